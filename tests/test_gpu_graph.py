"""Capture of ``rel_attn_fwd`` in a HIP graph (torch.cuda.CUDAGraph) at fixed
shapes: every replay, with new input values copied into the captured buffers
and eager work between replays, matches an eager call on the same buffers bit
for bit, and the first replay matches the oracle. The library reads no device
value on the host and records no memset, so a call is capturable."""

import pytest
import torch

import oracle
from gpu_util import compare, device_case, log
from paged_varlen_attention_gqa_amd.inputs import make_case

pytestmark = pytest.mark.gpu

CASES = {
    # decode batch with splits (balanced decode kernel + combine kernel)
    "decode_splits": dict(query_lens=[1] * 12 + [3], kv_lens=[(211 * i) % 1900 + 60 for i in range(13)],
                          num_heads=16, num_kv_heads=4, head_dim=128, block_size=16, rel_extent=256),
    # sliding window, one split: prefill kernel + in-workgroup decode split
    "mixed_window": dict(query_lens=[40, 1, 1, 2], kv_lens=[300, 900, 2000, 50], num_heads=16,
                         num_kv_heads=2, head_dim=128, block_size=16, rel_extent=64, window_size=(255, 0)),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    from paged_varlen_attention_gqa_amd import load_library

    load_library()


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replay(name):
    from paged_varlen_attention_gqa_amd import rel_attn_fwd
    from paged_varlen_attention_gqa_amd.relattn import rel_attn_num_splits, rel_attn_workspace_bytes

    spec = CASES[name]
    cases = [make_case(name=name, seed=s, **spec) for s in (5, 6, 7, 8)]
    kw = device_case(cases[0])
    base = {k: kw[k].clone() for k in ("key_cache", "value_cache")}
    T, H, D = kw["q"].shape
    local = spec.get("window_size", (-1, -1)) != (-1, -1)
    ns = rel_attn_num_splits(is_local=local, batch_size=len(spec["query_lens"]),
                             max_query_len=kw["max_seqlen_q"], num_heads=H,
                             num_kv_heads=spec["num_kv_heads"],
                             max_kv_len=kw["block_table"].shape[1] * spec["block_size"])
    need = rel_attn_workspace_bytes(ns, T, H, D)
    log(f"[graph] {name}: num_splits={ns} workspace={need} B")
    out = torch.empty_like(kw["q"])
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=kw["q"].device)
    rel_attn_fwd(**kw, num_splits=ns, out=out, workspace=ws)  # eager warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rel_attn_fwd(**kw, num_splits=ns, out=out, workspace=ws)
    torch.cuda.synchronize()
    for i, c in enumerate(cases):
        src = device_case(c)
        # new values in the captured buffers; the metadata stays the captured
        # one, so the caches keep the captured layout: new finite values in the
        # slots the captured call references, NaN in the others
        for k in ("q", "rel_logits"):
            kw[k].copy_(src[k])
        for k in ("key_cache", "value_cache"):
            used = torch.isfinite(base[k])
            vals = torch.where(torch.isfinite(src[k]), src[k], torch.full_like(src[k], 0.25))
            kw[k].copy_(torch.where(used, vals, torch.full_like(vals, float("nan"))))
        out.zero_()
        ref = rel_attn_fwd(**kw, num_splits=ns)  # eager, its own output and workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"  replay {i}: max |graph - eager| = {(out.float() - ref.float()).abs().max().item():.3e}")
        assert torch.equal(out, ref), f"{name}: replay {i} differs from the eager call"
        if i == 0:
            compare(out, oracle.oracle_attention(**cases[0].kwargs()), cases[0].dtype, what=f"{name} replay 0")
