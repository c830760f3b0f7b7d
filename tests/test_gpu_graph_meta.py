"""Graph replays whose request metadata changes between replays.

A serving loop captures the attention call once per batch-shape bucket (fixed
tensor shapes: token rows, batch slots, page-table width, page pool, the bound
``max_seqlen_q`` and ``num_splits``) and replays it every step with new
``cu_seqlens_q``, ``cache_seqlens`` and ``block_table`` contents (the vLLM
pull-request report on prhub.com.cn, 关联脉络, names piecewise CUDA-graph
capture for this op). The kernels derive every request's rows, key range and
work split from those device tensors, so one captured graph must serve any
step that fits its bucket: decode-only, mixed prefill and decode, padded
slots (no queries, no keys) and fully empty steps.

Per bucket the call is captured once; each step copies its case into the
captured buffers (rows past the step's tokens and pool slots it does not use
hold NaN), replays, and checks the step's rows against an eager call on the
same buffers (bit for bit) and against the fp64 oracle of the step's own
unpadded case. Eager calls run between replays."""

import pytest
import torch

import oracle
from gpu_util import compare, log
from paged_varlen_attention_gqa_amd.inputs import make_case

pytestmark = pytest.mark.gpu

BUCKETS = {
    # 16 decode slots, up to 2 query tokens each, 2048 keys of page table
    "decode16": dict(B=16, T=32, max_q=2, mb=128, pool=1200, H=32, Hkv=8, E=256, bs=16, window=(-1, -1),
                     steps=[
                         ([1] * 16, [2048, 1, 17, 500, 1999, 64, 1024, 300, 2, 1500, 777, 16, 33, 1000, 250, 1200]),
                         ([2, 1, 0, 1, 2, 0, 1, 1, 0, 2, 1, 1, 0, 0, 1, 2],
                          [100, 2048, 0, 5, 2, 40, 1, 900, 0, 1800, 60, 3, 0, 7, 333, 2000]),
                         ([1, 1, 2] + [0] * 13, [2048, 129, 2] + [0] * 13),
                         ([0] * 16, [0] * 16),
                         ([0] * 16, [50] * 16),
                         ([1] * 16, [2048] * 8 + [1] * 8),
                     ]),
    # 4 slots of chunked prefill (up to 320 queries), 1280 keys of page table
    "chunked4": dict(B=4, T=640, max_q=320, mb=80, pool=200, H=16, Hkv=2, E=128, bs=16, window=(-1, -1),
                     steps=[
                         ([320, 1, 200, 64], [1280, 700, 200, 900]),
                         ([1, 1, 1, 1], [1000, 3, 1280, 50]),
                         ([0, 300, 0, 17], [0, 300, 10, 1100]),
                         ([0, 0, 0, 0], [0, 0, 0, 0]),
                         ([320, 320, 0, 0], [320, 1280, 0, 0]),
                     ]),
    # sliding window (127, 0), 8 slots mixing prefill chunks and decode
    "window8": dict(B=8, T=160, max_q=96, mb=64, pool=300, H=16, Hkv=4, E=64, bs=16, window=(127, 0),
                    steps=[
                        ([96, 1, 1, 2, 40, 1, 0, 19], [1024, 1000, 5, 2, 40, 600, 0, 300]),
                        ([1] * 8, [1024, 128, 127, 1, 900, 64, 129, 1000]),
                        ([50] + [0] * 7, [50] + [0] * 7),
                        ([0] * 8, [0] * 8),
                    ]),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    from paged_varlen_attention_gqa_amd import load_library

    load_library()


def _step_case(bk, i, qlens, kvlens):
    return make_case(name=f"step{i}", query_lens=qlens, kv_lens=kvlens, num_heads=bk["H"],
                     num_kv_heads=bk["Hkv"], head_dim=128, block_size=bk["bs"], rel_extent=bk["E"],
                     window_size=bk["window"], seed=200 + i, pool_pages=bk["pool"],
                     max_blocks_per_seq=bk["mb"], max_seqlen_q=bk["max_q"])


@pytest.mark.parametrize("name", sorted(BUCKETS))
def test_graph_varying_metadata(name):
    from paged_varlen_attention_gqa_amd import rel_attn_fwd
    from paged_varlen_attention_gqa_amd.relattn import rel_attn_num_splits, rel_attn_workspace_bytes

    bk = BUCKETS[name]
    dev = torch.device("cuda:0")
    B, T, H, Hkv, E, bs, mb, pool = bk["B"], bk["T"], bk["H"], bk["Hkv"], bk["E"], bk["bs"], bk["mb"], bk["pool"]
    nan = float("nan")
    # the captured buffers, at the bucket's shapes
    buf = dict(
        q=torch.full((T, H, 128), nan, dtype=torch.bfloat16, device=dev),
        key_cache=torch.full((pool, bs, Hkv, 128), nan, dtype=torch.bfloat16, device=dev),
        value_cache=torch.full((pool, bs, Hkv, 128), nan, dtype=torch.bfloat16, device=dev),
        block_table=torch.zeros((B, mb), dtype=torch.int32, device=dev),
        cache_seqlens=torch.zeros((B,), dtype=torch.int32, device=dev),
        cu_seqlens_q=torch.zeros((B + 1,), dtype=torch.int32, device=dev),
        rel_logits=torch.full((T, H, E), nan, dtype=torch.bfloat16, device=dev),
    )
    fixed = dict(max_seqlen_q=bk["max_q"], softmax_scale=128 ** -0.5, causal=True, window_size=bk["window"],
                 rel_extent=E)
    local = bk["window"] != (-1, -1)
    ns = rel_attn_num_splits(is_local=local, batch_size=B, max_query_len=bk["max_q"], num_heads=H,
                             num_kv_heads=Hkv, max_kv_len=mb * bs)
    need = rel_attn_workspace_bytes(ns, T, H, 128)
    out = torch.full((T, H, 128), nan, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    log(f"[graph-meta] {name}: B={B} T={T} max_q={bk['max_q']} num_splits={ns} workspace={need} B")

    def load(case):
        t = case.num_tokens
        for k in ("q", "rel_logits"):
            buf[k].fill_(nan)
            buf[k][:t].copy_(getattr(case, k))
        for k in ("key_cache", "value_cache", "block_table", "cache_seqlens", "cu_seqlens_q"):
            buf[k].copy_(getattr(case, k))

    cases = [_step_case(bk, i, q, kv) for i, (q, kv) in enumerate(bk["steps"])]
    load(cases[0])
    rel_attn_fwd(**buf, **fixed, num_splits=ns, out=out, workspace=ws)  # eager warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rel_attn_fwd(**buf, **fixed, num_splits=ns, out=out, workspace=ws)
    torch.cuda.synchronize()

    # every step once, then the first steps again after the small ones
    order = list(range(len(cases))) + [0, 1]
    for n, i in enumerate(order):
        case = cases[i]
        t = case.num_tokens
        log(f"  replay {n}: step {i} query_lens={case.query_lens()} kv_lens={case.kv_lens()}")
        load(case)
        out.fill_(nan)
        ref = rel_attn_fwd(**buf, **fixed, num_splits=ns)  # eager, its own output and workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out[:t]
        assert torch.equal(got, ref[:t]), f"{name}: replay {n} (step {i}) differs from the eager call"
        if t > 0:
            compare(got, oracle.oracle_attention(**case.kwargs()), case.dtype, what=f"{name} replay {n} step {i}")
