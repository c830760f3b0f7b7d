"""rel_attn_fwd_noalloc, the entry point for callers that cannot allocate: its
output equals rel_attn_fwd's (same kernels, same split count: bit for bit)
and the fp64 oracle's within the bf16 tolerance, on two calls in a row, the
second smaller, both through the split path that uses the library's static
scratch array. Calls whose workspace exceeds the array are refused before any
device work (CPU-side checks in test_abi.py)."""

import pytest
import torch

import oracle
from gpu_util import compare, device_case, log
from paged_varlen_attention_gqa_amd import (RelAttnError, rel_attn_fwd, rel_attn_fwd_noalloc,
                                           rel_attn_noalloc_scratch_bytes, rel_attn_workspace_bytes)
from paged_varlen_attention_gqa_amd.inputs import make_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    from paged_varlen_attention_gqa_amd import load_library

    load_library()


# first a larger mixed batch (decode requests and a 96-token prefill chunk),
# then a smaller decode-only batch
CASES = [
    (dict(name="noalloc_big", query_lens=[1] * 20 + [96, 3], kv_lens=[(311 * i) % 3000 + 40 for i in range(20)] + [900, 77],
          num_heads=32, num_kv_heads=8, head_dim=128, block_size=16, rel_extent=256, seed=21), 12),
    (dict(name="noalloc_small", query_lens=[1] * 5, kv_lens=[700, 31, 2000, 129, 64], num_heads=16,
          num_kv_heads=4, head_dim=128, block_size=16, rel_extent=128, seed=22), 5),
]


def test_noalloc_matches_fwd_twice():
    limit = rel_attn_noalloc_scratch_bytes()
    assert limit == 32 << 20
    for spec, splits in CASES:
        case = make_case(**spec)
        need = rel_attn_workspace_bytes(splits, case.num_tokens, case.num_heads, case.head_dim)
        log(f"[noalloc] {case.name}: T={case.num_tokens} splits={splits} workspace {need} of {limit} bytes")
        assert 0 < need <= limit
        kw = device_case(case)
        ref = rel_attn_fwd(**kw, num_splits=splits)
        out = torch.full_like(kw["q"], float("nan"))
        got = rel_attn_fwd_noalloc(**kw, num_splits=splits, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got, ref), f"{case.name}: noalloc output differs from rel_attn_fwd"
        compare(got, oracle.oracle_attention(**case.kwargs()), case.dtype, what=f"{case.name} noalloc")


def test_noalloc_one_split_and_too_large():
    """One split needs no scratch; a workspace past the limit is refused with an error."""
    case = make_case(**CASES[1][0])
    kw = device_case(case)
    got = rel_attn_fwd_noalloc(**kw, num_splits=1)
    ref = rel_attn_fwd(**kw, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    big = make_case(name="noalloc_too_big", query_lens=[4096], kv_lens=[4096], num_heads=32, num_kv_heads=8,
                    head_dim=128, block_size=16, rel_extent=0, seed=23)
    assert rel_attn_workspace_bytes(2, big.num_tokens, big.num_heads, big.head_dim) > rel_attn_noalloc_scratch_bytes()
    with pytest.raises(RelAttnError, match="workspace"):
        rel_attn_fwd_noalloc(**device_case(big), num_splits=2)
