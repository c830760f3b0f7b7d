"""``rel_attn_fwd_lse`` (return_lse=True): the output at the parity tolerance
and each row's natural-log log-sum-exp against the fp64 oracle's, -inf
exactly for rows without visible keys. The call always runs split (one split
is taken as two), so this covers every kernel's split path with the merge
writing the log-sum-exps."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import compare, device_case, log
from paged_varlen_attention_gqa_amd import rel_attn_fwd
from paged_varlen_attention_gqa_amd.inputs import make_case, make_config

pytestmark = pytest.mark.gpu

# as for the split partials: fp32 score arithmetic over bf16 inputs
LSE_TOL = {torch.bfloat16: 1e-2, torch.float32: 1e-4}

def _no_keys():
    # requests 0 and 1 get cache length 0 on the device: their rows see no key
    case = make_case(name="no_keys", query_lens=[1, 20, 0, 1, 3], kv_lens=[40, 20, 10, 300, 50],
                     num_heads=8, num_kv_heads=2, head_dim=128, block_size=16, rel_extent=16)
    return case, {"cache_seqlens": torch.tensor([0, 0, 10, 300, 50], dtype=torch.int32)}


CASES = {
    "tiny_fp32": lambda: (make_config("tiny_fp32"), {}),
    "decode_b64_small": lambda: (make_config("decode_b64", scale=1 / 8), {}),
    "prefill_small": lambda: (make_config("prefill_chunked", scale=1 / 8), {}),
    "mixed_window_small": lambda: (make_config("mixed_window", scale=1 / 8), {}),
    "no_keys": _no_keys,
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    from paged_varlen_attention_gqa_amd import load_library

    load_library()


@pytest.mark.parametrize("splits", [None, 1, 7])
@pytest.mark.parametrize("name", sorted(CASES))
def test_fwd_lse(name, splits):
    case, over = CASES[name]()
    log(f"[lse] {name} splits={splits}: T={case.num_tokens} H={case.num_heads}")
    kw = device_case(case)
    kw.update({k: v.cuda() for k, v in over.items()})
    out, lse = rel_attn_fwd(**kw, num_splits=splits, return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.oracle_attention(**{**case.kwargs(), **over}, return_lse=True)
    compare(out, ref, case.dtype, what=f"{name} out")
    got = lse.cpu().double().numpy()
    assert np.array_equal(np.isneginf(got), np.isneginf(ref_lse)), "rows without keys differ"
    fin = ~np.isneginf(ref_lse)
    err = np.abs(got[fin] - ref_lse[fin]) if fin.any() else np.zeros(1)
    log(f"  {name}: lse max_abs={err.max():.3e} (tol {LSE_TOL[case.dtype]:g})")
    assert np.isfinite(got[fin]).all()
    assert err.max() <= LSE_TOL[case.dtype]
