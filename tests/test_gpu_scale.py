"""Parity at softmax scales other than 1/sqrt(head_dim), with a wide bias (std 2).

The docs.vllm.ai ``inkling_fa4_rel_attention`` signature takes ``softmax_scale``
as a free argument, and the prhub.com.cn report's ``score_mod_rel_bias`` adds
the bias to the already-scaled score: the bias itself is never scaled. Scales
whose reciprocal is not a bf16 number (0.49806, 0.0707, 0.3) and ones whose
reciprocal is (1.0, 0.125) take different selection operands in the prefill
kernel; zero and negative scales go to the general kernel. Every output is
compared with the fp64 oracle.
"""

import pytest
import torch

import oracle
from gpu_util import compare, log, run_gpu
from paged_varlen_attention_gqa_amd.inputs import make_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    from paged_varlen_attention_gqa_amd import load_library

    load_library()


SHAPES = {
    # prefill-shaped: two requests of 200 and 64 queries (G = 8), E = 256
    "prefill": dict(query_lens=[200, 64], kv_lens=[700, 64], num_heads=16, num_kv_heads=2,
                    head_dim=128, block_size=16, rel_extent=256),
    # mixed decode and prefill requests (G = 8)
    "mixed": dict(query_lens=[1, 300, 1, 2], kv_lens=[2000, 900, 37, 500], num_heads=32, num_kv_heads=4,
                  head_dim=128, block_size=16, rel_extent=300),
    # decode-shaped: 8 single-token requests (G = 4)
    "decode": dict(query_lens=[1] * 8, kv_lens=[100, 3000, 517, 64, 2048, 1, 999, 1500], num_heads=32,
                   num_kv_heads=8, head_dim=128, block_size=16, rel_extent=512),
}
SCALES = [0.49806, 0.0707, 0.3, 1.0, 0.125]


@pytest.mark.parametrize("scale", SCALES, ids=[f"s{s:g}" for s in SCALES])
@pytest.mark.parametrize("shape", sorted(SHAPES))
def test_scale(shape, scale):
    case = make_case(name=f"{shape}_scale", softmax_scale=scale, rel_std=2.0, seed=11, **SHAPES[shape])
    log(f"[scale] {shape} softmax_scale={scale} rel_std=2")
    got = run_gpu(case)
    ref = oracle.oracle_attention(**case.kwargs())
    compare(got, ref, case.dtype, what=f"{shape} scale={scale}")


@pytest.mark.parametrize("scale", [0.0, -0.05])
def test_non_positive_scale(scale):
    """softmax_scale 0 (scores are the bias alone) and a negative scale."""
    case = make_case(name="nonpos_scale", softmax_scale=scale, rel_std=2.0, seed=12, **SHAPES["mixed"])
    log(f"[scale] mixed softmax_scale={scale}")
    got = run_gpu(case)
    ref = oracle.oracle_attention(**case.kwargs())
    compare(got, ref, case.dtype, what=f"mixed scale={scale}")


def test_scale_with_splits():
    """A non-default scale through the split path (partials and merge)."""
    case = make_case(name="split_scale", softmax_scale=0.3, rel_std=2.0, seed=13, **SHAPES["prefill"])
    got = run_gpu(case, num_splits=3)
    ref = oracle.oracle_attention(**case.kwargs())
    compare(got, ref, case.dtype, what="prefill scale=0.3 splits=3")
