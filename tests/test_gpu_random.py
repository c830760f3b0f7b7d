"""Seeded random shapes against the oracle: batch sizes, query and KV lengths
(decode-shaped, prefill-shaped and mixed), GQA group sizes 1-16, head dims 64
and 128, block sizes (powers of two and not), relative extents (0, below 8,
around the lengths, past them), causal or not, windows on either side, fp32
and bf16, and split counts. Each case runs through rel_attn_fwd and is
compared element by element with the fp64 oracle at the parity tolerance.

A second set aims at the bf16 prefill kernel: longer query chunks over longer
caches, relative extents from 8 to past the lengths (so that key tiles fall
inside, across and outside the bias band, and bias runs reach the first and
last rows of rel_logits), group sizes 2-16, block sizes 16-64, windows, and
a bias of standard deviation up to 2."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import compare, device_case, log
from paged_varlen_attention_gqa_amd import rel_attn_fwd
from paged_varlen_attention_gqa_amd.inputs import make_case

pytestmark = pytest.mark.gpu

N_CASES = 40


def _spec(i: int) -> dict:
    r = np.random.default_rng(1000 + i)
    B = int(r.integers(1, 9))
    kind = r.choice(["decode", "prefill", "mixed"])
    q_lens, kv_lens = [], []
    for _ in range(B):
        if kind == "decode" or (kind == "mixed" and r.random() < 0.5):
            s = int(r.integers(1, 4))
        else:
            s = int(r.integers(5, 200))
        L = s + int(r.integers(0, 700))
        q_lens.append(s)
        kv_lens.append(L)
    Hkv = int(r.choice([1, 2, 4, 8]))
    G = int(r.choice([1, 2, 4, 8, 16]))
    D = int(r.choice([64, 128, 128]))
    bs = int(r.choice([16, 16, 32, 64, 7, 1]))
    E = int(r.choice([0, 5, 8, 13, 64, 300, 1000]))
    causal = bool(r.random() < 0.8)
    wl = int(r.choice([-1, -1, 0, 17, 128]))
    wr = int(r.choice([-1, -1, 0, 9])) if not causal else -1
    dtype = torch.float32 if r.random() < 0.2 else torch.bfloat16
    splits = [None, 1, 2, 5][int(r.integers(0, 4))]
    return dict(spec=dict(name=f"rand{i}", query_lens=q_lens, kv_lens=kv_lens, num_heads=Hkv * G,
                          num_kv_heads=Hkv, head_dim=D, block_size=bs, rel_extent=E, causal=causal,
                          window_size=(wl, wr), dtype=dtype, seed=i),
                splits=splits)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    from paged_varlen_attention_gqa_amd import load_library

    load_library()


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    d = _spec(i)
    case = make_case(**d["spec"])
    log(f"[random {i}] q={case.query_lens()} kv={case.kv_lens()} H={case.num_heads} Hkv={case.num_kv_heads} "
        f"D={case.head_dim} bs={case.block_size} E={case.rel_extent} causal={case.causal} "
        f"window={case.window_size} {case.dtype} splits={d['splits']}")
    kw = device_case(case)
    out = rel_attn_fwd(**kw, num_splits=d["splits"])
    torch.cuda.synchronize()
    ref = oracle.oracle_attention(**case.kwargs())
    compare(out, ref, case.dtype, what=f"random {i}")


N_PREFILL_CASES = 24


def _prefill_spec(i: int) -> dict:
    r = np.random.default_rng(5000 + i)
    B = int(r.integers(1, 5))
    q_lens, kv_lens = [], []
    for _ in range(B):
        s = int(r.integers(17, 700)) if r.random() < 0.8 else int(r.integers(1, 3))
        q_lens.append(s)
        kv_lens.append(s + int(r.integers(0, 2500)))
    Hkv = int(r.choice([1, 2, 4, 8]))
    G = int(r.choice([2, 4, 8, 16]))
    bs = int(r.choice([16, 32, 64]))
    E = int(r.choice([8, 13, 64, 100, 257, 1000, 4096]))
    causal = bool(r.random() < 0.85)
    wl = int(r.choice([-1, -1, -1, 31, 700]))
    wr = int(r.choice([-1, -1, 5])) if not causal else -1
    splits = [None, 1, 3][int(r.integers(0, 3))]
    return dict(spec=dict(name=f"randp{i}", query_lens=q_lens, kv_lens=kv_lens, num_heads=Hkv * G,
                          num_kv_heads=Hkv, head_dim=128, block_size=bs, rel_extent=E, causal=causal,
                          window_size=(wl, wr), rel_std=float(r.choice([1.0, 2.0])), seed=100 + i),
                splits=splits)


@pytest.mark.parametrize("i", range(N_PREFILL_CASES))
def test_random_prefill_case(i):
    d = _prefill_spec(i)
    case = make_case(**d["spec"])
    log(f"[random prefill {i}] q={case.query_lens()} kv={case.kv_lens()} H={case.num_heads} "
        f"Hkv={case.num_kv_heads} bs={case.block_size} E={case.rel_extent} causal={case.causal} "
        f"window={case.window_size} splits={d['splits']}")
    kw = device_case(case)
    out = rel_attn_fwd(**kw, num_splits=d["splits"])
    torch.cuda.synchronize()
    ref = oracle.oracle_attention(**case.kwargs())
    compare(out, ref, case.dtype, what=f"random prefill {i}")
