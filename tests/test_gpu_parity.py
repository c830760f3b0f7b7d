"""Parity of the HIP path with the fp64 oracle on the same seeded inputs.

Small and reduced-size workloads are compared on every output; the full-size
workloads (the sizes the benchmark times, in its launch configuration) are
compared on every output the oracle finishes quickly and on sampled rows
otherwise.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, compare, device_case, log, run_gpu
from paged_varlen_attention_gqa_amd.inputs import config_spec, make_case, make_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    from paged_varlen_attention_gqa_amd import load_library

    load_library()  # fails loudly when librelattn.so is missing


def _check(case, tokens=None, what=None, **over):
    what = what or case.name
    log(f"[parity] {what}: T={case.num_tokens} H={case.num_heads} Hkv={case.num_kv_heads} "
        f"D={case.head_dim} bs={case.block_size} E={case.rel_extent} over={over}")
    got = run_gpu(case, **over)
    ref = oracle.oracle_attention(**case.kwargs(), tokens=tokens)
    return compare(got, ref, case.dtype, tokens=tokens, what=what)


# ---- the five workloads at reduced size (every output) ----
REDUCED = [("tiny_fp32", 1.0), ("decode_b64", 1 / 8), ("prefill_chunked", 1 / 8),
           ("mixed_window", 1 / 8), ("decode_long_b1", 1 / 16)]


@pytest.mark.parametrize("name,scale", REDUCED, ids=[n for n, _ in REDUCED])
def test_reduced(name, scale):
    _check(make_config(name, scale=scale), what=f"{name}@{scale:g}")


# ---- full-size workloads ----
def test_full_tiny_fp32():
    _check(make_config("tiny_fp32"))


def test_full_decode_b64():
    _check(make_config("decode_b64"))


def test_full_decode_long_b1():
    _check(make_config("decode_long_b1"))


@pytest.mark.parametrize("name", ["decode_1m_b1_kv4", "decode_1m_b1_kv8"])
def test_full_decode_1m_b1(name):
    """Batch-1 decode over 2^20 keys (512 splits), 4 and 8 KV heads."""
    _check(make_config(name))


def _run_of_tokens(rng, S, n):
    """n consecutive query tokens of a request with S tokens, starting at a
    random multiple of n: with G query heads per KV head they are n * G
    consecutive packed rows, so every row position of a block of that many
    rows is compared."""
    start = n * int(rng.integers(0, S // n))
    return range(start, start + n)


def test_full_prefill_chunked_sampled():
    case = make_config("prefill_chunked")
    cu = case.cu_seqlens_q.tolist()
    rng = np.random.default_rng(0)
    tokens = set()
    for b in range(case.batch_size):
        S = cu[b + 1] - cu[b]
        picks = list(rng.choice(S, 12, replace=False)) + [0, S - 1] + list(_run_of_tokens(rng, S, 32))
        tokens.update(cu[b] + int(i) for i in picks)
    _check(case, tokens=tokens, what="prefill_chunked sampled")


def test_full_mixed_window_sampled():
    case = make_config("mixed_window")
    cu = case.cu_seqlens_q.tolist()
    rng = np.random.default_rng(1)
    tokens = set(range(cu[8], cu[-1]))  # every decode token
    for b in range(8):
        S = cu[b + 1] - cu[b]
        picks = list(rng.choice(S, 3, replace=False)) + [0, S - 1]
        if b % 2 == 0:
            picks += list(_run_of_tokens(rng, S, 32))
        tokens.update(cu[b] + int(i) for i in picks)
    _check(case, tokens=tokens, what="mixed_window sampled")


# ---- edge cases ----
EDGE = [
    dict(name="g1_noncausal", query_lens=[3, 40], kv_lens=[50, 40], num_heads=4, num_kv_heads=4,
         head_dim=128, block_size=16, rel_extent=20, causal=False),
    dict(name="g16_window_both", query_lens=[5, 1, 70], kv_lens=[130, 77, 200], num_heads=32,
         num_kv_heads=2, head_dim=128, block_size=16, rel_extent=50, causal=False, window_size=(33, 9)),
    dict(name="d64_bs64", query_lens=[1, 9, 33], kv_lens=[300, 65, 129], num_heads=8, num_kv_heads=2,
         head_dim=64, block_size=64, rel_extent=100),
    dict(name="odd_block_size", query_lens=[2, 17], kv_lens=[45, 99], num_heads=8, num_kv_heads=4,
         head_dim=128, block_size=7, rel_extent=13),
    dict(name="block_size_1", query_lens=[4, 1], kv_lens=[20, 31], num_heads=4, num_kv_heads=2,
         head_dim=64, block_size=1, rel_extent=8),
    dict(name="no_bias", query_lens=[6, 1], kv_lens=[66, 1000], num_heads=16, num_kv_heads=4,
         head_dim=128, block_size=16, rel_extent=0),
    dict(name="extent_beyond_len", query_lens=[8, 1], kv_lens=[30, 41], num_heads=8, num_kv_heads=8,
         head_dim=128, block_size=16, rel_extent=500),
    dict(name="empty_request", query_lens=[0, 5, 0, 1], kv_lens=[10, 5, 0, 3], num_heads=8,
         num_kv_heads=2, head_dim=128, block_size=16, rel_extent=4),
    dict(name="window_left_only", query_lens=[64, 1], kv_lens=[256, 900], num_heads=8, num_kv_heads=1,
         head_dim=128, block_size=16, rel_extent=64, window_size=(100, -1)),
    dict(name="fp32_d128_window", query_lens=[3, 20], kv_lens=[77, 20], num_heads=6, num_kv_heads=3,
         head_dim=128, block_size=16, rel_extent=40, window_size=(10, 0), dtype=torch.float32),
    dict(name="decode_extent_2", query_lens=[1, 1, 2], kv_lens=[40, 300, 17], num_heads=8,
         num_kv_heads=2, head_dim=128, block_size=16, rel_extent=2),
    dict(name="decode_extent_7", query_lens=[1, 3, 1], kv_lens=[40, 300, 17], num_heads=8,
         num_kv_heads=2, head_dim=128, block_size=16, rel_extent=7),
    dict(name="decode_extent_8", query_lens=[1, 3, 1], kv_lens=[40, 300, 9], num_heads=8,
         num_kv_heads=2, head_dim=128, block_size=16, rel_extent=8),
    dict(name="decode_extent_9_first_rows", query_lens=[1, 1], kv_lens=[5, 600], num_heads=4,
         num_kv_heads=1, head_dim=128, block_size=32, rel_extent=9),
    dict(name="decode_b80_mixed_lengths", query_lens=[1] * 76 + [2, 3, 1, 4],
         kv_lens=[(37 * i) % 700 + 1 for i in range(80)], num_heads=16, num_kv_heads=4, head_dim=128,
         block_size=16, rel_extent=64),
    dict(name="prefill_edge_rows_e8", query_lens=[40, 33], kv_lens=[40, 100], num_heads=8, num_kv_heads=2,
         head_dim=128, block_size=16, rel_extent=8),
    dict(name="prefill_edge_rows_e13_g8", query_lens=[25, 64], kv_lens=[25, 64], num_heads=16, num_kv_heads=2,
         head_dim=128, block_size=16, rel_extent=13),
    dict(name="prefill_extent_5", query_lens=[30], kv_lens=[50], num_heads=8, num_kv_heads=2,
         head_dim=128, block_size=16, rel_extent=5),
    dict(name="decode_window_wg_split", query_lens=[1, 2, 4, 1, 1], kv_lens=[700, 900, 1500, 2000, 40],
         num_heads=16, num_kv_heads=4, head_dim=128, block_size=16, rel_extent=64, window_size=(300, 0)),
    dict(name="decode_window_long_g8", query_lens=[1, 1, 2], kv_lens=[9000, 5000, 7000], num_heads=32,
         num_kv_heads=4, head_dim=128, block_size=64, rel_extent=2048, window_size=(4095, 0)),
    dict(name="fp32_noncausal_g4", query_lens=[1, 7], kv_lens=[90, 7], num_heads=8, num_kv_heads=2,
         head_dim=64, block_size=8, rel_extent=5, causal=False, dtype=torch.float32),
    # prefill with pages of more than 64 keys (a 64-key tile starts inside a page)
    dict(name="prefill_block_128", query_lens=[70, 130], kv_lens=[300, 501], num_heads=16, num_kv_heads=2,
         head_dim=128, block_size=128, rel_extent=200),
    dict(name="prefill_block_256_window", query_lens=[50, 9], kv_lens=[700, 260], num_heads=8, num_kv_heads=1,
         head_dim=128, block_size=256, rel_extent=64, window_size=(300, 0)),
]


@pytest.mark.parametrize("spec", EDGE, ids=[e["name"] for e in EDGE])
def test_edge(spec):
    spec = dict(spec)
    spec.setdefault("pool_pages", None)
    _check(make_case(**spec))


@pytest.mark.parametrize("splits", [1, 2, 3, 8, 37, 128, 300, 512])
def test_split_counts(splits):
    """Any split count gives the same result (the balanced decode kernel for
    this batch: at most 64 requests)."""
    case = make_case(name="splits", query_lens=[1, 1, 4, 1], kv_lens=[3000, 17, 700, 5000],
                     num_heads=16, num_kv_heads=4, head_dim=128, block_size=16, rel_extent=600)
    _check(case, num_splits=splits, what=f"splits={splits}")


def test_max_seqlen_bucketed():
    """A loose max_seqlen_q bound (next power of two, and more) gives the same output."""
    case = make_case(name="bucket", query_lens=[5, 17, 1], kv_lens=[40, 90, 20], num_heads=8,
                     num_kv_heads=2, head_dim=128, block_size=16, rel_extent=32)
    a = run_gpu(case)
    b = run_gpu(case, max_seqlen_q=32)
    c = run_gpu(case, max_seqlen_q=1000)
    assert torch.equal(a, b) and torch.equal(a, c)


def test_page_permutation_bitwise():
    """Moving pages to other physical slots (and relabelling the table) changes no bit."""
    case = make_case(name="perm", query_lens=[1, 30, 2], kv_lens=[500, 300, 1200], num_heads=16,
                     num_kv_heads=4, head_dim=128, block_size=16, rel_extent=256, pool_pages=200)
    a = run_gpu(case)
    g = torch.Generator().manual_seed(7)
    perm = torch.randperm(case.key_cache.shape[0], generator=g)
    kc = torch.empty_like(case.key_cache)
    vc = torch.empty_like(case.value_cache)
    kc[perm] = case.key_cache
    vc[perm] = case.value_cache
    bt = perm[case.block_table.long()].to(torch.int32)
    b = run_gpu(case, key_cache=kc.cuda(), value_cache=vc.cuda(), block_table=bt.cuda())
    assert torch.equal(a, b)


def test_kv_shorter_than_queries_gives_zero_rows():
    """Rows whose position is negative (L_b < S_b) see no key and come out as zeros."""
    case = make_case(name="short", query_lens=[4], kv_lens=[4], num_heads=4, num_kv_heads=2,
                     head_dim=128, block_size=16, rel_extent=4)
    kw = device_case(case)
    kw["cache_seqlens"] = torch.tensor([2], dtype=torch.int32, device="cuda")
    from paged_varlen_attention_gqa_amd import rel_attn_fwd

    out = rel_attn_fwd(**kw)
    torch.cuda.synchronize()
    ref_kw = case.kwargs()
    ref_kw["cache_seqlens"] = torch.tensor([2], dtype=torch.int32)
    ref = oracle.oracle_attention(**ref_kw)
    compare(out, ref, case.dtype, what="L<S")
    assert torch.count_nonzero(out[:2]) == 0


def test_preallocated_out_and_determinism():
    case = make_config("decode_b64", scale=1 / 16)
    kw = device_case(case)
    from paged_varlen_attention_gqa_amd import rel_attn_fwd

    out = torch.full_like(kw["q"], float("nan"))
    r = rel_attn_fwd(**kw, out=out)
    assert r.data_ptr() == out.data_ptr()
    r2 = rel_attn_fwd(**kw)
    torch.cuda.synchronize()
    assert torch.equal(r, r2)


@pytest.mark.parametrize("splits", [1, 4])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_requests_without_keys_give_zeros(splits, dtype):
    """Requests whose cache length is 0 (one decode query, a 20-query chunk)
    see no key: their rows are zeros, written over a NaN-filled output."""
    case = make_case(name="no_keys", query_lens=[1, 20, 1, 3], kv_lens=[40, 20, 300, 50],
                     num_heads=8, num_kv_heads=2, head_dim=128, block_size=16, rel_extent=16,
                     dtype=dtype)
    lens = torch.tensor([0, 0, 300, 50], dtype=torch.int32)
    kw = device_case(case)
    kw["cache_seqlens"] = lens.cuda()
    from paged_varlen_attention_gqa_amd import rel_attn_fwd

    out = torch.full_like(kw["q"], float("nan"))
    rel_attn_fwd(**kw, num_splits=splits, out=out)
    torch.cuda.synchronize()
    ref_kw = case.kwargs()
    ref_kw["cache_seqlens"] = lens
    ref = oracle.oracle_attention(**ref_kw)
    compare(out, ref, case.dtype, what=f"no keys splits={splits}")
    assert torch.count_nonzero(out[:21]) == 0


def test_cache_over_4gb():
    """K/V caches past 4 GB (the prefill kernel's per-page resources): the
    pages of a small case are placed at the far end of a 4.6 GB pool."""
    case = make_case(name="wide_cache", query_lens=[100, 1, 70], kv_lens=[300, 90, 70], num_heads=16,
                     num_kv_heads=8, head_dim=128, block_size=16, rel_extent=64, seed=3)
    big = 150000  # pages of 32 KB: 4.6 GB per cache
    kw = device_case(case)
    bt = case.block_table.clone()
    used = sorted(set(int(x) for x in bt.flatten().tolist()))
    remap = {p: big - 1 - 5 * i for i, p in enumerate(used)}
    bt_big = bt.clone().apply_(lambda x: remap[int(x)])
    log(f"[parity] wide_cache: {len(used)} pages mapped to {min(remap.values())}..{max(remap.values())} of {big}")
    for name in ("key_cache", "value_cache"):
        small = kw[name]
        pool = torch.empty((big,) + tuple(small.shape[1:]), dtype=small.dtype, device=small.device)
        src = torch.tensor(used, dtype=torch.int64, device=small.device)
        dst = torch.tensor([remap[p] for p in used], dtype=torch.int64, device=small.device)
        pool[dst] = small[src]
        kw[name] = pool
    kw["block_table"] = bt_big.to(kw["q"].device)
    from paged_varlen_attention_gqa_amd import rel_attn_fwd

    got = rel_attn_fwd(**kw)
    torch.cuda.synchronize()
    ref = oracle.oracle_attention(**case.kwargs())
    compare(got, ref, case.dtype, what="wide_cache")
