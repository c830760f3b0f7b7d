"""Pins for the fp64 oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` function takes the three oracle entry points (so that the
mutation test can hand it a deliberately broken copy of the oracle) and raises
``AssertionError`` when the oracle disagrees with the pinned fact. The pins
never call the HIP library.
"""

from __future__ import annotations

import json
import os

import numpy as np
import torch

from paged_varlen_attention_gqa_amd.inputs import make_case

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_cases.json")


def load_golden():
    with open(GOLDEN) as f:
        data = json.load(f)
    out = []
    for c in data["cases"]:
        def t(x, dtype=torch.float64):
            arr = np.array(x, dtype=object)
            arr = np.where(arr == None, np.nan, arr).astype(np.float64)  # noqa: E711
            return torch.from_numpy(arr).to(dtype)

        kw = dict(
            q=t(c["q"]), key_cache=t(c["key_cache"]), value_cache=t(c["value_cache"]),
            block_table=torch.tensor(c["block_table"], dtype=torch.int32),
            cache_seqlens=torch.tensor(c["cache_seqlens"], dtype=torch.int32),
            cu_seqlens_q=torch.tensor(c["cu_seqlens_q"], dtype=torch.int32),
            max_seqlen_q=max(np.diff(c["cu_seqlens_q"])),
            softmax_scale=float(c["softmax_scale"]), causal=bool(c["causal"]),
            window_size=tuple(c["window_size"]), rel_extent=int(c["rel_extent"]),
            rel_logits=t(c["rel_logits"]),
        )
        out.append((c["name"], kw, np.array(c["expected_out"], dtype=np.float64)))
    return out


def load_golden_lse():
    """(name, kwargs, expected_lse) of every golden case; "-inf" marks a row with no visible key."""
    with open(GOLDEN) as f:
        data = json.load(f)
    lses = {c["name"]: np.array([[float(x) for x in row] for row in c["expected_lse"]]) for c in data["cases"]}
    return [(name, kw, lses[name]) for name, kw, _ in load_golden()]


def small_case(seed=0, **over):
    spec = dict(query_lens=[3, 1, 6], kv_lens=[9, 13, 6], num_heads=4, num_kv_heads=2, head_dim=8,
                block_size=4, rel_extent=5, causal=True, window_size=(-1, -1),
                dtype=torch.float32, seed=seed)
    spec.update(over)
    return make_case(**spec)


def _sdpa_ref(case, mask_fn):
    """Per request, SDPA (library routine, fp64) over logically gathered, GQA-expanded K/V."""
    T, H, D = case.q.shape
    G = case.num_heads // case.num_kv_heads
    out = np.zeros((T, H, D))
    cu = case.cu_seqlens_q.tolist()
    for b, L in enumerate(case.cache_seqlens.tolist()):
        S = cu[b + 1] - cu[b]
        if S == 0:
            continue
        bs = case.block_size
        pages = case.block_table[b, : (L + bs - 1) // bs].long()
        K = case.key_cache[pages].reshape(-1, case.num_kv_heads, D)[:L].double()
        V = case.value_cache[pages].reshape(-1, case.num_kv_heads, D)[:L].double()
        K = K.repeat_interleave(G, dim=1).permute(1, 0, 2).contiguous()  # (H, L, D)
        V = V.repeat_interleave(G, dim=1).permute(1, 0, 2).contiguous()
        Q = case.q[cu[b]: cu[b + 1]].double().permute(1, 0, 2).contiguous()  # (H, S, D)
        m = mask_fn(S, L)
        o = torch.nn.functional.scaled_dot_product_attention(
            Q, K, V, attn_mask=m, scale=case.softmax_scale) if m is not None else \
            torch.nn.functional.scaled_dot_product_attention(
                Q, K, V, is_causal=True, scale=case.softmax_scale)
        out[cu[b]: cu[b + 1]] = o.permute(1, 0, 2).numpy()
    return out


def _forms(oa, ob, osc):
    """The three forms of the oracle, each as a plain attention function."""
    return [oa, ob, lambda **kw: osc(**kw, num_splits=3)]


def pin_golden(oa, ob, osc):
    for name, kw, exp in load_golden():
        got = oa(**kw)
        assert np.allclose(got, exp, rtol=0, atol=1e-12), (name, got, exp)
        got_b = ob(**kw)
        assert np.allclose(got_b, exp, rtol=0, atol=1e-12), ("bruteforce", name, got_b, exp)
        got_s = osc(**kw, num_splits=2)
        assert np.allclose(got_s, exp, rtol=0, atol=1e-12), ("split", name, got_s, exp)


def pin_sdpa_no_bias(oa, ob, osc):
    """rel_extent = 0 (and rel_logits = 0) reduce to SDPA with a bottom-right causal mask."""
    for f in _forms(oa, ob, osc):
        case = small_case(rel_extent=0, seed=1)

        def causal_br(S, L):  # keys j <= i + (L - S): torch.tril with a diagonal offset
            return torch.tril(torch.ones(S, L, dtype=torch.bool), diagonal=L - S)

        ref = _sdpa_ref(case, causal_br)
        got = f(**case.kwargs())
        assert np.allclose(got, ref, rtol=0, atol=1e-12), np.abs(got - ref).max()
        case2 = small_case(seed=2)
        case2.rel_logits.zero_()
        ref2 = _sdpa_ref(case2, causal_br)
        got2 = f(**case2.kwargs())
        assert np.allclose(got2, ref2, rtol=0, atol=1e-12)
        # sliding window (left, right) as a band: torch.triu/tril offsets
        case3 = small_case(rel_extent=0, seed=3, window_size=(2, 1), causal=False)

        def band(S, L):
            o = L - S
            ones = torch.ones(S, L, dtype=torch.bool)
            return torch.tril(ones, diagonal=o + 1) & torch.triu(ones, diagonal=o - 2)

        ref3 = _sdpa_ref(case3, band)
        got3 = f(**case3.kwargs())
        assert np.allclose(got3, ref3, rtol=0, atol=1e-12), np.abs(got3 - ref3).max()


def pin_top_left_causal(oa, ob, osc):
    """With S_b = L_b the bottom-right causal mask is the usual top-left one (is_causal=True)."""
    for f in _forms(oa, ob, osc):
        case = small_case(query_lens=[7, 4], kv_lens=[7, 4], rel_extent=0, seed=4)
        ref = _sdpa_ref(case, lambda S, L: None)
        got = f(**case.kwargs())
        assert np.allclose(got, ref, rtol=0, atol=1e-12)


def pin_one_hot_bias(oa, ob, osc):
    """A single huge bias entry at distance d0 selects key p - d0 (closed form)."""
    for f in _forms(oa, ob, osc):
        case = small_case(seed=5, qkv_std=0.05, rel_extent=8, query_lens=[4, 2], kv_lens=[12, 9])
        case.rel_logits.zero_()
        T, H, _ = case.q.shape
        cu = case.cu_seqlens_q.tolist()
        d0s = {}
        for b, L in enumerate(case.cache_seqlens.tolist()):
            S = cu[b + 1] - cu[b]
            for i in range(S):
                t = cu[b] + i
                p = i + L - S
                for h in range(H):
                    d0 = (3 * t + h) % min(8, p + 1)
                    case.rel_logits[t, h, d0] = 60.0
                    d0s[(t, h)] = (b, p - d0)
        got = f(**case.kwargs())
        G = case.num_heads // case.num_kv_heads
        for (t, h), (b, j) in d0s.items():
            page = int(case.block_table[b, j // case.block_size])
            v = case.value_cache[page, j % case.block_size, h // G].double().numpy()
            assert np.allclose(got[t, h], v, rtol=0, atol=1e-20 + 1e-12), (t, h, got[t, h], v)


def pin_single_visible_key(oa, ob, osc):
    """Window (0, 0): only key p is visible, so the output is exactly that V row."""
    for f in _forms(oa, ob, osc):
        case = small_case(seed=6, window_size=(0, 0))
        got = f(**case.kwargs())
        cu = case.cu_seqlens_q.tolist()
        G = case.num_heads // case.num_kv_heads
        for b, L in enumerate(case.cache_seqlens.tolist()):
            S = cu[b + 1] - cu[b]
            for i in range(S):
                p = i + L - S
                page = int(case.block_table[b, p // case.block_size])
                for h in range(case.num_heads):
                    v = case.value_cache[page, p % case.block_size, h // G].double().numpy()
                    assert np.array_equal(got[cu[b] + i, h], v)


def pin_gqa_expansion(oa, ob, osc):
    """Repeating each KV head G times (repeat_interleave) and calling with H KV heads changes nothing."""
    for f in _forms(oa, ob, osc):
        case = small_case(seed=7, num_heads=8, num_kv_heads=2)
        ref = f(**case.kwargs())
        kw = case.kwargs()
        kw["key_cache"] = case.key_cache.repeat_interleave(4, dim=2)
        kw["value_cache"] = case.value_cache.repeat_interleave(4, dim=2)
        got = f(**kw)
        assert np.allclose(got, ref, rtol=0, atol=1e-13)


def pin_page_permutation(oa, ob, osc):
    """Relabelling physical pages (moving their contents) leaves the output unchanged."""
    for f in _forms(oa, ob, osc):
        case = small_case(seed=8, pool_pages=40)
        ref = f(**case.kwargs())
        g = torch.Generator().manual_seed(123)
        perm = torch.randperm(case.key_cache.shape[0], generator=g)  # new page id for old page i
        kw = case.kwargs()
        kc = torch.empty_like(case.key_cache)
        vc = torch.empty_like(case.value_cache)
        kc[perm] = case.key_cache
        vc[perm] = case.value_cache
        kw["key_cache"], kw["value_cache"] = kc, vc
        kw["block_table"] = perm[case.block_table.long()].to(torch.int32)
        got = f(**kw)
        assert np.array_equal(got, ref)


def pin_constant_bias(oa, ob, osc):
    """A bias constant over every reachable distance cancels in the softmax."""
    for f in _forms(oa, ob, osc):
        case = small_case(seed=9, rel_extent=32)
        ref_kw = case.kwargs()
        ref_kw["rel_extent"] = 0
        ref = f(**ref_kw)
        case.rel_logits.copy_(torch.full_like(case.rel_logits, 2.5))
        got = f(**case.kwargs())
        assert np.allclose(got, ref, rtol=0, atol=1e-12)


def pin_extent_endpoint(oa, ob, osc):
    """Distance E-1 is biased and distance E is not (half-open range)."""
    for f in _forms(oa, ob, osc):
        case = small_case(seed=10, rel_extent=3, query_lens=[1], kv_lens=[6], qkv_std=0.01)
        case.rel_logits.zero_()
        case.rel_logits[0, :, 2] = 50.0  # d = 2 = E-1 -> key p-2 dominates
        got = f(**case.kwargs())
        p = 5
        G = case.num_heads // case.num_kv_heads
        for h in range(case.num_heads):
            j = p - 2
            page = int(case.block_table[0, j // case.block_size])
            v = case.value_cache[page, j % case.block_size, h // G].double().numpy()
            assert np.allclose(got[0, h], v, atol=1e-12)
        # same tensor seen with rel_extent = 2: the entry at d = 2 is now out of range
        kw = case.kwargs()
        kw["rel_extent"] = 2
        kw["rel_logits"] = case.rel_logits[:, :, :2].contiguous()
        kw0 = case.kwargs()
        kw0["rel_extent"] = 0
        assert np.allclose(f(**kw), f(**kw0), atol=1e-12)


def pin_split_combine(oa, ob, osc):
    """The split-KV log-sum-exp merge reproduces the one-pass result for any split count."""
    case = small_case(seed=11, query_lens=[3, 2], kv_lens=[17, 11])
    ref = oa(**case.kwargs())
    for k in (1, 2, 3, 7, 40):
        got = osc(**case.kwargs(), num_splits=k)
        assert np.allclose(got, ref, rtol=0, atol=1e-12), k


def pin_request_order(oa, ob, osc):
    """Reordering requests permutes the output rows the same way."""
    for f in _forms(oa, ob, osc):
        case = small_case(seed=12)
        ref = f(**case.kwargs())
        order = [2, 0, 1]
        cu = case.cu_seqlens_q.tolist()
        rows = [list(range(cu[b], cu[b + 1])) for b in range(3)]
        new_rows = sum((rows[b] for b in order), [])
        kw = case.kwargs()
        kw["q"] = case.q[new_rows]
        kw["rel_logits"] = case.rel_logits[new_rows]
        kw["block_table"] = case.block_table[order]
        kw["cache_seqlens"] = case.cache_seqlens[order]
        lens = [len(rows[b]) for b in order]
        kw["cu_seqlens_q"] = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
        got = f(**kw)
        assert np.allclose(got, ref[new_rows], rtol=0, atol=1e-13)


def pin_bruteforce(oa, ob, osc):
    """The scalar-loop form and the vectorised form agree on tiny cases of every mask mode."""
    modes = [(True, (-1, -1)), (False, (-1, -1)), (True, (3, 0)), (False, (2, 2)), (True, (-1, 1)),
             (False, (-1, 0)), (False, (0, -1))]
    i = 0
    for causal, win in modes:
        for E in (0, 1, 7, 30):
            for H, Hkv in ((2, 2), (4, 2), (4, 1)):
                for bs in (1, 4, 16):
                    i += 1
                    if i % 3:  # a third of the grid keeps the CPU suite short
                        continue
                    case = small_case(seed=100 + i, causal=causal, window_size=win, rel_extent=E,
                                      num_heads=H, num_kv_heads=Hkv, block_size=bs,
                                      query_lens=[2, 1, 4], kv_lens=[5, 9, 4], head_dim=4,
                                      dtype=torch.bfloat16 if i % 2 else torch.float32)
                    a = oa(**case.kwargs())
                    b = ob(**case.kwargs())
                    assert np.allclose(a, b, rtol=0, atol=1e-12), (causal, win, E, H, Hkv, bs)


def _same_lse(got, exp, atol):
    """Equal within atol, with -inf exactly where the expected value is -inf."""
    got = np.asarray(got, dtype=np.float64)
    exp = np.asarray(exp, dtype=np.float64)
    assert got.shape == exp.shape, (got.shape, exp.shape)
    assert np.array_equal(np.isneginf(got), np.isneginf(exp)), (got, exp)
    fin = np.isfinite(exp)
    assert np.all(np.isfinite(got[fin])), got
    assert np.allclose(got[fin], exp[fin], rtol=0, atol=atol), np.abs(got[fin] - exp[fin]).max()


def pin_lse_golden(oa, ob, osc):
    """Log-sum-exp of the hand-derived cases (ln 4, ln 5, ..., -inf for a row with no key)."""
    for name, kw, exp in load_golden_lse():
        _, lse = oa(**kw, return_lse=True)
        _same_lse(lse, exp, 1e-12)


def _mask_count(S, L, causal, window):
    """Visible-key mask (S, L) built from torch.tril / torch.triu band offsets (query i at p = i + L - S)."""
    o = L - S
    m = torch.ones(S, L, dtype=torch.bool)
    if causal:
        m &= torch.tril(torch.ones(S, L, dtype=torch.bool), diagonal=o)
    wl, wr = window
    if wl >= 0:
        m &= torch.triu(torch.ones(S, L, dtype=torch.bool), diagonal=o - wl)
    if wr >= 0:
        m &= torch.tril(torch.ones(S, L, dtype=torch.bool), diagonal=o + wr)
    return m


def pin_lse_uniform(oa, ob, osc):
    """q = 0 and no bias make every visible score 0, so the log-sum-exp is ln(visible keys)."""
    for causal, win in ((True, (-1, -1)), (True, (3, 0)), (False, (2, 1)), (False, (-1, -1))):
        case = small_case(seed=20, rel_extent=0, causal=causal, window_size=win,
                          query_lens=[3, 1, 6, 2], kv_lens=[9, 13, 6, 2])
        case.cache_seqlens[3] = 1  # two queries over one key: the first sits at p = -1
        case.q.zero_()
        _, lse = oa(**case.kwargs(), return_lse=True)
        cu = case.cu_seqlens_q.tolist()
        for b, L in enumerate(case.cache_seqlens.tolist()):
            S = cu[b + 1] - cu[b]
            n = _mask_count(S, L, causal, win).sum(dim=1).numpy().astype(np.float64)
            exp = np.where(n > 0, np.log(np.maximum(n, 1.0)), -np.inf)
            for h in range(case.num_heads):
                _same_lse(lse[cu[b]:cu[b + 1], h], exp, 1e-12)


def pin_lse_single_key(oa, ob, osc):
    """Window (0, 0): one visible key, so the log-sum-exp is that key's own score."""
    case = small_case(seed=21, window_size=(0, 0))
    _, lse = oa(**case.kwargs(), return_lse=True)
    cu = case.cu_seqlens_q.tolist()
    G = case.num_heads // case.num_kv_heads
    for b, L in enumerate(case.cache_seqlens.tolist()):
        S = cu[b + 1] - cu[b]
        for i in range(S):
            t, p = cu[b] + i, i + L - S
            page = int(case.block_table[b, p // case.block_size])
            for h in range(case.num_heads):
                k = case.key_cache[page, p % case.block_size, h // G].double()
                s = case.softmax_scale * float(torch.dot(case.q[t, h].double(), k)) + \
                    float(case.rel_logits[t, h, 0])
                assert abs(lse[t, h] - s) <= 1e-12, (t, h, lse[t, h], s)


def pin_lse_logsumexp(oa, ob, osc):
    """torch.logsumexp (a library reduction) over the fp64 masked score matrix built with torch ops."""
    for causal, win in ((True, (-1, -1)), (False, (2, 3)), (True, (4, 0))):
        case = small_case(seed=22, rel_extent=6, causal=causal, window_size=win, rel_std=3.0,
                          query_lens=[3, 1, 6, 2], kv_lens=[9, 13, 6, 2])
        case.cache_seqlens[3] = 1  # two queries over one key: the first sits at p = -1
        _, lse = oa(**case.kwargs(), return_lse=True)
        cu = case.cu_seqlens_q.tolist()
        G = case.num_heads // case.num_kv_heads
        E = case.rel_extent
        for b, L in enumerate(case.cache_seqlens.tolist()):
            S = cu[b + 1] - cu[b]
            bs = case.block_size
            pages = case.block_table[b, : (L + bs - 1) // bs].long()
            K = case.key_cache[pages].reshape(-1, case.num_kv_heads, case.head_dim)[:L].double()
            Q = case.q[cu[b]: cu[b + 1]].double()
            dist = (torch.arange(S)[:, None] + (L - S)) - torch.arange(L)[None, :]
            mask = _mask_count(S, L, causal, win)
            for h in range(case.num_heads):
                sc = case.softmax_scale * (Q[:, h, :] @ K[:, h // G, :].T)
                R = case.rel_logits[cu[b]: cu[b + 1], h, :].double()
                inr = (dist >= 0) & (dist < E)
                bias = torch.gather(R, 1, dist.clamp(0, E - 1)) * inr
                sc = torch.where(mask, sc + bias, torch.tensor(float("-inf"), dtype=torch.float64))
                exp = torch.logsumexp(sc, dim=1).numpy()
                _same_lse(lse[cu[b]:cu[b + 1], h], exp, 1e-12)


ALL_PINS = [pin_golden, pin_sdpa_no_bias, pin_top_left_causal, pin_one_hot_bias,
            pin_single_visible_key, pin_gqa_expansion, pin_page_permutation, pin_constant_bias,
            pin_extent_endpoint, pin_split_combine, pin_request_order, pin_lse_golden,
            pin_lse_uniform, pin_lse_single_key, pin_lse_logsumexp, pin_bruteforce]

# Pins that do not compare two forms of the oracle with each other
INDEPENDENT_PINS = [p for p in ALL_PINS if p is not pin_bruteforce]


def run_pin(pin, mod):
    pin(mod.oracle_attention, mod.oracle_bruteforce, mod.oracle_split_combine)
