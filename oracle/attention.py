"""fp64 reference implementations (test infrastructure only; see the package docstring).

Notation (shared with the pages' ``score_mod_rel_bias`` snippet, prhub.com.cn
report on vLLM PR #48858, "key source snippets"):

* request ``b`` owns packed query rows ``cu_seqlens_q[b] .. cu_seqlens_q[b+1]``
  (``S_b`` of them) and ``L_b = cache_seqlens[b]`` cached keys;
* query ``i`` of request ``b`` sits at absolute position ``p = i + L_b - S_b``
  (``seqlen_k - seqlen_q`` offset of the snippet);
* its global row is ``t = cu_seqlens_q[b] + i`` (``offset_q + q_idx``);
* for key ``j`` the distance is ``d = p - j`` (``rel_dist``);
* the bias is ``rel_logits[t, h, d]`` when ``0 <= d < rel_extent``, else 0,
  and the score is ``softmax_scale * <q, k> + bias``;
* logical key ``j`` of request ``b`` lives at
  ``cache[block_table[b, j // block_size], j % block_size]`` (paged cache of
  the docs.vllm.ai ``inkling_fa4_rel_attention`` signature).
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = float("-inf")


def _f64(x) -> np.ndarray:
    """Exact upcast of a host tensor (fp32 or bf16) or array to float64."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().cpu().to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _ints(x) -> np.ndarray:
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().cpu().to(torch.int64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.int64)


def visible_keys(p: int, L: int, causal: bool, window_size) -> tuple:
    """Half-open range ``[lo, hi)`` of keys query position ``p`` may attend to.

    Keys exist for ``0 <= j < L``. Causal keeps ``j <= p`` (queries are the last
    tokens of the sequence, so the causal diagonal is bottom-right aligned).
    A window ``(left, right)`` keeps ``p - left <= j <= p + right``; a negative
    side is unbounded, so ``(-1, -1)`` is no window (docs.vllm.ai
    ``inkling_fa4_rel_attention``: ``(-1, -1)`` is mapped to "no window").
    Every constraint is an interval, so the visible set is one interval.
    """
    wl, wr = window_size
    lo, hi = 0, L
    if causal:
        hi = min(hi, p + 1)
    if wl >= 0:
        lo = max(lo, p - wl)
    if wr >= 0:
        hi = min(hi, p + wr + 1)
    return lo, max(lo, hi)


def _requests(cu_seqlens_q, cache_seqlens):
    cu = _ints(cu_seqlens_q)
    Ls = _ints(cache_seqlens)
    for b in range(len(Ls)):
        t0 = int(cu[b])
        S = int(cu[b + 1] - cu[b])
        L = int(Ls[b])
        yield b, t0, S, L


def _logical_kv(cache: np.ndarray, block_table: np.ndarray, b: int, L: int) -> np.ndarray:
    """Logical ``(L, num_kv_heads, head_dim)`` rows of request ``b`` gathered through its pages."""
    bs = cache.shape[1]
    npages = (L + bs - 1) // bs
    pages = block_table[b, :npages]
    return cache[pages].reshape(npages * bs, cache.shape[2], cache.shape[3])[:L]


def _scores(qh, K, R, p, L, softmax_scale, causal, window_size, rel_extent):
    """Masked scores ``(rows, L)`` for one query head: scale*q.k + bias, -inf where not visible.

    ``qh``: (rows, D) queries; ``K``: (L, D) logical keys of the head's KV head;
    ``R``: (rows, rel_extent) bias rows; ``p``: (rows,) absolute positions.
    """
    j = np.arange(L)
    s = softmax_scale * (qh @ K.T)
    if rel_extent > 0:
        d = p[:, None] - j[None, :]
        in_range = (d >= 0) & (d < rel_extent)
        bias = np.take_along_axis(R, np.clip(d, 0, rel_extent - 1), axis=1)
        s = s + np.where(in_range, bias, 0.0)
    vis = np.zeros((len(p), L), dtype=bool)
    for r, pr in enumerate(p):
        lo, hi = visible_keys(int(pr), L, causal, window_size)
        vis[r, lo:hi] = True
    return np.where(vis, s, NEG_INF), vis


def oracle_attention(q, key_cache, value_cache, *, block_table, cache_seqlens, cu_seqlens_q,
                     max_seqlen_q, softmax_scale, causal, window_size, rel_extent, rel_logits,
                     tokens=None, return_lse=False):
    """Plain definition, evaluated in float64, vectorised per (request, query head).

    out[t, h] = sum_j e^{s_j - m} V_j / sum_j e^{s_j - m} over the visible keys
    j, with s_j = softmax_scale * <q[t,h], K_j> + bias_j and m = max_j s_j; zero
    when no key is visible. ``tokens`` (optional iterable of packed row
    indices) restricts the work to those rows; other rows of the result are
    NaN. ``max_seqlen_q`` is a scheduling bound only and does not change the
    result. Returns ``out`` (T, H, D) float64, and ``lse`` (T, H) (the natural
    log of the softmax denominator including the max, -inf when empty) when
    ``return_lse``.
    """
    del max_seqlen_q
    bt = _ints(block_table)
    T, H, D = q.shape
    Hkv = key_cache.shape[2]
    G = H // Hkv
    out = np.full((T, H, D), np.nan)
    lse = np.full((T, H), np.nan)
    want = None if tokens is None else np.zeros(T, dtype=bool)
    if want is not None:
        want[np.asarray(list(tokens), dtype=np.int64)] = True
    E = int(rel_extent)
    for b, t0, S, L in _requests(cu_seqlens_q, cache_seqlens):
        rows = np.arange(S)
        if want is not None:
            rows = rows[want[t0:t0 + S]]
        if len(rows) == 0:
            continue
        p = rows + (L - S)
        Kb = _f64(_logical_kv(key_cache, bt, b, L)) if L > 0 else np.zeros((0, Hkv, D))
        Vb = _f64(_logical_kv(value_cache, bt, b, L)) if L > 0 else np.zeros((0, Hkv, D))
        for h in range(H):
            g = h // G
            qh = _f64(q[t0 + rows, h, :])
            R = _f64(rel_logits[t0 + rows, h, :]) if E > 0 else None
            s, vis = _scores(qh, Kb[:, g, :], R, p, L, softmax_scale, causal, window_size, E)
            has = vis.any(axis=1)
            m = np.where(has, np.max(s, axis=1, initial=NEG_INF), 0.0)
            w = np.where(vis, np.exp(s - m[:, None]), 0.0)
            l = w.sum(axis=1)
            o = np.zeros((len(rows), D))
            o[has] = (w[has] @ Vb[:, g, :]) / l[has, None]
            out[t0 + rows, h, :] = o
            lse[t0 + rows, h] = np.where(has, m + np.log(np.where(has, l, 1.0)), NEG_INF)
    return (out, lse) if return_lse else out


def oracle_split_combine(q, key_cache, value_cache, *, block_table, cache_seqlens, cu_seqlens_q,
                         max_seqlen_q, softmax_scale, causal, window_size, rel_extent, rel_logits,
                         num_splits):
    """Split-KV form of the same result (the ``num_splits`` argument of the pages' API).

    Each query's visible keys are cut into ``num_splits`` contiguous chunks of
    near-equal size. Per chunk ``k``: the normalised partial output
    ``o_k = sum e^{s-m_k} V / l_k`` and ``lse_k = m_k + ln l_k`` (-inf and zero
    output for an empty chunk). They are merged with
    ``LSE = ln sum_k e^{lse_k}`` and ``out = sum_k e^{lse_k - LSE} o_k``.
    """
    del max_seqlen_q
    bt = _ints(block_table)
    T, H, D = q.shape
    Hkv = key_cache.shape[2]
    G = H // Hkv
    E = int(rel_extent)
    out = np.zeros((T, H, D))
    for b, t0, S, L in _requests(cu_seqlens_q, cache_seqlens):
        if S == 0:
            continue
        rows = np.arange(S)
        p = rows + (L - S)
        Kb = _f64(_logical_kv(key_cache, bt, b, L)) if L > 0 else np.zeros((0, Hkv, D))
        Vb = _f64(_logical_kv(value_cache, bt, b, L)) if L > 0 else np.zeros((0, Hkv, D))
        for h in range(H):
            g = h // G
            R = _f64(rel_logits[t0 + rows, h, :]) if E > 0 else None
            s, vis = _scores(_f64(q[t0 + rows, h, :]), Kb[:, g, :], R, p, L, softmax_scale,
                             causal, window_size, E)
            for r in range(S):
                keys = np.nonzero(vis[r])[0]
                lses, parts = [], []
                for chunk in np.array_split(keys, num_splits):
                    if len(chunk) == 0:
                        lses.append(NEG_INF)
                        parts.append(np.zeros(D))
                        continue
                    m_k = s[r, chunk].max()
                    w = np.exp(s[r, chunk] - m_k)
                    l_k = w.sum()
                    parts.append((w @ Vb[chunk, g, :]) / l_k)
                    lses.append(m_k + math.log(l_k))
                lses = np.asarray(lses)
                if np.all(np.isneginf(lses)):
                    continue
                mx = lses.max()
                LSE = mx + math.log(np.exp(lses - mx).sum())
                out[t0 + r, h, :] = sum(math.exp(lk - LSE) * pk for lk, pk in zip(lses, parts))
    return out


def oracle_bruteforce(q, key_cache, value_cache, *, block_table, cache_seqlens, cu_seqlens_q,
                      max_seqlen_q, softmax_scale, causal, window_size, rel_extent, rel_logits):
    """Scalar loops over every (token, head, key); tiny inputs only.

    Written independently of :func:`oracle_attention`: each key is fetched
    through its page, each mask condition is tested per key, and the bias of
    key ``j`` is the entry at distance ``d = p - j`` of the query's
    ``rel_logits`` row when ``0 <= d < rel_extent``, else 0.
    """
    del max_seqlen_q
    bt = _ints(block_table).tolist()
    cu = _ints(cu_seqlens_q).tolist()
    Ls = _ints(cache_seqlens).tolist()
    qv = _f64(q)
    kc = _f64(key_cache)
    vc = _f64(value_cache)
    rl = _f64(rel_logits) if rel_extent > 0 else None
    T, H, D = qv.shape
    Hkv = kc.shape[2]
    bs = kc.shape[1]
    wl, wr = window_size
    out = np.zeros((T, H, D))
    for b in range(len(Ls)):
        S = cu[b + 1] - cu[b]
        L = Ls[b]
        for i in range(S):
            t = cu[b] + i
            p = i + L - S
            for h in range(H):
                g = h // (H // Hkv)
                scores, vrows = [], []
                for j in range(L):
                    if causal and j > p:
                        continue
                    if wl >= 0 and j < p - wl:
                        continue
                    if wr >= 0 and j > p + wr:
                        continue
                    page = bt[b][j // bs]
                    slot = j % bs
                    dot = 0.0
                    for e in range(D):
                        dot += qv[t, h, e] * kc[page, slot, g, e]
                    # the distance of key j behind the query; only
                    # distances 0 .. rel_extent-1 have a bias entry
                    d = p - j
                    bias = rl[t, h, d] if 0 <= d < rel_extent else 0.0
                    scores.append(softmax_scale * dot + bias)
                    vrows.append(vc[page, slot, g, :])
                if not scores:
                    continue
                m = max(scores)
                ws = [math.exp(s - m) for s in scores]
                den = sum(ws)
                acc = np.zeros(D)
                for w_, v in zip(ws, vrows):
                    acc += w_ * v
                out[t, h, :] = acc / den
    return out
