"""Algorithmic work of one call: the bytes the method must move and the flops
it must do, counting only what the definition touches.

* K/V bytes: every key that some query row of the request may see, once per
  KV head, for K and for V (``2 * Hkv * D * elem`` bytes per key).
* bias bytes: every ``rel_logits`` entry whose distance ``d = p - j`` is in
  ``[0, rel_extent)`` for a visible key (each entry is read at most once).
* q and out: read and written once.
* block table: one int32 per page holding a visible key; cu_seqlens_q and
  cache_seqlens: read once.
* flops: ``4 * head_dim`` per visible (query head, key) pair (2 for q.k and 2
  for p.v).

Masked pairs, padding, split-KV partials and re-reads are not counted, so
these figures are lower bounds for any implementation.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class Work:
    kv_bytes: int
    bias_bytes: int
    qo_bytes: int
    meta_bytes: int
    pairs: int          # visible (query head, key) pairs
    flops: int

    @property
    def bytes(self) -> int:
        return self.kv_bytes + self.bias_bytes + self.qo_bytes + self.meta_bytes


def _ranges(p: np.ndarray, L: int, causal: bool, window_size) -> tuple:
    wl, wr = window_size
    lo = np.zeros_like(p)
    hi = np.full_like(p, L)
    if causal:
        hi = np.minimum(hi, p + 1)
    if wl >= 0:
        lo = np.maximum(lo, p - wl)
    if wr >= 0:
        hi = np.minimum(hi, p + wr + 1)
    hi = np.maximum(hi, lo)
    return lo, hi


def count_work(*, query_lens, kv_lens, num_heads: int, num_kv_heads: int, head_dim: int,
               block_size: int, rel_extent: int, causal: bool, window_size, elem_bytes: int) -> Work:
    H, Hkv, D, E, bs = num_heads, num_kv_heads, head_dim, rel_extent, block_size
    kv = bias = pairs = meta = 0
    T = 0
    for S, L in zip(query_lens, kv_lens):
        S, L = int(S), int(L)
        T += S
        meta += 8  # cu_seqlens_q entry + cache_seqlens entry
        if S == 0:
            continue
        p = np.arange(S, dtype=np.int64) + (L - S)
        lo, hi = _ranges(p, L, causal, window_size)
        n = hi - lo
        pairs += int(n.sum()) * H
        if n.sum() == 0:
            continue
        klo, khi = int(lo[n > 0].min()), int(hi[n > 0].max())
        kv += (khi - klo) * 2 * Hkv * D * elem_bytes
        meta += ((khi - 1) // bs - klo // bs + 1) * 4
        if E > 0:
            # visible keys with 0 <= p - j < E  <=>  j in [max(lo, p-E+1), min(hi, p+1))
            blo = np.maximum(lo, p - E + 1)
            bhi = np.minimum(hi, p + 1)
            bias += int(np.maximum(bhi - blo, 0).sum()) * H * elem_bytes
    qo = 2 * T * H * D * elem_bytes
    return Work(kv_bytes=kv, bias_bytes=bias, qo_bytes=qo, meta_bytes=meta + 4, pairs=pairs,
                flops=4 * D * pairs)


def case_work(case) -> Work:
    return count_work(query_lens=case.query_lens(), kv_lens=case.kv_lens(), num_heads=case.num_heads,
                      num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                      block_size=case.block_size, rel_extent=case.rel_extent, causal=case.causal,
                      window_size=case.window_size, elem_bytes=case.q.element_size())
