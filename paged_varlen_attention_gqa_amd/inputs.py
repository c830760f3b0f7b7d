"""Seeded synthetic workloads for paged, variable-length GQA attention with a
per-token relative-position bias.

This module only draws random numbers and lays them out in the shapes the
operation takes; it holds none of the attention arithmetic. Both the fp64
oracle (tests) and the HIP path (tests, bench) are fed from it.

Shapes follow the op's documented signature (docs.vllm.ai API page for
``vllm.models.inkling.nvidia.ops.fa4_rel_attention``, function
``inkling_fa4_rel_attention``, its docstring):

* ``q``            ``(num_tokens, num_heads, head_dim)``
* ``key_cache``    ``(num_blocks, block_size, num_kv_heads, head_dim)``
* ``value_cache``  same as ``key_cache``
* ``block_table``  ``(batch, max_blocks_per_seq)`` int32 page ids
* ``cache_seqlens`` ``(batch,)`` int32 KV length per request
* ``cu_seqlens_q`` ``(batch + 1,)`` int32 prefix sums of query lengths
* ``rel_logits``   ``(num_tokens, num_heads, rel_extent)``

Recipe (every tensor has its own named random stream, so adding or resizing
one tensor never changes another):

* Random numbers come from NumPy's PCG64, one generator per
  ``(seed, stream, sub, chunk)`` built with ``SeedSequence``. Normal values
  are drawn in chunks of ``2**20`` float32 values, so the result does not
  depend on how many threads draw them.
* Normal values are drawn as float32 ``standard_normal * std`` and rounded
  once, round-to-nearest-even, to bf16 (kept float32 for fp32 workloads).
* Queries of request ``b`` are the last ``S_b`` of its ``L_b`` tokens.
* Logical K and V of request ``b`` are drawn as ``(L_b, num_kv_heads,
  head_dim)`` and scattered to the request's pages in ``block_table`` order.
  Pool slots that no request uses, and the slots of a request's last page at
  positions ``>= L_b``, hold NaN; unused ``block_table`` entries point at
  page 0 (they are never read).
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

CHUNK = 1 << 20

# stream ids
_S_LENGTHS = 1
_S_PAGES = 2
_S_Q = 3
_S_K = 4
_S_V = 5
_S_REL = 6

_POOL = ThreadPoolExecutor(max_workers=8)


def _gen(seed: int, stream: int, sub: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, sub, chunk])))


def normal_f32(n: int, seed: int, stream: int, sub: int = 0, std: float = 1.0) -> np.ndarray:
    """``n`` float32 values ~ N(0, std^2), drawn chunk by chunk (thread-count independent)."""
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(c: int) -> None:
        s = c * CHUNK
        e = min(n, s + CHUNK)
        _gen(seed, stream, sub, c).standard_normal(e - s, dtype=np.float32, out=out[s:e])
        if std != 1.0:
            out[s:e] *= np.float32(std)

    list(_POOL.map(work, range(nchunks)))
    return out


def normal_tensor(shape, dtype: torch.dtype, seed: int, stream: int, sub: int = 0,
                  std: float = 1.0) -> torch.Tensor:
    n = int(np.prod(shape)) if len(shape) else 1
    x = torch.from_numpy(normal_f32(n, seed, stream, sub, std)).reshape(shape)
    return x if dtype == torch.float32 else x.to(dtype)  # RNE cast


@dataclass
class AttnCase:
    """One call's worth of inputs (host tensors) plus its scalar arguments."""

    name: str
    q: torch.Tensor
    key_cache: torch.Tensor
    value_cache: torch.Tensor
    block_table: torch.Tensor
    cache_seqlens: torch.Tensor
    cu_seqlens_q: torch.Tensor
    rel_logits: torch.Tensor
    max_seqlen_q: int
    softmax_scale: float
    causal: bool
    window_size: tuple
    rel_extent: int
    meta: dict = field(default_factory=dict)

    @property
    def dtype(self) -> torch.dtype:
        return self.q.dtype

    @property
    def num_tokens(self) -> int:
        return self.q.shape[0]

    @property
    def num_heads(self) -> int:
        return self.q.shape[1]

    @property
    def head_dim(self) -> int:
        return self.q.shape[2]

    @property
    def num_kv_heads(self) -> int:
        return self.key_cache.shape[2]

    @property
    def block_size(self) -> int:
        return self.key_cache.shape[1]

    @property
    def batch_size(self) -> int:
        return self.cache_seqlens.shape[0]

    def query_lens(self) -> list:
        cu = self.cu_seqlens_q.tolist()
        return [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]

    def kv_lens(self) -> list:
        return self.cache_seqlens.tolist()

    def kwargs(self) -> dict:
        """Keyword arguments shared by the oracle and the binding."""
        return dict(
            q=self.q, key_cache=self.key_cache, value_cache=self.value_cache,
            block_table=self.block_table, cache_seqlens=self.cache_seqlens,
            cu_seqlens_q=self.cu_seqlens_q, max_seqlen_q=self.max_seqlen_q,
            softmax_scale=self.softmax_scale, causal=self.causal,
            window_size=self.window_size, rel_extent=self.rel_extent,
            rel_logits=self.rel_logits,
        )


def make_case(*, name: str = "custom", query_lens, kv_lens, num_heads: int, num_kv_heads: int,
              head_dim: int, block_size: int, rel_extent: int, causal: bool = True,
              window_size=(-1, -1), softmax_scale: float | None = None,
              dtype: torch.dtype = torch.bfloat16, seed: int = 0, pool_pages: int | None = None,
              qkv_std: float = 1.0, rel_std: float = 1.0, max_blocks_per_seq: int | None = None,
              nan_fill: bool = True, max_seqlen_q: int | None = None) -> AttnCase:
    """Build a seeded case. ``query_lens[b] <= kv_lens[b]`` (queries are the last tokens).

    ``pool_pages``: number of physical pages; default = exactly the pages needed.
    Pages are a random sample without replacement from the pool, in random order.
    """
    query_lens = [int(x) for x in query_lens]
    kv_lens = [int(x) for x in kv_lens]
    B = len(kv_lens)
    assert len(query_lens) == B
    for s, l in zip(query_lens, kv_lens):
        assert 0 <= s <= l, (s, l)
    assert num_heads % num_kv_heads == 0
    bs = block_size
    pages_per = [(l + bs - 1) // bs for l in kv_lens]
    need = sum(pages_per)
    pool = need if pool_pages is None else int(pool_pages)
    assert pool >= need and pool >= 1
    mb = max(1, max(pages_per) if pages_per else 1)
    if max_blocks_per_seq is not None:
        assert max_blocks_per_seq >= mb
        mb = max_blocks_per_seq
    T = sum(query_lens)
    H, Hkv, D, E = num_heads, num_kv_heads, head_dim, rel_extent

    # page permutation: a random sample of `need` distinct pages of the pool, in random order
    perm = _gen(seed, _S_PAGES, 0, 0).permutation(pool)[:need].astype(np.int64)
    block_table = torch.zeros((B, mb), dtype=torch.int32)
    off = 0
    for b in range(B):
        block_table[b, : pages_per[b]] = torch.from_numpy(perm[off: off + pages_per[b]].astype(np.int32))
        off += pages_per[b]

    q = normal_tensor((T, H, D), dtype, seed, _S_Q, 0, qkv_std)

    fill = float("nan") if nan_fill else 0.0
    key_cache = torch.full((pool, bs, Hkv, D), fill, dtype=dtype)
    value_cache = torch.full((pool, bs, Hkv, D), fill, dtype=dtype)
    for b in range(B):
        L = kv_lens[b]
        if L == 0:
            continue
        pages = block_table[b, : pages_per[b]].long()
        for cache, stream in ((key_cache, _S_K), (value_cache, _S_V)):
            x = normal_tensor((L, Hkv, D), dtype, seed, stream, b, qkv_std)
            padded = torch.full((pages_per[b] * bs, Hkv, D), fill, dtype=dtype)
            padded[:L] = x
            cache[pages] = padded.reshape(pages_per[b], bs, Hkv, D)

    rel_logits = normal_tensor((T, H, E), dtype, seed, _S_REL, 0, rel_std)

    cu = [0]
    for s in query_lens:
        cu.append(cu[-1] + s)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if max_seqlen_q is None:
        max_seqlen_q = max(query_lens) if query_lens else 0
    return AttnCase(
        name=name, q=q, key_cache=key_cache, value_cache=value_cache, block_table=block_table,
        cache_seqlens=torch.tensor(kv_lens, dtype=torch.int32),
        cu_seqlens_q=torch.tensor(cu, dtype=torch.int32), rel_logits=rel_logits,
        max_seqlen_q=int(max_seqlen_q), softmax_scale=float(softmax_scale), causal=bool(causal),
        window_size=tuple(int(w) for w in window_size), rel_extent=int(E),
        meta=dict(seed=seed, pool_pages=pool, qkv_std=qkv_std, rel_std=rel_std),
    )


def _uniform_ints(n: int, lo: int, hi: int, seed: int, sub: int = 0) -> list:
    """``n`` integers uniform on the inclusive range [lo, hi]."""
    return [int(x) for x in _gen(seed, _S_LENGTHS, sub, 0).integers(lo, hi + 1, size=n)]


# The five named workloads. Sizes are the ones the workloads are quoted at; the
# `scale` argument shrinks them for quick parity runs (documented per config).
CONFIG_NAMES = ("tiny_fp32", "decode_b64", "prefill_chunked", "mixed_window", "decode_long_b1",
                "decode_1m_b1_kv4", "decode_1m_b1_kv8")


def config_spec(name: str, scale: float = 1.0, seed: int = 0) -> dict:
    """Arguments for :func:`make_case` for a named workload.

    ``scale < 1`` shrinks KV/query lengths (and pools) proportionally for quick
    parity runs while keeping head counts, head_dim, block_size and masks.
    """
    def sc(x: int, lo: int = 1) -> int:
        return max(lo, int(round(x * scale)))

    if name == "tiny_fp32":
        return dict(name=name, query_lens=[5, 17], kv_lens=[37, 70], num_heads=4, num_kv_heads=2,
                    head_dim=64, block_size=16, rel_extent=32, causal=True, window_size=(-1, -1),
                    softmax_scale=1.0 / math.sqrt(64), dtype=torch.float32, seed=seed, pool_pages=8)
    if name == "decode_b64":
        lens = _uniform_ints(64, sc(1024), sc(8192), seed)
        return dict(name=name, query_lens=[1] * 64, kv_lens=lens, num_heads=32, num_kv_heads=8,
                    head_dim=128, block_size=16, rel_extent=1024, causal=True, window_size=(-1, -1),
                    softmax_scale=1.0 / math.sqrt(128), dtype=torch.bfloat16, seed=seed,
                    pool_pages=max(sc(40000), sum((l + 15) // 16 for l in lens)))
    if name == "prefill_chunked":
        S = sc(2048, 16)
        prior = [0, sc(1024, 0), sc(2048, 0), sc(4096, 0)]
        return dict(name=name, query_lens=[S] * 4, kv_lens=[S + p for p in prior], num_heads=64,
                    num_kv_heads=8, head_dim=128, block_size=16, rel_extent=sc(4096), causal=True,
                    window_size=(-1, -1), softmax_scale=1.0 / math.sqrt(128), dtype=torch.bfloat16,
                    seed=seed, rel_std=0.5)
    if name == "mixed_window":
        dec = _uniform_ints(56, sc(2048), sc(32768), seed)
        S, Lp = sc(512, 2), sc(4096, 2)
        win = sc(4096) - 1
        return dict(name=name, query_lens=[S] * 8 + [1] * 56, kv_lens=[Lp] * 8 + dec, num_heads=32,
                    num_kv_heads=4, head_dim=128, block_size=16, rel_extent=sc(2048), causal=True,
                    window_size=(win, 0), softmax_scale=1.0 / math.sqrt(128), dtype=torch.bfloat16,
                    seed=seed)
    if name == "decode_long_b1":
        L = sc(262144, 64)
        return dict(name=name, query_lens=[1], kv_lens=[L], num_heads=32, num_kv_heads=4,
                    head_dim=128, block_size=64, rel_extent=sc(8192), causal=True,
                    window_size=(-1, -1), softmax_scale=1.0 / math.sqrt(128), dtype=torch.bfloat16,
                    seed=seed, pool_pages=max(sc(4096), (L + 63) // 64))
    if name in ("decode_1m_b1_kv4", "decode_1m_b1_kv8"):
        # batch-1 decode over a million keys, with 4 or 8 KV heads (the page
        # quotes its split caps per KV-head count and measures to 1M tokens)
        L = sc(1 << 20, 64)
        return dict(name=name, query_lens=[1], kv_lens=[L], num_heads=32,
                    num_kv_heads=4 if name.endswith("kv4") else 8, head_dim=128, block_size=64,
                    rel_extent=sc(8192), causal=True, window_size=(-1, -1),
                    softmax_scale=1.0 / math.sqrt(128), dtype=torch.bfloat16, seed=seed,
                    pool_pages=(L + 63) // 64)
    raise KeyError(name)


def make_config(name: str, scale: float = 1.0, seed: int = 0) -> AttnCase:
    return make_case(**config_spec(name, scale, seed))
