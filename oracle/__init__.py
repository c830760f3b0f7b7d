"""fp64 CPU oracle for paged, variable-length GQA attention with a per-token
relative-position bias.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP library and imports
nothing from it.

What it computes is written out from the pages:

* docs.vllm.ai API page for ``vllm.models.inkling.nvidia.ops.fa4_rel_attention``,
  ``inkling_fa4_rel_attention`` (signature and docstring): tensor shapes, the
  paged cache reached through ``block_table`` and ``cache_seqlens``, the
  packed queries described by ``cu_seqlens_q``, ``softmax_scale``, ``causal``,
  ``window_size`` with ``(-1, -1)`` meaning no window.
* prhub.com.cn report on vLLM PR #48858, section "key source snippets",
  the ``score_mod_rel_bias`` device function: the query's absolute position is
  its index plus ``seqlen_k - seqlen_q``; the distance ``d`` is that position
  minus the key index; the bias row is the packed (global) token row and the
  query head; the bias is the stored value when ``d`` lies in
  ``[0, rel_extent)`` and zero otherwise; it is added to the scaled score.

Readings where the pages are silent (each is pinned by a test):
GQA maps query head ``h`` to KV head ``h // (num_heads // num_kv_heads)``;
windows are inclusive ``[p - left, p + right]``; a query with no visible key
outputs zeros.

Every function here has at least one pin in ``tests/test_oracle_pins.py``; none
is "parity unpinned". The log-sum-exp that ``oracle_attention(..., return_lse=True)``
returns is pinned by hand-derived values (``tests/golden/hand_cases.json``),
``ln n`` for ``n`` equal scores, a single visible key's own score, and
``torch.logsumexp`` over the masked fp64 score matrix.
"""

from .attention import (  # noqa: F401
    oracle_attention,
    oracle_bruteforce,
    oracle_split_combine,
    visible_keys,
)
