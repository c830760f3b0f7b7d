"""Paged, variable-length GQA attention with a per-token relative-position bias
for AMD Instinct MI355X (gfx950).

The compute path is librelattn.so (hand-written HIP kernels behind a C ABI,
include/rel_attn.h); ``relattn`` is its ctypes binding. ``inputs`` draws
seeded synthetic workloads; ``work`` counts the algorithmic bytes and flops
of a call.
"""

from .relattn import (  # noqa: F401
    RelAttnError,
    load_library,
    rel_attn_combine,
    rel_attn_fwd,
    rel_attn_fwd_noalloc,
    rel_attn_fwd_splits,
    rel_attn_noalloc_scratch_bytes,
    rel_attn_num_splits,
    rel_attn_strerror,
    rel_attn_workspace_bytes,
    split_partials,
)
