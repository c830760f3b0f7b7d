"""Helpers for GPU parity tests: move a seeded case to the device, call the HIP
library through its binding, compare with the fp64 oracle at the stated
tolerances."""

from __future__ import annotations

import sys

import numpy as np
import torch

# bf16 workloads: max-abs <= 2e-2 and mean-abs <= 2e-3 against the fp64 oracle;
# fp32 workloads: max-abs <= 1e-4.
TOL = {torch.bfloat16: (2e-2, 2e-3), torch.float32: (1e-4, 1e-4)}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def device_case(case, device="cuda:0"):
    """Device copies of every tensor argument (same keyword names as the oracle)."""
    kw = case.kwargs()
    out = {}
    for k, v in kw.items():
        out[k] = v.to(device) if isinstance(v, torch.Tensor) else v
    return out


def run_gpu(case, device="cuda:0", **over):
    from paged_varlen_attention_gqa_amd import rel_attn_fwd

    kw = device_case(case, device)
    kw.update(over)
    out = rel_attn_fwd(**kw)
    torch.cuda.synchronize()
    return out


def compare(got: torch.Tensor, ref: np.ndarray, dtype, tokens=None, what=""):
    """Element-wise comparison on the selected token rows; returns (max_abs, mean_abs)."""
    g = got.detach().cpu().to(torch.float64).numpy()
    if tokens is not None:
        idx = np.asarray(sorted(tokens), dtype=np.int64)
        g = g[idx]
        ref = ref[idx]
    assert np.isfinite(g).all(), f"{what}: non-finite values in the HIP output"
    err = np.abs(g - ref)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    tmax, tmean = TOL[dtype]
    log(f"  {what}: max_abs={mx:.3e} mean_abs={mean:.3e} (tol {tmax:g}/{tmean:g})")
    assert mx <= tmax, f"{what}: max-abs {mx} > {tmax}"
    assert mean <= tmean, f"{what}: mean-abs {mean} > {tmean}"
    return mx, mean
