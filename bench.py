"""Benchmark: paged varlen GQA attention with the per-token relative bias on one MI355X.

A step is one attention call over one batch of synthetic, seeded input that
is resident in HBM before timing starts: ``rel_attn_fwd_splits`` (the
attention kernels) followed, when the call splits the key range, by
``rel_attn_combine`` -- together exactly what ``rel_attn_fwd`` launches.
Default workload: batched decode, 64 requests x 1 query token, KV lengths
uniform in [1024, 8192], 32 query / 8 KV heads, head_dim 128, block_size 16,
rel_extent 1024, bf16.

Prints ONE JSON line. ``value`` is the algorithmic bytes of a step (K/V rows
of visible keys, in-range bias, q, out, page-table entries) divided by the
wall-clock step time. ``roofline`` divides the same algorithmic figure (or
the flops, for the compute-bound prefill workload) by the attention stage's
own average duration, from HIP events recorded around it on the stream its
kernels run on, and compares that with MI355X's published peak. Its
``traffic`` is the HBM-side bytes per launch measured by rocprofv3 counters
(FETCH_SIZE, WRITE_SIZE, scaled by the same counters' reading for a plain copy
of known size), read from the committed counter summary under profiles/ when
that summary was taken on the current kernel sources, else null.
``cpu_baseline`` times the fp64 CPU oracle on a bounded sample of the same
workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from paged_varlen_attention_gqa_amd import (rel_attn_combine, rel_attn_fwd_splits,  # noqa: E402
                                           rel_attn_num_splits, rel_attn_workspace_bytes)
from paged_varlen_attention_gqa_amd.inputs import config_spec, make_case  # noqa: E402
from paged_varlen_attention_gqa_amd.work import case_work  # noqa: E402

METRIC = "rel-bias paged attn: decode KV GB/s + prefill TFLOP/s, % of MI355X roofline"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP32_MFMA_PEAK_TFLOPS = 157.3

DESCRIPTIONS = {
    "decode_b64": "batched decode: 64 requests x 1 query, KV lens U[1024,8192], H=32 Hkv=8 D=128 "
                  "bs=16, 40000-page pool, causal, rel_extent=1024, bf16",
    "prefill_chunked": "chunked causal prefill: 4 requests x 2048 queries over prior context "
                       "0/1024/2048/4096, H=64 Hkv=8 D=128 bs=16, rel_extent=4096, bf16",
    "mixed_window": "mixed sliding-window batch: 8 prefills (512 queries over KV 4096) + 56 decodes "
                    "(KV U[2048,32768]), window (4095,0), H=32 Hkv=4 D=128 bs=16, rel_extent=2048, bf16",
    "decode_long_b1": "batch-1 long-context decode: 1 query over 262144 keys, H=32 Hkv=4 D=128 "
                      "bs=64, rel_extent=8192, bf16, split-KV + LSE combine",
    "decode_1m_b1_kv4": "batch-1 decode over 1048576 keys, H=32 Hkv=4 D=128 bs=64, rel_extent=8192, bf16, "
                        "split-KV + LSE combine",
    "decode_1m_b1_kv8": "batch-1 decode over 1048576 keys, H=32 Hkv=8 D=128 bs=64, rel_extent=8192, bf16, "
                        "split-KV + LSE combine",
    "tiny_fp32": "tiny fp32 correctness case: 2 requests, query lens 5/17, KV lens 37/70, H=4 Hkv=2 "
                 "D=64 bs=16, rel_extent=32",
}
# the bound of the stage's dominant kernel (mixed_window: the prefill kernel,
# about 80% of the stage)
BOUND = {"decode_b64": "hbm", "decode_long_b1": "hbm", "mixed_window": "mfma",
         "decode_1m_b1_kv4": "hbm", "decode_1m_b1_kv8": "hbm",
         "prefill_chunked": "mfma", "tiny_fp32": "hbm"}


# Kernel sources whose code decides the attention stage's memory traffic, per
# workload; a counter summary is valid only for the sources it was taken on.
CSRC = os.path.join(ROOT, "paged_varlen_attention_gqa_amd", "csrc")
STAGE_SOURCES = {
    "decode_b64": ["attn_decode.hip"],
    "decode_long_b1": ["attn_decode.hip"],
    "decode_1m_b1_kv4": ["attn_decode.hip"],
    "decode_1m_b1_kv8": ["attn_decode.hip"],
    "prefill_chunked": ["attn_decode.hip", "attn_prefill.hip"],
    "mixed_window": ["attn_decode.hip", "attn_prefill.hip"],
    "tiny_fp32": ["attn_general.hip"],
}
STAGE_KERNELS = {
    "decode_b64": "attn_decode_balanced_kernel",
    "decode_long_b1": "attn_decode_balanced_kernel",
    "decode_1m_b1_kv4": "attn_decode_balanced_kernel",
    "decode_1m_b1_kv8": "attn_decode_balanced_kernel",
    "prefill_chunked": "attn_decode_wg_split_kernel (no work: rows > 16) + attn_prefill_kernel",
    "mixed_window": "attn_decode_wg_split_kernel + attn_prefill_kernel",
    "tiny_fp32": "attn_general_kernel",
}
COPY_BYTES = 2 << 30  # the plain copy that calibrates the HBM counters


def sources_digest(name: str) -> str:
    h = hashlib.sha256()
    for f in STAGE_SOURCES[name] + ["device_common.h", "api.cpp"]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(name: str):
    """HBM bytes per launch of the attention stage from profiles/hbm_traffic_<name>.txt
    (``key: value`` lines), or None when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith((" ", "#")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256") != sources_digest(name):
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(case, name: str, budget_s: float = 20.0) -> dict:
    """Time the fp64 oracle on a bounded sample of the same workload (whole requests
    for decode workloads, a token sample otherwise); scaled to GB/s or TFLOP/s.
    The oracle runs on one thread (its BLAS pool limited to 1), so ``cores`` is 1."""
    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1):
        return _cpu_baseline(case, name, budget_s)


def _cpu_baseline(case, name: str, budget_s: float) -> dict:
    import oracle
    from paged_varlen_attention_gqa_amd.work import count_work

    cu = case.cu_seqlens_q.tolist()
    B = case.batch_size
    qlens, klens = case.query_lens(), case.kv_lens()
    order = list(range(B))
    done, t_total = [], 0.0
    elem = case.q.element_size()
    bound = BOUND[name]
    # passes over the requests until about 10 s of CPU time (a workload the
    # oracle finishes sooner is repeated, for a steadier figure), at most budget_s
    passes = 0
    while t_total < min(10.0, budget_s):
        passes += 1
        for b in order:
            toks = list(range(cu[b], cu[b + 1]))
            if bound == "mfma":  # a bounded token sample of this request
                toks = toks[-8:]
            if not toks:
                continue
            t0 = time.perf_counter()
            oracle.oracle_attention(**case.kwargs(), tokens=toks)
            t_total += time.perf_counter() - t0
            done.append((b, len(toks)))
            if t_total > budget_s:
                break
        if t_total > budget_s or not done:
            break
    w = count_work(query_lens=[n for _, n in done], kv_lens=[klens[b] for b, _ in done],
                   num_heads=case.num_heads, num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                   block_size=case.block_size, rel_extent=case.rel_extent, causal=case.causal,
                   window_size=case.window_size, elem_bytes=elem)
    cores = 1
    if bound == "mfma":
        value, unit = w.flops / t_total / 1e12, "TFLOP/s"
    else:
        value, unit = w.bytes / t_total / 1e9, "GB/s"
    ntok = sum(n for _, n in done)
    nreq = len(set(b for b, _ in done))
    return {"value": round(value, 6), "unit": unit, "cores": cores, "kind": "oracle",
            "sample": f"{nreq} of {B} requests ({ntok} query tokens over {passes} pass(es), the last 8 of "
                      f"each request for prefill), fp64 NumPy oracle, {t_total:.1f} s" if bound == "mfma" else
                      f"{nreq} of {B} requests ({ntok} query tokens over {passes} pass(es)), fp64 NumPy "
                      f"oracle, {t_total:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="decode_b64", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--num-splits", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="extra calls after the timed ones, each after a 1 GiB write that flushes the "
                         "L2 and the 256 MB last-level cache (reported as stage_us_cold_mean)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 2 GiB copy first (for HBM counter runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this path has no "
              f"multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(2)
    name = args.config
    dev = torch.device("cuda:0")
    _log(f"[bench] generating {name}")
    case = make_case(**config_spec(name))
    work = case_work(case)
    kw = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in case.kwargs().items()}
    wl, wr = case.window_size
    splits = args.num_splits or rel_attn_num_splits(
        is_local=(wl >= 0 or wr >= 0), batch_size=case.batch_size, max_query_len=case.max_seqlen_q,
        num_heads=case.num_heads, num_kv_heads=case.num_kv_heads, max_kv_len=max(case.kv_lens()))
    out = torch.empty_like(kw["q"])
    need = rel_attn_workspace_bytes(splits, case.num_tokens, case.num_heads, case.head_dim)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    if args.copy_calibration:
        # a plain copy of known size, for scaling the HBM counters of a
        # profiling run (2 GiB read + 2 GiB written, far beyond the caches)
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        _log(f"[bench] copy calibration: {COPY_BYTES} bytes read + written, 3 times")
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        rel_attn_fwd_splits(**kw, num_splits=splits, out=out, workspace=ws)
        if ev is not None:
            ev[1].record(stream)
        if splits > 1:
            rel_attn_combine(ws, out, splits)

    _log(f"[bench] warmup {args.warmup} (num_splits={splits})")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    _log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_ms = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
    ms_per_step = wall * 1e3 / args.steps
    # the same stage with no input left in the caches: a 1 GiB write before
    # each call (outside the events, not part of the timed steps)
    cold_ms = np.array([])
    if args.cold_steps > 0:
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        cevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.cold_steps)]
        for ev in cevs:
            scratch.fill_(0.0)
            step(ev)
        torch.cuda.synchronize()
        cold_ms = np.array([e0.elapsed_time(e1) for e0, e1 in cevs])
        del scratch
    gbs = work.bytes / (ms_per_step * 1e-3) / 1e9
    tflops = work.flops / (ms_per_step * 1e-3) / 1e12
    avg_call_s = float(stage_ms.mean()) * 1e-3
    traffic = measured_traffic(name)
    bound = BOUND[name]
    if bound == "mfma":
        peak = BF16_MFMA_PEAK_TFLOPS if case.dtype == torch.bfloat16 else FP32_MFMA_PEAK_TFLOPS
        ach = work.flops / avg_call_s / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 3), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "traffic": traffic}
        value, unit = tflops, "TFLOP/s"
    else:
        ach = work.bytes / avg_call_s / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic}
        value, unit = gbs, "GB/s"
    res = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if case.dtype == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": f"{name}: {DESCRIPTIONS[name]}", "num_splits": splits,
                   "algorithmic_bytes": work.bytes, "algorithmic_flops": work.flops,
                   "stage_kernels": STAGE_KERNELS[name],
                   "stage_us_mean": round(float(stage_ms.mean()) * 1e3, 2),
                   "stage_us_min": round(float(stage_ms.min()) * 1e3, 2),
                   "stage_us_cold_mean": round(float(cold_ms.mean()) * 1e3, 2) if cold_ms.size else None,
                   "tflops": round(tflops, 3), "gbs": round(gbs, 2)},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        _log("[bench] timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(case, name)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
