"""Benchmark: paged varlen GQA attention with the per-token relative bias on one MI355X.

A step is one ``rel_attn_fwd`` call over one batch of synthetic, seeded
input that is resident in HBM before timing starts: the attention kernels
and, when the call splits the key range, the combine kernel.

The metric has two halves, decode KV bandwidth and prefill TFLOP/s, and the
default run times both, each for exactly ``--steps`` steps:
  * the headline: batched decode, 64 requests x 1 query token, KV lengths
    uniform in [1024, 8192], 32 query / 8 KV heads, head_dim 128, block_size
    16, rel_extent 1024, bf16 (``value`` in GB/s);
  * chunked causal prefill, 4 requests x 2048 queries over prior context
    0/1024/2048/4096, 64 query / 8 KV heads, rel_extent 4096, bf16, reported
    under ``config.prefill`` (TFLOP/s, with its own roofline and CPU baseline).
``--config NAME`` times one workload alone.

Prints ONE JSON line. ``value`` is the algorithmic bytes of a step (K/V rows
of visible keys, in-range bias, q, out, page-table entries) divided by the
wall-clock step time (the timed steps run back to back, with nothing
recorded between them). ``roofline`` divides the same algorithmic figure (or
the flops, for the compute-bound prefill workload) by the average duration
of the attention kernels (``rel_attn_fwd_splits``; the combine kernel runs
after the second event), from HIP events recorded around them in a second,
untimed pass of as many steps, on the stream they run on, and compares that
with MI355X's published peak. Its
``traffic`` is the HBM-side bytes per launch measured by rocprofv3 counters
(FETCH_SIZE, WRITE_SIZE, scaled by the same counters' reading for a plain copy
of known size), read from the committed counter summary under profiles/ when
that summary was taken on the current kernel sources, else null.
``cpu_baseline`` times the fp64 CPU oracle, unchanged, on a bounded sample of
the same workload over the host's cores (at most 16), before the GPU is
touched.
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

from paged_varlen_attention_gqa_amd import (rel_attn_combine, rel_attn_fwd,  # noqa: E402
                                           rel_attn_fwd_splits, rel_attn_num_splits,
                                           rel_attn_workspace_bytes)
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
    "decode_b64": "attn_decode_balanced_kernel + combine_kernel",
    "decode_long_b1": "attn_decode_balanced_kernel + combine_kernel",
    "decode_1m_b1_kv4": "attn_decode_balanced_kernel + combine_kernel",
    "decode_1m_b1_kv8": "attn_decode_balanced_kernel + combine_kernel",
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


# ---- CPU baseline: the fp64 oracle on the host's cores ----
# The pool is forked before this process touches the GPU, so that no worker
# holds a device handle; workers inherit the case through _POOL_CASE.
_POOL_CASE = None
_POOL_LIMIT = None


def _pool_init():
    from threadpoolctl import threadpool_limits

    global _POOL_LIMIT
    _POOL_LIMIT = threadpool_limits(limits=1)  # one BLAS thread per worker


def _pool_task(toks):
    import oracle

    oracle.oracle_attention(**_POOL_CASE.kwargs(), tokens=toks)
    return len(toks)


def host_cores() -> int:
    """Cores this process may use, capped at 16 (one GPU's share of a box)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown CPU"."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(case, name: str, target_s: float = 10.0, budget_s: float = 20.0) -> dict:
    """Time the fp64 oracle, unchanged, on a bounded sample of the same workload over the
    host's cores (a forked pool, one BLAS thread per worker): whole requests for decode
    workloads, the last 16 tokens of each request (in tasks of 2) for prefill workloads.
    Passes over the sample repeat until about ``target_s`` of wall time (at most
    ``budget_s``); the figure is the sample's algorithmic work over the wall time."""
    import multiprocessing as mp

    from paged_varlen_attention_gqa_amd.work import count_work

    global _POOL_CASE
    cu = case.cu_seqlens_q.tolist()
    B = case.batch_size
    klens = case.kv_lens()
    bound = BOUND[name]
    tasks, task_req = [], []
    for b in range(B):
        toks = list(range(cu[b], cu[b + 1]))
        if not toks:
            continue
        if bound == "mfma":
            toks = toks[-16:]
            for i in range(0, len(toks), 2):
                tasks.append(toks[i:i + 2])
                task_req.append(b)
        else:
            tasks.append(toks)
            task_req.append(b)
    cores = min(host_cores(), len(tasks))
    _POOL_CASE = case
    ctx = mp.get_context("fork")
    done_q, done_k = [], []
    wall, passes = 0.0, 0
    with ctx.Pool(cores, initializer=_pool_init) as pool:
        while wall < target_s and passes < 1000:
            t0 = time.perf_counter()
            counts = pool.map(_pool_task, tasks, chunksize=1)
            wall += time.perf_counter() - t0
            passes += 1
            for b, n in zip(task_req, counts):
                done_q.append(n)
                done_k.append(klens[b])
            if wall > budget_s:
                break
    _POOL_CASE = None
    w = count_work(query_lens=done_q, kv_lens=done_k, num_heads=case.num_heads,
                   num_kv_heads=case.num_kv_heads, head_dim=case.head_dim, block_size=case.block_size,
                   rel_extent=case.rel_extent, causal=case.causal, window_size=case.window_size,
                   elem_bytes=case.q.element_size())
    if bound == "mfma":
        value, unit = w.flops / wall / 1e12, "TFLOP/s"
        what = f"the last 16 query tokens of each of the {B} requests"
    else:
        value, unit = w.bytes / wall / 1e9, "GB/s"
        what = f"all {B} requests"
    return {"value": round(value, 6), "unit": unit, "cores": cores, "kind": "oracle",
            "sample": f"{what} ({sum(done_q)} query tokens over {passes} pass(es)), fp64 NumPy oracle in a "
                      f"pool of {cores} processes on {cpu_model()}, {wall:.1f} s wall"}


# ---- GPU timing of one workload ----
def time_workload(name: str, case, args, dev, splits_override=None) -> dict:
    """Warm-up, then exactly ``args.steps`` timed steps; stage durations from HIP events on
    the stream the kernels run on; then the same stage after cache flushes."""
    work = case_work(case)
    kw = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in case.kwargs().items()}
    wl, wr = case.window_size
    splits = splits_override or rel_attn_num_splits(
        is_local=(wl >= 0 or wr >= 0), batch_size=case.batch_size, max_query_len=case.max_seqlen_q,
        num_heads=case.num_heads, num_kv_heads=case.num_kv_heads, max_kv_len=max(case.kv_lens()))
    out = torch.empty_like(kw["q"])
    need = rel_attn_workspace_bytes(splits, case.num_tokens, case.num_heads, case.head_dim)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is None:
            rel_attn_fwd(**kw, num_splits=splits, out=out, workspace=ws)
            return
        # the same launches, the attention kernels between the events
        ev[0].record(stream)
        rel_attn_fwd_splits(**kw, num_splits=splits, out=out, workspace=ws)
        ev[1].record(stream)
        if splits > 1:
            rel_attn_combine(ws, out, splits)

    _log(f"[bench] {name}: warmup {args.warmup} (num_splits={splits})")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    _log(f"[bench] {name}: timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    # the duration of each call, from events around it (a pass of its own, so
    # that the event records do not sit between the timed steps)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    stage_ms = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
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
    del kw, out, ws
    return {
        "value": value, "unit": unit, "ms_per_step": ms_per_step, "roofline": roof,
        "config": {"workload": f"{name}: {DESCRIPTIONS[name]}", "num_splits": splits,
                   "algorithmic_bytes": work.bytes, "algorithmic_flops": work.flops,
                   "stage_kernels": STAGE_KERNELS[name],
                   "stage_us_mean": round(float(stage_ms.mean()) * 1e3, 2),
                   "stage_us_min": round(float(stage_ms.min()) * 1e3, 2),
                   "stage_us_cold_mean": round(float(cold_ms.mean()) * 1e3, 2) if cold_ms.size else None,
                   "tflops": round(tflops, 3), "gbs": round(gbs, 2)},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default=None, choices=sorted(DESCRIPTIONS),
                    help="time this workload alone (default: decode_b64 as the headline, with "
                         "prefill_chunked timed in the same run under config.prefill)")
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
    headline = args.config or "decode_b64"
    names = [headline] if args.config else [headline, "prefill_chunked"]
    cases = {}
    for n in names:
        _log(f"[bench] generating {n}")
        cases[n] = make_case(**config_spec(n))
    # the CPU baseline runs before this process touches the GPU (its pool is forked)
    cpu = {}
    if not args.no_cpu_baseline:
        for n in names:
            _log(f"[bench] timing the CPU oracle on a bounded sample of {n}")
            cpu[n] = cpu_baseline(cases[n], n)
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
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
    results = {}
    for n in names:
        results[n] = time_workload(n, cases[n], args, dev,
                                   splits_override=args.num_splits if n == headline else None)
        torch.cuda.empty_cache()
    h = results[headline]
    case = cases[headline]
    res = {
        "metric": METRIC, "value": round(h["value"], 3), "unit": h["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(h["ms_per_step"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if case.dtype == torch.bfloat16 else "f32", "data": "synthetic",
        "config": h["config"],
        "roofline": h["roofline"],
    }
    for n in names[1:]:
        r = results[n]
        extra = dict(r["config"])
        extra.update({"value": round(r["value"], 3), "unit": r["unit"], "steps": args.steps,
                      "ms_per_step": round(r["ms_per_step"], 5), "roofline": r["roofline"]})
        if n in cpu:
            extra["cpu_baseline"] = cpu[n]
        res["config"]["prefill" if n == "prefill_chunked" else n] = extra
    if headline in cpu:
        res["cpu_baseline"] = cpu[headline]
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
