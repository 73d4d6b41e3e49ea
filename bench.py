#!/usr/bin/env python3
"""Benchmark: batched paged-KV MLA decode (absorbed form) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload deepseek]

A step is one pass of the whole decode path (fused decode kernel + split
merge) over one batch.  The timed region runs K steps back to back; every step
reads a different copy ("layer") of the KV cache and query, cycling over
enough copies to exceed the 256 MB last-level cache, so KV bytes come from HBM
as they would across the layers of a real model.  Inputs are seeded synthetic
bf16 (N(0,1)*0.5) with the workload's shapes; they are resident in HBM before
the timed region starts.  Prints one JSON line.

Timing.  The timed region is K steps back to back between two HIP events
(created without the system-scope fence); ms_per_step is their interval over
K.  During those same K steps the library's timing records are on: every
workgroup of every decode and merge launch stores its start and end on the
GPU's 100 MHz real-time counter (plain stores to its own words: no events or
atomics between or inside the steps, which would change how the launches run;
measured cost under 1% of a step).  The decode launches' duration of a step is
its merge's first block start minus its decode's first workgroup start (the
kernels run back to back, so this is the dispatch-to-next-dispatch duration a
rocprofv3 kernel trace reports; the next step's start when a step has no
merge), averaged over exactly the timed steps; the in-kernel span (first
workgroup start to last workgroup end) is reported beside it.  A second pass of 64
steps, recorded the same way, gives the per-step median and p10/p90 from the
intervals between consecutive launch starts.  The default warm-up (1000
steps, under 0.1 s) runs the GPU into its steady clock state: after an idle
period the first few hundred steps run at another speed before they settle.

Roofline of the dominant kernel (the fused decode kernel): algorithmic bytes
per launch = 1152 B per unique KV token + query (1152 B per head) + output
(1024 B + 4 B lse per head) + page-table bytes (flops: 2176 per attended token
and head), divided by the kernel's mean span.  The line refuses to print if a
decode kernel measured longer than the step that contains it.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2516.6    # MI355X dense bf16 MFMA, TFLOP/s (256 CU x 4096 flop/clk x 2.4 GHz)
MALL_BYTES = 256 << 20

WORKLOAD_DESC = {
    "deepseek": "DeepSeek-V3-shaped decode: batch 64, 128 heads, kv_lora_rank 512, rope 64, "
                "page_size 64, kv_len uniform [1024,4096], random page table",
    "long": "long-context split-KV: batch 8, 128 heads, 512/64, page_size 64, kv_len 32768",
    "ragged": "ragged decode (16-head share of a 128-head model): batch 256, 16 heads, 512/64, "
              "page_size 1, kv_len lognormal(median 1024, sigma 1) clipped [1,16384]",
    "cascade": "cascade shared-prefix decode: batch 128, 128 heads, 512/64, page_size 64, "
               "8192-token shared prefix + suffix uniform [64,1024]",
    "tiny": "tiny decode: batch 4, 16 heads, 512/64, page_size 16, kv_len {1,17,64,200}",
    "qo": "several query tokens per request: batch 64, 4 new tokens each (causal among them), "
          "16 heads, 512/64, page_size 64, kv_len uniform [1024,4096]",
}


class HipEvents:
    """HIP events without the system-scope fence, through the HIP runtime that
    torch has loaded (torch's own events record with the fence)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        import torch
        self._c = ctypes
        self._hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib",
                                             "libamdhip64.so"))

    def create(self):
        e = self._c.c_void_p()
        rc = self._hip.hipEventCreateWithFlags(self._c.byref(e), self.DISABLE_SYSTEM_FENCE)
        assert rc == 0, rc
        return e

    def record(self, e, stream: int):
        rc = self._hip.hipEventRecord(e, self._c.c_void_p(stream))
        assert rc == 0, rc

    def elapsed(self, a, b) -> float:
        ms = self._c.c_float(0.0)
        rc = self._hip.hipEventElapsedTime(self._c.byref(ms), a, b)
        assert rc == 0, rc
        return float(ms.value)

    def destroy(self, e):
        self._hip.hipEventDestroy(e)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "paged_kv_mla_amd", "csrc"))):
        with open(os.path.join(ROOT, "paged_kv_mla_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def workload_counts(inp, kv_row_bytes: int = 1152):
    """Attended tokens (per query token, summed), unique KV rows and
    algorithmic bytes/flops of one step (kv_row_bytes: one token's ckv + kpe
    row, 1152 in bf16, 576 in fp8)."""
    H = inp.num_heads
    B = inp.batch
    rows = B   # query rows of H heads
    if hasattr(inp, "prefix_lens"):
        attended = inp.attended_tokens()
        unique = inp.unique_tokens()
        idx_bytes = 4 * (len(inp.prefix_indices) + len(inp.kv_indices)) + 8 * B
    elif getattr(inp, "qo_indptr", None) is not None:
        # query token j of n sees kv_len - n + 1 + j tokens; the cache is read once
        n = np.diff(inp.qo_indptr).astype(np.int64)
        L = inp.kv_lens.astype(np.int64)
        attended = int(np.sum(n * (L - n + 1) + n * (n - 1) // 2))
        unique = int(L.sum())
        rows = int(inp.qo_indptr[-1])
        idx_bytes = 4 * len(inp.kv_indices) + 12 * B
    else:
        attended = unique = inp.total_tokens
        idx_bytes = 4 * len(inp.kv_indices) + 8 * B
    alg_bytes = unique * kv_row_bytes + idx_bytes + rows * H * (1152 + 1024 + 4)
    alg_flops = 2176.0 * H * attended
    return attended, unique, alg_bytes, alg_flops


def cpu_baseline(inp, budget_s: float = 12.0):
    """Time the fp64 oracle on the host (a reported baseline, not a target)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    is_cas = hasattr(inp, "prefix_lens")
    is_qo = getattr(inp, "qo_indptr", None) is not None
    done_tokens = 0
    reqs = 0
    t0 = time.perf_counter()
    b = 0
    while True:
        sl = slice(b, b + 1)
        sc = (inp.ckv_scale, inp.kpe_scale) if inp.ckv8 is not None else None
        ckv, kpe = (inp.ckv8, inp.kpe8) if sc else (inp.ckv, inp.kpe)
        if is_cas:
            g = inp.group_of(b)
            oracle.attend_cascade(
                inp.q_nope[sl], inp.q_pe[sl], ckv, kpe, inp.page_size,
                np.array([0, 1], np.int32),
                np.array([0, inp.prefix_indptr[g + 1] - inp.prefix_indptr[g]], np.int32),
                inp.prefix_indices[inp.prefix_indptr[g]:inp.prefix_indptr[g + 1]],
                inp.prefix_lens[g:g + 1],
                np.array([0, inp.kv_indptr[b + 1] - inp.kv_indptr[b]], np.int32),
                inp.kv_indices[inp.kv_indptr[b]:inp.kv_indptr[b + 1]], inp.kv_lens[sl],
                kv_scales=sc)
            done_tokens += int(inp.prefix_lens[g]) + int(inp.kv_lens[b])
        elif is_qo:
            q0, q1 = int(inp.qo_indptr[b]), int(inp.qo_indptr[b + 1])
            ip = np.array([0, inp.kv_indptr[b + 1] - inp.kv_indptr[b]], np.int32)
            oracle.attend_qo(inp.q_nope[q0:q1], inp.q_pe[q0:q1], ckv, kpe,
                             np.array([0, q1 - q0], np.int32), ip,
                             inp.kv_indices[inp.kv_indptr[b]:inp.kv_indptr[b + 1]],
                             inp.kv_lens[sl], inp.page_size, sm_scale=inp.sm_scale,
                             kv_scales=sc)
            n, L = q1 - q0, int(inp.kv_lens[b])
            done_tokens += n * (L - n + 1) + n * (n - 1) // 2
        else:
            ip = np.array([0, inp.kv_indptr[b + 1] - inp.kv_indptr[b]], np.int32)
            oracle.attend_flat(inp.q_nope[sl], inp.q_pe[sl], ckv, kpe, ip,
                               inp.kv_indices[inp.kv_indptr[b]:inp.kv_indptr[b + 1]],
                               inp.kv_lens[sl], inp.page_size, sm_scale=inp.sm_scale,
                               kv_scales=sc)
            done_tokens += int(inp.kv_lens[b])
        reqs += 1
        b = (b + 1) % inp.batch
        el = time.perf_counter() - t0
        if el >= budget_s or reqs >= 64 * inp.batch:
            break
    return {"value": done_tokens / el, "unit": "KV-tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{reqs} requests of the same workload in order (cycling), fp64 numpy, "
                      f"{el:.1f} s wall"}


def load_traffic(workload: str, launches_tokens: int, kv: str = "bf16"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    suffix = "" if kv == "bf16" else "_" + kv
    path = os.path.join(ROOT, "profiles", f"traffic_decode_{workload}{suffix}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="deepseek", choices=sorted(WORKLOAD_DESC))
    ap.add_argument("--layers", type=int, default=0,
                    help="KV copies cycled over (0: enough to exceed the last-level cache)")
    ap.add_argument("--kv", default="bf16", choices=["bf16", "fp8"],
                    help="KV-cache element type: bf16, or OCP E4M3 codes with per-tensor "
                         "scales (queries and outputs stay bf16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for HBM counter calibration)")
    ap.add_argument("--gemm-calibration", action="store_true",
                    help="only time a plain bf16 GEMM (8192^3, the PyTorch/hipBLASLt "
                         "library path): the dense MFMA rate a library reaches on this GPU")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return

    if args.gemm_calibration:
        n = 8192
        a = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
        b = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
        for _ in range(5):
            c = a @ b
        torch.cuda.synchronize()
        hip = HipEvents()
        e0, e1 = hip.create(), hip.create()
        sh = int(torch.cuda.current_stream().cuda_stream)
        reps = 50
        hip.record(e0, sh)
        for _ in range(reps):
            c = a @ b
        hip.record(e1, sh)
        torch.cuda.synchronize()
        ms = hip.elapsed(e0, e1) / reps
        tfs = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
        del c
        print(json.dumps({"gemm": "bf16 8192x8192x8192 (torch.matmul)", "ms": round(ms, 4),
                          "tflops": round(tfs, 1), "frac_of_peak": round(tfs / MFMA_BF16_PEAK_TFS, 4)}))
        return

    import paged_kv_mla_amd as pk
    from mla_workloads import make_config, quantize_kv_fp8

    fp8 = args.kv == "fp8"
    t0 = time.perf_counter()
    inp = make_config(args.workload)
    if fp8:
        inp = quantize_kv_fp8(inp)
    gen_s = time.perf_counter() - t0
    attended, unique, alg_bytes, alg_flops = workload_counts(inp, 576 if fp8 else 1152)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")

    def dev8(codes):
        return torch.from_numpy(np.ascontiguousarray(codes)).to("cuda")

    pool_bytes = (inp.ckv8.nbytes + inp.kpe8.nbytes) if fp8 else (inp.ckv.nbytes + inp.kpe.nbytes)
    layers = args.layers or max(2, math.ceil(3 * MALL_BYTES / pool_bytes))
    ckv0, kpe0 = (dev8(inp.ckv8), dev8(inp.kpe8)) if fp8 else (dev(inp.ckv), dev(inp.kpe))
    qn0, qp0 = dev(inp.q_nope), dev(inp.q_pe)
    ckvs = [ckv0] + [ckv0.clone() for _ in range(layers - 1)]
    kpes = [kpe0] + [kpe0.clone() for _ in range(layers - 1)]
    qns = [qn0] + [qn0.clone() for _ in range(layers - 1)]
    qps = [qp0] + [qp0.clone() for _ in range(layers - 1)]
    B, H = inp.batch, inp.num_heads
    R = int(inp.qo_indptr[-1]) if getattr(inp, "qo_indptr", None) is not None else B
    outs = [torch.empty((R, H, 512), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
    lses = [torch.empty((R, H), dtype=torch.float32, device="cuda") for _ in range(layers)]
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    plan = pk.plan_for(inp)
    plan_ms = (time.perf_counter() - t0) * 1e3

    stream = torch.cuda.current_stream()
    sh = int(stream.cuda_stream)

    def step(i):
        k = i % layers
        if fp8:
            plan.run_fp8_ptrs(qns[k].data_ptr(), qps[k].data_ptr(), ckvs[k].data_ptr(),
                              kpes[k].data_ptr(), 512, 64, inp.ckv_scale, inp.kpe_scale,
                              outs[k].data_ptr(), lses[k].data_ptr(), sh)
        else:
            plan.run_ptrs(qns[k].data_ptr(), qps[k].data_ptr(), ckvs[k].data_ptr(),
                          kpes[k].data_ptr(), outs[k].data_ptr(), lses[k].data_ptr(), sh)

    hip = HipEvents()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def timed_total(first, n):
        # the K timed steps, with one event before and one after them: an
        # event recorded between two steps delays the next step's dispatch
        e0, e1 = hip.create(), hip.create()
        torch.cuda.synchronize()
        hip.record(e0, sh)
        for i in range(n):
            step(first + i)
        hip.record(e1, sh)
        torch.cuda.synchronize()
        t = hip.elapsed(e0, e1)
        hip.destroy(e0)
        hip.destroy(e1)
        return t

    if args.steps > 256:
        print("--steps is at most 256 (the library keeps 256 timing records)", file=sys.stderr)
        sys.exit(2)
    plan.set_timing(True)
    total_ms = timed_total(args.warmup, args.steps)
    spans_us, t_start, t_merge = plan.timing_runs()
    ms_per_step = total_ms / args.steps
    durs = [t_merge[i] - t_start[i] if t_merge[i] >= 0 else t_start[i + 1] - t_start[i]
            for i in range(len(t_start)) if t_merge[i] >= 0 or i + 1 < len(t_start)]
    # per-step statistics: a second pass of 64 steps, back to back (no event
    # between the steps), from the intervals between launch starts
    stats_steps = 64
    plan.set_timing(True)
    total2_ms = timed_total(args.warmup + args.steps, stats_steps)
    _, starts_us, _ = plan.timing_runs()
    plan.set_timing(False)
    if len(spans_us) != args.steps or len(starts_us) != stats_steps:
        print(f"timing records: {len(spans_us)} and {len(starts_us)} runs", file=sys.stderr)
        sys.exit(3)
    per_step = np.diff(starts_us) * 1e-3           # ms, launch start to launch start
    kern_avg_ms = float(np.mean(durs)) * 1e-3
    span_avg_ms = float(np.mean(spans_us)) * 1e-3
    # the decode launches' own span must fit in the step that contains them;
    # their start-to-next-start duration can exceed it only under a profiler
    # that spaces the kernels (counter collection)
    if span_avg_ms > ms_per_step or span_avg_ms <= 0.0:
        print(f"inconsistent timing: decode span {span_avg_ms:.5f} ms against a step of "
              f"{ms_per_step:.5f} ms", file=sys.stderr)
        sys.exit(3)
    if kern_avg_ms > ms_per_step:
        print(f"note: decode {kern_avg_ms:.5f} ms exceeds the step of {ms_per_step:.5f} ms "
              f"(kernels spaced by a profiler?)", file=sys.stderr)

    value = attended / (ms_per_step * 1e-3)
    tflops = alg_flops / (ms_per_step * 1e-3) / 1e12
    # binding roof of the whole step
    t_hbm = alg_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = alg_flops / (MFMA_BF16_PEAK_TFS * 1e12)
    step_bound = "hbm" if t_hbm >= t_mfma else "mfma"
    # dominant kernel roofline
    if step_bound == "hbm":
        achieved = alg_bytes / (kern_avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = alg_flops / (kern_avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFS, 4)}
    roof["traffic"] = load_traffic(args.workload, attended, args.kv)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_budget)

    line = {
        "metric": "MLA paged decode KV-tokens/s (absorbed form), 1 MI355X",
        "value": round(value, 1),
        "unit": "KV-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 queries, fp8 e4m3 KV (per-tensor scales)" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_DESC[args.workload], "batch": B, "num_heads": H,
                   "query_rows": R,
                   "page_size": inp.page_size, "kv_cache": args.kv,
                   "attended_kv_tokens": attended,
                   "unique_kv_tokens": unique, "kv_copies_cycled": layers},
        "tflops": round(tflops, 2),
        "step_roofline_frac": round(max(t_hbm, t_mfma) / (ms_per_step * 1e-3), 4),
        "ms_per_step_median": round(float(np.median(per_step)), 5),
        "ms_per_step_p10": round(float(np.percentile(per_step, 10)), 5),
        "ms_per_step_p90": round(float(np.percentile(per_step, 90)), 5),
        "per_step_stats_steps": int(len(per_step)),
        "per_step_stats_source": "second pass of 64 steps, back to back: intervals between "
                                 "consecutive decode launch starts (in-kernel real-time stamps)",
        "decode_kernel_ms": round(kern_avg_ms, 5),
        "decode_kernel_source": "the K timed steps: first merge block start minus first decode "
                                "workgroup start (in-kernel real-time stamps), mean",
        "decode_span_ms": round(span_avg_ms, 5),
        "ms_per_step_timing_pass": round(total2_ms / stats_steps, 5),
        "alg_bytes_per_step": int(alg_bytes),
        "alg_flops_per_step": alg_flops,
        "plan_host_ms": round(plan_ms, 2),
        "input_gen_s": round(gen_s, 1),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
