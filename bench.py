"""Throughput of the exact attention forward on one MI355X.

One step = one fa_fwd launch over the whole workload (all steps of the hot
path: schedule, K/V loads, Q K^T, mask, softmax with conditional rescaling,
exp2, P V, epilogue), inputs resident in HBM before the timed region.
Default workload: causal attention, B=1, H=16, S=32768, D=128 (bf16 in,
bf16 O + fp32 LSE out).  The metric is TFLOP/s with the usual convention
4*B*H*S^2*D, halved for causal, and its fraction of the dense bf16 MFMA peak.
The S=8192 causal workload (B=2, H=16, D=128) the metric also names is timed
the same way and reported under "secondary".

Timing follows the FlashAttention-4 paper's protocol (appendix A.1: warm up,
then time repeated runs and report the mean): about a second of untimed
back-to-back steps so the clock settles (--settle-s), W untimed warm-up steps, then K
timed steps bracketed by torch.cuda.synchronize(); each launch is also
bracketed by HIP events on the launch stream for the per-launch kernel time
used by the roofline figure.

The cpu_baseline leg times the fp64 oracle (test infrastructure) on a
bounded sample of query rows of the same workload on the host cores.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
  python bench.py --backward [--table]     # the backward pass (fa_bwd_general)
  python bench.py --mfma-ceiling           # the matrix-unit ceiling alone

After the timed steps the bench line also carries the measured ceiling
(roofline.attainable, fa_mfma_ceiling): the forward's own product sequence
alone on every CU, operands in registers, and its clock; frac_of_attainable
is the kernel's rate against it (the lds_fed figures read the operands from
LDS as the forward does).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


FORWARD_SOURCES = ("fa_fwd.hip", "fa_tile.h", "fa_sched.h", "exp2_poly.h", "fa_host.h")


def kernel_sources_sha256() -> str:
    """Hash of the sources the forward kernel is built from, to tell whether a
    stored counter measurement still describes the current kernel."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_attention_forward_04_amd", "csrc")
    for name in FORWARD_SOURCES:
        h.update(name.encode())
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE profile
    (scaled by the copy-kernel calibration), or None if there is none for this
    workload or the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    return rec.get("hbm_bytes")


DEFAULT_WORKLOAD = "long_b1h16s32768d128_causal"
SECONDARY_WORKLOAD = "causal_b2h16s8192d128"


def settle(torch, step, seconds):
    """Run the step back to back, untimed, for about `seconds` of wall time.

    Under sustained matrix-core load the GPU's clock and power state take a
    fraction of a second to settle; a handful of warm-up launches of a
    sub-millisecond kernel end before that, and the timed steps then run
    partly at the idle clock (the 8k causal workload reads about 20% low).
    Returns the number of launches made."""
    if seconds <= 0:
        return 0
    torch.cuda.synchronize()
    n = 0
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        step()
        n += 1
        if n % 4 == 0:   # keep the launch queue short so the loop tracks GPU time
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def time_workload(fa, torch, w, steps, warmup, tuning=None, num_splits=None, settle_s=0.0):
    from attn_inputs import make, make_qk, flops
    dev = torch.device("cuda:0")
    extra = {}
    if w.q_range:   # queries with lengths of their own
        q, k, v, cu, cu_k, S, S_k = make_qk(w)
        extra = dict(cu_seqlens_k=torch.from_numpy(cu_k).to(dev), max_seqlen_k=S_k)
    else:
        q, k, v, cu, S = make(w)
    dq, dk, dv = q.to(dev), k.to(dev), v.to(dev)
    dcu = None if cu is None else torch.from_numpy(cu).to(dev)
    o = torch.empty(tuple(dq.shape[:-1]) + (w.head_dim_v,), dtype=dq.dtype, device=dev)
    T = dq.shape[0] if cu is not None else None
    lse = torch.empty((w.H, T) if cu is not None else (w.B, w.H, w.S), dtype=torch.float32,
                      device=dev)
    fl = flops(w, None if w.q_range else cu)

    if num_splits is not None:   # split-KV: one workspace for every step
        n_sp = num_splits
        if n_sp == 0:
            import ctypes
            c = ctypes.c_int(1)
            fa.load().fa_splitkv_auto_splits_gqa(w.B, w.H, w.kv_heads, S,
                                                 extra.get("max_seqlen_k", S), w.D,
                                                 ctypes.byref(c))
            n_sp = c.value
        nbytes = fa.splitkv_workspace_size(w.B, w.H, S, extra.get("max_seqlen_k", S),
                                           w.head_dim_v, n_sp)
        extra = dict(extra, num_splits=n_sp,
                     workspace=torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev))

    def step():
        fa.attention(dq, dk, dv, causal=w.causal, scale=w.scale, cu_seqlens=dcu,
                     max_seqlen=S if cu is not None else None, out=o, lse_out=lse,
                     tuning=tuning, **extra)

    n_settle = settle(torch, step, settle_s)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = [a.elapsed_time(b) for a, b in ev]
    from attn_inputs import io_bytes
    return {
        "flops": fl,
        "bytes": io_bytes(w, None if w.q_range else cu),
        "num_splits": extra.get("num_splits", 1),
        "ms_per_step": wall * 1e3 / steps,
        "kernel_ms_mean": float(np.mean(kernel_ms)),
        "kernel_ms_median": float(np.median(kernel_ms)),
        "kernel_ms_min": float(np.min(kernel_ms)),
        "settle_launches": n_settle,
        "inputs": (q, k, v, cu),
    }


BACKWARD_WORKLOADS = ["causal_b2h16s8192d128", "long_b1h16s32768d128_causal",
                      "dense_b2h16s2048d128", "dense_b2h16s2048d128_causal",
                      "gqa_b2h32kv8s8192d128_causal", "varlen_16x512to8192_h32d128_causal",
                      "smoke_b1h8s512d64_causal", "mixed_16x_q1to2048_k512to8192_h16d128_causal",
                      "wide_b2h16s8192d256_spread3", "hd192v128_b2h16s8192_causal"]


def time_backward(fa, torch, w, steps, warmup, settle_s=0.0):
    """Time the backward (fa_bwd_general, or fa_bwd_hd for the (192, 128) head
    dimensions: its dQ kernel and its dK/dV kernel) on a workload, after one
    forward launch that provides o and lse.  Flops follow the usual backward
    convention: five products per block (S, dP, dV, dQ, dK), 2.5x the
    forward's when D_v = D."""
    from attn_inputs import draw_dout, flops, make, make_qk
    dev = torch.device("cuda:0")
    dcu_k, ms_k = None, None
    if w.q_range:   # queries with lengths of their own
        q, k, v, cu, cu_k, S, S_k = make_qk(w)
        dcu_k, ms_k = torch.from_numpy(cu_k).to(dev), S_k
    else:
        q, k, v, cu, S = make(w)
    dq_, dk_, dv_ = q.to(dev), k.to(dev), v.to(dev)
    dcu = None if cu is None else torch.from_numpy(cu).to(dev)
    ms = S if cu is not None else None
    o, lse = fa.attention(dq_, dk_, dv_, causal=w.causal, scale=w.scale, cu_seqlens=dcu,
                          max_seqlen=ms, cu_seqlens_k=dcu_k, max_seqlen_k=ms_k)
    g = draw_dout(tuple(o.shape), w.seed).to(dev)
    gq, gk, gv = torch.empty_like(dq_), torch.empty_like(dk_), torch.empty_like(dv_)
    delta = torch.empty_like(lse)

    def step():
        fa.attention_backward(dq_, dk_, dv_, o, lse, g, causal=w.causal, scale=w.scale,
                              cu_seqlens=dcu, max_seqlen=ms, dq=gq, dk=gk, dv=gv, delta=delta,
                              cu_seqlens_k=dcu_k, max_seqlen_k=ms_k)

    settle(torch, step, settle_s)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = [a.elapsed_time(b) for a, b in ev]
    # five products per block: S and dQ, dK contract or produce D-wide rows,
    # dP and dV D_v-wide ones (2.5x the forward when D_v = D)
    D, Dv = w.D, w.head_dim_v
    fl = flops(w, None if w.q_range else cu) * (3 * D + 2 * Dv) / (D + Dv)
    return {"workload": w.name, "pass": "backward", "flops": fl,
            "ms_per_step": round(wall * 1e3 / steps, 4),
            "kernel_ms_mean": round(float(np.mean(kernel_ms)), 4),
            "kernel_ms_median": round(float(np.median(kernel_ms)), 4),
            "TFLOP/s": round(fl / (float(np.mean(kernel_ms)) * 1e-3) / 1e12, 1),
            "pct_of_peak": round(100 * fl / (float(np.mean(kernel_ms)) * 1e-3) / 1e12
                                 / PEAK_BF16_TFLOPS, 2)}


def cpu_baseline(w, inputs, target_s=15.0):
    """Time the fp64 oracle on a bounded, seeded sample of query rows."""
    import oracle
    q, k, v, cu = inputs
    rng = np.random.default_rng(12345)
    if cu is None:
        nrows = w.B * w.H * w.S
        keys_of = (lambda r: (r % w.S) + 1) if w.causal else (lambda r: np.full_like(r, w.S))
    else:
        T = int(cu[-1])
        nrows = w.H * T
        starts = np.asarray(cu[:-1])

        def keys_of(r):
            t = r % T
            b = np.searchsorted(cu, t, side="right") - 1
            L = cu[b + 1] - cu[b]
            return (t - starts[b] + 1) if w.causal else L
    # calibrate on a small batch, then size the sample to about target_s
    n = 64
    total_rows, total_flops, total_s = 0, 0.0, 0.0
    while total_s < target_s and n > 0:
        rows = rng.choice(nrows, n, replace=False)
        t0 = time.perf_counter()
        oracle.attention_rows_bf16(q, k, v, rows, w.scale, w.causal, cu)
        dt = time.perf_counter() - t0
        total_s += dt
        total_rows += n
        total_flops += float(np.sum(2.0 * (w.D + w.head_dim_v) * keys_of(rows)))
        rate = n / max(dt, 1e-6)
        n = int(min(max(rate * (target_s - total_s), 0), 20000))
    return {
        "value": total_flops / total_s / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "%d random query rows (all their keys) of %s, fp64, %.1f s" % (
            total_rows, w.name, total_s),
    }


CEILING_BLOCKS = 8192   # 64-key blocks per wave: about 10 ms per ceiling launch


def settle_ceiling(fa, seconds):
    """Untimed ceiling launches for about this many seconds (clock settle)."""
    t0 = time.time()
    while time.time() - t0 < seconds:
        fa.mfma_ceiling(0, CEILING_BLOCKS, 5)


def ceiling_record(mode, c):
    return {"mfma_ceiling": "registers" if mode == 0 else "lds_fed",
            "TFLOP/s": round(c["tflops"], 2), "best_TFLOP/s": round(c["best_tflops"], 2),
            "ms": round(c["ms"], 4), "cus": c["workers"], "products": c["products"],
            "clock_mhz": round(c["clock_mhz"], 1),
            "cycles_per_product": round(c["cycles_per_product"], 2),
            "frac_of_nominal_peak": round(c["tflops"] / PEAK_BF16_TFLOPS, 4),
            "peak_at_measured_clock": round(4096 * c["workers"] * c["clock_mhz"] * 1e-6, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="untimed back-to-back steps for this many seconds before the warm-up "
                         "steps, so that the timed steps run at the settled clock (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--tau", type=float, default=None)
    ap.add_argument("--exp2-emu", type=int, default=None)
    ap.add_argument("--schedule", type=int, default=None)
    ap.add_argument("--table", action="store_true",
                    help="time every named workload (one JSON line each) instead of the "
                         "single bench line")
    ap.add_argument("--gemm-reference", action="store_true",
                    help="only time torch's bf16 matmul (hipBLASLt) on large shapes, as context "
                         "for the MFMA fraction the attention kernel reaches")
    ap.add_argument("--num-splits", type=int, default=None,
                    help="run the workload through split-KV (fa_fwd_splitkv) with this many "
                         "key splits (0: the library's choice for the device)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (fa_bwd) on --workload, or with --table on "
                         "every workload it supports (one JSON line each)")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only run the matrix-unit ceiling microbenchmark (the D = 128 "
                         "forward's product sequence alone, operands in registers and from LDS)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="leave the measured ceiling (roofline.attainable) out of the bench line")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (3 times); used to "
                         "scale the FETCH_SIZE / WRITE_SIZE counters of a profiler run")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the attention forward runs on a single MI355X "
              "(every (sequence, head, row-tile) is independent; see the sharding notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_forward_04_amd as fa
    from attn_inputs import WORKLOADS
    if not torch.cuda.is_available():
        print("no GPU", file=sys.stderr)
        sys.exit(1)
    fa.load()

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "launches": 3}))
        return

    if args.mfma_ceiling:
        settle_ceiling(fa, 1.0)
        for mode in (0, 1):
            c = fa.mfma_ceiling(mode, CEILING_BLOCKS, 7)
            print(json.dumps(ceiling_record(mode, c)), flush=True)
        return

    if args.gemm_reference:
        for (m, n, kk) in [(4096, 4096, 4096), (8192, 8192, 8192), (16384, 16384, 8192)]:
            a = torch.randn(m, kk, dtype=torch.bfloat16, device="cuda")
            b = torch.randn(kk, n, dtype=torch.bfloat16, device="cuda")
            for _ in range(5):
                c = a @ b
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(20):
                c = a @ b
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 20
            print(json.dumps({"gemm_bf16": [m, n, kk], "ms": round(ms, 4),
                              "TFLOP/s": round(2.0 * m * n * kk / ms / 1e9, 1)}), flush=True)
            del a, b, c
        return

    tuning = None
    if args.tau is not None or args.exp2_emu is not None or args.schedule is not None:
        tuning = fa.default_tuning()
        if args.tau is not None:
            tuning.tau = args.tau
        if args.exp2_emu is not None:
            tuning.exp2_emu = args.exp2_emu
        if args.schedule is not None:
            tuning.schedule = args.schedule

    if args.backward:
        names = BACKWARD_WORKLOADS if args.table else [args.workload]
        for name in names:
            print(json.dumps(time_backward(fa, torch, WORKLOADS[name], args.steps, args.warmup,
                                            args.settle_s)),
                  flush=True)
        return

    if args.table:
        for name, wl in WORKLOADS.items():
            # workloads with few query rows per sequence also run split-KV
            for sp in ([None, 0] if wl.q_range else [None]):
                rr = time_workload(fa, torch, wl, args.steps, args.warmup, tuning, num_splits=sp,
                                   settle_s=args.settle_s)
                v = rr["flops"] / (rr["kernel_ms_mean"] * 1e-3) / 1e12
                print(json.dumps({"workload": name, "num_splits": rr["num_splits"],
                                  "kernel_ms_mean": round(rr["kernel_ms_mean"], 4),
                                  "kernel_ms_median": round(rr["kernel_ms_median"], 4),
                                  "TFLOP/s": round(v, 1),
                                  "pct_of_peak": round(100 * v / PEAK_BF16_TFLOPS, 2),
                                  "GB/s": round(rr["bytes"] / (rr["kernel_ms_mean"] * 1e-3) / 1e9, 1),
                                  "flops": rr["flops"]}), flush=True)
        return

    w = WORKLOADS[args.workload]
    r = time_workload(fa, torch, w, args.steps, args.warmup, tuning, num_splits=args.num_splits,
                      settle_s=args.settle_s)
    value = r["flops"] / (r["ms_per_step"] * 1e-3) / 1e12
    achieved = r["flops"] / (r["kernel_ms_mean"] * 1e-3) / 1e12
    out = {
        "metric": "attention fwd TFLOP/s (bf16) + % of MFMA peak, S=8k/32k D=128 causal",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"seconds": args.settle_s, "launches": r["settle_launches"]},
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": w.name, "B": w.B, "H": w.H, "S": w.S, "D": w.D,
                   "causal": w.causal, "seed": w.seed, "flops_per_step": r["flops"],
                   "num_splits": r["num_splits"],
                   "io_GB_per_s": round(r["bytes"] / (r["kernel_ms_mean"] * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(w.name),
                     "kernel_ms_mean": round(r["kernel_ms_mean"], 4),
                     "kernel_ms_median": round(r["kernel_ms_median"], 4),
                     "kernel_ms_min": round(r["kernel_ms_min"], 4)},
    }
    # the peak's inputs as the device reports them (CU count, peak shader clock)
    dev = fa.device_info()
    out["roofline"]["device"] = {
        "cus": dev["cus"], "peak_clock_mhz": dev["peak_clock_mhz"],
        "peak_from_device": round(4096 * dev["cus"] * dev["peak_clock_mhz"] * 1e-6, 1)}
    if not args.no_ceiling:
        # right after the timed steps, at the clock the GPU has settled to
        c0 = fa.mfma_ceiling(0, CEILING_BLOCKS, 7)
        c1 = fa.mfma_ceiling(1, CEILING_BLOCKS, 7)
        rf = out["roofline"]
        rf["attainable"] = round(c0["tflops"], 2)
        rf["frac_of_attainable"] = round(achieved / c0["tflops"], 4)
        rf["attainable_lds_fed"] = round(c1["tflops"], 2)
        rf["frac_of_attainable_lds_fed"] = round(achieved / c1["tflops"], 4)
        rf["ceiling"] = {"what": "fa_mfma_ceiling: the forward's 32 products per 64-key block "
                                 "alone, one 8-wave workgroup per CU",
                         "cus": c0["workers"],
                         "clock_mhz": round(c0["clock_mhz"], 1),
                         "clock_mhz_lds_fed": round(c1["clock_mhz"], 1),
                         "cycles_per_product": round(c0["cycles_per_product"], 2),
                         "cycles_per_product_lds_fed": round(c1["cycles_per_product"], 2),
                         "peak_at_measured_clock": round(
                             4096 * c0["workers"] * c0["clock_mhz"] * 1e-6, 1)}
    if not args.no_secondary and args.workload == DEFAULT_WORKLOAD:
        w2 = WORKLOADS[SECONDARY_WORKLOAD]
        r2 = time_workload(fa, torch, w2, args.steps, args.warmup, tuning, settle_s=args.settle_s)
        v2 = r2["flops"] / (r2["ms_per_step"] * 1e-3) / 1e12
        out["secondary"] = {"workload": w2.name, "value": round(v2, 2), "unit": "TFLOP/s",
                            "pct_of_peak": round(100 * v2 / PEAK_BF16_TFLOPS, 2),
                            "ms_per_step": round(r2["ms_per_step"], 4),
                            "kernel_ms_mean": round(r2["kernel_ms_mean"], 4)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, r["inputs"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
