"""Benchmark of the u4 group-64 affine quantized matmul hot path on one GPU.

Headline (`value`): the 14B-shaped decode step at M = 1, fused QKV GEMV + fused
gate+up+SwiGLU GEMV (hidden 5120, 40 q heads / 8 kv heads of 128, intermediate 13824),
u4 group-64 weights, seeded synthetic inputs resident in HBM.  One step = one fused-QKV
call and one fused-gate+up call on the next layer of a 48-layer rotating pool (4.8 GB,
far above the 256 MB last-level cache), each step with its own activation vector.  The
timed region replays a HIP graph holding all K steps, bracketed by device
synchronisation; the value is algorithmic bytes moved per second (packed codes + bf16
scales/biases + activations + outputs).

Also reported, each timed the same way (HIP graphs on one stream, events around them):
  * prefill GEMM at M = 2048 on the 14B layer (fused QKV, fused gate+up+SwiGLU) in
    TFLOP/s against the bf16 MFMA peak, with a dense bf16 torch.matmul of the same shape
    as context;
  * the 24B-dense-shaped decode step (40 layers of QKV + gate+up + down, fresh x per
    step, each layer's down on that layer's h);
  * the 35B-A3B-shaped MoE decode layer (top-8 of 256 experts gathered in place, stage 1
    gate+up+SwiGLU and stage 2 down + weighted combine, fresh routing per step and layer).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--pool", type=int, default=48, help="layer copies in the rotating weight pool")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-steps", type=int, default=2)
    ap.add_argument("--kernel-reps", type=int, default=1000,
                    help="launches per graph when timing one kernel on its own")
    ap.add_argument("--prefill-reps", type=int, default=20)
    ap.add_argument("--step24-steps", type=int, default=20)
    ap.add_argument("--moe-steps", type=int, default=20)
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the prefill, 24B-step and MoE measurements")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM traffic summary (" + COUNTERS_SUMMARY + ") from the counter "
                         "collections of two rocprofv3 --pmc runs of this script (FETCH_SIZE, WRITE_SIZE), "
                         "then exit; needs no GPU")
    return ap.parse_args()


KERNEL_SOURCES = ["gemm_affine_u4_amd/csrc/gemv_step.hip", "gemm_affine_u4_amd/csrc/qmm_step.h",
                  "gemm_affine_u4_amd/csrc/gemv_u4.hip", "gemm_affine_u4_amd/csrc/qmm_device.h"]
COUNTERS_SUMMARY = "profiles/gemv_step_decode_14B_hbm_counters.md"


def counted_traffic(key: str, summary: str = None):
    """HBM bytes per launch measured by the committed counter runs (FETCH_SIZE and
    WRITE_SIZE, calibrated on a device copy), or None if the kernel sources changed
    since they were taken."""
    import re
    try:
        text = open(summary or os.path.join(ROOT, COUNTERS_SUMMARY)).read()
        if re.search(r"source_sha256_16: (\w+)", text).group(1) != _source_hash():
            return None
        return int(re.search(rf"traffic_bytes_per_launch\.{key}: (\d+)", text).group(1))
    except (OSError, AttributeError):
        return None


COUNTER_CMD = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 rocprofv3 --pmc {c} --output-format csv "
               "-d $REPO/gpurun_out/prof_{n} -o {n} -- python3 $REPO/bench.py --steps 20 --warmup 2 "
               "--kernel-reps 20 --no-cpu-baseline --headline-only")


def _source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def summarize_counters(fetch_csv: str, write_csv: str, out: str = None) -> str:
    """HBM bytes per launch of the decode kernels from FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for the bench's 2 GiB device copy
    (2 GiB read and 2 GiB written); writes COUNTERS_SUMMARY and returns its text."""
    import csv
    sh = __import__("synth").DENSE_14B
    K, I, rows_qkv = sh.K, sh.I, sh.qkv_rows
    b_qkv = weight_bytes(rows_qkv, K) + K * 2 + rows_qkv * 2
    b_gu = weight_bytes(2 * I, K) + K * 2 + I * 2

    def values(path, match):
        v = [float(r["Counter_Value"]) for r in csv.DictReader(open(path)) if match in r["Kernel_Name"]]
        if not v:
            raise SystemExit(f"{path}: no dispatch of {match}")
        return v

    def mean_of(path, match):
        v = values(path, match)
        return sum(v) / len(v), len(v)

    def copies(path):
        # the bench's ten 2 GiB device copies: the ten largest readings of the copy kernel
        # (the plans' host-to-device uploads run it too, on a few KB)
        v = sorted(values(path, "__amd_rocclr_copyBuffer"))[-10:]
        if len(v) < 10 or v[0] < 0.9 * v[-1]:
            raise SystemExit(f"{path}: the ten device copies are not the largest copy dispatches")
        return sum(v) / len(v)

    known = 2 * 2 ** 30 / 1024
    cf, cw = copies(fetch_csv), copies(write_csv)
    ff, fw = known / cf, known / cw
    if not (0.25 <= ff <= 8 and 0.25 <= fw <= 8):
        raise SystemExit(f"calibration factors {ff:.4g}, {fw:.4g}: the 2 GiB device copies are missing")
    lines = [f"copy calibration: FETCH_SIZE {cf:.1f} KiB, WRITE_SIZE {cw:.1f} KiB for a 2 GiB device copy -> "
             f"factors fetch {ff:.4f}, write {fw:.4f}"]
    keys = []
    for key, what, match, alg in [
            ("step", "one-launch 14B step (fused QKV + fused gate+up+SwiGLU, K=5120)",
             "qmm::step::gemv_step_single_inline_kernel<true>", b_qkv + b_gu),
            ("gate_up", "per-call fused gate+up+SwiGLU GEMV (K=5120, I=13824)",
             "qmm::b4::gemv_u4_s1_kernel<32, 5, 2, false, 1, 1>", b_gu),
            ("qkv", "per-call fused QKV GEMV (K=5120, 7168 rows)", "qmm::b4::gemv_u4_s1_kernel<32, 5, 1, false, 1, 1>",
             b_qkv)]:
        fk, nf = mean_of(fetch_csv, match)
        wk, nw = mean_of(write_csv, match)
        t = (fk * ff + wk * fw) * 1024
        lines.append(f"{what}: FETCH_SIZE {fk:.1f} KiB x {ff:.4f} + WRITE_SIZE {wk:.1f} KiB x {fw:.4f} = "
                     f"{t:.0f} B per launch; algorithmic {alg} B; ratio {t / alg:.4f} (n={nf},{nw})")
        keys.append(f"traffic_bytes_per_launch.{key}: {t:.0f}")
    h = _source_hash()
    text = "\n".join([
        "# Decode GEMV kernels, 14B-shaped step — HBM traffic counters (rocprofv3 --pmc)", "",
        "Two counter runs, one counter each (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch):", "",
        "    " + COUNTER_CMD.format(c="FETCH_SIZE", n="fetch"),
        "    " + COUNTER_CMD.format(c="WRITE_SIZE", n="write"), "",
        "Summarised by `python3 bench.py --summarize-counters <fetch_counter_collection.csv> "
        "<write_counter_collection.csv>`.  Calibration: bench.py runs ten 2 GiB device-to-device copies "
        "(`__amd_rocclr_copyBuffer`, 2 GiB read and 2 GiB written each); the counters' readings for that copy "
        "give the factors applied to the kernels.  Traffic per launch = the mean over all launches of that "
        "kernel (the 48-layer pool rotates, so every launch streams its weights from HBM).", "",
        *["    " + ln for ln in lines], "",
        "Machine-readable (read by bench.py; valid only while the kernel sources hash to the value below, "
        "otherwise bench.py reports traffic as null):", "",
        f"    source_sha256_16: {h}", *["    " + k for k in keys], ""])
    with open(out or os.path.join(ROOT, COUNTERS_SUMMARY), "w") as f:
        f.write(text)
    return text


def weight_bytes(rows: int, K: int) -> int:
    return rows * K // 2 + 2 * rows * (K // 64) * 2


class Timer:
    """HIP graphs captured and replayed on one stream, timed with events on that stream."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def capture(self, fn, n):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(self.stream):
            fn(0)  # touch once outside capture
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=self.stream):
                for i in range(n):
                    fn(i)
        torch.cuda.synchronize()
        return g

    def replay_ms(self, g, reps=1):
        torch = self.torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):
            e0.record(self.stream)
            for _ in range(reps):
                g.replay()
            e1.record(self.stream)
        e1.synchronize()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def per_call_ms(self, fn, n):
        """Average duration of one call of fn over a graph of n calls (after one warm replay)."""
        g = self.capture(fn, n)
        self.replay_ms(g)
        ms = self.replay_ms(g) / n
        del g
        return ms


def _progress(msg):
    """One line per finished leg on stderr (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = _args()
    if args.summarize_counters:
        print(summarize_counters(*args.summarize_counters))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: --gpus must be 1 (no multi-GPU path is built)",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)

    import torch
    import gemm_affine_u4_amd as qmm
    import synth

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    qmm.load_library()
    dev = torch.device("cuda:0")
    sh = synth.DENSE_14B
    K, I, q_out, kv_out = sh.K, sh.I, sh.q_out, sh.kv_out
    rows_qkv, rows_gu = sh.qkv_rows, 2 * I

    # ---- inputs: one seeded layer, replicated into a rotating pool --------------------
    w_qkv = synth.gen_weight(synth.CFG_14B, 0, synth.PROJ_QKV, rows_qkv, K)
    w_gu = synth.gen_weight(synth.CFG_14B, 0, synth.PROJ_GATE_UP, rows_gu, K)

    P = args.pool
    pq = pool_of(torch, dev, w_qkv, P)
    pg = pool_of(torch, dev, w_gu, P)
    NX = 16
    xs = torch.from_numpy(np.concatenate([synth.gen_x(synth.CFG_14B, 0, s, 1, K) for s in range(NX)]).view(np.int16)).to(dev)
    q = torch.empty((1, q_out), dtype=torch.bfloat16, device=dev)
    k = torch.empty((1, kv_out), dtype=torch.bfloat16, device=dev)
    v = torch.empty((1, kv_out), dtype=torch.bfloat16, device=dev)
    h = torch.empty((1, I), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    bytes_qkv = weight_bytes(rows_qkv, K) + K * 2 + rows_qkv * 2
    bytes_gu = weight_bytes(rows_gu, K) + K * 2 + I * 2
    bytes_step = bytes_qkv + bytes_gu

    stream = torch.cuda.Stream()
    T = Timer(torch, stream)

    # the step: fused QKV and fused gate+up+SwiGLU of one token in one launch (a planned
    # decode step); step i reads layer i % P of the pool and activation row i % NX, so one
    # plan per (layer, row) pair that occurs
    NP = P * NX // math.gcd(P, NX)
    plans = []
    for j in range(NP):
        L, x = j % P, xs[j % NX]
        pr = [qmm.step_fused_qkv(x, pq[0][L], pq[1][L], pq[2][L], q, k, v),
              qmm.step_gate_up_swiglu(x, pg[0][L], pg[1][L], pg[2][L], h)]
        mem = torch.empty(qmm.qmm_step_plan_bytes(pr), dtype=torch.uint8, device=dev)
        qmm.qmm_step_plan(pr, mem, stream=stream)
        plans.append((pr, mem))

    def step(i):
        pr, mem = plans[i % NP]
        qmm.qmm_step_run(pr, mem, stream=stream)

    def per_call_step(i):
        L = i % P
        x = xs[i % NX]
        qmm.qmm_fused_qkv(x, pq[0][L], pq[1][L], pq[2][L], q, k, v, stream=stream)
        qmm.qmm_fused_gate_up_swiglu(x, pg[0][L], pg[1][L], pg[2][L], h, stream=stream)

    def gate_up_only(i):
        L = i % P
        qmm.qmm_fused_gate_up_swiglu(xs[i % NX], pg[0][L], pg[1][L], pg[2][L], h, stream=stream)

    def qkv_only(i):
        L = i % P
        qmm.qmm_fused_qkv(xs[i % NX], pq[0][L], pq[1][L], pq[2][L], q, k, v, stream=stream)

    # warmup (eager), then the timed graph of exactly K steps
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()
    g_step = T.capture(step, args.steps)
    with torch.cuda.stream(stream):
        g_step.replay()
    torch.cuda.synchronize()
    ms_total = T.replay_ms(g_step)
    del g_step
    ms_per_step = ms_total / args.steps
    _progress(f"headline step: {ms_per_step * 1e3:.2f} us")
    value = bytes_step / (ms_per_step * 1e-3) / 1e9
    # one launch per step: the step kernel's average launch duration is the step time

    # the same work as two per-call launches, and each of them alone
    ms_pc = T.per_call_ms(per_call_step, args.kernel_reps)
    ms_gu = T.per_call_ms(gate_up_only, args.kernel_reps)
    ms_qkv = T.per_call_ms(qkv_only, args.kernel_reps)
    ach_gu = bytes_gu / (ms_gu * 1e-3) / 1e9
    ach_qkv = bytes_qkv / (ms_qkv * 1e-3) / 1e9

    copy_gbs = device_copy_gbs(torch, dev)
    read_ceiling = hbm_read_ceiling(torch, dev, T)
    _progress("per-call kernels and read ceilings done")

    result = {
        "metric": "achieved HBM GB/s (% of peak) fused u4 GEMV M=1; prefill GEMM TFLOP/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u4 weights, bf16 activations, fp32 accumulate",
        "data": "synthetic (seeded: codes uniform 0..15, scales U[0.001,0.01] bf16, bias=-8*scale, x~N(0,1) bf16)",
        "config": {"workload": "14B-shaped decode M=1: fused QKV [7168 x 5120] + fused gate+up+SwiGLU "
                               "[27648 x 5120], u4 g64, 48-layer rotating pool, one planned launch per step",
                   "global_batch": 1, "seq_len": 1, "parallelism": "none (1 GPU)",
                   "bytes_per_step": bytes_step, "pool_layers": P},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm",
                     "kernel": "gemv_step_single_inline_kernel<true> (the whole step in one launch: fused QKV "
                               "+ fused gate+up+SwiGLU, K=5120)",
                     "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": counted_traffic("step"),
                     "bytes_per_launch": bytes_step, "avg_launch_us": ms_per_step * 1e3},
        "kernels": {"one_launch_step": {"avg_launch_us": ms_per_step * 1e3, "GB/s": round(value, 1),
                                        "bytes_per_launch": bytes_step},
                    "per_call_step": {"us_per_step": ms_pc * 1e3, "launches": 2,
                                      "GB/s": round(bytes_step / (ms_pc * 1e-3) / 1e9, 1)},
                    "fused_qkv_gemv": {"avg_launch_us": ms_qkv * 1e3, "GB/s": round(ach_qkv, 1),
                                       "bytes_per_launch": bytes_qkv},
                    "fused_gate_up_gemv": {"avg_launch_us": ms_gu * 1e3, "GB/s": round(ach_gu, 1),
                                           "bytes_per_launch": bytes_gu}},
        "device_copy_GBps": round(copy_gbs, 1),
        "hbm_read_ceiling_GBps": read_ceiling,
    }
    c100 = read_ceiling["100MB"]["GB/s"]
    result["pct_of_read_ceiling_100MB"] = round(100 * value / c100, 2)

    if not args.headline_only:
        result["mfma_ceiling"] = mfma_ceiling(torch, dev, T)
        _progress("mfma_ceiling done")
        result["qkv_rope"] = bench_rope(torch, qmm, synth, T, dev, pq, args.prefill_reps)
        _progress("qkv_rope done")
        result["prefill_gemm"] = bench_prefill(torch, qmm, synth, T, dev, pq, pg, args.prefill_reps)
        _progress("prefill_gemm done")
        result["small_batch"] = bench_small_batch(torch, qmm, synth, T, dev, pq, pg)
        _progress("small_batch done")
        del pq, pg
        torch.cuda.empty_cache()
        result["decode_24B_step"] = bench_step_24b(torch, qmm, synth, T, dev, args.step24_steps)
        _progress("decode_24B_step done")
        torch.cuda.empty_cache()
        result["moe_35B_layer"] = bench_moe(torch, qmm, synth, T, dev, args.moe_steps)
        _progress("moe_35B_layer done")
        torch.cuda.empty_cache()
        result["moe_35B_prefill"] = bench_moe_prefill(torch, qmm, synth, T, dev, args.prefill_reps)
        _progress("moe_35B_prefill done")
        torch.cuda.empty_cache()
        result["formats"] = bench_formats(torch, qmm, synth, T, dev, args.prefill_reps)
        _progress("formats done")
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_sample_steps, w_qkv, w_gu, bytes_step)
        _progress("cpu_baseline done")

    print(json.dumps(result), flush=True)


def up(torch, dev, a):
    return torch.from_numpy(a.view(np.int32) if a.dtype == np.uint32 else a.view(np.int16)).to(dev)


def pool_of(torch, dev, w, P):
    """P device copies of one seeded weight: [P, rows, ...] for codes, scales, biases."""
    out = []
    for arr in (w.codes, w.scales, w.biases):
        t = up(torch, dev, arr)
        stack = torch.empty((P,) + tuple(t.shape), dtype=t.dtype, device=dev)
        stack.copy_(t.unsqueeze(0).expand_as(stack))
        out.append(stack)
    return out


def _ceiling_lib():
    import ctypes
    path = os.path.join(ROOT, "gemm_affine_u4_amd", "libqmm_ceiling.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m gemm_affine_u4_amd.build`")
    lib = ctypes.CDLL(path)
    lib.qmm_ceiling_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p]
    lib.qmm_ceiling_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return lib


def hbm_read_ceiling(torch, dev, T):
    """Plain streaming read (no compute, 16-byte non-temporal loads) per launch size, timed
    like the kernels: a HIP graph of launches, each on its own slice of a 2 GiB pool (8x the
    last-level cache), and one 4 GiB buffer.  Best over launch shapes (waves per CU, 1 KB
    loads in flight per wave, a contiguous slice per wave or interleaved groups): the rate a
    single launch of that many bytes reaches on this GPU, the ceiling a GEMV of that size
    per launch can approach."""
    lib = _ceiling_lib()
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    st = T.stream.cuda_stream
    shapes = [(256 * b, u, il) for b in (2, 4, 8) for u in (2, 4) for il in (0, 1)]

    def best_of(fn_for, n, nbytes):
        best = None
        for blocks, unroll, il in shapes:
            ms = T.per_call_ms(fn_for(blocks, unroll, il), n)
            gbs = nbytes / (ms * 1e-3) / 1e9
            if best is None or gbs > best[0]:
                best = (gbs, blocks // 256 * 4, unroll, il, ms * 1e3)
        return {"GB/s": round(best[0], 1), "us": round(best[4], 2), "waves_per_cu": best[1],
                "loads_in_flight_per_wave": best[2], "partition": "interleaved" if best[3] else "contiguous"}

    pool = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    pool.fill_(1)
    out = {}
    for name, nbytes in [("20MB", 20 << 20), ("80MB", 80 << 20), ("100MB", 100 << 20), ("168MB", 168 << 20)]:
        nsl = (2 << 30) // nbytes

        def fn_for(blocks, unroll, il, nbytes=nbytes, nsl=nsl):
            return lambda i: lib.qmm_ceiling_read(pool.data_ptr() + (i % nsl) * nbytes, nbytes, blocks, unroll, il,
                                                  sink.data_ptr(), st)
        out[name] = best_of(fn_for, max(2 * nsl, 40), nbytes)
    del pool
    torch.cuda.empty_cache()
    big = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    big.fill_(1)
    out["4GiB"] = best_of(lambda b, u, il: (lambda i: lib.qmm_ceiling_read(big.data_ptr(), 4 << 30, b, u, il,
                                                                          sink.data_ptr(), st)), 4, 4 << 30)
    del big
    torch.cuda.empty_cache()
    return out


def mfma_ceiling(torch, dev, T):
    """Register-only loop of v_mfma_f32_32x32x16_bf16 (four independent accumulators per wave,
    8 waves per SIMD): the bf16 matrix rate this GPU sustains, next to the published peak."""
    lib = _ceiling_lib()
    sink = torch.zeros(256, dtype=torch.float32, device=dev)
    st = T.stream.cuda_stream
    blocks, iters = 256 * 8, 4000
    ms = T.per_call_ms(lambda i: lib.qmm_ceiling_mfma(blocks, iters, sink.data_ptr(), st), 5)
    flop = blocks * 4 * 4 * iters * 32768.0
    tf = flop / (ms * 1e-3) / 1e12
    return {"TFLOP/s": round(tf, 1), "frac_of_bf16_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
            "kernel": "v_mfma_f32_32x32x16_bf16 register loop, 32 waves per CU"}


def device_copy_gbs(torch, dev):
    """Plain device copy of 2 GB: the read+write ceiling a simple kernel reaches."""
    src = torch.empty(1 << 30, dtype=torch.int16, device=dev)
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    e1.synchronize()
    gbs = 10 * 2 * src.numel() * 2 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbs


def bench_prefill(torch, qmm, synth, T, dev, pq, pg, reps):
    """Prefill GEMM at M = 2048 on the 14B layer 0: fused QKV and fused gate+up+SwiGLU,
    plus a dense bf16 torch.matmul of each shape (context only)."""
    sh = synth.DENSE_14B
    M, K, I = synth.PREFILL_M, sh.K, sh.I
    x = up(torch, dev, synth.gen_x(synth.CFG_PREFILL, 0, 0, M, K))
    q = torch.empty((M, sh.q_out), dtype=torch.bfloat16, device=dev)
    k = torch.empty((M, sh.kv_out), dtype=torch.bfloat16, device=dev)
    v = torch.empty((M, sh.kv_out), dtype=torch.bfloat16, device=dev)
    h = torch.empty((M, I), dtype=torch.bfloat16, device=dev)
    st = T.stream
    ms_qkv = T.per_call_ms(lambda i: qmm.qmm_fused_qkv(x, pq[0][0], pq[1][0], pq[2][0], q, k, v, stream=st), reps)
    ms_gu = T.per_call_ms(lambda i: qmm.qmm_fused_gate_up_swiglu(x, pg[0][0], pg[1][0], pg[2][0], h, stream=st), reps)
    fl_qkv = 2.0 * M * sh.qkv_rows * K
    fl_gu = 2.0 * M * 2 * I * K

    def dense(N):
        a = torch.randn((M, K), device=dev, dtype=torch.bfloat16)
        b = torch.randn((K, N), device=dev, dtype=torch.bfloat16)  # contiguous [K, N]
        c = torch.empty((M, N), device=dev, dtype=torch.bfloat16)
        ms = T.per_call_ms(lambda i: torch.matmul(a, b, out=c), reps)
        del a, b, c
        return ms

    ms_dq, ms_dg = dense(sh.qkv_rows), dense(2 * I)

    def rec(ms, fl, name):
        tf = fl / (ms * 1e-3) / 1e12
        return {"kernel": name, "avg_launch_us": round(ms * 1e3, 2), "TFLOP/s": round(tf, 1),
                "frac_of_bf16_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4), "flop": fl}

    return {"workload": f"M={M} x K={K}: fused QKV [{sh.qkv_rows} rows] and fused gate+up+SwiGLU "
                        f"[{2 * I} rows], bf16 out, u4 g64 weights of the 14B layer",
            "peak_TFLOPs": BF16_MFMA_PEAK_TFLOPS,
            "fused_qkv": rec(ms_qkv, fl_qkv, "gemm_u4_kernel<QKV>"),
            "fused_gate_up": rec(ms_gu, fl_gu, "gemm_u4_kernel<SWIGLU>"),
            "context_torch_bf16_matmul": {"qkv_shape": rec(ms_dq, fl_qkv, "torch.matmul bf16 (hipBLASLt)"),
                                          "gate_up_shape": rec(ms_dg, fl_gu, "torch.matmul bf16 (hipBLASLt)")}}


def bench_small_batch(torch, qmm, synth, T, dev, pq, pg):
    """Decode of a small batch (M activation rows) on the 14B layer: fused QKV (plain and
    with rotary embedding) and fused gate+up+SwiGLU over the rotating weight pool, per M;
    M = 1 is the GEMV, 2..32 the small-batch kernel, above it whichever of the
    small-batch kernel and the prefill GEMM is estimated faster."""
    sh = synth.DENSE_14B
    rs = synth.ROPE_14B  # the same 7168-row fused QKV, with its rotary layout
    K, I = sh.K, sh.I
    P = pq[0].shape[0]
    st = T.stream
    wbytes = (sh.qkv_rows + 2 * I) * (K // 2 + (K // 64) * 4)
    tab = up(torch, dev, synth.gen_rope_table(synth.ROPE_MAX_POS, rs.rot, rs.base).view(np.int32)).view(torch.float32)
    out = {}
    for M in (1, 2, 4, 8, 16, 32, 64):
        x = up(torch, dev, synth.gen_x(synth.CFG_14B, 0, 0, M, K))
        q = torch.empty((M, sh.q_out), dtype=torch.bfloat16, device=dev)
        k = torch.empty((M, sh.kv_out), dtype=torch.bfloat16, device=dev)
        v = torch.empty((M, sh.kv_out), dtype=torch.bfloat16, device=dev)
        h = torch.empty((M, I), dtype=torch.bfloat16, device=dev)
        ms_q = T.per_call_ms(lambda i: qmm.qmm_fused_qkv(x, pq[0][i % P], pq[1][i % P], pq[2][i % P], q, k, v,
                                                         stream=st), 2 * P)
        ms_g = T.per_call_ms(lambda i: qmm.qmm_fused_gate_up_swiglu(x, pg[0][i % P], pg[1][i % P], pg[2][i % P], h,
                                                                    stream=st), 2 * P)
        pos = torch.from_numpy(synth.gen_positions(synth.CFG_14B, 0, M, synth.ROPE_MAX_POS).astype(np.int32)).to(dev)
        qr, kr, vr = (q.view(M, rs.n_q, rs.head_dim), k.view(M, rs.n_kv, rs.head_dim),
                      v.view(M, rs.n_kv, rs.head_dim))
        ms_r = T.per_call_ms(lambda i: qmm.qmm_fused_qkv_rope(x, pq[0][i % P], pq[1][i % P], pq[2][i % P], qr, kr, vr,
                                                              pos, tab, rs.rot, stream=st), 2 * P)
        us = (ms_q + ms_g) * 1e3
        out[f"M={M}"] = {"qkv_us": round(ms_q * 1e3, 2), "qkv_rope_us": round(ms_r * 1e3, 2),
                         "gate_up_us": round(ms_g * 1e3, 2),
                         "weights_GB/s": round(wbytes / (us * 1e-6) / 1e9, 1),
                         "kernel": "gemv" if M == 1 else ("gemv, two rows" if M == 2
                                                          else "bmv" if M <= 32 else "bmv or gemm (estimate)")}
    return {"workload": "14B layer decode of M sequences: fused QKV [7168 x 5120] + fused gate+up+SwiGLU "
                        "[27648 x 5120], u4 g64, rotating 48-layer pool", **out}


def bench_rope(torch, qmm, synth, T, dev, pq, reps):
    """Fused QKV + split + rotary embedding on the 14B layer shape (40 q / 8 kv heads x 128,
    full rotary), decode M=1 over the rotating weight pool and prefill M=2048, each next
    to the plain fused QKV call on the same weights (the epilogue's cost is the gap)."""
    sh = synth.ROPE_14B
    K, hd = sh.K, sh.head_dim
    P = pq[0].shape[0]
    tab = up(torch, dev, synth.gen_rope_table(synth.ROPE_MAX_POS, sh.rot, sh.base).view(np.int32)).view(torch.float32)
    out = {}
    for M in (1, synth.PREFILL_M):
        x = up(torch, dev, synth.gen_x(synth.CFG_14B, 0, 0, M, K))
        pos = torch.from_numpy(synth.gen_positions(synth.CFG_14B, 0, M, synth.ROPE_MAX_POS)).to(dev)
        q = torch.empty((M, sh.n_q, hd), dtype=torch.bfloat16, device=dev)
        k = torch.empty((M, sh.n_kv, hd), dtype=torch.bfloat16, device=dev)
        v = torch.empty((M, sh.n_kv, hd), dtype=torch.bfloat16, device=dev)
        st = T.stream
        n = 4 * P if M == 1 else reps

        def rope(i):
            l = i % P
            qmm.qmm_fused_qkv_rope(x, pq[0][l], pq[1][l], pq[2][l], q, k, v, pos, tab, sh.rot, stream=st)

        def plain(i):
            l = i % P
            qmm.qmm_fused_qkv(x, pq[0][l], pq[1][l], pq[2][l], q.view(M, -1), k.view(M, -1), v.view(M, -1),
                              stream=st)

        ms_r = T.per_call_ms(rope, n)
        ms_p = T.per_call_ms(plain, n)
        b = weight_bytes(sh.rows, K) + M * K * 2 + M * sh.rows * 2
        fl = 2.0 * M * sh.rows * K
        key = "decode_M1" if M == 1 else f"prefill_M{M}"
        out[key] = {"rope_us": round(ms_r * 1e3, 3), "plain_qkv_us": round(ms_p * 1e3, 3),
                    "rope_over_plain": round(ms_r / ms_p, 4),
                    ("GB/s" if M == 1 else "TFLOP/s"): round((b / (ms_r * 1e-3) / 1e9) if M == 1
                                                             else (fl / (ms_r * 1e-3) / 1e12), 1)}
        del x, q, k, v
    return {"workload": f"fused QKV + RoPE, {sh.n_q} q / {sh.n_kv} kv heads x {hd}, rotary {sh.rot}, "
                        f"K={K}; decode M=1 over a {P}-layer pool and prefill M={synth.PREFILL_M}", **out}


def bench_formats(torch, qmm, synth, T, dev, reps):
    """The other formats of the affine family on the 14B gate+up shape (27648 rows,
    K=5120): decode M=1 (GB/s, over a rotating pool larger than the last-level cache) and
    prefill M=2048 (TFLOP/s), for each code width at group 64 and for u4 at groups 32/128."""
    sh = synth.DENSE_14B
    K, I = sh.K, sh.I
    rows = 2 * I
    out = {}
    x1 = up(torch, dev, synth.gen_x(synth.CFG_14B, 0, 0, 1, K))
    xm = up(torch, dev, synth.gen_x(synth.CFG_14B, 0, 0, synth.PREFILL_M, K))
    h1 = torch.empty((1, I), dtype=torch.bfloat16, device=dev)
    hm = torch.empty((synth.PREFILL_M, I), dtype=torch.bfloat16, device=dev)
    st = T.stream
    for bits, G in ((2, 64), (3, 64), (4, 64), (6, 64), (8, 64), (qmm.QMM_FP8_E4M3, 64), (4, 32), (4, 128)):
        fp8 = bits == qmm.QMM_FP8_E4M3
        w = synth.gen_weight(synth.CFG_14B, 0, synth.PROJ_GATE_UP, rows, K, bits="e4m3" if fp8 else bits, group=G)
        b = rows * K * (8 if fp8 else bits) // 8 + 2 * rows * (K // G) * 2
        P = max(2, -(-768 * 2 ** 20 // b))
        pool = pool_of(torch, dev, w, P)
        del w

        def dec(i):
            l = i % P
            qmm.qmm_fused_gate_up_swiglu_fmt(bits, G, x1, pool[0][l], pool[1][l], pool[2][l], h1, stream=st)

        def pre(i):
            qmm.qmm_fused_gate_up_swiglu_fmt(bits, G, xm, pool[0][0], pool[1][0], pool[2][0], hm, stream=st)

        ms_d = T.per_call_ms(dec, 4 * P)
        ms_p = T.per_call_ms(pre, reps)
        bd = b + K * 2 + I * 2
        fl = 2.0 * synth.PREFILL_M * rows * K
        out[f"fp8e4m3_g{G}" if fp8 else f"u{bits}_g{G}"] = {"bits_per_weight": round(8 * b / (rows * K), 3),
                                "decode_us": round(ms_d * 1e3, 3),
                                "decode_GB/s": round(bd / (ms_d * 1e-3) / 1e9, 1),
                                "prefill_us": round(ms_p * 1e3, 1),
                                "prefill_TFLOP/s": round(fl / (ms_p * 1e-3) / 1e12, 1)}
        del pool
        torch.cuda.empty_cache()
    return {"workload": f"fused gate+up+SwiGLU [{rows} x {K}] in each format: decode M=1 over a pool of "
                        f">= 768 MB, prefill M={synth.PREFILL_M}", **out}


def bench_step_24b(torch, qmm, synth, T, dev, n_steps):
    """24B-dense-shaped decode step: 40 layers of fused QKV + fused gate+up+SwiGLU + down,
    each step with fresh x; a layer's down reads that layer's h.  Run as a planned step
    (two launches: every QKV and gate+up, then every down) and, for comparison, as one
    launch per projection."""
    sh = synth.DENSE_24B
    K, I = sh.K, sh.I
    L = 40
    w_qkv = synth.gen_weight(synth.CFG_24B, 0, synth.PROJ_QKV, sh.qkv_rows, K)
    w_gu = synth.gen_weight(synth.CFG_24B, 0, synth.PROJ_GATE_UP, 2 * I, K)
    w_dn = synth.gen_weight(synth.CFG_24B, 0, synth.PROJ_DOWN, K, I)
    pq, pg, pd = pool_of(torch, dev, w_qkv, L), pool_of(torch, dev, w_gu, L), pool_of(torch, dev, w_dn, L)
    del w_qkv, w_gu, w_dn
    xs = up(torch, dev, np.concatenate([synth.gen_x(synth.CFG_24B, 0, s, 1, K) for s in range(n_steps)]))
    # per-layer outputs: a planned step's outputs may not overlap, and a layer's down reads
    # that layer's h
    qs = torch.empty((L, sh.q_out), dtype=torch.bfloat16, device=dev)
    ks = torch.empty((L, sh.kv_out), dtype=torch.bfloat16, device=dev)
    vs = torch.empty((L, sh.kv_out), dtype=torch.bfloat16, device=dev)
    hs = torch.empty((L, I), dtype=torch.bfloat16, device=dev)
    ys = torch.empty((L, K), dtype=torch.bfloat16, device=dev)
    st = T.stream

    # the planned step: level 0 = every layer's QKV and gate+up (they read x), level 1 =
    # every layer's down (it waits for its layer's gate+up): two launches per step
    plans = []
    for s_ in range(n_steps):
        x = xs[s_]
        pr = []
        for l in range(L):
            pr.append(qmm.step_fused_qkv(x, pq[0][l], pq[1][l], pq[2][l], qs[l], ks[l], vs[l]))
            pr.append(qmm.step_gate_up_swiglu(x, pg[0][l], pg[1][l], pg[2][l], hs[l]))
            pr.append(qmm.step_linear(hs[l], pd[0][l], pd[1][l], pd[2][l], ys[l], wait_for=len(pr) - 1))
        mem = torch.empty(qmm.qmm_step_plan_bytes(pr), dtype=torch.uint8, device=dev)
        qmm.qmm_step_plan(pr, mem, stream=st)
        plans.append((pr, mem))

    def one_step(s_):
        pr, mem = plans[s_ % n_steps]
        qmm.qmm_step_run(pr, mem, stream=st)

    def per_call_step(s_):
        x = xs[s_ % n_steps]
        for l in range(L):
            qmm.qmm_fused_qkv(x, pq[0][l], pq[1][l], pq[2][l], qs[l], ks[l], vs[l], stream=st)
            qmm.qmm_fused_gate_up_swiglu(x, pg[0][l], pg[1][l], pg[2][l], hs[l], stream=st)
            qmm.qmm_linear(hs[l], pd[0][l], pd[1][l], pd[2][l], ys[l], stream=st)

    g = T.capture(one_step, n_steps)
    T.replay_ms(g)
    ms = T.replay_ms(g) / n_steps
    del g
    g = T.capture(per_call_step, n_steps)
    T.replay_ms(g)
    ms_pc = T.replay_ms(g) / n_steps
    del g
    b_qkv = weight_bytes(sh.qkv_rows, K) + K * 2 + sh.qkv_rows * 2
    b_gu = weight_bytes(2 * I, K) + K * 2 + I * 2
    b_dn = weight_bytes(K, I) + I * 2 + K * 2
    b_step = L * (b_qkv + b_gu + b_dn)
    gbs = b_step / (ms * 1e-3) / 1e9
    # each projection on its own (a graph of one kind of call over the 40 layers)
    x0 = xs[0]
    ms_q = T.per_call_ms(lambda i: qmm.qmm_fused_qkv(x0, pq[0][i % L], pq[1][i % L], pq[2][i % L], qs[0], ks[0],
                                                     vs[0], stream=st), 4 * L)
    ms_g = T.per_call_ms(lambda i: qmm.qmm_fused_gate_up_swiglu(x0, pg[0][i % L], pg[1][i % L], pg[2][i % L],
                                                                hs[0], stream=st), 4 * L)
    ms_d = T.per_call_ms(lambda i: qmm.qmm_linear(hs[0], pd[0][i % L], pd[1][i % L], pd[2][i % L], ys[0],
                                                  stream=st), 4 * L)
    kern = {name: {"avg_launch_us": round(t * 1e3, 3), "GB/s": round(b / (t * 1e-3) / 1e9, 1)}
            for name, t, b in (("fused_qkv", ms_q, b_qkv), ("fused_gate_up", ms_g, b_gu), ("down", ms_d, b_dn))}
    return {"workload": f"24B-dense decode step M=1: {L} layers x (QKV [{sh.qkv_rows}x{K}] + gate+up "
                        f"[{2 * I}x{K}] + down [{K}x{I}]), fresh x per step, {n_steps} steps in one graph",
            "ms_per_step": round(ms, 4), "bytes_per_step": b_step, "GB/s": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "launches_per_step": 2,
            "per_call": {"ms_per_step": round(ms_pc, 4), "launches_per_step": 3 * L,
                         "GB/s": round(b_step / (ms_pc * 1e-3) / 1e9, 1)},
            "kernels": kern,
            "per_call_step_over_kernel_sum": round(ms_pc / (L * (ms_q + ms_g + ms_d)), 4)}


def read_ceiling_sequence(torch, dev, T, sizes):
    """The plain streaming read (qmm_ceiling_read) as a sequence of launches of the given
    byte sizes, each on its own slice of a 2 GiB pool, timed like the kernels (a HIP graph):
    microseconds per sequence, best over launch shapes.  The ceiling of a path that is that
    many launches of those sizes."""
    lib = _ceiling_lib()
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    st = T.stream.cuda_stream
    sizes = [(b + 1023) // 1024 * 1024 for b in sizes]
    pool = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    pool.fill_(1)
    per_seq = sum(sizes)
    nseq = (2 << 30) // per_seq
    best = None
    for blocks in (256, 512, 1024, 2048):
        for unroll in (1, 2, 4):
            def fn(i, blocks=blocks, unroll=unroll):
                base = pool.data_ptr() + (i % nseq) * per_seq
                for b in sizes:
                    lib.qmm_ceiling_read(base, b, blocks, unroll, 1, sink.data_ptr(), st)
                    base += b
            us = T.per_call_ms(fn, min(nseq, 200)) * 1e3
            best = us if best is None else min(best, us)
    del pool
    torch.cuda.empty_cache()
    return best


def bench_moe(torch, qmm, synth, T, dev, n_steps):
    """35B-A3B-shaped MoE decode: per layer, stage 1 (gathered gate+up+SwiGLU of the 8
    routed experts) and stage 2 (gathered down + weighted combine), over a 40-layer pool
    of in-place expert grids, fresh routing per step and layer (the layer call
    qmm_moe_layer: two launches)."""
    sh = synth.MOE_35B
    H, E, Ie, topk = sh.hidden, sh.E, sh.I, sh.topk
    L = 40
    g_gu = synth.gen_expert_grid(synth.CFG_MOE, 0, synth.PROJ_MOE_GATE_UP, E, 2 * Ie, H)
    g_dn = synth.gen_expert_grid(synth.CFG_MOE, 0, synth.PROJ_MOE_DOWN, E, H, Ie)
    pgu, pdn = pool_of(torch, dev, g_gu, L), pool_of(torch, dev, g_dn, L)
    del g_gu, g_dn
    ids = np.zeros((n_steps, L, topk), np.int32)
    pw = np.zeros((n_steps, L, topk), np.float32)
    for s in range(n_steps):
        for l in range(L):
            ids[s, l], pw[s, l] = synth.gen_routing(synth.CFG_MOE, l, s, E, topk)
    ids_d = torch.from_numpy(ids).to(dev)
    pw_d = torch.from_numpy(pw).to(dev)
    xs = up(torch, dev, np.concatenate([synth.gen_x(synth.CFG_MOE, 0, s, 1, H) for s in range(n_steps)]))
    hk = torch.empty((topk, Ie), dtype=torch.bfloat16, device=dev)
    y = torch.empty((H,), dtype=torch.bfloat16, device=dev)
    st = T.stream

    def layer_call(s):
        s %= n_steps
        for l in range(L):
            qmm.qmm_moe_layer(xs[s], pgu[0][l], pgu[1][l], pgu[2][l], pdn[0][l], pdn[1][l], pdn[2][l], ids_d[s, l],
                              pw_d[s, l], hk, y, stream=st)

    g = T.capture(layer_call, n_steps)
    T.replay_ms(g)
    ms_layer = T.replay_ms(g) / (n_steps * L)
    del g
    b_layer = (topk * (weight_bytes(2 * Ie, H) + weight_bytes(H, Ie))
               + H * 2 + 2 * topk * Ie * 2 + H * 2 + topk * 8)
    gbs = b_layer / (ms_layer * 1e-3) / 1e9
    b1 = topk * weight_bytes(2 * Ie, H) + H * 2 + topk * Ie * 2 + topk * 4
    ceil_us = read_ceiling_sequence(torch, dev, T, [b1, b_layer - b1])
    return {"workload": f"35B-A3B-shaped MoE decode M=1: top-{topk} of {E} experts, hidden {H}, expert I {Ie}, "
                        f"{L}-layer pool, fresh routing per step and layer, {n_steps} steps in one graph",
            "us_per_layer": round(ms_layer * 1e3, 3), "bytes_per_layer": b_layer, "GB/s": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "launches_per_layer": 2,
            "read_ceiling_two_launches_us": round(ceil_us, 3),
            "frac_of_read_ceiling": round(ceil_us / (ms_layer * 1e3), 4)}


def bench_moe_prefill(torch, qmm, synth, T, dev, reps):
    """35B-A3B-shaped MoE prefill at 2048 tokens: routing, stage 1 (gathered gate+up+SwiGLU
    GEMM) and stage 2 (gathered down GEMM + combine) per layer, over a 4-layer pool of
    in-place expert grids (each layer's grids exceed the last-level cache)."""
    sh = synth.MOE_35B
    H, E, Ie, topk = sh.hidden, sh.E, sh.I, sh.topk
    M = synth.MOE_PREFILL_M
    L = 4
    g_gu = synth.gen_expert_grid(synth.CFG_MOE, 0, synth.PROJ_MOE_GATE_UP, E, 2 * Ie, H)
    g_dn = synth.gen_expert_grid(synth.CFG_MOE, 0, synth.PROJ_MOE_DOWN, E, H, Ie)
    pgu, pdn = pool_of(torch, dev, g_gu, L), pool_of(torch, dev, g_dn, L)
    del g_gu, g_dn
    ids_np, p_np = synth.gen_prefill_routing(synth.CFG_MOE, 0, M, E, topk)
    ids = torch.from_numpy(ids_np).to(dev)
    pw = torch.from_numpy(p_np).to(dev)
    x = up(torch, dev, synth.gen_x(synth.CFG_MOE, 0, 0, M, H))
    h = torch.empty((M, topk, Ie), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(qmm.qmm_moe_prefill_workspace_bytes(M, topk, E, H), dtype=torch.uint8, device=dev)
    st = T.stream

    def route(i):
        qmm.qmm_moe_route(ids, E, ws, stream=st)

    def s1(i):
        l = i % L
        qmm.qmm_moe_prefill(qmm.QMM_MOE_GATE_UP_SWIGLU, x, pgu[0][l], pgu[1][l], pgu[2][l], ids, ws, h, stream=st)

    def s2(i):
        l = i % L
        qmm.qmm_moe_prefill(qmm.QMM_MOE_DOWN_COMBINE, h, pdn[0][l], pdn[1][l], pdn[2][l], ids, ws, y,
                            expert_w=pw, stream=st)

    def layer(i):
        route(i)
        s1(i)
        s2(i)

    route(0)
    torch.cuda.synchronize()
    # one untimed pass of every measurement below first: the first graphs of this leg run
    # 3-8 % slower than the same graphs replayed right after them
    for fn in (route, s1, s2, layer):
        T.per_call_ms(fn, reps)
    ms_route = T.per_call_ms(route, reps)
    ms_s1 = T.per_call_ms(s1, reps)
    ms_s2 = T.per_call_ms(s2, reps)
    ms_layer = T.per_call_ms(layer, reps)
    # smaller batches (the first Ms tokens of the same routing)
    small = {}
    for Ms in (1, 4, 16, 64, 256, 512):
        ids_s, x_s, h_s, y_s, pw_s = ids[:Ms], x[:Ms], h[:Ms], y[:Ms], pw[:Ms]

        def layer_s(i, ids_s=ids_s, x_s=x_s, h_s=h_s, y_s=y_s, pw_s=pw_s):
            l = i % L
            qmm.qmm_moe_route(ids_s, E, ws, stream=st)
            qmm.qmm_moe_prefill(qmm.QMM_MOE_GATE_UP_SWIGLU, x_s, pgu[0][l], pgu[1][l], pgu[2][l], ids_s, ws, h_s,
                                stream=st)
            qmm.qmm_moe_prefill(qmm.QMM_MOE_DOWN_COMBINE, h_s, pdn[0][l], pdn[1][l], pdn[2][l], ids_s, ws, y_s,
                                expert_w=pw_s, stream=st)
        u_s = len(np.unique(ids_np[:Ms]))
        b_s = u_s * (weight_bytes(2 * Ie, H) + weight_bytes(H, Ie))
        ms_s = T.per_call_ms(layer_s, reps)
        small[f"M={Ms}"] = {"us_per_layer": round(ms_s * 1e3, 2), "experts_used": u_s,
                            "expert_weight_GB/s": round(b_s / (ms_s * 1e-3) / 1e9, 1)}
    P = int((ids_np >= 0).sum())
    used = np.unique(ids_np)
    fl1 = 2.0 * P * 2 * Ie * H
    fl2 = 2.0 * P * H * Ie
    b1 = len(used) * weight_bytes(2 * Ie, H) + M * H * 2 + P * Ie * 2
    b2 = len(used) * weight_bytes(H, Ie) + P * Ie * 2 + M * H * 2
    del pgu, pdn

    def rec(ms, fl, b):
        return {"avg_us": round(ms * 1e3, 2), "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 1),
                "GB/s": round(b / (ms * 1e-3) / 1e9, 1), "flop": fl, "bytes": b}

    counts = np.bincount(ids_np.ravel(), minlength=E)
    return {"workload": f"35B-A3B-shaped MoE prefill: {M} tokens x top-{topk} of {E} experts, hidden {H}, "
                        f"expert I {Ie}; pairs per expert min {counts.min()} mean {counts.mean():.0f} "
                        f"max {counts.max()}; {L}-layer pool",
            "us_per_layer": round(ms_layer * 1e3, 2),
            "TFLOP/s_per_layer": round((fl1 + fl2) / (ms_layer * 1e-3) / 1e12, 1),
            "route": {"avg_us": round(ms_route * 1e3, 2)},
            "gate_up_swiglu": rec(ms_s1, fl1, b1),
            "down_combine": rec(ms_s2, fl2, b2),
            "small_batches": {"note": "route + both stages per layer for the first M tokens of the same "
                                      "routing; M * topk <= 288 runs pair by pair on the decode gather "
                                      "kernels, above it the batch is routed onto the weight-stationary "
                                      "gathered kernel", **small}}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(n_steps, w_qkv, w_gu, bytes_step, runs: int = 5):
    """The fp64 oracle, as it stands, on the same layer: one run = n_steps full decode steps
    (fused QKV + fused gate+up+SwiGLU), median of `runs` runs, with BLAS on every available
    core and on one thread.  The oracle's dequantization is NumPy elementwise work (one
    thread); its dot products are BLAS calls, which use the BLAS thread count."""
    from threadpoolctl import threadpool_info, threadpool_limits
    import synth
    from oracle import qmm_oracle as orc

    sh = synth.DENSE_14B
    x = synth.gen_x(synth.CFG_14B, 0, 0, 1, sh.K)
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()

    def timed(threads):
        ts = []
        with threadpool_limits(limits=threads):
            for _ in range(runs):
                t0 = time.perf_counter()
                for _ in range(n_steps):
                    orc.fused_qkv(x, w_qkv.codes, w_qkv.scales, w_qkv.biases, sh.q_out, sh.kv_out)
                    orc.gate_up_swiglu(x, w_gu.codes, w_gu.scales, w_gu.biases, sh.I)
                ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    t_all = timed(avail)
    t_one = timed(1)
    blas = [{"api": d.get("internal_api"), "num_threads": d.get("num_threads")} for d in threadpool_info()]
    gbs_all = bytes_step * n_steps / t_all / 1e9
    gbs_one = bytes_step * n_steps / t_one / 1e9
    return {"value": round(gbs_all, 4), "unit": "GB/s", "cores": avail, "kind": "oracle",
            "sample": f"{n_steps} full 14B-shaped decode steps (fused QKV + gate+up+SwiGLU) per run, fp64 NumPy, "
                      f"median of {runs} runs; BLAS on {avail} threads: {t_all:.2f} s per run",
            "one_thread": {"value": round(gbs_one, 4), "unit": "GB/s", "cores": 1,
                           "seconds_per_run": round(t_one, 3)},
            "seconds_per_run": round(t_all, 3),
            "host": _cpu_model(), "host_cpus": os.cpu_count(), "affinity_cpus": avail, "blas": blas,
            "env": {k: os.environ[k] for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
                    if k in os.environ}}


if __name__ == "__main__":
    main()
