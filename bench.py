#!/usr/bin/env python3
"""Benchmark of the MLA attend-and-combine hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  prefill  B=4, T=4096, 64 heads: rotary prologue + causal flash attention
           (mla_attend_prefill), then o_proj on the [16384, 8192] output;
  decode   B=64, L=8192 cached keys, query at position 8192: split attention +
           merge (mla_attend_decode), then o_proj on the [64, 8192] output.
Inputs are generated on the GPU before the timed region and stay resident.
Every call is timed with HIP events on the stream the library launches on.

Prints ONE JSON line.  `value` is the causal prefill attention throughput
(algorithmic flops 2*(128+64+128)*T(T+1)/2*B*H per call / call time).  The
decode figure (algorithmic bytes: every cached K/V byte once, plus q and the
output / call time) and the o_proj figures sit beside it.
"""
import argparse
import json
import math
import os
import statistics
import sys
import time

REPO = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, REPO)

PEAK_BF16_TFLOPS = 2516.6   # dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBPS = 8000.0      # HBM3E
METRIC = "MLA prefill TFLOP/s (causal) + % bf16 MFMA peak; decode HBM GB/s, 1 GPU"
CSRC = os.path.join(REPO, "transformer_attention_mla_amd", "csrc")

# HBM bytes per launch at this file's workloads, from two rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE) scaled by what the same counters read for a
# copy of known size (FETCH_SIZE counts half the bytes read, WRITE_SIZE all the
# bytes written).  Each figure holds only for the kernel source it was taken on,
# identified by a hash of its files; after any change the figure is dropped.
MEASURED_TRAFFIC = {
    "prefill_kernel": ("627c9cd07391280c", ("mla_prefill.hip", "mla_device.h", "mla_internal.h"),
                       2000857886, "profiles/prefill_kernel_B4_T4096_H64.txt"),
    "decode_split_kernel": ("b78a42ed2d076e13", ("mla_decode.hip", "mla_device.h", "mla_internal.h"),
                            21477804714, "profiles/decode_split_kernel_B64_L8192_H64.txt"),
    "decode_split_kernel_shared_kpe": ("b78a42ed2d076e13", ("mla_decode.hip", "mla_device.h", "mla_internal.h"),
                                       17249596301, "profiles/decode_split_kernel_shared_kpe_B64_L8192_H64.txt"),
    "latent_decode_kernel": ("cb36bcf1f93f9034", ("mla_latent.hip", "mla_device.h", "mla_internal.h"),
                             657394973, "profiles/latent_decode_kernel_B64_L8192_H64.txt"),
}
# o_proj GEMM kernels at K = 8192, N = 7168 (the split-K reduce kernel, shared
# by several paths, is left out), M = 16384 and M = 64.
_OPROJ_SRC = ("2c293fa82d067509", ("mla_oproj.hip", "mla_device.h", "mla_internal.h"))
_OPROJ_PROFILE = "profiles/oproj_kernel_M16384_K8192_N7168_and_M64.txt"
for _k, _v in {"oproj_bf16_M16384": 3204206167, "oproj_bf16_M64": 140699657,
               "oproj_fp8_M16384": 176252089 + 3193876463, "oproj_fp8_M64": 81981659,
               "oproj_fp8_dyn_M16384": 1728777594 + 411079737, "oproj_fp8_dyn_M64": 70560848 + 1647659}.items():
    MEASURED_TRAFFIC[_k] = _OPROJ_SRC + (_v, _OPROJ_PROFILE)


def measured_traffic(kernel):
    import hashlib
    digest, files, nbytes, _ = MEASURED_TRAFFIC[kernel]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return nbytes if h.hexdigest()[:16] == digest else None


def measured_copy_gbps(torch, dev, reps=5):
    """Device copy rate on this GPU: 1 GiB read and 1 GiB written by an
    elementwise kernel, best of a few runs (bytes read + written per second)."""
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.neg(src, out=dst)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del src, dst
    return 2.0 * (1 << 30) / (best * 1e-3) / 1e9


def measured_mfma_tflops(mla, torch, dev, kind=0, reps=5):
    """Matrix-core rate this GPU sustains with every compute unit busy (the
    library's probe: MFMA chains on register operands, no memory traffic;
    kind 0 bf16, kind 1 e4m3 on fixed operands, kinds 2 and 3 the same on
    random operands that change with every instruction), median of a few
    launches of about 5 ms each."""
    iters = 32768 if kind in (0, 2) else 16384
    out = torch.empty(mla.MLA_MFMA_PROBE_OUT, dtype=torch.float32, device=dev)
    mla.mla_mfma_probe(iters, kind, out=out)
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        mla.mla_mfma_probe(iters, kind, out=out)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del out
    return mla.mla_mfma_probe_flops(iters, kind) / (statistics.median(times) * 1e-3) / 1e12


def clock_under_load(fn, torch, seconds=2.5):
    """Graphics clock of the GPU while `fn` (one call of a kernel path) runs back
    to back for about `seconds`: `amd-smi metric -c` sampled from a thread, the
    median over samples of each XCD's current clock.  None when amd-smi is not
    available or reports no clock."""
    import json
    import shutil
    import subprocess
    import threading

    smi = shutil.which("amd-smi") or ("/opt/rocm/bin/amd-smi" if os.path.exists("/opt/rocm/bin/amd-smi") else None)
    if smi is None:
        return None
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            try:
                r = subprocess.run([smi, "metric", "-g", "0", "-c", "--json"], capture_output=True,
                                   text=True, timeout=30)
                clk = json.loads(r.stdout)["gpu_data"][0]["clock"]
                xcd = [v["clk"]["value"] for k, v in sorted(clk.items()) if k.startswith("gfx_")]
                if xcd and all(isinstance(x, (int, float)) for x in xcd):
                    samples.append(xcd)
            except Exception:
                return

    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    th = threading.Thread(target=poll, daemon=True)
    t0 = time.perf_counter()
    th.start()
    while time.perf_counter() - t0 < seconds or (not samples and time.perf_counter() - t0 < 4 * seconds):
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=60)
    if len(samples) < 2:
        return None
    samples = samples[1:]  # the first sample may straddle the start of the load
    per_xcd = [statistics.median(col) for col in zip(*samples)]
    return {"mhz_median": statistics.median(per_xcd), "mhz_per_xcd": per_xcd, "samples": len(samples),
            "source": "amd-smi metric -c (current gfx clock per XCD), sampled while the call repeats"}


class Timer:
    """Median call time with HIP events on the current stream, warm and cold.

    warm: back-to-back calls (inputs and weights may sit in the 256 MB MALL and
    the L2s).  cold: before each timed call, outside the event pair, a 512 MB
    scratch buffer is written, which evicts the MALL and the L2s, so the call
    reads its inputs and weights from HBM -- and also leaves the caches full of
    dirty lines, whose write-back the call's reads then pay for.  cold_clean:
    the same write, then a read of a second 512 MB buffer (a sum), so the
    caches hold neither the call's inputs nor dirty lines."""

    def __init__(self, torch, dev):
        self.torch = torch
        self.scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        self.clean = torch.ones(64 << 20, dtype=torch.float64, device=dev)  # 512 MB
        self.sink = torch.empty((), dtype=torch.float64, device=dev)

    def flush(self, clean=False):
        self.scratch.fill_(1)
        if clean:
            self.torch.sum(self.clean, 0, out=self.sink)

    def median(self, fn, calls, cold=False, untimed=3, clean=False):
        torch = self.torch
        for _ in range(untimed):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(calls)]
        for a, b in ev:
            if cold:
                self.flush(clean)
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in ev)
        return t[len(t) // 2]

    def both(self, fn, calls):
        return {"cold": self.median(fn, calls, cold=True),
                "cold_clean": self.median(fn, calls, cold=True, clean=True),
                "warm": self.median(fn, calls)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def prefill_flops(B, H, T):
    return 2.0 * (128 + 64 + 128) * T * (T + 1) / 2 * B * H


def decode_bytes(B, H, L):
    return B * H * (L * (192 + 128) * 2 + (128 + 64) * 2 + 128 * 2)


def oproj_flops(M, K, N):
    return 2.0 * M * K * N


def oproj_bytes(M, K, N):
    return (M * K + N * K + M * N) * 2


def cpu_baseline(d, B, H, T, R, scale, budget_s):
    """Time the oracle on a bounded sample of the prefill workload: every row
    of the first n (sequence, head) units in sequence-major order, n chosen
    from a one-unit calibration so the sample takes about budget_s seconds."""
    import numpy as np
    import oracle
    from transformer_attention_mla_amd import inputs

    threads = oracle.default_threads()
    cache = {}

    def seq_inputs(nb):
        if nb not in cache:
            sl = lambda t: inputs.bits(t[0:nb])
            cache.clear()
            cache[nb] = (sl(d["q_nope"]), sl(d["q_pe"]), sl(d["k_nope"]), sl(d["k_pe"]), sl(d["v"]))
        return cache[nb]

    def run(n):
        nb = (n + H - 1) // H
        qn, qp, kn, kp, v = seq_inputs(nb)
        units = np.arange(n, dtype=np.int32)
        sel = np.stack([np.repeat(units // H, T), np.repeat(units % H, T),
                        np.tile(np.arange(T, dtype=np.int32), n)], 1).astype(np.int32)
        t0 = time.perf_counter()
        oracle.prefill_rows(qn, qp, kn, kp, v, R, scale, sel, nthreads=threads)
        return time.perf_counter() - t0

    t1 = run(1)
    n = max(1, min(B * H, int(budget_s / max(t1, 1e-3))))
    tn = t1 if n == 1 else run(n)
    flops = prefill_flops(1, n, T)
    last_b, last_h = (n - 1) // H, (n - 1) % H
    return {"value": flops / tn / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"every row of the first {n} (sequence, head) units in sequence-major order "
                      f"(through sequence {last_b}, head {last_h}) of the B={B} T={T} H={H} "
                      f"workload; {flops / 1e9:.1f} GFLOP in {tn:.2f} s, fp64",
            "seconds": round(tn, 3)}


def cpu_baseline_decode(dd, Bd, Hd, L, q_pos, R, scale, budget_s):
    """Time the oracle's decode on a bounded sample of the decode workload:
    every head of the first nb sequences, nb chosen from a one-sequence
    calibration for about budget_s seconds (all of them when the whole
    workload takes less, as it does on a many-core host: the oracle streams
    the 21.5 GB cache in well under a second); GB/s on the same algorithmic
    bytes as the GPU figure (every cached key and value byte of those
    (sequence, head) units once, plus q and the output)."""
    import numpy as np
    import oracle
    from transformer_attention_mla_amd import inputs

    threads = oracle.default_threads()

    def run(nb):
        sl = lambda t: inputs.bits(t[0:nb])
        qn, qp, kc, vc = sl(dd["q_nope"]), sl(dd["q_pe"]), sl(dd["k_cache"]), sl(dd["v_cache"])
        sel = np.stack([np.repeat(np.arange(nb, dtype=np.int32), Hd),
                        np.tile(np.arange(Hd, dtype=np.int32), nb)], 1).astype(np.int32)
        t0 = time.perf_counter()
        oracle.decode_rows(qn, qp, kc, vc, R, q_pos, scale, sel, nthreads=threads)
        return time.perf_counter() - t0

    t1 = run(1)
    nb = max(1, min(Bd, int(budget_s / max(t1, 1e-3))))
    tn = t1 if nb == 1 else run(nb)
    nbytes = decode_bytes(nb, Hd, L)
    return {"value": nbytes / tn / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"all {Hd} heads of the first {nb} sequences of the B={Bd} L={L} decode "
                      f"workload; {nbytes / 1e9:.2f} GB of cached keys and values in {tn:.2f} s, "
                      f"fp64", "seconds": round(tn, 3)}


def other_configs(mla, inputs, w_o, scale, dev, timer):
    """Prefill attention and o_proj at the other prefill workloads (T = 64,
    1024 with plain rotary angles; T = 16384 with the YaRN table), each call
    timed with HIP events after 3 untimed ones; median per call, cold (MALL
    and L2 flushed before each call) and warm (back to back); 200 calls at
    T <= 1024, 10 at T = 16384.  Reported beside the main line, not part of
    it."""
    import torch

    out = {}
    for w in (1, 2, 4):
        wl = inputs.WORKLOADS[w]
        B, H, T = wl["B"], wl["H"], wl["T"]
        print(f"other config: workload {w} (B={B} T={T})", file=sys.stderr, flush=True)
        d = inputs.prefill_inputs(B, H, T, workload=w, device=dev)
        d["v"] = inputs.to_v_blocked(d["v"])  # the layout mla_up_project writes with MLA_V_BLOCKED
        o = torch.empty((B, T, H * 128), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(mla.mla_prefill_workspace_bytes(B, H, T), dtype=torch.uint8, device=dev)
        M, K_O, N_O = B * T, H * 128, w_o.shape[0]
        y = torch.empty((M, N_O), dtype=torch.bfloat16, device=dev)
        ws_o = torch.empty(max(16, mla.mla_out_proj_workspace_bytes(M, K_O, N_O)), dtype=torch.uint8,
                           device=dev)
        fa = lambda: mla.mla_attend_prefill(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"],
                                            d["R"], scale, out=o, workspace=ws, v_blocked=True)
        fo = lambda: mla.mla_out_proj(o.view(M, K_O), w_o, y=y, workspace=ws_o)

        calls = 200 if T <= 1024 else 10
        ta, to = timer.both(fa, calls), timer.both(fo, calls)
        fl_a, fl_o = prefill_flops(B, H, T), oproj_flops(M, K_O, N_O)
        ob = oproj_bytes(M, K_O, N_O)
        out[f"prefill_B{B}_T{T}_H{H}"] = {
            "attention_ms": ta["cold"], "attention_ms_cold_clean": ta["cold_clean"],
            "attention_ms_warm": ta["warm"],
            "attention_tflops": fl_a / ta["cold"] / 1e9,
            "attention_tflops_warm": fl_a / ta["warm"] / 1e9,
            "attention_frac_peak": fl_a / ta["cold"] / 1e9 / PEAK_BF16_TFLOPS,
            "oproj_ms_cold": to["cold"], "oproj_ms_cold_clean": to["cold_clean"], "oproj_ms_warm": to["warm"],
            "oproj_tflops_cold": fl_o / to["cold"] / 1e9, "oproj_tflops_warm": fl_o / to["warm"] / 1e9,
            "oproj_gbps_cold": ob / to["cold"] / 1e6, "oproj_gbps_warm": ob / to["warm"] / 1e6,
            "calls": calls, "rope": wl["rope"]}
        del d, o, ws, y, ws_o
        torch.cuda.empty_cache()
    # A chunk of 4096 positions after 12288 cached ones (64 heads): append the
    # chunk's keys into the shared-rotary cache, then attend over all 16384.
    B, H, T, past = 1, 64, 4096, 12288
    L = past + T
    print(f"other config: chunked prefill (T={T} after {past})", file=sys.stderr, flush=True)
    c = inputs.chunk_inputs(B, H, T, past, seed=7000, device=dev)
    q_nope, q_pe, k_nope, k_pe, v = (c[k] for k in ("q_nope", "q_pe", "k_nope", "k_pe", "v"))
    kc, pc, vc, R = c["k_nope_cache"], c["kpe_cache"], c["v_cache"], c["R"]
    o = torch.empty((B, T, H * 128), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(mla.mla_prefill_chunk_workspace_bytes(T), dtype=torch.uint8, device=dev)
    fapp = lambda: mla.mla_append_kv(k_nope, k_pe, v, R, past, kc, pc, vc)
    fatt = lambda: mla.mla_attend_prefill_chunk(q_nope, q_pe, kc, pc, vc, R, past, scale, out=o,
                                                workspace=ws)
    tapp, tatt = timer.median(fapp, 10), timer.median(fatt, 10)
    fl = 2.0 * (128 + 64 + 128) * B * H * (T * past + T * (T + 1) / 2)
    out[f"prefill_chunk_B{B}_T{T}_past{past}_H{H}"] = {
        "append_ms": tapp, "attention_ms": tatt, "attention_tflops": fl / tatt / 1e9,
        "attention_frac_peak": fl / tatt / 1e9 / PEAK_BF16_TFLOPS}
    del c, q_nope, q_pe, k_nope, k_pe, v, kc, pc, vc, o, ws
    torch.cuda.empty_cache()
    # The up-projection in front of the prefill at B=4, T=4096, 64 heads: q
    # from the rank-1536 latent, nope key and value from the rank-512 latent.
    B, T, H = 4, 4096, 64
    print(f"other config: up-projection (B={B} T={T})", file=sys.stderr, flush=True)
    d = inputs.up_project_inputs(B, T, H, workload=3, device=dev)
    outs = [torch.empty((B, H, T, w), dtype=torch.bfloat16, device=dev) for w in (128, 64, 128)]
    outs.append(torch.empty((B, H, (T + 15) // 16, 128, 16), dtype=torch.bfloat16, device=dev))
    fup = lambda: mla.mla_up_project(d["q_lat"], d["ckv"], d["w_q_b"], d["w_kv_b"], outs=outs,
                                     v_blocked=True)
    tup = timer.both(fup, 10)
    fl = 2.0 * B * T * (1536 * H * 192 + 512 * H * 256)
    nbytes = 2 * (B * T * (1536 + 512) + H * 192 * 1536 + H * 256 * 512 + B * H * T * (128 + 64 + 128 + 128))
    out[f"up_project_B{B}_T{T}_H{H}"] = {
        "ms_cold": tup["cold"], "ms_cold_clean": tup["cold_clean"], "ms_warm": tup["warm"], "tflops_cold": fl / tup["cold"] / 1e9,
        "tflops_warm": fl / tup["warm"] / 1e9, "frac_peak_cold": fl / tup["cold"] / 1e9 / PEAK_BF16_TFLOPS,
        "hbm_gbps_cold": nbytes / tup["cold"] / 1e6, "per_call": f"{fl:.4e} flops, {nbytes} bytes"}
    del d, outs
    torch.cuda.empty_cache()
    # Attention feeding the FP8 o_proj at B=4, T=4096, 64 heads: the bf16
    # output quantized by a separate pass (mla_attend_prefill, then
    # mla_out_proj_fp8_dyn), against the output quantized in the attention's
    # epilogue (mla_attend_prefill_fp8, then mla_out_proj_fp8_q).
    B, H, T = 4, 64, 4096
    M, K_O = B * T, H * 128
    print(f"other config: attention -> FP8 o_proj (B={B} T={T})", file=sys.stderr, flush=True)
    d = inputs.prefill_inputs(B, H, T, workload=3, device=dev)
    w8, sc = inputs.out_proj_weight_fp8(inputs.D_MODEL, K_O, workload=3, device=dev)
    N_O = w8.shape[0]
    ws = torch.empty(mla.mla_prefill_workspace_bytes(B, H, T), dtype=torch.uint8, device=dev)
    o16 = torch.empty((B, T, K_O), dtype=torch.bfloat16, device=dev)
    o8 = torch.empty((B, T, K_O), dtype=torch.uint8, device=dev)
    osT = torch.empty((H, mla.mla_act_scale_stride(M)), dtype=torch.float32, device=dev)
    y = torch.empty((M, N_O), dtype=torch.bfloat16, device=dev)
    ws_d = torch.empty(max(16, mla.mla_out_proj_fp8_dyn_workspace_bytes(M, K_O, N_O)), dtype=torch.uint8,
                       device=dev)
    args = (d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], inputs.to_v_blocked(d["v"]), d["R"], scale)
    fa16 = lambda: mla.mla_attend_prefill(*args, out=o16, workspace=ws, v_blocked=True)
    fdyn = lambda: mla.mla_out_proj_fp8_dyn(o16.view(M, K_O), w8, sc, y=y, workspace=ws_d)
    fa8 = lambda: mla.mla_attend_prefill_fp8(*args, out8=o8, out_scaleT=osT, workspace=ws,
                                             v_blocked=True)
    fq = lambda: mla.mla_out_proj_fp8_q(o8.view(M, K_O), osT, w8, sc, y=y)
    # the four calls interleaved, 10 rounds after 3 untimed ones; median per call
    fns = (fa16, fdyn, fa8, fq)
    for _ in range(3):
        for f in fns:
            f()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
          for _ in range(10)]
    for row in ev:
        for (a, b), f in zip(row, fns):
            a.record()
            f()
            b.record()
    torch.cuda.synchronize()
    t16, tdyn, t8, tq = (statistics.median(row[i][0].elapsed_time(row[i][1]) for row in ev)
                         for i in range(len(fns)))
    fl_a, fl_o = prefill_flops(B, H, T), oproj_flops(M, K_O, N_O)
    out[f"attention_to_fp8_oproj_B{B}_T{T}_H{H}"] = {
        "separate_quantization_ms": {"attention": t16, "oproj_fp8_dyn": tdyn, "total": t16 + tdyn},
        "quantized_in_epilogue_ms": {"attention_fp8_out": t8, "oproj_fp8_q": tq, "total": t8 + tq},
        "total_tflops": {"separate": (fl_a + fl_o) / (t16 + tdyn) / 1e9,
                         "in_epilogue": (fl_a + fl_o) / (t8 + tq) / 1e9}}
    del d, w8, sc, ws, o16, o8, osT, y, ws_d
    torch.cuda.empty_cache()
    return out


def decode_shared_kpe_bytes(B, H, L):
    return B * H * L * (128 + 128) * 2 + B * L * 64 * 2 + B * H * ((128 + 64) * 2 + 128 * 2)


def decode_shared_kpe_figures(mla, inputs, scale, dev, calls=10):
    """Decode at B=64, H=64, L=8192 with the shared-rotary cache layout (nope
    keys per head, one rotated rope key per position for all heads): median
    call time and HBM rate on its algorithmic bytes (every cached byte once,
    q in, output out).  Reported beside the main line, not part of it."""
    import torch

    wd = inputs.WORKLOADS[5]
    B, H, L, q_pos = wd["B"], wd["H"], wd["L"], wd["q_pos"]
    print("decode, shared-rotary cache layout", file=sys.stderr, flush=True)
    d = inputs.decode_shared_kpe_inputs(B, H, L, q_pos, workload=5, device=dev)
    out = torch.empty((B, H * 128), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(16, mla.mla_decode_workspace_bytes(B, H, L, 0)), dtype=torch.uint8,
                     device=dev)
    f = lambda: mla.mla_attend_decode_shared_kpe(d["q_nope"], d["q_pe"], d["k_nope_cache"],
                                                 d["kpe_cache"], d["v_cache"], d["R"], q_pos, scale,
                                                 out=out, workspace=ws)
    for _ in range(3):
        f()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(calls)]
    for a, b in ev:
        a.record()
        f()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)[calls // 2]
    nb = decode_shared_kpe_bytes(B, H, L)
    del d
    torch.cuda.empty_cache()
    return {"workload": f"decode B={B} L={L} H={H} q_pos={q_pos}, k_nope [B,H,L,128] + shared "
                        f"rotated k_pe [B,L,64] + V [B,H,L,128]",
            "attention_ms": t, "hbm_gbps": nb / t / 1e6, "frac_hbm": nb / t / 1e6 / PEAK_HBM_GBPS,
            "per_launch": f"{nb} bytes",
            "traffic": measured_traffic("decode_split_kernel_shared_kpe")}


def decode_latent_bytes(B, H, L):
    """Every cached byte once (latent 512 + rotated rope key 64 per position),
    kv_b_proj once, queries in, outputs out."""
    return B * L * (512 + 64) * 2 + H * 256 * 512 * 2 + B * H * ((128 + 64) * 2 + 128 * 2)


def decode_latent_flops(B, H, L):
    """Scores over 576 dims and the mix over 512 per (head, position), plus the
    query absorption (128 x 512) and the value expansion (512 x 128) per head."""
    return 2.0 * B * H * (L * (576 + 512) + 2 * 128 * 512)


def decode_latent_figures(mla, inputs, scale, dev, calls=20):
    """Decode at B=64, H=64, L=8192 against the latent cache (512-wide latent
    and the rotated rope key per position, kv_b_proj [64*256, 512]): median
    call time of the whole entry point (absorb, attend, merge, expand) and its
    rates on the algorithmic bytes and flops.  Reported beside the main line."""
    import torch

    wd = inputs.WORKLOADS[5]
    B, H, L, q_pos = wd["B"], wd["H"], wd["L"], wd["q_pos"]
    print("decode, latent cache", file=sys.stderr, flush=True)
    d = inputs.decode_latent_inputs(B, H, L, q_pos, workload=5, device=dev)
    out = torch.empty((B, H * 128), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(mla.mla_decode_latent_workspace_bytes(B, H, L, 0), dtype=torch.uint8,
                     device=dev)
    f = lambda: mla.mla_attend_decode_latent(d["q_nope"], d["q_pe"], d["ckv"], d["kpe"],
                                             d["w_kv_b"], d["R"], q_pos, scale, out=out,
                                             workspace=ws)
    for _ in range(3):
        f()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(calls)]
    for a, b in ev:
        a.record()
        f()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)[calls // 2]
    nb, nf = decode_latent_bytes(B, H, L), decode_latent_flops(B, H, L)
    del d
    torch.cuda.empty_cache()
    return {"workload": f"decode B={B} L={L} H={H} q_pos={q_pos}, latent cache [B,L,512] + "
                        f"rotated k_pe [B,L,64], kv_b_proj [{H * 256},512]",
            "call_ms": t, "hbm_gbps": nb / t / 1e6, "frac_hbm": nb / t / 1e6 / PEAK_HBM_GBPS,
            "tflops": nf / t / 1e9, "per_call": f"{nb} bytes, {nf:.4e} flops",
            "traffic": measured_traffic("latent_decode_kernel")}


def oproj_figures(mla, inputs, w_o, dev, timer, calls=20):
    """o_proj with the bf16 weight at M = 64 (decode) and M = 16384 (prefill),
    timed alone: median time cold (MALL and L2 flushed before each call) and
    warm (back to back), GB/s on x + w + y, TFLOP/s."""
    import torch

    N, K = w_o.shape
    res = {}
    for M in (64, 16384):
        print(f"o_proj bf16 M={M}", file=sys.stderr, flush=True)
        x = inputs.normal_bf16((M, K), 90 + M, device=dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(16, mla.mla_out_proj_workspace_bytes(M, K, N)), dtype=torch.uint8,
                         device=dev)
        t = timer.both(lambda: mla.mla_out_proj(x, w_o, y=y, workspace=ws), calls)
        nb = oproj_bytes(M, K, N)
        res[f"M{M}"] = {"ms_cold": t["cold"], "ms_cold_clean": t["cold_clean"], "ms_warm": t["warm"],
                        "gbps_cold": nb / t["cold"] / 1e6, "gbps_warm": nb / t["warm"] / 1e6,
                        "tflops_cold": oproj_flops(M, K, N) / t["cold"] / 1e9,
                        "tflops_warm": oproj_flops(M, K, N) / t["warm"] / 1e9, "bytes": nb,
                        "traffic": measured_traffic(f"oproj_bf16_M{M}") if N == 7168 and K == 8192 else None}
        del x, y, ws
    torch.cuda.empty_cache()
    return res


def oproj_fp8_figures(mla, inputs, dev, timer, calls=20):
    """o_proj with the FP8 checkpoint weight ([7168, 8192] e4m3 + float32 block
    scales; at M = 64 (decode) dequantized to bf16 as it is loaded, at M =
    16384 (prefill) dequantized once per call into the workspace before the
    bf16 product): median time cold and warm, GB/s on x + w8 + scales + y,
    TFLOP/s."""
    import torch

    K, N = 64 * 128, inputs.D_MODEL
    w8, sc = inputs.out_proj_weight_fp8(N, K, workload=3, device=dev)
    res = {}
    for M in (64, 16384):
        print(f"o_proj fp8 M={M}", file=sys.stderr, flush=True)
        x = inputs.normal_bf16((M, K), 90 + M, device=dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(16, mla.mla_out_proj_fp8_workspace_bytes(M, K, N)), dtype=torch.uint8,
                         device=dev)
        f = lambda: mla.mla_out_proj_fp8(x, w8, sc, y=y, workspace=ws)
        t = timer.both(f, calls)
        nb = M * K * 2 + N * K + sc.numel() * 4 + M * N * 2
        res[f"M{M}"] = {"ms_cold": t["cold"], "ms_cold_clean": t["cold_clean"], "ms_warm": t["warm"],
                        "gbps_cold": nb / t["cold"] / 1e6, "gbps_warm": nb / t["warm"] / 1e6,
                        "tflops_cold": oproj_flops(M, K, N) / t["cold"] / 1e9,
                        "tflops_warm": oproj_flops(M, K, N) / t["warm"] / 1e9, "bytes": nb,
                        "traffic": measured_traffic(f"oproj_fp8_M{M}")}
        del x, y, ws
    del w8, sc
    torch.cuda.empty_cache()
    return res


def oproj_fp8_dyn_figures(mla, inputs, dev, timer, calls=20):
    """o_proj with FP8 activations and the FP8 checkpoint weight on the FP8
    matrix cores (x quantized per row and 128-column block, then the e4m3 x
    e4m3 product with both block scales applied per 128-deep slab), at M = 64
    and M = 16384: the whole call (both kernels), median time cold and warm;
    GB/s on x + w8 + scales + y (the algorithmic bytes: the quantized copy of
    x is an intermediate), TFLOP/s."""
    import torch

    K, N = 64 * 128, inputs.D_MODEL
    w8, sc = inputs.out_proj_weight_fp8(N, K, workload=3, device=dev)
    res = {}
    for M in (64, 16384):
        print(f"o_proj fp8 dynamic M={M}", file=sys.stderr, flush=True)
        x = inputs.normal_bf16((M, K), 90 + M, device=dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(16, mla.mla_out_proj_fp8_dyn_workspace_bytes(M, K, N)),
                         dtype=torch.uint8, device=dev)
        f = lambda: mla.mla_out_proj_fp8_dyn(x, w8, sc, y=y, workspace=ws)
        t = timer.both(f, calls)
        nb = M * K * 2 + N * K + sc.numel() * 4 + M * N * 2
        res[f"M{M}"] = {"ms_cold": t["cold"], "ms_cold_clean": t["cold_clean"], "ms_warm": t["warm"],
                        "gbps_cold": nb / t["cold"] / 1e6, "gbps_warm": nb / t["warm"] / 1e6,
                        "tflops_cold": oproj_flops(M, K, N) / t["cold"] / 1e9,
                        "tflops_warm": oproj_flops(M, K, N) / t["warm"] / 1e9, "bytes": nb,
                        "traffic": measured_traffic(f"oproj_fp8_dyn_M{M}"),
                        "traffic_note": "quantization kernel + GEMM kernel per call (the split-K "
                                        "reduce at M = 64 not included)"}
        del x, y, ws
    del w8, sc
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--decode-splits", type=int, default=0)
    ap.add_argument("--only", choices=["prefill", "decode", "all"], default="all")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the extra figures: prefill at T=64, 1024 and 16384, and decode "
                         "with the shared-rotary cache layout")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip sampling the graphics clock (amd-smi) under the prefill and the probe "
                         "(--no-other-configs skips it as well)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="before the steps, run a plain streaming kernel over 1 GiB (read 1 GiB, "
                         "write 1 GiB) three times, to scale hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path to measure (heads and sequences would shard with one exchange after "
              "o_proj).", file=sys.stderr)
        sys.exit(2)

    import torch
    import transformer_attention_mla_amd as mla
    from transformer_attention_mla_amd import inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    scale = float(inputs.SOFTMAX_SCALE)
    wp, wd = inputs.WORKLOADS[3], inputs.WORKLOADS[5]
    B, H, T = wp["B"], wp["H"], wp["T"]
    Bd, Hd, L, q_pos = wd["B"], wd["H"], wd["L"], wd["q_pos"]
    K_O, N_O = H * 128, inputs.D_MODEL
    do_p = args.only in ("prefill", "all")
    do_d = args.only in ("decode", "all")

    # ---- inputs, resident in HBM before timing
    print("generating inputs", file=sys.stderr, flush=True)
    w_o = inputs.out_proj_weight(N_O, K_O, workload=3, device=dev)
    if do_p:
        d = inputs.prefill_inputs(B, H, T, workload=3, device=dev)
        # values key-blocked, as mla_up_project writes them with MLA_V_BLOCKED (the
        # oracle leg below takes the same values in [B, H, T, 128])
        v_blk = inputs.to_v_blocked(d["v"])
        attn_out = torch.empty((B, T, H * 128), dtype=torch.bfloat16, device=dev)
        y_p = torch.empty((B * T, N_O), dtype=torch.bfloat16, device=dev)
        ws_p = torch.empty(mla.mla_prefill_workspace_bytes(B, H, T), dtype=torch.uint8, device=dev)
        ws_op = torch.empty(max(16, mla.mla_out_proj_workspace_bytes(B * T, K_O, N_O)),
                            dtype=torch.uint8, device=dev)
    if do_d:
        dd = inputs.decode_inputs(Bd, Hd, L, q_pos, workload=5, device=dev)
        dec_out = torch.empty((Bd, Hd * 128), dtype=torch.bfloat16, device=dev)
        y_d = torch.empty((Bd, N_O), dtype=torch.bfloat16, device=dev)
        ws_d = torch.empty(max(16, mla.mla_decode_workspace_bytes(Bd, Hd, L, args.decode_splits)),
                           dtype=torch.uint8, device=dev)
        ws_od = torch.empty(max(16, mla.mla_out_proj_workspace_bytes(Bd, K_O, N_O)),
                            dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    names = []
    if do_p:
        names += ["prefill_attention", "prefill_oproj"]
    if do_d:
        names += ["decode_attention", "decode_oproj"]
    n_ev = args.steps
    ev = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n_ev)] for k in names}

    def step(i=None):
        def timed(name, fn):
            if i is not None:
                ev[name][i][0].record()
            fn()
            if i is not None:
                ev[name][i][1].record()
        if do_p:
            timed("prefill_attention", lambda: mla.mla_attend_prefill(
                d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], v_blk, d["R"], scale,
                out=attn_out, workspace=ws_p, v_blocked=True))
            timed("prefill_oproj", lambda: mla.mla_out_proj(
                attn_out.view(B * T, K_O), w_o, y=y_p, workspace=ws_op))
        if do_d:
            timed("decode_attention", lambda: mla.mla_attend_decode(
                dd["q_nope"], dd["q_pe"], dd["k_cache"], dd["v_cache"], dd["R"], q_pos, scale,
                num_splits=args.decode_splits, out=dec_out, workspace=ws_d))
            timed("decode_oproj", lambda: mla.mla_out_proj(dec_out, w_o, y=y_d, workspace=ws_od))

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    print("warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("timing", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {k: sorted(a.elapsed_time(b) for a, b in ev[k]) for k in names}
    avg = {k: sum(v) / len(v) for k, v in ms.items()}
    med = {k: v[len(v) // 2] for k, v in ms.items()}
    print("timed: " + ", ".join(f"{k} {avg[k]:.3f} ms" for k in names), file=sys.stderr, flush=True)

    res = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    cfg = {"workload": "", "heads": H}
    parts = []
    if do_p:
        fa = prefill_flops(B, H, T)
        fo = oproj_flops(B * T, K_O, N_O)
        ta = avg["prefill_attention"] / 1e3
        to = avg["prefill_oproj"] / 1e3
        res["value"] = fa / ta / 1e12
        res["unit"] = "TFLOP/s"
        res["prefill"] = {
            "attention_ms": avg["prefill_attention"], "attention_ms_median": med["prefill_attention"],
            "attention_tflops": fa / ta / 1e12, "attention_frac_peak": fa / ta / 1e12 / PEAK_BF16_TFLOPS,
            "oproj_ms": avg["prefill_oproj"], "oproj_tflops": fo / to / 1e12,
            "oproj_frac_peak": fo / to / 1e12 / PEAK_BF16_TFLOPS,
            "attention_plus_oproj_tflops": (fa + fo) / (ta + to) / 1e12}
        mfma_fixed = measured_mfma_tflops(mla, torch, dev, kind=0)
        mfma_tf = measured_mfma_tflops(mla, torch, dev, kind=2)
        res["measured_mfma_tflops"] = {
            "bf16_random_operands": mfma_tf, "bf16": mfma_fixed,
            "fp8_e4m3_random_operands": measured_mfma_tflops(mla, torch, dev, kind=3),
            "fp8_e4m3": measured_mfma_tflops(mla, torch, dev, kind=1)}
        if not (args.no_clock or args.no_other_configs):  # the profiled runs leave it out too
            probe_out = torch.empty(mla.MLA_MFMA_PROBE_OUT, dtype=torch.float32, device=dev)
            res["clock_under_load"] = {
                "prefill_attention": clock_under_load(lambda: mla.mla_attend_prefill(
                    d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], v_blk, d["R"], scale,
                    out=attn_out, workspace=ws_p, v_blocked=True), torch),
                "mfma_probe_bf16": clock_under_load(lambda: mla.mla_mfma_probe(32768, 0, out=probe_out), torch),
                "mfma_probe_bf16_random_operands": clock_under_load(
                    lambda: mla.mla_mfma_probe(32768, 2, out=probe_out), torch)}
            del probe_out
        res["prefill"]["exp_count"] = B * H * T * (T + 1) // 2
        res["roofline"] = {"bound": "mfma", "achieved": fa / ta / 1e12, "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": fa / ta / 1e12 / PEAK_BF16_TFLOPS,
                           "traffic": measured_traffic("prefill_kernel"),
                           "kernel": "prefill_kernel (+ rope_prep_kernel)",
                           "per_launch": f"{fa:.4e} causal flops",
                           "measured_mfma_tflops": mfma_tf,
                           "measured_mfma_operands": "random, changing with every instruction (probe kind 2)",
                           "frac_of_measured_mfma": fa / ta / 1e12 / mfma_tf,
                           "measured_mfma_tflops_fixed_operands": mfma_fixed}
        parts.append(f"prefill B={B} T={T} H={H} causal + o_proj [{B * T}x{K_O}]x[{K_O}x{N_O}]")
        cfg.update({"prefill_batch": B, "prefill_seq_len": T,
                    "prefill_v_layout": "key-blocked [B,H,T/16,128,16] (MLA_V_BLOCKED)"})
    if do_d:
        bd = decode_bytes(Bd, Hd, L)
        td = avg["decode_attention"] / 1e3
        tod = avg["decode_oproj"] / 1e3
        bo = oproj_bytes(Bd, K_O, N_O)
        res["decode"] = {
            "attention_ms": avg["decode_attention"], "attention_ms_median": med["decode_attention"],
            "hbm_gbps": bd / td / 1e9, "frac_hbm": bd / td / 1e9 / PEAK_HBM_GBPS,
            "splits": mla.mla_decode_splits(Bd, Hd, L, args.decode_splits),
            "oproj_ms": avg["decode_oproj"], "oproj_gbps": bo / tod / 1e9}
        copy_gbps = measured_copy_gbps(torch, dev)
        res["roofline_decode"] = {"bound": "hbm", "achieved": bd / td / 1e9, "peak": PEAK_HBM_GBPS,
                                  "unit": "GB/s", "frac": bd / td / 1e9 / PEAK_HBM_GBPS,
                                  "traffic": (measured_traffic("decode_split_kernel")
                                              if args.decode_splits == 0 else None),
                                  "kernel": "decode_split_kernel",
                                  "per_launch": f"{bd} bytes",
                                  "measured_copy_gbps": copy_gbps,
                                  "frac_of_measured_copy": bd / td / 1e9 / copy_gbps}
        parts.append(f"decode B={Bd} L={L} H={Hd} q_pos={q_pos} + o_proj [{Bd}x{K_O}]x[{K_O}x{N_O}]")
        cfg.update({"decode_batch": Bd, "decode_kv_len": L})
        if not do_p:
            res["value"] = bd / td / 1e9
            res["unit"] = "GB/s"
            res["roofline"] = res.pop("roofline_decode")
    cfg["workload"] = "; ".join(parts)
    res["config"] = cfg

    if not args.no_other_configs:
        timer = Timer(torch, dev)
        if do_p:
            res["other_configs"] = other_configs(mla, inputs, w_o, scale, dev, timer)
        if do_d:
            res["decode_shared_kpe"] = decode_shared_kpe_figures(mla, inputs, scale, dev)
            res["decode_latent"] = decode_latent_figures(mla, inputs, scale, dev)
        res["oproj"] = oproj_figures(mla, inputs, w_o, dev, timer)
        res["oproj_fp8"] = oproj_fp8_figures(mla, inputs, dev, timer)
        res["oproj_fp8_dyn"] = oproj_fp8_dyn_figures(mla, inputs, dev, timer)
        del timer
        torch.cuda.empty_cache()

    if do_p and not args.no_cpu_baseline:
        print("cpu baseline", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(d, B, H, T, d["R"].cpu().numpy(), scale, args.cpu_budget)
        if do_d:
            print("cpu baseline, decode", file=sys.stderr, flush=True)
            res["cpu_baseline"]["decode"] = cpu_baseline_decode(
                dd, Bd, Hd, L, q_pos, dd["R"].cpu().numpy(), scale, args.cpu_budget / 3)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
