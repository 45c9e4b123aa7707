#!/usr/bin/env python
"""Benchmark of the block-wise mixed-precision quantized matmul on one MI355X.

Workload: the seven linears of a Llama-3-70B-shaped decoder layer
(q/o 8192x8192, k/v 1024x8192, gate/up 28672x8192, down 8192x28672), random
N(0, 0.02) bf16 weights with 1% outlier input columns x10, block bitwidths
drawn i.i.d. from {0:5%, 1:10%, 2:60%, 3:15%, 4:8%, 8:2%} (labelled "about
2.1 bits"), random row/column permutations, x ~ N(0, 1) bf16.  Seed 0.

A step is one decode pass (M = 1) through all seven packed linears: the
activation gather, on-the-fly dequantization, matrix-core product and row
scatter of every linear, issued as a decoder layer issues them (q, k, v on
one activation in one grouped call, o, gate and up on one activation in one
grouped call, down), captured in one HIP graph that holds one step per
weight copy (a model's decode graph holds all its layers) and replayed.  The same step as seven separate calls, each on its own
activation, is reported beside it (decode_separate_calls).  The packed weights of the layer are cloned R times (R * packed >=
1 GiB) and the copies are rotated step by step so that the 256 MB Infinity
Cache cannot serve them.  value = effective weight GB/s = packed weight bytes
(codes + scales/zero points + bit map/offsets) of the layer / step time.

Also reported, each timed in its own leg of the same run:
  prefill : M = 2048 through all seven linears, grouped as the decode step is
            (q/k/v and gate/up each one gather and one GEMM launch), TFLOP/s
            and fraction of the 2.5 PFLOP/s dense bf16 matrix-core peak; the
            same as seven separate calls beside it;
  decode_m16: the same layer step at M = 16;
  pack    : quantize-pack of the seven matrices (kernel time: the descriptors
            are planned on the host beforehand), bytes moved and fraction of
            8 TB/s;
  roofline: the decode kernel on the largest linear (gate_proj), bytes per
            launch / average launch time, against 8 TB/s, over >= 1 GiB of
            rotating gate_proj copies;
  read_probe: a plain streaming-read kernel over 4 GiB, what reads reach;
  cpu_baseline: the CPU oracle (numpy) on a bounded sample of block rows of
            every linear, its pack, dequantize and fp64 matmul phases timed
            separately (median of 3), the decode rate as GB/s;
  configs : one record per (matrix, M) of the smaller workloads: Llama-3-8B
            q_proj and MLP decodes at M = 1, 8, 16, 64 (GB/s, fraction of HBM,
            p10/p90 over replays) and the Llama-3-8B down_proj prefill at
            M = 512, 2048, 8192 (TFLOP/s, fraction of the matrix-core peak),
            and the 70B layer's linears one by one at M = 16;
  context : torch's dense bf16 GEMM (hipBLASLt) at prefill shapes and a 1 GiB
            device copy, as what plain library code reaches on this GPU;
  clocks  : GPU shader and memory clocks (rocm-smi) before and after.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]

Auxiliary modes for rocprofv3 runs (bench.py reads back the HBM traffic of
the decode kernel):
  --only-decode NAME --calls C [--m M] : pack one linear of the layer, clone
                                  it to >= 1 GiB of copies, run C decode calls
                                  (M = 1, or M <= 64) rotating over the copies
                                  and exit;
  --only-configs                : only the per-matrix config lines (for a
                                  kernel trace of the small-M decodes);
  --only-pack NAME --calls C    : quantize-pack one linear of the layer C
                                  times (W resident) and exit;
  --only-prefill NAME --calls C : the same with prefill calls (M = 2048);
  --copy-bytes B                : copy B bytes device to device a few times
                                  (the calibration of the byte counters);
  --rows-sweep                  : the M = 1 decode kernel of the roofline leg
                                  on the first 1 .. 448 block rows of gate_proj
                                  (fixed cost per call against streaming rate).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective weight GB/s & %HBM peak at M=1; TFLOP/s & %MFMA peak at M=2048"
PREFILL_M = 2048
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
WORKLOAD = "llama3-70b-layer"
# grouped calls of one decoder layer's decode step (linears that read the same activation)
LAYER_GROUPS = (("q_proj", "k_proj", "v_proj"), ("o_proj",), ("gate_proj", "up_proj"), ("down_proj",))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_m1_traffic.json")
GEMV_SOURCES = ("block_wise_mixed_amd/csrc/msq_gemv.hip", "block_wise_mixed_amd/csrc/msq_dequant.h")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for p in GEMV_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(expected_sha: str):
    """HBM bytes per launch of the decode kernel from the committed rocprofv3 counter runs,
    or None when they were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != expected_sha:
        return None
    return t.get("hbm_bytes_per_launch")


def decode_bytes(pw, M: int) -> int:
    """Algorithmic bytes of one decode of one linear: packed weight + x + y."""
    return pw.packed_bytes + 2 * M * pw.K + 4 * M * pw.N


def prefill_flops(pw, M: int) -> int:
    """2 * M * 64 * 128 per block that is not pruned."""
    live = int((pw.bits != 0).sum().item())
    return 2 * M * 64 * 128 * live


def pct(v, q):
    """q-th percentile (0..100) of a list, nearest rank."""
    import numpy as np
    return float(np.percentile(np.asarray(v, dtype=np.float64), q, method="nearest"))


def replay_times_us(torch, graphs, reps: int, per_replay: int):
    """Replay graphs[k % len] reps times, each bracketed by its own events on the
    current stream (the library launches on it); returns per-launch microseconds
    of every replay (replay time / per_replay)."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for k in range(reps):
        graphs[k % len(graphs)].replay()
        evs[k + 1].record()
    torch.cuda.synchronize()
    return [evs[k].elapsed_time(evs[k + 1]) * 1e3 / per_replay for k in range(reps)]


def gpu_clocks():
    """Current shader / memory clocks as rocm-smi reports them (None if unavailable)."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=20)
        d = json.loads(r.stdout)
        card = d[sorted(d)[0]]
        out = {}
        for k, v in card.items():  # e.g. "sclk clock speed:": "(2400Mhz)"
            kl = k.lower()
            for clk in ("sclk", "mclk", "fclk", "socclk"):
                if kl.startswith(clk) and "speed" in kl:
                    out[clk] = str(v).strip("()")
        return out or None
    except Exception:  # pragma: no cover - context only
        return None


def bf16_dev(torch, np, a, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def decode_record(msq, torch, np, pw, x, M, rec, reps=10, options=None):
    """M <= 64 decode of one matrix in a HIP graph over >= 1 GiB of rotating copies."""
    dev = x.device
    y = torch.empty((M, pw.N), dtype=torch.float32, device=dev)
    ws = torch.empty(max(msq.workspace_bytes(M, pw.N, pw.K, options=options), 256),
                     dtype=torch.uint8, device=dev)
    R = max(2, min(256, int(np.ceil((1 << 30) / pw.packed_bytes))))
    cps = [pw] + [pw.clone() for _ in range(R - 1)]
    msq.gemm(x, pw, out=y, workspace=ws, options=options)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in cps:
            msq.gemm(x, c, out=y, workspace=ws, options=options)
    g.replay()
    ts = replay_times_us(torch, [g], reps, R)
    us = pct(ts, 50)
    db = decode_bytes(pw, M)
    rec.update({"us_per_call": round(us, 3), "us_p10": round(pct(ts, 10), 3),
                "us_p90": round(pct(ts, 90), 3), "weight_copies": R,
                "decode_bytes": db,
                "gbps_effective": round(pw.packed_bytes / (us * 1e-6) / 1e9, 1),
                "hbm_frac": round(db / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)})
    del g, cps
    return rec


def rows_sweep(msq, synth, torch, np, dev, log):
    """The roofline leg's kernel (M = 1, whole block rows, one K range: the
    workgroups reorder x themselves) on the first k block rows of gate_proj
    (W rows 0 .. 64k - 1, their bit-map rows and the restriction of perm_row),
    k = 1 .. 448: how the call time grows from one workgroup to the full
    matrix separates the per-call fixed cost (launch, start-up, drain) from
    the streaming rate."""
    mi = synth.matrix_inputs(WORKLOAD, "gate_proj")
    x = bf16_dev(torch, np, mi.x(1), dev)
    opt = {"gemv_split": 1}
    out = []
    for k in (1, 2, 4, 8, 16, 32, 64, 128, 192, 256, 320, 384, 448):
        N = 64 * k
        prow = mi.perm_row[mi.perm_row < N].astype(np.int32)
        pw = msq.quantize_pack(bf16_dev(torch, np, mi.W[:N], dev), np.ascontiguousarray(mi.bits[:k]),
                               prow, mi.perm_col)
        rec = {"block_rows": k, "N": N, "K": mi.K, "workgroups": k}
        decode_record(msq, torch, np, pw, x, 1, rec, options=opt)
        log(f"rows sweep k={k}: {rec['us_per_call']} us, {rec['gbps_effective']} GB/s")
        out.append(rec)
        del pw
        torch.cuda.empty_cache()
    return out


def config_legs(msq, synth, torch, np, dev, log, only_decode=False):
    """Per-matrix lines of the smaller workloads: the Llama-3-8B q_proj and MLP
    decodes (M = 1, 8, 16, 64), the Llama-3-8B down_proj prefill (M = 512, 2048,
    8192), and the 70B layer's linears one by one at M = 16.  Decodes rotate
    >= 1 GiB of weight copies inside one HIP graph per (matrix, M); prefills run
    eagerly on two copies."""
    out = []
    legs = [("llama3-8b-q_proj", (1,)), ("llama3-8b-mlp", (1, 8, 16, 64)),
            ("llama3-70b-layer", (16,))]
    if not only_decode:
        legs.append(("llama3-8b-down_proj-prefill", (512, 2048, 8192)))
    for wname, Ms in legs:
        wl = synth.WORKLOADS[wname]
        for mi_idx, m in enumerate(wl.matrices):
            mi = synth.matrix_inputs(wname, mi_idx)
            pw = msq.quantize_pack(bf16_dev(torch, np, mi.W, dev), mi.bits, mi.perm_row, mi.perm_col)
            for M in Ms:
                x = bf16_dev(torch, np, mi.x(M), dev)
                rec = {"workload": wname, "matrix": m.name, "N": m.N, "K": m.K, "M": M,
                       "mean_bits": round(mi.mean_bits, 4)}
                if M <= 64:
                    decode_record(msq, torch, np, pw, x, M, rec)
                else:
                    y = torch.empty((M, pw.N), dtype=torch.float32, device=dev)
                    ws = torch.empty(max(msq.workspace_bytes(M, pw.N, pw.K), 256), dtype=torch.uint8,
                                     device=dev)
                    cps = [pw, pw.clone()]
                    msq.gemm(x, pw, out=y, workspace=ws)
                    torch.cuda.synchronize()
                    reps = 6
                    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
                    evs[0].record()
                    for k in range(reps):
                        msq.gemm(x, cps[k % 2], out=y, workspace=ws)
                        evs[k + 1].record()
                    torch.cuda.synchronize()
                    ts = [evs[k].elapsed_time(evs[k + 1]) * 1e3 for k in range(reps)]
                    us = pct(ts, 50)
                    tf = prefill_flops(pw, M) / (us * 1e-6) / 1e12
                    rec.update({"us_per_call": round(us, 1), "us_p10": round(pct(ts, 10), 1),
                                "us_p90": round(pct(ts, 90), 1), "flops": prefill_flops(pw, M),
                                "tflops": round(tf, 1), "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)})
                    del cps, y, ws
                log(f"{wname} {m.name} M={M}: " + ", ".join(
                    f"{k}={v}" for k, v in rec.items()
                    if k in ("us_per_call", "us_p10", "us_p90", "gbps_effective", "hbm_frac", "tflops",
                             "mfma_frac")))
                out.append(rec)
                del x
            del pw
            torch.cuda.empty_cache()
    return out


def read_probe_leg(torch, dev, log):
    """A plain streaming-read kernel (libmsq_probe.so) over a 4 GiB buffer: the
    best of a few grid sizes, GB/s read.  What reads reach on this GPU, beside the
    8 TB/s peak; not a denominator."""
    import ctypes
    path = os.path.join(ROOT, "block_wise_mixed_amd", "libmsq_probe.so")
    lib = ctypes.CDLL(path)
    lib.msq_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                   ctypes.c_void_p]
    lib.msq_probe_read.restype = ctypes.c_int
    n = 4 << 30
    buf = torch.empty(n, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    out = torch.empty(1 << 16, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    res = []
    for wgs in (1024, 2048, 4096, 8192, 16384):
        assert lib.msq_probe_read(buf.data_ptr(), n, out.data_ptr(), wgs, stream) == 0
        torch.cuda.synchronize()
        reps = 5
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        evs[0].record()
        for k in range(reps):
            assert lib.msq_probe_read(buf.data_ptr(), n, out.data_ptr(), wgs, stream) == 0
            evs[k + 1].record()
        torch.cuda.synchronize()
        ts = [evs[k].elapsed_time(evs[k + 1]) * 1e3 for k in range(reps)]
        us = pct(ts, 50)
        res.append({"workgroups": wgs, "us": round(us, 1), "gbps": round(n / (us * 1e-6) / 1e9, 1)})
    best = max(res, key=lambda r: r["gbps"])
    log(f"read probe: best {best['gbps']} GB/s ({best['workgroups']} workgroups)")
    del buf, out
    torch.cuda.empty_cache()
    return {"bytes": n, "best_gbps": best["gbps"], "best_frac": round(best["gbps"] / HBM_PEAK_GBPS, 4),
            "sweep": res, "note": "16-byte streaming loads, grid-stride, 256 threads per workgroup"}


def achievable_context(torch, dev, log):
    """What plain library code reaches on the same GPU, as context for the
    fractions (not a denominator): torch's dense bf16 GEMM (hipBLASLt) at the
    prefill shapes, and a device-to-device copy of 1 GiB (read + write)."""
    res = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gemms = []
    for name, M, N, K in (("llama3-8b down_proj", 2048, 4096, 14336),
                          ("llama3-70b gate_proj", 2048, 28672, 8192),
                          ("llama3-70b down_proj", 2048, 8192, 28672)):
        a = torch.randn(M, K, device=dev).to(torch.bfloat16)
        b = torch.randn(N, K, device=dev).to(torch.bfloat16)
        c = torch.matmul(a, b.t())
        torch.cuda.synchronize()
        reps = 5
        e0.record()
        for _ in range(reps):
            c = torch.matmul(a, b.t())
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
        gemms.append({"shape": f"{name} M={M} N={N} K={K}", "us": round(us, 1), "tflops": round(tf, 1),
                      "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)})
        log(f"context: dense bf16 torch.matmul {name}: {tf:.0f} TFLOP/s")
        del a, b, c
    res["dense_bf16_gemm"] = gemms
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    reps = 5
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    res["device_copy_1GiB"] = {"us": round(us, 1), "gbps_read_plus_write": round(2 * n / (us * 1e-6) / 1e9, 1)}
    log(f"context: device copy {2 * n / (us * 1e-6) / 1e9:.0f} GB/s read+write")
    del src, dst
    torch.cuda.empty_cache()
    res["note"] = ("achievable context only; the fractions above use the published peaks "
                   "(8 TB/s HBM, 2.5 PFLOP/s dense bf16)")
    return res


def alloc_leg(msq, synth, torch, log):
    """Bitwidth allocation (batched greedy) for every block of a Llama-3-70B-shaped
    model (80 layers of the seven linears: 8355840 blocks of 64x128) at an average
    of 2.1 bits, on synthetic utilities; wall time of msq_allocate_bits, which
    synchronises with the host after every iteration."""
    blocks = 80 * (2 * 8192 * 8192 + 2 * 1024 * 8192 + 3 * 28672 * 8192) // (64 * 128)
    u = torch.from_numpy(synth.draw_alloc_utility(blocks, 70)).cuda()
    budget = int(2.1 * blocks)
    ws = torch.empty(msq.alloc_workspace_bytes(blocks), dtype=torch.uint8, device=u.device)
    msq.allocate_bits(u, budget, workspace=ws)
    torch.cuda.synchronize()
    times, iters = [], 0
    for _ in range(3):
        t0 = time.perf_counter()
        bits, iters = msq.allocate_bits(u, budget, workspace=ws)
        times.append(time.perf_counter() - t0)
    ms = 1e3 * sorted(times)[1]
    mean_bits = float(bits.double().mean())
    log(f"alloc: {blocks} blocks, {iters} iterations, {ms:.1f} ms, mean {mean_bits:.4f} bits")
    del u, ws, bits
    return {"blocks": blocks, "budget_mean_bits": 2.1, "mean_bits": round(mean_bits, 4),
            "iterations": iters, "ms": round(ms, 2),
            "note": "batched greedy over a 70B model's blocks, synthetic utilities; median of 3"}


def tile16_leg(msq, synth, torch, np, log):
    """A TileQuant-style weight (tiles at 8 or 16 bits, 70/30) of the Llama-3-8B gate_proj
    shape (14336 x 4096): M = 1 decode in a HIP graph over rotating copies, and M = 2048
    prefill; the quantized kernels plus the k_tile16 pass for the bf16 tiles."""
    c = synth.random_case(14336, 4096, 90, dist={8: 0.7, 16: 0.3})
    pw = msq.quantize_pack(c.W, c.bits, c.perm_row, c.perm_col)
    dev = pw.bits.device
    out = {"N": c.N, "K": c.K, "mix": "8-bit 0.7, 16-bit 0.3", "tile16_blocks": pw.tile16_blocks,
           "mean_bits": round(float(c.bits.astype(np.float64).mean()), 4)}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    x = torch.from_numpy(c.x(1).view(np.int16)).view(torch.bfloat16).to(dev)
    y = torch.empty((1, c.N), dtype=torch.float32, device=dev)
    ws = torch.empty(max(msq.workspace_bytes(1, c.N, c.K), 256), dtype=torch.uint8, device=dev)
    R = max(2, min(64, int(np.ceil((1 << 30) / pw.packed_bytes))))
    cps = [pw] + [pw.clone() for _ in range(R - 1)]
    msq.gemm(x, pw, out=y, workspace=ws)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for cp in cps:
            msq.gemm(x, cp, out=y, workspace=ws)
    g.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(3):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (3 * R)
    out.update({"decode_us": round(us, 3), "decode_gbps": round(decode_bytes(pw, 1) / (us * 1e-6) / 1e9, 1)})
    del g, cps
    M = 2048
    x = torch.from_numpy(c.x(M).view(np.int16)).view(torch.bfloat16).to(dev)
    y = torch.empty((M, c.N), dtype=torch.float32, device=dev)
    ws = torch.empty(max(msq.workspace_bytes(M, c.N, c.K), 256), dtype=torch.uint8, device=dev)
    msq.gemm(x, pw, out=y, workspace=ws)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(3):
        msq.gemm(x, pw, out=y, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / 3
    flops = 2.0 * M * c.N * c.K * float((c.bits != 0).mean())
    out.update({"prefill_M": M, "prefill_us": round(us, 1),
                "prefill_tflops": round(flops / (us * 1e-6) / 1e12, 1)})
    log(f"tile16 (8/16 mix): decode {out['decode_us']} us ({out['decode_gbps']} GB/s), "
        f"prefill M=2048 {out['prefill_us']} us ({out['prefill_tflops']} TFLOP/s)")
    return out


def reorder_leg(msq, torch, log):
    """Channel reordering for one gate_proj-shaped saliency map (28672 x 8192 fp32,
    940 MB, read once): time per call over 5 calls bracketed by events."""
    N, K = 28672, 8192
    S = torch.rand((N, K), dtype=torch.float32, device="cuda")
    ws = torch.empty(int(msq.load_library().msq_reorder_workspace_bytes(N, K)), dtype=torch.uint8,
                     device="cuda")
    msq.reorder_channels(S, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        msq.reorder_channels(S, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    gbps = N * K * 4 / (ms * 1e-3) / 1e9
    log(f"reorder: {N}x{K} saliency, {ms:.3f} ms, {gbps:.0f} GB/s of saliency read")
    del S, ws
    return {"N": N, "K": K, "ms": round(ms, 4), "gbps_saliency": round(gbps, 1),
            "note": "row and column sums in one pass over the fp32 map, two radix sorts"}


def cpu_baseline(inputs, target_s: float = 7.0):
    """The oracle on a bounded sample of every linear, phase by phase (median of 3).

    Sample: the first rows_per block rows of each of the seven linears (rows_per
    calibrated so that one pass over all phases takes about target_s seconds).
    Phases, each timed on its own:
      pack        oracle.quantize (reorder, scales, zero points, codes) + oracle.pack;
      dequantize  oracle.unpack + oracle.dequantize (fp64 W-hat);
      matmul M=1  oracle.matmul, fp64, x gathered through perm_col;
      matmul M=2048 the same on the first 256 rows of the first linear's sample.
    value = decode rate in GB/s of packed weight = sample packed bytes /
    (dequantize + matmul at M = 1), the CPU counterpart of the GPU decode.
    """
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1

    def sample(rows_per):
        out = []
        for mi in inputs:
            brs = np.arange(min(rows_per, mi.N // 64))
            out.append((mi, brs))
        return out

    def phases(smp):
        """One pass of every phase over the sample: (times dict, packed bytes, weights)."""
        t = {"pack": 0.0, "dequantize": 0.0, "matmul_m1": 0.0}
        packed_b = weights = 0
        keep = None
        for mi, brs in smp:
            t0 = time.perf_counter()
            q = oracle.quantize(mi.W, mi.bits, mi.perm_row, mi.perm_col, block_rows=brs, check=False)
            sub_bits = mi.bits[brs]
            off, codes = oracle.pack(q["q"], sub_bits)
            t1 = time.perf_counter()
            qq = oracle.unpack(codes, sub_bits, off)
            What = oracle.dequantize(qq, q["s"], q["z"])
            t2 = time.perf_counter()
            oracle.matmul(oracle.bf16_to_f32(mi.x(1)), What, mi.perm_col)
            t3 = time.perf_counter()
            t["pack"] += t1 - t0
            t["dequantize"] += t2 - t1
            t["matmul_m1"] += t3 - t2
            live = int((sub_bits != 0).sum())
            packed_b += codes.size + 320 * live + 5 * sub_bits.size
            weights += What.size
            if keep is None:
                keep = (mi, What[:256])
        return t, packed_b, weights, keep

    t1, _, _, _ = phases(sample(1))  # calibration
    per_row = sum(t1.values())
    rows_per = int(max(1, min(448, round(target_s / max(per_row, 1e-3)))))
    smp = sample(rows_per)
    runs = [phases(smp) for _ in range(3)]
    med = {k: float(np.median([r[0][k] for r in runs])) for k in runs[0][0]}
    packed_b, weights, (mi0, W256) = runs[0][1], runs[0][2], runs[0][3]
    x2048 = oracle.bf16_to_f32(mi0.x(PREFILL_M))
    mm = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.matmul(x2048, W256, mi0.perm_col)
        mm.append(time.perf_counter() - t0)
    mm_s = float(np.median(mm))
    mm_flops = 2.0 * PREFILL_M * W256.shape[0] * W256.shape[1]
    decode_s = med["dequantize"] + med["matmul_m1"]
    return {"value": round(packed_b / decode_s / 1e9, 4), "unit": "GB/s",
            "cores": int(blas_threads), "kind": "oracle",
            "sample": f"first {rows_per} block rows of each of the 7 linears "
                      f"({weights} weights, {packed_b / 1e6:.1f} MB packed), M=1; value = packed "
                      f"bytes / (dequantize + fp64 matmul); phases median of 3",
            "phases_s": {k: round(v, 4) for k, v in med.items()},
            "pack_gbps_w_read": round(2.0 * weights / med["pack"] / 1e9, 4),
            "matmul_m2048": {"rows": int(W256.shape[0]), "K": int(W256.shape[1]),
                             "s": round(mm_s, 4), "tflops": round(mm_flops / mm_s / 1e12, 4)}}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--prefill-steps", type=int, default=6)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-matrix lines of the smaller workloads and the context leg")
    ap.add_argument("--only-decode", default=None, metavar="NAME")
    ap.add_argument("--only-prefill", default=None, metavar="NAME")
    ap.add_argument("--only-configs", action="store_true")
    ap.add_argument("--only-pack", default=None, metavar="NAME")
    ap.add_argument("--calls", type=int, default=20)
    ap.add_argument("--m", type=int, default=1, help="M of --only-decode (default 1)")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--rows-sweep", action="store_true",
                    help="only the M = 1 decode on the first 1 .. 448 block rows of gate_proj")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path here (block rows "
              "would shard across GPUs, x replicated, y gathered). Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import block_wise_mixed_amd as msq
    from block_wise_mixed_amd import synth

    msq.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS[WORKLOAD]
    names = [m.name for m in wl.matrices]

    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_bytes} bytes 5 times")
        return 0
    if args.only_pack is not None:
        mi = synth.matrix_inputs(WORKLOAD, names.index(args.only_pack))
        Wd = bf16_dev(torch, np, mi.W, dev)
        pw = msq.allocate_packed(mi.N, mi.K, mi.bits, mi.perm_row, mi.perm_col, device=dev)
        torch.cuda.synchronize()
        for _ in range(args.calls):
            msq.pack_into(Wd, pw)
        torch.cuda.synchronize()
        log(f"{args.calls} packs of {args.only_pack}: {msq.pack_bytes(pw)} bytes moved per pack")
        return 0
    if args.rows_sweep:
        print(json.dumps({"rows_sweep": rows_sweep(msq, synth, torch, np, dev, log)}), flush=True)
        return 0
    if args.only_configs:
        recs = config_legs(msq, synth, torch, np, dev, log, only_decode=True)
        print(json.dumps({"configs": recs}), flush=True)
        return 0
    if args.only_prefill is not None or args.only_decode is not None:
        name = args.only_prefill if args.only_prefill is not None else args.only_decode
        mi = synth.matrix_inputs(WORKLOAD, names.index(name))
        pw = msq.quantize_pack(bf16_dev(torch, np, mi.W, dev), mi.bits, mi.perm_row, mi.perm_col)
        M = PREFILL_M if args.only_prefill is not None else args.m
        # decode: rotate >= 1 GiB of copies, as the roofline leg does
        R = 1 if M > 64 else max(2, int(np.ceil((1 << 30) / pw.packed_bytes)))
        cps = [pw] + [pw.clone() for _ in range(R - 1)]
        x = bf16_dev(torch, np, mi.x(M), dev)
        y = torch.empty((M, pw.N), dtype=torch.float32, device=dev)
        ws = torch.empty(max(msq.workspace_bytes(M, pw.N, pw.K), 256), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        for k in range(args.calls):
            msq.gemm(x, cps[k % R], out=y, workspace=ws)
        torch.cuda.synchronize()
        log(f"{args.calls} calls (M = {M}) on {name} over {R} copies: "
            f"{decode_bytes(pw, M) if M <= 64 else prefill_flops(pw, M)} algorithmic "
            f"{'bytes' if M <= 64 else 'flops'} per call")
        return 0

    clocks_before = gpu_clocks()

    # ---- inputs and pack leg: descriptors planned on the host first, then the
    # seven pack launches back to back between two events ------------------------------
    inputs, packed, Wds = [], [], []
    for mi_idx, m in enumerate(wl.matrices):
        mi = synth.matrix_inputs(WORKLOAD, mi_idx)
        log(f"inputs {m.name} {m.N}x{m.K} mean bits {mi.mean_bits:.3f}")
        inputs.append(mi)
        Wds.append(bf16_dev(torch, np, mi.W, dev))
        packed.append(msq.allocate_packed(m.N, m.K, mi.bits, mi.perm_row, mi.perm_col, device=dev))
    for W, pw in zip(Wds, packed):  # warm-up pass (first launch, page-in)
        msq.pack_into(W, pw)
    torch.cuda.synchronize()
    pack_reps = 3
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(pack_reps + 1)]
    evs[0].record()
    for k in range(pack_reps):
        for W, pw in zip(Wds, packed):
            msq.pack_into(W, pw)
        evs[k + 1].record()
    torch.cuda.synchronize()
    pack_ts = [evs[k].elapsed_time(evs[k + 1]) for k in range(pack_reps)]
    pack_ms = pct(pack_ts, 50)
    p_bytes = sum(msq.pack_bytes(pw) for pw in packed)
    w_bytes = sum(2 * pw.N * pw.K for pw in packed)
    pack = {"ms": round(pack_ms, 4), "ms_p10": round(pct(pack_ts, 10), 4),
            "ms_p90": round(pct(pack_ts, 90), 4), "weight_bytes": w_bytes, "pack_bytes": p_bytes,
            "gbps_read": round(w_bytes / (pack_ms * 1e-3) / 1e9, 1),
            "gbps_moved": round(p_bytes / (pack_ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(p_bytes / (pack_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "note": "msq_quantize_pack of the 7 matrices back to back (k_block_offsets + k_pack_rows each), "
                    "asynchronous, descriptors planned on the host beforehand; median of 3"}
    log(f"pack: {pack_ms:.3f} ms for 7 matrices, {pack['gbps_moved']} GB/s moved "
        f"({pack['hbm_frac']:.3f} of HBM)")
    del Wds
    torch.cuda.empty_cache()

    layer_packed = sum(p.packed_bytes for p in packed)
    mean_bits = float(sum(int(p.bits.to(torch.int64).sum().item()) for p in packed) /
                      sum(p.bits.numel() for p in packed))
    R = max(2, int(np.ceil((1 << 30) / layer_packed)))
    log(f"layer packed {layer_packed / 1e6:.1f} MB, {R} copies for cache rotation")
    copies = [packed] + [[p.clone() for p in packed] for _ in range(R - 1)]

    # ---- decode leg (M = 1), one HIP graph per weight copy -----------------------------
    layer_groups = [[names.index(n) for n in grp] for grp in LAYER_GROUPS]

    def layer_buffers(M):
        xs = [bf16_dev(torch, np, mi.x(M), dev) for mi in inputs]
        ys = [torch.empty((M, p.N), dtype=torch.float32, device=dev) for p in packed]
        wss = [torch.empty(max(msq.workspace_bytes(M, p.N, p.K), 256), dtype=torch.uint8, device=dev)
               for p in packed]
        gws = [torch.empty(max(msq.group_workspace_bytes(M, [packed[i] for i in grp]), 256),
                           dtype=torch.uint8, device=dev) for grp in layer_groups]
        return xs, ys, wss, gws

    def make_steps(bufs):
        xs, ys, wss, gws = bufs

        # The layer's linears in the order and grouping a decoder layer calls them:
        # q, k, v read one activation (one grouped call), then o, then gate, up read
        # one activation (one grouped call), then down.
        def grouped(ws_copy):
            for grp, gw in zip(layer_groups, gws):
                x = xs[grp[0]]  # the group's shared activation
                if len(grp) == 1:
                    msq.gemm(x, ws_copy[grp[0]], out=ys[grp[0]], workspace=wss[grp[0]])
                else:
                    msq.gemm_group([x] * len(grp), [ws_copy[i] for i in grp],
                                   outs=[ys[i] for i in grp], workspace=gw)

        def single(ws_copy):
            for i, p in enumerate(ws_copy):
                msq.gemm(xs[i], p, out=ys[i], workspace=wss[i])
        return grouped, single

    def time_steps(step_fn, steps, warmup):
        """Time exactly `steps` steps.  One HIP graph holds R steps, one per weight
        copy in rotation order (a model's decode graph holds all its layers, so a
        graph launch per layer step would overstate the launch cost); steps % R
        leftover steps replay one-step graphs.  Events bracket every replay on
        the current stream; per-step times are replay time / steps in it."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for cp in copies:
                step_fn(cp)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all):
            for cp in copies:
                step_fn(cp)
        singles = []
        for cp in copies[:steps % R]:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step_fn(cp)
            singles.append(g)
        torch.cuda.synchronize()
        for s in range(max(1, (warmup + R - 1) // R)):
            g_all.replay()
        torch.cuda.synchronize()
        plan = [(g_all, R)] * (steps // R) + [(g, 1) for g in singles]
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(plan) + 1)]
        t0 = time.perf_counter()
        evs[0].record()
        for k, (g, _) in enumerate(plan):
            g.replay()
            evs[k + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = evs[0].elapsed_time(evs[len(plan)]) / steps
        per = []
        for k, (_, n) in enumerate(plan):
            per += [evs[k].elapsed_time(evs[k + 1]) / n] * n
        del g_all, singles
        return ms, wall, per

    M = 1
    bufs1 = layer_buffers(M)
    step_grouped, step_single = make_steps(bufs1)
    ms_single, _, _ = time_steps(step_single, args.steps, args.warmup)
    log(f"decode step, seven separate calls: {ms_single * 1e3:.1f} us")
    ms_per_step, t_wall, per_step = time_steps(step_grouped, args.steps, args.warmup)
    step_decode_bytes = sum(decode_bytes(p, M) for p in packed)
    value = layer_packed / (ms_per_step * 1e-3) / 1e9
    hbm_frac = step_decode_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS
    log(f"decode step {ms_per_step * 1e3:.1f} us, {value:.1f} GB/s effective, {hbm_frac:.3f} of HBM")
    decode_single = {"ms_per_step": round(ms_single, 5),
                     "value": round(layer_packed / (ms_single * 1e-3) / 1e9, 2),
                     "note": "the seven linears as seven msq_gemm calls, each with its own activation"}
    step_stats = {"us_p10": round(pct(per_step, 10) * 1e3, 2), "us_p50": round(pct(per_step, 50) * 1e3, 2),
                  "us_p90": round(pct(per_step, 90) * 1e3, 2)}

    # ---- the same step at M = 16 -------------------------------------------------------
    bufs16 = layer_buffers(16)
    step16, _ = make_steps(bufs16)
    ms16, _, per16 = time_steps(step16, max(10, args.steps // 2), args.warmup)
    db16 = sum(decode_bytes(p, 16) for p in packed)
    decode_m16 = {"M": 16, "ms_per_step": round(ms16, 5),
                  "gbps_effective": round(layer_packed / (ms16 * 1e-3) / 1e9, 1),
                  "hbm_frac": round(db16 / (ms16 * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                  "us_p10": round(pct(per16, 10) * 1e3, 2), "us_p90": round(pct(per16, 90) * 1e3, 2),
                  "grouping": "as the M = 1 step (q/k/v and gate/up: one gather and one decode "
                              "launch per group)"}
    log(f"decode step M=16 {ms16 * 1e3:.1f} us, {decode_m16['hbm_frac']:.3f} of HBM")
    del bufs16

    # ---- roofline leg: the decode kernel on gate_proj over >= 1 GiB of its copies --------
    gi = names.index("gate_proj")
    xs1, ys1, wss1, _ = bufs1
    R_gate = max(2, int(np.ceil((1 << 30) / packed[gi].packed_bytes)))
    gate_copies = [copies[k][gi] for k in range(min(R, R_gate))]
    gate_copies += [packed[gi].clone() for _ in range(R_gate - len(gate_copies))]
    L = 2 * R_gate
    g_roof = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_roof):
        for k in range(L):
            msq.gemm(xs1[gi], gate_copies[k % R_gate], out=ys1[gi], workspace=wss1[gi])
    g_roof.replay()
    roof_ts = replay_times_us(torch, [g_roof], 10, L)
    launch_us = pct(roof_ts, 50)
    per_launch = decode_bytes(packed[gi], M)
    achieved = per_launch / (launch_us * 1e-6) / 1e9
    sha = kernel_source_sha()
    traffic = measured_traffic(sha)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic,
                "kernel": "msq_gemm M=1 on gate_proj 28672x8192: one k_gemv_m1 launch per call "
                          "(launch gaps inside the graph included)",
                "bytes_per_launch": per_launch, "avg_launch_us": round(launch_us, 3),
                "launch_us_p10": round(pct(roof_ts, 10), 3), "launch_us_p90": round(pct(roof_ts, 90), 3),
                "weight_copies": R_gate, "launches_per_graph": L, "kernel_sha": sha}
    log(f"roofline: {launch_us:.2f} us/launch over {R_gate} copies, {achieved:.0f} GB/s")
    del g_roof, gate_copies

    read_probe = read_probe_leg(torch, dev, log)

    # ---- prefill leg (M = 2048) --------------------------------------------------------
    prefill = None
    if not args.no_prefill:
        Mp = PREFILL_M
        xp = [bf16_dev(torch, np, mi.x(Mp), dev) for mi in inputs]
        yp = [torch.empty((Mp, p.N), dtype=torch.float32, device=dev) for p in packed]
        wsp = [torch.empty(max(msq.workspace_bytes(Mp, p.N, p.K), 256), dtype=torch.uint8,
                           device=dev) for p in packed]
        gwsp = [torch.empty(max(msq.group_workspace_bytes(Mp, [packed[i] for i in grp]), 256),
                            dtype=torch.uint8, device=dev) for grp in layer_groups]

        def prefill_grouped(cp):
            # q, k, v (and gate, up) in one gather and one GEMM launch each
            for grp, gw in zip(layer_groups, gwsp):
                x = xp[grp[0]]
                msq.gemm_group([x] * len(grp), [cp[i] for i in grp],
                               outs=[yp[i] for i in grp], workspace=gw)

        def prefill_single(cp):
            for i, p in enumerate(cp):
                msq.gemm(xp[i], p, out=yp[i], workspace=wsp[i])

        def time_prefill(step_fn):
            step_fn(packed)
            torch.cuda.synchronize()
            n = args.prefill_steps
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
            evs[0].record()
            for s in range(n):
                step_fn(copies[s % R])
                evs[s + 1].record()
            torch.cuda.synchronize()
            per = [evs[s].elapsed_time(evs[s + 1]) for s in range(n)]
            return evs[0].elapsed_time(evs[n]) / n, per

        ms_single_p, _ = time_prefill(prefill_single)
        ms_p, per_p = time_prefill(prefill_grouped)
        flops = sum(prefill_flops(p, Mp) for p in packed)
        tflops = flops / (ms_p * 1e-3) / 1e12
        prefill = {"M": Mp, "ms_per_step": round(ms_p, 4), "tflops": round(tflops, 2),
                   "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                   "peak_tflops": MFMA_BF16_PEAK_TFLOPS, "flops_per_step": flops,
                   "ms_p10": round(pct(per_p, 10), 4), "ms_p90": round(pct(per_p, 90), 4),
                   "grouping": "q/k/v and gate/up grouped as in the decode step",
                   "ms_per_step_separate_calls": round(ms_single_p, 4)}
        log(f"prefill M={Mp}: {ms_p:.3f} ms/step grouped, {tflops:.1f} TFLOP/s "
            f"({ms_single_p:.3f} ms/step as separate calls)")
        del xp, yp, wsp, gwsp

    alloc = alloc_leg(msq, synth, torch, log)
    reorder = reorder_leg(msq, torch, log)
    tile16 = tile16_leg(msq, synth, torch, np, log)
    clocks_after = gpu_clocks()

    configs, context = None, None
    if not args.no_configs:
        del copies, bufs1
        torch.cuda.empty_cache()
        configs = config_legs(msq, synth, torch, np, dev, log)
        context = achievable_context(torch, dev, log)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(inputs)
        log(f"cpu baseline {cpu['value']} GB/s; phases {cpu['phases_s']}")

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3-70b-layer decode M=1: q,o 8192x8192; k,v 1024x8192; "
                               "gate,up 28672x8192; down 8192x28672",
                   "M": M, "mean_bits": round(mean_bits, 4), "packed_bytes": layer_packed,
                   "decode_bytes": step_decode_bytes, "weight_copies": R,
                   "timing": f"one HIP graph of {R} steps (one per weight copy), events around every timed replay"},
        "hbm_frac": round(hbm_frac, 4),
        "step_spread": step_stats,
        "decode_separate_calls": decode_single,
        "decode_m16": decode_m16,
        "prefill": prefill,
        "pack": pack,
        "alloc": alloc,
        "reorder": reorder,
        "tile16": tile16,
        "roofline": roofline,
        "read_probe": read_probe,
        "cpu_baseline": cpu,
        "configs": configs,
        "context": context,
        "clocks": {"before": clocks_before, "after_gpu_legs": clocks_after},
        "wall_s_timed": round(t_wall, 4),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
