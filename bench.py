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
grouped call, down), captured once per weight copy in a HIP graph and
replayed.  The same step as seven separate calls, each on its own
activation, is reported beside it (decode_separate_calls).  The packed weights of the layer are cloned R times (R * packed >=
1 GiB) and the copies are rotated step by step so that the 256 MB Infinity
Cache cannot serve them.  value = effective weight GB/s = packed weight bytes
(codes + scales/zero points + bit map/offsets) of the layer / step time.

Also reported, each timed in its own leg of the same run:
  prefill : M = 2048 through all seven linears, grouped as the decode step is
            (q/k/v and gate/up each one gather and one GEMM launch), TFLOP/s
            and fraction of the 2.5 PFLOP/s dense bf16 matrix-core peak; the
            same as seven separate calls beside it;
  pack    : quantize-pack throughput over the seven matrices;
  roofline: the decode kernel on the largest linear (gate_proj), bytes per
            launch / average launch time, against 8 TB/s;
  cpu_baseline: the CPU oracle (numpy) decoding a bounded sample of block
            rows of every linear, scaled to GB/s;
  configs : one record per (matrix, M) of the smaller workloads: Llama-3-8B
            q_proj and MLP decodes at M = 1, 16, 64 (GB/s, fraction of HBM)
            and the Llama-3-8B down_proj prefill at M = 512, 2048, 8192
            (TFLOP/s, fraction of the matrix-core peak);
  context : torch's dense bf16 GEMM (hipBLASLt) at prefill shapes and a 1 GiB
            device copy, as what plain library code reaches on this GPU.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]

Auxiliary modes for rocprofv3 counter runs (bench.py reads back the HBM
traffic of the decode kernel):
  --only-decode NAME --calls C  : pack one linear of the layer, run C decode
                                  calls (M = 1) and exit;
  --only-prefill NAME --calls C : the same with prefill calls (M = 2048);
  --copy-bytes B                : copy B bytes device to device a few times
                                  (the calibration of the byte counters).
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


def config_legs(msq, synth, torch, np, dev, log):
    """Per-matrix lines of the smaller workloads: the Llama-3-8B q_proj and MLP
    decodes (M = 1, 16, 64) and the Llama-3-8B down_proj prefill (M = 512, 2048,
    8192).  Decodes rotate >= 1 GiB of weight copies inside one HIP graph per
    (matrix, M); prefills run eagerly on two copies."""
    out = []
    for wname, Ms in (("llama3-8b-q_proj", (1,)), ("llama3-8b-mlp", (1, 16, 64)),
                      ("llama3-8b-down_proj-prefill", (512, 2048, 8192))):
        wl = synth.WORKLOADS[wname]
        for mi_idx, m in enumerate(wl.matrices):
            mi = synth.matrix_inputs(wname, mi_idx)
            Wd = torch.from_numpy(mi.W.view(np.int16)).view(torch.bfloat16).to(dev)
            pw = msq.quantize_pack(Wd, mi.bits, mi.perm_row, mi.perm_col)
            del Wd
            for M in Ms:
                x = torch.from_numpy(mi.x(M).view(np.int16)).view(torch.bfloat16).to(dev)
                y = torch.empty((M, pw.N), dtype=torch.float32, device=dev)
                ws = torch.empty(max(msq.workspace_bytes(M, pw.N, pw.K), 256), dtype=torch.uint8,
                                 device=dev)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                rec = {"workload": wname, "matrix": m.name, "N": m.N, "K": m.K, "M": M,
                       "mean_bits": round(mi.mean_bits, 4)}
                if M <= 64:
                    R = max(2, min(256, int(np.ceil((1 << 30) / pw.packed_bytes))))
                    cps = [pw] + [pw.clone() for _ in range(R - 1)]
                    msq.gemm(x, pw, out=y, workspace=ws)
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        for c in cps:
                            msq.gemm(x, c, out=y, workspace=ws)
                    g.replay()
                    torch.cuda.synchronize()
                    reps = 3
                    e0.record()
                    for _ in range(reps):
                        g.replay()
                    e1.record()
                    torch.cuda.synchronize()
                    us = e0.elapsed_time(e1) * 1e3 / (reps * R)
                    db = decode_bytes(pw, M)
                    rec.update({"us_per_call": round(us, 3), "weight_copies": R,
                                "gbps_effective": round(pw.packed_bytes / (us * 1e-6) / 1e9, 1),
                                "hbm_frac": round(db / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)})
                    del g, cps
                else:
                    cps = [pw, pw.clone()]
                    msq.gemm(x, pw, out=y, workspace=ws)
                    torch.cuda.synchronize()
                    reps = 6
                    e0.record()
                    for k in range(reps):
                        msq.gemm(x, cps[k % 2], out=y, workspace=ws)
                    e1.record()
                    torch.cuda.synchronize()
                    us = e0.elapsed_time(e1) * 1e3 / reps
                    tf = prefill_flops(pw, M) / (us * 1e-6) / 1e12
                    rec.update({"us_per_call": round(us, 1), "tflops": round(tf, 1),
                                "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)})
                    del cps
                log(f"{wname} {m.name} M={M}: " + ", ".join(f"{k}={v}" for k, v in rec.items()
                                                             if k in ("us_per_call", "gbps_effective",
                                                                      "hbm_frac", "tflops", "mfma_frac")))
                out.append(rec)
                del x, y, ws
            del pw
            torch.cuda.empty_cache()
    return out


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


def cpu_baseline(inputs, target_s: float = 12.0):
    """The oracle decoding a sample of block rows of every linear (M = 1).

    Per linear: the oracle quantizes and packs the sampled block rows (not
    timed), then the timed part unpacks their codes, dequantizes in fp64 and
    multiplies (the oracle's decode).  The sample grows until it takes about
    target_s seconds in total; the rate is sample packed bytes / time.
    """
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    def run(rows_per):
        t_sum = b_sum = 0.0
        n_rows = 0
        for mi in inputs:
            brs = np.arange(min(rows_per, mi.N // 64))
            q = oracle.quantize(mi.W, mi.bits, mi.perm_row, mi.perm_col, block_rows=brs,
                                check=False)
            sub_bits = mi.bits[brs]
            off, codes = oracle.pack(q["q"], sub_bits)
            x = mi.x(1)
            t0 = time.perf_counter()
            qq = oracle.unpack(codes, sub_bits, off)
            What = oracle.dequantize(qq, q["s"], q["z"])
            oracle.matmul(oracle.bf16_to_f32(x), What, mi.perm_col)
            t_sum += time.perf_counter() - t0
            live = int((sub_bits != 0).sum())
            b_sum += codes.size + 320 * live + 5 * sub_bits.size
            n_rows += brs.size * 64
        return t_sum, b_sum, n_rows

    t1, _, _ = run(1)  # calibration
    rows_per = int(max(1, min(448, round(target_s / max(t1, 1e-3)))))
    total_t, total_b, sample_rows = run(rows_per)
    return {"value": round(total_b / total_t / 1e9, 4), "unit": "GB/s",
            "cores": int(blas_threads), "kind": "oracle",
            "sample": f"first {rows_per} block rows ({sample_rows} output rows total) of each of "
                      f"the 7 linears, M=1: unpack + fp64 dequantize + fp64 matmul; "
                      f"{total_t:.2f} s for {total_b / 1e6:.1f} MB packed"}


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
    ap.add_argument("--calls", type=int, default=20)
    ap.add_argument("--copy-bytes", type=int, default=0)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(block rows would shard across GPUs; see the design notes). Run with --gpus 1.",
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

    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_bytes} bytes 5 times")
        return 0
    if args.only_prefill is not None:
        names = [m.name for m in wl.matrices]
        mi = synth.matrix_inputs(WORKLOAD, names.index(args.only_prefill))
        Wd = torch.from_numpy(mi.W.view(np.int16)).view(torch.bfloat16).to(dev)
        pw = msq.quantize_pack(Wd, mi.bits, mi.perm_row, mi.perm_col)
        del Wd
        M = PREFILL_M
        x = torch.from_numpy(mi.x(M).view(np.int16)).view(torch.bfloat16).to(dev)
        y = torch.empty((M, pw.N), dtype=torch.float32, device=dev)
        ws = torch.empty(max(msq.workspace_bytes(M, pw.N, pw.K), 256), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        for _ in range(args.calls):
            msq.gemm(x, pw, out=y, workspace=ws)
        torch.cuda.synchronize()
        log(f"{args.calls} prefill calls (M = {M}) on {args.only_prefill}")
        return 0
    if args.only_decode is not None:
        names = [m.name for m in wl.matrices]
        mi = synth.matrix_inputs(WORKLOAD, names.index(args.only_decode))
        Wd = torch.from_numpy(mi.W.view(np.int16)).view(torch.bfloat16).to(dev)
        pw = msq.quantize_pack(Wd, mi.bits, mi.perm_row, mi.perm_col)
        del Wd
        x = torch.from_numpy(mi.x(1).view(np.int16)).view(torch.bfloat16).to(dev)
        y = torch.empty((1, pw.N), dtype=torch.float32, device=dev)
        ws = torch.empty(max(msq.workspace_bytes(1, pw.N, pw.K), 256), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        for _ in range(args.calls):
            msq.gemm(x, pw, out=y, workspace=ws)
        torch.cuda.synchronize()
        log(f"{args.calls} decode calls on {args.only_decode}: {decode_bytes(pw, 1)} algorithmic "
            f"bytes per call")
        return 0

    # ---- inputs and pack leg -----------------------------------------------------------
    inputs, packed = [], []
    pack_ms = 0.0
    w_bytes = 0
    for mi_idx, m in enumerate(wl.matrices):
        mi = synth.matrix_inputs(WORKLOAD, mi_idx)
        log(f"pack {m.name} {m.N}x{m.K} mean bits {mi.mean_bits:.3f}")
        Wd = torch.from_numpy(mi.W.view(np.int16)).view(torch.bfloat16).to(dev)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        pw = msq.quantize_pack(Wd, mi.bits, mi.perm_row, mi.perm_col)
        e1.record()
        torch.cuda.synchronize()
        pack_ms += e0.elapsed_time(e1)
        w_bytes += 2 * m.N * m.K
        del Wd
        inputs.append(mi)
        packed.append(pw)
    torch.cuda.empty_cache()
    layer_packed = sum(p.packed_bytes for p in packed)
    mean_bits = float(sum(int(p.bits.to(torch.int64).sum().item()) for p in packed) /
                      sum(p.bits.numel() for p in packed))
    R = max(2, int(np.ceil((1 << 30) / layer_packed)))
    log(f"layer packed {layer_packed / 1e6:.1f} MB, {R} copies for cache rotation")
    copies = [packed] + [[p.clone() for p in packed] for _ in range(R - 1)]

    # ---- decode leg (M = 1), one HIP graph per weight copy -----------------------------
    M = 1
    xs = [torch.from_numpy(mi.x(M).view(np.int16)).view(torch.bfloat16).to(dev) for mi in inputs]
    ys = [torch.empty((M, p.N), dtype=torch.float32, device=dev) for p in packed]
    wss = [torch.empty(max(msq.workspace_bytes(M, p.N, p.K), 256), dtype=torch.uint8, device=dev)
           for p in packed]

    # The layer's linears in the order and grouping a decoder layer calls them:
    # q, k, v read one activation (one grouped call), then o, then gate, up read
    # one activation (one grouped call), then down.
    names = [m.name for m in wl.matrices]
    layer_groups = [[names.index(n) for n in grp] for grp in LAYER_GROUPS]
    gws = [torch.empty(max(msq.group_workspace_bytes(M, [packed[i] for i in grp]), 256),
                       dtype=torch.uint8, device=dev) for grp in layer_groups]

    def decode_step_grouped(ws_copy):
        for grp, gw in zip(layer_groups, gws):
            x = xs[grp[0]]  # the group's shared activation
            if len(grp) == 1:
                msq.gemm(x, ws_copy[grp[0]], out=ys[grp[0]], workspace=wss[grp[0]])
            else:
                msq.gemm_group([x] * len(grp), [ws_copy[i] for i in grp],
                               outs=[ys[i] for i in grp], workspace=gw)

    def decode_step_single(ws_copy):
        for i, p in enumerate(ws_copy):
            msq.gemm(xs[i], p, out=ys[i], workspace=wss[i])

    def time_steps(step_fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for cp in copies:
                step_fn(cp)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for cp in copies:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step_fn(cp)
            graphs.append(g)
        torch.cuda.synchronize()
        for s in range(args.warmup):
            graphs[s % R].replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for s in range(args.steps):
            graphs[s % R].replay()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = e0.elapsed_time(e1) / args.steps
        del graphs
        return ms, wall

    ms_single, _ = time_steps(decode_step_single)
    log(f"decode step, seven separate calls: {ms_single * 1e3:.1f} us")
    ms_per_step, t_wall = time_steps(decode_step_grouped)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    step_decode_bytes = sum(decode_bytes(p, M) for p in packed)
    value = layer_packed / (ms_per_step * 1e-3) / 1e9
    hbm_frac = step_decode_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS
    log(f"decode step {ms_per_step * 1e3:.1f} us, {value:.1f} GB/s effective, {hbm_frac:.3f} of HBM")
    decode_single = {"ms_per_step": round(ms_single, 5),
                     "value": round(layer_packed / (ms_single * 1e-3) / 1e9, 2),
                     "note": "the seven linears as seven msq_gemm calls, each with its own activation"}

    # ---- roofline leg: decode kernel on gate_proj, rotating copies --------------------
    gi = [m.name for m in wl.matrices].index("gate_proj")
    L = 4 * R
    g_roof = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_roof):
        for k in range(L):
            msq.gemm(xs[gi], copies[k % R][gi], out=ys[gi], workspace=wss[gi])
    g_roof.replay()
    torch.cuda.synchronize()
    reps = 5
    e0.record()
    for _ in range(reps):
        g_roof.replay()
    e1.record()
    torch.cuda.synchronize()
    launch_us = e0.elapsed_time(e1) * 1e3 / (reps * L)
    per_launch = decode_bytes(packed[gi], M)
    achieved = per_launch / (launch_us * 1e-6) / 1e9
    sha = kernel_source_sha()
    traffic = measured_traffic(sha)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic,
                "kernel": "msq_gemm M=1 on gate_proj 28672x8192: k_gemv_m1 reordering x in its "
                          "workgroups (one launch per call, launch gaps included)",
                "bytes_per_launch": per_launch, "avg_launch_us": round(launch_us, 3),
                "kernel_sha": sha}
    log(f"roofline: {launch_us:.2f} us/launch, {achieved:.0f} GB/s")

    # ---- prefill leg (M = 2048) --------------------------------------------------------
    prefill = None
    if not args.no_prefill:
        Mp = PREFILL_M
        del g_roof
        xp = [torch.from_numpy(mi.x(Mp).view(np.int16)).view(torch.bfloat16).to(dev) for mi in inputs]
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
            e0.record()
            for s in range(args.prefill_steps):
                step_fn(copies[s % R])
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / args.prefill_steps

        ms_single = time_prefill(prefill_single)
        ms_p = time_prefill(prefill_grouped)
        flops = sum(prefill_flops(p, Mp) for p in packed)
        tflops = flops / (ms_p * 1e-3) / 1e12
        prefill = {"M": Mp, "ms_per_step": round(ms_p, 4), "tflops": round(tflops, 2),
                   "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                   "peak_tflops": MFMA_BF16_PEAK_TFLOPS, "flops_per_step": flops,
                   "grouping": "q/k/v and gate/up grouped as in the decode step",
                   "ms_per_step_separate_calls": round(ms_single, 4)}
        log(f"prefill M={Mp}: {ms_p:.3f} ms/step grouped, {tflops:.1f} TFLOP/s "
            f"({ms_single:.3f} ms/step as separate calls)")
        del xp, yp, wsp, gwsp

    pack = {"ms": round(pack_ms, 3), "weight_bytes": w_bytes,
            "gbps_read": round(w_bytes / (pack_ms * 1e-3) / 1e9, 1),
            "note": "host-side descriptor validation included"}

    alloc = alloc_leg(msq, synth, torch, log)
    reorder = reorder_leg(msq, torch, log)
    tile16 = tile16_leg(msq, synth, torch, np, log)

    configs, context = None, None
    if not args.no_configs:
        del copies
        torch.cuda.empty_cache()
        configs = config_legs(msq, synth, torch, np, dev, log)
        context = achievable_context(torch, dev, log)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(inputs)
        log(f"cpu baseline {cpu['value']} GB/s")

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3-70b-layer decode M=1: q,o 8192x8192; k,v 1024x8192; "
                               "gate,up 28672x8192; down 8192x28672",
                   "M": M, "mean_bits": round(mean_bits, 4), "packed_bytes": layer_packed,
                   "decode_bytes": step_decode_bytes, "weight_copies": R,
                   "timing": "HIP graph per weight copy, events around the timed replays"},
        "hbm_frac": round(hbm_frac, 4),
        "decode_separate_calls": decode_single,
        "prefill": prefill,
        "pack": pack,
        "alloc": alloc,
        "reorder": reorder,
        "tile16": tile16,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "configs": configs,
        "context": context,
        "wall_s_timed": round(t_wall, 4),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
