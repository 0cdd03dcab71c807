#!/usr/bin/env python3
"""Benchmark of the packed b-bit weight path on one MI355X.

One step = one pass of the whole path over the synthetic workload:
  1. quantize + pack the five 4096x4096 decode matrices (b = 4, 5, 6, 7, 8);
  2. unpack them back to int32 codes;
  3. quantize + pack the four 8192x8192 prefill matrices (b = 5, 6, 8, 12);
  4. GEMM x[2048, 8192] . W^T for each prefill matrix;
  5. decode: for each of 8 tokens, GEMV x_t[1, 4096] . W^T for each decode
     matrix; token t reads its own copy of the five packed matrices (copy 0 is
     the one step 1 writes; copies 1..7 hold the same bits, written before
     timing), 503 MB in all, so no launch finds its weights in the 256 MB
     last-level cache.
The 40 GEMV launches form one timed group: one pair of HIP events costs about
4.5 us, which spread over only five launches would add ~0.9 us to each.

Reported ``value`` is the metric's first half: packed-weight GB/s of the M=1
GEMV (sum of packed bytes over the sum of the GEMV kernel times, measured with
HIP events on the launch stream).  The GEMM's TFLOP/s (the metric's second
half) is reported in ``roofline_gemm``.  Every input is resident in HBM before
the timed region.  The CPU baseline is the oracle's fp64 GEMV on the same
decode matrices, timed on the host cores.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores

# decode: the five matrices for `tokens` decode tokens, token t reading copy t
# of the packed matrices (copies x 63 MB > the 256 MB last-level cache)
DECODE = dict(N=4096, K=4096, bits=(4, 5, 6, 7, 8), M=1, tokens=8)
PREFILL = dict(N=8192, K=8192, bits=(5, 6, 8, 12), M=2048)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_traffic.json")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-stack", action="store_true",
                   help="skip the context measurement over the 448-matrix layer stack")
    p.add_argument("--sweep", action="store_true",
                   help="instead of the step: every bit width 2..15 on the 28672x8192 matrix "
                        "(quantize + pack, GEMV at M=1 and 16, GEMM at M=256), one JSON line")
    p.add_argument("--copy-calibration", action="store_true",
                   help="after the timed steps, copy 256 MiB device to device once (a plain copy "
                        "of known size for scaling hardware byte counters)")
    return p.parse_args()


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixed_precision_weight_dq_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f in ("gemv_batch.hip", "gemv_kernels.hpp", "gemm_tiles.hpp", "common.hpp"):
            # code only: whole-line comments do not change the kernel
            for line in open(os.path.join(csrc, f), "rb"):
                if not line.lstrip().startswith(b"//"):
                    h.update(line)
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per batched decode launch from the committed rocprofv3 counter
    summary, if it was taken on the current source of that kernel; else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != kernel_source_digest():
        return None
    return rec.get("bytes_per_launch_avg")


def stack_context(torch, dq, workload, dev, stream):
    """Context for the GEMV figure, outside the timed steps: the 448-matrix
    layer stack (64 layers x 4 x 5120x5120, 2 x 17408x5120, 5120x17408 at the
    knee bit allocation), weights drawn on the GPU (seeded) and quantized once;
    then GEMV at M = 1 and M = 8 over every matrix in layer order."""
    shapes, recipe = workload.stack_shapes(), workload.stack_bits()
    gen = torch.Generator(device=dev)
    packs, total, sums = [], 0, []
    for idx, ((N, K), b) in enumerate(zip(shapes, recipe)):
        gen.manual_seed(3000 + idx)
        W = (torch.randn((N, K), generator=gen, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
        sums.append(dq.row_sumsq(W)[1])  # mean(w^2) for the allocation context
        P, S = dq.quantize_pack(W, b)
        packs.append((P, S, K, b, N))
        total += N * K * b // 8
        del W
    torch.cuda.synchronize()
    sumsq = torch.cat(sums).cpu().numpy()
    del sums
    xs = {K: torch.from_numpy(workload.activations(3, K, 8, K).view(np.int16)).view(torch.bfloat16).to(dev)
          for K in {k for _, k in shapes}}
    ys = {(N, M): torch.empty((M, N), dtype=torch.float32, device=dev)
          for N in {n for n, _ in shapes} for M in (1, 8)}
    out = {}
    lib = dq.load()
    for M in (1, 8):
        # C entry point with prepared arguments (the tensor wrapper's checks
        # would cost the host more than the smaller GEMVs take)
        calls = [(xs[K].data_ptr(), M, P.data_ptr(), S.data_ptr(), N, K, b, ys[(N, M)].data_ptr(),
                  stream.cuda_stream) for P, S, K, b, N in packs]

        def one_pass():
            for a in calls:
                if lib.dq_gemv(*a):
                    raise RuntimeError("dq_gemv failed")
        one_pass()
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            one_pass()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = float(np.median(ts))
        out["m%d" % M] = {"ms_per_pass": round(ms, 3), "gbs": round(total / (ms * 1e-3) / 1e9, 1),
                          "frac_of_hbm_peak": round(total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    # batched: one dq_gemv_batched per layer (its 7 matrices), and one per
    # group of matrices a layer can multiply at once (q/k/v on one activation,
    # o, gate/up on one activation, down); every item its own output
    per_layer = 7
    yl = {M: [torch.empty((M, N), dtype=torch.float32, device=dev) for N, _ in shapes[:per_layer]]
          for M in (1, 8)}
    groupings = {"layer": [list(range(per_layer))], "dependency_groups": [[0, 1, 2], [3], [4, 5], [6]]}
    keep = []
    for M in (1, 8):
        for gname, groups in groupings.items():
            calls = []
            for l0 in range(0, len(packs), per_layer):
                for grp in groups:
                    arr = (dq.DQGemvItem * len(grp))()
                    for i, j in enumerate(grp):
                        P, S, K, b, N = packs[l0 + j]
                        arr[i] = dq.DQGemvItem(xs[K].data_ptr(), P.data_ptr(), S.data_ptr(),
                                               yl[M][j].data_ptr(), N, K, b)
                    keep.append(arr)
                    calls.append((ctypes.addressof(arr), len(grp), M, stream.cuda_stream))

            def one_pass(calls=calls):
                for a in calls:
                    if lib.dq_gemv_batched(*a):
                        raise RuntimeError("dq_gemv_batched failed")
            one_pass()
            torch.cuda.synchronize()
            ts = []
            for _ in range(3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                one_pass()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            ms = float(np.median(ts))
            out["m%d_batched_per_%s" % (M, gname)] = {
                "ms_per_pass": round(ms, 3), "launches_per_pass": len(calls),
                "gbs": round(total / (ms * 1e-3) / 1e9, 1),
                "frac_of_hbm_peak": round(total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del packs, keep
    out["packed_gb"] = round(total / 1e9, 3)
    out["what"] = ("decode GEMV over the 448-matrix layer stack (17.8 GB packed, mostly 6-bit), "
                   "every matrix in layer order per pass: m1/m8 one dq_gemv launch per matrix; "
                   "*_batched_per_layer one dq_gemv_batched launch per layer (7 matrices); "
                   "*_batched_per_dependency_groups one per group a layer multiplies at once "
                   "(q/k/v, o, gate/up, down: 4 per layer); packed-weight GB/s; context, not "
                   "the value")
    return out, sumsq


def allocation_context(dq, workload, sumsq, reps: int = 20):
    """The allocation step on the 448-matrix stack, outside the timed steps:
    sensitivities from the GPU-measured sum(w^2) of every matrix and synthetic
    Hessian traces, then the full-mode recipe at 5.7 bits per parameter (the
    DynaQuant knee) and the hardware-native one at the same budget."""
    params = np.array([n * k for n, k in workload.stack_shapes()], dtype=np.int64)
    h = workload.hessian_traces(3, len(params))
    sens = dq.sensitivity(h, sumsq, params)
    budget = int(5.7 * int(params.sum()))
    out = {}
    for name, levels in (("full", dq.FULL_LEVELS), ("native", dq.NATIVE_LEVELS)):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            bits, steps, loss = dq.allocate_bits(sens, params, levels, budget)
            ts.append(time.perf_counter() - t0)
        hist = {str(b): int((bits == b).sum()) for b in sorted(set(bits.tolist()))}
        out[name] = {
            "recipe": hist, "steps": len(steps),
            "avg_bits": round(float((bits.astype(np.int64) * params).sum()) / float(params.sum()), 4),
            "call_us": round(float(np.median(ts)) * 1e6, 1),
        }
    out["what"] = ("water-filling allocation over the 448 matrices at 5.7 bits per parameter: "
                   "sum(w^2) measured on the GPU (dq_row_sumsq), synthetic Hessian traces, host "
                   "call time of dq_allocate_bits (Python marshalling included)")
    return out, (sens, params, budget)


def asym_context(torch, dq, stream, W2, X1t, W4, X4, reps: int):
    """The asymmetric (zero-point) variant, outside the timed steps, on the
    step's own inputs: quantize + pack of the five 4096^2 decode matrices, the
    decode group (8 tokens x 5 GEMVs on 8 rotated copies) and the b = 6
    prefill GEMM, each beside the symmetric figure of the same run."""
    Nd, Kd = next(iter(W2.values())).shape
    q = {b: dq.quantize_pack_asym(W, b) for b, W in W2.items()}
    copies = [q] + [{b: (P.clone(), S, Z) for b, (P, S, Z) in q.items()} for _ in range(len(X1t) - 1)]
    ys = {b: torch.empty((1, Nd), dtype=torch.float32, device=W.device) for b, W in W2.items()}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    def quant():
        for b, W in W2.items():
            dq.quantize_pack_asym(W, b)

    # raw C calls with the addresses taken beforehand (the tensor wrappers'
    # checks cost more host time than a 4096^2 GEMV takes on the GPU)
    cs = stream.cuda_stream
    lib = dq.load()
    calls = []
    for t, X in enumerate(X1t):
        for b, (P, S, Z) in copies[t].items():
            calls.append((lib.dq_gemv_asym, (X.data_ptr(), 1, P.data_ptr(), S.data_ptr(),
                                             Z.data_ptr(), Nd, Kd, b, ys[b].data_ptr(), cs)))

    def decode():
        for fn, a in calls:
            fn(*a)

    # the same products as one dq_gemv_batched launch per token
    tables = []
    for t, X in enumerate(X1t):
        arr = (dq.DQGemvItem * len(copies[t]))()
        for i, (b, (P, S, Z)) in enumerate(copies[t].items()):
            arr[i] = dq.DQGemvItem(X.data_ptr(), P.data_ptr(), S.data_ptr(), ys[b].data_ptr(), Nd, Kd,
                                   b, 0, Z.data_ptr())
        tables.append(arr)

    def decode_batched():
        for arr in tables:
            if lib.dq_gemv_batched(ctypes.addressof(arr), len(arr), 1, cs):
                raise RuntimeError("dq_gemv_batched failed")

    b6 = 6
    P6, S6, Z6 = dq.quantize_pack_asym(W4[b6], b6)
    Y = torch.empty((X4.shape[0], P6.shape[0]), dtype=torch.float32, device=X4.device)

    def gemm():
        dq.gemm_asym(X4, P6, S6, Z6, X4.shape[1], b6, y=Y)

    t_q, t_d, t_g = timed(quant), timed(decode), timed(gemm)
    t_b = timed(decode_batched)
    dec_bytes = len(X1t) * sum(Nd * Kd * b // 8 for b in W2)
    q_bytes = sum(Nd * Kd * (16 + b) // 8 for b in W2)
    M, K = X4.shape
    N = P6.shape[0]
    return {"quantize_pack_4096_gbs": round(q_bytes / (t_q * 1e-3) / 1e9, 1),
            "gemv_m1_gbs": round(dec_bytes / (t_b * 1e-3) / 1e9, 1),
            "gemv_m1_per_launch_us": round(t_b / len(X1t) * 1e3, 3),
            "gemv_m1_per_matrix_gbs": round(dec_bytes / (t_d * 1e-3) / 1e9, 1),
            "gemm_2048_b6_tflops": round(2.0 * M * N * K / (t_g * 1e-3) / 1e12, 1),
            "what": "asymmetric scheme on the step's inputs: quantize+pack (read + write bytes), "
                    "decode GEMV M=1 over 8 tokens x b=4..8 on rotated copies, one "
                    "dq_gemv_batched launch per token (packed-weight GB/s; per_matrix: one "
                    "dq_gemv_asym launch per matrix), prefill GEMM M=2048 b=6; the products "
                    "subtract each row's zero point from its codes; median of the step count, "
                    "outside the timed steps"}


def group_context(torch, dq, stream, W2, X1t, W4, X4, reps: int, group: int = 128):
    """Group-wise scales (one per 128 codes), outside the timed steps, on the
    step's own inputs: quantize + pack of the five decode matrices, the decode
    group (8 tokens x 5 GEMVs on rotated copies) and the b = 6 prefill GEMM."""
    Nd, Kd = next(iter(W2.values())).shape
    q = {b: dq.quantize_pack_group(W, b, group) for b, W in W2.items()}
    copies = [q] + [{b: (P.clone(), S) for b, (P, S) in q.items()} for _ in range(len(X1t) - 1)]
    ys = {b: torch.empty((1, Nd), dtype=torch.float32, device=W.device) for b, W in W2.items()}
    cs = stream.cuda_stream
    lib = dq.load()
    calls = [(lib.dq_gemv_group, (X.data_ptr(), 1, P.data_ptr(), S.data_ptr(), Nd, Kd, b, group,
                                  ys[b].data_ptr(), cs))
             for t, X in enumerate(X1t) for b, (P, S) in copies[t].items()]
    # M = 16 (the token activations stacked twice): group-wise scales in the
    # matrix-core GEMV, and the per-row scheme on the same matrices beside it
    X16 = torch.cat([X1t[i % len(X1t)] for i in range(16)], 0).contiguous()
    y16 = torch.empty((16, Nd), dtype=torch.float32, device=X16.device)
    sym = {b: dq.quantize_pack(W, b) for b, W in W2.items()}
    sym_copies = [sym] + [{b: (P.clone(), S) for b, (P, S) in sym.items()} for _ in range(len(X1t) - 1)]
    calls16 = [(lib.dq_gemv_group, (X16.data_ptr(), 16, P.data_ptr(), S.data_ptr(), Nd, Kd, b, group,
                                    y16.data_ptr(), cs))
               for t in range(len(X1t)) for b, (P, S) in copies[t].items()]
    calls16_sym = [(lib.dq_gemv, (X16.data_ptr(), 16, P.data_ptr(), S.data_ptr(), Nd, Kd, b,
                                  y16.data_ptr(), cs))
                   for t in range(len(X1t)) for b, (P, S) in sym_copies[t].items()]

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    def quant():
        for b, W in W2.items():
            dq.quantize_pack_group(W, b, group)

    def decode():
        for fn, a in calls:
            fn(*a)

    # the same products as one dq_gemv_batched launch per token
    tables = []
    for t, X in enumerate(X1t):
        arr = (dq.DQGemvItem * len(copies[t]))()
        for i, (b, (P, S)) in enumerate(copies[t].items()):
            arr[i] = dq.DQGemvItem(X.data_ptr(), P.data_ptr(), S.data_ptr(), ys[b].data_ptr(), Nd, Kd,
                                   b, group, 0)
        tables.append(arr)

    def decode_batched():
        for arr in tables:
            if lib.dq_gemv_batched(ctypes.addressof(arr), len(arr), 1, cs):
                raise RuntimeError("dq_gemv_batched failed")

    def decode16():
        for fn, a in calls16:
            fn(*a)

    def decode16_sym():
        for fn, a in calls16_sym:
            fn(*a)

    P6, S6 = dq.quantize_pack_group(W4[6], 6, group)
    Y = torch.empty((X4.shape[0], P6.shape[0]), dtype=torch.float32, device=X4.device)

    def gemm():
        dq.gemm_group(X4, P6, S6, X4.shape[1], 6, group, Y)

    t_q, t_d, t_g = timed(quant), timed(decode), timed(gemm)
    t_b = timed(decode_batched)
    t_16, t_16s = timed(decode16), timed(decode16_sym)
    G = -(-Kd // group)
    dec_bytes = len(X1t) * sum(Nd * (Kd * b // 8 + G * 4) for b in W2)
    payload = len(X1t) * sum(Nd * Kd * b // 8 for b in W2)
    q_bytes = sum(Nd * (Kd * (16 + b) // 8 + G * 4) for b in W2)
    M, K = X4.shape
    N = P6.shape[0]
    return {"group": group,
            "quantize_pack_4096_gbs": round(q_bytes / (t_q * 1e-3) / 1e9, 1),
            "gemv_m1_gbs": round(dec_bytes / (t_b * 1e-3) / 1e9, 1),
            "gemv_m1_per_launch_us": round(t_b / len(tables) * 1e3, 3),
            "gemv_m1_per_matrix_gbs": round(dec_bytes / (t_d * 1e-3) / 1e9, 1),
            "gemv_m16_packed_gbs": round(payload / (t_16 * 1e-3) / 1e9, 1),
            "gemv_m16_per_row_scales_packed_gbs": round(payload / (t_16s * 1e-3) / 1e9, 1),
            "gemm_2048_b6_tflops": round(2.0 * M * N * K / (t_g * 1e-3) / 1e12, 1),
            "what": "group-wise scales (g=128) on the step's inputs: quantize+pack (read + write "
                    "bytes), decode GEMV M=1 over 8 tokens x b=4..8 on rotated copies, one "
                    "dq_gemv_batched launch per token (packed words + group scales per second; "
                    "per_matrix: one dq_gemv_group launch per matrix), the same at M=16 (packed words per second; "
                    "beside it the per-row scheme on the same matrices), prefill GEMM M=2048 b=6 (pipelined 128-row tiles, each group folded in as it ends); "
                    "median of the step count, outside the timed steps"}


def packed_file_context(torch, dq, stream, packs, reps: int = 5):
    """The on-disk format, outside the timed steps: the five packed decode
    matrices written to a temporary file, mapped, checked and copied back into
    device buffers (pageable host memory -> HBM over PCIe; the file sits in the
    page cache after the write)."""
    import tempfile
    mats = [("decode_b%d" % b, P.shape[0], K, b, P.cpu().numpy(), S.cpu().numpy())
            for b, (P, S, K) in packs.items()]
    nbytes = sum(m[4].nbytes + m[5].nbytes for m in mats)
    with tempfile.TemporaryDirectory() as d:
        path = d + "/decode.dqw"
        t0 = time.perf_counter()
        dq.write_packed_file(path, mats)
        t_write = time.perf_counter() - t0
        dst = [(torch.empty_like(P), torch.empty_like(S)) for P, S, _ in packs.values()]
        with dq.PackedFile(path) as pf:
            t0 = time.perf_counter()
            ok = all(pf.verify(i) for i in range(len(pf)))
            t_verify = time.perf_counter() - t0
            ts = []
            for _ in range(reps):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for i, (P, S) in enumerate(dst):
                    dq._check(dq.load().dq_file_load(pf._h, i, P.data_ptr(), S.data_ptr(),
                                                     stream.cuda_stream), "dq_file_load")
                torch.cuda.synchronize()
                ts.append(time.perf_counter() - t0)
        same = all(torch.equal(a, P) and torch.equal(b, S)
                   for (a, b), (P, S, _) in zip(dst, packs.values()))
    t_load = float(np.median(ts))
    return {"bytes": nbytes, "write_gbs": round(nbytes / t_write / 1e9, 2),
            "verify_gbs": round(nbytes / t_verify / 1e9, 2),
            "load_to_hbm_gbs": round(nbytes / t_load / 1e9, 2), "checksums_ok": ok,
            "loaded_equal": bool(same),
            "what": "five packed 4096x4096 decode matrices (b=4..8) + scales: file write, "
                    "FNV-1a verify, and dq_file_load of every entry into HBM (page cache -> "
                    "pageable hipMemcpyAsync; PCIe-bound, context only)"}


def row_sumsq_context(torch, dq, stream, mats, reps: int):
    """dq_row_sumsq over the given bf16 matrices back to back (more bytes than
    the 256 MB last-level cache, so each is read from HBM), median of reps."""
    nbytes = sum(w.numel() * 2 + w.shape[0] * 8 for w in mats)
    rows = [torch.empty((w.shape[0],), dtype=torch.float64, device=w.device) for w in mats]
    tot = [torch.empty((1,), dtype=torch.float64, device=w.device) for w in mats]

    def group(with_total):
        for w, r, t in zip(mats, rows, tot):
            dq._check(dq.dq_row_sumsq(w.data_ptr(), dq.DQ_BF16, w.shape[0], w.shape[1],
                                      r.data_ptr(), t.data_ptr() if with_total else 0,
                                      stream.cuda_stream), "dq_row_sumsq")

    def timed(with_total):
        group(with_total)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            group(with_total)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))
    ms_rows, ms_tot = timed(False), timed(True)
    g = nbytes / (ms_rows * 1e-3) / 1e9
    return {"kernel": "dq_row_sumsq row sums over %d bf16 %dx%d matrices back to back"
                      % (len(mats), mats[0].shape[0], mats[0].shape[1]),
            "bound": "hbm", "gbs": round(g, 1), "frac_of_hbm_peak": round(g / HBM_PEAK_GBS, 4),
            "per_matrix_us": round(ms_rows / len(mats) * 1e3, 2),
            "with_matrix_total_us": round(ms_tot / len(mats) * 1e3, 2),
            "bytes": "N*K*2 read + N*8 written per matrix"}


def attainable_read(torch, dq, dev, stream, gemv_group, read_bufs, flush, reps: int,
                    per_matrix_group=None, per_matrix_launches: int = 0):
    """Context for the GEMV figure, outside the timed steps: the decode GEMV
    launches of a step (one batched launch per token) against a plain
    streaming read (dq_stream_read) of the same packed bytes in as many
    launches (each token's buffer), each group timed after the same
    cache-flushing GEMM; the same matrices with one dq_gemv launch each; plus
    the read rate of a 1 GiB buffer and the back-to-back launch floor.  The
    read's share count is the best of four."""
    nbytes = sum(b.numel() * b.element_size() for b in read_bufs)
    n = len(read_bufs)

    def timed(group):
        ts = []
        for _ in range(reps):
            flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            group()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    parts = {}
    for per in (256, 512, 1024, 2048):
        outs = [torch.empty((max(1, min(65536, b.numel() * b.element_size() // 16 // per)),),
                            dtype=torch.int32, device=dev) for b in read_bufs]
        lib = dq.load()
        calls = [(lib.dq_stream_read, (b.data_ptr(), b.numel() * b.element_size(), o.data_ptr(),
                                       o.shape[0], stream.cuda_stream)) for b, o in zip(read_bufs, outs)]
        parts[per] = (outs, timed(lambda calls=calls: [fn(*a) for fn, a in calls]))
    per, (outs, read_ms) = min(parts.items(), key=lambda kv: kv[1][1])
    gemv_ms = timed(gemv_group)
    single_ms = timed(per_matrix_group) if per_matrix_group is not None else None
    big = torch.empty(1 << 28, dtype=torch.int32, device=dev).fill_(1)
    big_out = torch.empty((65536,), dtype=torch.int32, device=dev)
    dq.stream_read(big, 65536, big_out)
    torch.cuda.synchronize()
    big_ms = timed(lambda: dq.stream_read(big, 65536, big_out))
    # launch floor: n back-to-back reads of 16 KB (1024 workgroups) from the same buffer
    tiny = (lib.dq_stream_read, (big.data_ptr(), 16384, big_out.data_ptr(), 1024, stream.cuda_stream))
    floor_ms = timed(lambda: [tiny[0](*tiny[1]) for _ in range(n)])
    del big
    read_gbs = nbytes / (read_ms * 1e-3) / 1e9
    gemv_gbs = nbytes / (gemv_ms * 1e-3) / 1e9
    out = {
        "what": "plain streaming read (dq_stream_read) of the step's %d token buffers (each the "
                "five packed 4096x4096 matrices b=4..8 of one token, 63 MB), one launch each, vs "
                "the %d batched GEMV launches on them; each group after the same b=6 prefill "
                "GEMM, median of %d; bytes = packed words; context, not the value" % (n, n, reps),
        "read_gbs": round(read_gbs, 1),
        "read_per_launch_us": round(read_ms / n * 1e3, 3),
        "read_shares": sorted({o.shape[0] for o in outs}),
        "gemv_gbs": round(gemv_gbs, 1),
        "gemv_per_launch_us": round(gemv_ms / n * 1e3, 3),
        "gemv_frac_of_read": round(gemv_gbs / read_gbs, 4),
        "read_1gib_gbs": round((1 << 30) / (big_ms * 1e-3) / 1e9, 1),
        "launch_floor_us": round(floor_ms / n * 1e3, 3),
        "launch_floor_what": "per-launch time of %d back-to-back 16 KB plain reads: the fixed "
                             "cost every launch pays here" % n,
    }
    if single_ms is not None:
        out["per_matrix"] = {
            "gbs": round(nbytes / (single_ms * 1e-3) / 1e9, 1),
            "per_launch_us": round(single_ms / per_matrix_launches * 1e3, 3),
            "frac_of_hbm_peak": round(nbytes / (single_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "what": "the same 40 matrix products as one dq_gemv launch each (the per-matrix "
                    "figure), same flush and timing"}
    return out


def cpu_baseline(decode_w, x1, target_s: float, allocation=None):
    """The oracle's fp64 GEMV (unpack bit by bit + dot product) over the decode
    matrices, repeated until about target_s seconds of CPU time; and, given the
    stack's allocation inputs, the oracle's allocator on them."""
    import oracle
    from oracle import recipe as orc
    alloc = None
    if allocation is not None:
        sens, params, budget = allocation
        alloc = {}
        for name, levels in (("full", orc.FULL_LEVELS), ("native", orc.NATIVE_LEVELS)):
            t0 = time.perf_counter()
            orc.allocate(sens, params, levels, budget)
            alloc[name + "_ms"] = round((time.perf_counter() - t0) * 1e3, 2)
    packs = []
    for b, w in decode_w.items():
        p, s, _ = oracle.quantize_pack(w, b)
        packs.append((b, p, s))
    done_bytes, reps = 0, 0
    t0 = time.perf_counter()
    while True:
        for b, p, s in packs:
            oracle.matmul(x1, p, s, DECODE["N"], DECODE["K"], b)
            done_bytes += DECODE["N"] * DECODE["K"] * b // 8
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    # one host thread, one pass over the b = 6 decode matrix
    cores = oracle.max_threads()
    b6p = next((p, s) for b, p, s in packs if b == 6)
    oracle.set_threads(1)
    try:
        t1 = time.perf_counter()
        oracle.matmul(x1, b6p[0], b6p[1], DECODE["N"], DECODE["K"], 6)
        one_thread = DECODE["N"] * DECODE["K"] * 6 / 8 / (time.perf_counter() - t1) / 1e9
    finally:
        oracle.set_threads(cores)
    # the oracle's asymmetric and group-wise products on one decode matrix
    # (b = 6), beside the GPU figures of the same variants
    variants = {}
    w6 = decode_w[6]
    N, K = DECODE["N"], DECODE["K"]
    for name, prep, run in (
            ("asymmetric", lambda: oracle.quantize_pack_asym(w6, 6)[:3],
             lambda q: oracle.matmul_asym(x1, q[0], q[1], q[2], N, K, 6)),
            ("group_scales_128", lambda: oracle.quantize_pack_group(w6, 6, 128)[:2],
             lambda q: oracle.matmul_group(x1, q[0], q[1], N, K, 6, 128))):
        q = prep()
        t0 = time.perf_counter()
        run(q)
        variants[name + "_gemv_gbs"] = round(N * K * 6 / 8 / (time.perf_counter() - t0) / 1e9, 4)
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "one_thread_b6_gbs": round(one_thread, 4),
            "sample": "fp64 GEMV M=1 over the five 4096x4096 decode matrices (b=4..8), "
                      "%d passes, %.1f s" % (reps, el),
            "cpu": cpu, "allocation_oracle": alloc, "variants_oracle": variants}


def device_info(torch, dev) -> dict:
    """What the run ran on (the peaks above are MI355X's published figures)."""
    p = torch.cuda.get_device_properties(dev)
    info = {"name": p.name, "compute_units": p.multi_processor_count,
            "memory_gb": round(p.total_memory / 1e9, 1)}
    arch = getattr(p, "gcnArchName", None)
    if arch:
        info["arch"] = arch
    # peak engine clock as the runtime reports it (hipDeviceAttributeClockRate,
    # enum value 5, in kHz; looked up through the library's handle, so it is the
    # HIP runtime the library runs on), and the dense bf16 matrix peak scaled to
    # it from 2.5 PFLOP/s at 2.4 GHz on 256 CUs
    try:
        import ctypes
        import mixed_precision_weight_dq_amd as dq
        khz = ctypes.c_int(0)
        if dq.load().hipDeviceGetAttribute(ctypes.byref(khz), 5, ctypes.c_int(dev.index or 0)) == 0 \
                and khz.value > 0:
            info["peak_clock_mhz"] = round(khz.value / 1e3)
            info["bf16_peak_at_that_clock_tflops"] = round(
                MFMA_BF16_PEAK_TFLOPS * khz.value / 2.4e6 * p.multi_processor_count / 256, 1)
    except (OSError, AttributeError):
        pass
    return info


def sweep(torch, dq, workload, dev, stream, reps: int):
    """Workload 5 at every width: W[28672, 8192] Student-t(5) (std 0.02), x N(0, 1).
    Each launch is timed alone with HIP events right after a cache-flushing bf16
    GEMM (so its operands come from HBM), median of `reps`; per-launch times
    include the launch overhead of one kernel."""
    wl = workload.WORKLOADS[5]
    N, K = wl.N, wl.K
    W = torch.from_numpy(workload.workload_weights(wl, 0).view(np.int16)).view(torch.bfloat16).to(dev)
    x16 = torch.from_numpy(workload.activations(5, 0, 256, K).view(np.int16)).view(torch.bfloat16).to(dev)
    ga = torch.randn((4096, 8192), device=dev).to(torch.bfloat16)
    gb = torch.randn((8192, 4096), device=dev).to(torch.bfloat16)

    def timed(fn):
        ts = []
        for _ in range(reps):
            torch.matmul(ga, gb)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(ts))

    rows = []
    for b in range(2, 16):
        rb = dq.packed_row_bytes(K, b)
        P = torch.empty((N, rb // 4), dtype=torch.int32, device=dev)
        S = torch.empty((N,), dtype=torch.float32, device=dev)
        dq.quantize_pack(W, b, P, S)
        y1 = torch.empty((1, N), dtype=torch.float32, device=dev)
        y16 = torch.empty((16, N), dtype=torch.float32, device=dev)
        y256 = torch.empty((256, N), dtype=torch.float32, device=dev)
        x1, xs = x16[:1], x16[:16]
        tq = timed(lambda: dq.quantize_pack(W, b, P, S))
        t1 = timed(lambda: dq.gemv(x1, P, S, K, b, y1))
        t16 = timed(lambda: dq.gemv(xs, P, S, K, b, y16))
        tg = timed(lambda: dq.gemm(x16, P, S, K, b, y256))
        packed = N * K * b / 8
        rows.append({
            "bits": b, "packed_mb": round(packed / 1e6, 1),
            "quantize_us": round(tq, 1), "quantize_gbs": round((N * K * 2 + N * rb) / tq / 1e3, 1),
            "gemv_m1_us": round(t1, 1), "gemv_m1_gbs": round(packed / t1 / 1e3, 1),
            "gemv_m16_us": round(t16, 1), "gemv_m16_gbs": round(packed / t16 / 1e3, 1),
            "gemm_m256_us": round(tg, 1), "gemm_m256_tflops": round(2.0 * 256 * N * K / tg / 1e6, 1),
        })
        del P, S, y1, y16, y256
    return {
        "sweep": "workload 5: W 28672x8192 bf16 Student-t(5) std 0.02, x N(0,1); every bit width",
        "timing": "one launch after a cache-flushing bf16 GEMM, HIP events, median of %d; "
                  "includes one launch overhead" % reps,
        "peaks": {"hbm_gbs": HBM_PEAK_GBS, "bf16_tflops": MFMA_BF16_PEAK_TFLOPS},
        "device": device_info(torch, dev),
        "rows": rows,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library runs on one GPU, with no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixed_precision_weight_dq_amd as dq
    import workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    if args.sweep:
        print(json.dumps(sweep(torch, dq, workload, dev, stream, reps=max(5, args.steps // 4))))
        return

    def bf16(u16):
        return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- inputs (seeded, synthetic), resident in HBM before timing
    wl2, wl4 = workload.WORKLOADS[2], workload.WORKLOADS[4]
    decode_np = {b: workload.workload_weights(wl2, i) for i, b in enumerate(DECODE["bits"])}
    x1_np = workload.activations(2, 0, DECODE["M"], DECODE["K"])
    W2 = {b: bf16(w) for b, w in decode_np.items()}
    X1 = bf16(x1_np)
    X1t = [X1] + [bf16(workload.activations(2, t, DECODE["M"], DECODE["K"]))
                  for t in range(1, DECODE["tokens"])]
    W4 = {b: bf16(workload.workload_weights(wl4, i)) for i, b in enumerate(PREFILL["bits"])}
    X4 = bf16(workload.activations(4, 0, PREFILL["M"], PREFILL["K"]))

    def rw(K, b):
        return dq.packed_row_bytes(K, b) // 4

    # each token's five packed matrices lie back to back in one buffer (token t
    # reads copy t), so a plain read of exactly those bytes is one launch too
    words = {b: DECODE["N"] * rw(DECODE["K"], b) for b in W2}
    tok_bufs = [torch.empty((sum(words.values()),), dtype=torch.int32, device=dev)
                for _ in range(DECODE["tokens"])]

    def token_views(buf):
        out, off = {}, 0
        for b in W2:
            out[b] = buf[off:off + words[b]].view(DECODE["N"], rw(DECODE["K"], b))
            off += words[b]
        return out
    P2t = [token_views(buf) for buf in tok_bufs]
    P2 = P2t[0]
    S2 = {b: torch.empty((DECODE["N"],), dtype=torch.float32, device=dev) for b in W2}
    Q2 = {b: torch.empty((DECODE["N"], DECODE["K"]), dtype=torch.int32, device=dev) for b in W2}
    Y1 = {b: torch.empty((1, DECODE["N"]), dtype=torch.float32, device=dev) for b in W2}
    for b in W2:
        dq.quantize_pack(W2[b], b, P2[b], S2[b])
    for t in range(1, DECODE["tokens"]):
        tok_bufs[t].copy_(tok_bufs[0])
    P4 = {b: torch.empty((PREFILL["N"], rw(PREFILL["K"], b)), dtype=torch.int32, device=dev) for b in W4}
    S4 = {b: torch.empty((PREFILL["N"],), dtype=torch.float32, device=dev) for b in W4}
    Y4 = torch.empty((PREFILL["M"], PREFILL["N"]), dtype=torch.float32, device=dev)

    ops = []  # (kind, b, callable)
    for b in W2:
        ops.append(("quantize_pack_4096", b, lambda b=b: dq.quantize_pack(W2[b], b, P2[b], S2[b])))
    for b in W2:
        ops.append(("unpack_4096", b, lambda b=b: dq._check(dq.dq_unpack(
            P2[b].data_ptr(), 0, DECODE["N"], DECODE["K"], b, Q2[b].data_ptr(), 0,
            stream.cuda_stream), "dq_unpack")))
    for b in W4:
        ops.append(("quantize_pack_8192", b, lambda b=b: dq.quantize_pack(W4[b], b, P4[b], S4[b])))
    for b in W4:  # one event group per GEMM (each runs for hundreds of microseconds)
        ops.append(("gemm_2048_b%d" % b, b, lambda b=b: dq.gemm(X4, P4[b], S4[b], PREFILL["K"], b, Y4)))
    decode = [(X1t[t], P2t[t][b], S2[b], b, Y1[b]) for t in range(DECODE["tokens"]) for b in W2]
    # the decode launches go through the C entry points with their arguments
    # taken beforehand: the tensor wrappers' checks cost the host more time
    # than a decode launch takes on the GPU, and a host-bound loop would time
    # the host (the submission cost is measured and reported below).  The
    # step's decode: one dq_gemv_batched per token over its five matrices.
    lib = dq.load()
    decode_calls = [(lib.dq_gemv, (xt.data_ptr(), 1, pt.data_ptr(), st.data_ptr(), DECODE["N"],
                                   DECODE["K"], b, yt.data_ptr(), stream.cuda_stream))
                    for xt, pt, st, b, yt in decode]
    token_items = []
    for t in range(DECODE["tokens"]):
        arr = (dq.DQGemvItem * len(W2))()
        for i, b in enumerate(W2):
            arr[i] = dq.DQGemvItem(X1t[t].data_ptr(), P2t[t][b].data_ptr(), S2[b].data_ptr(),
                                   Y1[b].data_ptr(), DECODE["N"], DECODE["K"], b)
        token_items.append(arr)
    batch_calls = [(lib.dq_gemv_batched, (ctypes.addressof(arr), len(W2), 1, stream.cuda_stream))
                   for arr in token_items]

    def launch(fn, a):
        status = fn(*a)
        if status:
            raise dq.DQError(status, fn.__name__)

    for fn, a in batch_calls:
        ops.append(("gemv_m1", 0, lambda fn=fn, a=a: launch(fn, a)))

    # one HIP event at every group boundary (events between every launch would
    # add their own dispatch gaps to the tiny GEMV launches)
    kinds = []
    for kind, _, _ in ops:
        if not kinds or kinds[-1] != kind:
            kinds.append(kind)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kinds) + 1)]
          for _ in range(args.steps)]

    def step(events=None):
        g = 0
        if events is not None:
            events[0].record(stream)
        for i, (kind, _, fn) in enumerate(ops):
            fn()
            last = i + 1 == len(ops) or ops[i + 1][0] != kind
            if last:
                g += 1
                if events is not None:
                    events[g].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-group time (ms) averaged over steps, split evenly over the group's launches
    group_ms = {kind: float(np.mean([ev[s][g].elapsed_time(ev[s][g + 1]) for s in range(args.steps)]))
                for g, kind in enumerate(kinds)}
    count = {kind: sum(1 for k, _, _ in ops if k == kind) for kind in kinds}

    # host time to issue the decode launches, taken while a GEMM keeps the GPU
    # busy: below the GPU's per-launch time, the decode group is not host-bound
    b6 = PREFILL["bits"][1]
    host_us = []
    for _ in range(5):
        dq.gemm(X4, P4[b6], S4[b6], PREFILL["K"], b6, Y4)
        t0 = time.perf_counter()
        for fn, a in batch_calls:
            launch(fn, a)
        host_us.append((time.perf_counter() - t0) / len(batch_calls) * 1e6)
        torch.cuda.synchronize()

    Nd, Kd = DECODE["N"], DECODE["K"]
    Np, Kp, Mp = PREFILL["N"], PREFILL["K"], PREFILL["M"]
    gemv_bytes = DECODE["tokens"] * sum(Nd * Kd * b // 8 for b in DECODE["bits"])
    gemv_ms = group_ms["gemv_m1"]
    value = gemv_bytes / (gemv_ms * 1e-3) / 1e9
    gemm_flop = 2.0 * Mp * Np * Kp
    gemm_ms = {b: group_ms["gemm_2048_b%d" % b] for b in PREFILL["bits"]}
    gemm_tflops = {b: gemm_flop / (t * 1e-3) / 1e12 for b, t in gemm_ms.items()}
    gemm_le9_ms = float(np.mean([t for b, t in gemm_ms.items() if b <= 9]))
    gemm_le9 = gemm_flop / (gemm_le9_ms * 1e-3) / 1e12
    # every width of the config (b = 12 included): algorithmic flops over the
    # mean launch time of all four
    gemm_all_ms = float(np.mean(list(gemm_ms.values())))
    gemm_all = gemm_flop / (gemm_all_ms * 1e-3) / 1e12

    # context for the GEMM figure, outside the timed steps: the plain bf16
    # library GEMM (torch.matmul -> hipBLASLt) on the same shape and GPU, with
    # the dense bf16 weights the prefill matrices were quantized from, in the
    # operand layout of the packed weights (each output's weights contiguous
    # along K: x @ W^T as a transposed view of W [N, K]) and, beside it, with
    # W^T made contiguous ([K, N]), which the library runs with other kernels
    def library_tflops(b_operand):
        for _ in range(3):
            torch.matmul(X4, b_operand)
        torch.cuda.synchronize()
        lib_ms = []
        for _ in range(7):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            torch.matmul(X4, b_operand)
            e1.record(stream)
            torch.cuda.synchronize()
            lib_ms.append(e0.elapsed_time(e1))
        return 2.0 * PREFILL["M"] * PREFILL["N"] * PREFILL["K"] / (float(np.median(lib_ms)) * 1e-3) / 1e12
    W6 = W4[PREFILL["bits"][1]]
    lib_tflops = library_tflops(W6.t())
    WT = W6.t().contiguous()
    lib_nn_tflops = library_tflops(WT)
    del WT, W6

    def gbs(kind, bits, N, K, read_bits, write_bits):
        """(read + write) bytes of the group's launches over the group time"""
        total = sum(N * K * (read_bits(b) + write_bits(b)) / 8 for b in bits)
        return round(total / (group_ms[kind] * 1e-3) / 1e9, 1)

    traffic = recorded_traffic()
    out = {
        "metric": "packed-weight GB/s & % HBM peak (M=1 GEMV); TFLOP/s & % MFMA peak (M=2048)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; bf16 W ~ N(0, 0.02^2) with 0.1% x20 outliers, x ~ N(0, 1))",
        "config": {
            "workload": "decode GEMV 4096x4096 b=4..8 M=1 (value) + prefill GEMM "
                        "M=2048 N=K=8192 b=5,6,8,12 (roofline_gemm)",
            "gemv": {"N": Nd, "K": Kd, "M": 1, "bits": list(DECODE["bits"]),
                     "tokens": DECODE["tokens"], "weight_copies": DECODE["tokens"]},
            "gemm": {"N": Np, "K": Kp, "M": Mp, "bits": list(PREFILL["bits"]),
                     "mfma_dtype": "bf16", "accumulate": "f32"},
            "step": "quantize+pack(5 decode) -> unpack(5) -> quantize+pack(4 prefill) -> "
                    "gemm(4) -> decode 8 tokens x one batched GEMV over the 5 matrices, token t on "
                    "copy t of the packed weights",
            "timing": "HIP events at group boundaries on the launch stream; per-launch "
                      "figures are group time / launches (inter-launch gaps included); decode "
                      "launches through the C entry point with prepared arguments",
        },
        "roofline": {
            "kernel": "dq_gemv_batched M=1 N=K=4096 (gemv_xres_batch_kernel; 8 launches back to "
                      "back, one per token, each over that token's five matrices b=4..8 on its "
                      "own copy of the weights)",
            "bound": "hbm",
            "achieved": round(value, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(value / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "per_launch_us": round(gemv_ms / count["gemv_m1"] * 1e3, 3),
            "host_submit_us_per_launch": round(float(np.median(host_us)), 3),
        },
        "roofline_gemm": {
            "kernel": "dq_gemm M=2048 N=K=8192, b=5,6,8 (b=12 listed in per_bits)",
            "bound": "mfma",
            "achieved": round(gemm_le9, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_le9 / MFMA_BF16_PEAK_TFLOPS, 4),
            "all_widths": {
                "achieved": round(gemm_all, 2),
                "frac": round(gemm_all / MFMA_BF16_PEAK_TFLOPS, 4),
                "what": "the same over all four widths of the config (b = 5, 6, 8, 12): "
                        "algorithmic flops over the mean launch time",
            },
            "per_bits": {str(b): round(v, 1) for b, v in gemm_tflops.items()},
            "note": "algorithmic 2*M*N*K flops; b >= 10 issues twice the MFMA work (exact hi/lo "
                    "bf16 split), so its ceiling is half the peak",
            "per_launch_us": round(gemm_le9_ms * 1e3, 2),
            "library_bf16_reference": {
                "tflops": round(lib_tflops, 1),
                "what": "torch.matmul bf16 x[2048,8192] @ W^T (W [8192,8192] row-major, the packed "
                        "weights' layout, passed as a transposed view; hipBLASLt, bf16 output) on the "
                        "same GPU in the same run, untimed by the steps",
                "w_t_contiguous_tflops": round(lib_nn_tflops, 1),
                "w_t_contiguous_what": "the same product with W^T made contiguous [8192,8192] first",
            },
        },
        "groups_ms": {kind: round(group_ms[kind], 5) for kind in kinds},
        "throughput_gbs": {
            "quantize_pack_4096": gbs("quantize_pack_4096", DECODE["bits"], Nd, Kd,
                                      lambda b: 16, lambda b: b),
            "unpack_4096": gbs("unpack_4096", DECODE["bits"], Nd, Kd, lambda b: b, lambda b: 32),
            "quantize_pack_8192": gbs("quantize_pack_8192", PREFILL["bits"], Np, Kp,
                                      lambda b: 16, lambda b: b),
        },
        "cpu_baseline": None,
        "device": device_info(torch, dev),
    }
    if args.copy_calibration:
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = src.numel() * 4
    b6 = PREFILL["bits"][1]
    out["roofline"]["attainable_read"] = attainable_read(
        torch, dq, dev, stream,
        lambda: [launch(fn, a) for fn, a in batch_calls],
        tok_bufs,
        lambda: dq.gemm(X4, P4[b6], S4[b6], PREFILL["K"], b6, Y4), reps=max(5, args.steps),
        per_matrix_group=lambda: [launch(fn, a) for fn, a in decode_calls],
        per_matrix_launches=len(decode_calls))
    # cache-hot figure, labelled as such: the same 8 launches with every token
    # reading copy 0 (63 MB, inside the 256 MB last-level cache after the first token)
    hot_items = []
    for t in range(DECODE["tokens"]):
        arr = (dq.DQGemvItem * len(W2))()
        for i, b in enumerate(W2):
            arr[i] = dq.DQGemvItem(X1t[t].data_ptr(), P2t[0][b].data_ptr(), S2[b].data_ptr(),
                                   Y1[b].data_ptr(), DECODE["N"], DECODE["K"], b)
        hot_items.append(arr)
    hot_calls = [(lib.dq_gemv_batched, (ctypes.addressof(arr), len(W2), 1, stream.cuda_stream))
                 for arr in hot_items]
    hot_ms = []
    for _ in range(max(5, args.steps)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for fn, a in hot_calls:
            launch(fn, a)
        e1.record(stream)
        torch.cuda.synchronize()
        hot_ms.append(e0.elapsed_time(e1))
    hot = float(np.median(hot_ms))
    out["roofline"]["cache_hot"] = {
        "gbs": round(gemv_bytes / (hot * 1e-3) / 1e9, 1),
        "per_launch_us": round(hot / len(hot_calls) * 1e3, 3),
        "what": "cache-hot: the 8 batched decode launches all on copy 0 of the five packed "
                "matrices (63 MB, re-read from the last-level cache), median of the step count; "
                "context, not the value"}
    out["allocation"] = {"row_sumsq": row_sumsq_context(torch, dq, stream, list(W4.values()),
                                                        reps=max(5, args.steps))}
    out["asymmetric"] = asym_context(torch, dq, stream, W2, X1t, W4, X4, reps=max(5, args.steps))
    out["group_scales"] = group_context(torch, dq, stream, W2, X1t, W4, X4, reps=max(5, args.steps))
    out["packed_file"] = packed_file_context(
        torch, dq, stream, {b: (P2[b], S2[b], DECODE["K"]) for b in W2})
    if not args.no_stack:
        del P4, W4, X4, Y4, Q2
        torch.cuda.empty_cache()
        out["roofline"]["context_layer_stack"], stack_sumsq = stack_context(
            torch, dq, workload, dev, stream)
        out["allocation"]["stack_recipe"], alloc_inputs = allocation_context(dq, workload,
                                                                             stack_sumsq)
    else:
        alloc_inputs = None
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(decode_np, x1_np, args.cpu_seconds, alloc_inputs)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
