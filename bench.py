"""Benchmark of the Fairy2i widely-linear hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--prewarm-s S] [--no-cpu-baseline] [--no-stack] [--no-mlp]

Workload: the LLaMA-2 7B attention projection (R 4096 x 4096 -> U, W 2048 x 2048 complex),
T = 2 residual stages, bf16 activations, all inputs synthetic and seeded (workloads.py).

One step is one pass of every stage of the path over one batch of inputs:
  1. quantize + pack the layer (split, projection, axis scales, residual stages, packing);
  2. decode GEMV at batch 1 over a pool of P = 256 distinct copies of the packed layer (1 GiB,
     four times the 256 MB Infinity Cache, so every pass streams from HBM and no segment gains
     from the pool reads of the one before it, as a decode step over a 1.6 GB stack would not),
     stored back to back and run as one strided-batch launch (fairy2i_gemv_strided): x is turned
     into its exact fp6 digit form once (fairy2i_x_digits_f6; the pool's layers share x, as q, k
     and v do), then the fp4-MFMA GEMV runs over the pool; the same with the int8 digit form and
     the int8-MFMA GEMV;
  3. the bf16-MFMA GEMV over the pool at batch 1, 4 and 16;
  4. prefill: per-token int8 activation quantization of 2048 tokens and the int8-MFMA GEMM;
  5. the real form of the quantized layer (dequantize, the fake-quant forward);
  6. quantize + pack with per-tensor axis scales (the other scale granularity).
Each segment is captured once into a HIP graph and replayed on torch's current stream, with
HIP events on that stream around every replay; inputs are resident in HBM before the timed
region starts.

`value` is the headline metric: algorithmic HBM bytes of the batch-1 decode segment (fp6 digit
form + fp4 GEMV launch) divided by its time (GB/s).  The JSON line also carries the roofline
of that GEMV kernel -- its launches timed, after the steps, in one graph of 8 back-to-back passes
over the pool, so that graph-launch latency between segments does not count as kernel time --
the other legs (GB/s, TOPS, params/s; the same pool through the grouped call, 48 layers per
launch; one launch per layer; fairy2i_gemv on the bf16 x as given, AUTO, at batch 1 and 2; the
prefill GEMM on the 11008 x 4096 layer and on zero-valued data; the 32-layer stack's quantizer
and decode step, the latter also on the fp4 kernel with and without its digit passes; the MLP
shapes at T = 2 and 3) and the CPU oracle timed on a bounded sample of the same workload.
Progress lines go to stderr; stdout carries the one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, TOP/s
METRIC = "packed 2-bit widely-linear GEMV HBM GB/s (% peak) + prefill GEMM int8 TOPS"
POOL_BYTES = 2 ** 30     # 4x the 256 MB Infinity Cache: every pass streams from HBM


def progress(msg: str) -> None:
    """A progress line on stderr (stdout carries only the result line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stack", action="store_true", help="skip the 32-layer stack legs")
    ap.add_argument("--no-mlp", action="store_true", help="skip the MLP-shape decode legs")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--prewarm-s", type=float, default=0.3,
                    help="seconds of untimed whole steps before the warm-up steps (clock ramp)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one 256 MiB device copy (counter calibration for profiles)")
    return ap.parse_args()


ROOF_PASSES = 8           # passes over the pool per roofline graph
ROOF_WARM = 40            # untimed replays first (~60 ms of the same launches)
ROOF_REPLAYS = 3
TRAFFIC_PROFILE = "profiles/gemv_strided_pool_attention4096_T2_hbm_traffic.md"


def measured_traffic_per_layer():
    """HBM bytes per layer of the batch-1 fp4 GEMV launch, from the committed FETCH_SIZE / WRITE_SIZE
    summary (copy-calibrated), or None when the kernel source changed since it was taken."""
    import hashlib
    import re
    here = os.path.dirname(os.path.abspath(__file__))
    try:
        text = open(os.path.join(here, TRAFFIC_PROFILE)).read()
        total = int(re.search(r"traffic_bytes_per_launch: (\d+)", text).group(1))
        layers = int(re.search(r"layers_per_launch: (\d+)", text).group(1))
        src, digest = re.search(r"kernel_source: (\S+) sha256 ([0-9a-f]+)", text).groups()
        now = hashlib.sha256(open(os.path.join(here, src), "rb").read()).hexdigest()
    except (OSError, AttributeError, ValueError):
        return None
    return total / layers if now == digest else None


def gemv_bytes(n, m, T, B, x_bytes=2, y_bytes=4):
    """Algorithmic bytes of one GEMV: codes + fp32 scales + x + y."""
    return T * n * m // 2 + n * T * 2 * 2 * 4 + B * 2 * m * x_bytes + B * 2 * n * y_bytes


def host_info():
    """The measuring host's CPU: logical cores, the cores this process may run on, the CPU model
    and the BLAS thread count NumPy uses."""
    info = {"cpu_count": os.cpu_count(), "affinity": None, "model": None, "blas_threads": None}
    try:
        info["affinity"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["model"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        info["blas_threads"] = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:                                      # pragma: no cover
        pass
    return info


def cpu_baseline(R, T, x1, budget_s, prefill):
    """The oracle (float64 NumPy) on the measuring machine's host cores, on bounded samples of the
    same workload: the batch-1 GEMV of the attention layer (repeated until `budget_s` is spent;
    `value`), the quantizer on a row sample, and the prefill path (activation quantization, the
    integer GEMM and its epilogue) on a token sample of the 4096 x 4096 prefill layer."""
    import oracle
    host = host_info()
    cores = host["blas_threads"] or host["affinity"] or host["cpu_count"] or 1
    n, m = R.shape[0] // 2, R.shape[1] // 2
    rows = np.arange(128)
    sub = np.concatenate([R[rows], R[n + rows]])
    t0 = time.perf_counter()
    oracle.quantize(sub, T)
    tq = time.perf_counter() - t0
    codes, s32, _, _ = oracle.quantize(R, T)               # setup, not timed
    reps, t_gemv = 0, 0.0
    while t_gemv < budget_s or reps == 0:
        t0 = time.perf_counter()
        oracle.gemv_ref(codes, s32, x1)
        t_gemv += time.perf_counter() - t0
        reps += 1
    per = t_gemv / reps
    Rp, xp = prefill                                       # prefill layer and its activations
    pc, ps, _, _ = oracle.quantize(Rp, T)                  # setup, not timed
    ntok = 256
    t0 = time.perf_counter()
    q, d = oracle.act_quant_ref(xp[:ntok])
    P = oracle.gemm_int_ref(pc, q)
    oracle.gemm_epilogue_ref(P, ps, d)
    tg = time.perf_counter() - t0
    pn, pm = Rp.shape[0] // 2, Rp.shape[1] // 2
    issued = 16 * T * pn * pm * ntok
    return {
        "value": gemv_bytes(n, m, T, 1) / per / 1e9, "unit": "GB/s", "cores": int(cores),
        "kind": "oracle",
        "sample": f"{reps} x oracle gemv_ref of the full {2*n}x{2*m} layer at batch 1 "
                  f"({per*1e3:.1f} ms each); quantizer on {len(rows)} of {n} complex rows "
                  f"took {tq:.3f} s ({len(rows)*m*4/tq/1e6:.2f} M real params/s); prefill "
                  f"(act-quant + integer GEMM + epilogue) of {ntok} of 2048 tokens on the "
                  f"{2*pn}x{2*pm} layer took {tg:.3f} s",
        "host": host,
        "legs": {"gemv_b1": {"GB/s": round(gemv_bytes(n, m, T, 1) / per / 1e9, 5), "s_per_call": round(per, 4)},
                 "quantize": {"real_params_per_s": round(len(rows) * m * 4 / tq, 1), "s": round(tq, 4)},
                 "gemm": {"tokens": ntok, "s": round(tg, 4), "issued_TOPS": round(issued / tg / 1e12, 6),
                          "useful_TOPS": round(issued / 2 / tg / 1e12, 6)}},
    }


def stack_legs(f2, torch, dev, T, reps):
    """The LLaMA-2 7B linear stack (32 layers x 7 projections, 6.48e9 real weights): quantize all
    224 matrices (grouped calls, the matrices of one shape sharing launches; and, for comparison,
    one call per matrix), then one decode step (grouped launches per shared input, the stack's default
    kernel) at batch 1 and batch 8, each captured in a HIP graph.  The weights are the pinned
    generator's (workloads.stack_layer: NumPy, seed 5000 + 7 L + p, N(0, 0.02^2)), drawn on host
    threads and copied to the GPU (25.9 GB in all), the same matrices the GPU parity test samples;
    the decode inputs are workloads.activations with seed 6000 + 7 L + g.  Runs outside the timed
    step."""
    import concurrent.futures
    import workloads
    from widely_linear_gemv_amd.stack import DecodeStep, GROUPS, PROJECTIONS
    R, out = [], []
    keys = [(L, p) for L in range(32) for p in range(len(PROJECTIONS))]
    workers = min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1))
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:      # NumPy's generator releases the GIL
        for k0 in range(0, len(keys), 2 * workers):               # bounded host memory
            for w in ex.map(lambda key: workloads.stack_layer(*key).weight(), keys[k0:k0 + 2 * workers]):
                R.append(torch.from_numpy(w).to(dev))
    gen_s = time.perf_counter() - t0
    for (L, p) in keys:
        _, rows, cols, _ = PROJECTIONS[p]
        n, m = rows // 2, cols // 2
        out.append({"packed": torch.empty((f2.fairy2i_packed_bytes(n, m, T),), dtype=torch.uint8, device=dev),
                    "scales": torch.empty((n, T, 2, 2), dtype=torch.float32, device=dev)})

    by_shape = {}                   # grouped calls: the matrices of one shape share launches
    for r, o in zip(R, out):
        by_shape.setdefault(tuple(r.shape), []).append((r, o))

    def quantize_all():
        for items in by_shape.values():
            f2.fairy2i_quantize_grouped([r for r, _ in items], T, packed=[o["packed"] for _, o in items],
                                        scales=[o["scales"] for _, o in items])

    def quantize_each():
        for r, o in zip(R, out):
            f2.fairy2i_quantize(r, T, packed=o["packed"], scales=o["scales"])

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=torch.cuda.Stream()):
            fn()
        g.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps          # ms

    t_q = timed(quantize_all)
    t_q1 = timed(quantize_each)
    layers = [[(out[7 * L + p]["packed"], out[7 * L + p]["scales"]) for p in range(7)] for L in range(32)]
    r_bytes = sum(r.numel() * 4 for r in R)
    legs = {"stack_quantize": {"matrices": 224, "launches": sum((len(v) + 31) // 32 for v in by_shape.values()),
                               "ms": round(t_q, 3), "R_GB/s": round(r_bytes / (t_q * 1e-3) / 1e9, 1),
                               "one_call_per_matrix_ms": round(t_q1, 3),
                               "real_params_per_s": round(sum(r.numel() for r in R) / (t_q * 1e-3), 1),
                               "weights": f"pinned NumPy generator (seed 5000 + 7 L + p), drawn on {workers} "
                                          f"host threads in {gen_s:.1f} s"}}
    del R
    for B in (1, 8):
        xs = []
        for L in range(32):
            lx = []
            for gi in range(GROUPS):
                cols = next(c for (_, _, c, grp) in PROJECTIONS if grp == gi)
                a = workloads.activations(B, cols, workloads.stack_x_seed(L, gi))
                lx.append(torch.from_numpy(a.bf16_bits.view(np.int16)).to(dev).view(torch.bfloat16))
            xs.append(lx)
        step = DecodeStep(layers, xs)
        t = timed(step.run)
        nbytes = sum(gemv_bytes(rows // 2, cols // 2, T, B) for L in range(32) for (_, rows, cols, _) in PROJECTIONS)
        legs[f"stack_decode_b{B}"] = {"gemvs": 224, "launches": 128, "us": round(t * 1e3, 1),
                                      "GB/s": round(nbytes / (t * 1e-3) / 1e9, 1), "bytes": nbytes,
                                      "kernel": "AUTO: fp4 matrix cores, each wave digitizing its own chunks of x on chip"
                                                if B == 1 else "AUTO: bf16 matrix cores"}
        if B == 1:
            # the fp4 kernel: with its digit pass in the step (256 launches), and on x already
            # in digit form (the 128 GEMV launches alone, for inputs a producer writes in that form)
            for given, key, note in ((False, "stack_decode_b1_f4", "fp4 matrix cores, fp6 digit pass per group"),
                                     (True, "stack_decode_b1_f4_digits_given",
                                      "fp4 matrix cores on x already in fp6 digit form (digit passes outside the step)")):
                fstep = DecodeStep(layers, xs, algo=f2.GEMV_MFMA_F4, digits_given=given)
                tf = timed(fstep.run)
                legs[key] = {"gemvs": 224, "launches": 128 if given else 256, "us": round(tf * 1e3, 1),
                             "GB/s": round(nbytes / (tf * 1e-3) / 1e9, 1), "kernel": note}
                del fstep
    return legs


MLP_POOL_BYTES = 2 ** 30     # 4x the Infinity Cache per MLP pool, as for the attention pool


def mlp_legs(f2, torch, workloads, dev, reps=5):
    """The LLaMA-2 7B MLP decode GEMVs: gate/up (11008 x 4096, outlier weights) and down
    (4096 x 11008) quantized at T = 2 and T = 3, at batch 1 (fp4 matrix cores on the fp6 digit form)
    and batch 8 (bf16 matrix cores, shared x).  Each case streams a pool of >= 1 GiB of copies of
    its quantized layer (as the attention pool: four times the Infinity Cache, and launches long
    enough that one launch's ramp and tail are a small part of it) as one strided-batch launch per
    pass, four passes per HIP graph, replayed for ~50 ms first so the clocks have settled.  Runs
    outside the timed step."""
    legs = {}
    for name, layer in (("gate_up", workloads.MLP_GATE_UP), ("down", workloads.MLP_DOWN)):
        R = torch.from_numpy(layer.weight()).to(dev)
        n, m = layer.n, layer.m
        for T in (2, 3):
            q = f2.fairy2i_quantize(R, T)
            P = max(1, -(-MLP_POOL_BYTES // q["packed"].numel()))
            pool = q["packed"].unsqueeze(0).repeat(P, 1).contiguous()
            spool = q["scales"].unsqueeze(0).repeat(P, 1, 1, 1, 1).contiguous()
            for B in (1, 8):
                a = workloads.activations(B, 2 * m, workloads.MLP_X_SEEDS[name])
                x = torch.from_numpy(a.bf16_bits.view(np.int16)).to(dev).view(torch.bfloat16)
                y = torch.empty((P, B, 2 * n), dtype=torch.float32, device=dev)
                if B <= 2:
                    xd = f2.fairy2i_x_digits_f6(x)
                    kern = "fp4 matrix cores (fp6 digit form of x, made once)"

                    def fn():
                        f2.fairy2i_gemv_strided(pool, spool, xd, y, algo=f2.GEMV_MFMA_F4)
                else:
                    kern = "bf16 matrix cores (shared x)"

                    def fn():
                        f2.fairy2i_gemv_strided(pool, spool, x, y, algo=f2.GEMV_MFMA_BF16)
                fn()
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=torch.cuda.Stream()):
                    for _ in range(4):
                        fn()
                t_w = time.perf_counter()
                while time.perf_counter() - t_w < 0.05:
                    g.replay()
                    torch.cuda.synchronize()
                stream = torch.cuda.current_stream()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / (reps * 4)
                nbytes = P * gemv_bytes(n, m, T, B)
                legs[f"mlp_{name}_T{T}_b{B}"] = {
                    "shape": f"{2 * n}x{2 * m}", "layers_per_launch": P, "us_per_launch": round(us, 2),
                    "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                    "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "kernel": kern}
            del pool, spool, q
        del R
    torch.cuda.empty_cache()
    return legs


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this path has no "
              f"multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    import widely_linear_gemv_amd as f2
    from widely_linear_gemv_amd import build as _build

    if not os.path.exists(f2.LIB_PATH):
        _build.build()
    f2.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    layer = workloads.ATTN
    n, m, T = layer.n, layer.m, 2
    R_np = layer.weight()
    R = torch.from_numpy(R_np).to(dev)
    q0 = f2.fairy2i_quantize(R, T)
    layer_bytes = q0["packed"].numel()
    P = max(1, -(-POOL_BYTES // layer_bytes))
    pool = q0["packed"].unsqueeze(0).repeat(P, 1).contiguous()
    spool = q0["scales"].unsqueeze(0).repeat(P, 1, 1, 1, 1).contiguous()
    xs = {}
    for B in (1, 4, 16):
        a = workloads.activations(B, 2 * m, workloads.ATTN_X_SEEDS[B])
        xs[B] = torch.from_numpy(a.bf16_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    ys = {B: torch.empty((B, 2 * n), dtype=torch.float32, device=dev) for B in xs}
    Ntok = workloads.PREFILL_TOKENS
    xp_np = workloads.activations(Ntok, 2 * m, workloads.PREFILL_X_SEED)
    xp = torch.from_numpy(xp_np.bf16_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    qp = torch.empty((Ntok, 2 * m), dtype=torch.int8, device=dev)
    dp = torch.empty((Ntok,), dtype=torch.float32, device=dev)
    # the two prefill layers (4096 x 4096 and 11008 x 4096), quantized once before timing
    Rp_np = [L.weight() for L in workloads.PREFILL_LAYERS]
    qpre = [f2.fairy2i_quantize(torch.from_numpy(r).to(dev), T) for r in Rp_np]
    ypre = [torch.empty((Ntok, L.rows), dtype=torch.float32, device=dev) for L in workloads.PREFILL_LAYERS]
    qout = {"packed": torch.empty_like(q0["packed"]), "scales": torch.empty_like(q0["scales"])}

    if args.calib_copy:
        a = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    # Each segment of the step is captured once into a HIP graph (all outputs preallocated, no
    # memset nodes), so the timed region measures GPU work rather than Python launch overhead.
    def seg_quantize():
        f2.fairy2i_quantize(R, T, packed=qout["packed"], scales=qout["scales"])

    ypool = {B: torch.empty((P, B, 2 * n), dtype=torch.float32, device=dev) for B in xs}
    items = {B: [(pool[p], spool[p], xs[B], ypool[B][p]) for p in range(P)] for B in xs}

    def seg_gemv(B):
        def run():
            f2.fairy2i_gemv_strided(pool, spool, xs[B], ypool[B], algo=f2.GEMV_MFMA)
        return run

    xd1 = f2.XDigits(torch.empty((f2.fairy2i_x_digits_bytes(m, 1),), dtype=torch.uint8, device=dev), 1, m)
    items_i8 = [(pool[p], spool[p], xd1, ypool[1][p]) for p in range(P)]

    def seg_decode_i8():               # the batch-1 decode path: digit form, then the GEMV
        f2.fairy2i_x_digits(xs[1], out=xd1)
        f2.fairy2i_gemv_strided(pool, spool, xd1, ypool[1], algo=f2.GEMV_MFMA_I8)

    def seg_gemv_i8():                 # the GEMV launch alone (kernel time)
        f2.fairy2i_gemv_strided(pool, spool, xd1, ypool[1], algo=f2.GEMV_MFMA_I8)

    xf1 = f2.XDigits(torch.empty((f2.fairy2i_x_digits_f6_bytes(m, 1),), dtype=torch.uint8, device=dev), 1, m,
                     f2.X_DIGITS_F6)
    items_f4 = [(pool[p], spool[p], xf1, ypool[1][p]) for p in range(P)]

    def seg_decode_f4():               # the batch-1 decode path on the fp4 matrix cores
        f2.fairy2i_x_digits_f6(xs[1], out=xf1)
        f2.fairy2i_gemv_strided(pool, spool, xf1, ypool[1], algo=f2.GEMV_MFMA_F4)

    def seg_gemv_f4():
        f2.fairy2i_gemv_strided(pool, spool, xf1, ypool[1], algo=f2.GEMV_MFMA_F4)

    def grouped_f4():                  # the same layers through the grouped call (<= 48 per launch)
        f2.fairy2i_gemv_grouped(items_f4, algo=f2.GEMV_MFMA_F4)

    def single_layers():               # one launch per layer (latency-bound small kernels)
        for p in range(P):
            f2.fairy2i_gemv(pool[p], spool[p], xf1, y=ys[1], algo=f2.GEMV_MFMA_F4)

    Rhat = torch.empty((2 * n, 2 * m), dtype=torch.float32, device=dev)

    def seg_dequant():                 # the real form of the layer (fake-quant forward)
        f2.fairy2i_dequantize(q0["packed"], q0["scales"], m, R=Rhat)

    ws_t = torch.empty((f2.fairy2i_quantize_tensor_workspace_bytes(n, m, T),), dtype=torch.uint8, device=dev)

    def seg_quantize_tensor():         # the per-tensor-scale quantizer (2T + 1 launches)
        f2.fairy2i_quantize_tensor(R, T, workspace=ws_t, packed=qout["packed"], scales=qout["scales"])

    def seg_act_quant():
        f2.fairy2i_act_quant(xp, q=qp, delta=dp)

    def seg_gemm():                    # the 4096 x 4096 prefill layer
        f2.fairy2i_gemm(qpre[0]["packed"], qpre[0]["scales"], qp, x_scale=dp, y=ypre[0])

    def gemm_mlp():                    # the 11008 x 4096 prefill layer (timed outside the step)
        f2.fairy2i_gemm(qpre[1]["packed"], qpre[1]["scales"], qp, x_scale=dp, y=ypre[1])

    segments = [seg_quantize, seg_decode_f4, seg_gemv_f4, seg_decode_i8, seg_gemv_i8, seg_gemv(1),
                seg_gemv(4), seg_gemv(16), seg_act_quant, seg_gemm, seg_dequant, seg_quantize_tensor,
                grouped_f4, single_layers]
    NSEG = len(segments) - 2
    for fn in segments:                     # eager warm-up (also loads every kernel)
        fn()
    torch.cuda.synchronize()
    graphs = []
    cap = torch.cuda.Stream()
    for fn in segments:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            fn()
        graphs.append(g)
    torch.cuda.synchronize()

    single_graph = graphs.pop()
    grouped_graph = graphs.pop()

    def step():
        e = [ev()]
        for g in graphs:
            g.replay()
            e.append(ev())
        return e

    # The GPU's clocks settle only after tens of milliseconds of sustained load (the first ~20 ms of
    # back-to-back pool passes run ~10 % slower): replay whole steps for --prewarm-s seconds first.
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < args.prewarm_s:
        step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    seg = np.zeros(NSEG)
    t0 = time.perf_counter()
    progress(f"warm-up done; timing {args.steps} steps")
    all_events = [step() for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for e in all_events:
        seg += np.array([e[k].elapsed_time(e[k + 1]) for k in range(NSEG)])   # ms
    seg /= args.steps
    ms_step = float(np.sum(seg))
    # outside the timed step: the same pool as separate single-layer launches (one per layer)
    single_graph.replay()
    torch.cuda.synchronize()
    e0 = ev()
    for _ in range(3):
        single_graph.replay()
    e1 = ev()
    torch.cuda.synchronize()
    single_us = e0.elapsed_time(e1) * 1e3 / (3 * P)
    # outside the timed step: the pool through the grouped call (48 layers per launch)
    for _ in range(5):
        grouped_graph.replay()
    torch.cuda.synchronize()
    e0 = ev()
    for _ in range(5):
        grouped_graph.replay()
    e1 = ev()
    torch.cuda.synchronize()
    grouped_us = e0.elapsed_time(e1) * 1e3 / 5
    # outside the timed step: the roofline's kernel time.  One graph holds ROOF_PASSES passes of
    # the strided fp4 launch over the pool back to back, so the launch time is the kernel's own
    # (no graph-launch latency between segments).
    roof_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(roof_graph, stream=cap):
        for _ in range(ROOF_PASSES):
            seg_gemv_f4()
    for _ in range(ROOF_WARM):
        roof_graph.replay()
    torch.cuda.synchronize()
    e0 = ev()
    for _ in range(ROOF_REPLAYS):
        roof_graph.replay()
    e1 = ev()
    torch.cuda.synchronize()

    def kernel_us(fn, calls=8, warm=20, replays=3):
        """Per-call time of fn's launches run back to back: `calls` calls in one graph, replayed
        after `warm` untimed replays (no graph-launch latency between the calls)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for _ in range(calls):
                fn()
        for _ in range(warm):
            g.replay()
        torch.cuda.synchronize()
        a = ev()
        for _ in range(replays):
            g.replay()
        b = ev()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (replays * calls)

    # the pool through fairy2i_gemv on the bf16 x as it is (AUTO: the fp4 kernel building its
    # digits on chip for a launch this large), batch 1 and 2
    x2 = xs[4][:2].contiguous()
    ypool2 = torch.empty((P, 2, 2 * n), dtype=torch.float32, device=dev)

    def auto_b1():
        f2.fairy2i_gemv_strided(pool, spool, xs[1], ypool[1])

    def auto_b2():
        f2.fairy2i_gemv_strided(pool, spool, x2, ypool2)

    def auto_b4():                     # AUTO at batch 4: fp4 code planes on x split into fp8 parts
        f2.fairy2i_gemv_strided(pool, spool, xs[4], ypool[4])

    # the same GEMM launch on all-zero activations and codes 0x55 (one plane all zero, the other +1):
    # the same instructions and memory traffic with little switching, so the chip holds a higher clock
    q_zero = torch.zeros_like(qp)
    packed_55 = torch.full_like(qpre[0]["packed"], 0x55)
    y_zero = torch.empty_like(ypre[0])

    def gemm_zero_data():
        f2.fairy2i_gemm(packed_55, qpre[0]["scales"], q_zero, x_scale=dp, y=y_zero)

    k_us = {"quantize": kernel_us(seg_quantize), "act_quant": kernel_us(seg_act_quant),
            "gemm_zero_data": kernel_us(gemm_zero_data),
            "auto_b1": kernel_us(auto_b1, warm=40), "auto_b2": kernel_us(auto_b2, warm=40),
            "auto_b4": kernel_us(auto_b4, warm=40),
            "gemm": kernel_us(seg_gemm), "dequantize": kernel_us(seg_dequant),
            "quantize_per_tensor": kernel_us(seg_quantize_tensor), "gemm_mlp": kernel_us(gemm_mlp)}
    ops_mlp = 16 * T * workloads.PREFILL_LAYERS[1].n * m * Ntok        # issued int8 ops

    t_quant, t_decf4, t_f4, t_dec, t_i8, t_b1, t_b4, t_b16, t_aq, t_gemm, t_deq, t_qt = seg    # ms
    bytes_b = {B: gemv_bytes(n, m, T, B) for B in (1, 4, 16)}
    gemv_ms = {1: t_b1, 4: t_b4, 16: t_b16}
    gbs = {B: P * bytes_b[B] / (gemv_ms[B] * 1e-3) / 1e9 for B in (1, 4, 16)}
    launches = 1                               # one strided-batch launch per pool pass
    per_launch_us = {B: gemv_ms[B] * 1e3 / launches for B in (1, 4, 16)}
    # batch-1 decode through a digit form of x (made once per x, shared by the pool's layers as
    # q, k and v share theirs), then the strided-batch GEMV launch
    bytes_pool = P * bytes_b[1]
    f4_gbs = bytes_pool / (t_decf4 * 1e-3) / 1e9
    f4_launch_us = t_f4 * 1e3 / launches
    roof_launch_us = e0.elapsed_time(e1) * 1e3 / (ROOF_REPLAYS * ROOF_PASSES * launches)
    roof_gbs = bytes_pool / launches / (roof_launch_us * 1e-6) / 1e9
    f4_launch_gbs = bytes_pool / launches / (f4_launch_us * 1e-6) / 1e9
    i8_gbs = bytes_pool / (t_dec * 1e-3) / 1e9
    i8_launch_us = t_i8 * 1e3 / launches
    i8_launch_gbs = bytes_pool / launches / (i8_launch_us * 1e-6) / 1e9
    traffic_layer = measured_traffic_per_layer()
    issued_ops = 16 * T * n * m * Ntok
    gemm_tops = issued_ops / (t_gemm * 1e-3) / 1e12
    quant_params = 4 * n * m
    quant_read = quant_params * 4 + layer_bytes + n * T * 4 * 4

    out = {
        "metric": METRIC,
        "value": round(f4_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "LLaMA-2 7B attention projection R 4096x4096 -> U,W 2048x2048, T=2; "
                        "decode GEMV batch 1 (value), 4, 16 over a pool of distinct layer copies "
                        "stored back to back (one strided-batch launch per pass); "
                        "quantize+pack; prefill act-quant + int8 GEMM over 2048 tokens",
            "rows": 2 * n, "cols": 2 * m, "T": T, "batch": 1, "pool_layers": P,
            "x_dtype": "bf16", "y_dtype": "f32",
            "gemv_kernel": "fp4 x fp6 MFMA (sum/difference sign planes) on the exact fp6 digit form "
                           "of x, one strided-batch launch over the pool",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_gemv_f4_mixed (strided batch over the pool, batch 1; one wave per tile, the last 1536 tiles four waves each)",
            "achieved": round(roof_gbs, 2),
            "us_per_launch": round(roof_launch_us, 3),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(roof_gbs / HBM_PEAK_GBS, 4),
            "traffic": (None if traffic_layer is None
                        else int(round(traffic_layer * P / launches))),
        },
        "legs": {
            "gemv_b1_i8": {"GB/s": round(i8_gbs, 2), "segment_us": round(t_dec * 1e3, 3),
                           "us_per_launch": round(i8_launch_us, 3), "launch_GB/s": round(i8_launch_gbs, 2),
                           "layers_per_launch": P / launches, "bytes_per_layer": bytes_b[1]},
            "gemv_b1_f4": {"GB/s": round(f4_gbs, 2), "segment_us": round(t_decf4 * 1e3, 3),
                           "us_per_launch": round(f4_launch_us, 3), "launch_GB/s": round(f4_launch_gbs, 2),
                           "layers_per_launch": P / launches, "bytes_per_layer": bytes_b[1]},
            "gemv_b1": {"GB/s": round(gbs[1], 2), "us_per_launch": round(per_launch_us[1], 3),
                        "layers_per_launch": P / launches, "bytes_per_layer": bytes_b[1]},
            "gemv_b4": {"GB/s": round(gbs[4], 2), "us_per_launch": round(per_launch_us[4], 3),
                        "layers_per_launch": P / launches, "bytes_per_layer": bytes_b[4]},
            "gemv_b16": {"GB/s": round(gbs[16], 2), "us_per_launch": round(per_launch_us[16], 3),
                         "layers_per_launch": P / launches, "bytes_per_layer": bytes_b[16]},
            "gemv_b1_bf16x_auto": {"us_per_launch": round(k_us["auto_b1"], 3),
                                   "GB/s": round(bytes_pool / (k_us["auto_b1"] * 1e-6) / 1e9, 2),
                                   "kernel": "fp4 MFMA, digit records built on chip from the bf16 x (AUTO)"},
            "gemv_b2_bf16x_auto": {"us_per_launch": round(k_us["auto_b2"], 3),
                                   "GB/s": round(P * gemv_bytes(n, m, T, 2) / (k_us["auto_b2"] * 1e-6) / 1e9, 2),
                                   "kernel": "fp4 MFMA, digit records built on chip from the bf16 x (AUTO)"},
            "gemv_b4_bf16x_auto": {"us_per_launch": round(k_us["auto_b4"], 3),
                                   "GB/s": round(P * bytes_b[4] / (k_us["auto_b4"] * 1e-6) / 1e9, 2),
                                   "kernel": "fp4 MFMA on x split into two fp8 parts with per-block scales (AUTO)"},
            "gemv_b1_f4_grouped": {"us_per_pass": round(grouped_us, 3), "launches_per_pass": -(-P // 48),
                                   "GB/s": round(bytes_pool / (grouped_us * 1e-6) / 1e9, 2)},
            "gemv_b1_single_layer_launch": {"us_per_launch": round(single_us, 3),
                                            "GB/s": round(bytes_b[1] / (single_us * 1e-6) / 1e9, 2)},
            "quantize": {"us": round(t_quant * 1e3, 2),
                         "real_params_per_s": round(quant_params / (t_quant * 1e-3), 1),
                         "GB/s": round(quant_read / (t_quant * 1e-3) / 1e9, 2),
                         "kernel_us": round(k_us["quantize"], 2),
                         "kernel_GB/s": round(quant_read / (k_us["quantize"] * 1e-6) / 1e9, 2)},
            "quantize_per_tensor": {"us": round(t_qt * 1e3, 2),
                                    "real_params_per_s": round(quant_params / (t_qt * 1e-3), 1),
                                    "kernel_us": round(k_us["quantize_per_tensor"], 2)},
            "act_quant": {"us": round(t_aq * 1e3, 2),
                          "GB/s": round((Ntok * 2 * m * 3 + Ntok * 4) / (t_aq * 1e-3) / 1e9, 2),
                          "kernel_us": round(k_us["act_quant"], 2),
                          "kernel_GB/s": round((Ntok * 2 * m * 3 + Ntok * 4) / (k_us["act_quant"] * 1e-6) / 1e9, 2)},
            "gemm": {"us": round(t_gemm * 1e3, 2), "issued_TOPS": round(gemm_tops, 2),
                     "useful_TOPS": round(gemm_tops / 2, 2),
                     "frac_of_int8_peak": round(gemm_tops / INT8_PEAK_TOPS, 4),
                     "issued_ops": issued_ops,
                     "kernel_us": round(k_us["gemm"], 2),
                     "kernel_issued_TOPS": round(issued_ops / (k_us["gemm"] * 1e-6) / 1e12, 2),
                     "kernel_frac_of_int8_peak": round(issued_ops / (k_us["gemm"] * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4)},
            "gemm_zero_data": {
                "kernel_us": round(k_us["gemm_zero_data"], 2),
                "kernel_frac_of_int8_peak": round(issued_ops / (k_us["gemm_zero_data"] * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4),
                "note": "4096x4096 layer, zero activations and codes 0x55: the launch of the gemm leg with "
                        "low switching activity (higher clock under the power limit)"},
            "gemm_11008x4096": {
                "issued_ops": ops_mlp, "kernel_us": round(k_us["gemm_mlp"], 2),
                "kernel_issued_TOPS": round(ops_mlp / (k_us["gemm_mlp"] * 1e-6) / 1e12, 2),
                "kernel_useful_TOPS": round(ops_mlp / 2 / (k_us["gemm_mlp"] * 1e-6) / 1e12, 2),
                "kernel_frac_of_int8_peak": round(ops_mlp / (k_us["gemm_mlp"] * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4)},
            "dequantize": {"us": round(t_deq * 1e3, 2),
                           "GB/s": round((layer_bytes + n * T * 16 + 4 * n * m * 4) / (t_deq * 1e-3) / 1e9, 2),
                           "kernel_us": round(k_us["dequantize"], 2),
                           "kernel_GB/s": round((layer_bytes + n * T * 16 + 4 * n * m * 4) / (k_us["dequantize"] * 1e-6) / 1e9, 2)},
            "wall_s": round(wall, 3),
        },
    }
    progress("steps and kernel legs done")
    if not args.no_stack:
        progress("32-layer stack legs")
        out["legs"].update(stack_legs(f2, torch, dev, T, reps=5))
    if not args.no_mlp:
        progress("MLP-shape decode legs")
        out["legs"].update(mlp_legs(f2, torch, workloads, dev))
    if not args.no_cpu_baseline:
        progress("CPU oracle baseline")
        x1 = workloads.activations(1, 2 * m, workloads.ATTN_X_SEEDS[1]).values
        out["cpu_baseline"] = cpu_baseline(R_np, T, x1, args.cpu_seconds, (Rp_np[0], xp_np.values))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
