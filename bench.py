#!/usr/bin/env python3
"""Benchmark of the NVFP4 block-scaled GEMM library on one MI355X.

Step = one W4A4 NVFP4 GEMM D = alpha (A.SFA)(B.SFB)^T at M = N = K = 8192 with
BF16 output: A and B are BF16 N(0,1) tensors quantized on the device by the
library's quantizer, A straight into the layout the GEMM reads
(nvfp4_quantize_tiled) and B prepared once (both untimed), all inputs resident
in HBM when the timed region starts. One step is one nvfp4_gemm_w4a4_tiled
call, the GEMM kernel. `value` is TFLOP/s (2 M N K per step). The same GEMM
on a row-major A (nvfp4_gemm_w4a4: a tile copy of A, then the GEMM) is timed
too and reported in `config`. The default 50 warm-up steps (about 40 ms)
bring the chip to its steady clock under this load; the first ~25 calls after
idle run up to 10 % slower while the clock ramps.

Extra figures in the same JSON line: W4A16 decode (M = 1) achieved HBM GB/s on
the 27B-class layer shapes with weights rotated over >= 1 GiB (CUDA-graph
replay), the prefill W4A4 with on-device activation quantization, and the
other square sizes. `roofline` describes the dominant kernel, the W4A4 GEMM
kernel (the whole step);
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps 100] [--warmup 50] [--no-extras] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 GEMM TFLOP/s & % MFMA peak at 8k³; W4A16 M=1 achieved HBM GB/s"
PEAK_F16_TFLOPS = 2500.0          # MI355X dense FP16/BF16 MFMA (published)
PEAK_HBM_GBS = 8000.0             # MI355X HBM3E (published)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "w4a4_8192_traffic.json")
KERNEL_SOURCES = ["nvfp4_block_scaled_amd/csrc/gemm_w4a4.hip", "nvfp4_block_scaled_amd/csrc/common.hpp"]


def kernel_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def time_calls(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / steps


def quantized_square(nv, S, operand, gen, tiled=False):
    """Device NVFP4 operand quantized by the library from the seeded BF16 tensor: (codes, scales,
    g, inv_g), or (activation in the tile layout, g, inv_g) with tiled=True."""
    import torch
    x = gen(S, operand)
    if isinstance(x, tuple):
        x = x[0]
    xd = torch.from_numpy(x).cuda().view(torch.bfloat16)
    res = nv.nvfp4_quantize_tiled(xd) if tiled else nv.nvfp4_quantize(xd)
    del xd
    return res


def w4a4_square(nv, S, steps, warmup, gen=None, standard_too=False):
    """Step = the W4A4 GEMM on A as the quantizer emits it for the GEMM (the tile layout,
    nvfp4_quantize_tiled) and B prepared once: nvfp4_gemm_w4a4_tiled. With standard_too, also
    time nvfp4_gemm_w4a4 on A in the row-major layout (the tile copy + the same GEMM)."""
    import numpy as np
    import torch
    import synth
    gen = gen or synth.square_normal
    at, gA, _ = quantized_square(nv, S, "A", gen, tiled=True)
    cb, sb, gB, _ = quantized_square(nv, S, "B", gen)
    wp, _ = nv.nvfp4_prepare_weight(cb, sb, "ue4m3")
    del cb, sb
    alpha = float(np.float32(1.0) / np.float32(np.float32(gA.item()) * np.float32(gB.item())))
    out = torch.empty((S, S), dtype=torch.bfloat16, device="cuda")
    ms = time_calls(lambda: nv.nvfp4_gemm_w4a4_tiled(at, S, wp, S, S, alpha, None, "bf16", out), steps, warmup)
    if not standard_too:
        return ms, 2.0 * S ** 3 / (ms * 1e-3) / 1e12
    # the same GEMM with a per-column alpha (a weight with per-column scales)
    ac = torch.from_numpy(np.random.default_rng(7).uniform(0.5, 2.0, S).astype(np.float32)).cuda()
    ms_col = time_calls(lambda: nv.nvfp4_gemm_w4a4_tiled(at, S, wp, S, S, alpha, None, "bf16", out, alpha_col=ac),
                        steps, warmup)
    del at
    ca, sa, _, _ = quantized_square(nv, S, "A", gen)
    ws = torch.empty(nv.workspace_bytes(nv.OP_W4A4, S, S, S), dtype=torch.uint8, device="cuda")
    ms_std = time_calls(lambda: nv.nvfp4_gemm_w4a4(ca, sa, wp, S, S, alpha, None, "bf16", out, ws), steps, warmup)
    return ms, 2.0 * S ** 3 / (ms * 1e-3) / 1e12, ms_std, ms_col


def w4a16_m1(nv, j, reps=3, per_column=False):
    """M = 1 decode on shape j, weights rotated over >= 1 GiB, replayed from a CUDA graph
    (per_column: with a per-column alpha as well)."""
    import numpy as np
    import torch
    import synth
    N, K = synth.DECODE_SHAPES[j]
    w = torch.from_numpy(synth.decode_weight(j)).cuda().view(torch.bfloat16)
    cw, sw, gW, _ = nv.nvfp4_quantize(w)
    del w
    wp, _ = nv.nvfp4_prepare_weight(cw, sw, "ue4m3")
    del cw, sw
    nbytes = wp.numel()
    R = max(2, -(-(1 << 30) // nbytes))
    copies = [wp] + [wp.clone() for _ in range(R - 1)]
    x = torch.from_numpy(synth.decode_activation(1, j, 0)).cuda().view(torch.bfloat16)
    alpha = float(np.float32(1.0) / np.float32(gW.item()))
    out = torch.empty((1, N), dtype=torch.bfloat16, device="cuda")
    ws = nv.workspace(nv.OP_W4A16, 1, N, K)
    ac = None
    if per_column:
        ac = torch.from_numpy(np.random.default_rng(7).uniform(0.5, 2.0, N).astype(np.float32)).cuda()
    for c in copies:
        nv.nvfp4_gemm_w4a16(x, c, N, K, alpha, out=out, ws=ws, alpha_col=ac)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            for c in copies:
                nv.nvfp4_gemm_w4a16(x, c, N, K, alpha, out=out, ws=ws, alpha_col=ac)
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        g.replay()
        e.record()
        e.synchronize()
        t = s.elapsed_time(e) / R
        best = t if best is None else min(best, t)
    weight_bytes = N * K // 2 + N * K // 16
    all_bytes = weight_bytes + 2 * K + 2 * N
    del copies, g
    torch.cuda.empty_cache()
    return dict(N=N, K=K, us=round(best * 1e3, 2), rotated_copies=R,
                GBps=round(all_bytes / (best * 1e-3) / 1e9, 1),
                weight_GBps=round(weight_bytes / (best * 1e-3) / 1e9, 1),
                hbm_frac=round(all_bytes / (best * 1e-3) / 1e9 / PEAK_HBM_GBS, 3))


def w4a16_m_sweep(nv, j, steps, warmup):
    """W4A16 on layer shape j at the batch sizes M > 1 of the decode workload (weights
    rotated over >= 1 GiB so every call streams them from HBM)."""
    import numpy as np
    import torch
    import synth
    N, K = synth.DECODE_SHAPES[j]
    w = torch.from_numpy(synth.decode_weight(j)).cuda().view(torch.bfloat16)
    cw, sw, gW, _ = nv.nvfp4_quantize(w)
    del w
    wp, _ = nv.nvfp4_prepare_weight(cw, sw, "ue4m3")
    del cw, sw
    R = max(2, -(-(1 << 30) // wp.numel()))
    copies = [wp] + [wp.clone() for _ in range(R - 1)]
    alpha = float(np.float32(1.0) / np.float32(gW.item()))
    res = []
    for i, M in enumerate(synth.DECODE_MS):
        if M == 1:
            continue
        x = torch.from_numpy(synth.decode_activation(M, j, i)).cuda().view(torch.bfloat16)
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ws = nv.workspace(nv.OP_W4A16, M, N, K)
        k = [0]

        def step():
            nv.nvfp4_gemm_w4a16(x, copies[k[0] % R], N, K, alpha, out=out, ws=ws)
            k[0] += 1
        ms = time_calls(step, max(steps, R), max(warmup, R))
        byts = N * K * 9 // 16 + 2 * M * K + 2 * M * N
        r = dict(M=M, N=N, K=K, us=round(ms * 1e3, 2), TFLOPs=round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1),
                 GBps=round(byts / (ms * 1e-3) / 1e9, 1))
        log(f"[bench] W4A16 M={M} {N}x{K}: {r}")
        res.append(r)
    del copies
    torch.cuda.empty_cache()
    return res


def prefill(nv, steps, warmup):
    import numpy as np
    import torch
    import synth
    x, _ = synth.prefill_activation()
    xd = torch.from_numpy(x).cuda().view(torch.bfloat16)
    w = torch.from_numpy(synth.prefill_weight()).cuda().view(torch.bfloat16)
    cw, sw, gW, _ = nv.nvfp4_quantize(w)
    wp, _ = nv.nvfp4_prepare_weight(cw, sw, "ue4m3")
    del w, cw, sw
    M, K = x.shape
    N = synth.PREFILL_W[0]
    alpha_w = float(np.float32(1.0) / np.float32(gW.item()))
    at = torch.empty(nv.lib().nvfp4_tiled_activation_bytes(M, K), dtype=torch.uint8, device="cuda")
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((M, K // 16), dtype=torch.uint8, device="cuda")
    g = torch.empty(1, dtype=torch.float32, device="cuda")
    ig = torch.empty(1, dtype=torch.float32, device="cuda")
    qws = torch.empty(nv.workspace_bytes(nv.OP_QUANTIZE, M, 0, K), dtype=torch.uint8, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    gws = torch.empty(nv.workspace_bytes(nv.OP_W4A4, M, N, K), dtype=torch.uint8, device="cuda")

    def quant():
        nv.nvfp4_quantize_tiled(xd, at, g, ig, qws)

    def gemm():
        nv.nvfp4_gemm_w4a4_tiled(at, M, wp, N, K, alpha_w, ig, "bf16", out)

    def step():
        quant()
        gemm()

    def step_row_major():
        nv.nvfp4_quantize(xd, codes, scales, g, ig, qws)
        nv.nvfp4_gemm_w4a4(codes, scales, wp, N, K, alpha_w, ig, "bf16", out, gws)
    # two-pass prefill: value and residual passes under one g, one contraction over 2K
    a2 = torch.empty(nv.lib().nvfp4_tiled_activation_bytes(M, 2 * K), dtype=torch.uint8, device="cuda")

    def quant2():
        nv.nvfp4_quantize_two_pass_tiled(xd, a2, g, ig, qws)

    def gemm2():
        nv.nvfp4_gemm_w4a4_two_pass_tiled(a2, M, wp, N, K, alpha_w, ig, "bf16", out)

    def step2():
        quant2()
        gemm2()
    q_ms = time_calls(quant, steps, warmup)
    g_ms = time_calls(gemm, steps, warmup)
    t_ms = time_calls(step, steps, warmup)
    r_ms = time_calls(step_row_major, steps, warmup)
    q2_ms = time_calls(quant2, steps, warmup)
    g2_ms = time_calls(gemm2, steps, warmup)
    t2_ms = time_calls(step2, steps, warmup)
    q_bytes = M * K * 2 + M * K // 2 + M * K // 16
    return dict(M=M, N=N, K=K, quantize_us=round(q_ms * 1e3, 1),
                quantize_GBps=round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
                gemm_ms=round(g_ms, 4), gemm_TFLOPs=round(2.0 * M * N * K / (g_ms * 1e-3) / 1e12, 1),
                total_ms=round(t_ms, 4), total_TFLOPs=round(2.0 * M * N * K / (t_ms * 1e-3) / 1e12, 1),
                row_major_path_ms=round(r_ms, 4),
                two_pass=dict(quantize_us=round(q2_ms * 1e3, 1), gemm_ms=round(g2_ms, 4),
                              gemm_TFLOPs_2K=round(4.0 * M * N * K / (g2_ms * 1e-3) / 1e12, 1),
                              total_ms=round(t2_ms, 4)))


def cpu_baseline(S=8192, rows=2048, cols=8192):
    """The oracle, as it stands, on a bounded sample of the 8k W4A4 workload:
    `rows` rows of A against `cols` rows of B over the full K (exact int64-chunked)."""
    import numpy as np
    import synth
    from oracle import gemm, quantize
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    xa = synth.square_normal(S, "A")
    xb = synth.square_normal(S, "B")
    gA, gB = quantize.global_scale(xa), quantize.global_scale(xb)
    a, sa = quantize.quantize_rows_with_g(xa[:rows], gA)
    b, sb = quantize.quantize_rows_with_g(xb[:cols], gB)
    del xa, xb
    alpha = np.float32(1.0) / np.float32(gA * gB)
    t0 = time.perf_counter()
    gemm.w4a4_exact(a, sa, b, sb, alpha)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * cols * S
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=int(threads), kind="oracle",
                sample=f"exact int64-chunked oracle, {rows} rows of A x {cols} rows of B, K={S} "
                       f"(of the {S}^3 problem), decode + GEMM timed: {dt:.2f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--size", type=int, default=8192)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the W4A16 M = 1 decode shapes (one JSON line; for profiling the decode kernels)")
    ap.add_argument("--sweep-only", action="store_true",
                    help="only the W4A16 M > 1 layer sweep (one JSON line; for profiling the MFMA kernels)")
    ap.add_argument("--large", action="store_true", help="also time the 32768^3 square (about 4 GiB of device memory)")
    ap.add_argument("--copy-ref", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_ref:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_ref_bytes_read": 1 << 30, "copy_ref_bytes_written": 1 << 30}), flush=True)
        return
    import nvfp4_block_scaled_amd as nv
    nv.init()
    if args.decode_only:
        import synth
        print(json.dumps({"w4a16_m1": [w4a16_m1(nv, j) for j in range(len(synth.DECODE_SHAPES))]}), flush=True)
        return
    if args.sweep_only:
        import synth
        print(json.dumps({"w4a16_m_sweep": [r for j in range(len(synth.DECODE_SHAPES))
                                            for r in w4a16_m_sweep(nv, j, args.steps, args.warmup)]}), flush=True)
        return
    S = args.size
    log(f"[bench] W4A4 {S}^3 bf16: {args.warmup} warmup + {args.steps} timed steps")
    ms, tflops, ms_std, ms_col = w4a4_square(nv, S, args.steps, args.warmup, standard_too=True)
    std_tflops = 2.0 * S ** 3 / (ms_std * 1e-3) / 1e12
    log(f"[bench] W4A4 {S}^3: {ms:.4f} ms/step, {tflops:.1f} TFLOP/s (A from nvfp4_quantize_tiled); "
        f"row-major A through nvfp4_gemm_w4a4 (tile copy + GEMM): {ms_std:.4f} ms, {std_tflops:.1f} TFLOP/s; "
        f"with a per-column alpha: {ms_col:.4f} ms")

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_hash") == kernel_hash() and tr.get("size") == S:
            traffic = tr.get("hbm_bytes_per_launch")

    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"W4A4 NVFP4 GEMM M=N=K={S}, A and B quantized on device from BF16 N(0,1) "
                               f"(per-16 E4M3 scale amax/6, per-tensor global scale), alpha=1/(gA gB), BF16 out",
                   "M": S, "N": S, "K": S, "out": "bf16",
                   "a_layout": "tile layout emitted by nvfp4_quantize_tiled (untimed, like B's prepare)",
                   "row_major_a_call_ms": round(ms_std, 5)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_F16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "gemm_kernel (the whole step)"},
    }
    if not args.no_extras:
        import synth
        extras = {}
        dec = []
        for j in range(len(synth.DECODE_SHAPES)):
            r = w4a16_m1(nv, j)
            log(f"[bench] W4A16 M=1 {r['N']}x{r['K']}: {r['us']} us, {r['GBps']} GB/s")
            dec.append(r)
        extras["w4a16_m1"] = dec
        r = w4a16_m1(nv, 2, per_column=True)
        log(f"[bench] W4A16 M=1 {r['N']}x{r['K']} with a per-column alpha: {r['us']} us")
        extras["per_column_alpha"] = {"w4a4_tiled_ms": round(ms_col, 5),
                                      "w4a4_tiled_TFLOPs": round(2.0 * S ** 3 / (ms_col * 1e-3) / 1e12, 1),
                                      "w4a16_m1": r}
        pf = prefill(nv, max(5, args.steps // 2), args.warmup)
        log(f"[bench] prefill: {pf}")
        extras["prefill_w4a4"] = pf
        extras["w4a16_m_sweep"] = [r for j in range(len(synth.DECODE_SHAPES))
                                   for r in w4a16_m_sweep(nv, j, args.steps, args.warmup)]
        sweep = {}
        for s2 in (2048, 4096):
            m2, t2 = w4a4_square(nv, s2, args.steps, args.warmup)
            sweep[str(s2)] = dict(ms=round(m2, 4), TFLOPs=round(t2, 1))
            log(f"[bench] W4A4 {s2}^3: {m2:.4f} ms, {t2:.1f} TFLOP/s")
        large = [16384] + ([32768] if args.large else [])
        for s2 in large:
            # 1 % of rows x8 and 1 % of 16-blocks zeroed, as the large-square workload states
            m2, t2 = w4a4_square(nv, s2, max(5, args.steps // 10), max(3, args.warmup // 10), gen=synth.square_large)
            sweep[str(s2)] = dict(ms=round(m2, 4), TFLOPs=round(t2, 1), inputs="outlier rows and zero blocks")
            log(f"[bench] W4A4 {s2}^3 (outliers, zero blocks): {m2:.4f} ms, {t2:.1f} TFLOP/s")
        extras["w4a4_square"] = sweep
        result["extras"] = extras
    torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(S)
        log(f"[bench] cpu_baseline: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
