#!/usr/bin/env python3
"""Benchmark of the NVFP4 block-scaled GEMM library on one MI355X.

Step = one W4A4 NVFP4 GEMM D = alpha (A.SFA)(B.SFB)^T at M = N = K = 8192 with
BF16 output: A and B are BF16 N(0,1) tensors quantized on the device by the
library's quantizer, A straight into the layout the GEMM reads
(nvfp4_quantize_tiled) and B prepared once (both untimed), all inputs resident
in HBM when the timed region starts. One step is one nvfp4_gemm_w4a4_tiled
call, the GEMM kernel. `value` is TFLOP/s (2 M N K per step) from the mean step
time; the minimum is reported beside it. The default 50 warm-up steps (about
40 ms) bring the chip to its steady clock under this load; the first ~25
calls after idle run up to 10 % slower while the clock ramps. After the timed
steps the same call runs for 3 s while amdsmi samples the shader clock and
power (the driver refreshes them about once a second): the peak at the clock
the chip holds, 256 CUs x 4 SIMDs x 1024 FLOP/clk x f, is reported beside the
2.5 PFLOP/s one.

Extra figures in the same JSON line (`extras`): W4A16 decode (M = 1) achieved
HBM GB/s on the 27B-class layer shapes and the W4A16 batch sweep, both from
graph replays over weights rotated across >= 1 GiB; the prefill W4A4 with
on-device activation quantization (one- and two-pass, and the tail schedules:
quadrants, K split, dynamic); the other square sizes up to 32768^3; and a
context line with torch's own dense BF16 GEMM at 8192^3 on the same device.
`roofline` describes the dominant kernel, the W4A4 GEMM kernel (the whole
step); `cpu_baseline` times the CPU oracle on a bounded sample of the same
workload, with further legs (2048^3 in full, the prefill GEMM, decode GEMVs).

Usage: python bench.py [--gpus 1] [--steps 100] [--warmup 50] [--no-extras] [--no-large] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 GEMM TFLOP/s & % MFMA peak at 8k³; W4A16 M=1 achieved HBM GB/s"
PEAK_F16_TFLOPS = 2500.0          # MI355X dense FP16/BF16 MFMA (published)
PEAK_HBM_GBS = 8000.0             # MI355X HBM3E (published)
FLOP_PER_CLK = 256 * 4 * 1024     # CUs x SIMDs x dense FP16 FLOP per SIMD per clock
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


class ClockSampler:
    """Samples the GPU's shader (GFX) clock and socket power with amdsmi in a background thread.
    The driver refreshes these values about once a second, so only a region of a few seconds
    gives meaningful samples (sustained_clock); no-op when amdsmi is not available."""

    def __init__(self, period=0.05):
        self.period, self.samples, self._stop = period, [], threading.Event()
        self.ok = False
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            amdsmi.amdsmi_get_clock_info(self._h, amdsmi.AmdSmiClkType.GFX)
            self.ok = True
        except Exception as e:          # no amdsmi, no permission: report no clock
            self.err = repr(e)

    def _run(self):
        a = self._amdsmi
        t0 = time.perf_counter()
        while not self._stop.is_set():
            try:
                c = a.amdsmi_get_clock_info(self._h, a.AmdSmiClkType.GFX)
                p = a.amdsmi_get_power_info(self._h)
                w = p.get("current_socket_power", p.get("socket_power"))
                self.samples.append((time.perf_counter() - t0, float(c.get("clk", 0)),
                                     float(w) if isinstance(w, (int, float)) else None))
            except Exception:
                pass
            time.sleep(self.period)

    def __enter__(self):
        if self.ok:
            self._t = threading.Thread(target=self._run, daemon=True)
            self._t.start()
        return self

    def __exit__(self, *exc):
        if self.ok:
            self._stop.set()
            self._t.join()

    def stats(self, after=0.0):
        """Median clock and power of the samples taken `after` seconds into the region."""
        s = [x for x in self.samples if x[0] >= after and x[1] > 0]
        if not self.ok or not s:
            return None
        c = sorted(x[1] for x in s)
        w = sorted(x[2] for x in s if x[2] is not None)
        out = dict(samples=len(c), median_MHz=c[len(c) // 2], min_MHz=c[0], max_MHz=c[-1])
        if w:
            out["median_socket_power_W"] = w[len(w) // 2]
        return out


def sustained_clock(fn, seconds=3.0, settle=1.2):
    """The shader clock and power the chip holds under a loop of fn: fn is called back to back for
    `seconds` while amdsmi is sampled, and the samples after the first `settle` seconds (the clock
    ramp and the driver's one-second refresh) are summarised, with the loop's own ms per call."""
    import torch
    sampler = ClockSampler()
    if not sampler.ok:
        return None
    n = 0
    with sampler:
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        s.record()
        while time.perf_counter() - t0 < seconds:
            for _ in range(20):
                fn()
            n += 20
            torch.cuda.synchronize()
        e.record()
        e.synchronize()
    st = sampler.stats(after=settle)
    if st is not None:
        st.update(seconds=seconds, settle_s=settle, loop_ms_per_call=round(s.elapsed_time(e) / n, 5))
    return st


def time_steps(fn, steps, warmup, sampler=None, warm_s=0.0):
    """Warm-up, then `steps` calls bracketed by synchronisations and by one HIP event before and
    one after, on the launch stream: the mean ms per call over that region. Then a second run of
    up to 10 groups of g = max(1, min(10, steps // 10)) consecutive calls, with an event between
    groups only, for the fastest group's ms per call (an event between every two calls costs a
    few microseconds, which would inflate short calls). Returns (mean ms, fastest group's ms per
    call). The warm-up is `warmup` calls, continued until at least `warm_s` seconds have passed
    (short calls need many more than `warmup` to bring the clock to where it settles under
    load)."""
    import torch
    t0 = time.time()
    n = 0
    while n < warmup or time.time() - t0 < warm_s:
        fn()
        n += 1
        if n % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ctx = sampler if sampler is not None else _Null()
    with ctx:
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        e1.synchronize()
    torch.cuda.synchronize()
    mean = e0.elapsed_time(e1) / steps
    g = max(1, min(10, steps // 10))
    k = min(10, max(1, steps // g))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(k + 1)]
    ev[0].record()
    for i in range(k):
        for _ in range(g):
            fn()
        ev[i + 1].record()
    ev[-1].synchronize()
    torch.cuda.synchronize()
    return mean, min(ev[i].elapsed_time(ev[i + 1]) for i in range(k)) / g


class _Null:
    def __enter__(self):
        return self

    def __exit__(self, *exc):
        pass


def time_calls(fn, steps, warmup, warm_s=0.0):
    return time_steps(fn, steps, warmup, warm_s=warm_s)[0]


# untimed warm-up of the short legs (the 2048^3 and 4096^3 squares, the prefill parts): at
# least this long, so that they are timed at the clock the chip settles at, as the headline is
WARM_S_SHORT = 0.3


def graph_time(calls, reps=3):
    """Per-call ms of a list of thunks captured once in a CUDA (HIP) graph and replayed (best of
    reps): kernel time without host launch costs."""
    import torch
    for c in calls:
        c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            for c in calls:
                c()
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        g.replay()
        e.record()
        e.synchronize()
        t = s.elapsed_time(e) / len(calls)
        best = t if best is None else min(best, t)
    del g
    return best


def quantized_square(nv, S, operand, gen, tiled=False):
    """Device NVFP4 operand quantized by the library from the BF16 tensor gen(S, operand) (a host
    numpy array or a device tensor): (codes, scales, g, inv_g), or (tiled A, g, inv_g)."""
    import torch
    x = gen(S, operand)
    if isinstance(x, tuple):
        x = x[0]
    xd = x if isinstance(x, torch.Tensor) else torch.from_numpy(x).cuda().view(torch.bfloat16)
    res = nv.nvfp4_quantize_tiled(xd) if tiled else nv.nvfp4_quantize(xd)
    del xd, x
    return res


def square_large_device(S, operand):
    """The large square workload drawn on the device (seeded Philox): N(0,1), 1 % of the rows x8,
    each 16-block zeroed with probability 0.01 (zero wins); BF16 [S][S]. The same recipe as the
    host generator, drawn where the tensor lives (a 32768^2 host draw takes minutes)."""
    import math
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed((300 if operand == "A" else 400) + int(math.log2(S)))
    x = torch.randn((S, S), generator=g, device="cuda", dtype=torch.float32)
    rows = torch.randperm(S, generator=g, device="cuda")[:math.ceil(0.01 * S)]
    x[rows] *= 8.0
    zero = torch.rand((S, S // 16), generator=g, device="cuda") < 0.01
    x.view(S, S // 16, 16)[zero] = 0.0
    out = x.to(torch.bfloat16)
    del x, zero
    return out


def w4a4_square(nv, S, steps, warmup, gen=None, standard_too=False, clock=False, warm_s=0.0):
    """Step = the W4A4 GEMM on A as the quantizer emits it for the GEMM (the tile layout,
    nvfp4_quantize_tiled) and B prepared once: nvfp4_gemm_w4a4_tiled with the library's config.
    Returns dict(ms, ms_min, TFLOPs, ...); with standard_too, also the per-column-alpha call and
    nvfp4_gemm_w4a4 on the row-major A (tile copy + the same GEMM)."""
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
    gws = nv.workspace(nv.OP_W4A4_TILED, S, S, S)
    cfg = nv.get_config(nv.OP_W4A4_TILED, S, S, S)
    step = lambda: nv.nvfp4_gemm_w4a4_tiled(at, S, wp, S, S, alpha, None, "bf16", out, ws=gws)
    ms, ms_min = time_steps(step, steps, warmup, warm_s=warm_s)
    fl = 2.0 * S ** 3
    r = dict(ms=round(ms, 5), ms_min=round(ms_min, 5), TFLOPs=round(fl / (ms * 1e-3) / 1e12, 1),
             TFLOPs_at_min=round(fl / (ms_min * 1e-3) / 1e12, 1), config=cfg.as_dict())
    if warm_s:
        r["warmup_min_s"] = warm_s
    if clock:
        r["sustained_clock"] = sustained_clock(step)
    if standard_too:
        ac = torch.from_numpy(np.random.default_rng(7).uniform(0.5, 2.0, S).astype(np.float32)).cuda()
        ms_col = time_calls(lambda: nv.nvfp4_gemm_w4a4_tiled(at, S, wp, S, S, alpha, None, "bf16", out, alpha_col=ac,
                                                             ws=gws), steps, warmup)
        del at
        ca, sa, _, _ = quantized_square(nv, S, "A", gen)
        ws = nv.workspace(nv.OP_W4A4, S, S, S)
        ms_std = time_calls(lambda: nv.nvfp4_gemm_w4a4(ca, sa, wp, S, S, alpha, None, "bf16", out, ws), steps, warmup)
        r.update(per_column_alpha_ms=round(ms_col, 5), row_major_a_ms=round(ms_std, 5))
    return r


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
    best = graph_time([lambda c=c: nv.nvfp4_gemm_w4a16(x, c, N, K, alpha, out=out, ws=ws, alpha_col=ac)
                       for c in copies], reps)
    weight_bytes = N * K // 2 + N * K // 16
    all_bytes = weight_bytes + 2 * K + 2 * N
    del copies
    torch.cuda.empty_cache()
    return dict(N=N, K=K, us=round(best * 1e3, 2), rotated_copies=R,
                GBps=round(all_bytes / (best * 1e-3) / 1e9, 1),
                weight_GBps=round(weight_bytes / (best * 1e-3) / 1e9, 1),
                hbm_frac=round(all_bytes / (best * 1e-3) / 1e9 / PEAK_HBM_GBS, 3))


def w4a16_m_sweep(nv, j):
    """W4A16 on layer shape j at the batch sizes M > 1 of the decode workload: graph replays over
    weight copies rotated across >= 1 GiB, so every call streams its weight from HBM and the time
    is the kernels' (the eager calls' host launch cost is not counted)."""
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
        ms = graph_time([lambda c=c: nv.nvfp4_gemm_w4a16(x, c, N, K, alpha, out=out, ws=ws) for c in copies])
        byts = N * K * 9 // 16 + 2 * M * K + 2 * M * N
        fl = 2.0 * M * N * K
        r = dict(M=M, N=N, K=K, us=round(ms * 1e3, 2), TFLOPs=round(fl / (ms * 1e-3) / 1e12, 1),
                 GBps=round(byts / (ms * 1e-3) / 1e9, 1), hbm_frac=round(byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
                 mfma_frac=round(fl / (ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 3),
                 config=nv.get_config(nv.OP_W4A16, M, N, K).as_dict())
        log(f"[bench] W4A16 M={M} {N}x{K}: {r['us']} us")
        res.append(r)
    del copies
    torch.cuda.empty_cache()
    return res


def prefill(nv, steps, warmup):
    """The prefill workload: x [8192][5120] quantized on the device into the tile layout, then the
    W4A4 GEMM against a prepared [17408][5120] weight with alpha = 1/gW times the device 1/gA.
    Times the parts, the step, the row-major path, the two-pass variant, and the GEMM under each
    schedule of its last, partial round of tiles."""
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
    gws = nv.workspace(nv.OP_W4A4, M, N, K)
    tws = nv.workspace(nv.OP_W4A4_TILED, M, N, K)
    cfg = nv.get_config(nv.OP_W4A4_TILED, M, N, K)

    def quant():
        nv.nvfp4_quantize_tiled(xd, at, g, ig, qws)

    def gemm():
        nv.nvfp4_gemm_w4a4_tiled(at, M, wp, N, K, alpha_w, ig, "bf16", out, ws=tws)

    def step():
        quant()
        gemm()

    def step_row_major():
        nv.nvfp4_quantize(xd, codes, scales, g, ig, qws)
        nv.nvfp4_gemm_w4a4(codes, scales, wp, N, K, alpha_w, ig, "bf16", out, gws)
    a2 = torch.empty(nv.lib().nvfp4_tiled_activation_bytes(M, 2 * K), dtype=torch.uint8, device="cuda")

    def quant2():
        nv.nvfp4_quantize_two_pass_tiled(xd, a2, g, ig, qws)

    tws2 = nv.workspace(nv.OP_W4A4_TILED, M, N, 2 * K)

    def gemm2():
        nv.nvfp4_gemm_w4a4_two_pass_tiled(a2, M, wp, N, K, alpha_w, ig, "bf16", out, ws=tws2)

    def step2():
        quant2()
        gemm2()
    W = WARM_S_SHORT
    q_ms, q_min = time_steps(quant, steps, warmup, warm_s=W)
    g_ms, g_min = time_steps(gemm, steps, warmup, warm_s=W)
    t_ms, t_min = time_steps(step, steps, warmup, warm_s=W)
    r_ms = time_calls(step_row_major, steps, warmup, warm_s=W)
    q2_ms = time_calls(quant2, steps, warmup, warm_s=W)
    g2_ms = time_calls(gemm2, steps, warmup, warm_s=W)
    t2_ms = time_calls(step2, steps, warmup, warm_s=W)
    sched = {}
    for name, c in (("quadrants", nv.make_config(nv.KERNEL_W4A4_TILES, 256, 256, nv.TAIL_QUADRANTS)),
                    ("split2", nv.make_config(nv.KERNEL_W4A4_TILES, 256, 256, nv.TAIL_SPLIT, 2)),
                    ("split4", nv.make_config(nv.KERNEL_W4A4_TILES, 256, 256, nv.TAIL_SPLIT, 4)),
                    ("one_more_round", nv.make_config(nv.KERNEL_W4A4_TILES, 256, 256)),
                    ("quadrants_dynamic", nv.make_config(nv.KERNEL_W4A4_TILES, 256, 256, nv.TAIL_QUADRANTS,
                                                         dynamic=1)),
                    ("split2_dynamic", nv.make_config(nv.KERNEL_W4A4_TILES, 256, 256, nv.TAIL_SPLIT, 2,
                                                      dynamic=1))):
        ws = nv.workspace(nv.OP_W4A4_TILED, M, N, K, config=c)
        ms = time_calls(lambda: nv.nvfp4_gemm_w4a4_tiled(at, M, wp, N, K, alpha_w, ig, "bf16", out, config=c, ws=ws),
                        steps, warmup, warm_s=W)
        sched[name] = round(ms, 4)
    q_bytes = M * K * 2 + M * K // 2 + M * K // 16
    fl = 2.0 * M * N * K
    return dict(M=M, N=N, K=K, config=cfg.as_dict(), warmup_min_s=W, quantize_us=round(q_ms * 1e3, 1),
                quantize_us_min=round(q_min * 1e3, 1), quantize_GBps=round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
                quantize_hbm_frac=round(q_bytes / (q_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
                gemm_ms=round(g_ms, 4), gemm_ms_min=round(g_min, 4), gemm_TFLOPs=round(fl / (g_ms * 1e-3) / 1e12, 1),
                total_ms=round(t_ms, 4), total_ms_min=round(t_min, 4),
                total_TFLOPs=round(fl / (t_ms * 1e-3) / 1e12, 1), row_major_path_ms=round(r_ms, 4),
                tail_schedules_gemm_ms=sched,
                two_pass=dict(quantize_us=round(q2_ms * 1e3, 1), gemm_ms=round(g2_ms, 4),
                              gemm_TFLOPs_2K=round(2 * fl / (g2_ms * 1e-3) / 1e12, 1), total_ms=round(t2_ms, 4)))


def torch_bf16_context(S=8192, steps=20, warmup=10):
    """Context only (not the target): torch's dense BF16 GEMM (its BLAS library) at S^3 on the
    same device, the B operand contiguous."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    a = torch.randn((S, S), generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randn((S, S), generator=g, device="cuda").to(torch.bfloat16)
    c = torch.empty((S, S), dtype=torch.bfloat16, device="cuda")
    ms = time_calls(lambda: torch.matmul(a, b, out=c), steps, warmup)
    del a, b, c
    torch.cuda.empty_cache()
    return dict(op=f"torch.matmul bf16 {S}^3 (dense BF16, context only)", ms=round(ms, 4),
                TFLOPs=round(2.0 * S ** 3 / (ms * 1e-3) / 1e12, 1))


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(S=8192, rows=2048, cols=8192):
    """The oracle, as it stands, on a bounded sample of the 8k W4A4 workload: `rows` rows of A
    against `cols` rows of B over the full K (exact int64-chunked), plus legs: 2048^3 in full,
    the prefill GEMM on a sample of its rows, and decode-once + GEMV at M = 1 per layer shape."""
    import numpy as np
    import synth
    from oracle import gemm, quantize
    threads = _blas_threads()
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
    legs = {}
    # 2048^3, the whole problem
    S2 = 2048
    xa, xb = synth.square_normal(S2, "A"), synth.square_normal(S2, "B")
    a2, sa2, gA2, _ = quantize.quantize(xa)
    b2, sb2, gB2, _ = quantize.quantize(xb)
    t0 = time.perf_counter()
    gemm.w4a4_exact(a2, sa2, b2, sb2, np.float32(1.0) / np.float32(gA2 * gB2))
    d2 = time.perf_counter() - t0
    legs["w4a4_2048_full"] = dict(s=round(d2, 3), TFLOPs=round(2.0 * S2 ** 3 / d2 / 1e12, 4))
    # the prefill GEMM: 1024 of its 8192 rows against the whole weight
    xp, _ = synth.prefill_activation()
    gp = quantize.global_scale(xp)
    ap, sap = quantize.quantize_rows_with_g(xp[:1024], gp)
    wcodes, wsc, gw, _ = quantize.quantize(synth.prefill_weight())
    t0 = time.perf_counter()
    gemm.w4a4_exact(ap, sap, wcodes, wsc, np.float32(1.0) / np.float32(gp * gw))
    d3 = time.perf_counter() - t0
    Np, Kp = synth.PREFILL_W
    legs["prefill_1024_rows"] = dict(s=round(d3, 3), TFLOPs=round(2.0 * 1024 * Np * Kp / d3 / 1e12, 4),
                                     full_extrapolated_s=round(d3 * 8, 2))
    del xp, ap, sap, wcodes, wsc
    # decode: the weight decoded once, then the M = 1 GEMV, per layer shape
    dec = []
    for j, (N, K) in enumerate(synth.DECODE_SHAPES):
        wc, ws_, gw, _ = quantize.quantize(synth.decode_weight(j))
        x1 = synth.decode_activation(1, j, 0)
        t0 = time.perf_counter()
        gemm.w4a16(x1, wc, ws_, np.float32(1.0) / gw)
        dd = time.perf_counter() - t0
        nb = N * K * 9 // 16 + 2 * K + 2 * N
        dec.append(dict(N=N, K=K, s=round(dd, 3), GBps=round(nb / dd / 1e9, 3)))
        del wc, ws_
    legs["w4a16_m1_decode_plus_gemv"] = dec
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=int(threads), kind="oracle",
                cpu_model=_cpu_model(),
                sample=f"exact int64-chunked oracle, {rows} rows of A x {cols} rows of B, K={S} "
                       f"(of the {S}^3 problem), decode + GEMM timed: {dt:.2f} s", legs=legs)


def main():
    global WARM_S_SHORT
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--size", type=int, default=8192)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-large", action="store_true", help="skip the 16384^3 and 32768^3 squares")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the W4A16 M = 1 decode shapes (one JSON line; for profiling the decode kernels)")
    ap.add_argument("--sweep-only", action="store_true",
                    help="only the W4A16 M > 1 layer sweep (one JSON line; for profiling the MFMA kernels)")
    ap.add_argument("--warm-s", type=float, default=WARM_S_SHORT,
                    help="least untimed warm-up of the short legs, in seconds (0 under a profiler)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the prefill leg (one JSON line; for profiling the quantizer and its GEMM)")
    ap.add_argument("--square-only", type=int, default=0,
                    help="only the W4A4 square of this size (one JSON line; for profiling at 16k / 32k)")
    ap.add_argument("--copy-ref", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (calibrates HBM byte counters)")
    args = ap.parse_args()
    WARM_S_SHORT = args.warm_s
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
    import synth
    if args.decode_only:
        print(json.dumps({"w4a16_m1": [w4a16_m1(nv, j) for j in range(len(synth.DECODE_SHAPES))]}), flush=True)
        return
    if args.sweep_only:
        print(json.dumps({"w4a16_m_sweep": [r for j in range(len(synth.DECODE_SHAPES))
                                            for r in w4a16_m_sweep(nv, j)]}), flush=True)
        return
    if args.prefill_only:
        print(json.dumps({"prefill_w4a4": prefill(nv, max(10, args.steps // 2), args.warmup)}), flush=True)
        return
    if args.square_only:
        s2 = args.square_only
        gen = square_large_device if s2 >= 16384 else None
        print(json.dumps({"w4a4_square": {str(s2): w4a4_square(nv, s2, args.steps, args.warmup, gen=gen)}}),
              flush=True)
        return
    S = args.size
    log(f"[bench] W4A4 {S}^3 bf16: {args.warmup} warmup + {args.steps} timed steps")
    head = w4a4_square(nv, S, args.steps, args.warmup, standard_too=True, clock=not args.no_extras)
    ms, tflops = head["ms"], head["TFLOPs"]
    clk = head.get("sustained_clock")
    log(f"[bench] W4A4 {S}^3: {head}")

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_hash") == kernel_hash() and tr.get("size") == S:
            traffic = tr.get("hbm_bytes_per_launch")
    roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_F16_TFLOPS, 4), "traffic": traffic,
            "kernel": "gemm_kernel (the whole step)", "algorithmic_flop_per_launch": 2.0 * S ** 3,
            "launch_ms_mean": ms, "launch_ms_min": head["ms_min"]}
    if clk:
        # the peak at the clock the chip holds under this loop (power-capped below 2.4 GHz)
        peak_clk = FLOP_PER_CLK * clk["median_MHz"] * 1e6 / 1e12
        roof.update(sclk_MHz_sustained=clk["median_MHz"], peak_at_sclk=round(peak_clk, 1),
                    frac_at_sclk=round(tflops / peak_clk, 4))
    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"W4A4 NVFP4 GEMM M=N=K={S}, A and B quantized on device from BF16 N(0,1) "
                               f"(per-16 E4M3 scale amax/6, per-tensor global scale), alpha=1/(gA gB), BF16 out",
                   "M": S, "N": S, "K": S, "out": "bf16",
                   "a_layout": "tile layout emitted by nvfp4_quantize_tiled (untimed, like B's prepare)",
                   "ms_min": head["ms_min"], "row_major_a_call_ms": head["row_major_a_ms"],
                   "launch_config": head["config"]},
        "roofline": roof,
    }
    if not args.no_extras:
        extras = {"headline": head}
        dec = []
        for j in range(len(synth.DECODE_SHAPES)):
            r = w4a16_m1(nv, j)
            log(f"[bench] W4A16 M=1 {r['N']}x{r['K']}: {r['us']} us, {r['GBps']} GB/s")
            dec.append(r)
        extras["w4a16_m1"] = dec
        r = w4a16_m1(nv, 2, per_column=True)
        log(f"[bench] W4A16 M=1 {r['N']}x{r['K']} with a per-column alpha: {r['us']} us")
        extras["per_column_alpha"] = {"w4a4_tiled_ms": head["per_column_alpha_ms"],
                                      "w4a4_tiled_TFLOPs": round(2.0 * S ** 3 / (head["per_column_alpha_ms"] * 1e-3)
                                                                 / 1e12, 1),
                                      "w4a16_m1": r}
        pf = prefill(nv, max(10, args.steps // 2), args.warmup)
        log(f"[bench] prefill: {pf}")
        extras["prefill_w4a4"] = pf
        extras["w4a16_m_sweep"] = [r for j in range(len(synth.DECODE_SHAPES)) for r in w4a16_m_sweep(nv, j)]
        sweep = {}
        for s2 in (2048, 4096):
            sweep[str(s2)] = w4a4_square(nv, s2, args.steps, args.warmup, warm_s=WARM_S_SHORT)
            log(f"[bench] W4A4 {s2}^3: {sweep[str(s2)]}")
        if not args.no_large:
            for s2 in (16384, 32768):
                r = w4a4_square(nv, s2, max(5, args.steps // 10), max(3, args.warmup // 10), gen=square_large_device)
                r.update(inputs="outlier rows and zero blocks (drawn on the device)")
                sweep[str(s2)] = r
                log(f"[bench] W4A4 {s2}^3: {r}")
                torch.cuda.empty_cache()
        extras["w4a4_square"] = sweep
        extras["context"] = torch_bf16_context()
        log(f"[bench] context: {extras['context']}")
        result["extras"] = extras
    torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(S)
        log(f"[bench] cpu_baseline: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
