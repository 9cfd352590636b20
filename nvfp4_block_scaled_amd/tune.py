"""Tuning sweep for the launch configurations of the GEMMs (the tuned table of csrc/config.hip).

On the current device, every valid configuration of each benchmark shape is timed back to back
(W4A16: graph replays over weight copies rotated across >= 1 GiB, so each call streams its
weight from HBM and no Python launch cost is counted; W4A4 on its tiled entry with the K-split
workspace). Where the fastest beats the heuristic's own config by more than 3 %, it becomes a
table entry keyed by the device's CU count, consecutive W4A16 batch sizes with the same winner
merged into one M range:

    python -m nvfp4_block_scaled_amd.tune [--out nvfp4_block_scaled_amd/csrc/tuned_table.inc]

Entries of other CU counts already in the file are kept. Rebuild the library afterwards.
Inputs are synthetic (N(0, 1) activations, N(0, 0.02) weights, quantized on the device).
"""
import argparse
import json
import os
import re
import sys

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
import nvfp4_block_scaled_amd as nv  # noqa: E402

LAYERS = [(6144, 5120), (5120, 5120), (34816, 5120), (5120, 17408)]
W4A16_MS = [1, 2, 4, 8, 16, 32, 48, 64, 96, 128, 192, 256, 384, 512, 768, 1024]
W4A4_SHAPES = [(8192, 17408, 5120), (2048, 17408, 5120), (8192, 5120, 17408), (8192, 34816, 5120),
               (8192, 6144, 5120), (8192, 5120, 5120), (2048, 2048, 2048), (4096, 4096, 4096),
               (8192, 8192, 8192), (16384, 16384, 16384)]
KNAMES = {nv.KERNEL_W4A4_TILES: "NVFP4_KERNEL_W4A4_TILES", nv.KERNEL_W4A16_DECODE: "NVFP4_KERNEL_W4A16_DECODE",
          nv.KERNEL_W4A16_SKINNY: "NVFP4_KERNEL_W4A16_SKINNY", nv.KERNEL_W4A16_TILES: "NVFP4_KERNEL_W4A16_TILES"}
TNAMES = {nv.TAIL_NONE: "NVFP4_TAIL_NONE", nv.TAIL_QUADRANTS: "NVFP4_TAIL_QUADRANTS", nv.TAIL_SPLIT: "NVFP4_TAIL_SPLIT"}


def _time(fn, calls, reps=3):
    for _ in range(max(5, calls // 2)):
        fn()
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(calls):
            fn()
        e.record()
        e.synchronize()
        t = s.elapsed_time(e) * 1e3 / calls
        best = t if best is None else min(best, t)
    return best


def _w4a16_candidates(M, K):
    c = []
    if M <= 4 and M * K * 2 <= 64 * 1024:
        c.append(nv.make_config(nv.KERNEL_W4A16_DECODE))
    if M <= 64:
        c.append(nv.make_config(nv.KERNEL_W4A16_SKINNY))
    for tm, tn in ((256, 256), (128, 256), (128, 128)):
        c.append(nv.make_config(nv.KERNEL_W4A16_TILES, tm, tn))
    return c


def _w4a4_candidates(K):
    c = [nv.make_config(nv.KERNEL_W4A4_TILES, 128, 128), nv.make_config(nv.KERNEL_W4A4_TILES, 256, 256),
         nv.make_config(nv.KERNEL_W4A4_TILES, 256, 256, nv.TAIL_QUADRANTS)]
    for S in (2, 3, 4):
        if S <= K // 64:
            c.append(nv.make_config(nv.KERNEL_W4A4_TILES, 256, 256, nv.TAIL_SPLIT, S))
    return c


def _key(c):
    return (c.kernel, c.tile_m, c.tile_n, c.tail, c.split_k, c.dynamic)


def _graph_time(calls, reps=3):
    """Per-call time of `calls` (a list of thunks) captured once in a graph and replayed: kernel time
    without the Python launch cost, which dominates a few-microsecond call timed eagerly."""
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
        t = s.elapsed_time(e) * 1e3 / len(calls)
        best = t if best is None else min(best, t)
    del g
    return best


def tune_w4a16(cus, log):
    rows = []
    for N, K in LAYERS:
        w = (0.02 * torch.randn(N, K, device="cuda")).to(torch.bfloat16)
        cw, sw, gW, _ = nv.nvfp4_quantize(w)
        wp, _ = nv.nvfp4_prepare_weight(cw, sw, "ue4m3")
        del w, cw, sw
        R = max(2, -(-(1 << 30) // wp.numel()))
        copies = [wp] + [wp.clone() for _ in range(R - 1)]
        for M in W4A16_MS:
            x = torch.randn(M, K, device="cuda").to(torch.bfloat16)
            out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            res = []
            for cfg in _w4a16_candidates(M, K):
                ws = nv.workspace(nv.OP_W4A16, M, N, K, config=cfg)
                calls = [lambda c=c, cfg=cfg, ws=ws: nv.nvfp4_gemm_w4a16(x, c, N, K, 1.0, out=out, ws=ws, config=cfg)
                         for c in copies]
                res.append((_graph_time(calls), cfg))
            rows.append(_pick(nv.OP_W4A16, M, N, K, cus, res, log))
        del copies
        torch.cuda.empty_cache()
    return [r for r in rows if r is not None]


def _pick(op, M, N, K, cus, res, log, margin=0.03):
    """The row for the table when the fastest config beats the heuristic's by more than `margin`."""
    heur = nv.get_config(op if op != nv.OP_W4A4 else nv.OP_W4A4_TILED, M, N, K, -cus)
    heur_t = [t for t, c in res if _key(c)[:5] == _key(heur)[:5]]
    best_t, best = min(res, key=lambda r: r[0])
    gain = heur_t[0] / best_t - 1 if heur_t else None
    log(dict(op="w4a16" if op == nv.OP_W4A16 else "w4a4", M=M, N=N, K=K, best_us=round(best_t, 2),
             best=best.as_dict(), heuristic=heur.as_dict(), heuristic_us=round(heur_t[0], 2) if heur_t else None,
             gain=round(gain, 4) if gain is not None else None, all={str(_key(c)): round(t, 2) for t, c in res}))
    if gain is None or gain > margin:
        return (op, N, K, M, best)
    return None


def tune_w4a4(cus, log):
    rows = []
    for M, N, K in W4A4_SHAPES:
        x = torch.randn(M, K, device="cuda").to(torch.bfloat16)
        w = (0.02 * torch.randn(N, K, device="cuda")).to(torch.bfloat16)
        at, _, ig = nv.nvfp4_quantize_tiled(x)
        cw, sw, _, _ = nv.nvfp4_quantize(w)
        wp, _ = nv.nvfp4_prepare_weight(cw, sw, "ue4m3")
        del x, w, cw, sw
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        flops = 2.0 * M * N * K
        calls = max(5, min(50, int(2e13 / flops)))
        res = []
        for cfg in _w4a4_candidates(K):
            ws = torch.empty(max(256, nv.workspace_bytes(nv.OP_W4A4_TILED, M, N, K, cfg)), dtype=torch.uint8,
                             device="cuda")
            us = _time(lambda: nv.nvfp4_gemm_w4a4_tiled(at, M, wp, N, K, 1.0, ig, "bf16", out, config=cfg, ws=ws),
                       calls)
            res.append((us, cfg))
        rows.append(_pick(nv.OP_W4A4, M, N, K, cus, res, log))
        del at, wp, out
        torch.cuda.empty_cache()
    return [r for r in rows if r is not None]


def _entry(cus, op, N, K, lo, hi, c):
    opname = "NVFP4_OP_W4A4" if op == nv.OP_W4A4 else "NVFP4_OP_W4A16"
    return (f"{{{cus}, {opname}, {N}, {K}, {lo}, {hi}, {{{KNAMES[c.kernel]}, {c.tile_m}, {c.tile_n}, "
            f"{TNAMES[c.tail]}, {c.split_k}, {c.dynamic}, {cus}, 0}}}},")


def table_lines(cus, rows):
    """Entries for one CU count; W4A16 batch sizes of one shape that are neighbours in W4A16_MS
    and have the same winner become one M range (from the first to the last measured M)."""
    lines = []
    i = 0
    while i < len(rows):
        op, N, K, M, c = rows[i]
        j = i
        while (j + 1 < len(rows) and rows[j + 1][:3] == (op, N, K) and op == nv.OP_W4A16
               and _key(rows[j + 1][4]) == _key(c)
               and W4A16_MS.index(rows[j + 1][3]) == W4A16_MS.index(rows[j][3]) + 1):
            j += 1
        lines.append(_entry(cus, op, N, K, M, rows[j][3], c))
        i = j + 1
    return lines


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=os.path.join(HERE, "csrc", "tuned_table.inc"))
    ap.add_argument("--log", default=None, help="JSON lines of every timing")
    args = ap.parse_args()
    nv.init()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    logf = open(args.log, "w") if args.log else None

    def log(row):
        print(json.dumps(row), flush=True)
        if logf:
            logf.write(json.dumps(row) + "\n")
            logf.flush()
    rows = tune_w4a4(cus, log) + tune_w4a16(cus, log)
    keep = []
    if os.path.exists(args.out):
        with open(args.out) as f:
            keep = [ln.rstrip("\n") for ln in f if ln.startswith("{") and not ln.startswith(f"{{{cus},")]
    header = [
        "// Tuned launch configurations: entries of kTuned in config.hip,",
        "// {cus, op, N, K, m_lo, m_hi, {kernel, tile_m, tile_n, tail, split_k, dynamic, num_cus, source}}.",
        "// Written by nvfp4_block_scaled_amd/tune.py (the fastest valid config of each benchmark shape,",
        "// timed on a device with `cus` CUs).",
    ]
    with open(args.out, "w") as f:
        f.write("\n".join(header + keep + table_lines(cus, rows)) + "\n")
    print(f"wrote {args.out}", flush=True)


if __name__ == "__main__":
    main()
