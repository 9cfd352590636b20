"""Shared helpers for the GPU parity tests (the tolerance of the NVFP4 GEMM
outputs, host <-> device moves, quantize-then-verify of inputs, and the oracle run over
row or tile blocks on the host's cores for full-size checks)."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch
from threadpoolctl import threadpool_limits

from oracle import formats, gemm, quantize

# Error bound for FP32 outputs: |gpu - ref| <= 1e-5 * sum_k |alpha a b| + 1e-6 per
# element (ref exact). BF16 outputs add the round-to-nearest-even half ulp of
# the FP32 value: 2**-8 |ref| + (1 + 2**-8) * (FP32 bound).
REL = 1e-5
ABS = 1e-6


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def bound(ref, sum_abs, bf16):
    tol = REL * sum_abs + ABS
    if bf16:
        tol = 2.0 ** -8 * np.abs(ref) + (1 + 2.0 ** -8) * tol
    return tol


def _close_block(got, ref, sum_abs, bf16):
    """Per-block pieces of assert_close: None if the NaN patterns differ, else
    (n_bad, worst excess, its err, tol, ref, got, squared error sum, squared ref sum)."""
    nan_ref = np.isnan(ref)
    if not np.array_equal(np.isnan(got), nan_ref):
        return None
    if nan_ref.any():
        ok = ~nan_ref
        got, ref, sum_abs = got[ok], ref[ok], sum_abs[ok]
    if ref.size == 0:
        return 0, -np.inf, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0
    diff = got - ref
    err = np.abs(diff)
    tol = bound(ref, sum_abs, bf16)
    excess = err - tol
    i = int(np.argmax(excess))
    return (int(np.count_nonzero(excess > 0)), excess.flat[i], err.flat[i], tol.flat[i], ref.flat[i],
            got.flat[i], float(np.dot(diff.ravel(), diff.ravel())), float(np.dot(ref.ravel(), ref.ravel())))


def assert_close(got, ref, sum_abs, bf16, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    sum_abs = np.asarray(sum_abs, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.ndim == 2 and ref.size > (1 << 22):
        step = max(1, (1 << 20) // ref.shape[1])
        parts = _on_host_cores(lambda r: _close_block(got[r:r + step], ref[r:r + step], sum_abs[r:r + step], bf16),
                               range(0, ref.shape[0], step))
    else:
        parts = [_close_block(got, ref, sum_abs, bf16)]
    assert all(p is not None for p in parts), f"{what}: NaN pattern differs"
    n_bad = sum(p[0] for p in parts)
    if n_bad:
        w = max(parts, key=lambda p: p[1])
        n_ok = int(np.count_nonzero(~np.isnan(ref)))
        raise AssertionError(f"{what}: {n_bad} of {n_ok} outside the bound; worst err {w[2]:.3e} "
                             f"tol {w[3]:.3e} ref {w[4]:.6e} got {w[5]:.6e}")
    # the pages' own, looser checks (TileLang PR #3290, 'Tests'): relative Frobenius error
    num, den = sum(p[6] for p in parts), sum(p[7] for p in parts)
    if den > 0:
        rel = np.sqrt(num / den)
        assert rel <= 2.5e-3, f"{what}: relative Frobenius error {rel}"


def gpu_quantize_checked(nv, x_bits, sample_rows):
    """Quantize BF16 bits on the GPU (product path); check g, inv_g and the sampled rows'
    bytes against the oracle's own quantization of the same BF16 rows.

    Returns the device tensors (codes, scales, g, inv_g) and the oracle's g."""
    xd = dev(x_bits).view(torch.bfloat16)
    codes, scales, g, inv_g = nv.nvfp4_quantize(xd)
    g_ref = quantize.global_scale(x_bits)
    assert np.float32(g.item()) == g_ref
    assert np.float32(inv_g.item()) == np.float32(np.float32(1.0) / g_ref)
    c_ref, s_ref = quantize.quantize_rows_with_g(x_bits[sample_rows], g_ref)
    np.testing.assert_array_equal(codes[torch.as_tensor(sample_rows).cuda()].cpu().numpy(), c_ref)
    np.testing.assert_array_equal(scales[torch.as_tensor(sample_rows).cuda()].cpu().numpy(), s_ref)
    return codes, scales, g, inv_g, g_ref


def e4m3_scales_from_targets(t):
    return formats.round_e4m3_byte(t)


def alpha_ab(gA, gB):
    """alpha = fl(1 / fl(gA * gB)) in FP32."""
    return np.float32(np.float32(1.0) / np.float32(np.float32(gA) * np.float32(gB)))


def _workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _on_host_cores(fn, items):
    """fn over items in host threads, one BLAS thread each (the blocks are independent)."""
    with threadpool_limits(1), ThreadPoolExecutor(_workers()) as ex:
        return list(ex.map(fn, items))


def oracle_quantize_full(x_bits, rows_per_block=256):
    """The oracle's quantization of a whole tensor: its global scale, then
    quantize_rows_with_g on blocks of rows (given g, each row is quantized on its own).

    Returns (codes, scales, g)."""
    g = quantize.global_scale(x_bits)
    parts = _on_host_cores(lambda r: quantize.quantize_rows_with_g(x_bits[r:r + rows_per_block], g),
                           range(0, x_bits.shape[0], rows_per_block))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]), g


def oracle_w4a4_exact_blocked(a, sa, b, sb, alpha, tile=2048):
    """gemm.w4a4_exact on tile x tile blocks of D (an output element depends only on its
    row of A and its row of B); returns (D, sum_abs) like the unblocked call."""
    M, N = a.shape[0], b.shape[0]
    D = np.empty((M, N))
    S = np.empty((M, N))

    def run(rc):
        r, c = rc
        al = alpha[c:c + tile] if np.ndim(alpha) else alpha      # a per-column alpha goes with its columns
        d, t = gemm.w4a4_exact(a[r:r + tile], sa[r:r + tile], b[c:c + tile], sb[c:c + tile], al)
        D[r:r + tile, c:c + tile] = d
        S[r:r + tile, c:c + tile] = t
    _on_host_cores(run, [(r, c) for r in range(0, M, tile) for c in range(0, N, tile)])
    return D, S


def oracle_w4a16_blocked(x, w_codes, w_scales, alpha, cols=2048):
    """gemm.w4a16 on blocks of weight rows (output columns); returns (y, sum_abs)."""
    M, N = x.shape[0], w_codes.shape[0]
    y = np.empty((M, N))
    S = np.empty((M, N))

    def run(c):
        al = alpha[c:c + cols] if np.ndim(alpha) else alpha
        yy, t = gemm.w4a16(x, w_codes[c:c + cols], w_scales[c:c + cols], al)
        y[:, c:c + cols] = yy
        S[:, c:c + cols] = t
    _on_host_cores(run, range(0, N, cols))
    return y, S
