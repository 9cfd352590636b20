"""Shared helpers for the GPU parity tests (the tolerance of the NVFP4 GEMM
outputs, host <-> device moves, and quantize-then-verify of inputs)."""
import numpy as np
import torch

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


def assert_close(got, ref, sum_abs, bf16, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), f"{what}: NaN pattern differs"
    ok = ~nan_ref
    err = np.abs(got[ok] - ref[ok])
    tol = bound(ref[ok], sum_abs[ok], bf16)
    bad = err > tol
    if bad.any():
        i = np.argmax(err - tol)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside the bound; worst err {err[i]:.3e} "
                             f"tol {tol[i]:.3e} ref {ref[ok][i]:.6e} got {got[ok][i]:.6e}")
    # the pages' own, looser checks (TileLang PR #3290, 'Tests'): relative Frobenius error
    if ref[ok].size and np.linalg.norm(ref[ok]) > 0:
        rel = np.linalg.norm(got[ok] - ref[ok]) / np.linalg.norm(ref[ok])
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
