"""NVFP4 GEMMs on the CPU: W4A4 D = alpha (A.SFA)(B.SFB)^T and W4A16 y = alpha x (W.SFW)^T.

Test infrastructure (see the package docstring).

Definitions followed:
* Colfax article, introduction and "Version 2" (input shapes): A is M x K and B
  is N x K in 4-bit E2M1 with one 8-bit scale per 16 K-elements (SFA M x K/16,
  SFB N x K/16); the product accumulates in FP32 and the epilogue multiplies by
  alpha in FP32 before converting to the output type ("Version 3").
* TileLang PR #3290, "Summary": W4A16 keeps the activations x [M, K] in BF16
  and multiplies by the dequantized NVFP4 weight W [N, K] with a global or a
  per-column scale. Here alpha is either one FP32 value or an FP32 vector [N],
  one value per output column (column_alpha forms it), for both GEMMs.

Exact evaluation of W4A4. With v = E2M1 value and s = E4M3 value, 2v is an
integer in {0, +-1, +-2, +-3, +-4, +-6, +-8, +-12} and 2**9 s is an integer in
[0, 229376], so A^ = (2v)(2**9 s) is an integer with |A^| < 2**22 and every
product A^ B^ is below 2**44. Summing at most 512 of them stays below 2**53,
so a float64 matmul over K-chunks of 512 is exact in any summation order; the
chunk sums are added in int64. D = alpha * S * 2**-20.
"""
import numpy as np

from . import formats

_CHUNK = 512


def decode_nvfp4(codes_packed, scale_bytes, scale_kind="e4m3"):
    """[rows][K/2] packed codes + [rows][K/16] scale bytes -> float64 [rows][K] values code * scale."""
    codes = formats.unpack_nibbles(codes_packed)
    rows, K = codes.shape
    dec = formats.decode_e4m3 if scale_kind == "e4m3" else formats.decode_ue4m3
    s = dec(scale_bytes).reshape(rows, K // 16)
    v = formats.decode_e2m1(codes).reshape(rows, K // 16, 16)
    with np.errstate(invalid="ignore"):
        return (v * s[:, :, None]).reshape(rows, K)


def _integer_operand(codes_packed, scale_bytes, scale_kind):
    """(2 * fp4) * (2**9 * scale) as exact float64 integers, plus a per-row NaN flag."""
    codes = formats.unpack_nibbles(codes_packed)
    rows, K = codes.shape
    dec = formats.decode_e4m3 if scale_kind == "e4m3" else formats.decode_ue4m3
    s = dec(scale_bytes).reshape(rows, K // 16)
    nan_row = np.isnan(s).any(axis=1)
    s_int = np.where(np.isnan(s), 0.0, s) * 512.0
    v2 = formats.decode_e2m1(codes).reshape(rows, K // 16, 16) * 2.0
    return (v2 * s_int[:, :, None]).reshape(rows, K), nan_row


def w4a4_exact(a_codes, a_scales, b_codes, b_scales, alpha, a_kind="e4m3", b_kind="e4m3"):
    """Exact W4A4 result (float64, one final rounding) and sum_k |alpha a b| for the error bound.

    A rows or B rows holding a NaN scale give NaN outputs (NaN propagates).
    """
    ai, a_nan = _integer_operand(a_codes, a_scales, a_kind)
    bi, b_nan = _integer_operand(b_codes, b_scales, b_kind)
    M, K = ai.shape
    N = bi.shape[0]
    assert bi.shape[1] == K
    S = np.zeros((M, N), dtype=np.int64)
    T = np.zeros((M, N), dtype=np.int64)
    for k0 in range(0, K, _CHUNK):
        a = ai[:, k0:k0 + _CHUNK]
        b = bi[:, k0:k0 + _CHUNK]
        S += (a @ b.T).astype(np.int64)
        T += (np.abs(a) @ np.abs(b).T).astype(np.int64)
    al = _alpha64(alpha, N)
    D = S.astype(np.float64) * 2.0 ** -20 * al
    sum_abs = T.astype(np.float64) * 2.0 ** -20 * np.abs(al)
    D[a_nan, :] = np.nan
    D[:, b_nan] = np.nan
    return D, sum_abs


def w4a4_float64(a_codes, a_scales, b_codes, b_scales, alpha, a_kind="e4m3", b_kind="e4m3"):
    """Second, independent evaluation: decode to float64 and multiply directly."""
    a = decode_nvfp4(a_codes, a_scales, a_kind)
    b = decode_nvfp4(b_codes, b_scales, b_kind)
    return (a @ b.T) * _alpha64(alpha, b.shape[0])


def w4a16(x_bf16_bits, w_codes, w_scales, alpha, w_kind="e4m3"):
    """y = alpha * x W~^T in float64 (products exact; float64 summation) and sum_k |alpha x w|."""
    x = formats.bf16_bits_to_f32(x_bf16_bits).astype(np.float64)
    w = decode_nvfp4(w_codes, w_scales, w_kind)
    al = _alpha64(alpha, w.shape[0])
    y = (x @ w.T) * al
    with np.errstate(invalid="ignore"):
        sum_abs = (np.abs(x) @ np.abs(w).T) * np.abs(al)
    return y, sum_abs


def _alpha64(alpha, N):
    """alpha as float64: a scalar (rounded to FP32 first), or an FP32 vector of the N columns."""
    al = np.asarray(alpha)
    if al.ndim == 0:
        return float(np.float32(al))
    assert al.shape == (N,) and al.dtype == np.float32, "per-column alpha: float32 [N]"
    return al.astype(np.float64)


def column_alpha(alpha_eff, alpha_col):
    """Per-column alpha: fl32(alpha_eff * alpha_col[n]) for every output column n."""
    return (np.float32(alpha_eff) * np.asarray(alpha_col, np.float32)).astype(np.float32)


def alpha_product(alpha_host, alpha_dev=None):
    """alpha_eff = alpha_host * alpha_dev rounded to FP32 (alpha_dev absent -> alpha_host)."""
    a = np.float32(alpha_host)
    if alpha_dev is None:
        return a
    return np.float32(a * np.float32(alpha_dev))


def w4a4_two_pass_exact(a1_codes, a1_scales, a2_codes, a2_scales, b_codes, b_scales, alpha, b_kind="e4m3"):
    """Two-pass W4A4: D = alpha (A1 + A2) W~^T with A1, A2 the value and residual passes of one
    activation under one global scale. Written as one contraction over 2K, [A1 | A2] against
    [W | W], so the exact evaluation and its error bound are w4a4_exact's."""
    a = np.concatenate([a1_codes, a2_codes], axis=1)
    sa = np.concatenate([a1_scales, a2_scales], axis=1)
    b = np.concatenate([b_codes, b_codes], axis=1)
    sb = np.concatenate([b_scales, b_scales], axis=1)
    return w4a4_exact(a, sa, b, sb, alpha, "e4m3", b_kind)
