"""BF16 -> NVFP4 quantizer (per-tensor global scale, per-16 E4M3 scale, E2M1 codes).

Test infrastructure (see the package docstring).

The pages name the format and the workloads (block scale = amax/6 of a 16-block
in E4M3, a per-tensor global scale; TileLang PR #3290, "Summary" and
"Follow-ups") but print no recipe. The reading taken, every operation an IEEE
binary32 operation with round-to-nearest-even, no fused multiply-add, no
denormal flush, in this order:

1. x: BF16 -> FP32 (exact).
2. amax_t = max |x| over the tensor; g = 2688 / amax_t (2688 = 448 * 6, so the
   block holding amax_t gets the largest E4M3 scale); g = 1 if amax_t == 0.
3. per 16-block: amax_b = max |x|; t = amax_b / 6; u = t * g;
   scale byte = E4M3 RNE of u, saturating at 448; a block with amax_b == 0 gets
   scale byte 0 (also when g is infinite).
4. s = value of that byte. If s == 0 every code of the block is 0x0. Otherwise
   r = g / s and, per element, v = x * r, code = signbit(x) << 3 | E2M1 RNE of
   |v| (ties to the even code, saturating at 6).
5. codes are packed two per byte (low nibble = even k); scales are UE4M3 bytes.
6. the dequantized tensor is codes * s / g, so the GEMM's alpha carries 1/g:
   inv_g = 1 / g in FP32.
"""
import numpy as np

from . import formats


def quantize(x_bf16_bits):
    """Quantize a [rows][K] BF16 tensor (uint16 bit patterns), K % 16 == 0.

    Returns (codes [rows][K/2] uint8, scales [rows][K/16] uint8 UE4M3,
    g float32, inv_g float32).
    """
    xb = np.asarray(x_bf16_bits, dtype=np.uint16)
    assert xb.ndim == 2 and xb.shape[1] % 16 == 0
    g = global_scale(xb)                                   # steps 1-2
    codes, scales = quantize_rows_with_g(xb, g)            # steps 3-5
    with np.errstate(divide="ignore"):
        inv_g = np.float32(np.float32(1.0) / g)            # step 6
    return codes, scales, g, inv_g


def global_scale(x_bf16_bits):
    """Step 2 alone: g for a BF16 tensor."""
    x = formats.bf16_bits_to_f32(np.asarray(x_bf16_bits, dtype=np.uint16))
    amax_t = np.float32(np.abs(x).max()) if x.size else np.float32(0)
    with np.errstate(divide="ignore", over="ignore"):
        return np.float32(np.float32(2688.0) / amax_t) if amax_t != 0 else np.float32(1.0)


def quantize_rows_with_g(x_bf16_bits, g):
    """Steps 3-5 for a subset of rows, given the tensor's global scale g (for row-sampled checks)."""
    xb = np.asarray(x_bf16_bits, dtype=np.uint16)
    rows, K = xb.shape
    return quantize_f32_rows_with_g(formats.bf16_bits_to_f32(xb).reshape(rows, K), g)


def quantize_f32_rows_with_g(x, g):
    """Steps 3-5 on FP32 values [rows][K] (the residual pass of the two-pass recipe below)."""
    x = np.asarray(x, dtype=np.float32)
    rows, K = x.shape
    f32 = np.float32
    g = f32(g)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        amax_b = np.abs(x).reshape(rows, K // 16, 16).max(axis=2).astype(np.float32)
        u = ((amax_b / f32(6.0)).astype(np.float32) * g).astype(np.float32)
    s_byte = formats.round_e4m3_byte(u)
    s_byte[amax_b == 0] = 0
    s = formats.decode_e4m3(s_byte).astype(np.float32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        r = np.where(s != 0, g / np.where(s != 0, s, f32(1)), f32(0)).astype(np.float32)
        v = (x.reshape(rows, K // 16, 16) * r[:, :, None]).astype(np.float32)
    mag = formats.round_e2m1_magnitude(np.abs(v))
    sign = np.signbit(x.reshape(rows, K // 16, 16)).astype(np.uint8)
    codes = (sign << 3) | mag
    codes[s == 0] = 0
    return formats.pack_nibbles(codes.reshape(rows, K)), s_byte.astype(np.uint8)


def dequantize_with_g(codes_packed, scale_bytes, g):
    """The FP32 value each code stands for: fl32(code * scale / g). code * scale is exact in FP32
    (at most 6 significant bits); the division by the global scale is the one rounding."""
    v = formats.decode_e2m1(formats.unpack_nibbles(codes_packed)).astype(np.float64)
    rows, K = v.shape
    s = formats.decode_e4m3(np.asarray(scale_bytes, dtype=np.uint8)).astype(np.float64)
    prod = (v.reshape(rows, K // 16, 16) * s[:, :, None]).reshape(rows, K).astype(np.float32)
    return (prod / np.float32(g)).astype(np.float32)


def two_pass_rows_with_g(x_bf16_bits, g):
    """Two NVFP4 passes over the activations, value then residual (TileLang PR #3290, "Follow-ups":
    the W4A4 prefill that quantizes activations in two passes). Pass 1 is the quantizer above;
    the residual r = fl32(x - dequantize(pass 1)) is quantized by the same steps under the same
    global scale g, so both passes share one alpha. Returns (codes1, scales1, codes2, scales2)."""
    xb = np.asarray(x_bf16_bits, dtype=np.uint16)
    rows, K = xb.shape
    x = formats.bf16_bits_to_f32(xb).reshape(rows, K)
    c1, s1 = quantize_f32_rows_with_g(x, g)
    r = (x - dequantize_with_g(c1, s1, g)).astype(np.float32)
    c2, s2 = quantize_f32_rows_with_g(r, g)
    return c1, s1, c2, s2


def two_pass(x_bf16_bits):
    """two_pass_rows_with_g over a whole tensor with its global scale: (c1, s1, c2, s2, g, 1/g)."""
    g = global_scale(x_bf16_bits)
    c1, s1, c2, s2 = two_pass_rows_with_g(x_bf16_bits, g)
    return c1, s1, c2, s2, g, np.float32(np.float32(1.0) / g)
