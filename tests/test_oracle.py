"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a relation printed on the pages,
a library routine (torch's float8_e4m3fn / bfloat16 casts), exact rational
arithmetic, brute force over tiny inputs, or a closed form worked by hand
(tests/golden/hand_worked.json).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats, gemm, prepared, quantize
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ E2M1

def test_e2m1_bf16_subnormal_relation():
    """TileLang PR #3290, 'Design: Weight layout': an E2M1 code placed in the BF16
    subnormal range reads as fp4 * 2**-126. Put the sign at bit 15 and the three
    exponent/mantissa bits at bits 8..6; torch's bfloat16 decodes the result."""
    codes = np.arange(16, dtype=np.uint16)
    bits = ((codes & 8) << 12) | ((codes & 7) << 6)
    vals = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(vals, formats.E2M1_TABLE * 2.0 ** -126)


def test_e2m1_eight_magnitudes():
    assert list(formats.E2M1_MAGNITUDES) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert np.signbit(formats.E2M1_TABLE[8]) and formats.E2M1_TABLE[8] == 0
    np.testing.assert_array_equal(formats.E2M1_TABLE[8:], -formats.E2M1_TABLE[:8])


# ------------------------------------------------------------------ E4M3

def test_e4m3_matches_torch_float8_e4m3fn():
    b = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = formats.E4M3_TABLE
    nan = np.isnan(b)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], b[~nan])


def test_e4m3_spot_values():
    v = formats.E4M3_TABLE
    assert v[0x38] == 1.0 and v[0x7E] == 448.0 and v[0x01] == 2.0 ** -9
    assert v[0x08] == 2.0 ** -6 and v[0x69] == 72.0 and v[0xB8] == -1.0


def test_e4m3_bf16_reencode_relation():
    """TileLang PR #3290, 'Design: Weight layout': each finite E4M3 scale has a byte b
    with bf16(0x7000 | b << 4) == scale * 2**119, subnormals included."""
    b = np.arange(256, dtype=np.uint32)
    pat = (0x7000 | (b << 4)) & 0xFFFF
    cand = torch.from_numpy(pat.astype(np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    cand = set(cand.tolist())
    for byte in range(1, 0x7F):
        s = formats.E4M3_TABLE[byte]
        assert s * 2.0 ** 119 in cand, hex(byte)


def test_ue4m3_rejects_sign_bit():
    v = formats.decode_ue4m3(np.array([0x38, 0xB8, 0x7F, 0x00]))
    assert v[0] == 1.0 and np.isnan(v[1]) and np.isnan(v[2]) and v[3] == 0.0


# ------------------------------------------------------------------ encoders

def _all_bf16_nonneg_finite():
    bits = np.arange(0, 0x7F80, dtype=np.uint32)          # +0 .. largest finite
    return (bits << 16).view(np.float32)


def test_round_e2m1_exhaustive_vs_brute_force():
    y = _all_bf16_nonneg_finite().astype(np.float64)
    got = formats.round_e2m1_magnitude(y)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    ys = np.minimum(y, 6.0)                              # saturation
    d = np.abs(ys[:, None] - mags[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # nearest; on a tie the even code index
    idx = np.where(cand.sum(axis=1) > 1, np.argmax(cand & (np.arange(8) % 2 == 0), axis=1), np.argmax(cand, axis=1))
    np.testing.assert_array_equal(got, idx.astype(np.uint8))


def test_round_e2m1_edges():
    y = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 1e30, np.inf, np.nan])
    np.testing.assert_array_equal(formats.round_e2m1_magnitude(y), [0, 2, 2, 4, 4, 6, 6, 7, 7, 7, 0])


def test_round_e4m3_vs_torch_cast():
    """torch's float8_e4m3fn cast is RNE; it turns values above the largest finite one
    into NaN, so inputs are clamped to 448 first (the saturation reading)."""
    y = _all_bf16_nonneg_finite()
    y = y[y <= 448.0]
    r = np.random.default_rng(5)
    extra = np.concatenate([r.uniform(0, 448, 200000), 2.0 ** r.uniform(-14, 8.8, 200000)]).astype(np.float32)
    y = np.concatenate([y, extra, np.float32([2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -6 - 2.0 ** -11])])
    ours = formats.round_e4m3_byte(y)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_round_e4m3_saturates():
    got = formats.round_e4m3_byte(np.array([448.0, 464.0, 470.0, 1000.0, np.inf, 0.0]))
    np.testing.assert_array_equal(got, [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x00])


def test_bf16_rounding_vs_torch():
    r = np.random.default_rng(3)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32),
                        (r.integers(0, 2 ** 32, 100000, dtype=np.uint64).astype(np.uint32)).view(np.float32)])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(formats.f32_to_bf16_bits(x), ref)


def test_pack_roundtrip_and_order():
    c = synth.random_codes(9, 4, 64)
    p = formats.pack_nibbles(c)
    assert p[0, 0] == (c[0, 0] | (c[0, 1] << 4))
    np.testing.assert_array_equal(formats.unpack_nibbles(p), c)


# ------------------------------------------------------------------ quantizer

def _bf16(vals):
    return formats.f32_to_bf16_bits(np.array(vals, dtype=np.float32))


@pytest.mark.parametrize("case", _golden("hand_worked.json")["quantize"], ids=lambda c: c["name"])
def test_quantizer_hand_worked(case):
    x = _bf16(case["x"]).reshape(1, -1)
    codes, scales, g, inv_g = quantize.quantize(x)
    assert list(scales[0]) == case["scales"]
    assert list(codes[0]) == case["codes_packed"]
    if "g_bits" in case:
        assert int(np.float32(g).view(np.uint32)) == int(case["g_bits"], 16)


def test_quantizer_g_values():
    _, _, g, inv_g = quantize.quantize(_bf16([6.0] + [0.0] * 15).reshape(1, -1))
    assert g == np.float32(448.0) and inv_g == np.float32(1.0 / 448.0)
    _, s, g, _ = quantize.quantize(np.zeros((2, 32), dtype=np.uint16))
    assert g == 1.0 and not s.any()


def test_quantizer_invariants_on_normal_data():
    x = synth.normal_bf16(11, 64, 512)
    codes, scales, g, inv_g = quantize.quantize(x)
    xf = formats.bf16_bits_to_f32(x).astype(np.float64)
    blocks = np.abs(xf).reshape(64, 32, 16).max(axis=2)
    # the block holding the tensor amax gets 448; none exceeds 448
    i = np.unravel_index(np.argmax(blocks), blocks.shape)
    assert scales[i] == 0x7E and scales.max() <= 0x7E
    # per element, |v - decoded code| is at most half the E2M1 grid step at v (unsaturated)
    s = formats.decode_e4m3(scales)
    c = formats.decode_e2m1(formats.unpack_nibbles(codes)).reshape(64, 32, 16)
    r = (np.float32(g) / s.astype(np.float32)).astype(np.float32)
    v = (xf.reshape(64, 32, 16).astype(np.float32) * r[:, :, None].astype(np.float32)).astype(np.float64)
    step = np.where(np.abs(v) < 2, 0.5, np.where(np.abs(v) < 4, 1.0, 2.0))
    unsat = np.abs(v) <= 6.0
    assert np.all(np.abs(v - c)[unsat] <= step[unsat] / 2)
    assert np.all(np.sign(c[c != 0]) == np.sign(v[c != 0]))
    # dequantized values track x: |x - c*s/g| <= (half step) * s/g
    deq = c * s[:, :, None] / float(g)
    assert np.all(np.abs(xf.reshape(64, 32, 16) - deq)[unsat] <= (step * s[:, :, None] / float(g))[unsat] * 0.5 * (1 + 1e-6))


def test_quantizer_zero_blocks_and_sign_of_zero():
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 1.0
    x[0, 1] = -1e-6
    bits = formats.f32_to_bf16_bits(x)
    codes, scales, _, _ = quantize.quantize(bits)
    # -1e-6 rounds to magnitude 0 but keeps its sign bit: code 0x8
    assert codes[0, 0] == (0x7 | (0x8 << 4))
    assert scales[0, 1] == 0 and not codes[0, 8:].any()


# ------------------------------------------------------------------ GEMM

def _encode_case(c):
    return (np.array(c["a_packed"], np.uint8)[None], np.array(c["a_scales"], np.uint8)[None],
            np.array(c["b_packed"], np.uint8)[None], np.array(c["b_scales"], np.uint8)[None])


@pytest.mark.parametrize("case", _golden("hand_worked.json")["gemm"], ids=lambda c: c["name"])
def test_gemm_hand_worked(case):
    a, sa, b, sb = _encode_case(case)
    D, _ = gemm.w4a4_exact(a, sa, b, sb, case["alpha"])
    assert D[0, 0] == case["D"]
    assert gemm.w4a4_float64(a, sa, b, sb, case["alpha"])[0, 0] == case["D"]


def _fraction_gemm(a_codes, a_scales, b_codes, b_scales, alpha):
    """Brute force in exact rationals, element by element."""
    def val(c):
        c = int(c)
        s = -1 if c & 8 else 1
        e, m = (c >> 1) & 3, c & 1
        mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
        return s * mag

    def sc(b):
        b = int(b)
        s = -1 if b & 0x80 else 1
        e, m = (b >> 3) & 15, b & 7
        mag = Fraction(m, 512) if e == 0 else Fraction(2) ** (e - 7) * (1 + Fraction(m, 8))
        return s * mag
    A = formats.unpack_nibbles(a_codes)
    B = formats.unpack_nibbles(b_codes)
    M, K = A.shape
    N = B.shape[0]
    out = np.empty((M, N), dtype=object)
    for i in range(M):
        for j in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += val(A[i, k]) * sc(a_scales[i, k // 16]) * val(B[j, k]) * sc(b_scales[j, k // 16])
            out[i, j] = Fraction(float(np.float32(alpha))) * acc
    return out


@pytest.mark.parametrize("K", [16, 32, 64])
def test_gemm_exact_vs_fractions(K):
    r = np.random.default_rng(K)
    M, N = 3, 4
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    a = formats.pack_nibbles(r.integers(0, 16, (M, K)))
    b = formats.pack_nibbles(r.integers(0, 16, (N, K)))
    sa = r.choice(finite, (M, K // 16)).astype(np.uint8)
    sb = r.choice(finite, (N, K // 16)).astype(np.uint8)
    alpha = 0.7
    D, _ = gemm.w4a4_exact(a, sa, b, sb, alpha)
    F = _fraction_gemm(a, sa, b, sb, alpha)
    for i in range(M):
        for j in range(N):
            assert D[i, j] == float(F[i, j])


def test_gemm_all_scale_bytes_exact():
    """Every finite scale byte and every code appears; exact vs rational brute force."""
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)   # 254 bytes
    K = 16 * 64
    sa = np.resize(finite, (2, K // 16)).astype(np.uint8)
    sb = np.resize(finite[::-1], (2, K // 16)).astype(np.uint8)
    codes = np.resize(np.arange(16, dtype=np.uint8), (2, K))
    a = formats.pack_nibbles(codes)
    b = formats.pack_nibbles(np.roll(codes, 3, axis=1))
    D, _ = gemm.w4a4_exact(a, sa, b, sb, 1.0)
    F = _fraction_gemm(a, sa, b, sb, 1.0)
    for i in range(2):
        for j in range(2):
            assert D[i, j] == float(F[i, j])


def test_gemm_exact_matches_float64_random():
    c = synth.small_random_case(64, 48, 256, seed=2)
    a = formats.pack_nibbles(c["a_codes"])
    b = formats.pack_nibbles(c["b_codes"])
    sa = formats.round_e4m3_byte(c["a_scale_targets"])
    sb = formats.round_e4m3_byte(c["b_scale_targets"])
    D, sum_abs = gemm.w4a4_exact(a, sa, b, sb, 0.5)
    D2 = gemm.w4a4_float64(a, sa, b, sb, 0.5)
    assert np.all(np.abs(D - D2) <= 1e-12 * sum_abs)


def test_gemm_sign_flip_identity_and_scale_doubling():
    r = np.random.default_rng(7)
    M, N, K = 32, 32, 64
    a = formats.pack_nibbles(r.integers(0, 16, (M, K)))
    b = formats.pack_nibbles(r.integers(0, 16, (N, K)))
    sa = formats.round_e4m3_byte(2.0 ** r.uniform(-3, 3, (M, K // 16)))
    sb = formats.round_e4m3_byte(2.0 ** r.uniform(-3, 3, (N, K // 16)))
    D, _ = gemm.w4a4_exact(a, sa, b, sb, 1.0)
    # xor 0x88 on every A byte flips every sign: D negates exactly
    Dn, _ = gemm.w4a4_exact(a ^ 0x88, sa, b, sb, 1.0)
    np.testing.assert_array_equal(Dn, -D)
    # scale byte + 8 (exponent + 1) doubles that block's contribution
    sa2 = sa.copy()
    sa2[:, 1] += 8
    Da, _ = gemm.w4a4_exact(a, sa, b, sb, 1.0)
    keep = sa.copy()
    keep[:, 1] = 0
    D0, _ = gemm.w4a4_exact(a, keep, b, sb, 1.0)
    D2, _ = gemm.w4a4_exact(a, sa2, b, sb, 1.0)
    np.testing.assert_array_equal(D2 - D0, 2 * (Da - D0))
    # identity A (1.0 on the diagonal, scale 1.0): D[m, n] = B~[n, m]
    eye = np.zeros((K, K), dtype=np.uint8)
    eye[np.arange(K), np.arange(K)] = 0x2
    ones = np.full((K, K // 16), 0x38, dtype=np.uint8)
    Di, _ = gemm.w4a4_exact(formats.pack_nibbles(eye), ones, b, sb, 1.0)
    np.testing.assert_array_equal(Di, gemm.decode_nvfp4(b, sb).T)


def test_gemm_nan_scale_propagates():
    a = np.full((2, 8), 0x22, np.uint8)
    b = np.full((3, 8), 0x22, np.uint8)
    sa = np.array([[0x38], [0x7F]], np.uint8)
    sb = np.array([[0x38], [0x38], [0xFF]], np.uint8)
    D, _ = gemm.w4a4_exact(a, sa, b, sb, 1.0)
    assert D[0, 0] == 16 and D[0, 1] == 16
    assert np.isnan(D[1]).all() and np.isnan(D[:, 2]).all()


def test_w4a16_one_hot_and_ones():
    r = np.random.default_rng(4)
    N, K = 32, 64
    w = formats.pack_nibbles(r.integers(0, 16, (N, K)))
    sw = formats.round_e4m3_byte(2.0 ** r.uniform(-3, 3, (N, K // 16)))
    Wd = gemm.decode_nvfp4(w, sw)
    x = np.zeros((2, K), np.float32)
    x[0, 5] = 1.0
    x[1, :] = 1.0
    y, _ = gemm.w4a16(formats.f32_to_bf16_bits(x), w, sw, 0.25)
    np.testing.assert_array_equal(y[0], 0.25 * Wd[:, 5])
    np.testing.assert_allclose(y[1], 0.25 * Wd.sum(axis=1), rtol=1e-15)


@pytest.mark.parametrize("case", _golden("hand_worked.json")["alpha"], ids=lambda c: c["name"])
def test_alpha_product_hand_worked(case):
    """alpha_eff = host alpha times the device scalar, one FP32 rounding (Colfax article,
    "Version 3": alpha is an FP32 scale of the accumulator); values worked out by hand."""
    a = gemm.alpha_product(case["alpha_host"], case["alpha_dev"])
    assert isinstance(a, np.float32)
    assert int(a.view(np.uint32)) == int(case["alpha_eff_bits"], 16)


def test_column_alpha_is_fp32_per_column():
    c = gemm.column_alpha(np.float32(1.0 / 3.0), [3.0, 0.1, -2.0, 0.0])
    third = np.float32(1.0 / 3.0)
    assert c.dtype == np.float32 and c.shape == (4,)
    assert c[0] == np.float32(third * np.float32(3.0)) and c[0] == 1.0        # 0x3EAAAAAB * 3 rounds to 1
    assert c[1] == np.float32(third * np.float32(0.1))
    assert c[2] == -2 * third and c[3] == 0.0


def test_per_column_alpha_w4a16_one_hot_zero_negative_scales():
    """A global or a per-column weight scale (TileLang PR #3290, "Summary"; its tests pair the
    per-column one with zero and negative block scales). A one-hot x = e_k reads out column
    by column y[n] = alpha[n] * W~[n, k]; M != N, so a scale applied along rows fails."""
    r = np.random.default_rng(41)
    N, K = 64, 128
    w = formats.pack_nibbles(r.integers(0, 16, (N, K)))
    sw = r.integers(0, 0x7F, (N, K // 16)).astype(np.uint8)       # E4M3 bytes below NaN, zero included
    sw[::3] |= 0x80                                                 # negative scales
    sw[1, :] = 0
    al = gemm.column_alpha(0.75, 2.0 ** r.integers(-4, 5, N) * r.choice([-1.0, 1.0], N))
    Wd = gemm.decode_nvfp4(w, sw)
    x = np.zeros((3, K), np.float32)
    x[0, 7] = 1.0
    x[1, 100] = 1.0
    x[2, :] = 1.0
    y, S = gemm.w4a16(formats.f32_to_bf16_bits(x), w, sw, al)
    np.testing.assert_array_equal(y[0], al.astype(np.float64) * Wd[:, 7])
    np.testing.assert_array_equal(y[1], al.astype(np.float64) * Wd[:, 100])
    assert not y[:, 1].any() and (Wd < 0).any()
    np.testing.assert_allclose(y[2], al.astype(np.float64) * Wd.sum(axis=1), rtol=1e-14)
    np.testing.assert_array_equal(S[0], np.abs(al.astype(np.float64) * Wd[:, 7]))


def test_per_column_alpha_w4a4_reduces_to_scalar_per_column():
    """Column n of the per-column result is the scalar-alpha result of that column alone
    (alpha[n]), and a vector of equal entries gives the scalar result bit for bit."""
    r = np.random.default_rng(53)
    a = formats.pack_nibbles(r.integers(0, 16, (48, 256)))
    sa = formats.round_e4m3_byte(2.0 ** r.uniform(-4, 4, (48, 16)))
    b = formats.pack_nibbles(r.integers(0, 16, (64, 256)))
    sb = formats.round_e4m3_byte(2.0 ** r.uniform(-4, 4, (64, 16)))
    al = gemm.column_alpha(0.37, r.uniform(-3, 3, 64))
    D, S = gemm.w4a4_exact(a, sa, b, sb, al)
    for n in (0, 5, 47, 48, 63):
        Dn, Sn = gemm.w4a4_exact(a, sa, b[n:n + 1], sb[n:n + 1], al[n])
        np.testing.assert_array_equal(D[:, n], Dn[:, 0])
        np.testing.assert_array_equal(S[:, n], Sn[:, 0])
    D1, _ = gemm.w4a4_exact(a, sa, b, sb, 0.37)
    Dv, _ = gemm.w4a4_exact(a, sa, b, sb, np.full(64, 0.37, np.float32))
    np.testing.assert_array_equal(D1, Dv)
    np.testing.assert_allclose(gemm.w4a4_float64(a, sa, b, sb, al), D, rtol=1e-12, atol=1e-30)


# ------------------------------------------------------------------ prepared layout

def test_prepared_size_matches_page_formula():
    fig = _golden("pages_figures.json")["prepared_weight_size"]
    for N, K in [(32, 64), (6144, 5120), (34816, 5120), (5120, 17408)]:
        assert prepared.prepared_bytes(N, K) == eval(fig["formula"], {}, {"N": N, "K": K})


def test_prepared_hand_checked_tile():
    """code(n, k) = (n + k) mod 16, N = 32, K = 128: two tiles, bytes checked by hand."""
    N, K = 32, 128
    n = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    codes = formats.pack_nibbles((n + k) % 16)
    scales = np.full((N, K // 16), 0x38, np.uint8)
    scales[3, 5] = 0x40
    prep, bad = prepared.prepare_weight(codes, scales)
    assert bad == 0 and prep.size == N * K // 2 + N * K // 16
    assert prep[0] == 0x10            # unit 0 = row 0, k 0,1 -> codes 0,1
    assert prep[16] == 0x21           # unit 1 = row 1, k 0,1 -> codes 1,2
    assert prep[16 * 15] == 0x0F      # unit 15 = row 15, k 0,1 -> codes 15,0
    assert prep[16 * 37 + 4] == 0xED  # unit 32 + 5 = row 5, k 32+8, 32+9 -> codes 13, 14
    assert prep[1024] == 0x10         # tile 1 (k 64..127), row 0, k 64,65 -> codes 0,1
    assert prep[1024 + 16 * 2 + 3] == ((2 + 64 + 6) % 16) | (((2 + 64 + 7) % 16) << 4)
    # scale (3, 5): tile 1 (blocks 4..7), row 3, block 1 -> 2048 + 128 + 4*3 + 1
    assert prep[2048 + 128 + 13] == 0x40
    off, nib, soff = prepared.prepared_offsets(3, 64 + 16 + 5, N, K)
    assert (off, nib, soff) == (1024 + 16 * 3 + 10, 1, 2048 + 128 + 13)
    off, nib, _ = prepared.prepared_offsets(5, 40, N, K)
    assert (off, nib) == (16 * 37 + 4, 0)


def test_prepared_bijection_and_folding():
    r = np.random.default_rng(8)
    N, K = 64, 192
    codes = formats.pack_nibbles(r.integers(0, 16, (N, K)))
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    scales = r.choice(finite, (N, K // 16)).astype(np.uint8)
    scales[0, 0] = 0x80   # -0
    scales[1, 1] = 0x00
    prep, bad = prepared.prepare_weight(codes, scales, "e4m3")
    assert bad == 0
    c2, s2 = prepared.unprepare(prep, N, K)
    # folded scales are magnitudes; decoded values are unchanged by the folding
    assert s2.max() <= 0x7E and not (s2 & 0x80).any()
    np.testing.assert_array_equal(gemm.decode_nvfp4(c2, s2), gemm.decode_nvfp4(codes, scales))
    assert not c2[0, :8].any() and not c2[1, 8:16].any()
    # the map is a permutation of the folded bytes
    fc, fs, _ = prepared.fold_scales(codes, scales, "e4m3")
    np.testing.assert_array_equal(c2, fc)
    np.testing.assert_array_equal(s2, fs)


def test_prepared_counts_bad_scales():
    codes = np.zeros((32, 32), np.uint8)
    s = np.full((32, 4), 0x38, np.uint8)
    s[0, 0] = 0x7F
    s[1, 1] = 0xFF
    _, bad = prepared.prepare_weight(codes, s, "e4m3")
    assert bad == 2
    s[2, 2] = 0xB8          # negative: valid E4M3, invalid UE4M3
    _, bad_u = prepared.prepare_weight(codes, s, "ue4m3")
    assert bad_u == 3


# ------------------------------------------------------------------ page figures

def test_input_footprint_formula():
    fig = _golden("pages_figures.json")["input_footprint_MB"]
    for S, mb in zip(fig["sizes"], fig["MB"]):
        assert 2 * (S * S // 2 + S * S // 16) / 2 ** 20 == mb


def test_weight_bandwidth_formula():
    fig = _golden("pages_figures.json")["weight_bandwidth"]
    for c in fig["cells"]:
        bw = prepared.prepared_bytes(c["N"], c["K"]) / (c["us"] * 1e-6) / 1e12
        assert abs(bw - c["TBps"]) < 0.01


# ------------------------------------------------------------------ two-pass prefill

def test_two_pass_on_grid_input_has_zero_residual():
    """Values on the E2M1 grid with block maximum 6 and tensor maximum 6: g = 448, every block
    scale is 448 (0x7E), the first pass is exact, so the residual pass is all zero."""
    r = np.random.default_rng(61)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    x = grid[r.integers(0, 8, (4, 64))] * r.choice([-1.0, 1.0], (4, 64))
    x[:, ::16] = 6.0
    c1, s1, c2, s2, g, _ = quantize.two_pass(formats.f32_to_bf16_bits(x.astype(np.float32)))
    assert g == np.float32(448.0) and np.all(s1 == 0x7E)
    np.testing.assert_array_equal(quantize.dequantize_with_g(c1, s1, g), x.astype(np.float32))
    assert not c2.any() and not s2.any()


def test_two_pass_reconstruction_bound_and_gain():
    """|x - deq1 - deq2| is at most the second pass's half grid step: (amax of the block's
    residual) / 6 times the E4M3 rounding slack, plus the FP32 rounding of the residual; over
    normal data the two passes cut the RMS error about tenfold."""
    x = synth.normal_bf16(62, 32, 512)
    c1, s1, c2, s2, g, _ = quantize.two_pass(x)
    xf = formats.bf16_bits_to_f32(x).astype(np.float64)
    d1 = quantize.dequantize_with_g(c1, s1, g).astype(np.float64)
    d2 = quantize.dequantize_with_g(c2, s2, g).astype(np.float64)
    res = (xf - d1).reshape(32, 32, 16)
    amax_r = np.abs(res).max(axis=2, keepdims=True)
    err = np.abs(xf - d1 - d2).reshape(32, 32, 16)
    assert np.all(err <= amax_r / 6 * (1 + 2.0 ** -3) + 2.0 ** -23 * np.abs(xf).reshape(32, 32, 16))
    e1 = np.sqrt(np.mean((xf - d1) ** 2))
    e2 = np.sqrt(np.mean((xf - d1 - d2) ** 2))
    assert e2 < e1 / 6


def test_dequantize_with_g_hand_values():
    # code 0x7 (6) and 0x9 (-0.5) under scale 0x38 (1.0) and g = 448: fl32(6 / 448), fl32(-0.5 / 448)
    d = quantize.dequantize_with_g(np.array([[0x97] + [0] * 7], np.uint8), np.array([[0x38]], np.uint8), 448.0)
    assert d[0, 0] == np.float32(np.float32(6.0) / np.float32(448.0))
    assert d[0, 1] == np.float32(np.float32(-0.5) / np.float32(448.0)) and not d[0, 2:].any()


def test_two_pass_gemm_is_the_sum_of_both_contractions():
    """D = alpha (A1 + A2) W~^T: the exact 2K contraction equals, to float64 rounding, the sum of
    the two float64 products decoded separately (an independent evaluation route)."""
    x = synth.normal_bf16(63, 24, 256)
    c1, s1, c2, s2, g, ig = quantize.two_pass(x)
    r = np.random.default_rng(64)
    w = formats.pack_nibbles(r.integers(0, 16, (40, 256)))
    sw = formats.round_e4m3_byte(2.0 ** r.uniform(-3, 3, (40, 16)))
    D, S = gemm.w4a4_two_pass_exact(c1, s1, c2, s2, w, sw, 0.5)
    ref = gemm.w4a4_float64(c1, s1, w, sw, 0.5) + gemm.w4a4_float64(c2, s2, w, sw, 0.5)
    np.testing.assert_allclose(D, ref, rtol=1e-12, atol=1e-300)
    one, _ = gemm.w4a4_exact(c1, s1, w, sw, 0.5)
    exact = (formats.bf16_bits_to_f32(x).astype(np.float64) * float(g)) @ gemm.decode_nvfp4(w, sw).T * 0.5
    assert np.linalg.norm(D - exact) < np.linalg.norm(one - exact) / 6
