"""Element formats of NVFP4: E2M1 codes, E4M3 / UE4M3 scale bytes, nibble packing, BF16.

Test infrastructure (see the package docstring). Plain numpy, written from the
definitions, not from any kernel.

Readings (the pages name the formats but print no bit layouts):

* E2M1 (4 bits, sign|e1 e0|m, exponent bias 1): e == 0 gives 0.5*m, otherwise
  2**(e-1) * (1 + m/2). The 8 magnitudes are {0, .5, 1, 1.5, 2, 3, 4, 6}; codes
  8..15 are the negatives, code 8 is -0. TileLang PR #3290, "Design: Weight
  layout", states that E2M1 codes placed in the BF16 subnormal range read as
  fp4 * 2**-126, which holds exactly for this encoding (pinned in the tests).
* E4M3 "fn" (sign|eeee|mmm, bias 7, no infinities, 0x7F/0xFF are NaN, max 448)
  as torch.float8_e4m3fn; UE4M3 is the same byte with the sign bit required to
  be 0 (TileLang PR #3290, "Changes": scales are float8_e4m3fn or UE4M3 bytes).
* Packing (Colfax article, "Version 2": 4 bits per element, two per byte along
  K): byte j of a row holds element 2j in bits 0..3 and element 2j+1 in bits
  4..7.
"""
import numpy as np

E2M1_MAX = 6.0
E4M3_MAX = 448.0


def e2m1_value(code):
    """Value of one 4-bit E2M1 code, from the closed form (sign, 2-bit exponent with bias 1, 1-bit mantissa)."""
    code = int(code)
    sign = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if sign else mag


# The 16-entry decode table, built from the closed form above.
E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E2M1_MAGNITUDES = E2M1_TABLE[:8].copy()


def e4m3_value(byte):
    """Value of one E4M3 ("fn") byte: bias 7, subnormals m*2**-9, 0x7F/0xFF NaN, no infinity."""
    byte = int(byte)
    sign = (byte >> 7) & 1
    e = (byte >> 3) & 15
    m = byte & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        mag = m * 2.0 ** -9
    else:
        mag = 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -mag if sign else mag


E4M3_TABLE = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)


def decode_e2m1(codes):
    """Unpacked codes (any integer array with values 0..15) -> float64 values."""
    return E2M1_TABLE[np.asarray(codes, dtype=np.int64)]


def decode_e4m3(scale_bytes):
    """E4M3 bytes -> float64 values (NaN for 0x7F / 0xFF)."""
    return E4M3_TABLE[np.asarray(scale_bytes, dtype=np.int64)]


def decode_ue4m3(scale_bytes):
    """UE4M3 bytes -> float64. A byte with bit 7 set is not a UE4M3 value and decodes as NaN."""
    b = np.asarray(scale_bytes, dtype=np.int64)
    v = E4M3_TABLE[b & 0x7F]
    return np.where(b & 0x80, np.nan, v)


def pack_nibbles(codes):
    """[rows][K] codes 0..15 -> [rows][K/2] bytes, element 2j in the low nibble of byte j."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """Inverse of pack_nibbles."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def round_e2m1_magnitude(y):
    """Nearest E2M1 magnitude code (0..7) of y >= 0, ties to the even code, saturating at 6.

    Within each binade of the E2M1 grid the spacing is a power of two (0.5 below
    2, 1 below 4, 2 above), so y/ulp is exact and np.rint (round half to even)
    rounds correctly; a tie on a binade edge lands on the even code (1.75 -> 2,
    3.5 -> 4, 5 -> 4, 0.25 -> 0). NaN gives code 0 (a stated rule; it arises only
    from 0 * inf in the degenerate-global-scale case of the quantizer).
    """
    y = np.asarray(y, dtype=np.float64)
    ulp = np.where(y < 2.0, 0.5, np.where(y < 4.0, 1.0, 2.0))
    with np.errstate(invalid="ignore"):
        q = np.rint(y / ulp) * ulp
    q = np.minimum(q, E2M1_MAX)
    q = np.where(np.isnan(y), 0.0, q)
    # value -> code via the decode table (magnitudes are distinct)
    code = np.zeros(q.shape, dtype=np.uint8)
    for c in range(8):
        code[q == E2M1_MAGNITUDES[c]] = c
    return code


def round_e4m3_byte(u):
    """Nearest E4M3 byte of u >= 0 (RNE, saturating to 448 = 0x7E; never NaN).

    The grid spacing in binade 2**e is 2**(e-3) for normal values and 2**-9 in
    the subnormal range (e < -6); dividing by that power of two is exact, so
    np.rint gives round-half-to-even on the grid. Values at or above the largest
    finite value saturate to 448 (464, the midpoint to the NaN slot, included).
    """
    u = np.asarray(u, dtype=np.float64)
    mant, ex = np.frexp(u)          # u = mant * 2**ex, mant in [0.5, 1)
    e = np.maximum(ex - 1, -6)      # floor(log2 u), clamped at the subnormal binade
    ulp = np.ldexp(1.0, e - 3)
    with np.errstate(invalid="ignore", over="ignore"):
        q = np.rint(u / ulp) * ulp
    q = np.where(u >= E4M3_MAX, E4M3_MAX, q)
    q = np.minimum(q, E4M3_MAX)
    q = np.where(u == 0.0, 0.0, q)
    # exact value -> byte
    byte = np.zeros(q.shape, dtype=np.uint8)
    sub = q < 2.0 ** -6
    byte[sub] = np.rint(q[sub] * 512.0).astype(np.uint8)
    qn = q[~sub]
    if qn.size:
        _, exn = np.frexp(qn)
        en = exn - 1
        m = np.rint(qn / np.ldexp(1.0, en) * 8.0 - 8.0).astype(np.int64)
        byte[~sub] = (((en + 7) << 3) | m).astype(np.uint8)
    return byte


def bf16_bits_to_f32(bits):
    """BF16 bit patterns (uint16) -> float32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def f32_to_bf16_bits(x):
    """float32 -> BF16 bits with round-to-nearest-even (NaN -> quiet NaN 0x7FC0)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    r[nan] = 0x7FC0
    return r
