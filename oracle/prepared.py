"""Byte map of the prepared weight (the library's W layout), with scale sign and zero folding.

Test infrastructure (see the package docstring).

Folding (TileLang PR #3290, "Design: Weight layout"): a block whose scale is
zero gets all-zero codes, a block whose scale is negative gets its code signs
flipped (code ^ 0x8) and the magnitude of the scale; the prepared copy has the
same size as the checkpoint tensors, N*K/2 + N*K/16 bytes.

Layout (this library's own design, written here as a plain index map). The
weight W [N][K] is cut into tiles of 32 rows (n) x 64 columns (k); tiles are
numbered t = (n // 32) * (K // 64) + (k // 64). The first N*K/2 bytes are the
code tiles, 1024 bytes each, as 64 units of 16 bytes: unit 32*h + r holds bytes
16h .. 16h+15 of row r's 32 packed bytes of the k-chunk (element 2j in the low
nibble of byte j, 2j+1 in the high), i.e. codes of k in [32h, 32h+32). So byte
j of row r sits at 16 * (32 * (j // 16) + r) + j % 16. The next N*K/16 bytes
are the scale tiles, 128 bytes each: byte 4*r + b of tile t is the (folded)
scale of row r, block b (k in [16b, 16b+16) of the chunk).

Scale-byte validity: for E4M3 input 0x7F and 0xFF are NaN; for UE4M3 input a
byte with bit 7 set is invalid, as is 0x7F. Invalid bytes are counted; their
block keeps its codes and gets scale byte 0x7F (NaN), so a GEMM over them
yields NaN rather than a silent number.
"""
import numpy as np

from . import formats

TILE_N = 32
TILE_K = 64


def fold_scales(codes_packed, scale_bytes, scale_kind="e4m3"):
    """Return (codes, scales, bad_count) after sign/zero folding (unchanged layout)."""
    codes = np.array(codes_packed, dtype=np.uint8, copy=True)
    sb = np.asarray(scale_bytes, dtype=np.uint8)
    N, K2 = codes.shape
    K = 2 * K2
    nb = K // 16
    assert sb.shape == (N, nb)
    mag = sb & 0x7F
    if scale_kind == "e4m3":
        bad = mag == 0x7F
        neg = ((sb & 0x80) != 0) & (mag != 0) & ~bad
        zero = mag == 0
    else:
        bad = ((sb & 0x80) != 0) | (sb == 0x7F)
        neg = np.zeros_like(bad)
        zero = (sb == 0)
    out_s = np.where(bad, 0x7F, np.where(zero, 0, mag)).astype(np.uint8)
    cb = codes.reshape(N, nb, 8)                 # 8 packed bytes per 16-block
    cb[neg] ^= 0x88
    cb[zero] = 0
    return cb.reshape(N, K2), out_s, int(bad.sum())


def prepare_weight(codes_packed, scale_bytes, scale_kind="e4m3"):
    """[N][K/2] packed codes + [N][K/16] scale bytes -> (prepared bytes, bad_count)."""
    codes, scales, bad = fold_scales(codes_packed, scale_bytes, scale_kind)
    N, K2 = codes.shape
    K = 2 * K2
    assert N % TILE_N == 0 and K % TILE_K == 0
    nt, kt = N // TILE_N, K // TILE_K
    out = np.empty(N * K2 + N * (K // 16), dtype=np.uint8)
    # code byte (n, j) -> tile (n//32, j//32), unit 32*((j%32)//16) + n%32, byte j%16
    c = codes.reshape(nt, TILE_N, kt, 2, 16).transpose(0, 2, 3, 1, 4)
    out[:N * K2] = c.reshape(-1)
    # scale byte (n, b) -> tile (n//32, b//4), in-tile offset 4*(n%32) + b%4
    s = scales.reshape(nt, TILE_N, kt, 4).transpose(0, 2, 1, 3)
    out[N * K2:] = s.reshape(-1)
    return out, bad


def prepared_offsets(n, k, N, K):
    """(code byte offset, nibble 0/1, scale byte offset) of element (n, k) -- the index map itself."""
    tile = (n // TILE_N) * (K // TILE_K) + (k // TILE_K)
    r = n % TILE_N
    kk = k % TILE_K
    j = kk // 2
    code_off = tile * 1024 + 16 * (32 * (j // 16) + r) + j % 16
    scale_off = N * K // 2 + tile * 128 + 4 * r + kk // 16
    return code_off, kk % 2, scale_off


def unprepare(prep, N, K):
    """Inverse map: prepared bytes -> ([N][K/2] codes, [N][K/16] scales)."""
    prep = np.asarray(prep, dtype=np.uint8)
    nt, kt = N // TILE_N, K // TILE_K
    c = prep[:N * K // 2].reshape(nt, kt, 2, TILE_N, 16).transpose(0, 3, 1, 2, 4).reshape(N, K // 2)
    s = prep[N * K // 2:].reshape(nt, kt, TILE_N, 4).transpose(0, 2, 1, 3).reshape(N, K // 16)
    return c.copy(), s.copy()


def prepared_bytes(N, K):
    return N * K // 2 + N * K // 16
