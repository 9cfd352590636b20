"""Seeded synthetic inputs for the NVFP4 GEMM workloads.

This module holds no NVFP4 arithmetic: it draws raw random numbers (code
indices, scale targets, normal activations) and rounds float32 to BF16 with
torch's own conversion. Quantization, packing and decoding live in the oracle
(for checks) and in the HIP library (for the product path); both start from
what this module returns. Every generator takes an explicit seed (numpy PCG64).

Workloads (sizes and distributions as the NVFP4 GEMM pages use them):

* "random codes" (small W4A4 case): uniformly random 4-bit codes (all 16,
  including -0) and one scale per 16 K-elements drawn log-uniform in
  [2**-4, 2**4] (rounded to E4M3 by the consumer).
* "normal" square W4A4: A and B ~ N(0, 1) in BF16, quantized by the consumer.
* "large" square W4A4: as "normal", then 1% of the rows are scaled by 8
  (outlier rows) and each 16-block is zeroed with probability 0.01.
* W4A16 decode: W ~ N(0, 0.02) [N, K] in BF16 (quantized by the consumer),
  x ~ N(0, 1) [M, K] in BF16, over the linear layers of a 27B-class model.
* prefill W4A4: x ~ N(0, 1) [8192, 5120] with 0.5% of the columns (26) scaled
  by 20, W ~ N(0, 0.02) [17408, 5120].
"""
import numpy as np

# (N, K) of the 27B-class linear layers: QKV, O, fused gate+up, down.
DECODE_SHAPES = [(6144, 5120), (5120, 5120), (34816, 5120), (5120, 17408)]
DECODE_MS = [1, 8, 32, 128, 1024]
PREFILL_X = (8192, 5120)
PREFILL_W = (17408, 5120)


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x):
    """float32 -> BF16 bit patterns (uint16) using torch's round-to-nearest-even cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def random_codes(seed, rows, K):
    """Unpacked 4-bit code indices, uniform over all 16 codes: uint8 [rows][K]."""
    return rng(seed).integers(0, 16, size=(rows, K), dtype=np.uint8)


def loguniform_scale_targets(seed, rows, nblocks, lo=-4.0, hi=4.0):
    """Scale targets 2**U, U ~ uniform(lo, hi): float32 [rows][nblocks] (not yet E4M3)."""
    return (2.0 ** rng(seed).uniform(lo, hi, size=(rows, nblocks))).astype(np.float32)


def normal_bf16(seed, rows, K, std=1.0, chunk_rows=1024):
    """N(0, std) float32 rounded to BF16: uint16 [rows][K].

    Large tensors are drawn in chunks of `chunk_rows` rows, chunk i from
    SeedSequence(seed).spawn(...)[i], so the result does not depend on memory.
    """
    if rows <= chunk_rows:
        x = rng(seed).standard_normal((rows, K), dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        return f32_to_bf16_bits(x)
    out = np.empty((rows, K), dtype=np.uint16)
    nchunks = (rows + chunk_rows - 1) // chunk_rows
    children = np.random.SeedSequence(seed).spawn(nchunks)
    for i, ss in enumerate(children):
        r0 = i * chunk_rows
        r1 = min(rows, r0 + chunk_rows)
        x = np.random.Generator(np.random.PCG64(ss)).standard_normal((r1 - r0, K), dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[r0:r1] = f32_to_bf16_bits(x)
    return out


# ---------------------------------------------------------------- workloads

def small_random_case(M=256, N=256, K=256, seed=0):
    """Random-code W4A4 case: codes and scale targets for A and B."""
    return dict(
        a_codes=random_codes(seed * 4 + 1, M, K),
        a_scale_targets=loguniform_scale_targets(seed * 4 + 2, M, K // 16),
        b_codes=random_codes(seed * 4 + 3, N, K),
        b_scale_targets=loguniform_scale_targets(seed * 4 + 4, N, K // 16),
    )


def square_normal(S, operand):
    """BF16 N(0,1) [S][S] for operand 'A' or 'B' of the normal square sweep."""
    base = 100 if operand == "A" else 200
    return normal_bf16(base + int(np.log2(S)), S, S)


def square_large(S, operand):
    """BF16 [S][S] of the large square case: N(0,1), 1% rows x8, 1% of 16-blocks zeroed.

    Returns (bits, outlier_rows, zero_block_mask).
    """
    base = 300 if operand == "A" else 400
    seed = base + int(np.log2(S))
    bits = normal_bf16(seed, S, S)
    r = rng(seed + 7919)
    n_out = int(np.ceil(0.01 * S))
    outlier_rows = np.sort(r.choice(S, n_out, replace=False))
    # x8 is exact in BF16 (a power of two); done in float32 and cast back
    sub = (bits[outlier_rows].astype(np.uint32) << 16).view(np.float32) * np.float32(8.0)
    bits[outlier_rows] = f32_to_bf16_bits(sub)
    zero_mask = r.random((S, S // 16)) < 0.01
    bits.reshape(S, S // 16, 16)[zero_mask] = 0
    return bits, outlier_rows, zero_mask


def decode_weight(j):
    """BF16 W ~ N(0, 0.02) for decode shape j: uint16 [N][K]."""
    N, K = DECODE_SHAPES[j]
    return normal_bf16(500 + j, N, K, std=0.02)


def decode_activation(M, j, i):
    """BF16 x ~ N(0, 1) [M][K] for decode shape j, M index i."""
    K = DECODE_SHAPES[j][1]
    return normal_bf16(600 + 10 * j + i, M, K)


def prefill_activation():
    """BF16 [8192][5120]: N(0,1) with 26 columns (0.5%, rounded) scaled by 20 in float32."""
    M, K = PREFILL_X
    x = rng(700).standard_normal((M, K), dtype=np.float32)
    cols = np.sort(rng(7001).choice(K, 26, replace=False))
    x[:, cols] *= np.float32(20.0)
    return f32_to_bf16_bits(x), cols


def prefill_weight():
    N, K = PREFILL_W
    return normal_bf16(701, N, K, std=0.02)
