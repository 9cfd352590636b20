"""GPU parity of the HIP library against the CPU oracle, through the C ABI.

Byte outputs (prepared weights, quantized codes and scales, g) must match
bit for bit; GEMM outputs must lie inside the stated FP32 / BF16 error bound
of the exact result (tests/gpu_helpers.py). All inputs are seeded (synth.py).
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_amd as nv
import synth
from oracle import formats, gemm, prepared, quantize
from gpu_helpers import (alpha_ab, assert_close, dev, gpu_quantize_checked, host, oracle_quantize_full,
                         oracle_w4a4_exact_blocked, oracle_w4a16_blocked)

pytestmark = pytest.mark.gpu


def _progress(msg):
    """A progress line for the long tests (visible with pytest -s)."""
    print(f"[progress] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _init():
    nv.init()


def _random_nvfp4(seed, rows, K, lo=-4, hi=4):
    codes = formats.pack_nibbles(synth.random_codes(seed, rows, K))
    scales = formats.round_e4m3_byte(synth.loguniform_scale_targets(seed + 1000, rows, K // 16, lo, hi))
    return codes, scales


def _prep(codes, scales, kind="e4m3"):
    wp, bad = nv.nvfp4_prepare_weight(dev(codes), dev(scales), kind, validate=False)
    torch.cuda.synchronize()
    return wp, int(bad.item())


# ------------------------------------------------------------------ prepare

@pytest.mark.parametrize("kind", ["e4m3", "ue4m3"])
def test_prepare_bit_exact(kind):
    N, K = 96, 320
    codes, _ = _random_nvfp4(1, N, K)
    r = np.random.default_rng(2)
    scales = r.integers(0, 256, (N, K // 16), dtype=np.uint8)   # every byte: negatives, zeros, NaNs
    wp, bad = _prep(codes, scales, kind)
    ref, bad_ref = prepared.prepare_weight(codes, scales, kind)
    np.testing.assert_array_equal(wp.cpu().numpy(), ref)
    assert bad == bad_ref and bad > 0


@pytest.mark.parametrize("kind,byte", [("e4m3", 0x7F), ("e4m3", 0xFF), ("ue4m3", 0x7F), ("ue4m3", 0x80)])
def test_prepare_rejects_invalid_scale_bytes(kind, byte):
    """Invalid scale bytes are an input error (TileLang PR #3290, "Changes", input validation):
    the binding synchronises after the prepare and raises ValueError naming the count."""
    N, K = 64, 128
    codes, scales = _random_nvfp4(4, N, K)
    scales[5, 2] = byte
    scales[63, 7] = byte
    with pytest.raises(ValueError, match="^2 scale bytes"):
        nv.nvfp4_prepare_weight(dev(codes), dev(scales), kind)
    scales[5, 2] = scales[63, 7] = 0x38
    wp, bad = nv.nvfp4_prepare_weight(dev(codes), dev(scales), kind)     # valid again: no error
    assert int(bad.item()) == 0


def test_prepare_decode_shape_bit_exact():
    N, K = synth.DECODE_SHAPES[0]
    codes, scales = _random_nvfp4(3, N, K)
    wp, bad = _prep(codes, scales)
    ref, _ = prepared.prepare_weight(codes, scales)
    assert bad == 0
    np.testing.assert_array_equal(wp.cpu().numpy(), ref)


# ------------------------------------------------------------------ quantize

@pytest.mark.parametrize("rows,K", [(1, 16), (3, 32), (77, 640), (256, 5120)])
def test_quantize_bit_exact(rows, K):
    x = synth.normal_bf16(rows * 7 + K, rows, K)
    codes, scales, g, inv_g = nv.nvfp4_quantize(dev(x).view(torch.bfloat16))
    c_ref, s_ref, g_ref, ig_ref = quantize.quantize(x)
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)
    np.testing.assert_array_equal(scales.cpu().numpy(), s_ref)
    assert np.float32(g.item()) == g_ref and np.float32(inv_g.item()) == ig_ref


def test_quantize_edge_values():
    # zeros, a zero block, ties on the E2M1 grid, tiny values, both signs, sign of zero
    vals = np.zeros((4, 64), np.float32)
    vals[0, :16] = [6, .25, .75, 1.25, 1.75, 2.5, 3.5, 5, -.25, -.75, -2.5, -5, .1, 5.9, 0, -0.0]
    vals[1, 16:32] = [1, .5, .400390625, -1] + [0] * 12
    vals[2, :] = np.linspace(-1e-3, 1e-3, 64)
    vals[3, 5] = -1e-30
    x = formats.f32_to_bf16_bits(vals)
    codes, scales, g, _ = nv.nvfp4_quantize(dev(x).view(torch.bfloat16))
    c_ref, s_ref, g_ref, _ = quantize.quantize(x)
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)
    np.testing.assert_array_equal(scales.cpu().numpy(), s_ref)
    z = np.zeros((2, 32), np.uint16)
    codes, scales, g, inv_g = nv.nvfp4_quantize(dev(z).view(torch.bfloat16))
    assert g.item() == 1.0 and not codes.any() and not scales.any()


def test_quantize_all_bf16_patterns():
    """Every finite BF16 value, in blocks of widely different magnitude: the E2M1
    rounding (hardware conversion in the library) against the oracle's stated rule."""
    b = np.arange(65536, dtype=np.uint32)
    b = b[((b >> 7) & 0xFF) != 0xFF].astype(np.uint16)          # drop Inf / NaN patterns
    r = np.random.default_rng(5)
    x = r.permutation(b)
    x = x[: x.size // 64 * 64].reshape(-1, 64)
    codes, scales, g, _ = nv.nvfp4_quantize(dev(x).view(torch.bfloat16))
    c_ref, s_ref, g_ref, _ = quantize.quantize(x)
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)
    np.testing.assert_array_equal(scales.cpu().numpy(), s_ref)
    assert np.float32(g.item()) == np.float32(g_ref)
    # the same patterns scaled into one binade per row, so many blocks sit near the top of the grid
    y = x.copy()
    y &= 0x807F
    y |= np.uint16(0x3F80)
    codes, scales, g, _ = nv.nvfp4_quantize(dev(y).view(torch.bfloat16))
    c_ref, s_ref, g_ref, _ = quantize.quantize(y)
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)
    np.testing.assert_array_equal(scales.cpu().numpy(), s_ref)


@pytest.mark.parametrize("rows,K", [(77, 320), (256, 5120), (1, 64)])
def test_quantize_tiled_matches_quantize_then_tile(rows, K):
    x = synth.normal_bf16(rows * 7 + K, rows, K)
    xd = dev(x).view(torch.bfloat16)
    at, g, ig = nv.nvfp4_quantize_tiled(xd)
    codes, scales, g2, ig2 = nv.nvfp4_quantize(xd)
    ref_t = nv.nvfp4_tile_activation(codes, scales)
    torch.cuda.synchronize()
    assert torch.equal(at, ref_t)
    assert g.item() == g2.item() and ig.item() == ig2.item()
    # and against the oracle: quantizer bytes in the prepared index map, padding rows zero
    c_ref, s_ref, _, _ = quantize.quantize(x)
    Mp = -(-rows // 32) * 32
    cp = np.zeros((Mp, K // 2), np.uint8)
    sp = np.zeros((Mp, K // 16), np.uint8)
    cp[:rows], sp[:rows] = c_ref, s_ref
    ref, _ = prepared.prepare_weight(cp, sp, "ue4m3")
    assert np.array_equal(host(at), ref)


def test_quantize_prefill_activation_full():
    x, _ = synth.prefill_activation()
    codes, scales, g, inv_g = nv.nvfp4_quantize(dev(x).view(torch.bfloat16))
    c_ref, s_ref, g_ref, ig_ref = quantize.quantize(x)
    assert np.float32(g.item()) == g_ref and np.float32(inv_g.item()) == ig_ref
    np.testing.assert_array_equal(scales.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)


_ORACLE_Q = {}


def _oracle_q(rows, K, two):
    """The oracle's one- or two-pass quantization of the seeded [rows][K] activation, cached."""
    key = (rows, K, two)
    if key not in _ORACLE_Q:
        x = synth.normal_bf16(7000 + rows, rows, K)
        _ORACLE_Q[key] = (x, quantize.two_pass(x) if two else quantize.quantize(x))
    return _ORACLE_Q[key]


@pytest.mark.parametrize("extra", [0, 1])
@pytest.mark.parametrize("form", ["row_major", "tiled", "two_pass"])
def test_quantize_at_and_past_register_capacity(form, extra):
    """The quantizer reads x once when its 32 x 64 tiles fit in the registers of one resident grid
    (5 tiles per wave, 16 waves per CU: 32 rows of 5120 columns per CU) and twice otherwise. At
    exactly that capacity (extra = 0: the one-read form with every register tile in use) and one
    row past it (extra = 1: the two-read form), every byte and g against the oracle, for the
    row-major, tiled and two-pass outputs."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    K = 5120
    rows = min(cus, 1024) * 32 + extra
    x, ref = _oracle_q(rows, K, form == "two_pass")
    _progress(f"quantize {form} rows={rows} K={K}")
    xd = dev(x).view(torch.bfloat16)
    Mp = -(-rows // 32) * 32
    if form == "row_major":
        codes, scales, g, ig = nv.nvfp4_quantize(xd)
        c_ref, s_ref, g_ref, ig_ref = ref
        np.testing.assert_array_equal(host(codes), c_ref)
        np.testing.assert_array_equal(host(scales), s_ref)
    elif form == "tiled":
        at, g, ig = nv.nvfp4_quantize_tiled(xd)
        c_ref, s_ref, g_ref, ig_ref = ref
        cp = np.zeros((Mp, K // 2), np.uint8)
        sp = np.zeros((Mp, K // 16), np.uint8)
        cp[:rows], sp[:rows] = c_ref, s_ref
        lay, _ = prepared.prepare_weight(cp, sp, "ue4m3")
        np.testing.assert_array_equal(host(at), lay)
    else:
        a2, g, ig = nv.nvfp4_quantize_two_pass_tiled(xd)
        c1, s1, c2, s2, g_ref, ig_ref = ref
        cp = np.zeros((Mp, K), np.uint8)
        sp = np.zeros((Mp, K // 8), np.uint8)
        cp[:rows], sp[:rows] = np.concatenate([c1, c2], axis=1), np.concatenate([s1, s2], axis=1)
        lay, _ = prepared.prepare_weight(cp, sp, "ue4m3")
        np.testing.assert_array_equal(host(a2), lay)
    assert np.float32(g.item()) == g_ref and np.float32(ig.item()) == ig_ref


@pytest.mark.parametrize("rows,K", [(256, 5120), (77, 640), (8192, 5120), (1, 64), (33, 17408)])
@pytest.mark.parametrize("form", ["row_major", "tiled", "two_pass"])
def test_quantize_writes_stay_in_bounds(form, rows, K):
    """Every output of the quantizer sits between guard bytes (one slab, the outputs carved out of
    it with guards before and after each): the guards are unchanged after the call, and the
    outputs equal those of a call on separately allocated buffers. Shapes whose tiles split into
    unequal per-workgroup runs (256 x 5120: 640 tiles as 213 runs of 3 and one of 1)."""
    G = 4096
    x = synth.normal_bf16(rows + 3 * K, rows, K)
    xd = dev(x).view(torch.bfloat16)
    if form == "row_major":
        sizes = [rows * K // 2, rows * K // 16]
    elif form == "tiled":
        sizes = [int(nv.lib().nvfp4_tiled_activation_bytes(rows, K))]
    else:
        sizes = [int(nv.lib().nvfp4_tiled_activation_bytes(rows, 2 * K))]
    sizes += [4, 4]                                        # g, inv_g
    total = G + sum(-(-n // 256) * 256 + G for n in sizes)
    slab = torch.full((total,), 0xA5, dtype=torch.uint8, device="cuda")
    views, off = [], G
    for n in sizes:
        views.append(slab[off:off + n])
        off += -(-n // 256) * 256 + G
    g, ig = views[-2].view(torch.float32), views[-1].view(torch.float32)
    if form == "row_major":
        nv.nvfp4_quantize(xd, views[0], views[1], g, ig)
        ref = nv.nvfp4_quantize(xd)
        outs = [views[0].view(rows, K // 2), views[1].view(rows, K // 16), g, ig]
    elif form == "tiled":
        nv.nvfp4_quantize_tiled(xd, views[0], g, ig)
        ref = nv.nvfp4_quantize_tiled(xd)
        outs = [views[0], g, ig]
    else:
        nv.nvfp4_quantize_two_pass_tiled(xd, views[0], g, ig)
        ref = nv.nvfp4_quantize_two_pass_tiled(xd)
        outs = [views[0], g, ig]
    torch.cuda.synchronize()
    mask = torch.ones(total, dtype=torch.bool, device="cuda")
    off = G
    for n in sizes:
        mask[off:off + n] = False
        off += -(-n // 256) * 256 + G
    assert bool((slab[mask] == 0xA5).all()), "a quantizer write landed outside its output"
    for a, b in zip(outs, ref):
        assert torch.equal(a.reshape(-1), b.reshape(-1))


def test_quantize_repeat_calls_new_maximum():
    """Calls in a row on one workspace, each input with a different tensor maximum (larger, then
    smaller, then zero): no call may see the previous call's per-workgroup maxima."""
    ws = torch.empty(nv.workspace_bytes(nv.OP_QUANTIZE, 2048, 0, 640), dtype=torch.uint8, device="cuda")
    for i, scale in enumerate([1.0, 50.0, 0.01, 0.0]):
        x = synth.normal_bf16(300 + i, 2048, 640, std=max(scale, 1e-3))
        if scale == 0.0:
            x[:] = 0
        xd = dev(x).view(torch.bfloat16)
        at, g, ig = nv.nvfp4_quantize_tiled(xd, ws=ws)
        torch.cuda.synchronize()
        c_ref, s_ref, g_ref, ig_ref = quantize.quantize(x)
        assert np.float32(g.item()) == g_ref, f"call {i}"
        cp = c_ref.reshape(2048, 320)
        lay, _ = prepared.prepare_weight(cp, s_ref, "ue4m3")
        np.testing.assert_array_equal(host(at), lay)


@pytest.mark.parametrize("fill", ["zeros", "ones", "a5", "after_two_read", "random"])
def test_quantize_workspace_any_initial_state(fill):
    """The one-read quantizer's barrier needs no workspace initialisation: whatever the workspace
    holds (zeros as nvfp4_workspace_init leaves it, all-ones bytes, a constant byte, what the
    two-read form leaves there, random bytes), several calls in a row give the oracle's bytes,
    with the tensor maximum changing from call to call."""
    n = nv.workspace_bytes(nv.OP_QUANTIZE, 256, 0, 5120)
    if fill == "zeros":
        ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    elif fill == "ones":
        ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
    elif fill == "a5":
        ws = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")
    elif fill == "random":
        ws = torch.from_numpy(np.random.default_rng(3).integers(0, 256, n, dtype=np.uint8)).cuda()
    else:
        ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
        big = synth.normal_bf16(5, 8256, 5120)             # past the register capacity: two reads
        nv.nvfp4_quantize_tiled(dev(big).view(torch.bfloat16), ws=ws)
    for i, std in enumerate([1.0, 3.0, 0.25]):
        x = synth.normal_bf16(400 + i, 256, 5120, std=std)
        at, g, ig = nv.nvfp4_quantize_tiled(dev(x).view(torch.bfloat16), ws=ws)
        torch.cuda.synchronize()
        c_ref, s_ref, g_ref, _ = quantize.quantize(x)
        assert np.float32(g.item()) == g_ref, f"{fill}: call {i}"
        lay, _ = prepared.prepare_weight(c_ref, s_ref, "ue4m3")
        np.testing.assert_array_equal(host(at), lay)


# ------------------------------------------------------------------ W4A4

def _w4a4(a, sa, b, sb, alpha, out_dtype, alpha_dev=None):
    N, K = b.shape[0], b.shape[1] * 2
    wp, bad = _prep(b, sb)
    assert bad == 0
    ad = None if alpha_dev is None else torch.tensor([alpha_dev], dtype=torch.float32, device="cuda")
    out = nv.nvfp4_gemm_w4a4(dev(a), dev(sa), wp, N, K, alpha, ad, out_dtype)
    torch.cuda.synchronize()
    return out


def test_w4a4_random_codes_256_f32_and_repeat():
    """Random codes (all 16) with log-uniform scales, 256^3, alpha = 1, FP32 out."""
    c = synth.small_random_case(256, 256, 256, seed=0)
    a, b = formats.pack_nibbles(c["a_codes"]), formats.pack_nibbles(c["b_codes"])
    sa, sb = formats.round_e4m3_byte(c["a_scale_targets"]), formats.round_e4m3_byte(c["b_scale_targets"])
    out = _w4a4(a, sa, b, sb, 1.0, "f32")
    D, S = gemm.w4a4_exact(a, sa, b, sb, 1.0)
    assert_close(host(out), D, S, bf16=False, what="256^3 f32")
    out2 = _w4a4(a, sa, b, sb, 1.0, "f32")
    assert torch.equal(out, out2)


@pytest.mark.parametrize("M,N,K", [(1, 32, 64), (300, 320, 192), (513, 256, 128), (77, 544, 320), (256, 512, 1024)])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_w4a4_ragged_shapes(M, N, K, out_dtype):
    a, sa = _random_nvfp4(M + 11, M, K)
    b, sb = _random_nvfp4(N + 13, N, K)
    alpha = 0.37
    out = _w4a4(a, sa, b, sb, alpha, out_dtype)
    D, S = gemm.w4a4_exact(a, sa, b, sb, alpha)
    assert_close(host(out), D, S, bf16=out_dtype == "bf16", what=f"{M}x{N}x{K}")


@pytest.mark.parametrize("out_dtype,pad", [("bf16", 3), ("f32", 4)])
def test_w4a4_big_tiles_ragged_strided_out(out_dtype, pad):
    """256 x 256 workgroup tiles (17 x 17 of them) with ragged rows and columns, written into
    an output whose rows are longer than N: BF16 rows of N + 3 (not 16-byte aligned, the
    element-store path) and FP32 rows of N + 4. The padding must stay untouched; full check."""
    M, N, K = 4100, 4128, 128
    a, sa = _random_nvfp4(M + 5, M, K)
    b, sb = _random_nvfp4(N + 6, N, K)
    wp, bad = _prep(b, sb)
    assert bad == 0
    dt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    big = torch.full((M, N + pad), -7.0, dtype=dt, device="cuda")
    out = nv.nvfp4_gemm_w4a4(dev(a), dev(sa), wp, N, K, 0.81, None, out_dtype, out=big[:, :N])
    torch.cuda.synchronize()
    assert torch.all(big[:, N:] == -7.0), "columns past N were written"
    D, S = gemm.w4a4_exact(a, sa, b, sb, 0.81)
    assert_close(host(out), D, S, bf16=out_dtype == "bf16", what=f"strided {out_dtype} {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(4000, 4192, 256), (8192, 8192, 128), (300, 8704, 192)])
def test_w4a4_bf16_aligned_padded_rows_ragged(M, N, K):
    """BF16 out on 256 x 256 tiles into rows 8 elements longer than N (16-byte aligned rows, the
    16-byte store path): every element inside D against the oracle, the padding columns
    untouched. Ragged M and N (last tiles part-filled), several tiles per workgroup (8192 x 8192:
    four rounds), and fewer tiles than CUs (300 x 8704)."""
    a, sa = _random_nvfp4(M + 31, M, K)
    b, sb = _random_nvfp4(N + 37, N, K)
    wp, bad = _prep(b, sb)
    assert bad == 0
    big = torch.full((M, N + 8), -3.0, dtype=torch.bfloat16, device="cuda")
    cfg = nv.make_config(nv.KERNEL_W4A4_TILES, 256, 256)
    out = nv.nvfp4_gemm_w4a4(dev(a), dev(sa), wp, N, K, 0.59, None, "bf16", out=big[:, :N], config=cfg)
    again = nv.nvfp4_gemm_w4a4(dev(a), dev(sa), wp, N, K, 0.59, None, "bf16", config=cfg)
    torch.cuda.synchronize()
    assert torch.all(big[:, N:] == -3.0), "columns past N were written"
    assert torch.equal(out, again)
    D, S = oracle_w4a4_exact_blocked(a, sa, b, sb, 0.59)
    assert_close(host(out), D, S, bf16=True, what=f"bf16 padded rows {M}x{N}x{K}")


def test_w4a4_last_round_quadrants_same_bits():
    """16 x 17 = 272 tiles of 256 x 256 on 256 CUs: the last 16 (at most half a round) run as
    128 x 128 quadrants on two workgroups per CU. Ragged both ways: the last tile row holds 160
    rows (lower quadrants part-filled), the last tile column 96 columns (right quadrants wholly
    outside D, skipped). Every output checked against the oracle, and the same bits as the
    columns of a wider W whose 16 x 32 tiles make whole rounds (the T = 4 kernel alone)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if 272 < cus or 2 * (272 % cus) > cus or (16 * 32) % cus != 0:
        pytest.skip(f"tile counts chosen for 256 CUs, this device has {cus}")
    M, N, K, Nw = 4000, 4192, 1024, 8192
    a, sa = _random_nvfp4(71, M, K)
    b, sb = _random_nvfp4(72, Nw, K)
    wp, _ = _prep(b[:N], sb[:N])
    wpw, _ = _prep(b, sb)
    A, SA = dev(a), dev(sa)
    quads = nv.make_config(nv.KERNEL_W4A4_TILES, 256, 256, nv.TAIL_QUADRANTS)
    out = nv.nvfp4_gemm_w4a4(A, SA, wp, N, K, 0.63, None, "bf16", config=quads)
    wide = nv.nvfp4_gemm_w4a4(A, SA, wpw, Nw, K, 0.63, None, "bf16")
    torch.cuda.synchronize()
    assert torch.equal(out, wide[:, :N]), "quadrant launch must give the T = 4 kernel's bits"
    D, S = oracle_w4a4_exact_blocked(a, sa, b[:N], sb[:N], 0.63)
    assert_close(host(out), D, S, bf16=True, what=f"last-round quadrants {M}x{N}x{K}")


_W4A4_CONFIGS = {
    "none": dict(tile_m=256, tile_n=256),
    "quadrants": dict(tile_m=256, tile_n=256, tail=nv.TAIL_QUADRANTS),
    "split2": dict(tile_m=256, tile_n=256, tail=nv.TAIL_SPLIT, split_k=2),
    "split7": dict(tile_m=256, tile_n=256, tail=nv.TAIL_SPLIT, split_k=7),
    "none_dynamic": dict(tile_m=256, tile_n=256, dynamic=1),
    "split3_dynamic": dict(tile_m=256, tile_n=256, tail=nv.TAIL_SPLIT, split_k=3, dynamic=1),
    "tiles128": dict(tile_m=128, tile_n=128),
}


@pytest.fixture(scope="module")
def _w4a4_config_case():
    """4000 x 4192 x 1088: 16 x 17 = 272 tiles of 256 x 256, ragged in both directions, K = 17
    chunks (so split ranges are unequal: 8 / 9 chunks, or 2-3 of 7)."""
    M, N, K = 4000, 4192, 1088
    a, sa = _random_nvfp4(171, M, K)
    b, sb = _random_nvfp4(172, N, K)
    wp, _ = _prep(b, sb)
    ac = _alpha_col(173, N)
    D, S = oracle_w4a4_exact_blocked(a, sa, b, sb, gemm.column_alpha(0.83, ac))
    return dict(M=M, N=N, K=K, A=dev(a), SA=dev(sa), wp=wp, ac=dev(ac), D=D, S=S)


@pytest.mark.parametrize("name", list(_W4A4_CONFIGS))
def test_w4a4_explicit_configs(_w4a4_config_case, name):
    """Every schedule the W4A4 config can ask for (TileLang PR #3290, "Tests": explicit configs),
    with a per-column alpha, FP32 out: the tail as one more round, as quadrants, or split along K
    with a fixed-order fix-up (row "split-K partials + fixed-order reduce"), and the dynamic
    (atomic-counter) schedule; each within the bound of the exact result and bit-identical on
    repeat. Schedules that run every element's MFMA sequence unchanged give the bits of the
    plain one."""
    c = _w4a4_config_case
    cfg = nv.make_config(nv.KERNEL_W4A4_TILES, **_W4A4_CONFIGS[name])
    run = lambda cf: nv.nvfp4_gemm_w4a4(c["A"], c["SA"], c["wp"], c["N"], c["K"], 0.83, None, "f32",
                                         alpha_col=c["ac"], config=cf)
    out, again = run(cfg), run(cfg)
    torch.cuda.synchronize()
    assert torch.equal(out, again), "repeat calls must be bit-identical"
    if name in ("none", "quadrants", "none_dynamic"):
        plain = run(nv.make_config(nv.KERNEL_W4A4_TILES, **_W4A4_CONFIGS["none"]))
        torch.cuda.synchronize()
        assert torch.equal(out, plain)
    assert_close(host(out), c["D"], c["S"], bf16=False, what=f"w4a4 config {name}")


def test_w4a4_all_tiles_split_2048():
    """2048^3 with every one of its 64 256 x 256 tiles split into 4 K ranges (no whole tile:
    the 256 work units are all ranges) and the BF16 epilogue in the fix-up; full check."""
    S = 2048
    xa, xb = synth.square_normal(S, "A"), synth.square_normal(S, "B")
    a, sa, gA, _ = quantize.quantize(xa)
    b, sb, gB, _ = quantize.quantize(xb)
    alpha = alpha_ab(gA, gB)
    wp, _ = _prep(b, sb, "ue4m3")
    cfg = nv.make_config(nv.KERNEL_W4A4_TILES, 256, 256, nv.TAIL_SPLIT, 4)
    out = nv.nvfp4_gemm_w4a4(dev(a), dev(sa), wp, S, S, float(alpha), None, "bf16", config=cfg)
    torch.cuda.synchronize()
    D, Sabs = oracle_w4a4_exact_blocked(a, sa, b, sb, alpha)
    assert_close(host(out), D, Sabs, bf16=True, what="2048^3 all tiles split")


def test_w4a4_config_errors():
    """Invalid explicit configs return NVFP4_ERR_VALUE (ValueError) before any launch; an explicit
    K-split without a workspace returns NVFP4_ERR_WORKSPACE."""
    M, N, K = 256, 256, 128
    a, sa = _random_nvfp4(5, M, K)
    b, sb = _random_nvfp4(6, N, K)
    wp, _ = _prep(b, sb)
    A, SA = dev(a), dev(sa)
    bad = [dict(tile_m=256, tile_n=128), dict(tile_m=192, tile_n=192), dict(tile_m=128, tile_n=128, dynamic=1),
           dict(tile_m=256, tile_n=256, tail=nv.TAIL_SPLIT, split_k=1),
           dict(tile_m=256, tile_n=256, tail=nv.TAIL_SPLIT, split_k=3),           # K has 2 chunks
           dict(tile_m=256, tile_n=256, tail=7), dict(kernel=nv.KERNEL_W4A16_SKINNY, tile_m=256, tile_n=256)]
    for kw in bad:
        kw = dict(kernel=nv.KERNEL_W4A4_TILES, **kw) if "kernel" not in kw else kw
        cfg = nv.make_config(**kw)
        st = nv.lib().nvfp4_gemm_w4a4(nv._ptr(A), nv._ptr(SA), nv._ptr(wp), M, N, K, 1.0, None, None,
                                      nv._ptr(torch.empty(1, device="cuda")), nv.OUT_F32, N, ctypes.byref(cfg),
                                      nv._ptr(torch.empty(1 << 20, dtype=torch.uint8, device="cuda")), 1 << 20,
                                      None)
        assert st == nv.ERR_VALUE, kw
    at = nv.nvfp4_tile_activation(A, SA)
    split = nv.make_config(nv.KERNEL_W4A4_TILES, 256, 256, nv.TAIL_SPLIT, 2)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    st = nv.lib().nvfp4_gemm_w4a4_tiled(nv._ptr(at), nv._ptr(wp), M, N, K, 1.0, None, None, nv._ptr(out), nv.OUT_F32,
                                        N, ctypes.byref(split), None, 0, None)
    assert st == nv.ERR_WORKSPACE
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,N,K,kernel,tile", [
    (1, 320, 640, nv.KERNEL_W4A16_SKINNY, (0, 0)), (3, 320, 640, nv.KERNEL_W4A16_TILES, (128, 128)),
    (4, 4160, 2048, nv.KERNEL_W4A16_DECODE, (0, 0)), (20, 4160, 2048, nv.KERNEL_W4A16_TILES, (128, 256)),
    (64, 2080, 1024, nv.KERNEL_W4A16_TILES, (256, 256)), (100, 2080, 1024, nv.KERNEL_W4A16_TILES, (128, 128)),
    (300, 8224, 640, nv.KERNEL_W4A16_TILES, (128, 256)), (40, 8224, 640, nv.KERNEL_W4A16_SKINNY, (0, 0))])
def test_w4a16_explicit_configs(M, N, K, kernel, tile):
    """Each W4A16 kernel forced on shapes where the heuristic picks another (TileLang PR #3290,
    "Tests": explicit configs): full check against the oracle."""
    x, b, sb, wp, alpha = _w4a16_case(M, N, K, M * 3 + N + K)
    cfg = nv.make_config(kernel, tile[0], tile[1])
    out = nv.nvfp4_gemm_w4a16(dev(x).view(torch.bfloat16), wp, N, K, alpha, config=cfg)
    torch.cuda.synchronize()
    y, S = gemm.w4a16(x, b, sb, alpha)
    assert_close(host(out), y, S, bf16=True, what=f"w4a16 config {kernel} {tile} M={M}")


@pytest.mark.parametrize("M,K", [(64, 128), (77, 320), (1, 64)])
def test_tile_activation_bytes_match_oracle_layout(M, K):
    """The activation tile layout is the prepared-weight index map (no folds needed:
    positive, non-zero scales), rows past M zero."""
    a, sa = _random_nvfp4(M * 13 + K, M, K)
    at = nv.nvfp4_tile_activation(dev(a), dev(sa))
    torch.cuda.synchronize()
    Mp = -(-M // 32) * 32
    a_pad = np.zeros((Mp, K // 2), np.uint8)
    s_pad = np.zeros((Mp, K // 16), np.uint8)
    a_pad[:M], s_pad[:M] = a, sa
    ref, bad = prepared.prepare_weight(a_pad, s_pad, "e4m3")
    assert bad == 0
    assert np.array_equal(host(at), ref)


@pytest.mark.parametrize("M,N,K", [(300, 320, 192), (2048, 2048, 512)])
def test_w4a4_tiled_entry_matches_standard(M, N, K):
    a, sa = _random_nvfp4(M + N, M, K)
    b, sb = _random_nvfp4(M + N + 1, N, K)
    wp, _ = _prep(b, sb)
    std = nv.nvfp4_gemm_w4a4(dev(a), dev(sa), wp, N, K, 0.5, None, "bf16")
    at = nv.nvfp4_tile_activation(dev(a), dev(sa))
    til = nv.nvfp4_gemm_w4a4_tiled(at, M, wp, N, K, 0.5, None, "bf16")
    torch.cuda.synchronize()
    assert torch.equal(std, til)


def test_w4a4_closed_forms():
    M = N = 64
    K = 256
    ones = np.full((M, K // 2), 0x22, np.uint8)
    s1 = np.full((M, K // 16), 0x38, np.uint8)
    out = _w4a4(ones, s1, ones, s1, 1.0, "f32")
    assert (host(out) == K).all()
    # largest magnitude, exactly representable: K * 2688^2
    six = np.full((M, K // 2), 0x77, np.uint8)
    smax = np.full((M, K // 16), 0x7E, np.uint8)
    out = _w4a4(six, smax, six, smax, 1.0, "f32")
    assert (host(out) == K * 2688.0 ** 2).all()
    # identity A picks rows of B~
    eye = np.zeros((K, K), np.uint8)
    eye[np.arange(K), np.arange(K)] = 0x2
    b, sb = _random_nvfp4(5, N, K)
    out = _w4a4(formats.pack_nibbles(eye), np.full((K, K // 16), 0x38, np.uint8), b, sb, 1.0, "f32")
    np.testing.assert_array_equal(host(out), gemm.decode_nvfp4(b, sb).T)
    # alpha from a device scalar multiplies in FP32
    out = _w4a4(ones, s1, ones, s1, 0.5, "f32", alpha_dev=0.25)
    assert (host(out) == K * 0.125).all()


def test_w4a4_nan_scale_propagates_to_its_row():
    M, N, K = 64, 64, 128
    a, sa = _random_nvfp4(21, M, K)
    b, sb = _random_nvfp4(22, N, K)
    sa[7, 3] = 0x7F
    out = host(_w4a4(a, sa, b, sb, 1.0, "f32"))
    assert np.isnan(out[7]).all() and not np.isnan(np.delete(out, 7, axis=0)).any()


def test_w4a4_normal_2048_bf16_full():
    S = 2048
    xa, xb = synth.square_normal(S, "A"), synth.square_normal(S, "B")
    a, sa, gA, _ = quantize.quantize(xa)
    b, sb, gB, _ = quantize.quantize(xb)
    alpha = alpha_ab(gA, gB)
    out = _w4a4(a, sa, b, sb, float(alpha), "bf16")
    D, Sabs = gemm.w4a4_exact(a, sa, b, sb, alpha)
    assert_close(host(out), D, Sabs, bf16=True, what="2048^3 bf16")


def test_w4a4_normal_8192_full():
    """8192^3 in the benchmark's launch configuration (A quantized into the tile layout,
    B quantized and prepared, nvfp4_gemm_w4a4_tiled into BF16), every output checked.
    The row-major quantizer's bytes are checked in full against the oracle's, and the
    row-major GEMM entry must give the same bits as the tiled one."""
    S = 8192
    xa, xb = synth.square_normal(S, "A"), synth.square_normal(S, "B")
    xad = dev(xa).view(torch.bfloat16)
    at, gA_t, _ = nv.nvfp4_quantize_tiled(xad)
    ca, sa, gA_d, _ = nv.nvfp4_quantize(xad)
    cb, sb, gB_d, _ = nv.nvfp4_quantize(dev(xb).view(torch.bfloat16))
    wp, bad = nv.nvfp4_prepare_weight(cb, sb, "ue4m3")
    a_ref, sa_ref, gA = oracle_quantize_full(xa)
    b_ref, sb_ref, gB = oracle_quantize_full(xb)
    assert np.float32(gA_t.item()) == gA and np.float32(gA_d.item()) == gA and np.float32(gB_d.item()) == gB
    np.testing.assert_array_equal(host(ca), a_ref)
    np.testing.assert_array_equal(host(sa), sa_ref)
    np.testing.assert_array_equal(host(cb), b_ref)
    np.testing.assert_array_equal(host(sb), sb_ref)
    del xad, cb, sb
    alpha = alpha_ab(gA, gB)
    out = nv.nvfp4_gemm_w4a4_tiled(at, S, wp, S, S, float(alpha), None, "bf16")
    std = nv.nvfp4_gemm_w4a4(ca, sa, wp, S, S, float(alpha), None, "bf16")
    torch.cuda.synchronize()
    assert int(bad.item()) == 0
    assert torch.equal(out, std), "tiled and row-major entries differ"
    del std, ca, sa, at, wp
    D, Sabs = oracle_w4a4_exact_blocked(a_ref, sa_ref, b_ref, sb_ref, alpha)
    assert_close(host(out), D, Sabs, bf16=True, what="8192^3 full")


def test_w4a4_normal_4096_full():
    """4096^3 (square sweep) in the benchmark's launch configuration: A quantized into the
    tile layout, B quantized and prepared, nvfp4_gemm_w4a4_tiled into BF16; every output
    checked, every quantized byte bit-exact."""
    S = 4096
    xa, xb = synth.square_normal(S, "A"), synth.square_normal(S, "B")
    at, gA_t, _ = nv.nvfp4_quantize_tiled(dev(xa).view(torch.bfloat16))
    cb, sb, gB_d, _ = nv.nvfp4_quantize(dev(xb).view(torch.bfloat16))
    a_ref, sa_ref, gA = oracle_quantize_full(xa)
    b_ref, sb_ref, gB = oracle_quantize_full(xb)
    assert np.float32(gA_t.item()) == gA and np.float32(gB_d.item()) == gB
    np.testing.assert_array_equal(host(cb), b_ref)
    np.testing.assert_array_equal(host(sb), sb_ref)
    # the tile layout is the prepared-weight index map; the quantizer's scales are positive and
    # its zero-scale blocks already have zero codes, so the folds change nothing
    tiled_ref, _ = prepared.prepare_weight(a_ref, sa_ref, "ue4m3")
    np.testing.assert_array_equal(host(at), tiled_ref)
    wp, _ = nv.nvfp4_prepare_weight(cb, sb, "ue4m3")
    alpha = alpha_ab(gA, gB)
    out = nv.nvfp4_gemm_w4a4_tiled(at, S, wp, S, S, float(alpha), None, "bf16")
    torch.cuda.synchronize()
    D, Sabs = oracle_w4a4_exact_blocked(a_ref, sa_ref, b_ref, sb_ref, alpha)
    assert_close(host(out), D, Sabs, bf16=True, what="4096^3 full")


@pytest.mark.slow
@pytest.mark.timeout(1200)
def test_w4a4_large_32768_rows():
    """32768^3 with 1 % outlier rows (x8) and 1 % zeroed blocks, in the square benchmark's
    launch configuration (tiled A from the quantizer, prepared B, BF16 out). D is 2 GiB, so
    row offsets exceed 2^31 bytes: the check covers 256 random rows, 64 outlier rows and the
    first and last rows across all 32768 columns; B's quantized bytes are checked in full, A's
    on those rows, and the row-major entry must give the tiled entry's bits."""
    S = 32768
    _progress("32768^3: generating A")
    xa, outl, _ = synth.square_large(S, "A")
    r = np.random.default_rng(S)
    rows = np.unique(np.concatenate([r.choice(S, 256, replace=False), outl[:64], [0, S - 1]]))
    xad = dev(xa).view(torch.bfloat16)
    at, gA_t, _ = nv.nvfp4_quantize_tiled(xad)
    ca, sa, gA_d, _ = nv.nvfp4_quantize(xad)
    del xad
    gA = quantize.global_scale(xa)
    assert np.float32(gA_t.item()) == gA and np.float32(gA_d.item()) == gA
    a_ref, sa_ref = quantize.quantize_rows_with_g(xa[rows], gA)
    ridx = torch.as_tensor(rows).cuda()
    np.testing.assert_array_equal(host(ca[ridx]), a_ref)
    np.testing.assert_array_equal(host(sa[ridx]), sa_ref)
    del xa
    _progress("32768^3: generating B")
    xb, _, _ = synth.square_large(S, "B")
    cb, sb, gB_d, _ = nv.nvfp4_quantize(dev(xb).view(torch.bfloat16))
    _progress("32768^3: oracle quantization of B")
    b_ref, sb_ref, gB = oracle_quantize_full(xb)
    del xb
    assert np.float32(gB_d.item()) == gB
    np.testing.assert_array_equal(host(cb), b_ref)
    np.testing.assert_array_equal(host(sb), sb_ref)
    wp, _ = nv.nvfp4_prepare_weight(cb, sb, "ue4m3")
    del cb, sb
    alpha = alpha_ab(gA, gB)
    out = nv.nvfp4_gemm_w4a4_tiled(at, S, wp, S, S, float(alpha), None, "bf16")
    del at
    std = nv.nvfp4_gemm_w4a4(ca, sa, wp, S, S, float(alpha), None, "bf16")
    torch.cuda.synchronize()
    assert torch.equal(out, std), "tiled and row-major entries differ"
    del std, ca, sa, wp
    got = host(out[ridx])
    del out
    _progress("32768^3: oracle rows")
    D, Sabs = oracle_w4a4_exact_blocked(a_ref, sa_ref, b_ref, sb_ref, alpha, tile=1024)
    assert_close(got, D, Sabs, bf16=True, what="32768^3 rows")


@pytest.mark.slow
def test_w4a4_large_16384_rows():
    """16384^3 with 1 % outlier rows (x8) and 1 % zeroed blocks in both operands, in the
    square benchmark's launch configuration. D is 512 MiB, so the check covers 256 random rows
    and 64 outlier rows of D across all 16384 columns (every column of B, its zero blocks and
    outlier rows included); B's quantized bytes are checked in full, A's on those rows."""
    S = 16384
    xa, outl, _ = synth.square_large(S, "A")
    xb, _, _ = synth.square_large(S, "B")
    r = np.random.default_rng(S)
    rows = np.unique(np.concatenate([r.choice(S, 256, replace=False), outl[:64], [0, S - 1]]))
    at, gA_t, _ = nv.nvfp4_quantize_tiled(dev(xa).view(torch.bfloat16))
    ca, sa, _, _, gA = gpu_quantize_checked(nv, xa, rows)
    cb, sb, gB_d, _ = nv.nvfp4_quantize(dev(xb).view(torch.bfloat16))
    b_ref, sb_ref, gB = oracle_quantize_full(xb)
    assert np.float32(gA_t.item()) == gA and np.float32(gB_d.item()) == gB
    np.testing.assert_array_equal(host(cb), b_ref)
    np.testing.assert_array_equal(host(sb), sb_ref)
    wp, bad = nv.nvfp4_prepare_weight(cb, sb, "ue4m3")
    del cb, sb
    alpha = alpha_ab(gA, gB)
    out = nv.nvfp4_gemm_w4a4_tiled(at, S, wp, S, S, float(alpha), None, "bf16")
    std = nv.nvfp4_gemm_w4a4(ca, sa, wp, S, S, float(alpha), None, "bf16")
    torch.cuda.synchronize()
    assert int(bad.item()) == 0
    assert torch.equal(out, std), "tiled and row-major entries differ"
    del std, ca, sa, at, wp
    got = host(out[torch.as_tensor(rows).cuda()])
    a_ref, sa_ref = quantize.quantize_rows_with_g(xa[rows], gA)
    D, Sabs = oracle_w4a4_exact_blocked(a_ref, sa_ref, b_ref, sb_ref, alpha, tile=1024)
    assert_close(got, D, Sabs, bf16=True, what="16384^3 rows")


# ------------------------------------------------------------------ W4A16

_DECODE_W = {}


def _decode_weight(j):
    if j not in _DECODE_W:
        _DECODE_W[j] = synth.decode_weight(j)
    return _DECODE_W[j]


def _w4a16_case(M, N, K, seed, alpha=0.75):
    b, sb = _random_nvfp4(seed, N, K, -3, 3)
    x = synth.normal_bf16(seed + 1, M, K)
    wp, bad = _prep(b, sb)
    return x, b, sb, wp, alpha


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 12, 16, 17, 32, 64, 128, 300])
@pytest.mark.parametrize("N,K", [(96, 192), (320, 640)])
def test_w4a16_small_shapes(M, N, K):
    x, b, sb, wp, alpha = _w4a16_case(M, N, K, M * 31 + N)
    out = nv.nvfp4_gemm_w4a16(dev(x).view(torch.bfloat16), wp, N, K, alpha)
    torch.cuda.synchronize()
    y, S = gemm.w4a16(x, b, sb, alpha)
    assert_close(host(out), y, S, bf16=True, what=f"w4a16 M={M} {N}x{K}")


@pytest.mark.parametrize("M", [6, 16, 24, 33, 40, 48, 49, 64])
@pytest.mark.parametrize("N,K", [(17408, 4160), (17440, 1088), (2048, 8192)])
def test_w4a16_skinny_long_k(M, N, K):
    """4 < M <= 64 with many tiles per wave; full check. The row kernel stages x rows through
    LDS, padded to 8, 16, 32 or 64 (rows >= M zero); on 544 and 545 row groups (at least one
    per CU) M = 49 and 64 run the fragment kernel on its fragment-order copy of x (two x
    tiles), on 64 groups the row kernel. 544 row groups: 8 waves per workgroup, two groups
    each, 65 tiles over the waves. 545 groups (odd): 8 waves, one group each. 64 groups: 16
    waves (8 at 64 padded rows), 8 or 16 tiles each."""
    x, b, sb, wp, alpha = _w4a16_case(M, N, K, M * 7 + N + K)
    out = nv.nvfp4_gemm_w4a16(dev(x).view(torch.bfloat16), wp, N, K, alpha)
    torch.cuda.synchronize()
    y, S = gemm.w4a16(x, b, sb, alpha)
    assert_close(host(out), y, S, bf16=True, what=f"w4a16 skinny M={M} {N}x{K}")


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("N,K", [(16384, 256), (16416, 1088), (34048, 320), (35968, 192), (36896, 128),
                                 (65536, 128)])
def test_w4a16_wide_decode(M, N, K):
    """Many 32-row groups (>= 2 per CU): the one-group-per-workgroup decode path,
    including a K that leaves the last tile batch partly empty; full check. With
    256 CUs and M = 1, one whole round of 1024 workgroups runs first and the groups
    left over are cut: 34048 rows (40 left) into 8-row workgroups, 35968 (100 left)
    into 16-row ones; 36896 (129 left) and 65536 (two whole rounds) are not cut. The decode
    kernel is asked for explicitly: from M = 3 the library's own choice is the skinny kernel."""
    x, b, sb, wp, alpha = _w4a16_case(M, N, K, M * 7 + N)
    out = nv.nvfp4_gemm_w4a16(dev(x).view(torch.bfloat16), wp, N, K, alpha,
                              config=nv.make_config(nv.KERNEL_W4A16_DECODE))
    torch.cuda.synchronize()
    y, S = gemm.w4a16(x, b, sb, alpha)
    assert_close(host(out), y, S, bf16=True, what=f"wide decode M={M} {N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1000, 2080, 320), (100, 512, 1024), (65, 4096, 4160), (200, 34816, 192),
                                   (2600, 8224, 128), (256, 65792, 64), (300, 56320, 192),
                                   (700, 3008, 33792), (1024, 2048, 49152), (100, 8224, 16064)])
def test_w4a16_big_ragged(M, N, K):
    """Larger M with ragged rows and columns on the persistent MFMA path; full check.
    Fewer 128 x 128 tiles than CUs, each split along K with a fix-up: 1000 x 2080 x 320
    (136 tiles in 3 ranges of 5 chunks, so ranges straddle tiles), 100 x 512 x 1024 (4
    tiles in 8 aligned ranges), 65 x 4096 x 4160 (65 chunks in 8 unaligned ranges).
    256 x 256 tiles, the ones past the last full round split along K over all
    workgroups: 2600 x 8224 (107 of 363 tiles); 256 x 65792 x 64 (one tile of one
    chunk, so every other workgroup's range is empty); 300 x 56320 (184 ragged tiles,
    about two chunks each).
    Fewer 256 x 256 tiles than CUs with a long K, every tile split over all workgroups:
    700 x 3008 x 33792 (36 ragged tiles of 528 chunks, 74-75 per workgroup, so ranges
    straddle tiles) and 1024 x 2048 x 49152 (32 tiles, exactly 8 ranges of 96 per tile).
    128 x 256 tiles: 200 x 34816 x 192 (544 tiles of 128 x 128 would do; 272 of 128 x 256
    fill one round and leave 16 split three chunks over 256 workgroups, most of them empty;
    x from its fragment-order copy) and 100 x 8224 x 16064 (33 ragged tiles, all split,
    about 32 chunks per workgroup; x staged through LDS)."""
    x, b, sb, wp, alpha = _w4a16_case(M, N, K, M + N + K)
    out = nv.nvfp4_gemm_w4a16(dev(x).view(torch.bfloat16), wp, N, K, alpha)
    torch.cuda.synchronize()
    y, S = gemm.w4a16(x, b, sb, alpha)
    assert_close(host(out), y, S, bf16=True, what=f"w4a16 big {M}x{N}x{K}")


@pytest.mark.parametrize("M,K", [(4, 8192), (2, 16384), (1, 32768)])
def test_w4a16_decode_largest_lds(M, K):
    """The decode kernel stages x in LDS up to M * K * 2 = 64 KiB: the largest (M, K) at each
    M that still takes the decode path (asked for explicitly), with a few hundred weight rows;
    full check."""
    N = 320
    x, b, sb, wp, alpha = _w4a16_case(M, N, K, M * 13 + K)
    out = nv.nvfp4_gemm_w4a16(dev(x).view(torch.bfloat16), wp, N, K, alpha,
                              config=nv.make_config(nv.KERNEL_W4A16_DECODE))
    torch.cuda.synchronize()
    y, S = gemm.w4a16(x, b, sb, alpha)
    assert_close(host(out), y, S, bf16=True, what=f"decode LDS edge M={M} K={K}")


@pytest.mark.parametrize("M", [1, 3, 24, 100])
def test_w4a16_misaligned_x_is_copied(M):
    """x starting one BF16 element past a 16-byte boundary (TileLang PR #3290, "Tests": x not
    16-byte aligned): the binding copies it to an aligned buffer; the result must match the
    oracle on the same values."""
    N, K = 320, 640
    x, b, sb, wp, alpha = _w4a16_case(M, N, K, M * 5 + 11)
    flat = torch.zeros(M * K + 8, dtype=torch.bfloat16, device="cuda")
    xv = flat[1:1 + M * K].view(M, K)
    assert xv.data_ptr() % 16 == 2
    xv.copy_(dev(x).view(torch.bfloat16))
    out = nv.nvfp4_gemm_w4a16(xv, wp, N, K, alpha)
    torch.cuda.synchronize()
    y, S = gemm.w4a16(x, b, sb, alpha)
    assert_close(host(out), y, S, bf16=True, what=f"misaligned x M={M}")


def test_binding_rejects_bad_buffers_before_launch():
    """Caller-supplied outputs and scalars are checked (device, dtype, size) before the C call,
    so an undersized or host buffer never reaches a kernel."""
    N, K = 64, 128
    codes, scales = _random_nvfp4(8, N, K)
    cd, sd = dev(codes), dev(scales)
    with pytest.raises(ValueError):
        nv.nvfp4_prepare_weight(cd, sd, out=torch.empty(10, dtype=torch.uint8, device="cuda"))
    with pytest.raises(TypeError):
        nv.nvfp4_prepare_weight(cd, sd, out=torch.empty(N * K, dtype=torch.uint8))           # host
    with pytest.raises(TypeError):
        nv.nvfp4_prepare_weight(cd, sd, bad_count=torch.empty(1, dtype=torch.float32, device="cuda"))
    wp, _ = _prep(codes, scales)
    with pytest.raises(ValueError):      # too few columns
        nv.nvfp4_gemm_w4a4(cd, sd, wp, N, K, out=torch.empty((N, N - 32), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(TypeError):       # host output
        nv.nvfp4_gemm_w4a4(cd, sd, wp, N, K, out=torch.empty((N, N), dtype=torch.bfloat16))
    with pytest.raises(TypeError):       # wrong dtype
        nv.nvfp4_gemm_w4a4(cd, sd, wp, N, K, out=torch.empty((N, N), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):      # undersized workspace
        nv.nvfp4_gemm_w4a4(cd, sd, wp, N, K, ws=torch.empty(16, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):      # alpha_dev with no value
        nv.nvfp4_gemm_w4a4(cd, sd, wp, N, K, alpha_dev=torch.empty(0, dtype=torch.float32, device="cuda"))
    x = torch.zeros((2, K), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        nv.nvfp4_gemm_w4a16(x, wp, N, K, out=torch.empty((1, N), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        nv.nvfp4_quantize(x, codes=torch.empty(K // 2, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        nv.nvfp4_quantize(x, scales=torch.empty(1, dtype=torch.uint8, device="cuda"))
    with pytest.raises(TypeError):
        nv.nvfp4_quantize(x, g=torch.empty(1, dtype=torch.float64, device="cuda"))
    with pytest.raises(ValueError):
        nv.nvfp4_quantize_tiled(x, out=torch.empty(100, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        nv.nvfp4_quantize_tiled(x, ws=torch.empty(4, dtype=torch.uint8, device="cuda"))


# ------------------------------------------------------------------ per-column alpha

def _alpha_col(seed, N):
    """Per-column scales of both signs over 2^-6 .. 2^6, every 17th zero."""
    r = np.random.default_rng(seed)
    c = (2.0 ** r.uniform(-6, 6, N) * r.choice([-1.0, 1.0], N)).astype(np.float32)
    c[::17] = 0.0
    return c


@pytest.mark.parametrize("M,N,K,entry", [(300, 320, 192, "std"), (4000, 4192, 256, "std"),
                                         (4000, 4192, 256, "tiled"), (4100, 4128, 128, "tiled")])
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_w4a4_per_column_alpha(M, N, K, entry, out_dtype):
    """A global or a per-column weight scale (TileLang PR #3290, "Summary"): column n is scaled
    by fl32(alpha_eff * alpha_col[n]), alpha_eff = alpha * *alpha_dev. 128 x 128 tiles (300 x 320);
    256 x 256 tiles with the last round as quadrants and ragged edges; full check."""
    a, sa = _random_nvfp4(M + 3, M, K)
    b, sb = _random_nvfp4(N + 4, N, K)
    wp, _ = _prep(b, sb)
    ac = _alpha_col(M + N, N)
    ad = torch.tensor([1.5], dtype=torch.float32, device="cuda")
    if entry == "std":
        out = nv.nvfp4_gemm_w4a4(dev(a), dev(sa), wp, N, K, 0.3, ad, out_dtype, alpha_col=dev(ac))
    else:
        at = nv.nvfp4_tile_activation(dev(a), dev(sa))
        out = nv.nvfp4_gemm_w4a4_tiled(at, M, wp, N, K, 0.3, ad, out_dtype, alpha_col=dev(ac))
    torch.cuda.synchronize()
    al = gemm.column_alpha(gemm.alpha_product(0.3, np.float32(1.5)), ac)
    D, S = oracle_w4a4_exact_blocked(a, sa, b, sb, al)
    assert_close(host(out), D, S, bf16=out_dtype == "bf16", what=f"per-column alpha {entry} {M}x{N}x{K}")
    assert not host(out)[:, ::17].any(), "zero column scales give zero columns"


@pytest.mark.parametrize("M,N,K", [(1, 34816, 256), (3, 320, 640), (16, 17408, 1088), (24, 17408, 1088),
                                   (40, 2048, 1024), (56, 17408, 1088), (100, 512, 1024), (300, 56320, 192),
                                   (1000, 2080, 320)])
def test_w4a16_per_column_alpha_zero_negative_scales(M, N, K):
    """Per-column alpha with zero and negative block scales (the combination the pages' tests
    name) on every W4A16 path: decode with the cut tail (1 x 34816), M = 3, the row kernel at 16,
    32 (two row groups per workgroup) and 64 padded rows (16, 24, 40), the fragment kernel on
    its fragment-order copy (56 rows of a 544-group weight), the 128 x 128 split with a fix-up
    (100 x 512, 1000 x 2080), 256 x 256 tiles with split leftovers (300 x 56320); full check."""
    x, b, sb, _, alpha = _w4a16_case(M, N, K, M + N + K + 5)
    sb = sb.copy()
    sb[::5] |= 0x80
    sb[1::7] = 0
    wp, bad = _prep(b, sb)
    assert bad == 0
    ac = _alpha_col(N + K, N)
    ad = torch.tensor([0.75], dtype=torch.float32, device="cuda")
    out = nv.nvfp4_gemm_w4a16(dev(x).view(torch.bfloat16), wp, N, K, alpha, ad, alpha_col=dev(ac))
    torch.cuda.synchronize()
    al = gemm.column_alpha(gemm.alpha_product(alpha, np.float32(0.75)), ac)
    y, S = oracle_w4a16_blocked(x, b, sb, al)
    assert_close(host(out), y, S, bf16=True, what=f"w4a16 per-column alpha M={M} {N}x{K}")


_DECODE_Q = {}


def _decode_weight_oracle(j):
    """The oracle's quantization of decode weight j: (codes, scales, g), computed once."""
    if j not in _DECODE_Q:
        _DECODE_Q[j] = oracle_quantize_full(_decode_weight(j))
    return _DECODE_Q[j]


@pytest.mark.parametrize("j", range(4))
@pytest.mark.parametrize("mi", range(5))
def test_w4a16_decode_shapes(j, mi):
    """27B-class layer shapes with W ~ N(0, 0.02) quantized on the GPU (bytes checked
    bit-exact against the oracle's), x ~ N(0, 1); every output checked."""
    M = synth.DECODE_MS[mi]
    N, K = synth.DECODE_SHAPES[j]
    w = _decode_weight(j)
    x = synth.decode_activation(M, j, mi)
    cw, sw, gW_d, _ = nv.nvfp4_quantize(dev(w).view(torch.bfloat16))
    c_ref, s_ref, gW = _decode_weight_oracle(j)
    assert np.float32(gW_d.item()) == gW
    np.testing.assert_array_equal(host(cw), c_ref)
    np.testing.assert_array_equal(host(sw), s_ref)
    wp, bad = nv.nvfp4_prepare_weight(cw, sw, "ue4m3")
    alpha = np.float32(np.float32(1.0) / gW)
    out = nv.nvfp4_gemm_w4a16(dev(x).view(torch.bfloat16), wp, N, K, float(alpha))
    out2 = nv.nvfp4_gemm_w4a16(dev(x).view(torch.bfloat16), wp, N, K, float(alpha))
    torch.cuda.synchronize()
    assert int(bad.item()) == 0
    assert torch.equal(out, out2), "repeat calls must be bit-identical"
    y, S = oracle_w4a16_blocked(x, c_ref, s_ref, alpha)
    assert_close(host(out), y, S, bf16=True, what=f"decode {N}x{K} M={M}")


def test_w4a16_zero_negative_scales_and_strided_out():
    M, N, K = 3, 64, 256
    b, sb = _random_nvfp4(41, N, K)
    sb[0, :] = 0x00
    sb[1, :] |= 0x80            # negative scales
    sb[2, 1] = 0x80             # -0
    x = synth.normal_bf16(42, M, K)
    wp, bad = _prep(b, sb)
    assert bad == 0
    big = torch.zeros((M, N + 64), dtype=torch.bfloat16, device="cuda")
    out = nv.nvfp4_gemm_w4a16(dev(x).view(torch.bfloat16), wp, N, K, 1.0, out=big[:, :N])
    torch.cuda.synchronize()
    y, S = gemm.w4a16(x, b, sb, 1.0)
    assert_close(host(big[:, :N]), y, S, bf16=True, what="signed scales")
    assert (host(big[:, N:]) == 0).all()


@pytest.mark.parametrize("M", [5, 8, 16, 24, 40])
@pytest.mark.parametrize("N", [96, 17408])
def test_w4a16_row_kernel_scale_edges(M, N):
    """The row kernel at M <= 16 folds the power of two of each block scale into the code
    conversion and multiplies the block's MFMA result by the scale's frexp mantissa; at
    M = 24 and 40 (32 and 64 padded rows) it dequantizes in full. Zero, negative and -0
    scales, every E4M3 subnormal, the largest normal (448) against the largest codes, and a
    NaN scale byte (its column must come out NaN in every row). 3 row groups (16 waves each,
    8 at 64 rows) and 544 (8 waves, two groups per workgroup)."""
    K = 256
    b, sb = _random_nvfp4(91 + M, N, K)
    codes = synth.random_codes(92 + M, N, K)
    codes[3] = np.where(np.arange(K) % 2 == 0, 0x7, 0xF)        # +-6 against scale 448
    b = formats.pack_nibbles(codes)
    sb[0, :] = 0x00
    sb[1, :] |= 0x80                                             # negative scales
    sb[2, :] = np.arange(K // 16) % 7 + 1                         # subnormals 0x01 .. 0x07
    sb[3, :] = 0x7E
    sb[4, 1] = 0x7F                                              # NaN in block 1 of row 4
    sb[5, :] = 0x80                                              # -0
    sb[6, :] = np.arange(K // 16) % 2 + 0x07                     # largest subnormal / smallest normal
    x = synth.normal_bf16(93 + M, M, K)
    wp, bad = _prep(b, sb)
    assert bad == 1
    out = nv.nvfp4_gemm_w4a16(dev(x).view(torch.bfloat16), wp, N, K, 0.37)
    torch.cuda.synchronize()
    got = host(out)
    assert np.isnan(got[:, 4]).all(), "a NaN scale must make its column NaN"
    y, S = gemm.w4a16(x, b, sb, 0.37)
    assert_close(got, y, S, bf16=True, what=f"row kernel scale edges M={M} N={N}")


@pytest.mark.parametrize("M,N,K,tile", [(1, 5120, 5120, None), (128, 6144, 5120, (128, 128)),
                                        (256, 8192, 1024, (128, 256)), (512, 8192, 512, (256, 256))])
def test_w4a16_graph_capture_replay_matches_eager(M, N, K, tile):
    """Replays of a captured call against eager calls that share its workspace, bit for bit. With
    tiles, every tile is split along K (6144 x 5120 at M = 128: 48 tiles in 5 ranges each; 64
    tiles over 256 workgroups otherwise), so each call writes FP32 partials into the workspace
    and a second kernel adds them in a fixed order. The workspace starts as random bytes; two
    replays in a row and the eager calls in between must all agree."""
    x, b, sb, wp, alpha = _w4a16_case(M, N, K, 77 + M)
    cfg = None if tile is None else nv.make_config(nv.KERNEL_W4A16_TILES, tile_m=tile[0], tile_n=tile[1])
    xd = dev(x).view(torch.bfloat16).clone()
    ws = nv.workspace(nv.OP_W4A16, M, N, K, config=cfg)
    if ws is not None:
        ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, generator=torch.Generator().manual_seed(5)).to(ws.device))
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    nv.nvfp4_gemm_w4a16(xd, wp, N, K, alpha, out=out, ws=ws, config=cfg)   # warm-up outside capture
    torch.cuda.synchronize()
    y, S = gemm.w4a16(x, b, sb, alpha)
    assert_close(host(out), y, S, bf16=True, what=f"w4a16 graph warm-up M={M} {N}x{K}")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            nv.nvfp4_gemm_w4a16(xd, wp, N, K, alpha, out=out, ws=ws, config=cfg)
    torch.cuda.synchronize()
    for rep in range(3):
        xn = synth.normal_bf16(900 + rep, M, K)
        xd.copy_(dev(xn).view(torch.bfloat16))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        g.replay()                                     # the words now read complete for this epoch
        torch.cuda.synchronize()
        assert torch.equal(out, got)
        eager = nv.nvfp4_gemm_w4a16(dev(xn).view(torch.bfloat16), wp, N, K, alpha, ws=ws, config=cfg)
        torch.cuda.synchronize()
        assert torch.equal(got, eager)


@pytest.mark.parametrize("mode", ["no_workspace", "split", "split_dynamic"])
@pytest.mark.parametrize("two_pass", [False, True])
def test_prefill_graph_capture_replay_matches_eager(two_pass, mode):
    """The prefill step (on-device quantize into the tile layout, then the W4A4 GEMM with the
    device 1/gA) captured once in a graph and replayed on new activations: every replay the
    same bits as eager calls. 4000 x 4192 x 256 (K = 512 two-pass): 256 x 256 tiles plus a last
    round of 16 tiles, run as quadrants (the library's choice without a workspace: two GEMM
    launches), split along K with the fix-up (two launches), or split with the dynamic schedule
    (counter reset, GEMM, fix-up: three launches); one- and two-pass."""
    M, N, K = 4000, 4192, 256
    b, sb = _random_nvfp4(91, N, K, -3, 3)
    wp, _ = _prep(b, sb)
    quant = nv.nvfp4_quantize_two_pass_tiled if two_pass else nv.nvfp4_quantize_tiled
    gemm_fn = nv.nvfp4_gemm_w4a4_two_pass_tiled if two_pass else nv.nvfp4_gemm_w4a4_tiled
    Kc = 2 * K if two_pass else K
    cfg = None
    if mode != "no_workspace":
        cfg = nv.make_config(nv.KERNEL_W4A4_TILES, 256, 256, nv.TAIL_SPLIT, 2, dynamic=int(mode == "split_dynamic"))
    gws = None
    if mode != "no_workspace":
        gws = torch.empty(nv.workspace_bytes(nv.OP_W4A4_TILED, M, N, Kc, cfg), dtype=torch.uint8, device="cuda")
    xd = dev(synth.normal_bf16(92, M, K)).view(torch.bfloat16).clone()
    at, g, ig = quant(xd)                                   # buffers, and a warm-up outside capture
    ws = torch.empty(nv.workspace_bytes(nv.OP_QUANTIZE, M, 0, K), dtype=torch.uint8, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    gemm_fn(at, M, wp, N, K, 0.5, ig, "bf16", out, config=cfg, ws=gws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        with torch.cuda.graph(graph, stream=st):
            quant(xd, at, g, ig, ws)
            gemm_fn(at, M, wp, N, K, 0.5, ig, "bf16", out, config=cfg, ws=gws)
    torch.cuda.synchronize()
    for rep in range(3):
        xn = dev(synth.normal_bf16(930 + rep, M, K)).view(torch.bfloat16)
        xd.copy_(xn)
        graph.replay()
        torch.cuda.synchronize()
        at2, _, ig2 = quant(xn)
        eager = gemm_fn(at2, M, wp, N, K, 0.5, ig2, "bf16", config=cfg, ws=gws)
        torch.cuda.synchronize()
        assert torch.equal(at, at2) and torch.equal(ig, ig2)
        assert torch.equal(out, eager), f"replay {rep}"


# ------------------------------------------------------------------ prefill W4A4 with on-device quantize

def test_prefill_quantize_then_w4a4_full():
    """The prefill workload as the benchmark runs it: W quantized and prepared, then the timed
    pair nvfp4_quantize_tiled(x) -> nvfp4_gemm_w4a4_tiled with alpha = 1/gW on the host and
    inv_gA from the device. Quantized bytes of x and W bit-exact, every output checked."""
    x, _ = synth.prefill_activation()
    w = synth.prefill_weight()
    M, K = x.shape
    N = w.shape[0]
    cw, sw, gW_d, _ = nv.nvfp4_quantize(dev(w).view(torch.bfloat16))
    wp, bad = nv.nvfp4_prepare_weight(cw, sw, "ue4m3")
    xd = dev(x).view(torch.bfloat16)
    at, gA_t, inv_gA = nv.nvfp4_quantize_tiled(xd)
    ca, sa, _, _ = nv.nvfp4_quantize(xd)
    w_ref, sw_ref, gW = oracle_quantize_full(w)
    a_ref, sa_ref, gA = oracle_quantize_full(x)
    assert np.float32(gW_d.item()) == gW and np.float32(gA_t.item()) == gA
    assert np.float32(inv_gA.item()) == np.float32(np.float32(1.0) / gA)
    np.testing.assert_array_equal(host(cw), w_ref)
    np.testing.assert_array_equal(host(sw), sw_ref)
    np.testing.assert_array_equal(host(ca), a_ref)
    np.testing.assert_array_equal(host(sa), sa_ref)
    del cw, sw, ca, sa, xd
    alpha_w = np.float32(np.float32(1.0) / gW)
    out = nv.nvfp4_gemm_w4a4_tiled(at, M, wp, N, K, float(alpha_w), inv_gA, "bf16")
    torch.cuda.synchronize()
    assert int(bad.item()) == 0
    del at, wp
    alpha_eff = gemm.alpha_product(alpha_w, np.float32(np.float32(1.0) / gA))
    D, S = oracle_w4a4_exact_blocked(a_ref, sa_ref, w_ref, sw_ref, alpha_eff)
    assert_close(host(out), D, S, bf16=True, what="prefill full")


# ------------------------------------------------------------------ two-pass prefill

def _two_pass_layout_ref(x_bits):
    """The oracle's two passes, laid out as the [rows][2K] tile-layout activation."""
    c1, s1, c2, s2, g, ig = quantize.two_pass(x_bits)
    rows = x_bits.shape[0]
    Mp = -(-rows // 32) * 32
    cp = np.zeros((Mp, c1.shape[1] * 2), np.uint8)
    sp = np.zeros((Mp, s1.shape[1] * 2), np.uint8)
    cp[:rows], sp[:rows] = np.concatenate([c1, c2], axis=1), np.concatenate([s1, s2], axis=1)
    ref, _ = prepared.prepare_weight(cp, sp, "ue4m3")
    return ref, (c1, s1, c2, s2), g, ig


@pytest.mark.parametrize("rows,K", [(1, 64), (77, 320), (256, 5120)])
def test_quantize_two_pass_tiled_bit_exact(rows, K):
    """Value and residual passes under one g (the two-pass prefill of TileLang PR #3290,
    "Follow-ups"), every byte of the 2K-column tile layout against the oracle."""
    x = synth.normal_bf16(rows * 5 + K, rows, K)
    a2, g, ig = nv.nvfp4_quantize_two_pass_tiled(dev(x).view(torch.bfloat16))
    torch.cuda.synchronize()
    ref, (_, _, c2, _), g_ref, ig_ref = _two_pass_layout_ref(x)
    assert np.float32(g.item()) == g_ref and np.float32(ig.item()) == ig_ref
    assert c2.any(), "the residual pass is not empty on normal data"
    np.testing.assert_array_equal(host(a2), ref)


def test_quantize_two_pass_edge_values():
    """Blocks on the E2M1 grid (zero residual), an all-zero block, signed zeros and tiny values."""
    vals = np.zeros((2, 64), np.float32)
    vals[0, :16] = [6, 4, 3, 2, 1.5, 1, .5, 0, -6, -4, -3, -2, -1.5, -1, -.5, -0.0]
    vals[0, 32:48] = np.linspace(-1e-3, 1e-3, 16)
    vals[1, :] = np.linspace(-5.9, 5.7, 64)
    vals[1, 5] = -0.0
    x = formats.f32_to_bf16_bits(vals)
    a2, g, _ = nv.nvfp4_quantize_two_pass_tiled(dev(x).view(torch.bfloat16))
    torch.cuda.synchronize()
    ref, _, g_ref, _ = _two_pass_layout_ref(x)
    assert np.float32(g.item()) == g_ref
    np.testing.assert_array_equal(host(a2), ref)


@pytest.mark.parametrize("M,N,K,out_dtype", [(300, 320, 192, "f32"), (4000, 4192, 256, "bf16"),
                                             (8192, 17408, 5120, "bf16")])
def test_w4a4_two_pass_gemm(M, N, K, out_dtype):
    """D = alpha (A1 + A2) W^T from x through the two-pass quantizer and the two-pass GEMM,
    alpha = 1/(gA gW) as for the one-pass prefill, against the oracle's 2K contraction on its
    own quantization of x: 128 x 128 tiles, 256 x 256 tiles with ragged edges and the last
    round as quadrants, and the prefill layer shape (every output checked)."""
    x = synth.normal_bf16(M + N + K, M, K)
    b, sb = _random_nvfp4(N + 9, N, K, -3, 3)
    wp, _ = _prep(b, sb)
    a2, g, ig = nv.nvfp4_quantize_two_pass_tiled(dev(x).view(torch.bfloat16))
    out = nv.nvfp4_gemm_w4a4_two_pass_tiled(a2, M, wp, N, K, 0.25, ig, out_dtype)
    torch.cuda.synchronize()
    c1, s1, c2, s2, g_ref, ig_ref = quantize.two_pass(x)
    assert np.float32(ig.item()) == ig_ref
    alpha = gemm.alpha_product(0.25, ig_ref)
    D, S = oracle_w4a4_exact_blocked(np.concatenate([c1, c2], 1), np.concatenate([s1, s2], 1),
                                     np.concatenate([b, b], 1), np.concatenate([sb, sb], 1), alpha)
    assert_close(host(out), D, S, bf16=out_dtype == "bf16", what=f"two-pass {M}x{N}x{K}")
