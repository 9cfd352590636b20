"""Host-only checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments with the documented status before any
launch (no GPU needed: every case here fails in the host-side checks)."""
import ctypes
import os
import re

import pytest

import nvfp4_block_scaled_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = nv.lib()
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert sorted(nv.EXPORTED) == names


def test_status_strings():
    L = nv.lib()
    assert L.nvfp4_status_str(0) == b"ok"
    assert L.nvfp4_status_str(2) == b"bad shape"
    assert L.nvfp4_status_str(99) == b"unknown status"


def test_prepared_size():
    L = nv.lib()
    assert L.nvfp4_prepared_weight_bytes(34816, 5120) == 34816 * 5120 // 2 + 34816 * 5120 // 16
    assert L.nvfp4_prepared_weight_bytes(33, 64) == 0
    assert L.nvfp4_prepared_weight_bytes(32, 65) == 0
    assert L.nvfp4_prepared_weight_bytes(0, 64) == 0


FAKE = ctypes.c_void_p(0x10000)       # a non-null, 64 KiB-aligned value; never dereferenced
ODD = ctypes.c_void_p(0x10001)


def test_gemm_w4a4_argument_checks():
    f = nv.lib().nvfp4_gemm_w4a4
    need = nv.lib().nvfp4_workspace_bytes(nv.OP_W4A4, 64, 64, 128)
    ok = dict(a=FAKE, s=FAKE, w=FAKE, M=64, N=64, K=128, alpha=1.0, ad=None, ac=None, d=FAKE, dt=nv.OUT_BF16, ldd=64,
              ws=None, nws=0)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["a"], a["s"], a["w"], a["M"], a["N"], a["K"], a["alpha"], a["ad"], a["ac"], a["d"], a["dt"],
                 a["ldd"], a["ws"], a["nws"], None)
    assert call(dt=7) == nv.ERR_DTYPE
    assert call(K=96) == nv.ERR_SHAPE
    assert call(N=48) == nv.ERR_SHAPE
    assert call(M=-1) == nv.ERR_SHAPE
    assert call(ldd=32) == nv.ERR_SHAPE
    assert call(M=0) == nv.OK                     # empty: nothing to do, nothing launched
    assert call(a=None) == nv.ERR_NULL
    assert call(d=None) == nv.ERR_NULL
    assert call(alpha=float("nan")) == nv.ERR_VALUE
    assert call(alpha=float("inf")) == nv.ERR_VALUE
    assert call(a=ODD) == nv.ERR_ALIGN
    assert call(w=ODD) == nv.ERR_ALIGN
    assert call() == nv.ERR_WORKSPACE             # A is re-tiled into the workspace
    assert call(ws=FAKE, nws=need - 1) == nv.ERR_WORKSPACE
    assert call(ws=ODD, nws=need) == nv.ERR_ALIGN
    assert call(ac=ODD, ws=FAKE, nws=need) == nv.ERR_ALIGN   # per-column alpha: FP32 aligned
    assert call(ad=ODD, ws=FAKE, nws=need) == nv.ERR_ALIGN


def test_tile_activation_and_tiled_gemm_argument_checks():
    L = nv.lib()
    assert L.nvfp4_tiled_activation_bytes(33, 128) == 64 * 128 * 9 // 16
    assert L.nvfp4_tiled_activation_bytes(32, 96) == 0
    t = L.nvfp4_tile_activation
    assert t(FAKE, FAKE, 64, 96, FAKE, None) == nv.ERR_SHAPE
    assert t(FAKE, FAKE, -1, 128, FAKE, None) == nv.ERR_SHAPE
    assert t(FAKE, FAKE, 0, 128, FAKE, None) == nv.OK
    assert t(None, FAKE, 64, 128, FAKE, None) == nv.ERR_NULL
    assert t(FAKE, FAKE, 64, 128, None, None) == nv.ERR_NULL
    assert t(ODD, FAKE, 64, 128, FAKE, None) == nv.ERR_ALIGN
    assert t(FAKE, FAKE, 64, 128, ODD, None) == nv.ERR_ALIGN
    g = L.nvfp4_gemm_w4a4_tiled

    def call(at=FAKE, w=FAKE, M=64, N=64, K=128, alpha=1.0, ac=None, d=FAKE, dt=nv.OUT_BF16, ldd=64):
        return g(at, w, M, N, K, alpha, None, ac, d, dt, ldd, None)
    assert call(dt=5) == nv.ERR_DTYPE
    assert call(K=96) == nv.ERR_SHAPE
    assert call(N=40) == nv.ERR_SHAPE
    assert call(M=0) == nv.OK
    assert call(at=None) == nv.ERR_NULL
    assert call(w=None) == nv.ERR_NULL
    assert call(alpha=float("nan")) == nv.ERR_VALUE
    assert call(at=ODD) == nv.ERR_ALIGN
    assert call(d=ODD) == nv.ERR_ALIGN
    assert call(ac=ODD) == nv.ERR_ALIGN


def test_quantize_tiled_argument_checks():
    q = nv.lib().nvfp4_quantize_tiled
    assert q(FAKE, 64, 128, FAKE, None, None, FAKE, 4096, None) == nv.ERR_NULL      # g_dev
    assert q(FAKE, 64, 96, FAKE, FAKE, None, FAKE, 4096, None) == nv.ERR_SHAPE      # K % 64
    assert q(FAKE, -1, 128, FAKE, FAKE, None, FAKE, 4096, None) == nv.ERR_SHAPE
    assert q(None, 64, 128, FAKE, FAKE, None, FAKE, 4096, None) == nv.ERR_NULL
    assert q(FAKE, 64, 128, FAKE, FAKE, None, None, 0, None) == nv.ERR_WORKSPACE
    assert q(FAKE, 64, 128, ODD, FAKE, None, FAKE, 4096, None) == nv.ERR_ALIGN


def test_two_pass_argument_checks():
    L = nv.lib()
    q = L.nvfp4_quantize_two_pass_tiled
    assert q(FAKE, 64, 128, FAKE, None, None, FAKE, 4096, None) == nv.ERR_NULL      # g_dev
    assert q(FAKE, 64, 96, FAKE, FAKE, None, FAKE, 4096, None) == nv.ERR_SHAPE      # K % 64
    assert q(FAKE, 64, 128, FAKE, FAKE, None, None, 0, None) == nv.ERR_WORKSPACE
    assert q(FAKE, 64, 128, ODD, FAKE, None, FAKE, 4096, None) == nv.ERR_ALIGN
    g = L.nvfp4_gemm_w4a4_two_pass_tiled

    def call(at=FAKE, w=FAKE, M=64, N=64, K=128, alpha=1.0, ac=None, d=FAKE, dt=nv.OUT_BF16, ldd=64):
        return g(at, w, M, N, K, alpha, None, ac, d, dt, ldd, None)
    assert call(dt=3) == nv.ERR_DTYPE
    assert call(K=96) == nv.ERR_SHAPE
    assert call(M=0) == nv.OK
    assert call(at=None) == nv.ERR_NULL
    assert call(alpha=float("nan")) == nv.ERR_VALUE
    assert call(at=ODD) == nv.ERR_ALIGN
    assert call(ac=ODD) == nv.ERR_ALIGN


def test_gemm_w4a16_argument_checks():
    f = nv.lib().nvfp4_gemm_w4a16

    def call(x=FAKE, ldx=128, w=FAKE, M=1, N=64, K=128, alpha=1.0, ac=None, y=FAKE, ldy=64, ws=None, nws=0):
        return f(x, ldx, w, M, N, K, alpha, None, ac, y, ldy, ws, nws, None)
    assert call(K=100) == nv.ERR_SHAPE
    assert call(ldx=64) == nv.ERR_SHAPE
    assert call(ldy=32) == nv.ERR_SHAPE
    assert call(M=0) == nv.OK
    assert call(x=None) == nv.ERR_NULL
    assert call(alpha=float("-inf")) == nv.ERR_VALUE
    assert call(ldx=132) == nv.ERR_ALIGN
    assert call(x=ODD) == nv.ERR_ALIGN
    assert call(ac=ODD) == nv.ERR_ALIGN


def test_prepare_and_quantize_argument_checks():
    L = nv.lib()
    p = L.nvfp4_prepare_weight
    assert p(None, FAKE, nv.SCALE_E4M3, 32, 64, FAKE, None, None) == nv.ERR_NULL
    assert p(FAKE, FAKE, 5, 32, 64, FAKE, None, None) == nv.ERR_DTYPE
    assert p(FAKE, FAKE, nv.SCALE_E4M3, 33, 64, FAKE, None, None) == nv.ERR_SHAPE
    assert p(FAKE, FAKE, nv.SCALE_E4M3, 32, 96, FAKE, None, None) == nv.ERR_SHAPE
    assert p(ODD, FAKE, nv.SCALE_E4M3, 32, 64, FAKE, None, None) == nv.ERR_ALIGN
    q = L.nvfp4_quantize
    assert q(FAKE, 4, 32, FAKE, FAKE, None, None, FAKE, 4096, None) == nv.ERR_NULL
    assert q(FAKE, 4, 24, FAKE, FAKE, FAKE, None, FAKE, 4096, None) == nv.ERR_SHAPE
    assert q(FAKE, 4, 32, FAKE, FAKE, FAKE, None, None, 0, None) == nv.ERR_WORKSPACE
    assert q(FAKE, 4, 32, FAKE, FAKE, FAKE, None, FAKE, 16, None) == nv.ERR_WORKSPACE
    assert q(ODD, 4, 32, FAKE, FAKE, FAKE, None, FAKE, 4096, None) == nv.ERR_ALIGN


def test_workspace_sizes():
    L = nv.lib()
    # W4A4: A in the prepared tile layout, rows rounded up to 32
    assert L.nvfp4_workspace_bytes(nv.OP_W4A4, 8192, 8192, 8192) == 8192 * 8192 * 9 // 16
    assert L.nvfp4_workspace_bytes(nv.OP_W4A4, 33, 64, 128) == 64 * 128 * 9 // 16
    assert L.nvfp4_workspace_bytes(nv.OP_W4A4, 0, 64, 128) == 0
    assert L.nvfp4_workspace_bytes(nv.OP_QUANTIZE, 8192, 0, 5120) >= 4
    # W4A16 (no device here: the plan assumes 256 CUs). Decode (M <= 4) needs none; the
    # skinny kernel's x copy for 16 < M <= 64 is 32 rows x K BF16.
    assert L.nvfp4_workspace_bytes(nv.OP_W4A16, 1, 34816, 5120) == 0
    assert L.nvfp4_workspace_bytes(nv.OP_W4A16, 4, 34816, 5120) == 0
    assert L.nvfp4_workspace_bytes(nv.OP_W4A16, 16, 34816, 5120) == 0
    assert L.nvfp4_workspace_bytes(nv.OP_W4A16, 24, 17408, 4160) == 32 * 4160 * 2
    # M = 128 on 34816 x 5120: 136 tiles of 128 x 256, all split over 256 workgroups (two
    # 128 KiB partial slots each), then x for one 128-row tile in fragment order
    assert L.nvfp4_workspace_bytes(nv.OP_W4A16, 128, 34816, 5120) == 256 * 2 * 128 * 1024 + 128 * 5120 * 2
    # M = 1024: 544 tiles of 256 x 256, 512 in two whole rounds and 32 split (two 256 KiB
    # slots per workgroup), then x for four 256-row tiles
    assert L.nvfp4_workspace_bytes(nv.OP_W4A16, 1024, 34816, 5120) == 256 * 2 * 256 * 1024 + 1024 * 5120 * 2
    # 8192 rows on 256 x 256 tiles fill 32 x 32 = 1024 tiles, 4 whole rounds: x copy only
    assert L.nvfp4_workspace_bytes(nv.OP_W4A16, 8192, 8192, 1024) == 8192 * 1024 * 2
    assert L.nvfp4_workspace_bytes(7, 1, 1, 1) == 0
    assert L.nvfp4_workspace_init(None, 0, None) == nv.OK
    assert L.nvfp4_workspace_init(None, 64, None) == nv.ERR_NULL
    assert L.nvfp4_workspace_init(ODD, 64, None) == nv.ERR_ALIGN


def test_python_wrapper_type_errors():
    import torch
    with pytest.raises(TypeError):
        nv.nvfp4_gemm_w4a16(torch.zeros(2, 64), None, 32, 64)


def test_init_rejects_bad_device_index():
    L = nv.lib()
    assert L.nvfp4_init(-1) == nv.ERR_VALUE
    assert L.nvfp4_init(1 << 20) == nv.ERR_VALUE


def test_binding_rejects_host_tensors_before_any_launch():
    """Every caller-supplied tensor must be a device tensor: a host pointer handed to a kernel
    would fault the GPU, so the binding raises TypeError before calling the library."""
    import torch
    cpu8 = torch.zeros(64, 32, dtype=torch.uint8)
    with pytest.raises(TypeError):
        nv.nvfp4_prepare_weight(cpu8, torch.zeros(64, 4, dtype=torch.uint8))
    with pytest.raises(TypeError):
        nv.nvfp4_gemm_w4a4(cpu8, torch.zeros(64, 4, dtype=torch.uint8), torch.zeros(10, dtype=torch.uint8), 32, 64)
    with pytest.raises(TypeError):
        nv.nvfp4_gemm_w4a4_tiled(torch.zeros(4096, dtype=torch.uint8), 64, torch.zeros(10, dtype=torch.uint8), 32, 64)
    with pytest.raises(TypeError):
        nv.nvfp4_gemm_w4a16(torch.zeros(2, 64, dtype=torch.bfloat16), torch.zeros(10, dtype=torch.uint8), 32, 64)
    with pytest.raises(TypeError):
        nv.nvfp4_quantize(torch.zeros(2, 64, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        nv.nvfp4_quantize_tiled(torch.zeros(2, 64, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        nv.nvfp4_quantize_two_pass_tiled(torch.zeros(2, 64, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        nv.nvfp4_tile_activation(cpu8, torch.zeros(64, 4, dtype=torch.uint8))
