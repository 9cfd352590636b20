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
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)          # declarations only, not comments
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
QWS = 12544        # bytes of the quantizer workspace (nvfp4_workspace_bytes(NVFP4_OP_QUANTIZE, ...))
ODD = ctypes.c_void_p(0x10001)


def test_gemm_w4a4_argument_checks():
    f = nv.lib().nvfp4_gemm_w4a4
    need = nv.lib().nvfp4_workspace_bytes(nv.OP_W4A4, 64, 64, 128)
    ok = dict(a=FAKE, s=FAKE, w=FAKE, M=64, N=64, K=128, alpha=1.0, ad=None, ac=None, d=FAKE, dt=nv.OUT_BF16, ldd=64,
              ws=None, nws=0)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["a"], a["s"], a["w"], a["M"], a["N"], a["K"], a["alpha"], a["ad"], a["ac"], a["d"], a["dt"],
                 a["ldd"], None, a["ws"], a["nws"], None)
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
        return g(at, w, M, N, K, alpha, None, ac, d, dt, ldd, None, None, 0, None)
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
    assert q(FAKE, 64, 128, FAKE, None, None, FAKE, QWS, None) == nv.ERR_NULL      # g_dev
    assert q(FAKE, 64, 96, FAKE, FAKE, None, FAKE, QWS, None) == nv.ERR_SHAPE      # K % 64
    assert q(FAKE, -1, 128, FAKE, FAKE, None, FAKE, QWS, None) == nv.ERR_SHAPE
    assert q(None, 64, 128, FAKE, FAKE, None, FAKE, QWS, None) == nv.ERR_NULL
    assert q(FAKE, 64, 128, FAKE, FAKE, None, None, 0, None) == nv.ERR_WORKSPACE
    assert q(FAKE, 64, 128, ODD, FAKE, None, FAKE, QWS, None) == nv.ERR_ALIGN


def test_two_pass_argument_checks():
    L = nv.lib()
    q = L.nvfp4_quantize_two_pass_tiled
    assert q(FAKE, 64, 128, FAKE, None, None, FAKE, QWS, None) == nv.ERR_NULL      # g_dev
    assert q(FAKE, 64, 96, FAKE, FAKE, None, FAKE, QWS, None) == nv.ERR_SHAPE      # K % 64
    assert q(FAKE, 64, 128, FAKE, FAKE, None, None, 0, None) == nv.ERR_WORKSPACE
    assert q(FAKE, 64, 128, ODD, FAKE, None, FAKE, QWS, None) == nv.ERR_ALIGN
    g = L.nvfp4_gemm_w4a4_two_pass_tiled

    def call(at=FAKE, w=FAKE, M=64, N=64, K=128, alpha=1.0, ac=None, d=FAKE, dt=nv.OUT_BF16, ldd=64):
        return g(at, w, M, N, K, alpha, None, ac, d, dt, ldd, None, None, 0, None)
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
        return f(x, ldx, w, M, N, K, alpha, None, ac, y, ldy, None, ws, nws, None)
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
    assert q(FAKE, 4, 32, FAKE, FAKE, None, None, FAKE, QWS, None) == nv.ERR_NULL
    assert q(FAKE, 4, 24, FAKE, FAKE, FAKE, None, FAKE, QWS, None) == nv.ERR_SHAPE
    assert q(FAKE, 4, 32, FAKE, FAKE, FAKE, None, None, 0, None) == nv.ERR_WORKSPACE
    assert q(FAKE, 4, 32, FAKE, FAKE, FAKE, None, FAKE, 16, None) == nv.ERR_WORKSPACE
    assert q(ODD, 4, 32, FAKE, FAKE, FAKE, None, FAKE, QWS, None) == nv.ERR_ALIGN


def test_workspace_sizes():
    def heur_ws(op, M, N, K):   # the heuristic's config, whatever the tuned table holds
        c = nv.get_config(op, M, N, K, -256)
        return nv.lib().nvfp4_config_workspace_bytes(op, M, N, K, ctypes.byref(c))

    L = nv.lib()
    # W4A4: A in the prepared tile layout, rows rounded up to 32
    assert L.nvfp4_workspace_bytes(nv.OP_W4A4, 8192, 8192, 8192) == 8192 * 8192 * 9 // 16
    assert L.nvfp4_workspace_bytes(nv.OP_W4A4, 33, 64, 128) == 64 * 128 * 9 // 16
    assert L.nvfp4_workspace_bytes(nv.OP_W4A4, 0, 64, 128) == 0
    assert L.nvfp4_workspace_bytes(nv.OP_QUANTIZE, 8192, 0, 5120) == QWS   # any size: 12.25 KiB
    # W4A16 (no device here: the plan assumes 256 CUs). Decode (M <= 4) and the row kernel
    # (M <= 64, M <= 48 on weights of >= 256 row groups) need none; the fragment kernel's x
    # copy is roundup32(M) rows x K BF16.
    assert L.nvfp4_workspace_bytes(nv.OP_W4A16, 1, 34816, 5120) == 0
    assert L.nvfp4_workspace_bytes(nv.OP_W4A16, 4, 34816, 5120) == 0
    assert L.nvfp4_workspace_bytes(nv.OP_W4A16, 16, 34816, 5120) == 0
    assert L.nvfp4_workspace_bytes(nv.OP_W4A16, 24, 17408, 4160) == 0
    assert L.nvfp4_workspace_bytes(nv.OP_W4A16, 48, 34816, 5120) == 0
    assert heur_ws(nv.OP_W4A16, 64, 5120, 17408) == 0       # 160 row groups
    # the tuned table's 128 x 128 tiles there: 40 tiles split 6 ways, two 64 KiB slots per
    # workgroup, x through LDS
    assert L.nvfp4_workspace_bytes(nv.OP_W4A16, 64, 5120, 17408) == 240 * 2 * 64 * 1024
    assert L.nvfp4_workspace_bytes(nv.OP_W4A16, 49, 34816, 5120) == 64 * 5120 * 2
    assert L.nvfp4_workspace_bytes(nv.OP_W4A16, 64, 8192, 5120) == 64 * 5120 * 2   # 256 row groups
    # K past the row kernel's 32-bit weight offsets: the fragment kernel and its copy
    assert L.nvfp4_workspace_bytes(nv.OP_W4A16, 24, 64, (1 << 27) + 64) == 32 * ((1 << 27) + 64) * 2
    # M = 128 on 34816 x 5120: 136 tiles of 128 x 256, all split over 256 workgroups (two
    # 128 KiB partial slots each) in ranges of 42-43 chunks, short enough for x to go
    # through LDS: no copy of x
    assert L.nvfp4_workspace_bytes(nv.OP_W4A16, 128, 34816, 5120) == 256 * 2 * 128 * 1024
    # M = 1024 on 5120 x 17408: 80 tiles of 256 x 256, all split over 256 workgroups (two
    # 256 KiB slots each), then x for four 256-row tiles in fragment order
    assert heur_ws(nv.OP_W4A16, 1024, 5120, 17408) == 256 * 2 * 256 * 1024 + 1024 * 17408 * 2
    # the tuned table's 128 x 256 tiles there: 160 tiles all split over 256 workgroups (two
    # 128 KiB slots each) in 170-chunk ranges, x read from its fragment-order copy
    assert L.nvfp4_workspace_bytes(nv.OP_W4A16, 1024, 5120, 17408) == (256 * 2 * 128 * 1024
                                                                       + 1024 * 17408 * 2)
    # M = 1024 on 5120 x 5120 (128 x 256 tiles, 160 of them, all split into 50-chunk ranges):
    # x through LDS, the partials only
    assert heur_ws(nv.OP_W4A16, 1024, 5120, 5120) == 256 * 2 * 128 * 1024
    # the tuned table's 128 x 128 tiles there: 320 whole tiles, no split, x through LDS
    assert L.nvfp4_workspace_bytes(nv.OP_W4A16, 1024, 5120, 5120) == 0
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


def _golden_figures():
    import json
    with open(os.path.join(ROOT, "tests", "golden", "pages_figures.json")) as f:
        return json.load(f)


def test_get_config_heuristic_and_tile_counts():
    """The heuristic's tiles: 256 x 256 when they fill the CUs (8192^3: 1024 tiles, whole rounds,
    no tail), else 128 x 128. At 2048^2 that gives 16 x 16 = 256 tiles, the count the Colfax
    article gives for 128 x 128 tiles (section 'Version 6: 12 MMA Warps'); its 192 x 128 tile is
    not a shape of this library, so an explicit config asking for it is rejected."""
    c = nv.get_config(nv.OP_W4A4_TILED, 8192, 8192, 8192, 256)
    assert (c.kernel, c.tile_m, c.tile_n, c.tail, c.dynamic, c.num_cus, c.source) == \
        (nv.KERNEL_W4A4_TILES, 256, 256, nv.TAIL_NONE, 0, 256, nv.CONFIG_HEURISTIC)
    for case in _golden_figures()["tile_counts"]["cases"]:
        M, N = case["M"], case["N"]
        if case["tile_m"] == 128 and case["tile_n"] == 128:
            c = nv.get_config(nv.OP_W4A4_TILED, M, N, 2048, 256)
            assert (c.tile_m, c.tile_n) == (128, 128)
            assert -(-M // c.tile_m) * -(-N // c.tile_n) == case["tiles"]
        else:
            cfg = nv.make_config(nv.KERNEL_W4A4_TILES, case["tile_m"], case["tile_n"], num_cus=256)
            assert nv.lib().nvfp4_config_workspace_bytes(nv.OP_W4A4, M, N, 2048, ctypes.byref(cfg)) == 0
    # a last round of at most half the CUs: quadrants, or a two-way K split when K is long
    c = nv.get_config(nv.OP_W4A4_TILED, 8192, 16896, 5120, 256)   # 32 x 66 = 2112 tiles, 64 left over
    assert (c.tail, c.split_k, c.source) == (nv.TAIL_QUADRANTS, 0, nv.CONFIG_HEURISTIC)
    c = nv.get_config(nv.OP_W4A4_TILED, 8192, 5376, 17408, 256)   # 32 x 21 = 672 tiles, 160 left over
    assert c.tail == nv.TAIL_NONE
    c = nv.get_config(nv.OP_W4A4_TILED, 8192, 4608, 16384, 256)   # 32 x 18 = 576 tiles, 64 left over
    assert (c.tail, c.split_k) == (nv.TAIL_SPLIT, 2)
    c = nv.get_config(nv.OP_W4A16, 1, 5120, 5120, 256)
    assert c.kernel == nv.KERNEL_W4A16_DECODE
    # the heuristic's own choice (-256: no table); the tuned table may pick the row kernel
    assert nv.get_config(nv.OP_W4A16, 2, 5120, 5120, -256).kernel == nv.KERNEL_W4A16_DECODE
    assert nv.get_config(nv.OP_W4A16, 3, 5120, 5120, 256).kernel == nv.KERNEL_W4A16_SKINNY   # the row kernel
    c = nv.get_config(nv.OP_W4A16, 32, 5120, 5120, 256)
    assert c.kernel == nv.KERNEL_W4A16_SKINNY
    c = nv.get_config(nv.OP_W4A16, 1024, 34816, 5120, 256)
    assert (c.kernel, c.tile_m, c.tile_n) == (nv.KERNEL_W4A16_TILES, 256, 256)


def test_tuned_table_is_per_cu_count():
    """A tuned entry applies only on the CU count it was measured on (TileLang PR #3290,
    'Tests': the tuned table is not applied on another SM count)."""
    # 34816 x 5120 at M = 384: 128 x 256 tiles measured 20 % faster than the heuristic's 256 x 256
    tuned = nv.get_config(nv.OP_W4A16, 384, 34816, 5120, 256)
    heur = nv.get_config(nv.OP_W4A16, 384, 34816, 5120, -256)
    assert tuned.source == nv.CONFIG_TUNED and tuned.num_cus == 256
    assert (tuned.kernel, tuned.tile_m, tuned.tile_n) == (nv.KERNEL_W4A16_TILES, 128, 256)
    assert heur.source == nv.CONFIG_HEURISTIC and (heur.tile_m, heur.tile_n) == (256, 256)
    for cus in (304, 255, 80):
        c = nv.get_config(nv.OP_W4A16, 384, 34816, 5120, cus)
        assert c.source == nv.CONFIG_HEURISTIC and c.num_cus == cus
    # outside an entry's M range the heuristic applies on 256 CUs too
    assert nv.get_config(nv.OP_W4A16, 128, 34816, 5120, 256).source == nv.CONFIG_HEURISTIC


def test_configs_are_valid_for_every_shape():
    """Every config the library picks, for M = 1 .. 1024 on the decode layer shapes and the
    square sizes and on three CU counts, is one its own check accepts (a positive workspace
    size whenever the op needs one, and the same size through both queries)."""
    L = nv.lib()
    shapes = [(6144, 5120), (5120, 5120), (34816, 5120), (5120, 17408), (2048, 2048), (8192, 8192)]
    for cus in (256, 304, 80):
        for N, K in shapes:
            for M in (1, 2, 3, 4, 5, 8, 16, 17, 32, 33, 64, 65, 96, 128, 200, 256, 384, 512, 1000, 1024):
                for op in (nv.OP_W4A16, nv.OP_W4A4_TILED, nv.OP_W4A4):
                    c = nv.get_config(op, M, N, K, cus)
                    assert c.num_cus == cus
                    n = L.nvfp4_config_workspace_bytes(op, M, N, K, ctypes.byref(c))
                    if op == nv.OP_W4A4:
                        assert n >= L.nvfp4_tiled_activation_bytes(M, K) > 0, (op, M, N, K, cus)
                    if c.tail == nv.TAIL_SPLIT:
                        assert n >= c.split_k * 256 * 256 * 4 > 0


def test_explicit_config_checks():
    L = nv.lib()
    ws = L.nvfp4_config_workspace_bytes

    def w(op, M, N, K, **kw):
        return ws(op, M, N, K, ctypes.byref(nv.make_config(**kw)))
    # W4A4: 256 or 128 square tiles; tails and the dynamic schedule need 256 x 256 tiles
    assert w(nv.OP_W4A4_TILED, 4096, 4096, 4096, tile_m=256, tile_n=256, num_cus=256) == 0   # nothing to hold
    assert w(nv.OP_W4A4_TILED, 4096, 4096, 4096, tile_m=256, tile_n=256, dynamic=1, num_cus=256) == 256
    assert w(nv.OP_W4A4_TILED, 2048, 2048, 2048, tile_m=256, tile_n=256, tail=nv.TAIL_SPLIT, split_k=4,
             num_cus=256) == 64 * 4 * 256 * 256 * 4
    assert w(nv.OP_W4A4_TILED, 2048, 2048, 2048, tile_m=128, tile_n=128, tail=nv.TAIL_SPLIT, split_k=4,
             num_cus=256) == 0
    assert w(nv.OP_W4A4_TILED, 2048, 2048, 2048, tile_m=128, tile_n=128, dynamic=1, num_cus=256) == 0
    assert w(nv.OP_W4A4_TILED, 2048, 2048, 2048, tile_m=256, tile_n=256, tail=nv.TAIL_SPLIT, split_k=33,
             num_cus=256) == 0      # more ranges than K chunks
    assert w(nv.OP_W4A4_TILED, 2048, 2048, 2048, tile_m=256, tile_n=128, num_cus=256) == 0
    assert w(nv.OP_W4A4_TILED, 2048, 2048, 2048, kernel=nv.KERNEL_W4A16_TILES, tile_m=256, tile_n=256,
             num_cus=256) == 0
    # W4A16: the decode kernel while x fits its LDS, skinny up to M = 64, three tile shapes
    assert w(nv.OP_W4A16, 5, 5120, 5120, kernel=nv.KERNEL_W4A16_DECODE, num_cus=256) == 0
    assert w(nv.OP_W4A16, 65, 5120, 5120, kernel=nv.KERNEL_W4A16_SKINNY, num_cus=256) == 0
    assert w(nv.OP_W4A16, 24, 5120, 5120, kernel=nv.KERNEL_W4A16_SKINNY, num_cus=256) == 0      # row kernel
    assert w(nv.OP_W4A16, 56, 5120, 5120, kernel=nv.KERNEL_W4A16_SKINNY, num_cus=256) == 0      # 160 groups < CUs
    assert w(nv.OP_W4A16, 56, 5120, 5120, kernel=nv.KERNEL_W4A16_SKINNY, num_cus=64) == 64 * 5120 * 2  # fragment
    assert w(nv.OP_W4A16, 1, 5120, 5120, kernel=nv.KERNEL_W4A16_TILES, tile_m=256, tile_n=128, num_cus=256) == 0
    assert w(nv.OP_W4A16, 1, 5120, 5120, kernel=nv.KERNEL_AUTO, num_cus=256) == 0
    assert w(nv.OP_W4A16, 1, 5120, 5120, kernel=nv.KERNEL_W4A16_TILES, tile_m=128, tile_n=128, num_cus=256) > 0
