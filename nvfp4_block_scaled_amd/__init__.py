"""Python binding of libnvfp4.so, the gfx950 NVFP4 block-scaled GEMM library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/nvfp4.h. torch supplies device
memory and the current stream. There is no CPU fallback: without the built
library every call raises.

Entry points (same names as the C ABI):
  nvfp4_prepare_weight(w_codes, w_scales, scale_kind="e4m3", out=None, bad_count=None, validate=True)
  nvfp4_gemm_w4a4(a_codes, a_scales, w_prep, N, K, alpha=1.0, alpha_dev=None, out_dtype="bf16", out=None,
                  ws=None, alpha_col=None)
  nvfp4_gemm_w4a16(x, w_prep, N, K, alpha=1.0, alpha_dev=None, out=None, ws=None, alpha_col=None)
  nvfp4_quantize(x, codes=None, scales=None, g=None, inv_g=None, ws=None)
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DTYPE, ERR_VALUE, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_HIP = range(9)
SCALE_UE4M3, SCALE_E4M3 = 0, 1
OUT_F32, OUT_BF16 = 0, 1
OP_W4A4, OP_W4A16, OP_QUANTIZE, OP_W4A4_TILED = 0, 1, 2, 3
KERNEL_AUTO, KERNEL_W4A4_TILES, KERNEL_W4A16_DECODE, KERNEL_W4A16_SKINNY, KERNEL_W4A16_TILES = range(5)
TAIL_NONE, TAIL_QUADRANTS, TAIL_SPLIT = range(3)
CONFIG_HEURISTIC, CONFIG_TUNED, CONFIG_EXPLICIT = range(3)


class Config(ctypes.Structure):
    """nvfp4_config: a GEMM launch configuration (see include/nvfp4.h)."""
    _fields_ = [(n, ctypes.c_int32) for n in
                ("kernel", "tile_m", "tile_n", "tail", "split_k", "dynamic", "num_cus", "source")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}

    def __repr__(self):
        return f"Config({self.as_dict()})"


_CFG = ctypes.POINTER(Config)

# C signatures: (name, restype, argtypes)
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIGS = [
    ("nvfp4_init", ctypes.c_int, [ctypes.c_int]),
    ("nvfp4_status_str", ctypes.c_char_p, [ctypes.c_int]),
    ("nvfp4_prepared_weight_bytes", ctypes.c_size_t, [_I64, _I64]),
    ("nvfp4_workspace_bytes", ctypes.c_size_t, [ctypes.c_int, _I64, _I64, _I64]),
    ("nvfp4_get_config", ctypes.c_int, [ctypes.c_int, _I64, _I64, _I64, ctypes.c_int, _CFG]),
    ("nvfp4_config_workspace_bytes", ctypes.c_size_t, [ctypes.c_int, _I64, _I64, _I64, _CFG]),
    ("nvfp4_workspace_init", ctypes.c_int, [_P, ctypes.c_size_t, _P]),
    ("nvfp4_prepare_weight", ctypes.c_int, [_P, _P, ctypes.c_int, _I64, _I64, _P, _P, _P]),
    ("nvfp4_gemm_w4a4", ctypes.c_int,
     [_P, _P, _P, _I64, _I64, _I64, ctypes.c_float, _P, _P, _P, ctypes.c_int, _I64, _CFG, _P, ctypes.c_size_t, _P]),
    ("nvfp4_tiled_activation_bytes", ctypes.c_size_t, [_I64, _I64]),
    ("nvfp4_tile_activation", ctypes.c_int, [_P, _P, _I64, _I64, _P, _P]),
    ("nvfp4_gemm_w4a4_tiled", ctypes.c_int,
     [_P, _P, _I64, _I64, _I64, ctypes.c_float, _P, _P, _P, ctypes.c_int, _I64, _CFG, _P, ctypes.c_size_t, _P]),
    ("nvfp4_gemm_w4a16", ctypes.c_int,
     [_P, _I64, _P, _I64, _I64, _I64, ctypes.c_float, _P, _P, _P, _I64, _CFG, _P, ctypes.c_size_t, _P]),
    ("nvfp4_quantize", ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    ("nvfp4_quantize_tiled", ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    ("nvfp4_quantize_two_pass_tiled", ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    ("nvfp4_gemm_w4a4_two_pass_tiled", ctypes.c_int,
     [_P, _P, _I64, _I64, _I64, ctypes.c_float, _P, _P, _P, ctypes.c_int, _I64, _CFG, _P, ctypes.c_size_t, _P]),
    ("nvfp4_quantize_tiled_noalloc", ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _P]),
]
EXPORTED = [s[0] for s in _SIGS]

_lib = None


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m nvfp4_block_scaled_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, res, args in _SIGS:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class NVFP4Error(RuntimeError):
    pass


def _check(status):
    if status == OK:
        return
    msg = lib().nvfp4_status_str(status).decode()
    if status == ERR_DTYPE:
        raise TypeError(msg)
    if status in (ERR_SHAPE, ERR_ALIGN, ERR_VALUE, ERR_WORKSPACE, ERR_NULL):
        raise ValueError(msg)
    raise NVFP4Error(msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _on_device(t, name):
    """t must be a tensor on the current HIP device (the library launches on the current
    device's current stream, and a host pointer handed to a kernel would fault the GPU)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, not on the current device cuda:{torch.cuda.current_device()}")
    return t


def _dev(t, name):
    _on_device(t, name)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _nbytes(t):
    return t.numel() * t.element_size()


def _f32_dev(t, name, n=1):
    """None, or a contiguous float32 device tensor of at least n values."""
    if t is None:
        return None
    _dev(t, name)
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    if t.numel() < n:
        raise ValueError(f"{name} must hold at least {n} float32 values")
    return t


def _byte_buffer(t, name, nbytes):
    """A caller-supplied contiguous uint8 device buffer of at least nbytes bytes."""
    _dev(t, name)
    if t.dtype != torch.uint8:
        raise TypeError(f"{name} must be uint8")
    if t.numel() < nbytes:
        raise ValueError(f"{name} holds {t.numel()} bytes, {nbytes} are needed")
    return t


def _workspace_arg(ws, need, name="ws"):
    """(pointer, bytes) of a caller workspace; the library checks the size against `need`."""
    if ws is None:
        return None, 0
    _dev(ws, name)
    if _nbytes(ws) < need:
        raise ValueError(f"{name} holds {_nbytes(ws)} bytes, {need} are needed")
    return _ptr(ws), _nbytes(ws)


def _out_matrix(out, M, N, dtype, name="out"):
    """A caller-supplied output: device tensor [M][>= N] of dtype with unit column stride and
    rows at least N elements apart (a column slice of a wider matrix is fine)."""
    _on_device(out, name)
    if out.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}")
    if out.dim() != 2 or out.shape[0] != M or out.shape[1] < N:
        raise ValueError(f"{name} must be [{M}][>={N}], got {tuple(out.shape)}")
    if M > 0 and (out.stride(1) != 1 or (M > 1 and out.stride(0) < N)):
        raise ValueError(f"{name} needs unit column stride and a row stride >= {N}")
    return out


def init(device=None):
    """Per-device set-up (optional; the first call on a device does it too). Call it before
    capturing a graph whose first library call would otherwise be inside the capture."""
    if device is None:
        device = torch.cuda.current_device()
    elif isinstance(device, torch.device):
        device = device.index if device.index is not None else torch.cuda.current_device()
    _check(lib().nvfp4_init(int(device)))


def prepared_weight_bytes(N, K):
    return int(lib().nvfp4_prepared_weight_bytes(N, K))


def workspace_bytes(op, M, N, K, config=None):
    """Workspace bytes of a call with `config` (None: the library's choice)."""
    if config is None:
        return int(lib().nvfp4_workspace_bytes(op, M, N, K))
    return int(lib().nvfp4_config_workspace_bytes(op, M, N, K, ctypes.byref(_config(config))))


def get_config(op, M, N, K, num_cus=0):
    """The configuration a call without one uses (tuned table entry or heuristic) on a device
    with num_cus CUs (0: the current device's)."""
    c = Config()
    _check(lib().nvfp4_get_config(op, M, N, K, num_cus, ctypes.byref(c)))
    return c


def make_config(kernel=KERNEL_AUTO, tile_m=0, tile_n=0, tail=TAIL_NONE, split_k=0, dynamic=0, num_cus=0):
    """An explicit configuration for the GEMM calls' `config` argument."""
    return Config(kernel, tile_m, tile_n, tail, split_k, dynamic, num_cus, CONFIG_EXPLICIT)


def _config(config):
    if config is None:
        return None
    if isinstance(config, Config):
        return config
    if isinstance(config, dict):
        return make_config(**config)
    raise TypeError("config must be a Config, a dict of its fields, or None")


def _cfg_arg(config):
    c = _config(config)
    return None if c is None else ctypes.byref(c)


def workspace(op, M, N, K, device="cuda", config=None):
    """Allocate and zero a workspace for (op, M, N, K[, config]); None when the call needs none."""
    n = workspace_bytes(op, M, N, K, config)
    if n == 0:
        return None
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    _check(lib().nvfp4_workspace_init(_ptr(ws), n, _stream()))
    return ws


def _u8(t, name):
    t = _dev(t, name)
    if t.dtype in (torch.uint8, torch.int8):
        return t.view(torch.uint8)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    raise TypeError(f"{name} must hold bytes (uint8/int8/float8_e4m3fn), got {t.dtype}")


def nvfp4_prepare_weight(w_codes, w_scales, scale_kind="e4m3", out=None, bad_count=None, validate=True):
    """Prepared copy of a weight ([N][K/2] packed codes, [N][K/16] scale bytes).

    Returns (w_prep uint8 tensor, bad_count int32 device tensor). With validate (the default)
    the call synchronises once and raises ValueError when any scale byte is NaN (or, for
    UE4M3, has its sign bit set); validate=False leaves the count to the caller."""
    w_codes = _u8(w_codes, "w_codes")
    w_scales = _u8(w_scales, "w_scales")
    if w_codes.dim() != 2 or w_scales.dim() != 2:
        raise ValueError("w_codes and w_scales must be 2-D")
    N, K2 = w_codes.shape
    K = 2 * K2
    if tuple(w_scales.shape) != (N, K // 16):
        raise ValueError("w_scales must be [N][K/16]")
    kind = {"e4m3": SCALE_E4M3, "ue4m3": SCALE_UE4M3}.get(scale_kind)
    if kind is None:
        raise TypeError("scale_kind must be 'e4m3' or 'ue4m3'")
    nbytes = prepared_weight_bytes(N, K)
    if nbytes == 0:
        raise ValueError("N % 32 == 0 and K % 64 == 0 are required")
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=w_codes.device)
    else:
        _byte_buffer(out, "out", nbytes)
    if bad_count is None:
        bad_count = torch.empty(1, dtype=torch.int32, device=w_codes.device)
    else:
        _dev(bad_count, "bad_count")
        if bad_count.dtype != torch.int32 or bad_count.numel() < 1:
            raise TypeError("bad_count must be an int32 device tensor")
    _check(lib().nvfp4_prepare_weight(_ptr(w_codes), _ptr(w_scales), kind, N, K, _ptr(out), _ptr(bad_count),
                                      _stream()))
    if validate:
        n_bad = int(bad_count.item())        # synchronises the current stream
        if n_bad:
            raise ValueError(f"{n_bad} scale bytes are NaN or invalid for {scale_kind}")
    return out, bad_count


def _check_alpha_col(alpha_col, N):
    """A per-column scale: None, or a contiguous float32 device tensor of N values."""
    if alpha_col is None:
        return None
    if not isinstance(alpha_col, torch.Tensor) or alpha_col.dtype != torch.float32 or not alpha_col.is_cuda:
        raise TypeError("alpha_col must be a float32 device tensor")
    _dev(alpha_col, "alpha_col")
    if alpha_col.dim() != 1 or alpha_col.shape[0] != N:
        raise ValueError("alpha_col must be a contiguous [N] tensor")
    return alpha_col


def _out_dtype(out_dtype):
    od = {"bf16": (OUT_BF16, torch.bfloat16), "f32": (OUT_F32, torch.float32)}.get(out_dtype)
    if od is None:
        raise TypeError("out_dtype must be 'bf16' or 'f32'")
    return od


def _w_prep(w_prep, N, K):
    w_prep = _u8(w_prep, "w_prep")
    if w_prep.numel() != prepared_weight_bytes(N, K):
        raise ValueError("w_prep does not match (N, K)")
    return w_prep


def _ld(out, M, N):
    """Leading dimension passed for out: its row stride (any value serves a single row)."""
    return out.stride(0) if M > 1 else N


def _gemm_out(out, M, N, dtype, device):
    if out is None:
        return torch.empty((M, N), dtype=dtype, device=device)
    return _out_matrix(out, M, N, dtype)


def nvfp4_gemm_w4a4(a_codes, a_scales, w_prep, N, K, alpha=1.0, alpha_dev=None, out_dtype="bf16", out=None, ws=None,
                    alpha_col=None, config=None):
    a_codes = _u8(a_codes, "a_codes")
    a_scales = _u8(a_scales, "a_scales")
    M = a_codes.shape[0] if a_codes.dim() == 2 else 0
    if a_codes.dim() != 2 or a_codes.shape[1] * 2 != K or tuple(a_scales.shape) != (M, K // 16):
        raise ValueError("a_codes must be [M][K/2] and a_scales [M][K/16]")
    w_prep = _w_prep(w_prep, N, K)
    code, dtype = _out_dtype(out_dtype)
    out = _gemm_out(out, M, N, dtype, a_codes.device)
    alpha_dev = _f32_dev(alpha_dev, "alpha_dev")
    alpha_col = _check_alpha_col(alpha_col, N)
    need = workspace_bytes(OP_W4A4, M, N, K, config)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=a_codes.device)
    wsp, nws = _workspace_arg(ws, need)
    _check(lib().nvfp4_gemm_w4a4(_ptr(a_codes), _ptr(a_scales), _ptr(w_prep), M, N, K, float(alpha), _ptr(alpha_dev),
                                 _ptr(alpha_col), _ptr(out), code, _ld(out, M, N), _cfg_arg(config), wsp, nws,
                                 _stream()))
    return out


def nvfp4_tile_activation(a_codes, a_scales, out=None):
    """A ([M][K/2] codes, [M][K/16] scales) -> the tile layout (uint8, nvfp4_tiled_activation_bytes)."""
    a_codes = _u8(a_codes, "a_codes")
    a_scales = _u8(a_scales, "a_scales")
    if a_codes.dim() != 2 or a_scales.dim() != 2 or a_scales.shape != (a_codes.shape[0], a_codes.shape[1] // 8):
        raise ValueError("a_codes must be [M][K/2] and a_scales [M][K/16]")
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    n = int(lib().nvfp4_tiled_activation_bytes(M, K))
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=a_codes.device)
    else:
        _byte_buffer(out, "out", n)
    _check(lib().nvfp4_tile_activation(_ptr(a_codes), _ptr(a_scales), M, K, _ptr(out), _stream()))
    return out


def nvfp4_gemm_w4a4_tiled(a_tiled, M, w_prep, N, K, alpha=1.0, alpha_dev=None, out_dtype="bf16", out=None,
                          alpha_col=None, config=None, ws=None):
    """nvfp4_gemm_w4a4 on an activation already in the tile layout (nvfp4_tile_activation).

    ws: the K-split / scheduler workspace (workspace_bytes(OP_W4A4_TILED, M, N, K, config)); when
    None it is allocated for an explicit config, and left out otherwise (the library then runs its
    choice without one)."""
    a_tiled = _u8(a_tiled, "a_tiled")
    if a_tiled.numel() < int(lib().nvfp4_tiled_activation_bytes(M, K)):
        raise ValueError("a_tiled is smaller than nvfp4_tiled_activation_bytes(M, K)")
    w_prep = _w_prep(w_prep, N, K)
    code, dtype = _out_dtype(out_dtype)
    out = _gemm_out(out, M, N, dtype, a_tiled.device)
    alpha_dev = _f32_dev(alpha_dev, "alpha_dev")
    alpha_col = _check_alpha_col(alpha_col, N)
    need = workspace_bytes(OP_W4A4_TILED, M, N, K, config)
    if ws is None and need > 0 and config is not None:
        ws = torch.empty(need, dtype=torch.uint8, device=a_tiled.device)
    wsp, nws = _workspace_arg(ws, need)
    _check(lib().nvfp4_gemm_w4a4_tiled(_ptr(a_tiled), _ptr(w_prep), M, N, K, float(alpha), _ptr(alpha_dev),
                                       _ptr(alpha_col), _ptr(out), code, _ld(out, M, N), _cfg_arg(config), wsp, nws,
                                       _stream()))
    return out


def nvfp4_gemm_w4a16(x, w_prep, N, K, alpha=1.0, alpha_dev=None, out=None, ws=None, alpha_col=None, config=None):
    _on_device(x, "x")
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError("x must be [M][K]")
    if x.shape[0] > 0 and (x.stride(1) != 1 or x.data_ptr() % 16 != 0 or
                           (x.shape[0] > 1 and (x.stride(0) % 8 != 0 or x.stride(0) < K))):
        x = x.contiguous().clone()          # misaligned or strided activations are copied (one new allocation)
    M = x.shape[0]
    w_prep = _w_prep(w_prep, N, K)
    out = _gemm_out(out, M, N, torch.bfloat16, x.device)
    alpha_dev = _f32_dev(alpha_dev, "alpha_dev")
    alpha_col = _check_alpha_col(alpha_col, N)
    need = workspace_bytes(OP_W4A16, M, N, K, config)
    if ws is None and need > 0:
        ws = workspace(OP_W4A16, M, N, K, x.device, config)
    wsp, nws = _workspace_arg(ws, need)
    ldx = x.stride(0) if M > 1 else K
    _check(lib().nvfp4_gemm_w4a16(_ptr(x), ldx, _ptr(w_prep), M, N, K, float(alpha), _ptr(alpha_dev),
                                  _ptr(alpha_col), _ptr(out), _ld(out, M, N), _cfg_arg(config), wsp, nws, _stream()))
    return out


def _quantize_inputs(x, K_mult):
    x = _dev(x, "x")
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    if x.dim() != 2 or x.shape[1] % K_mult != 0:
        raise ValueError(f"x must be [rows][K] with K % {K_mult} == 0")
    return x


def _scalar_outs(g, inv_g, dev):
    g = torch.empty(1, dtype=torch.float32, device=dev) if g is None else _f32_dev(g, "g")
    inv_g = torch.empty(1, dtype=torch.float32, device=dev) if inv_g is None else _f32_dev(inv_g, "inv_g")
    return g, inv_g


def _quantize_ws(ws, rows, K, dev):
    need = workspace_bytes(OP_QUANTIZE, rows, 0, K)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    return _workspace_arg(ws, need)


def nvfp4_quantize(x, codes=None, scales=None, g=None, inv_g=None, ws=None):
    """BF16 [rows][K] -> (codes [rows][K/2] uint8, scales [rows][K/16] uint8, g, inv_g) on the device."""
    x = _quantize_inputs(x, 16)
    rows, K = x.shape
    dev = x.device
    if codes is None:
        codes = torch.empty((rows, K // 2), dtype=torch.uint8, device=dev)
    else:
        _byte_buffer(codes, "codes", rows * (K // 2))
    if scales is None:
        scales = torch.empty((rows, K // 16), dtype=torch.uint8, device=dev)
    else:
        _byte_buffer(scales, "scales", rows * (K // 16))
    g, inv_g = _scalar_outs(g, inv_g, dev)
    wsp, nws = _quantize_ws(ws, rows, K, dev)
    _check(lib().nvfp4_quantize(_ptr(x), rows, K, _ptr(codes), _ptr(scales), _ptr(g), _ptr(inv_g), wsp, nws,
                                _stream()))
    return codes, scales, g, inv_g


def nvfp4_quantize_tiled(x, out=None, g=None, inv_g=None, ws=None):
    """BF16 [rows][K] -> (activation in the tile layout (uint8), g, inv_g): nvfp4_quantize with its
    output written straight into the layout nvfp4_gemm_w4a4_tiled reads."""
    x = _quantize_inputs(x, 64)
    rows, K = x.shape
    dev = x.device
    n = int(lib().nvfp4_tiled_activation_bytes(rows, K))
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=dev)
    else:
        _byte_buffer(out, "out", n)
    g, inv_g = _scalar_outs(g, inv_g, dev)
    wsp, nws = _quantize_ws(ws, rows, K, dev)
    _check(lib().nvfp4_quantize_tiled(_ptr(x), rows, K, _ptr(out), _ptr(g), _ptr(inv_g), wsp, nws, _stream()))
    return out, g, inv_g


def nvfp4_quantize_tiled_noalloc(x, out, g, inv_g=None):
    """nvfp4_quantize_tiled with no workspace and no allocation: the caller passes every output
    (out: nvfp4_tiled_activation_bytes(rows, K) uint8; g and inv_g: float32 [1]); the library
    uses a static device array of its own for the quantizer's scratch."""
    x = _quantize_inputs(x, 64)
    rows, K = x.shape
    _byte_buffer(out, "out", int(lib().nvfp4_tiled_activation_bytes(rows, K)))
    if g is None:
        raise ValueError("g is required")
    _f32_dev(g, "g")
    _f32_dev(inv_g, "inv_g")
    _check(lib().nvfp4_quantize_tiled_noalloc(_ptr(x), rows, K, _ptr(out), _ptr(g), _ptr(inv_g), _stream()))
    return out, g, inv_g


def nvfp4_quantize_two_pass_tiled(x, out=None, g=None, inv_g=None, ws=None):
    """BF16 [rows][K] -> (two-pass activation in the tile layout of [rows][2K] (uint8), g, inv_g)."""
    x = _quantize_inputs(x, 64)
    rows, K = x.shape
    dev = x.device
    n = int(lib().nvfp4_tiled_activation_bytes(rows, 2 * K))
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=dev)
    else:
        _byte_buffer(out, "out", n)
    g, inv_g = _scalar_outs(g, inv_g, dev)
    wsp, nws = _quantize_ws(ws, rows, K, dev)
    _check(lib().nvfp4_quantize_two_pass_tiled(_ptr(x), rows, K, _ptr(out), _ptr(g), _ptr(inv_g), wsp, nws,
                                               _stream()))
    return out, g, inv_g


def nvfp4_gemm_w4a4_two_pass_tiled(a2_tiled, M, w_prep, N, K, alpha=1.0, alpha_dev=None, out_dtype="bf16", out=None,
                                   alpha_col=None, config=None, ws=None):
    """D = alpha (A1 + A2) W^T on a two-pass activation (nvfp4_quantize_two_pass_tiled, K per pass)."""
    a2_tiled = _u8(a2_tiled, "a2_tiled")
    if a2_tiled.numel() < int(lib().nvfp4_tiled_activation_bytes(M, 2 * K)):
        raise ValueError("a2_tiled is smaller than nvfp4_tiled_activation_bytes(M, 2K)")
    w_prep = _w_prep(w_prep, N, K)
    code, dtype = _out_dtype(out_dtype)
    out = _gemm_out(out, M, N, dtype, a2_tiled.device)
    alpha_dev = _f32_dev(alpha_dev, "alpha_dev")
    alpha_col = _check_alpha_col(alpha_col, N)
    need = workspace_bytes(OP_W4A4_TILED, M, N, 2 * K, config)
    if ws is None and need > 0 and config is not None:
        ws = torch.empty(need, dtype=torch.uint8, device=a2_tiled.device)
    wsp, nws = _workspace_arg(ws, need)
    _check(lib().nvfp4_gemm_w4a4_two_pass_tiled(_ptr(a2_tiled), _ptr(w_prep), M, N, K, float(alpha),
                                                _ptr(alpha_dev), _ptr(alpha_col), _ptr(out), code, _ld(out, M, N),
                                                _cfg_arg(config), wsp, nws, _stream()))
    return out
