"""The quantizer entry point that allocates nothing (nvfp4_quantize_tiled_noalloc), for callers
that cannot allocate: called through the C ABI, its bytes and global scale must equal those of
nvfp4_quantize_tiled (which takes a caller workspace) on the same input, on two calls in a row,
the second with a smaller input, and match the oracle's quantization."""
import ctypes

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_amd as nv
import synth
from gpu_helpers import dev, host
from oracle import prepared, quantize

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _noalloc(x):
    """One call of the no-alloc entry through the C ABI on fresh output buffers."""
    rows, K = x.shape
    n = int(nv.lib().nvfp4_tiled_activation_bytes(rows, K))
    out = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")        # garbage the call must overwrite
    g = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    ig = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    st = nv.lib().nvfp4_quantize_tiled_noalloc(_p(x), rows, K, _p(out), _p(g), _p(ig),
                                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == nv.OK, nv.lib().nvfp4_status_str(st)
    return out, g, ig


def test_noalloc_quantize_matches_workspace_entry_twice():
    assert nv.lib().nvfp4_init(torch.cuda.current_device()) == nv.OK
    # first call: a large activation; second: a smaller one with a smaller maximum, so a stale
    # tensor maximum left in the scratch by the first call would show in g and in every byte
    cases = [synth.normal_bf16(901, 1000, 5120), synth.normal_bf16(902, 77, 320, std=0.01)]
    for x_bits in cases:
        xd = dev(x_bits).view(torch.bfloat16)
        a, g, ig = _noalloc(xd)
        b, g2, ig2 = nv.nvfp4_quantize_tiled(xd)
        torch.cuda.synchronize()
        assert torch.equal(a, b), "no-alloc bytes differ from nvfp4_quantize_tiled"
        assert torch.equal(g, g2) and torch.equal(ig, ig2)
        c_ref, s_ref, g_ref, _ = quantize.quantize(x_bits)
        assert np.float32(g.item()) == g_ref
        rows, K = x_bits.shape
        Mp = -(-rows // 32) * 32
        c_pad = np.zeros((Mp, K // 2), np.uint8)
        s_pad = np.zeros((Mp, K // 16), np.uint8)
        c_pad[:rows], s_pad[:rows] = c_ref, s_ref
        ref, _ = prepared.prepare_weight(c_pad, s_pad, "ue4m3")
        np.testing.assert_array_equal(host(a), ref)


def test_noalloc_quantize_rejects_bad_arguments():
    L = nv.lib()
    x = torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty(int(L.nvfp4_tiled_activation_bytes(64, 128)), dtype=torch.uint8, device="cuda")
    g = torch.empty(1, dtype=torch.float32, device="cuda")
    assert L.nvfp4_quantize_tiled_noalloc(_p(x), 64, 96, _p(out), _p(g), None, None) == nv.ERR_SHAPE
    assert L.nvfp4_quantize_tiled_noalloc(_p(x), 64, 128, _p(out), None, None, None) == nv.ERR_NULL
    assert L.nvfp4_quantize_tiled_noalloc(None, 64, 128, _p(out), _p(g), None, None) == nv.ERR_NULL
    assert L.nvfp4_quantize_tiled_noalloc(ctypes.c_void_p(x.data_ptr() + 2), 64, 128, _p(out), _p(g), None,
                                          None) == nv.ERR_ALIGN
