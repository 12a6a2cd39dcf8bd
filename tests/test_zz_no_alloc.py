"""The allocation-free NVFP4 entry point (nvfp4_quantize_noalloc, amax
partials in the library's own per-GPU array) against the workspace entry
point nvfp4_quantize, through the C ABI, bit for bit: two calls in a row on
one GPU, the second on a smaller input, so the second runs on the array the
first left behind."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from gpu_util import announce, assert_same, f32bits, to_dev_bf16, u8

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _outs(rows, cols, dev):
    return (torch.full((rows, cols // 2), 0xA5, dtype=torch.uint8, device=dev),
            torch.full((rows, cols // 16), 0xA5, dtype=torch.uint8, device=dev),
            torch.full((1,), float("nan"), dtype=torch.float32, device=dev))


def test_nvfp4_noalloc_equals_workspace_entry(gpu, orc):
    lib = gpu.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ws = torch.empty((lib.nvfp4_workspace_size(),), dtype=torch.uint8, device="cuda")
    cases = [((4097, 7168), 9100, 3.0), ((33, 48), 9101, 0.25)]   # the second smaller
    for k, (shape, seed, std) in enumerate(cases):
        rows, cols = shape
        xb = workloads.random_bf16(shape, seed, std=std)
        xb[rows // 2, cols // 3] = workloads.bf16_from_float(1000.0 * std)   # the global amax
        x = to_dev_bf16(xb)
        announce(f"nvfp4_quantize_noalloc call {k} {shape}")
        q1, s1, g1 = _outs(rows, cols, "cuda")
        assert lib.nvfp4_quantize(_p(x), rows, cols, _p(q1), _p(s1), _p(g1), _p(ws), ws.numel(),
                                  stream) == 0
        q2, s2, g2 = _outs(rows, cols, "cuda")
        assert lib.nvfp4_quantize_noalloc(_p(x), rows, cols, _p(q2), _p(s2), _p(g2), stream) == 0
        torch.cuda.synchronize()
        assert_same(f"call {k} g", f32bits(g2), f32bits(g1))
        assert_same(f"call {k} s", u8(s2), u8(s1))
        assert_same(f"call {k} q", u8(q2), u8(q1))
        oq, os_, og = orc.nvfp4_quantize(xb)
        assert_same(f"call {k} g vs oracle", f32bits(g2), f32bits(og))
        assert_same(f"call {k} q vs oracle", u8(q2), oq)
        assert_same(f"call {k} s vs oracle", u8(s2), os_)


def test_nvfp4_noalloc_binding_and_empty(gpu, orc):
    xb = workloads.random_bf16((64, 512), 9102)
    announce("nvfp4_quantize_noalloc binding")
    q, s, g = gpu.nvfp4_quantize_noalloc(to_dev_bf16(xb))
    torch.cuda.synchronize()
    oq, os_, og = orc.nvfp4_quantize(xb)
    assert_same("binding q", u8(q), oq)
    assert_same("binding s", u8(s), os_)
    assert_same("binding g", f32bits(g), f32bits(og))
    lib = gpu.load()
    assert lib.nvfp4_quantize_noalloc(None, 0, 64, None, None, None, None) == 0
