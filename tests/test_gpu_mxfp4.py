"""GPU parity of MXFP4 (quantize with fused fake-quant, fake-quant only,
dequantize) against the CPU oracle, byte for byte, through the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

import block_scaled_precision_mxfp8_amd as mxq
import pins
import workloads
from gpu_util import announce, assert_same, bits16, to_dev_bf16, u8

pytestmark = pytest.mark.gpu


def check_mxfp4(gpu, orc, x_bits, name):
    announce(f"mxfp4 {name} {x_bits.shape}")
    x = to_dev_bf16(x_bits)
    q, s, fq = gpu.mxfp4_quantize(x, fake_quant=True)
    q_only, s_only = gpu.mxfp4_quantize(x)          # the quantize-only launch (own tile order)
    only = gpu.mxfp4_simulate_qat(x)
    torch.cuda.synchronize()
    oq, os_ = orc.mxfp4_quantize(x_bits)
    ofq = orc.mxfp4_dequantize(oq, os_)
    assert_same(f"{name} q", u8(q), oq)
    assert_same(f"{name} scale", u8(s), os_)
    assert_same(f"{name} q (quantize only)", u8(q_only), oq)
    assert_same(f"{name} scale (quantize only)", u8(s_only), os_)
    assert_same(f"{name} fq", bits16(fq), ofq)
    assert_same(f"{name} fake-quant only", bits16(only), ofq)
    dq = gpu.mxfp4_dequantize(q, s)
    torch.cuda.synchronize()
    assert_same(f"{name} dequant", bits16(dq), ofq)


def test_mxfp4_mx_small(gpu, orc):
    check_mxfp4(gpu, orc, workloads.mx_small(), "mx_small")


def test_mxfp4_every_value_every_scale(gpu, orc):
    """Every (bf16 value, reachable scale byte) pair, 8.3 M elements."""
    x, _ = pins.mx4_sweep_input()
    n = x.shape[0] // 16 * 16
    check_mxfp4(gpu, orc, np.ascontiguousarray(x[:n].reshape(-1, 512)), "sweep512")


def test_mxfp4_nonfinite_zero_subnormal(gpu, orc):
    rng = np.random.default_rng(2)
    x = workloads.random_bf16((64, 256), 4)
    x[0, 0:32] = 0                                   # all zero
    x[1, 32:64] = 0x8000                             # all -0
    x[2, 0:32] = rng.integers(1, 0x80, 32)           # bf16 subnormals only (scale byte 0)
    x[2, 32:64] = rng.integers(0, 0x180, 32)         # amax exponent field <= 2: byte clamped at 0
    x[2, 64:96] = rng.integers(0x8000, 0x8180, 32)
    x[3, 5] = 0x7FC0                                 # NaN
    x[3, 6] = 0xBF80                                 # -1 beside it
    x[4, 40] = 0xFF80                                # -Inf
    x[5, 70] = 0x7F80                                # +Inf
    x[6, 100] = 0x7F7F                               # max finite bf16 (scale byte 252)
    x[7, 0:32] = 0x0001                              # min subnormal
    x[8, 0:32] = rng.integers(0, 0x10000, 32).astype(np.uint16) & 0x7FFF | 0x8000
    x[9, 0:32] = 0x40E0                              # 7.0 everywhere: saturates to 6 at scale 1
    check_mxfp4(gpu, orc, x, "edge")


@pytest.mark.parametrize("rows", [1, 31, 33, 97])
@pytest.mark.parametrize("cols", [32, 96, 544, 7168])
def test_mxfp4_ragged(gpu, orc, rows, cols):
    check_mxfp4(gpu, orc, workloads.random_bf16((rows, cols), 7 * rows + cols), f"ragged{rows}x{cols}")


def test_mxfp4_act_16384_full(gpu, orc):
    """The [16384, 7168] activation in the launch configuration the bench times."""
    check_mxfp4(gpu, orc, workloads.act_16384(), "act_16384")


def test_mxfp4_dequant_all_nibbles_all_scales(gpu, orc):
    """Row r: scale byte r for every one of the 16 nibbles (bytes 253, 254
    overflow bf16 for the large nibbles; 255 is NaN)."""
    nib = np.tile(np.arange(16, dtype=np.uint8), (256, 4))              # [256, 64]
    q = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)          # [256, 32]
    s = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 2, axis=1)  # [256, 2]
    announce("mxfp4 dequant all nibbles")
    out = gpu.mxfp4_dequantize(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda())
    torch.cuda.synchronize()
    assert_same("mxfp4 dequant", bits16(out), orc.mxfp4_dequantize(q, s))


def test_mxfp4_guard_bands(gpu, orc):
    """Outputs placed between 0xA5 guard bytes: nothing outside them is written."""
    rows, cols, G = 37, 96, 256
    xb = workloads.random_bf16((rows, cols), 99)
    announce("mxfp4 guard bands")
    x = to_dev_bf16(xb)
    qb = torch.full((2 * G + rows * cols // 2,), 0xA5, dtype=torch.uint8, device="cuda")
    sb = torch.full((2 * G + rows * cols // 32,), 0xA5, dtype=torch.uint8, device="cuda")
    fb = torch.full((2 * G + rows * cols,), 0x5A5A, dtype=torch.int16, device="cuda")
    lib = gpu.load()
    st = lib.mxfp4_quantize(ctypes.c_void_p(x.data_ptr()), rows, cols,
                            ctypes.c_void_p(qb.data_ptr() + G), ctypes.c_void_p(sb.data_ptr() + G),
                            ctypes.c_void_p(fb.data_ptr() + 2 * G),
                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == mxq.MXQ_OK
    torch.cuda.synchronize()
    oq, os_ = orc.mxfp4_quantize(xb)
    qh, sh, fh = u8(qb), u8(sb), fb.cpu().numpy().view(np.uint16)
    for h, n, fill in ((qh, oq.size, 0xA5), (sh, os_.size, 0xA5), (fh, rows * cols, 0x5A5A)):
        assert np.all(h[:G] == fill) and np.all(h[G + n:] == fill)
    assert_same("guard q", qh[G:G + oq.size].reshape(oq.shape), oq)
    assert_same("guard s", sh[G:G + os_.size].reshape(os_.shape), os_)
    assert_same("guard fq", fh[G:G + rows * cols].reshape(rows, cols), orc.mxfp4_dequantize(oq, os_))


def test_mxfp4_simulate_qat_keeps_shape(gpu, orc):
    xb = workloads.random_bf16((6 * 8, 64), 5)
    x = to_dev_bf16(xb).view(6, 8, 64)
    out = gpu.mxfp4_simulate_qat(x)
    torch.cuda.synchronize()
    assert out.shape == (6, 8, 64)
    assert_same("simulate_qat 3-D", bits16(out.reshape(48, 64)), orc.mxfp4_fake_quant(xb))
