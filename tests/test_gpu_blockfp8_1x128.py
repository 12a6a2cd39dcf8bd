"""GPU parity of 1 x 128 block-FP8 (quantize with fused fake-quant, fake-quant
only, dequantize) against the CPU oracle, bit for bit."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import announce, assert_same, bits16, f32bits, to_dev_bf16, u8

pytestmark = pytest.mark.gpu


def check_1x128(gpu, orc, x_bits, name):
    announce(f"blockfp8 1x128 {name} {x_bits.shape}")
    x = to_dev_bf16(x_bits)
    q, S, fq = gpu.blockfp8_quantize_1x128(x, fake_quant=True)
    only = gpu.fp8_simulate_qat(x)
    torch.cuda.synchronize()
    oq, oS = orc.blockfp8_quantize_rect(x_bits, 1, 128)
    odq = orc.blockfp8_dequantize_rect(oq, oS, 1, 128)
    assert_same(f"{name} q", u8(q), oq)
    assert_same(f"{name} S", f32bits(S), f32bits(oS))
    assert_same(f"{name} fq", bits16(fq), odq)
    assert_same(f"{name} fake-quant only", bits16(only), odq)
    dq = gpu.blockfp8_dequantize_1x128(q, S)
    torch.cuda.synchronize()
    assert_same(f"{name} dequant", bits16(dq), odq)


@pytest.mark.parametrize("shape", [(64, 384), (33, 200), (1, 128), (17, 7168), (100, 8), (130, 1032)])
def test_1x128_shapes(gpu, orc, shape):
    check_1x128(gpu, orc, workloads.random_bf16(shape, 41 * shape[0] + shape[1]), f"s{shape}")


def test_1x128_edge_groups_and_division_paths(gpu, orc):
    """Zero, NaN, Inf and subnormal blocks; block maxima whose scale falls
    outside [2^-60, 2^60] (IEEE-division path) next to ordinary blocks."""
    rng = np.random.default_rng(6)
    x = workloads.random_bf16((40, 1024), 8)
    x[0, 0:128] = 0
    x[1, 128:256] = 0x8000
    x[2, 5] = 0x7FC0
    x[3, 300] = 0xFF80
    x[4, 0:128] = rng.integers(1, 0x80, 128)                       # bf16 subnormals only
    x[5, 0:128] = 0x0001                                            # min subnormal
    x[6, 128:256] = rng.integers(0x0080, 0x0400, 128)               # tiny normals: S < 2^-60
    x[7, 256:384] = rng.integers(0x7E00, 0x7F7F, 128)               # huge: S > 2^60
    x[8, 384:512] = 0x7F7F                                          # max finite everywhere
    x[9, 512:640] = np.where(np.arange(128) % 2 == 0, 0x43E0, 0xC3E0)  # +-448
    check_1x128(gpu, orc, x, "edge")


def test_1x128_act_16384_full(gpu, orc):
    """The [16384, 7168] activation, every output bit."""
    check_1x128(gpu, orc, workloads.act_16384(), "act_16384")


def test_1x128_dequant_arbitrary(gpu, orc):
    rng = np.random.default_rng(3)
    rows, cols = 64, 512
    q = rng.integers(0, 256, size=(rows, cols)).astype(np.uint8)
    q[:, :256] = np.arange(256, dtype=np.uint8)
    specials = np.array([0.0, 1e-45, 3e38, np.inf, np.nan, -1.0, 2.0 ** -130, 0.1], np.float32)
    S = rng.choice(specials, size=(rows, cols // 128)).astype(np.float32)
    S[::3] = rng.random((len(S[::3]), cols // 128)).astype(np.float32) * 4
    announce("blockfp8 1x128 dequant arbitrary")
    out = gpu.blockfp8_dequantize_1x128(torch.from_numpy(q).cuda(), torch.from_numpy(S).cuda())
    torch.cuda.synchronize()
    assert_same("1x128 dequant", bits16(out), orc.blockfp8_dequantize_rect(q, S, 1, 128))
