"""GPU parity of [G, K, N] block-FP8 (tiles per slice) against the CPU oracle."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import announce, assert_same, bits16, f32bits, u8

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [(3, 200, 136), (2, 128, 256), (4, 33, 8), (1, 130, 520),
                                   (8, 2048, 512)])
def test_gkn(gpu, orc, shape):
    G, K, N = shape
    xb = workloads.random_bf16((G * K, N), 17 * K + N).reshape(G, K, N)
    xb[0, :min(K, 128), :min(N, 128)] = 0             # one zero tile
    if G > 1:
        xb[1, 1, 1] = 0x7FC0                          # one NaN tile in slice 1
    announce(f"blockfp8 gkn {shape}")
    x = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).view(torch.bfloat16).cuda()
    q, S = gpu.blockfp8_quantize_gkn(x)
    dq = gpu.blockfp8_dequantize_gkn(q, S)
    torch.cuda.synchronize()
    oq, oS = orc.blockfp8_quantize_gkn(xb)
    assert_same("gkn q", u8(q), oq)
    assert_same("gkn S", f32bits(S), f32bits(oS))
    assert_same("gkn dq", bits16(dq), orc.blockfp8_dequantize_gkn(oq, oS))
