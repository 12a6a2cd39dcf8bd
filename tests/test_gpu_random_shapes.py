"""Seeded random shapes through every single-tensor entry point, against the
oracle byte for byte.  Row counts run from 1 to 700 (partial 32-row groups,
16-row tiles and 128-row bands), column counts from one group to 2112
(partial 512-, 256- and 128-column tiles).  The MX and block-FP8 inputs hold
one NaN, one -Inf and one all-zero 32-element group each, at seeded places;
the NVFP4 inputs stay finite, since one non-finite element makes its whole
tensor NaN.  The dequantizers read the GPU codes; their expected values come
from the oracle's codes, shown equal to those first."""
import numpy as np
import pytest

import workloads
from gpu_util import announce, assert_same, bits16, f32bits, to_dev_bf16, u8

pytestmark = pytest.mark.gpu


def _shapes(n, step, seed):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 701)), int(step * rng.integers(1, 2112 // step + 1)))
            for _ in range(n)]


MX_SHAPES = _shapes(12, 32, 101)
NV_SHAPES = _shapes(8, 16, 202)


def _mx_input(shape, seed):
    x = workloads.random_bf16(shape, seed, std=2.0)
    rng = np.random.default_rng(seed + 1)
    rows, cols = shape
    r = rng.integers(0, rows, 3)
    c = rng.integers(0, cols, 3)
    x[r[0], c[0]] = 0x7FC0                       # NaN
    x[r[1], c[1]] = 0xFF80                       # -Inf
    g0 = (int(c[2]) // 32) * 32
    x[r[2], g0:g0 + 32] = 0                      # an all-zero row group
    return x


@pytest.mark.parametrize("k,shape", list(enumerate(MX_SHAPES)))
def test_random_shape_mxfp8(gpu, orc, k, shape):
    xb = _mx_input(shape, 1000 + k)
    x = to_dev_bf16(xb)
    name = f"mx{shape}"
    announce(f"random shape MXFP8 {shape}")
    oqr, osr = orc.mxfp8_quantize_rowwise(xb)
    oqc, osc = orc.mxfp8_quantize_colwise(xb)
    oqt, ost = orc.mxfp8_quantize_colwise_t(xb)
    ofq = orc.mxfp8_dequantize(oqr, osr, 1)

    q, s, fq = gpu.quantize_rowwise(x, fake_quant=True)
    assert_same(f"{name} row q", u8(q), oqr)
    assert_same(f"{name} row s", u8(s), osr)
    assert_same(f"{name} row fq", bits16(fq), ofq)

    one = gpu.quantize_colwise(x, rowwise=True, fake_quant=True)
    assert_same(f"{name} one-pass q_col", u8(one["q_col"]), oqc)
    assert_same(f"{name} one-pass s_col", u8(one["s_col"]), osc)
    assert_same(f"{name} one-pass q_row", u8(one["q_row"]), oqr)
    assert_same(f"{name} one-pass s_row", u8(one["s_row"]), osr)
    assert_same(f"{name} one-pass fq", bits16(one["fq"]), ofq)

    t = gpu.quantize_colwise_t(x, rowwise=True, fake_quant=True)
    assert_same(f"{name} transposed q", u8(t["q_colT"]), oqt)
    assert_same(f"{name} transposed s", u8(t["s_colT"]), ost)
    assert_same(f"{name} transposed q_row", u8(t["q_row"]), oqr)
    assert_same(f"{name} transposed fq", bits16(t["fq"]), ofq)

    assert_same(f"{name} dequant rows", bits16(gpu.dequantize(q, s, axis=1)), ofq)
    assert_same(f"{name} dequant cols", bits16(gpu.dequantize(one["q_col"], one["s_col"], axis=0)),
                orc.mxfp8_dequantize(oqc, osc, 0))
    for axis in (1, 0):
        assert_same(f"{name} fake-quant axis {axis}", bits16(gpu.fake_quant(x, axis=axis)),
                    orc.mxfp8_fake_quant(xb, axis))


@pytest.mark.parametrize("k,shape", list(enumerate(MX_SHAPES)))
def test_random_shape_mxfp4_and_block_fp8(gpu, orc, k, shape):
    xb = _mx_input(shape, 2000 + k)
    x = to_dev_bf16(xb)
    name = f"fp{shape}"
    announce(f"random shape MXFP4 / block-FP8 {shape}")
    oq4, os4 = orc.mxfp4_quantize(xb)
    q4, s4, fq4 = gpu.mxfp4_quantize(x, fake_quant=True)
    assert_same(f"{name} mxfp4 q", u8(q4), oq4)
    assert_same(f"{name} mxfp4 s", u8(s4), os4)
    assert_same(f"{name} mxfp4 fq", bits16(fq4), orc.mxfp4_dequantize(oq4, os4))
    assert_same(f"{name} mxfp4 dequant", bits16(gpu.mxfp4_dequantize(q4, s4)),
                orc.mxfp4_dequantize(oq4, os4))

    oq, oS = orc.blockfp8_quantize(xb, 128)
    bq, bS = gpu.blockfp8_quantize(x)
    assert_same(f"{name} bfp8 q", u8(bq), oq)
    assert_same(f"{name} bfp8 S", f32bits(bS.cpu()), f32bits(oS))
    assert_same(f"{name} bfp8 dequant", bits16(gpu.blockfp8_dequantize(bq, bS)),
                orc.blockfp8_dequantize(oq, oS, 128))
    oq8, os8 = orc.blockfp8_to_mxfp8(oq, oS, 128)
    q8, s8 = gpu.blockfp8_to_mxfp8(bq, bS)
    assert_same(f"{name} requant q", u8(q8), oq8)
    assert_same(f"{name} requant s", u8(s8), os8)

    o1, oS1 = orc.blockfp8_quantize_rect(xb, 1, 128)
    q1, S1, fq1 = gpu.blockfp8_quantize_1x128(x, fake_quant=True)
    assert_same(f"{name} 1x128 q", u8(q1), o1)
    assert_same(f"{name} 1x128 S", f32bits(S1.cpu()), f32bits(oS1))
    assert_same(f"{name} 1x128 fq", bits16(fq1), orc.blockfp8_fake_quant_1x128(xb))
    assert_same(f"{name} 1x128 dequant", bits16(gpu.blockfp8_dequantize_1x128(q1, S1)),
                orc.blockfp8_dequantize_rect(o1, oS1, 1, 128))


@pytest.mark.parametrize("k,shape", list(enumerate(NV_SHAPES)))
def test_random_shape_nvfp4(gpu, orc, k, shape):
    xb = workloads.random_bf16(shape, 3000 + k, std=2.0)
    x = to_dev_bf16(xb)
    name = f"nv{shape}"
    announce(f"random shape NVFP4 {shape}")
    oq, os_, og = orc.nvfp4_quantize(xb)
    q, s, g = gpu.nvfp4_quantize(x)
    assert_same(f"{name} g", f32bits(g.cpu()), f32bits(og))
    assert_same(f"{name} q", u8(q), oq)
    assert_same(f"{name} s", u8(s), os_)
    assert_same(f"{name} dequant", bits16(gpu.nvfp4_dequantize(q, s, g)),
                orc.nvfp4_dequantize(oq, os_, og))
