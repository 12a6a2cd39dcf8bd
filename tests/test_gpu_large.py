"""GPU parity past 32-bit offsets: a [320000, 7168] bf16 tensor (4.59 GB, so
element and byte offsets cross 2^31 and 2^32) through the MXFP8 one-pass,
row-wise, dequantize, block-FP8 and NVFP4 paths.  Groups, tiles and blocks
are independent of the rest of the tensor, so 32- or 128-row slices at the
start, across the 2^31-element boundary and at the end are compared byte for
byte with the oracle run on just those rows (NVFP4's global scale spans the
tensor: every sampled slice holds the tensor's largest magnitude, so each
slice's own global scale equals the tensor's)."""
import numpy as np
import pytest
import torch

from gpu_util import announce, assert_same, f32bits

pytestmark = pytest.mark.gpu

R, C = 320000, 7168
BOUNDARY_ROW = (2 ** 31) // C // 128 * 128      # a 128-row band holding element 2^31
PEAK = 0x42C8                                    # bf16 100.0, above every N(0, 0.25) draw


def _bands(h):
    """h-aligned slice starts: the first rows, the slices around element 2^31
    (the 32-row slice at BOUNDARY_ROW + 64 straddles it), the last rows."""
    if h == 32:
        return [0, BOUNDARY_ROW, BOUNDARY_ROW + 64, R - 32]
    return [0, BOUNDARY_ROW, R - 128]


@pytest.fixture(scope="module")
def big():
    if torch.cuda.get_device_properties(0).total_memory < 64 * 2 ** 30:
        pytest.skip("needs a GPU with at least 64 GiB")
    g = torch.Generator(device="cuda")
    g.manual_seed(31)
    x = (torch.randn((R, C), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    xi = x.view(torch.int16)
    for r0 in sorted(set(_bands(32) + _bands(128))):
        xi[r0, 7] = PEAK                          # each sampled slice holds the global max
    assert BOUNDARY_ROW * C <= 2 ** 31 < (BOUNDARY_ROW + 128) * C
    yield x
    del x
    torch.cuda.empty_cache()


def _rows(t, r0, h):
    return t[r0:r0 + h].contiguous().cpu()


def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def test_large_mxfp8_one_pass_and_dequant(gpu, orc, big):
    announce(f"large one-pass [{R}, {C}]")
    out = gpu.quantize_colwise(big, rowwise=True, fake_quant=True)
    torch.cuda.synchronize()
    for r0 in _bands(32):
        xb = _bits(_rows(big, r0, 32))
        oqc, osc = orc.mxfp8_quantize_colwise(xb)
        oqr, osr = orc.mxfp8_quantize_rowwise(xb)
        assert_same(f"q_col@{r0}", _rows(out["q_col"], r0, 32).numpy(), oqc)
        assert_same(f"s_col@{r0}", _rows(out["s_col"], r0 // 32, 1).numpy(), osc)
        assert_same(f"q_row@{r0}", _rows(out["q_row"], r0, 32).numpy(), oqr)
        assert_same(f"s_row@{r0}", _rows(out["s_row"], r0, 32).numpy(), osr)
        assert_same(f"fq@{r0}", _bits(_rows(out["fq"], r0, 32)), orc.mxfp8_dequantize(oqr, osr, 1))
    announce("large dequantize, both axes")
    dq_r = gpu.dequantize(out["q_row"], out["s_row"], axis=1)
    torch.cuda.synchronize()
    for r0 in _bands(32):
        want = orc.mxfp8_dequantize(_rows(out["q_row"], r0, 32).numpy(),
                                    _rows(out["s_row"], r0, 32).numpy(), 1)
        assert_same(f"dequant rows@{r0}", _bits(_rows(dq_r, r0, 32)), want)
    del dq_r
    dq_c = gpu.dequantize(out["q_col"], out["s_col"], axis=0)
    torch.cuda.synchronize()
    for r0 in _bands(32):
        want = orc.mxfp8_dequantize(_rows(out["q_col"], r0, 32).numpy(),
                                    _rows(out["s_col"], r0 // 32, 1).numpy(), 0)
        assert_same(f"dequant cols@{r0}", _bits(_rows(dq_c, r0, 32)), want)


def test_large_rowwise_and_mxfp4(gpu, orc, big):
    announce(f"large row-wise + MXFP4 [{R}, {C}]")
    q, s = gpu.quantize_rowwise(big)
    q4, s4, fq4 = gpu.mxfp4_quantize(big, fake_quant=True)
    torch.cuda.synchronize()
    for r0 in _bands(32):
        xb = _bits(_rows(big, r0, 32))
        oq, os_ = orc.mxfp8_quantize_rowwise(xb)
        assert_same(f"row q@{r0}", _rows(q, r0, 32).numpy(), oq)
        assert_same(f"row s@{r0}", _rows(s, r0, 32).numpy(), os_)
        oq4, os4 = orc.mxfp4_quantize(xb)
        assert_same(f"mxfp4 q@{r0}", _rows(q4, r0, 32).numpy(), oq4)
        assert_same(f"mxfp4 s@{r0}", _rows(s4, r0, 32).numpy(), os4)
        assert_same(f"mxfp4 fq@{r0}", _bits(_rows(fq4, r0, 32)), orc.mxfp4_dequantize(oq4, os4))


def test_large_blockfp8_and_nvfp4(gpu, orc, big):
    announce(f"large block-FP8 [{R}, {C}]")
    bq, bS = gpu.blockfp8_quantize(big)
    torch.cuda.synchronize()
    for r0 in _bands(128):
        xb = _bits(_rows(big, r0, 128))
        oq, oS = orc.blockfp8_quantize(xb, 128)
        assert_same(f"bfp8 q@{r0}", _rows(bq, r0, 128).numpy(), oq)
        assert_same(f"bfp8 S@{r0}", f32bits(_rows(bS, r0 // 128, 1)), f32bits(oS))
    del bq, bS
    announce(f"large NVFP4 [{R}, {C}]")
    nq, ns, ng = gpu.nvfp4_quantize(big)
    torch.cuda.synchronize()
    for r0 in _bands(32):
        xb = _bits(_rows(big, r0, 32))
        oq, os_, og = orc.nvfp4_quantize(xb)
        assert_same(f"nvfp4 g@{r0}", f32bits(ng), f32bits(og))
        assert_same(f"nvfp4 q@{r0}", _rows(nq, r0, 32).numpy(), oq)
        assert_same(f"nvfp4 s@{r0}", _rows(ns, r0, 32).numpy(), os_)
