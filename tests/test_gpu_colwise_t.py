"""GPU parity of the transposed column-wise MXFP8 layout (with the optional
row-wise outputs of the same pass) against the CPU oracle, byte for byte."""
import ctypes

import numpy as np
import pytest
import torch

import block_scaled_precision_mxfp8_amd as mxq
import pins
import workloads
from gpu_util import announce, assert_same, bits16, to_dev_bf16, u8

pytestmark = pytest.mark.gpu


def check_colwise_t(gpu, orc, x_bits, name, rowwise=True, fake_quant=True, ldt=None):
    announce(f"colwise_t {name} {x_bits.shape} row={rowwise} fq={fake_quant} ldt={ldt}")
    x = to_dev_bf16(x_bits)
    out = gpu.quantize_colwise_t(x, rowwise=rowwise, fake_quant=fake_quant, ldt=ldt)
    torch.cuda.synchronize()
    oqt, ost = orc.mxfp8_quantize_colwise_t(x_bits)
    assert_same(f"{name} qt", u8(out["q_colT"]), oqt)
    assert_same(f"{name} st", u8(out["s_colT"]), ost)
    if rowwise or fake_quant:
        oqr, osr = orc.mxfp8_quantize_rowwise(x_bits)
        if rowwise:
            assert_same(f"{name} q_row", u8(out["q_row"]), oqr)
            assert_same(f"{name} s_row", u8(out["s_row"]), osr)
        if fake_quant:
            assert_same(f"{name} fq", bits16(out["fq"]), orc.mxfp8_dequantize(oqr, osr, 1))


@pytest.mark.parametrize("shape", [(64, 512), (33, 96), (1, 32), (100, 544), (130, 96),
                                   (4097, 544), (160, 7168), (256, 1024)])
def test_colwise_t_shapes(gpu, orc, shape):
    check_colwise_t(gpu, orc, workloads.random_bf16(shape, 31 * shape[0] + shape[1]), f"t{shape}")


@pytest.mark.parametrize("shape,pad", [((4096, 1024), 256), ((300, 544), 16), ((129, 7168), 4096)])
def test_colwise_t_padded_rows(gpu, orc, shape, pad):
    """q_colT rows spaced ldt = rows (rounded up to 16) + pad bytes apart: the
    view holds the same codes as the oracle's compact layout."""
    ldt = (shape[0] + 15) // 16 * 16 + pad
    check_colwise_t(gpu, orc, workloads.random_bf16(shape, shape[0] * 3 + pad), f"t-pad{pad}{shape}",
                    ldt=ldt)


@pytest.mark.parametrize("rowwise,fake_quant", [(False, False), (True, False), (False, True)])
def test_colwise_t_output_subsets(gpu, orc, rowwise, fake_quant):
    check_colwise_t(gpu, orc, workloads.random_bf16((200, 1056), 77), "subset", rowwise, fake_quant)


@pytest.mark.parametrize("shape", [(4229, 1056), (8192, 512), (130, 7168)])
def test_colwise_t_column_only_band_units(gpu, orc, shape):
    """Column-only launches order workgroups in units of 32 row bands per XCD:
    a partial last unit (4229 rows = 33 bands + 5 rows), exactly 2 units,
    and fewer bands than one unit over many segments."""
    check_colwise_t(gpu, orc, workloads.random_bf16(shape, shape[0] + 7 * shape[1]),
                    f"t-col-only{shape}", rowwise=False, fake_quant=False)


def test_colwise_t_act_16384_column_only(gpu, orc):
    """The [16384, 7168] activation, transposed column-wise only (the bench's
    column-only launch), every output byte."""
    check_colwise_t(gpu, orc, workloads.act_16384(), "act_16384 col-only", rowwise=False,
                    fake_quant=False)


def test_colwise_t_edge_values(gpu, orc):
    """Every (value, reachable scale) sweep group laid down a column, plus
    NaN and Inf columns."""
    x, _ = pins.mx_sweep_input()
    nb = x.shape[0] // 8192
    xb = np.ascontiguousarray(x[:nb * 8192].reshape(nb, 8192, 32).transpose(0, 2, 1)
                              .reshape(nb * 32, 8192))
    xb[5, 7] = 0x7FC0
    xb[40, 9] = 0xFF80
    check_colwise_t(gpu, orc, xb, "t-edge")


def test_colwise_t_act_16384_full(gpu, orc):
    """The [16384, 7168] activation: transposed column-wise, row-wise and
    fake-quant in one pass, every output byte."""
    check_colwise_t(gpu, orc, workloads.act_16384(), "act_16384")


def test_colwise_t_guard_bands(gpu, orc):
    """qt with ldt > rows: the bytes between rows and ldt of every qt row and
    the guard bytes around qt and st must survive."""
    rows, cols, ldt, G = 37, 96, 64, 256
    xb = workloads.random_bf16((rows, cols), 55)
    announce("colwise_t guard bands")
    x = to_dev_bf16(xb)
    nrg = (rows + 31) // 32
    qb = torch.full((2 * G + cols * ldt,), 0xA5, dtype=torch.uint8, device="cuda")
    sb = torch.full((2 * G + cols * nrg,), 0xA5, dtype=torch.uint8, device="cuda")
    lib = gpu.load()
    st = lib.mxq_quantize_colwise_t(ctypes.c_void_p(x.data_ptr()), rows, cols,
                                    ctypes.c_void_p(qb.data_ptr() + G), ldt,
                                    ctypes.c_void_p(sb.data_ptr() + G), None, None, None,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == mxq.MXQ_OK
    torch.cuda.synchronize()
    oqt, ost = orc.mxfp8_quantize_colwise_t(xb)
    qh, sh = u8(qb), u8(sb)
    assert np.all(qh[:G] == 0xA5) and np.all(qh[G + cols * ldt:] == 0xA5)
    assert np.all(sh[:G] == 0xA5) and np.all(sh[G + cols * nrg:] == 0xA5)
    qm = qh[G:G + cols * ldt].reshape(cols, ldt)
    assert_same("guard qt", qm[:, :rows], oqt)
    assert np.all(qm[:, rows:] == 0xA5)
    assert_same("guard st", sh[G:G + cols * nrg].reshape(cols, nrg), ost)


def test_colwise_t_binding_refuses_bad_ldt(gpu):
    x = to_dev_bf16(workloads.random_bf16((64, 96), 5))
    for ldt in (48, 72):  # below rows; not a multiple of 16
        with pytest.raises(ValueError):
            gpu.quantize_colwise_t(x, ldt=ldt)
