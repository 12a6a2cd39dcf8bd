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
    want = {}
    for r0 in _bands(32):
        xb = _bits(_rows(big, r0, 32))
        oqc, osc = orc.mxfp8_quantize_colwise(xb)
        oqr, osr = orc.mxfp8_quantize_rowwise(xb)
        want[r0] = (oqr, osr, oqc, osc)
        assert_same(f"q_col@{r0}", _rows(out["q_col"], r0, 32).numpy(), oqc)
        assert_same(f"s_col@{r0}", _rows(out["s_col"], r0 // 32, 1).numpy(), osc)
        assert_same(f"q_row@{r0}", _rows(out["q_row"], r0, 32).numpy(), oqr)
        assert_same(f"s_row@{r0}", _rows(out["s_row"], r0, 32).numpy(), osr)
        assert_same(f"fq@{r0}", _bits(_rows(out["fq"], r0, 32)), orc.mxfp8_dequantize(oqr, osr, 1))
    announce("large dequantize, both axes")
    # the dequantizers read the GPU codes; the expected values come from the
    # oracle's codes, shown equal to them on these rows above
    dq_r = gpu.dequantize(out["q_row"], out["s_row"], axis=1)
    torch.cuda.synchronize()
    for r0 in _bands(32):
        oqr, osr = want[r0][:2]
        assert_same(f"dequant rows@{r0}", _bits(_rows(dq_r, r0, 32)),
                    orc.mxfp8_dequantize(oqr, osr, 1))
    del dq_r
    dq_c = gpu.dequantize(out["q_col"], out["s_col"], axis=0)
    torch.cuda.synchronize()
    for r0 in _bands(32):
        oqc, osc = want[r0][2:]
        assert_same(f"dequant cols@{r0}", _bits(_rows(dq_c, r0, 32)),
                    orc.mxfp8_dequantize(oqc, osc, 0))


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


def test_large_colwise_t(gpu, orc, big):
    """The transposed column-wise layout past 32-bit offsets: qT is [C, R] =
    2.29 GB, so column c's codes start at byte c * R, above 2^31 from column
    6711 on.  Every column of each sampled 32-row band is compared, with the
    row-wise outputs of the same pass."""
    announce(f"large transposed one pass [{R}, {C}]")
    out = gpu.quantize_colwise_t(big, rowwise=True, fake_quant=True)
    torch.cuda.synchronize()
    for r0 in _bands(32):
        xb = _bits(_rows(big, r0, 32))
        oqt, ost = orc.mxfp8_quantize_colwise_t(xb)
        assert_same(f"qT@{r0}", out["q_colT"][:, r0:r0 + 32].contiguous().cpu().numpy(), oqt)
        assert_same(f"sT@{r0}", out["s_colT"][:, r0 // 32:r0 // 32 + 1].contiguous().cpu().numpy(),
                    ost)
        oqr, osr = orc.mxfp8_quantize_rowwise(xb)
        assert_same(f"q_row@{r0}", _rows(out["q_row"], r0, 32).numpy(), oqr)
        assert_same(f"s_row@{r0}", _rows(out["s_row"], r0, 32).numpy(), osr)
        assert_same(f"fq@{r0}", _bits(_rows(out["fq"], r0, 32)), orc.mxfp8_dequantize(oqr, osr, 1))
    del out
    announce(f"large transposed column-only [{R}, {C}]")
    out = gpu.quantize_colwise_t(big, rowwise=False, fake_quant=False)
    torch.cuda.synchronize()
    for r0 in _bands(32):
        oqt, ost = orc.mxfp8_quantize_colwise_t(_bits(_rows(big, r0, 32)))
        assert_same(f"qT only@{r0}", out["q_colT"][:, r0:r0 + 32].contiguous().cpu().numpy(), oqt)
        assert_same(f"sT only@{r0}",
                    out["s_colT"][:, r0 // 32:r0 // 32 + 1].contiguous().cpu().numpy(), ost)
    del out
    torch.cuda.empty_cache()


def test_large_fake_quant_both_axes(gpu, orc, big):
    for axis in (1, 0):
        announce(f"large MXFP8 fake-quant axis {axis} [{R}, {C}]")
        fq = gpu.fake_quant(big, axis=axis)
        torch.cuda.synchronize()
        for r0 in _bands(32):
            assert_same(f"fake-quant axis {axis}@{r0}", _bits(_rows(fq, r0, 32)),
                        orc.mxfp8_fake_quant(_bits(_rows(big, r0, 32)), axis))
        del fq
    torch.cuda.empty_cache()


def test_large_blockfp8_1x128(gpu, orc, big):
    announce(f"large 1x128 block-FP8 [{R}, {C}]")
    q, S, fq = gpu.blockfp8_quantize_1x128(big, fake_quant=True)
    torch.cuda.synchronize()
    want = {}
    for r0 in _bands(32):
        xb = _bits(_rows(big, r0, 32))
        oq, oS = orc.blockfp8_quantize_rect(xb, 1, 128)
        want[r0] = (oq, oS)
        assert_same(f"1x128 q@{r0}", _rows(q, r0, 32).numpy(), oq)
        assert_same(f"1x128 S@{r0}", f32bits(_rows(S, r0, 32)), f32bits(oS))
        assert_same(f"1x128 fq@{r0}", _bits(_rows(fq, r0, 32)),
                    orc.blockfp8_fake_quant_1x128(xb))
    del fq
    announce(f"large 1x128 block-FP8 dequantize and simulate-QAT [{R}, {C}]")
    dq = gpu.blockfp8_dequantize_1x128(q, S)
    torch.cuda.synchronize()
    for r0 in _bands(32):
        oq, oS = want[r0]
        assert_same(f"1x128 dq@{r0}", _bits(_rows(dq, r0, 32)),
                    orc.blockfp8_dequantize_rect(oq, oS, 1, 128))
    del dq, q, S
    qat = gpu.fp8_simulate_qat(big)
    torch.cuda.synchronize()
    for r0 in _bands(32):
        assert_same(f"1x128 qat@{r0}", _bits(_rows(qat, r0, 32)),
                    orc.blockfp8_fake_quant_1x128(_bits(_rows(big, r0, 32))))
    del qat
    torch.cuda.empty_cache()


def test_large_blockfp8_dequant_requant_and_gkn(gpu, orc, big):
    """Block-FP8 dequantization and the FP8 block -> MXFP8 pass read the
    [R, C] codes (1.15e9 bytes past 2^31 written as bf16); the same tensor
    viewed as a [20, 16000, 7168] stack goes through the [G, K, N] form."""
    announce(f"large block-FP8 dequantize + FP8 block -> MXFP8 [{R}, {C}]")
    bq, bS = gpu.blockfp8_quantize(big)
    dq = gpu.blockfp8_dequantize(bq, bS)
    q8, s8 = gpu.blockfp8_to_mxfp8(bq, bS)
    torch.cuda.synchronize()
    for r0 in _bands(128):
        oq, oS = orc.blockfp8_quantize(_bits(_rows(big, r0, 128)), 128)
        assert_same(f"bfp8 q@{r0}", _rows(bq, r0, 128).numpy(), oq)
        assert_same(f"bfp8 S@{r0}", f32bits(_rows(bS, r0 // 128, 1)), f32bits(oS))
        assert_same(f"bfp8 dq@{r0}", _bits(_rows(dq, r0, 128)), orc.blockfp8_dequantize(oq, oS, 128))
        oq8, os8 = orc.blockfp8_to_mxfp8(oq, oS, 128)
        assert_same(f"requant q@{r0}", _rows(q8, r0, 128).numpy(), oq8)
        assert_same(f"requant s@{r0}", _rows(s8, r0, 128).numpy(), os8)
    del bq, bS, dq, q8, s8
    G, K = 20, R * C // (20 * C)
    assert G * K == R and K % 128 == 0
    stack = big.view(G, K, C)
    announce(f"large block-FP8 [G, K, N] = [{G}, {K}, {C}]")
    gq, gS = gpu.blockfp8_quantize_gkn(stack)
    gd = gpu.blockfp8_dequantize_gkn(gq, gS)
    torch.cuda.synchronize()
    for r0 in _bands(128):
        g, k0 = r0 // K, r0 % K
        xb = _bits(stack[g, k0:k0 + 128].contiguous().cpu())[None]
        oq, oS = orc.blockfp8_quantize_gkn(xb, 128)
        assert_same(f"gkn q@{r0}", gq[g, k0:k0 + 128].contiguous().cpu().numpy(), oq[0])
        assert_same(f"gkn S@{r0}", f32bits(gS[g, k0 // 128:k0 // 128 + 1].contiguous().cpu()),
                    f32bits(oS[0]))
        assert_same(f"gkn dq@{r0}", _bits(gd[g, k0:k0 + 128].contiguous().cpu()),
                    orc.blockfp8_dequantize_gkn(oq, oS, 128)[0])
    del gq, gS, gd
    torch.cuda.empty_cache()


def test_large_fp4_dequantizers(gpu, orc, big):
    """MXFP4 and NVFP4 dequantization write bf16 past 2^31 elements."""
    announce(f"large MXFP4 dequantize [{R}, {C}]")
    q4, s4 = gpu.mxfp4_quantize(big)
    d4 = gpu.mxfp4_dequantize(q4, s4)
    torch.cuda.synchronize()
    for r0 in _bands(32):
        oq4, os4 = orc.mxfp4_quantize(_bits(_rows(big, r0, 32)))
        assert_same(f"mxfp4 q@{r0}", _rows(q4, r0, 32).numpy(), oq4)
        assert_same(f"mxfp4 s@{r0}", _rows(s4, r0, 32).numpy(), os4)
        assert_same(f"mxfp4 dq@{r0}", _bits(_rows(d4, r0, 32)), orc.mxfp4_dequantize(oq4, os4))
    del q4, s4, d4
    announce(f"large NVFP4 dequantize [{R}, {C}]")
    nq, ns, ng = gpu.nvfp4_quantize(big)
    nd = gpu.nvfp4_dequantize(nq, ns, ng)
    torch.cuda.synchronize()
    for r0 in _bands(32):
        oq, os_, og = orc.nvfp4_quantize(_bits(_rows(big, r0, 32)))
        assert_same(f"nvfp4 g@{r0}", f32bits(ng), f32bits(og))
        assert_same(f"nvfp4 q@{r0}", _rows(nq, r0, 32).numpy(), oq)
        assert_same(f"nvfp4 s@{r0}", _rows(ns, r0, 32).numpy(), os_)
        assert_same(f"nvfp4 dq@{r0}", _bits(_rows(nd, r0, 32)), orc.nvfp4_dequantize(oq, os_, og))
    del nq, ns, ng, nd
    torch.cuda.empty_cache()
