"""GPU parity: the HIP library (through its C ABI) against the CPU oracle,
byte for byte, on the same seeded inputs.  Floating-point outputs (bf16
dequantization / fake-quant, fp32 scales) are compared as bit patterns: the
bar is 0 ULP everywhere."""
import ctypes

import numpy as np
import pytest
import torch

import block_scaled_precision_mxfp8_amd as mxq
import pins
import workloads
from gpu_util import announce, assert_same, bits16, f32bits, parallel_map, to_dev_bf16, u8

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# MXFP8 row-wise
# ---------------------------------------------------------------------------

def check_rowwise(gpu, orc, x_bits, name, fake_quant=True):
    announce(f"rowwise {name} {x_bits.shape}")
    x = to_dev_bf16(x_bits)
    if fake_quant:
        q, s, fq = gpu.quantize_rowwise(x, fake_quant=True)
    else:
        q, s = gpu.quantize_rowwise(x)
    torch.cuda.synchronize()
    oq, os_ = orc.mxfp8_quantize_rowwise(x_bits)
    assert_same(f"{name} q", u8(q), oq)
    assert_same(f"{name} scale", u8(s), os_)
    if fake_quant:
        assert_same(f"{name} fq", bits16(fq), orc.mxfp8_dequantize(oq, os_, 1))
    return q, s


def test_rowwise_mx_small(gpu, orc):
    x = workloads.mx_small()
    q, s = check_rowwise(gpu, orc, x, "mx_small")
    announce("dequant mx_small")
    dq = gpu.dequantize(q, s, axis=1)
    torch.cuda.synchronize()
    # the expected values come from the oracle's own codes (check_rowwise has
    # shown them equal to the GPU codes the dequantizer read)
    oq, os_ = orc.mxfp8_quantize_rowwise(x)
    assert_same("mx_small dequant", bits16(dq), orc.mxfp8_dequantize(oq, os_, 1))


def test_rowwise_every_value_every_scale(gpu, orc):
    """Every (bf16 value, reachable scale byte) pair, 8.6 M elements."""
    x, _ = pins.mx_sweep_input()
    n = x.shape[0] // 16 * 16
    check_rowwise(gpu, orc, np.ascontiguousarray(x[:n].reshape(-1, 512)), "sweep512")
    check_rowwise(gpu, orc, np.ascontiguousarray(x[:4096]), "sweep32")


def test_rowwise_nonfinite_zero_subnormal(gpu, orc):
    rng = np.random.default_rng(1)
    x = workloads.random_bf16((64, 256), 3)
    x[0, 0:32] = 0                                   # all zero
    x[1, 32:64] = 0x8000                             # all -0
    x[2, 0:32] = rng.integers(1, 0x80, 32)           # bf16 subnormals only (scale byte 0)
    x[2, 32:64] = rng.integers(0, 0x480, 32)         # mixed tiny values, amax exponent <= 8
    x[2, 64:96] = rng.integers(0x8000, 0x8480, 32)
    x[3, 5] = 0x7FC0                                 # NaN
    x[4, 40] = 0xFF80                                # -Inf
    x[5, 70] = 0x7F80                                # +Inf
    x[6, 100] = 0x7F7F                               # max finite bf16 (scale byte 246)
    x[7, 0:32] = 0x0001                              # min subnormal
    x[8, 0:32] = rng.integers(0, 0x10000, 32).astype(np.uint16) & 0x7FFF | 0x8000
    sat, sat_scale, sat_codes = pins.mx_saturation_group()  # 500, 480, 464, 460 -> 0x7E
    x[9, 0:32] = sat[0]
    q, s = check_rowwise(gpu, orc, x, "edge")
    assert int(u8(s)[9, 0]) == sat_scale
    assert np.array_equal(u8(q)[9, 0:32].astype(np.int64), sat_codes)


@pytest.mark.parametrize("rows", [1, 31, 33, 97])
@pytest.mark.parametrize("cols", [32, 96, 544, 7168])
def test_rowwise_ragged(gpu, orc, rows, cols):
    check_rowwise(gpu, orc, workloads.random_bf16((rows, cols), rows * 1000 + cols, std=0.02),
                  f"ragged{rows}x{cols}")


def test_rowwise_weight_4097_full(gpu, orc):
    """The [4097, 7168] weight (pad-to-32-rows-then-crop case), every byte."""
    check_rowwise(gpu, orc, workloads.weight_4097(), "weight_4097", fake_quant=False)


@pytest.mark.parametrize("ldq", [104, 112])
def test_rowwise_strided_with_guard_bands(gpu, orc, ldq):
    """Row strides beyond cols on input and outputs; 0xA5 guard bytes around
    and between every output row must survive.  ldq 112 keeps code rows
    16-byte aligned (paired 16-byte stores), 104 does not (8-byte stores)."""
    rows, cols, ldx, lds, ldf = 37, 96, 128, 5, 112
    G = 256
    xb = workloads.random_bf16((rows, ldx), 77)
    announce(f"rowwise strided/guard ldq={ldq}")
    xd = to_dev_bf16(xb)
    qbuf = torch.full((G + rows * ldq + G,), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((G + rows * lds + G,), 0xA5, dtype=torch.uint8, device="cuda")
    fbuf = torch.full((G + rows * ldf + G,), 0x5A5A, dtype=torch.int16, device="cuda")
    lib = gpu.load()
    st = lib.mxq_quantize_rowwise(ctypes.c_void_p(xd.data_ptr()), rows, cols, ldx,
                                  ctypes.c_void_p(qbuf.data_ptr() + G), ldq,
                                  ctypes.c_void_p(sbuf.data_ptr() + G), lds,
                                  ctypes.c_void_p(fbuf.data_ptr() + 2 * G), ldf,
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == mxq.MXQ_OK
    torch.cuda.synchronize()
    oq, os_ = orc.mxfp8_quantize_rowwise(np.ascontiguousarray(xb[:, :cols]))
    ofq = orc.mxfp8_dequantize(oq, os_, 1)
    qh, sh, fh = u8(qbuf), u8(sbuf), fbuf.cpu().numpy().view(np.uint16)
    assert np.all(qh[:G] == 0xA5) and np.all(qh[G + rows * ldq:] == 0xA5)
    assert np.all(sh[:G] == 0xA5) and np.all(sh[G + rows * lds:] == 0xA5)
    assert np.all(fh[:G] == 0x5A5A) and np.all(fh[G + rows * ldf:] == 0x5A5A)
    qm = qh[G:G + rows * ldq].reshape(rows, ldq)
    sm = sh[G:G + rows * lds].reshape(rows, lds)
    fm = fh[G:G + rows * ldf].reshape(rows, ldf)
    assert_same("strided q", qm[:, :cols], oq)
    assert_same("strided s", sm[:, :cols // 32], os_)
    assert_same("strided fq", fm[:, :cols], ofq)
    assert np.all(qm[:, cols:] == 0xA5) and np.all(sm[:, cols // 32:] == 0xA5)
    assert np.all(fm[:, cols:] == 0x5A5A)


@pytest.mark.parametrize("rows,cols", [(4097, 224), (200, 96), (128, 128)])
def test_rowwise_padded_scale_tiles(gpu, orc, rows, cols):
    """Scales written into a zero-filled [roundup(rows, 128), roundup(cols/32, 4)]
    buffer: the compact scale sits top-left, every pad byte stays 0."""
    announce(f"rowwise padded scale {rows}x{cols}")
    xb = workloads.random_bf16((rows, cols), rows + cols)
    q, s = gpu.quantize_rowwise(to_dev_bf16(xb), scale_pad=(128, 4))
    torch.cuda.synchronize()
    oq, os_ = orc.mxfp8_quantize_rowwise(xb)
    ng = cols // 32
    assert s.shape == ((rows + 127) // 128 * 128, (ng + 3) // 4 * 4)
    sh = u8(s)
    assert_same("padded q", u8(q), oq)
    assert_same("padded scale", sh[:rows, :ng], os_)
    assert not sh[rows:].any() and not sh[:, ng:].any()


def test_mxfp8_quantize_adapter_and_param_names(gpu, orc):
    xb = workloads.random_bf16((2 * 48, 64), 9)
    announce("adapter 3-D")
    w = to_dev_bf16(xb).reshape(2, 48, 64)
    q, s = gpu.mxfp8_quantize(w)
    torch.cuda.synchronize()
    oq, os_ = orc.mxfp8_quantize_rowwise(xb)
    assert_same("adapter q", u8(q), oq)
    assert_same("adapter s", u8(s), os_)
    out = gpu.quantize_param("model.layers.0.mlp.down_proj.weight", w)
    assert [n for n, _ in out] == ["model.layers.0.mlp.down_proj.weight",
                                   "model.layers.0.mlp.down_proj.weight_scale_inv"]
    assert out[0][1].view(torch.float8_e4m3fn).dtype == torch.float8_e4m3fn
    assert out[1][1].view(torch.float8_e8m0fnu).shape == (96, 2)
    with pytest.raises(ValueError):
        gpu.quantize_param("model.bias", w)


# ---------------------------------------------------------------------------
# MXFP8 column-wise (+ row-wise + fake-quant in one pass)
# ---------------------------------------------------------------------------

def check_colwise(gpu, orc, xb, name):
    announce(f"colwise {name} {xb.shape}")
    x = to_dev_bf16(xb)
    out = gpu.quantize_colwise(x, rowwise=True, fake_quant=True)
    torch.cuda.synchronize()
    oqc, osc = orc.mxfp8_quantize_colwise(xb)
    assert_same(f"{name} q_col", u8(out["q_col"]), oqc)
    assert_same(f"{name} s_col", u8(out["s_col"]), osc)
    oqr, osr = orc.mxfp8_quantize_rowwise(xb)
    assert_same(f"{name} q_row", u8(out["q_row"]), oqr)
    assert_same(f"{name} s_row", u8(out["s_row"]), osr)
    assert_same(f"{name} fq", bits16(out["fq"]), orc.mxfp8_dequantize(oqr, osr, 1))
    # the column-only and the fq-without-codes variants give the same bytes
    c_only = gpu.quantize_colwise(x, rowwise=False, fake_quant=False)
    fq_only = gpu.quantize_colwise(x, rowwise=False, fake_quant=True)
    torch.cuda.synchronize()
    assert_same(f"{name} q_col (col only)", u8(c_only["q_col"]), oqc)
    assert_same(f"{name} fq (no row codes)", bits16(fq_only["fq"]), bits16(out["fq"]))


@pytest.mark.parametrize("shape", [(64, 512), (33, 96), (1, 32), (100, 544), (4097, 544),
                                   (160, 7168)])
def test_colwise_shapes(gpu, orc, shape):
    check_colwise(gpu, orc, workloads.random_bf16(shape, shape[0] + shape[1]), f"c{shape}")


def test_colwise_edge_values(gpu, orc):
    """Every (value, reachable scale) sweep group laid down a column."""
    x, _ = pins.mx_sweep_input()
    nb = x.shape[0] // 8192
    xb = np.ascontiguousarray(x[:nb * 8192].reshape(nb, 8192, 32).transpose(0, 2, 1)
                              .reshape(nb * 32, 8192))
    xb[5, 7] = 0x7FC0
    xb[40, 9] = 0xFF80
    check_colwise(gpu, orc, xb, "colwise-edge")


@pytest.mark.parametrize("offset", [0, 8])
def test_colwise_output_alignment_with_guard_bands(gpu, orc, offset):
    """Code outputs 16-byte aligned (paired 16-byte stores) or only 8-byte
    aligned (8-byte stores), odd row count; guard bytes around each output
    must survive."""
    rows, cols, G = 37, 96, 256
    xb = workloads.random_bf16((rows, cols), 4242)
    announce(f"colwise alignment offset={offset}")
    x = to_dev_bf16(xb)
    ng = (rows + 31) // 32
    bufs = {k: torch.full((2 * G + n,), 0xA5, dtype=torch.uint8, device="cuda")
            for k, n in (("qc", rows * cols), ("sc", ng * cols), ("qr", rows * cols),
                         ("sr", rows * cols // 32))}
    fbuf = torch.full((2 * G + rows * cols,), 0x5A5A, dtype=torch.int16, device="cuda")
    off = {"qc": G + offset, "sc": G, "qr": G + offset, "sr": G}
    lib = gpu.load()
    st = lib.mxq_quantize_colwise(
        ctypes.c_void_p(x.data_ptr()), rows, cols,
        *[ctypes.c_void_p(bufs[k].data_ptr() + off[k]) for k in ("qc", "sc", "qr", "sr")],
        ctypes.c_void_p(fbuf.data_ptr() + 2 * G), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == mxq.MXQ_OK
    torch.cuda.synchronize()
    oqc, osc = orc.mxfp8_quantize_colwise(xb)
    oqr, osr = orc.mxfp8_quantize_rowwise(xb)
    want = {"qc": oqc, "sc": osc, "qr": oqr, "sr": osr}
    for k, buf in bufs.items():
        h = u8(buf)
        n = want[k].size
        assert np.all(h[:off[k]] == 0xA5) and np.all(h[off[k] + n:] == 0xA5), k
        assert_same(f"aligned{offset} {k}", h[off[k]:off[k] + n].reshape(want[k].shape), want[k])
    fh = fbuf.cpu().numpy().view(np.uint16)
    assert np.all(fh[:G] == 0x5A5A) and np.all(fh[G + rows * cols:] == 0x5A5A)
    assert_same(f"aligned{offset} fq", fh[G:G + rows * cols].reshape(rows, cols),
                orc.mxfp8_dequantize(oqr, osr, 1))


def test_act_16384_rowwise_dequant_fakequant_full(gpu, orc):
    """The [16384, 7168] activation through the bench's other single-tensor
    launches, every output byte: row-wise quantize with fused fake-quant,
    fake-quant alone on both axes, dequantize on both axes."""
    xb = workloads.act_16384()
    announce("act_16384 row-wise + fake-quant")
    x = to_dev_bf16(xb)
    q, s, fq = gpu.quantize_rowwise(x, fake_quant=True)
    col = gpu.quantize_colwise(x, rowwise=False, fake_quant=False)
    torch.cuda.synchronize()
    oq, os_ = orc.mxfp8_quantize_rowwise(xb)
    oqc, osc = orc.mxfp8_quantize_colwise(xb)
    ofq_r = orc.mxfp8_dequantize(oq, os_, 1)
    ofq_c = orc.mxfp8_dequantize(oqc, osc, 0)
    assert_same("act row q", u8(q), oq)
    assert_same("act row s", u8(s), os_)
    assert_same("act row fq", bits16(fq), ofq_r)
    assert_same("act col q", u8(col["q_col"]), oqc)
    assert_same("act col s", u8(col["s_col"]), osc)
    del fq
    announce("act_16384 dequantize and fake-quant, both axes")
    for axis, qq, ss, want in ((1, q, s, ofq_r), (0, col["q_col"], col["s_col"], ofq_c)):
        dq = gpu.dequantize(qq, ss, axis=axis)
        fqa = gpu.fake_quant(x, axis=axis)
        torch.cuda.synchronize()
        assert_same(f"act dequant axis {axis}", bits16(dq), want)
        assert_same(f"act fake-quant axis {axis}", bits16(fqa), want)
        del dq, fqa


def test_colwise_act_16384_full(gpu, orc):
    """The [16384, 7168] activation: column-wise, row-wise and fake-quant in
    one pass, every output byte, in the launch configuration the bench times."""
    check_colwise(gpu, orc, workloads.act_16384(), "act_16384")


# ---------------------------------------------------------------------------
# dequantize / fake-quant
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("axis", [0, 1])
def test_dequant_all_codes_all_scales(gpu, orc, axis):
    if axis == 1:   # row r uses scale byte r for every code
        q = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
        s = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 8, axis=1)
    else:           # rows 32g..32g+31 use scale byte g for every code
        q = np.tile(np.arange(256, dtype=np.uint8), (256 * 32, 1))
        s = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 256, axis=1)
    announce(f"dequant all codes axis {axis}")
    out = gpu.dequantize(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(), axis=axis)
    torch.cuda.synchronize()
    assert_same(f"dequant axis {axis}", bits16(out), orc.mxfp8_dequantize(q, s, axis))


def test_dequant_hw_path_all_finite_pairs(gpu, orc):
    """Every non-NaN E4M3 code x every finite scale byte, laid out so no wave
    sees a NaN code or a NaN scale (the hardware-decode path)."""
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F] + [0, 0], dtype=np.uint8)
    q = np.tile(finite, (255, 1))                                  # [255, 256]
    s = np.repeat(np.arange(255, dtype=np.uint8)[:, None], 8, axis=1)
    announce("dequant hw path")
    out = gpu.dequantize(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(), axis=1)
    torch.cuda.synchronize()
    assert_same("dequant hw path", bits16(out), orc.mxfp8_dequantize(q, s, 1))


def test_dequant_colwise_hw_path_all_finite_pairs(gpu, orc):
    """Column groups, no NaN code or scale anywhere (the hardware-decode path):
    every non-NaN code meets every finite scale byte in every column, and the
    scale changes from column to column."""
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)   # 254
    G, cols = 255 * 8, 256
    g = np.arange(G)[:, None]
    s = ((g + np.arange(cols)[None, :]) % 255).astype(np.uint8)                      # [G, cols]
    j = np.arange(32)[None, :]
    idx = (32 * (np.arange(G)[:, None] // 255) + j) % 254                            # [G, 32]
    q = np.repeat(finite[idx].reshape(G * 32, 1), cols, axis=1)                      # [32G, cols]
    pairs = set(zip(np.repeat(s, 32, axis=0)[:, 0].tolist(), q[:, 0].tolist()))
    assert len(pairs) == 255 * 254  # column 0 alone already sees every pair
    announce("dequant colwise hw path")
    out = gpu.dequantize(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(), axis=0)
    torch.cuda.synchronize()
    assert_same("dequant colwise hw path", bits16(out), orc.mxfp8_dequantize(q, s, 0))


def test_e8m0_to_fp32_all_bytes_and_real_scales(gpu, orc):
    """The fp32 scale view: all 256 bytes, then the row scales of a real
    quantization (odd element count, float8_e8m0fnu input view)."""
    announce("e8m0 -> fp32")
    allb = torch.arange(256, dtype=torch.int32).to(torch.uint8).cuda()
    got = f32bits(gpu.e8m0_to_fp32(allb))
    want = f32bits(orc.e8m0_to_fp32(np.arange(256, dtype=np.uint8)))
    assert got[255] == 0x7FC00000
    assert_same("e8m0 all bytes", got[:255], want[:255])
    xb = workloads.random_bf16((37, 7168 - 32), 61)
    _, s = gpu.quantize_rowwise(to_dev_bf16(xb))
    got = gpu.e8m0_to_fp32(s.view(torch.float8_e8m0fnu))
    torch.cuda.synchronize()
    assert got.shape == s.shape and got.dtype == torch.float32
    assert_same("e8m0 real scales", f32bits(got), f32bits(orc.e8m0_to_fp32(u8(s))))


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("shape", [(256, 512), (33, 64), (100, 7168)])
def test_fake_quant(gpu, orc, axis, shape):
    xb = workloads.random_bf16(shape, 55 + axis)
    announce(f"fake_quant axis {axis} {shape}")
    out = gpu.fake_quant(to_dev_bf16(xb), axis=axis)
    torch.cuda.synchronize()
    assert_same(f"fake_quant {axis}", bits16(out), orc.mxfp8_fake_quant(xb, axis))


# ---------------------------------------------------------------------------
# grouped row-wise
# ---------------------------------------------------------------------------

def test_grouped_mixed_shapes(gpu, orc):
    shapes = [(64, 512), (1, 32), (33, 96), (0, 64), (97, 7168), (2048, 64), (5, 544), (300, 2048)]
    xs_b = [workloads.random_bf16(sh, 900 + i, std=0.02 * (i + 1)) if sh[0] else
            np.zeros(sh, np.uint16) for i, sh in enumerate(shapes)]
    announce("grouped mixed")
    xs = [to_dev_bf16(b) for b in xs_b]
    # one input is a column slice of a wider tensor (row stride > cols)
    wide = workloads.random_bf16((40, 256), 999)
    xs.append(to_dev_bf16(wide)[:, :128])
    xs_b.append(np.ascontiguousarray(wide[:, :128]))
    outs = gpu.quantize_rowwise_grouped(xs)
    torch.cuda.synchronize()
    for i, (b, (q, s)) in enumerate(zip(xs_b, outs)):
        if b.shape[0] == 0:
            continue
        oq, os_ = orc.mxfp8_quantize_rowwise(b)
        assert_same(f"grouped[{i}] q", u8(q), oq)
        assert_same(f"grouped[{i}] s", u8(s), os_)


@pytest.mark.timeout(900)
def test_grouped_moe_full(gpu, orc):
    """128 experts x {gate, up, down}: one grouped launch over all 384
    tensors, every output byte of every tensor against the oracle (the
    oracle runs tensor by tensor over host threads)."""
    shapes = workloads.moe_shapes()
    mult = workloads.moe_multipliers()
    announce("grouped moe_experts (384 tensors)")
    xs = [workloads.moe_tensor(i, r, c, mult[i // 3], "cuda") for i, (_, r, c) in enumerate(shapes)]
    outs = gpu.quantize_rowwise_grouped(xs)
    torch.cuda.synchronize()
    announce("grouped moe_experts: oracle on every tensor")

    def check(i):
        oq, os_ = orc.mxfp8_quantize_rowwise(bits16(xs[i]))
        assert_same(f"moe[{i}] {shapes[i][0]} q", u8(outs[i][0]), oq)
        assert_same(f"moe[{i}] {shapes[i][0]} s", u8(outs[i][1]), os_)
        return i

    assert parallel_map(check, range(len(xs))) == list(range(len(xs)))


# ---------------------------------------------------------------------------
# block-FP8 and NVFP4
# ---------------------------------------------------------------------------

def check_blockfp8(gpu, orc, xb, name):
    announce(f"blockfp8 {name} {xb.shape}")
    x = to_dev_bf16(xb)
    q, S = gpu.blockfp8_quantize(x)
    dq = gpu.blockfp8_dequantize(q, S)
    torch.cuda.synchronize()
    oq, oS = orc.blockfp8_quantize(xb, 128)
    assert_same(f"{name} S", f32bits(S), f32bits(oS))
    assert_same(f"{name} q", u8(q), oq)
    assert_same(f"{name} dq", bits16(dq), orc.blockfp8_dequantize(oq, oS, 128))


@pytest.mark.parametrize("shape", [(256, 384), (200, 296), (129, 8), (1, 1024), (1024, 1024)])
def test_blockfp8_shapes(gpu, orc, shape):
    xb = workloads.random_bf16(shape, 700 + shape[0])
    xb[:min(128, shape[0]), :min(128, shape[1])] = 0     # a zero tile
    check_blockfp8(gpu, orc, xb, f"b{shape}")


def test_blockfp8_nonfinite_and_tiny_tiles(gpu, orc):
    xb = workloads.random_bf16((256, 512), 71)
    xb[3, 3] = 0x7FC0                                      # NaN tile (0, 0)
    xb[130, 140] = 0xFF80                                  # -Inf tile (1, 1)
    xb[0:128, 256:384] = np.random.default_rng(2).integers(0, 0x80, (128, 128))  # subnormal amax
    xb[128:256, 384:512] = 0x0001
    check_blockfp8(gpu, orc, xb, "b-edge")


def bf16_of(v):
    return workloads.bf16_from_float(v)


def test_blockfp8_division_paths(gpu, orc):
    """Tiles on both sides of the reciprocal-division domain (scale in
    [2^-60, 2^60]) and signed zeros in each."""
    xb = workloads.random_bf16((128, 128 * 6), 72)
    amax = [2.0 ** -52, 2.0 ** -51, 1.0, 2.0 ** 68.5, 2.0 ** 69, 2.0 ** 120]  # S = amax/448
    for t, a in enumerate(amax):
        tile = xb[:, 128 * t:128 * (t + 1)].astype(np.int64)
        scale = a / 4.0
        vals = workloads.random_bf16((128, 128), 80 + t)
        tile[:] = workloads.bf16_bits((torch.from_numpy(vals.view(np.int16)).view(torch.bfloat16)
                                       .float().numpy() * scale).astype(np.float32))
        tile[5, 5] = bf16_of(a)
        tile[6, 6] = 0x8000                                         # -0
        tile[7, 7] = 0x0000
        tile[8, 8] = 0x8001                                         # -min subnormal
        xb[:, 128 * t:128 * (t + 1)] = tile
    check_blockfp8(gpu, orc, np.ascontiguousarray(xb), "b-divpaths")


def test_blockfp8_square_8192_full(gpu, orc):
    check_blockfp8(gpu, orc, workloads.square_8192(), "square_8192")


def check_nvfp4(gpu, orc, xb, name):
    announce(f"nvfp4 {name} {xb.shape}")
    x = to_dev_bf16(xb)
    q, s, g = gpu.nvfp4_quantize(x)
    dq = gpu.nvfp4_dequantize(q, s, g)
    torch.cuda.synchronize()
    oq, os_, og = orc.nvfp4_quantize(xb)
    assert_same(f"{name} g", f32bits(g), f32bits(og))
    assert_same(f"{name} s", u8(s), os_)
    assert_same(f"{name} q", u8(q), oq)
    assert_same(f"{name} dq", bits16(dq), orc.nvfp4_dequantize(oq, os_, og))


@pytest.mark.parametrize("shape", [(64, 256), (33, 48), (1, 16), (1024, 1024), (97, 7168)])
def test_nvfp4_shapes(gpu, orc, shape):
    check_nvfp4(gpu, orc, workloads.random_bf16(shape, 800 + shape[0]), f"n{shape}")


def test_nvfp4_degenerate(gpu, orc):
    z = np.zeros((8, 64), np.uint16)
    z[3, 5] = 0x8000
    check_nvfp4(gpu, orc, z, "zero")
    nf = workloads.random_bf16((8, 64), 5)
    nf[2, 9] = 0x7FC0
    check_nvfp4(gpu, orc, nf, "nan")
    tiny = (np.random.default_rng(3).integers(0, 0x100, (16, 64))).astype(np.uint16)
    check_nvfp4(gpu, orc, tiny, "tiny")
    big = workloads.random_bf16((16, 64), 6)
    big[0, 0] = 0x7F7F                                      # max finite bf16
    check_nvfp4(gpu, orc, big, "max")


@pytest.mark.parametrize("amax", [2.0 ** -48, 2.0 ** -40, 1.0, 2.0 ** 60, 2.0 ** 70])
def test_nvfp4_division_paths(gpu, orc, amax):
    """Global scales that put block effective scales on both sides of the
    reciprocal-division domain; signed zeros; zero blocks beside tiny ones."""
    x = workloads.random_bf16((64, 256), 90)
    xf = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float().numpy() * (amax / 8.0)
    xb = workloads.bf16_bits(xf.astype(np.float32))
    xb[0, 0] = bf16_of(amax)
    xb[1, :16] = 0                                                  # a zero block
    xb[2, 3] = 0x8000                                               # -0
    xb[3, 16:32] = 0x0001                                           # subnormal block
    check_nvfp4(gpu, orc, xb, f"n-divpaths-{amax:g}")


def test_nvfp4_square_8192_full(gpu, orc):
    check_nvfp4(gpu, orc, workloads.square_8192(), "square_8192")


def test_fp_dequant_arbitrary_codes(gpu, orc):
    """Dequantizers on codes/scales the quantizers never emit: every E4M3
    code against many fp32 scales (incl. 0, subnormal, huge, NaN), every
    E2M1 nibble against many block scales."""
    rng = np.random.default_rng(11)
    q = np.tile(np.arange(256, dtype=np.uint8), (256, 2))             # [256, 512]
    S = rng.standard_normal((2, 4)).astype(np.float32) * 1e3
    S[0, 0], S[0, 1], S[0, 2], S[0, 3] = 0.0, 1e-40, 3e38, np.nan
    S = np.abs(S)
    S[0, 3] = np.nan
    announce("blockfp8 dequant arbitrary")
    dq = gpu.blockfp8_dequantize(torch.from_numpy(q).cuda(), torch.from_numpy(S).cuda())
    torch.cuda.synchronize()
    assert_same("bfp8 dq arbitrary", bits16(dq), orc.blockfp8_dequantize(q, S, 128))
    qp = rng.integers(0, 256, (64, 128)).astype(np.uint8)              # cols = 256
    s = rng.integers(0, 256, (64, 16)).astype(np.uint8)
    for gval in (1.0, 2.5e-3, 1e-40, 7e36):
        g = np.array([gval], np.float32)
        announce(f"nvfp4 dequant arbitrary g={gval}")
        dq = gpu.nvfp4_dequantize(torch.from_numpy(qp).cuda(), torch.from_numpy(s).cuda(),
                                  torch.from_numpy(g).cuda())
        torch.cuda.synchronize()
        assert_same(f"nvfp4 dq g={gval}", bits16(dq), orc.nvfp4_dequantize(qp, s, g))


def test_workspaces_need_no_initial_contents(gpu, orc):
    """A workspace reused across calls (second call smaller) or filled with
    garbage gives the same bytes as the oracle."""
    ws = gpu.nvfp4_workspace("cuda")
    ws.fill_(0xFF)
    for shape, seed in (((256, 1024), 31), ((40, 64), 32)):
        xb = workloads.random_bf16(shape, seed)
        announce(f"nvfp4 workspace reuse {shape}")
        q, s, g = gpu.nvfp4_quantize(to_dev_bf16(xb), workspace=ws)
        torch.cuda.synchronize()
        oq, os_, og = orc.nvfp4_quantize(xb)
        assert_same(f"ws {shape} q", u8(q), oq)
        assert_same(f"ws {shape} s", u8(s), os_)
        assert_same(f"ws {shape} g", f32bits(g), f32bits(og))
    gws = gpu.grouped_workspace(3, "cuda")
    gws.fill_(0xA5)
    for shapes, seed in (([(64, 512), (33, 96), (100, 2048)], 41), ([(7, 32)], 42)):
        xs_b = [workloads.random_bf16(sh, seed + i) for i, sh in enumerate(shapes)]
        announce(f"grouped workspace reuse {shapes}")
        outs = gpu.quantize_rowwise_grouped([to_dev_bf16(b) for b in xs_b], workspace=gws)
        torch.cuda.synchronize()
        for b, (q, s) in zip(xs_b, outs):
            oq, os_ = orc.mxfp8_quantize_rowwise(b)
            assert_same("grouped reuse q", u8(q), oq)
            assert_same("grouped reuse s", u8(s), os_)
