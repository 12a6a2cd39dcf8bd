"""The CPU oracle against what the format definitions and the mathematics fix
(no GPU).  See pins.py for what each pin compares against."""
import numpy as np
import pytest

import pins
import workloads


def test_bf16_decode(orc):
    pins.pin_bf16_decode(orc)


def test_e4m3_decode(orc):
    pins.pin_e4m3_decode(orc)


def test_e8m0_decode(orc):
    pins.pin_e8m0_decode(orc)


def test_mx_saturation_golden(orc):
    pins.pin_mx_saturation(orc)


def test_e8m0_to_fp32_matches_torch_cast(orc):
    """The fp32 scale view against torch's float8_e8m0fnu -> float32 cast, all
    256 bytes (NaN for 0xFF, the subnormal 2^-127 for 0)."""
    import torch
    want = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).float()
    got = orc.e8m0_to_fp32(np.arange(256, dtype=np.uint8))
    w = want.numpy()
    assert np.isnan(got[255]) and np.isnan(w[255])
    assert np.array_equal(got[:255].view(np.uint32), w[:255].view(np.uint32))
    assert got[0].view(np.uint32) == 0x00400000 and got[127] == 1.0


def test_e2m1_decode(orc):
    pins.pin_e2m1_decode(orc)


def test_e4m3_encode_golden(orc):
    pins.pin_e4m3_encode_golden(orc)


def test_e4m3_encode_all_bf16_bruteforce(orc):
    pins.pin_e4m3_encode_bruteforce(orc)


def test_e2m1_encode(orc):
    pins.pin_e2m1_encode(orc)


def test_bf16_round(orc):
    pins.pin_bf16_round(orc)


def test_mx_sweep_every_value_every_scale(orc):
    """All (bf16 value, reachable scale byte) pairs through row-wise MXFP8."""
    pins.pin_mx_sweep(orc)


def test_mx_nonfinite_groups(orc):
    pins.pin_mx_nonfinite(orc)


def test_mx_small_edge_groups(orc):
    pins.pin_mx_edge_groups(orc)


@pytest.mark.parametrize("shape,seed", [((256, 512), 0), ((97, 1024), 11), ((33, 96), 12)])
def test_mx_max_code_band(orc, shape, seed):
    pins.pin_mx_max_code_band(orc, workloads.random_bf16(shape, seed))


def test_mx_max_code_band_t3(orc):
    pins.pin_mx_max_code_band(orc, workloads.act_16384(rows=64))


@pytest.mark.parametrize("rows", [1, 31, 33, 97, 4097])
def test_mx_padcrop_equals_direct(orc, rows):
    pins.pin_mx_padcrop(orc, workloads.random_bf16((rows, 256), 100 + rows, std=0.02))


@pytest.mark.parametrize("shape", [(64, 96), (33, 64), (1, 32), (100, 160), (31, 7)])
def test_mx_colwise_is_rowwise_of_transpose(orc, shape):
    pins.pin_mx_colwise_is_rowwise_of_transpose(orc, workloads.random_bf16(shape, 200 + shape[0]))


@pytest.mark.parametrize("shape", [(64, 96), (33, 64), (1, 32), (100, 160), (31, 7)])
def test_mx_colwise_t_is_rowwise_of_transpose(orc, shape):
    pins.pin_mx_colwise_t_is_rowwise_of_transpose(orc, workloads.random_bf16(shape, 250 + shape[0]))


def test_mx_dequant_all_codes_all_scales(orc):
    pins.pin_mx_dequant_vs_torch(orc)


@pytest.mark.parametrize("which", ["mx_small", "t3", "weight"])
def test_mx_roundtrip_and_idempotence(orc, which):
    if which == "mx_small":
        x = workloads.mx_small()
    elif which == "t3":
        x = workloads.act_16384(rows=128)
    else:
        x = workloads.weight_4097()[:256]
    pins.pin_mx_roundtrip(orc, np.ascontiguousarray(x))


def test_mx_fake_quant_is_dequant_of_quant(orc):
    pins.pin_mx_fake_quant(orc, workloads.act_16384(rows=64))


@pytest.mark.parametrize("shape,blk", [((256, 384), 128), ((200, 300), 128), ((64, 64), 32),
                                       ((129, 1), 128)])
def test_blockfp8(orc, shape, blk):
    x = workloads.random_bf16(shape, 300 + shape[0])
    x[:min(shape[0], blk), :min(shape[1], blk)] = 0  # one all-zero tile
    pins.pin_blockfp8(orc, x, blk)


def test_blockfp8_outliers(orc):
    pins.pin_blockfp8(orc, workloads.square_8192(n=256), 128)


@pytest.mark.parametrize("shape", [(64, 256), (33, 48), (1, 16)])
def test_nvfp4(orc, shape):
    pins.pin_nvfp4(orc, workloads.random_bf16(shape, 400 + shape[0]))


def test_nvfp4_outliers(orc):
    pins.pin_nvfp4(orc, workloads.square_8192(n=256))


def test_nvfp4_zero_tensor(orc):
    x = np.zeros((4, 32), np.uint16)
    x[1, 3] = 0x8000  # -0.0 keeps its sign
    q, s, g = orc.nvfp4_quantize(x)
    assert g[0] == 0 and np.all(s == 0)
    assert q[1, 1] == 0x80 and np.count_nonzero(q) == 1


def test_nvfp4_nonfinite_tensor(orc):
    x = workloads.random_bf16((4, 32), 5)
    x[2, 7] = 0x7F80
    q, s, g = orc.nvfp4_quantize(x)
    assert np.isnan(g[0]) and np.all(s == 0x7F)
    assert np.all((q & 0x7) == 0x7) and np.all(((q >> 4) & 0x7) == 0x7)


def test_blockfp8_nonfinite_tile(orc):
    x = workloads.random_bf16((128, 256), 6)
    x[5, 5] = 0x7FC0
    q, S = orc.blockfp8_quantize(x, 128)
    assert np.isnan(S[0, 0]) and np.isfinite(S[0, 1])
    assert np.all((q[:, :128] & 0x7F) == 0x7F)


def test_mx4_sweep_every_value_every_scale(orc):
    """All (bf16 value, reachable scale byte) pairs through MXFP4."""
    pins.pin_mx4_sweep(orc)


def test_mx4_nonfinite_groups_and_packing(orc):
    pins.pin_mx4_nonfinite(orc)


def test_mx4_small_edge_groups(orc):
    pins.pin_mx4_edge_groups(orc)


@pytest.mark.parametrize("which", ["normal", "t3", "weight"])
def test_mx4_max_nibble(orc, which):
    x = {"normal": lambda: workloads.random_bf16((97, 1024), 13),
         "t3": lambda: workloads.act_16384(rows=64),
         "weight": lambda: np.ascontiguousarray(workloads.weight_4097()[:128])}[which]()
    pins.pin_mx4_max_nibble(orc, x)


def test_mx4_dequant_all_nibbles_all_scales(orc):
    pins.pin_mx4_dequant_vs_torch(orc)


@pytest.mark.parametrize("which", ["mx_small", "t3", "weight"])
def test_mx4_roundtrip_and_idempotence(orc, which):
    if which == "mx_small":
        x = workloads.mx_small()
    elif which == "t3":
        x = workloads.act_16384(rows=128)
    else:
        x = workloads.weight_4097()[:256]
    pins.pin_mx4_roundtrip(orc, np.ascontiguousarray(x))


def test_requant_pow2_tiles_keep_codes(orc):
    pins.pin_requant_pow2_tiles(orc)


@pytest.mark.parametrize("which", ["normal", "outliers"])
def test_requant_matches_steps(orc, which):
    x = workloads.random_bf16((200, 384), 17) if which == "normal" else workloads.square_8192(n=256)
    pins.pin_requant_matches_steps(orc, x)


@pytest.mark.parametrize("shape", [(64, 384), (33, 200), (1, 128), (17, 7168)])
def test_blockfp8_1x128(orc, shape):
    x = workloads.random_bf16(shape, 500 + shape[0])
    x[3 % shape[0], :128] = 0                         # one all-zero group
    pins.pin_blockfp8_1x128(orc, x)


def test_blockfp8_1x128_t3(orc):
    pins.pin_blockfp8_1x128(orc, workloads.act_16384(rows=64))


def _moe_halves(seed):
    rng = np.random.default_rng(seed)
    xs = []
    for e in range(3):
        gate = workloads.random_bf16((32, 64), seed + 10 * e, std=0.02 * (1 + e))
        up = workloads.random_bf16((32, 64), seed + 10 * e + 1, std=0.05 * (1 + e))
        xs += [gate, up]
    return xs


def test_nvfp4_grouped_per_half(orc):
    """Per-half global scales (QAT form): each gate and each up its own group."""
    xs = _moe_halves(70)
    pins.pin_nvfp4_grouped(orc, xs, list(range(len(xs))), len(xs))


def test_nvfp4_grouped_shared_gate_up(orc):
    """One shared global scale per expert's gate and up (export form), plus an
    unused group."""
    xs = _moe_halves(80)
    pins.pin_nvfp4_grouped(orc, xs, [i // 2 for i in range(len(xs))], len(xs) // 2 + 1)


def test_nvfp4_grouped_nonfinite_member(orc):
    xs = _moe_halves(90)
    xs[3][5, 7] = 0x7FC0
    outs, gs = orc.nvfp4_quantize_grouped(xs, [i // 2 for i in range(len(xs))], 3)
    assert np.isnan(gs[1]) and np.isfinite(gs[0]) and np.isfinite(gs[2])
    assert np.all(outs[2][1] == 0x7F) and np.all(outs[3][1] == 0x7F)


@pytest.mark.parametrize("shape", [(3, 200, 136), (2, 128, 256), (4, 33, 8)])
def test_blockfp8_gkn(orc, shape):
    x = workloads.random_bf16((shape[0] * shape[1], shape[2]), 700 + shape[1]).reshape(shape)
    x[0, :min(shape[1], 128), :min(shape[2], 128)] = 0
    pins.pin_blockfp8_gkn(orc, x)
