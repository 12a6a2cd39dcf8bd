"""Element quotients on and next to the rounding midpoints, through the product
entry points, against the oracle bit for bit.

Block-FP8 rounds fl32(x / S), S = fl32(amax / 448), to E4M3, and NVFP4 rounds
fl32(x / eff), eff = fl32(E4M3(s) * g), to E2M1 (xorl PR #30, "Add FP8, NVFP4,
and QARL training and export", deep review, "What looked solid").  A divider
or converter that is off by one fp32 ulp, or breaks ties the wrong way, shows
only on quotients within an ulp of a midpoint between two codes.  The inputs
here are chosen so that every element's quotient is one: for every positive
bf16 amax, and every midpoint m, the bf16 values x nearest m * S (and their
neighbours) whose fp32 quotient lies within one ulp of m, exact ties included.
The selection uses numpy's fp32 arithmetic (and torch's E4M3 cast for the
NVFP4 block scale); the expected bytes come from the oracle alone.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import announce, assert_same, bits16, f32bits, to_dev_bf16, u8

pytestmark = pytest.mark.gpu

F32 = np.float32


def _e4m3_values():
    c = torch.arange(0, 127, dtype=torch.uint8)            # finite non-negative codes
    return c.view(torch.float8_e4m3fn).float().numpy().astype(F32)


def _midpoints(vals):
    v = np.sort(vals.astype(np.float64))
    return ((v[:-1] + v[1:]) / 2).astype(F32)              # exact in fp32


E4M3_MIDS = _midpoints(_e4m3_values())
E2M1_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], F32)


def _f32_of_bf16(b):
    return (b.astype(np.uint32) << 16).view(F32)


def near_midpoint_x(div, mids, limit):
    """For each divisor div[i] (fp32), the positive bf16 bit patterns x <= limit[i]
    with fl32(x / div[i]) within one ulp of a midpoint: a list of uint16 arrays."""
    p = (div.astype(np.float64)[:, None] * mids.astype(np.float64)[None, :]).astype(F32)
    base = workloads.bf16_bits(p).astype(np.int32)
    found = [[] for _ in range(len(div))]
    mb = mids.view(np.int32)[None, :]
    for d in (-2, -1, 0, 1, 2):
        xb = base + d
        ok = (xb > 0) & (xb < 0x7F80)
        xf = _f32_of_bf16(np.where(ok, xb, 0).astype(np.uint16))
        with np.errstate(all="ignore"):
            q = xf / div[:, None]                               # IEEE fp32 division
        hit = ok & (np.abs(q.view(np.int32) - mb) <= 1) & (xf <= limit[:, None])
        for i, j in zip(*np.nonzero(hit)):
            found[i].append(xb[i, j])
    return [np.unique(np.array(f, np.int64)).astype(np.uint16) for f in found]


def _with_signs(bits, rng):
    return bits | (rng.integers(0, 2, bits.shape) << 15).astype(np.uint16)


def _amax_candidates(lo=0x0080, hi=0x7F00, step=1):
    """Positive finite bf16 patterns (normal, so the quotients cover all
    binades; the division-path tests cover subnormal amax)."""
    return np.arange(lo, hi, step, dtype=np.int64).astype(np.uint16)


def test_blockfp8_1x128_quotients_at_midpoints(gpu, orc):
    rng = np.random.default_rng(4100)
    A = _amax_candidates()
    S = _f32_of_bf16(A) / F32(448.0)
    hits = near_midpoint_x(S, E4M3_MIDS, _f32_of_bf16(A))
    blocks = []
    for a, h in zip(A, hits):
        if len(h) == 0:
            continue
        h = h[h != a][:127]
        fill = rng.integers(0, 0x80, 127 - len(h)).astype(np.uint16)   # tiny values
        blk = np.concatenate([[a], h, fill]).astype(np.uint16)
        blocks.append(_with_signs(rng.permutation(blk), rng))
    assert len(blocks) > 1000, len(blocks)
    nb = len(blocks) // 2 * 2
    xb = np.stack(blocks[:nb]).reshape(nb // 2, 256)       # two 1 x 128 blocks per row
    announce(f"1x128 block-FP8 at midpoints {xb.shape}")
    q, S_, fq = gpu.blockfp8_quantize_1x128(to_dev_bf16(xb), fake_quant=True)
    torch.cuda.synchronize()
    oq, oS = orc.blockfp8_quantize_rect(xb, 1, 128)
    assert_same("1x128 S", f32bits(S_), f32bits(oS))
    assert_same("1x128 q", u8(q), oq)
    assert_same("1x128 fq", bits16(fq), orc.blockfp8_fake_quant_1x128(xb))


def test_blockfp8_128x128_quotients_at_midpoints(gpu, orc):
    rng = np.random.default_rng(4200)
    A = _amax_candidates(step=3)
    S = _f32_of_bf16(A) / F32(448.0)
    hits = near_midpoint_x(S, E4M3_MIDS, _f32_of_bf16(A))
    order = np.argsort([-len(h) for h in hits])[:48]       # the 48 richest tiles
    tiles = []
    for i in order:
        h = hits[i][hits[i] != A[i]]
        t = rng.integers(0, 0x80, 128 * 128).astype(np.uint16)
        pos = rng.choice(128 * 128, len(h) + 1, replace=False)
        t[pos] = np.concatenate([[A[i]], h])
        tiles.append(_with_signs(t, rng).reshape(128, 128))
    xb = np.ascontiguousarray(np.concatenate(tiles, axis=1))   # [128, 48 * 128]
    announce(f"128x128 block-FP8 at midpoints {xb.shape}")
    q, S_ = gpu.blockfp8_quantize(to_dev_bf16(xb))
    torch.cuda.synchronize()
    oq, oS = orc.blockfp8_quantize(xb, 128)
    assert_same("128x128 S", f32bits(S_), f32bits(oS))
    assert_same("128x128 q", u8(q), oq)


def _nvfp4_blocks(A_bits, rng):
    """Blocks of 16 for a tensor whose amax is the bf16 A_bits: for every block
    amax b <= A, the x with fl32(x / eff) within an ulp of an E2M1 midpoint."""
    A = _f32_of_bf16(np.array([A_bits], np.uint16))[0]
    g = F32(A / F32(2688.0))
    d = F32(F32(6.0) * g)
    b = np.arange(0x0080, A_bits + 1, dtype=np.int64).astype(np.uint16)
    bf = _f32_of_bf16(b)
    ratio = (bf / d).astype(F32)
    s = torch.from_numpy(ratio).clamp(0, 448).to(torch.float8_e4m3fn).float().numpy().astype(F32)
    eff = (s * g).astype(F32)
    keep = eff > 0
    hits = near_midpoint_x(eff[keep], E2M1_MIDS, bf[keep])
    blocks = []
    for bb, h in zip(b[keep], hits):
        h = h[h != bb][:15]
        if len(h) == 0:
            continue
        fill = rng.integers(0, 0x80, 15 - len(h)).astype(np.uint16)
        blocks.append(_with_signs(rng.permutation(np.concatenate([[bb], h, fill]).astype(np.uint16)),
                                  rng))
    return blocks


@pytest.mark.parametrize("amax", [1.0, 6.0, 448.0, 2.0 ** -30, 2.0 ** 40])
def test_nvfp4_quotients_at_midpoints(gpu, orc, amax):
    rng = np.random.default_rng(4300 + int(np.log2(amax)) + 64)
    A_bits = int(workloads.bf16_from_float(amax))
    blocks = _nvfp4_blocks(A_bits, rng)
    assert len(blocks) > 200, len(blocks)
    nb = len(blocks) // 16 * 16
    xb = np.stack(blocks[:nb]).reshape(nb // 16, 256)     # 16 blocks of 16 per row
    xb[0, 0] = A_bits                                      # the tensor amax itself
    announce(f"NVFP4 at midpoints, amax {amax}, {xb.shape}")
    q, s, g = gpu.nvfp4_quantize(to_dev_bf16(xb))
    dq = gpu.nvfp4_dequantize(q, s, g)
    torch.cuda.synchronize()
    oq, os_, og = orc.nvfp4_quantize(xb)
    assert_same("nvfp4 g", f32bits(g), f32bits(og))
    assert_same("nvfp4 s", u8(s), os_)
    assert_same("nvfp4 q", u8(q), oq)
    assert_same("nvfp4 dq", bits16(dq), orc.nvfp4_dequantize(oq, os_, og))
