"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with
  - hand-derived golden points (tests/golden/, each file cites its source),
  - torch's own fp8 / e8m0 / bf16 casts and decoders (an independent library),
  - brute-force nearest-value searches over every code of a format,
  - closed forms (the MX scale byte straight from the bf16 exponent bits),
  - invariants (pad-then-crop, column-wise = row-wise of the transpose,
    idempotence, round-trip error bound, tile-max maps to the max code).
The same pins run against deliberately broken builds of the oracle source in
test_oracle_mutants.py, to show each planted mistake fails at least one of them.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from conftest import read_golden

# ---------------------------------------------------------------------------
# independent references (torch decoders / casts, brute force)
# ---------------------------------------------------------------------------

ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def torch_bf16_values(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.double().numpy()


def torch_e4m3_values() -> np.ndarray:
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def torch_e8m0_values() -> np.ndarray:
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).double().numpy()


E4M3_POS = None


def e4m3_pos_values() -> np.ndarray:
    """Values of the finite non-negative E4M3 codes 0x00..0x7E, from torch."""
    global E4M3_POS
    if E4M3_POS is None:
        v = torch_e4m3_values()[:127]
        assert np.all(np.diff(v) > 0)
        E4M3_POS = v
    return E4M3_POS


E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])  # codes 0..7 (OCP E2M1)


def nearest_code(v: np.ndarray, pos_values: np.ndarray, sign_bit: int) -> np.ndarray:
    """Nearest finite code by exhaustive search over every non-negative code of
    the format (ties -> the even code, sign bit copied from v; beyond the max
    the nearest finite code is the max, i.e. saturation).  NaN and Inf are
    not handled here."""
    # Beyond twice the max, every such value has the max as its nearest code;
    # capping there keeps the float64 distances exact (no false ties).
    a = np.minimum(np.abs(v), 2 * pos_values[-1])
    best = np.zeros(a.shape, np.int64)
    bestd = np.full(a.shape, np.inf)
    for c, cv in enumerate(pos_values):
        d = np.abs(a - cv)
        better = d < bestd
        tie = (d == bestd) & (c % 2 == 0)
        take = better | tie
        best = np.where(take, c, best)
        bestd = np.where(take, d, bestd)
    return best | (np.signbit(v).astype(np.int64) * sign_bit)


def nearest_code_sorted(v: np.ndarray, pos_values: np.ndarray, sign_bit: int) -> np.ndarray:
    """Same result as nearest_code via binary search (for millions of values)."""
    a = np.abs(v)
    n = len(pos_values)
    hi = np.clip(np.searchsorted(pos_values, a, side="left"), 0, n - 1)
    lo = np.clip(hi - 1, 0, n - 1)
    dlo = np.abs(a - pos_values[lo])
    dhi = np.abs(pos_values[hi] - a)
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    return pick.astype(np.int64) | (np.signbit(v).astype(np.int64) * sign_bit)


def mx_scale_closed_form(group_bits: np.ndarray) -> np.ndarray:
    """E8M0 byte straight from bf16 bits: max(expfield(max magnitude) - 8, 0);
    0xFF when the group holds Inf/NaN (exponent field 0xFF).  Magnitude bit
    patterns order like magnitudes, so the max is an integer max."""
    mag = (group_bits.astype(np.int64) & 0x7FFF).max(axis=-1)
    e = mag >> 7
    return np.where(e == 0xFF, 0xFF, np.maximum(e - 8, 0))


def torch_e4m3_cast(v32: np.ndarray) -> np.ndarray:
    """torch's fp32 -> float8_e4m3fn cast after clamping to +-448 (saturation)."""
    t = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)


# ---------------------------------------------------------------------------
# format pins
# ---------------------------------------------------------------------------

def _parse_value(tok: str) -> float:
    tok = tok.strip()
    if "*2^" in tok:
        a, b = tok.split("*2^")
        return float(a) * 2.0 ** int(b)
    if tok.startswith("2^"):
        return 2.0 ** int(tok[2:])
    return float(tok)


def pin_bf16_decode(orc):
    ref = torch_bf16_values(ALL_BF16)
    got = np.array([orc.bf16_to_double(int(b)) for b in ALL_BF16])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    for bits, val in read_golden("bf16_decode_points.txt"):
        v = _parse_value(val)
        g = orc.bf16_to_double(int(bits, 16))
        assert (math.isnan(v) and math.isnan(g)) or (g == v and math.copysign(1, g) == math.copysign(1, v)), bits


def pin_e4m3_decode(orc):
    ref = torch_e4m3_values()
    got = np.array([orc.e4m3_to_double(c) for c in range(256)])
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def pin_e8m0_decode(orc):
    ref = torch_e8m0_values()
    got = np.array([orc.e8m0_to_double(b) for b in range(256)])
    assert math.isnan(got[255]) and math.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    for b, lg in read_golden("e8m0_decode_points.txt"):
        g = orc.e8m0_to_double(int(b))
        assert (lg == "nan" and math.isnan(g)) or g == 2.0 ** int(lg)


def pin_e2m1_decode(orc):
    got = np.array([orc.e2m1_to_double(n) for n in range(16)])
    assert np.array_equal(got[:8], E2M1_POS)
    assert np.array_equal(got[8:], -E2M1_POS)
    assert np.all(np.signbit(got[8:]))


def pin_e4m3_encode_golden(orc):
    for val, code, *_ in read_golden("e4m3_encode_points.txt"):
        assert orc.double_to_e4m3(float(val)) == int(code, 16), (val, code)


def pin_e4m3_encode_bruteforce(orc):
    """Every bf16 pattern through the E4M3 encoder vs an exhaustive nearest search."""
    v = torch_bf16_values(ALL_BF16)
    fin = np.isfinite(v)
    got = np.array([orc.double_to_e4m3(float(x)) for x in v])
    ref = nearest_code(v[fin], e4m3_pos_values(), 0x80)
    assert np.array_equal(got[fin], ref)
    sign = np.signbit(v).astype(np.int64) * 0x80
    assert np.array_equal(got[np.isnan(v)], (sign | 0x7F)[np.isnan(v)])
    assert np.array_equal(got[np.isinf(v)], (sign | 0x7E)[np.isinf(v)])
    # torch's own cast agrees once clamped (values are exact in fp32)
    assert np.array_equal(got[fin], torch_e4m3_cast(v[fin].astype(np.float32)))


def pin_e2m1_encode(orc):
    for val, code, *_ in read_golden("e2m1_encode_points.txt"):
        assert orc.double_to_e2m1(float(val)) == int(code, 16), (val, code)
    v = torch_bf16_values(ALL_BF16)
    fin = np.isfinite(v)
    got = np.array([orc.double_to_e2m1(float(x)) for x in v[fin]])
    assert np.array_equal(got, nearest_code(v[fin], E2M1_POS, 0x8))


def pin_bf16_round(orc, n_random: int = 100_000):
    """double -> bf16 RNE vs torch's fp32 -> bf16 cast on random fp32 patterns
    (exact in double), plus the boundaries around overflow and subnormals."""
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=n_random, dtype=np.uint64).astype(np.uint32)
    edge = np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0x7F7FFFFF, 0x00008000, 0x00018000,
                     0x00007FFF, 0x00000001, 0x007FFFFF, 0x3F808000, 0x3F818000, 0x80008000],
                    np.uint32)
    bits = np.concatenate([bits, edge])
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.double_to_bf16(float(x)) for x in f], np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# MXFP8 pins
# ---------------------------------------------------------------------------

def mx_sweep_input(scale_bytes=range(0, 247)):
    """Every bf16 magnitude (both signs) that can share a group with scale byte
    s, for each s: groups of 31 test values plus one anchor whose exponent
    field is s + 8 (mantissa all ones, so it is the group's amax)."""
    groups, expect_s = [], []
    for s in scale_bytes:
        e_anchor = s + 8 if s > 0 else 8
        anchor = (e_anchor << 7) | 0x7F
        mags = np.arange(0, anchor + 1, dtype=np.uint32)
        vals = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        pad = (-len(vals)) % 31
        vals = np.concatenate([vals, np.zeros(pad, np.uint16)]).reshape(-1, 31)
        g = np.concatenate([np.full((len(vals), 1), anchor, np.uint16), vals], axis=1)
        groups.append(g)
        expect_s.append(np.full(len(g), s))
    return np.concatenate(groups), np.concatenate(expect_s)


def pin_mx_sweep(orc, scale_bytes=range(0, 247)):
    """Row-wise MXFP8 over every (bf16 value, reachable scale byte) pair vs the
    closed-form scale and an exhaustive nearest search on x / 2^(s-127)."""
    x, s_exp = mx_sweep_input(scale_bytes)
    q, s = orc.mxfp8_quantize_rowwise(x)
    assert np.array_equal(s[:, 0].astype(np.int64), s_exp)
    assert np.array_equal(mx_scale_closed_form(x), s_exp)
    v = torch_bf16_values(x) * np.exp2(127.0 - s_exp)[:, None]  # exact power-of-two shift
    ref = nearest_code_sorted(v.ravel(), e4m3_pos_values(), 0x80).reshape(v.shape)
    assert np.array_equal(q.astype(np.int64), ref)


def pin_mx_nonfinite(orc):
    x = np.zeros((4, 64), np.uint16)
    x[0, :32] = np.arange(32, dtype=np.uint16) | 0x3F00
    x[0, 5] = 0x7FC0                       # NaN in group 0
    x[1, 40] = 0xFF80                      # -Inf in group 1
    x[1, 41] = 0xBF80                      # -1 beside it
    x[2, :] = 0x3F80
    q, s = orc.mxfp8_quantize_rowwise(x)
    assert s[0, 0] == 0xFF and s[1, 1] == 0xFF
    assert s[0, 1] == 0 and s[1, 0] == 0 and s[2, 0] == 127 - 8 + 0  # 1.0: floor(log2)=0
    assert np.all(q[0, :32] == 0x7F)
    assert q[1, 40] == 0xFF and q[1, 41] == 0xFF and q[1, 42] == 0x7F


def pin_mx_edge_groups(orc, x=None):
    import workloads
    if x is None:
        x = workloads.mx_small()
    q, s = orc.mxfp8_quantize_rowwise(x)
    for kind, r, c, want in read_golden("mx_small_edge_groups.txt"):
        r, c, want = int(r), int(c), int(want, 16)
        if kind == "scale":
            assert s[r, c] == want, (r, c)
        elif kind == "allq":
            assert np.all(q[r, 32 * c:32 * c + 32] == want)
        else:
            assert q[r, c] == want, (r, c)
    # every group: closed-form scale; torch cast of x / 2^(s-127) gives the codes
    groups = x.reshape(x.shape[0], -1, 32)
    assert np.array_equal(s.astype(np.int64), mx_scale_closed_form(groups))
    X = np.exp2(s.astype(np.float64) - 127.0)
    v = torch_bf16_values(x).reshape(groups.shape) / X[:, :, None]
    ref = torch_e4m3_cast(v.astype(np.float32)).reshape(x.shape)  # all v are exact in fp32
    assert np.array_equal(q.astype(np.int64), ref)


def mx_saturation_group():
    """The hand-derived saturation group of tests/golden/mx_saturation_group.txt:
    (x bits [1, 32], expected scale byte, expected codes [32])."""
    x = np.zeros((1, 32), np.uint16)
    codes = np.zeros(32, np.int64)
    scale = None
    for parts in read_golden("mx_saturation_group.txt"):
        if parts[0] == "scale":
            scale = int(parts[1], 16)
        else:
            i, bits, code = int(parts[0]), int(parts[1], 16), int(parts[2], 16)
            x[0, i], codes[i] = bits, code
    return x, scale, codes


def pin_mx_saturation(orc):
    """Values at and above E4M3's largest finite 448 saturate to 0x7E with their
    sign (hand-derived golden group)."""
    x, scale, codes = mx_saturation_group()
    q, s = orc.mxfp8_quantize_rowwise(x)
    assert int(s[0, 0]) == scale
    assert np.array_equal(q[0].astype(np.int64), codes)


def pin_mx_max_code_band(orc, x):
    """Power-of-two scale with exponent floor(log2 amax) - 8: the group max maps
    into [256, 512) before rounding, so its code lies in 0x78..0x7E whenever the
    scale byte is not clamped at 0."""
    q, s = orc.mxfp8_quantize_rowwise(x)
    mag = (q.reshape(q.shape[0], -1, 32) & 0x7F).max(axis=-1)
    unclamped = (mx_scale_closed_form(x.reshape(x.shape[0], -1, 32)) > 0) & (s != 0xFF)
    assert np.all((mag[unclamped] >= 0x78) & (mag[unclamped] <= 0x7E))


def pin_mx_padcrop(orc, x):
    q1, s1 = orc.mxfp8_quantize_rowwise(x)
    q2, s2 = orc.mxfp8_quantize_padcrop(x)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def pin_mx_colwise_is_rowwise_of_transpose(orc, x):
    rows, cols = x.shape
    qc, sc = orc.mxfp8_quantize_colwise(x)
    prow = (rows + 31) // 32 * 32
    xp = np.zeros((prow, cols), np.uint16)
    xp[:rows] = x
    qt, st = orc.mxfp8_quantize_rowwise(np.ascontiguousarray(xp.T))
    assert np.array_equal(qc, qt.T[:rows])
    assert np.array_equal(sc, st.T)


def pin_mx_colwise_t_is_rowwise_of_transpose(orc, x):
    """The transposed column-wise layout is row-wise MXFP8 of x transposed
    (rows zero-padded to a multiple of 32, then cropped)."""
    rows, cols = x.shape
    qt, st = orc.mxfp8_quantize_colwise_t(x)
    prow = (rows + 31) // 32 * 32
    xp = np.zeros((prow, cols), np.uint16)
    xp[:rows] = x
    qr, sr = orc.mxfp8_quantize_rowwise(np.ascontiguousarray(xp.T))
    assert np.array_equal(qt, qr[:, :rows])
    assert np.array_equal(st, sr)


def pin_mx_dequant_vs_torch(orc):
    """Every (code, scale byte) pair: bf16 RNE of the exact product, via torch
    (fp32 product is exact here; torch's fp32 -> bf16 cast is RNE)."""
    q = np.tile(np.arange(256, dtype=np.uint8), (256, 1))           # [256 scale rows, 256 codes]
    sc = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 8, axis=1)
    out = orc.mxfp8_dequantize(q, sc, axis=1)
    vals = torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).float()
    e = np.arange(256.0)
    e[255] = 127.0  # byte 0xFF is NaN; its rows are checked separately below
    scales = torch.from_numpy(np.exp2(e - 127.0).astype(np.float32))[:, None]
    ref = (vals * scales).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(torch_e4m3_values())[None, :] | (np.arange(256) == 255)[:, None]
    assert np.array_equal(out[~nan], ref[~nan])
    want_nan = np.where(q >= 0x80, 0xFFC0, 0x7FC0).astype(np.uint16)
    assert np.array_equal(out[nan], want_nan[nan])
    # column-wise axis uses scale [ceil(rows/32), cols]
    qc = np.full((64, 32), 0x38, np.uint8)
    scc = np.zeros((2, 32), np.uint8)
    scc[0, :] = 127
    scc[1, :] = 128
    oc = orc.mxfp8_dequantize(qc, scc, axis=0)
    assert np.all(oc[:32] == 0x3F80) and np.all(oc[32:] == 0x4000)


def pin_mx_roundtrip(orc, x):
    """Idempotence q(dq(q(x))) == q(x) and the round-trip bound:
    |dq - x| <= half an E4M3 ulp of x/X, times X, unless x/X > 464 (saturated:
    |dq - x| = |x| - 448 X)."""
    q, s = orc.mxfp8_quantize_rowwise(x)
    dq = orc.mxfp8_dequantize(q, s, axis=1)
    q2, s2 = orc.mxfp8_quantize_rowwise(dq)
    ok_groups = (s >= 3) | np.all(q.reshape(q.shape[0], -1, 32) & 0x7F == 0, axis=-1)
    okm = np.repeat(ok_groups, 32, axis=1)
    assert np.array_equal(q[okm], q2[okm]) and np.array_equal(s[ok_groups], s2[ok_groups])
    xv = torch_bf16_values(x)
    dv = torch_bf16_values(dq)
    X = np.repeat(np.exp2(s.astype(np.float64) - 127.0), 32, axis=1)
    t = np.abs(xv) / X
    e = np.floor(np.log2(np.maximum(t, 2.0 ** -6)))
    half_ulp = np.exp2(e - 3) / 2 * X
    sat = t > 464
    fin = np.isfinite(xv) & (s != 0xFF).repeat(32, axis=1) & okm
    err = np.abs(dv - xv)
    assert np.all(err[fin & ~sat] <= half_ulp[fin & ~sat])
    assert np.allclose(err[fin & sat], (np.abs(xv) - 448 * X)[fin & sat], rtol=0, atol=0)


# ---------------------------------------------------------------------------
# block-FP8 and NVFP4 pins
# ---------------------------------------------------------------------------

def torch_blockfp8(x: np.ndarray, blk: int, bc: int | None = None):
    """Block-FP8 written with torch ops over blk x bc tiles (square unless bc is
    given): fp32 amax / 448 per tile, fp32 x / S, clamp to +-448 and torch's
    E4M3 cast; zero tiles divide by 1."""
    br = blk
    bc = blk if bc is None else bc
    rows, cols = x.shape
    pr, pc = -(-rows // br) * br, -(-cols // bc) * bc
    xf = torch.zeros((pr, pc), dtype=torch.float32)
    xf[:rows, :cols] = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float()
    tiles = xf.reshape(pr // br, br, pc // bc, bc)
    amax = tiles.abs().amax(dim=(1, 3))
    S = amax / 448.0
    div = torch.where(amax == 0, torch.ones_like(S), S)
    t = tiles / div[:, None, :, None]
    q = t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    q = q.reshape(pr, pc)[:rows, :cols].numpy()
    return q, S.numpy()


def pin_mx_fake_quant(orc, x):
    """Fake quantization equals the dequantization of the quantization along
    the same axis (row groups with row scales, column groups with column
    scales), composed here from the separately pinned steps."""
    for axis in (0, 1):
        fq = orc.mxfp8_fake_quant(x, axis)
        q, s = orc.mxfp8_quantize_rowwise(x) if axis == 1 else orc.mxfp8_quantize_colwise(x)
        assert np.array_equal(fq, orc.mxfp8_dequantize(q, s, axis)), axis


def pin_blockfp8_1x128(orc, x):
    """1 x 128 activation blocks: torch composition, the row-group max maps to
    0x7E, dequantization via torch products, fake quant = dequant(quant)."""
    q, S = orc.blockfp8_quantize_rect(x, 1, 128)
    rq, rS = torch_blockfp8(x, 1, 128)
    assert np.array_equal(S.view(np.uint32), rS.view(np.uint32))
    assert np.array_equal(q, rq)
    rows, cols = x.shape
    mag = x.astype(np.int64) & 0x7FFF
    for j in range(S.shape[1]):
        blk = mag[:, 128 * j:128 * j + 128]
        r = np.nonzero(blk.max(axis=1) > 0)[0]
        c = np.argmax(blk[r], axis=1) + 128 * j
        assert np.all((q[r, c] & 0x7F) == 0x7E)
    dq = orc.blockfp8_dequantize_rect(q, S, 1, 128)
    Sx = np.repeat(S, 128, axis=1)[:, :cols]
    v = torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).float() * torch.from_numpy(Sx)
    assert np.array_equal(dq, v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(orc.blockfp8_fake_quant_1x128(x), dq)


def pin_blockfp8(orc, x, blk=128):
    q, S = orc.blockfp8_quantize(x, blk)
    rq, rS = torch_blockfp8(x, blk)
    assert np.array_equal(S.view(np.uint32), rS.view(np.uint32))
    assert np.array_equal(q, rq)
    # each tile's max-magnitude element maps to +-448 (0x7E)
    rows, cols = x.shape
    for bi in range(S.shape[0]):
        for bj in range(S.shape[1]):
            tile = x[bi * blk:(bi + 1) * blk, bj * blk:(bj + 1) * blk].astype(np.int64) & 0x7FFF
            if tile.max() == 0:
                continue
            r, c = np.unravel_index(np.argmax(tile), tile.shape)
            assert q[bi * blk + r, bj * blk + c] & 0x7F == 0x7E
    # dequantization: fp32 product then bf16 RNE, via torch
    dq = orc.blockfp8_dequantize(q, S, blk)
    Sx = np.repeat(np.repeat(S, blk, 0), blk, 1)[:rows, :cols]
    v = torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).float() * torch.from_numpy(Sx)
    ref = v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(dq, ref)


def numpy_nvfp4(x: np.ndarray):
    """NVFP4 written step by step in numpy fp32 scalars/arrays with torch's E4M3
    cast and a nearest search for E2M1."""
    rows, cols = x.shape
    xv = torch_bf16_values(x)
    A = np.float32(np.abs(xv).max())
    g = np.float32(A / np.float32(2688.0))
    blocks = np.abs(xv).reshape(rows, cols // 16, 16).max(axis=-1).astype(np.float32)
    if A == 0:
        s = np.zeros_like(blocks, dtype=np.int64)
    else:
        d = np.float32(np.float32(6.0) * g)
        ratio = (blocks / d).astype(np.float32)
        s = torch_e4m3_cast(ratio)
    sval = torch_e4m3_values()[s].astype(np.float32)
    eff = (sval * g).astype(np.float32)
    effx = np.repeat(eff, 16, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (xv.astype(np.float32) / effx).astype(np.float32)
    nib = nearest_code_sorted(t.astype(np.float64).ravel(), E2M1_POS, 0x8).reshape(rows, cols)
    nib = np.where(effx == 0, (np.signbit(xv).astype(np.int64) * 0x8), nib)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return packed, s.astype(np.uint8), np.array([g], np.float32)


def pin_nvfp4(orc, x):
    q, s, g = orc.nvfp4_quantize(x)
    rq, rs, rg = numpy_nvfp4(x)
    assert g.view(np.uint32)[0] == rg.view(np.uint32)[0]
    assert np.array_equal(s, rs)
    assert np.array_equal(q, rq)
    # the block holding the global amax gets scale 0x7E and its max nibble is 6
    mag = x.astype(np.int64) & 0x7FFF
    if mag.max() > 0:
        r, c = np.unravel_index(np.argmax(mag), mag.shape)
        assert s[r, c // 16] == 0x7E
        nib = (q[r, c // 2] >> (4 * (c % 2))) & 0xF
        assert nib & 0x7 == 0x7
    # dequantization, fp32 products then bf16 RNE, via torch
    dq = orc.nvfp4_dequantize(q, s, g)
    nibs = np.stack([q & 0xF, q >> 4], axis=-1).reshape(x.shape[0], -1)
    ev = torch.from_numpy(E2M1_POS.astype(np.float32))[torch.from_numpy((nibs & 7).astype(np.int64))]
    ev = torch.where(torch.from_numpy(nibs >= 8), -ev, ev)
    sv = torch.from_numpy(s.copy()).view(torch.float8_e4m3fn).float() * float(g[0])
    ref = (ev * sv.repeat_interleave(16, dim=1)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(dq, ref)


# ---------------------------------------------------------------------------
# MXFP4 pins
# ---------------------------------------------------------------------------

def unpack_nibbles(q: np.ndarray) -> np.ndarray:
    """[rows, cols/2] packed bytes -> [rows, cols] nibbles, element 2j from the
    low nibble of byte j."""
    n = np.empty((q.shape[0], 2 * q.shape[1]), np.int64)
    n[:, 0::2] = q & 0xF
    n[:, 1::2] = q >> 4
    return n


def mx4_scale_closed_form(group_bits: np.ndarray) -> np.ndarray:
    """E8M0 byte straight from bf16 bits: max(expfield(max magnitude) - 2, 0);
    0xFF when the group holds Inf/NaN."""
    mag = (group_bits.astype(np.int64) & 0x7FFF).max(axis=-1)
    e = mag >> 7
    return np.where(e == 0xFF, 0xFF, np.maximum(e - 2, 0))


def mx4_sweep_input(scale_bytes=range(0, 253)):
    """Every bf16 magnitude (both signs) that can share a group with scale byte
    s: groups of 31 test values plus one anchor whose exponent field is s + 2
    (mantissa all ones, so it is the group's amax)."""
    groups, expect_s = [], []
    for s in scale_bytes:
        e_anchor = s + 2 if s > 0 else 2
        anchor = (e_anchor << 7) | 0x7F
        mags = np.arange(0, anchor + 1, dtype=np.uint32)
        vals = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        pad = (-len(vals)) % 31
        vals = np.concatenate([vals, np.zeros(pad, np.uint16)]).reshape(-1, 31)
        g = np.concatenate([np.full((len(vals), 1), anchor, np.uint16), vals], axis=1)
        groups.append(g)
        expect_s.append(np.full(len(g), s))
    return np.concatenate(groups), np.concatenate(expect_s)


def pin_mx4_sweep(orc, scale_bytes=range(0, 253)):
    """MXFP4 over every (bf16 value, reachable scale byte) pair vs the closed-form
    scale and an exhaustive nearest search over the E2M1 values of x / 2^(s-127)."""
    x, s_exp = mx4_sweep_input(scale_bytes)
    q, s = orc.mxfp4_quantize(x)
    assert np.array_equal(s[:, 0].astype(np.int64), s_exp)
    assert np.array_equal(mx4_scale_closed_form(x), s_exp)
    v = torch_bf16_values(x) * np.exp2(127.0 - s_exp)[:, None]  # exact power-of-two shift
    ref = nearest_code(v.ravel(), E2M1_POS, 0x8).reshape(v.shape)
    assert np.array_equal(unpack_nibbles(q), ref)


def pin_mx4_nonfinite(orc):
    x = np.zeros((3, 64), np.uint16)
    x[0, :32] = np.arange(32, dtype=np.uint16) | 0x3F00
    x[0, 5] = 0x7FC0                       # NaN in group 0
    x[1, 40] = 0xFF80                      # -Inf in group 1
    x[1, 41] = 0xBF80                      # -1 beside it
    x[2, :] = 0x3F80                       # 1.0: byte floor(log2 1) - 2 + 127 = 125, nibble 4 -> 0x6
    q, s = orc.mxfp4_quantize(x)
    n = unpack_nibbles(q)
    assert s[0, 0] == 0xFF and s[1, 1] == 0xFF and s[0, 1] == 0 and s[1, 0] == 0
    assert np.all(n[0, :32] == 0x7)
    assert n[1, 40] == 0xF and n[1, 41] == 0xF and n[1, 42] == 0x7
    assert np.all(s[2] == 125) and np.all(n[2] == 0x6)
    # packing: element 2j in the low nibble (1.0 and 4.0 with scale 1 -> 0x62)
    y = np.zeros((1, 32), np.uint16)
    y[0, 0], y[0, 1] = 0x3F80, 0x4080
    qy, sy = orc.mxfp4_quantize(y)
    assert sy[0, 0] == 127 and qy[0, 0] == 0x62 and np.all(qy[0, 1:] == 0)


def pin_mx4_edge_groups(orc, x=None):
    import workloads
    if x is None:
        x = workloads.mx_small()
    q, s = orc.mxfp4_quantize(x)
    n = unpack_nibbles(q)
    for kind, r, c, want in read_golden("mxfp4_small_edge_groups.txt"):
        r, c, want = int(r), int(c), int(want, 16)
        if kind == "scale":
            assert s[r, c] == want, (r, c)
        elif kind == "allb":
            assert np.all(q[r, 16 * c:16 * c + 16] == want), (r, c)
        else:
            assert n[r, c] == want, (r, c)
    assert np.array_equal(s.astype(np.int64), mx4_scale_closed_form(x.reshape(x.shape[0], -1, 32)))


def pin_mx4_max_nibble(orc, x):
    """Scale exponent floor(log2 amax) - 2 puts the group max in [4, 8) before
    rounding, so its nibble magnitude is 0x6 (4) or 0x7 (6) unless the scale
    byte is clamped at 0."""
    q, s = orc.mxfp4_quantize(x)
    mag = (unpack_nibbles(q).reshape(x.shape[0], -1, 32) & 0x7).max(axis=-1)
    unclamped = (mx4_scale_closed_form(x.reshape(x.shape[0], -1, 32)) > 0) & (s != 0xFF)
    assert np.all((mag[unclamped] == 0x6) | (mag[unclamped] == 0x7))


def pin_mx4_dequant_vs_torch(orc):
    """Every (nibble, scale byte) pair: bf16 RNE of E2M1 value * 2^(b-127) via
    torch's fp32 product and cast (exact here, subnormals kept)."""
    nib = np.tile(np.arange(16, dtype=np.uint8), (256, 2))              # [256, 32] nibbles
    q = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)          # [256, 16] packed
    sc = np.arange(256, dtype=np.uint8)[:, None].copy()                 # one group per row
    out = orc.mxfp4_dequantize(q, sc)
    ev = np.where(nib >= 8, -E2M1_POS[nib & 7], E2M1_POS[nib & 7]).astype(np.float32)
    e = np.arange(256.0)
    e[255] = 127.0
    X = np.exp2(e - 127.0).astype(np.float32)[:, None]
    with np.errstate(over="ignore"):   # 6 * 2^127 overflows to Inf, as bf16 RNE does
        ref = torch.from_numpy(ev * X).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out[:255], ref[:255])
    assert np.array_equal(out[255], np.where(nib[255] >= 8, 0xFFC0, 0x7FC0).astype(np.uint16))


def pin_mx4_roundtrip(orc, x):
    """Idempotence q(dq(q(x))) == q(x) (E2M1 times a power of two is exact in
    bf16, so dq re-quantizes to itself) and the round-trip bound: |dq - x| <=
    half an E2M1 ulp of x/X (0.5 below 2, 1 below 4, 2 up to 6), times X,
    unless x/X > 6 (saturated: |dq - x| = |x| - 6 X); fake-quant equals
    dequantize(quantize(x))."""
    q, s = orc.mxfp4_quantize(x)
    dq = orc.mxfp4_dequantize(q, s)
    assert np.array_equal(orc.mxfp4_fake_quant(x), dq)
    fin_g = s != 0xFF
    q2, s2 = orc.mxfp4_quantize(dq)
    fm = np.repeat(fin_g, 16, axis=1)
    assert np.array_equal(s[fin_g], s2[fin_g]) and np.array_equal(q[fm], q2[fm])
    xv = torch_bf16_values(x)
    dv = torch_bf16_values(dq)
    X = np.repeat(np.exp2(s.astype(np.float64) - 127.0), 32, axis=1)
    t = np.abs(xv) / X
    half_ulp = np.where(t < 2, 0.25, np.where(t < 4, 0.5, 1.0)) * X
    sat = t > 6
    fin = np.isfinite(xv) & np.repeat(fin_g, 32, axis=1)
    err = np.abs(dv - xv)
    assert np.all(err[fin & ~sat] <= half_ulp[fin & ~sat])
    assert np.array_equal(err[fin & sat], (np.abs(xv) - 6 * X)[fin & sat])


# ---------------------------------------------------------------------------
# FP8 block -> BF16 -> MXFP8 re-quantization pins
# ---------------------------------------------------------------------------

def pin_requant_pow2_tiles(orc, rows=256, cols=384, seed=8):
    """Closed form: with a power-of-two tile scale S = 2^k, the bf16
    intermediate is exactly E4M3(q) * 2^k, and every MX group whose largest
    code magnitude lies in [256, 448] (codes 0x78..0x7E) gets scale byte
    k + 127 and its input codes back unchanged."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 256, size=(rows, cols)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x7E                      # no NaN codes
    tr, tc = -(-rows // 128), -(-cols // 128)
    k = rng.integers(-20, 20, size=(tr, tc))
    S = np.exp2(k.astype(np.float64)).astype(np.float32)
    q8, s8 = orc.blockfp8_to_mxfp8(q, S)
    gmax = (q.reshape(rows, cols // 32, 32) & 0x7F).max(axis=-1)
    kk = np.repeat(np.repeat(k, 128, 0), 128, 1)[:rows, :cols][:, ::32]
    big = (gmax >= 0x78) & (gmax <= 0x7E)
    assert big.any()
    assert np.array_equal(s8[big].astype(np.int64), kk[big] + 127)
    bm = np.repeat(big, 32, axis=1)
    assert np.array_equal(q8[bm], q[bm])


def pin_requant_matches_steps(orc, x):
    """Against torch: the block-FP8 dequantization as torch fp32 products and
    its bf16 cast, then the row-wise MXFP8 of that bf16 tensor through the
    (separately pinned) row-wise oracle."""
    q, S = orc.blockfp8_quantize(x, 128)
    rows, cols = q.shape
    Sx = np.repeat(np.repeat(S, 128, 0), 128, 1)[:rows, :cols]
    v = torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).float() * torch.from_numpy(Sx)
    bf = v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q8, s8 = orc.blockfp8_to_mxfp8(q, S)
    rq, rs = orc.mxfp8_quantize_rowwise(bf)
    assert np.array_equal(q8, rq) and np.array_equal(s8, rs)


def pin_nvfp4_grouped(orc, xs, groups, n_groups):
    """Grouped NVFP4: each group's g is fl32(max over its members / 2688) (the
    numpy composition), each member equals single-tensor NVFP4 of that member
    after the group's largest value is planted into a copy of it (which makes
    the single-tensor amax the group's, leaving every other block unchanged),
    and a one-tensor group equals nvfp4_quantize exactly."""
    outs, gs = orc.nvfp4_quantize_grouped(xs, groups, n_groups)
    mags = [torch_bf16_values(x) for x in xs]
    for j in range(n_groups):
        members = [i for i in range(len(xs)) if groups[i] == j]
        if not members:
            assert gs[j] == 0
            continue
        A = np.float32(max(np.abs(mags[i]).max() for i in members))
        assert gs[j].view(np.uint32) == np.float32(A / np.float32(2688.0)).view(np.uint32)
        for i in members:
            q, s = outs[i]
            if len(members) == 1:
                rq, rs, rg = orc.nvfp4_quantize(xs[i])
                assert np.array_equal(q, rq) and np.array_equal(s, rs)
                continue
            # plant the group max into an extra block-aligned row of this member
            x = xs[i]
            amax_bits = max((xs[k].astype(np.int64) & 0x7FFF).max() for k in members)
            extra = np.zeros((1, x.shape[1]), np.uint16)
            extra[0, 0] = amax_bits
            rq, rs, rg = orc.nvfp4_quantize(np.concatenate([x, extra]))
            assert rg.view(np.uint32)[0] == gs[j].view(np.uint32)
            assert np.array_equal(q, rq[:-1]) and np.array_equal(s, rs[:-1])


def pin_blockfp8_gkn(orc, x3):
    """[G, K, N] block-FP8: every slice equals the torch composition of
    128 x 128 block-FP8 on that slice alone (no tile crosses a slice), and
    dequantization per slice matches torch's products."""
    q, S = orc.blockfp8_quantize_gkn(x3)
    dq = orc.blockfp8_dequantize_gkn(q, S)
    for g in range(x3.shape[0]):
        rq, rS = torch_blockfp8(np.ascontiguousarray(x3[g]), 128)
        assert np.array_equal(S[g].view(np.uint32), rS.view(np.uint32))
        assert np.array_equal(q[g], rq)
        K, N = x3.shape[1:]
        Sx = np.repeat(np.repeat(S[g], 128, 0), 128, 1)[:K, :N]
        v = torch.from_numpy(q[g].copy()).view(torch.float8_e4m3fn).float() * torch.from_numpy(Sx)
        assert np.array_equal(dq[g], v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
