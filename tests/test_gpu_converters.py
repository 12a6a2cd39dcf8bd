"""Every fp32 input the kernels can give the library's fp32 -> E4M3, E2M1 and
bf16 converters, through those converters on the GPU, against the CPU
oracle's encoders (bit for bit).

The block-FP8 (128 x 128 and 1 x 128), NVFP4, FP8 -> MXFP8 and dequantization
paths round full-precision fp32 values -- quotients x / S and x / eff, block
scale ratios b / (6g), fp32 products -- with gfx950 converts or with bit
arithmetic (mxq_device.hpp).  These sweeps cover each converter's whole input
domain, pattern by pattern:

  cvt_fp8x2_f32 (v_cvt_pk_fp8_f32 after a clamp to +-448) and
  e4m3_mag_from_f32: every fp32 in [0, 512] and its negation, then every
      4099th pattern up to +Inf (quotients x / S stay within 448 (1 + 2^-23);
      the NVFP4 block-scale ratio b / (6g) within a few ulps of 449);
  cvt_fp4x2_f32 (v_cvt_scalef32_pk_fp4_f32, scale 1) and e2m1_mag_from_f32:
      every fp32 in [0, 16] and its negation, then every 4099th pattern up to
      +Inf (x / eff stays below 9: eff is the block scale's E4M3 rounding
      times g);
  bf16x2_rne (v_cvt_pk_bf16_f32) and bf16_rne: every non-NaN fp32 (both
      signs; products of any size, subnormals and overflow to Inf included).

NaN never reaches these converters (the kernels route NaN groups, tiles and
tensors to their own exact code).  The oracle runs over host threads; the
comparison happens on the GPU, one chunk of patterns at a time.
"""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import announce, parallel_map

pytestmark = pytest.mark.gpu

CHUNK = 1 << 26


@pytest.fixture(scope="module")
def sweep(gpu):
    import sweep_lib
    return sweep_lib.load()


def _oracle(orc, fmt, first, n, stride):
    """The oracle's encodings of patterns first + i * stride, over host threads."""
    out = np.empty((n,), np.uint16 if fmt == "bf16" else np.uint8)
    parts = 64
    step = -(-n // parts)
    spans = [(a, min(n, a + step)) for a in range(0, n, step)]

    def run(span):
        a, b = span
        orc.f32_bits_to(fmt, first + a * stride, b - a, stride, out=out[a:b])

    parallel_map(run, spans)
    return out


def _first_mismatch(name, ok, first, stride, got, want):
    bad = torch.nonzero(~ok).flatten()[:6].cpu().tolist()
    rows = [(hex(first + i * stride), hex(int(got[i])), hex(int(want[i]))) for i in bad]
    raise AssertionError(f"{name}: {int((~ok).sum())} mismatching patterns; first "
                         f"(pattern, got, want): {rows}")


def _run(sweep, orc, fmt, first, n, stride=1):
    """One run of patterns, in chunks: device converters against the oracle."""
    fn = getattr(sweep, f"cvt_sweep_{fmt}")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for c0 in range(0, n, CHUNK):
        m = min(CHUNK, n - c0)
        f0 = first + c0 * stride
        hw = torch.empty((m,), dtype=torch.int32, device="cuda")
        sw = torch.empty((m,), dtype=torch.int16 if fmt == "bf16" else torch.uint8,
                         device="cuda")
        rc = fn(f0, m, stride, ctypes.c_void_p(hw.data_ptr()), ctypes.c_void_p(sw.data_ptr()),
                stream)
        assert rc == 0, f"cvt_sweep_{fmt} launch status {rc}"
        want_h = _oracle(orc, fmt, f0, m, stride)
        if fmt == "bf16":
            want = torch.from_numpy(want_h.view(np.int16)).to("cuda").to(torch.int32) & 0xFFFF
            hwl = hw & 0xFFFF
            hwh = (hw >> 16) & 0xFFFF
            checks = {"bf16x2_rne(t) low half": (hwl, want),
                      "bf16x2_rne(-t) high half": (hwh, want | 0x8000),
                      "bf16_rne(t)": (sw.to(torch.int32) & 0xFFFF, want)}
        else:
            want = torch.from_numpy(want_h).to("cuda").to(torch.int32)
            b = [(hw >> (8 * k)) & 0xFF for k in range(4)]
            if fmt == "e4m3":
                neg = want | 0x80
                checks = {"cvt_fp8x2_f32 lo(t)": (b[0], want), "cvt_fp8x2_f32 lo(-t)": (b[1], neg),
                          "cvt_fp8x2_f32 hi(-t)": (b[2], neg), "cvt_fp8x2_f32 hi(t)": (b[3], want),
                          "e4m3_mag_from_f32(t)": (sw.to(torch.int32), want)}
            else:
                neg = want | 0x8
                checks = {"cvt_fp4x2_f32 byte0 (t, -t)": (b[0], want | (neg << 4)),
                          "cvt_fp4x2_f32 byte1 (-t, t)": (b[1], neg | (want << 4)),
                          "cvt_fp4x2_f32 byte2 (t, t)": (b[2], want | (want << 4)),
                          "cvt_fp4x2_f32 byte3 (-t, -t)": (b[3], neg | (neg << 4)),
                          "e2m1_mag_from_f32(t)": (sw.to(torch.int32), want)}
        for name, (got, exp) in checks.items():
            ok = got == exp
            if not bool(ok.all()):
                _first_mismatch(f"{fmt} {name}", ok, f0, stride, got, exp)
        del hw, sw, want


def _oracle_is_sign_symmetric(orc, fmt, first, n):
    """The expectations for -t are the oracle's code for t with the sign bit
    set; check that reading on a slice of the negative patterns."""
    pos = _oracle(orc, fmt, first, n, 1).astype(np.int64)
    neg = _oracle(orc, fmt, first | 0x80000000, n, 1).astype(np.int64)
    bit = {"e4m3": 0x80, "e2m1": 0x8, "bf16": 0x8000}[fmt]
    assert np.array_equal(neg, pos | bit)


@pytest.mark.timeout(900)
def test_fp32_to_e4m3_every_input(sweep, orc):
    _oracle_is_sign_symmetric(orc, "e4m3", 0x43DF0000, 1 << 20)
    announce("converter sweep: fp32 -> E4M3, [0, 512]")
    _run(sweep, orc, "e4m3", 0, 0x44000000 + 1)
    announce("converter sweep: fp32 -> E4M3, (512, +Inf] sampled")
    _run(sweep, orc, "e4m3", 0x44000000, (0x7F800000 - 0x44000000) // 4099 + 1, 4099)
    _run(sweep, orc, "e4m3", 0x7F7FFFFF, 2)   # the largest finite value and +Inf


@pytest.mark.timeout(900)
def test_fp32_to_e2m1_every_input(sweep, orc):
    _oracle_is_sign_symmetric(orc, "e2m1", 0x40BF0000, 1 << 20)
    announce("converter sweep: fp32 -> E2M1, [0, 16]")
    _run(sweep, orc, "e2m1", 0, 0x41800000 + 1)
    announce("converter sweep: fp32 -> E2M1, (16, +Inf] sampled")
    _run(sweep, orc, "e2m1", 0x41800000, (0x7F800000 - 0x41800000) // 4099 + 1, 4099)
    _run(sweep, orc, "e2m1", 0x7F7FFFFF, 2)


@pytest.mark.timeout(1200)
def test_fp32_to_bf16_every_input(sweep, orc):
    _oracle_is_sign_symmetric(orc, "bf16", 0x3F7F0000, 1 << 20)
    announce("converter sweep: fp32 -> bf16, every non-NaN pattern")
    _run(sweep, orc, "bf16", 0, 0x7F800000 + 1)
