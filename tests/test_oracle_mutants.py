"""Plant one mistake at a time in a copy of the oracle's C source (on the CPU)
and check that the pins catch it: each mutant must fail at least one pin."""
import numpy as np
import pytest

import oracle
import pins
import workloads

# (name, exact text in the oracle source, replacement)
MUTANTS = [
    ("scale exponent off by one", "floor_log2(amax) - 8;", "floor_log2(amax) - 7;"),
    ("scale clamp at 2^-126", "E4M3's largest power of two */\n    if (E < -127) E = -127;",
     "E4M3's largest power of two */\n    if (E < -126) E = -126;"),
    ("zero group scale 1.0", "if (amax == 0.0) return 0;\n    int E = floor_log2(amax) - 8;",
     "if (amax == 0.0) return 127;\n    int E = floor_log2(amax) - 8;"),
    ("Inf not a NaN group",
     "mx_scale_byte(const double *vals, int n)\n{\n    double amax = 0.0;\n    for (int i = 0; i < n; ++i) {\n        double a = fabs(vals[i]);\n        if (!isfinite(a)) return 0xFF;",
     "mx_scale_byte(const double *vals, int n)\n{\n    double amax = 0.0;\n    for (int i = 0; i < n; ++i) {\n        double a = fabs(vals[i]);\n        if (isnan(a)) return 0xFF;"),
    ("mxfp4 Inf not a NaN group",
     "mx4_scale_byte(const double *vals, int n)\n{\n    double amax = 0.0;\n    for (int i = 0; i < n; ++i) {\n        double a = fabs(vals[i]);\n        if (!isfinite(a)) return 0xFF;",
     "mx4_scale_byte(const double *vals, int n)\n{\n    double amax = 0.0;\n    for (int i = 0; i < n; ++i) {\n        double a = fabs(vals[i]);\n        if (isnan(a)) return 0xFF;"),
    ("E4M3 ties away from zero",
     "double quantum = ldexp(1.0, E - 3);     /* 3 fraction bits */\n    double n = nearbyint(a / quantum);",
     "double quantum = ldexp(1.0, E - 3);     /* 3 fraction bits */\n    double n = round(a / quantum);"),
    ("E4M3 subnormal quantum", "if (E < -6) E = -6; ", "if (E < -7) E = -7; "),
    ("E4M3 no saturation below 480", "if (r > 448.0) return sign | 0x7E;", "if (r > 480.0) return sign | 0x7E;"),
    ("E4M3 drops sign of small codes", "if (r < ldexp(1.0, -6)) return sign | (uint8_t)n;",
     "if (r < ldexp(1.0, -6)) return (uint8_t)n;"),
    ("bf16 rounding flushes subnormals", "if (E < -126) E = -126;", "if (E < -126) return sign;"),
    ("dequant scale index", "axis == 1 ? scale[r * (cols / MX_GROUP) + c / MX_GROUP]",
     "axis == 1 ? scale[r * (cols / MX_GROUP) + (c % (cols / MX_GROUP))]"),
    ("mxfp4 dequant scale index", "uint8_t s = scale[r * (cols / MX_GROUP) + c / MX_GROUP];",
     "uint8_t s = scale[r * (cols / MX_GROUP) + (c % (cols / MX_GROUP))];"),
    ("colwise scale transposed", "scale[j * cols + c] = s;", "scale[c * nrg + j] = s;"),
    ("colwise_t scale index", "st[c * nrg + j] = s[j * cols + c];", "st[c * nrg + j] = s[c];"),
    ("requant skips the bf16 rounding", "    orc_blockfp8_dequantize(q, scale, rows, cols, blk, bf);\n    orc_mxfp8_quantize_rowwise(bf, rows, cols, q8, scale8);",
     "    orc_blockfp8_dequantize(q, scale, rows, cols, blk, bf);\n    for (int64_t i = 0; i < rows * cols; ++i) bf[i] = (uint16_t)(bf[i] & 0xFFF0);\n    orc_mxfp8_quantize_rowwise(bf, rows, cols, q8, scale8);"),
    ("rect tiles index rows by bc", "float S = scale[(r / br) * tc + c / bc];",
     "float S = scale[(r / bc) * tc + c / bc];"),
    ("nvfp4 group amax over the first member only",
     "for (int32_t i = 0; i < n; ++i) nv_amax(xs[i], rows[i] * cols[i], &A[group[i]], &nf[group[i]]);",
     "for (int32_t i = 0; i < n; ++i) if (A[group[i]] == 0.0) nv_amax(xs[i], rows[i] * cols[i], &A[group[i]], &nf[group[i]]);"),
    ("gkn tiles cross slices", "orc_blockfp8_quantize(x + g * K * N, K, N, blk, q + g * K * N, scale + g * ts);",
     "orc_blockfp8_quantize(x + g * K * N, K, N, blk, q + g * K * N, scale + g * ts);\n    if (G > 1 && K % blk) orc_blockfp8_quantize(x, G * K, N, blk, q, scale);"),
    ("colwise group stride", "q[(r0 + i) * cols + c] = mx_encode(g[i], s);",
     "q[(r0 + i) * cols + c] = mx_encode(g[i], (uint8_t)(s + (i == 31)));"),
    ("blockfp8 divisor 447", "S = (float)amax / 448.0f;", "S = (float)amax / 447.0f;"),
    ("blockfp8 zero tile unguarded", "divisor = (amax == 0.0) ? 1.0f : S;", "divisor = S;"),
    ("blockfp8 reciprocal multiply", "float t = xf / divisor;", "float t = xf * (1.0f / divisor);"),
    ("nvfp4 global 2687", "float g = (float)A / 2688.0f;", "float g = (float)A / 2687.0f;"),
    ("nvfp4 nibble order", "                    (uint8_t)(nib[i] | (nib[i + 1] << 4));",
     "                    (uint8_t)(nib[i + 1] | (nib[i] << 4));"),
    ("mxfp4 scale exponent -1", "int E = floor_log2(amax) - 2;", "int E = floor_log2(amax) - 1;"),
    ("mxfp4 nibble order", "/ 2] = (uint8_t)(nib[i] | (nib[i + 1] << 4));",
     "/ 2] = (uint8_t)(nib[i + 1] | (nib[i] << 4));"),
    ("mxfp4 NaN group nibble", "? (uint8_t)((signbit(g[i]) ? 0x8 : 0) | 0x7)",
     "? (uint8_t)((signbit(g[i]) ? 0x8 : 0) | 0x6)"),
    ("mxfp4 dequant reads the high nibble first", "(c % 2 == 0) ? (byte & 0xF) : (byte >> 4);",
     "(c % 2 == 0) ? (byte >> 4) : (byte & 0xF);"),
    ("mxfp4 scale clamp at 2^-126", "E2M1's largest power of two */\n    if (E < -127) E = -127;",
     "E2M1's largest power of two */\n    if (E < -126) E = -126;"),
    ("mxfp4 zero group scale 1.0", "if (amax == 0.0) return 0;\n    int E = floor_log2(amax) - 2;",
     "if (amax == 0.0) return 127;\n    int E = floor_log2(amax) - 2;"),
    ("nvfp4 eff divides", "float eff = (float)orc_e4m3_to_double(s) * g;",
     "float eff = (float)orc_e4m3_to_double(s) / g;"),
    ("nvfp4 block scale without 6", "float d = 6.0f * g;", "float d = 4.0f * g;"),
    ("e2m1 saturates at 4", "if (r > 6.0) return sign | 0x7;", "if (r > 4.0) return sign | 0x6;"),
    ("e2m1 quantum", "if (E < 0) E = 0; ", "if (E < -1) E = -1; "),
    ("dequant NaN sign", "o = (uint16_t)((code & 0x80) ? 0xFFC0 : 0x7FC0);", "o = (uint16_t)0x7FC0;"),
    ("fake-quant axis 0 dequantizes along rows", "orc_mxfp8_dequantize(q, s, rows, cols, axis, out);",
     "orc_mxfp8_dequantize(q, s, rows, cols, 1, out);"),
    ("1x128 fake-quant dequantizes with 128x128 tile scales",
     "orc_blockfp8_dequantize_rect(q, S, rows, cols, 1, 128, out);",
     "orc_blockfp8_dequantize_rect(q, S, rows, cols, 128, 128, out);"),
    ("grouped NVFP4 encodes with group 0's scale",
     "nv_quantize_given(xs[i], rows[i], cols[i], gs[group[i]], nf[group[i]], qs[i], ss[i]);",
     "nv_quantize_given(xs[i], rows[i], cols[i], gs[0], nf[0], qs[i], ss[i]);"),
]


def all_pins(orc):
    """Every pin, at sizes that keep one pass to a few seconds."""
    pins.pin_bf16_decode(orc)
    pins.pin_e4m3_decode(orc)
    pins.pin_e8m0_decode(orc)
    pins.pin_e2m1_decode(orc)
    pins.pin_e4m3_encode_golden(orc)
    pins.pin_e4m3_encode_bruteforce(orc)
    pins.pin_e2m1_encode(orc)
    pins.pin_bf16_round(orc, n_random=20_000)
    pins.pin_mx_sweep(orc, scale_bytes=list(range(0, 24)) + list(range(24, 247, 11)))
    pins.pin_mx_nonfinite(orc)
    pins.pin_mx_edge_groups(orc)
    pins.pin_mx_saturation(orc)
    x = workloads.random_bf16((97, 256), 17)
    pins.pin_mx_max_code_band(orc, x)
    pins.pin_mx_padcrop(orc, x)
    pins.pin_mx_colwise_is_rowwise_of_transpose(orc, workloads.random_bf16((70, 96), 18))
    pins.pin_mx_colwise_t_is_rowwise_of_transpose(orc, workloads.random_bf16((70, 96), 18))
    pins.pin_mx_dequant_vs_torch(orc)
    pins.pin_mx_roundtrip(orc, workloads.mx_small())
    pins.pin_mx_fake_quant(orc, workloads.random_bf16((70, 96), 19))
    pins.pin_blockfp8(orc, workloads.random_bf16((200, 300), 19), 128)
    z = workloads.random_bf16((128, 256), 20)
    z[:, :128] = 0
    pins.pin_blockfp8(orc, z, 128)
    pins.pin_nvfp4(orc, workloads.random_bf16((64, 256), 21))
    pins.pin_requant_pow2_tiles(orc)
    pins.pin_blockfp8_gkn(orc, workloads.random_bf16((3 * 200, 136), 900).reshape(3, 200, 136))
    hx = [workloads.random_bf16((32, 64), 600 + i, std=0.02 * (1 + i)) for i in range(4)]
    pins.pin_nvfp4_grouped(orc, hx, [0, 0, 1, 1], 3)
    y = workloads.random_bf16((33, 200), 533)
    y[3, :128] = 0
    pins.pin_blockfp8_1x128(orc, y)
    pins.pin_requant_matches_steps(orc, workloads.random_bf16((200, 384), 17))
    pins.pin_mx4_sweep(orc, scale_bytes=list(range(0, 20)) + list(range(20, 253, 13)))
    pins.pin_mx4_nonfinite(orc)
    pins.pin_mx4_edge_groups(orc)
    pins.pin_mx4_max_nibble(orc, x)
    pins.pin_mx4_dequant_vs_torch(orc)
    pins.pin_mx4_roundtrip(orc, workloads.mx_small())


def test_unmutated_source_passes_all_pins(tmp_path):
    all_pins(oracle.build_variant(oracle.source_text(), str(tmp_path / "orc_same.so")))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = oracle.source_text()
    assert src.count(old) == 1, f"mutation site not unique/found: {old!r}"
    orc = oracle.build_variant(src.replace(old, new), str(tmp_path / "orc_mut.so"))
    with pytest.raises(AssertionError):
        with np.errstate(all="ignore"):
            all_pins(orc)
