"""CPU oracle for the block-scaled quantizers -- TEST INFRASTRUCTURE ONLY.

The C file ``mxq_oracle.c`` beside this module is the plain single-threaded
definition of every output byte (MXFP8 row-/column-wise with pad-then-crop,
dequantization and fake-quant, grouped row-wise, MXFP4, 128x128 block-FP8,
NVFP4).
This module only marshals numpy arrays into it through ctypes.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  The HIP product path never imports it and the
two share no code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxq_oracle.c")
_LIB = os.path.join(_HERE, "libmxq_oracle.so")

# Strict IEEE: no contraction into FMA, no fast-math, SSE arithmetic (x86-64
# default, FLT_EVAL_METHOD == 0), no flush-to-zero.
CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
          "-fexcess-precision=standard", "-Wall", "-Wextra", "-shared", "-fPIC"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libmxq_oracle.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_i64 = ctypes.c_int64


def _p(a: np.ndarray, ct):
    assert a.flags["C_CONTIGUOUS"], "oracle buffers must be C-contiguous"
    return a.ctypes.data_as(ct)


def _bits16(x) -> np.ndarray:
    x = np.ascontiguousarray(x)
    assert x.dtype == np.uint16 and x.ndim == 2, "bf16 inputs are passed as uint16 [rows, cols]"
    return x


class Oracle:
    """numpy-facing wrapper over one build of the oracle library.

    The tests also build deliberately broken copies of the C source and wrap
    them in this class, to show that the pins catch planted mistakes."""

    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_double.restype = ctypes.c_double
        L.orc_double_to_bf16.argtypes = [ctypes.c_double]
        L.orc_double_to_bf16.restype = ctypes.c_uint16
        L.orc_e4m3_to_double.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_to_double.restype = ctypes.c_double
        L.orc_double_to_e4m3.argtypes = [ctypes.c_double]
        L.orc_double_to_e4m3.restype = ctypes.c_uint8
        L.orc_e8m0_to_double.argtypes = [ctypes.c_uint8]
        L.orc_e8m0_to_double.restype = ctypes.c_double
        L.orc_e2m1_to_double.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_to_double.restype = ctypes.c_double
        L.orc_double_to_e2m1.argtypes = [ctypes.c_double]
        L.orc_double_to_e2m1.restype = ctypes.c_uint8
        for nm, outp in (("orc_f32_bits_to_e4m3", _u8p), ("orc_f32_bits_to_e2m1", _u8p),
                         ("orc_f32_bits_to_bf16", _u16p)):
            getattr(L, nm).argtypes = [ctypes.c_uint32, _i64, ctypes.c_uint32, outp]
            getattr(L, nm).restype = None
        L.orc_mxfp8_quantize_rowwise.argtypes = [_u16p, _i64, _i64, _u8p, _u8p]
        L.orc_mxfp8_quantize_rowwise.restype = None
        L.orc_mxfp8_quantize_padcrop.argtypes = [_u16p, _i64, _i64, _u8p, _u8p]
        L.orc_mxfp8_quantize_padcrop.restype = ctypes.c_int
        L.orc_mxfp8_quantize_colwise.argtypes = [_u16p, _i64, _i64, _u8p, _u8p]
        L.orc_mxfp8_quantize_colwise.restype = None
        L.orc_mxfp8_quantize_colwise_t.argtypes = [_u16p, _i64, _i64, _u8p, _u8p]
        L.orc_mxfp8_quantize_colwise_t.restype = ctypes.c_int
        L.orc_mxfp8_dequantize.argtypes = [_u8p, _u8p, _i64, _i64, ctypes.c_int, _u16p]
        L.orc_mxfp8_dequantize.restype = None
        L.orc_mxfp8_fake_quant.argtypes = [_u16p, _i64, _i64, ctypes.c_int, _u16p]
        L.orc_mxfp8_fake_quant.restype = ctypes.c_int
        L.orc_mxfp4_quantize.argtypes = [_u16p, _i64, _i64, _u8p, _u8p]
        L.orc_mxfp4_quantize.restype = None
        L.orc_mxfp4_dequantize.argtypes = [_u8p, _u8p, _i64, _i64, _u16p]
        L.orc_mxfp4_dequantize.restype = None
        L.orc_mxfp4_fake_quant.argtypes = [_u16p, _i64, _i64, _u16p]
        L.orc_mxfp4_fake_quant.restype = ctypes.c_int
        L.orc_blockfp8_quantize_rect.argtypes = [_u16p, _i64, _i64, ctypes.c_int32,
                                                 ctypes.c_int32, _u8p, _f32p]
        L.orc_blockfp8_quantize_rect.restype = None
        L.orc_blockfp8_dequantize_rect.argtypes = [_u8p, _f32p, _i64, _i64, ctypes.c_int32,
                                                   ctypes.c_int32, _u16p]
        L.orc_blockfp8_dequantize_rect.restype = None
        L.orc_blockfp8_fake_quant_1x128.argtypes = [_u16p, _i64, _i64, _u16p]
        L.orc_blockfp8_fake_quant_1x128.restype = ctypes.c_int
        L.orc_blockfp8_quantize_gkn.argtypes = [_u16p, _i64, _i64, _i64, ctypes.c_int32, _u8p,
                                                _f32p]
        L.orc_blockfp8_quantize_gkn.restype = None
        L.orc_blockfp8_dequantize_gkn.argtypes = [_u8p, _f32p, _i64, _i64, _i64, ctypes.c_int32,
                                                  _u16p]
        L.orc_blockfp8_dequantize_gkn.restype = None
        L.orc_blockfp8_quantize.argtypes = [_u16p, _i64, _i64, ctypes.c_int32, _u8p, _f32p]
        L.orc_blockfp8_quantize.restype = None
        L.orc_blockfp8_dequantize.argtypes = [_u8p, _f32p, _i64, _i64, ctypes.c_int32, _u16p]
        L.orc_blockfp8_dequantize.restype = None
        L.orc_blockfp8_to_mxfp8.argtypes = [_u8p, _f32p, _i64, _i64, ctypes.c_int32, _u8p, _u8p]
        L.orc_blockfp8_to_mxfp8.restype = ctypes.c_int
        L.orc_nvfp4_quantize.argtypes = [_u16p, _i64, _i64, _u8p, _u8p, _f32p]
        L.orc_nvfp4_quantize.restype = None
        L.orc_nvfp4_quantize_grouped.argtypes = [ctypes.c_int32, ctypes.POINTER(_u16p),
                                                 ctypes.POINTER(_i64), ctypes.POINTER(_i64),
                                                 ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                                                 ctypes.POINTER(_u8p), ctypes.POINTER(_u8p), _f32p]
        L.orc_nvfp4_quantize_grouped.restype = ctypes.c_int
        L.orc_nvfp4_dequantize.argtypes = [_u8p, _u8p, _f32p, _i64, _i64, _u16p]
        L.orc_nvfp4_dequantize.restype = None
        self.L = L
        self.path = path

    # ---- element encoders over runs of fp32 bit patterns -------------------
    def f32_bits_to(self, fmt: str, first: int, n: int, stride: int = 1, out=None) -> np.ndarray:
        """Encodings (fmt 'e4m3', 'e2m1' or 'bf16') of the fp32 values with
        bit patterns first + i * stride, i < n, into out (or a new array)."""
        dt = np.uint16 if fmt == "bf16" else np.uint8
        if out is None:
            out = np.empty((n,), dt)
        assert out.dtype == dt and out.size >= n and out.flags["C_CONTIGUOUS"]
        assert 0 <= first and first + (n - 1) * stride <= 0xFFFFFFFF
        fn = getattr(self.L, f"orc_f32_bits_to_{fmt}")
        fn(int(first), int(n), int(stride), _p(out, _u16p if fmt == "bf16" else _u8p))
        return out

    # ---- scalar codecs ----------------------------------------------------
    def bf16_to_double(self, b: int) -> float:
        return self.L.orc_bf16_to_double(int(b))

    def double_to_bf16(self, v: float) -> int:
        return self.L.orc_double_to_bf16(float(v))

    def e4m3_to_double(self, c: int) -> float:
        return self.L.orc_e4m3_to_double(int(c))

    def double_to_e4m3(self, v: float) -> int:
        return self.L.orc_double_to_e4m3(float(v))

    def e8m0_to_double(self, b: int) -> float:
        return self.L.orc_e8m0_to_double(int(b))

    def e8m0_to_fp32(self, scale: np.ndarray) -> np.ndarray:
        """E8M0 bytes as fp32 values (the fp32 scale storage of "V4 mxfp4"'s
        PR description): each byte's exact value 2^(b - 127), NaN for 0xFF.
        Every such value is exact in fp32 (2^-127 as a subnormal)."""
        table = np.array([self.e8m0_to_double(b) for b in range(256)], dtype=np.float64)
        return table.astype(np.float32)[np.asarray(scale, dtype=np.uint8)]

    def e2m1_to_double(self, n: int) -> float:
        return self.L.orc_e2m1_to_double(int(n))

    def double_to_e2m1(self, v: float) -> int:
        return self.L.orc_double_to_e2m1(float(v))

    # ---- MXFP8 ------------------------------------------------------------
    def mxfp8_quantize_rowwise(self, x: np.ndarray):
        """x: uint16 bf16 bits [rows, cols], cols % 32 == 0 ->
        (q [rows, cols] u8, scale [rows, cols/32] u8)."""
        x = _bits16(x)
        rows, cols = x.shape
        assert cols % 32 == 0
        q = np.empty((rows, cols), np.uint8)
        s = np.empty((rows, cols // 32), np.uint8)
        self.L.orc_mxfp8_quantize_rowwise(_p(x, _u16p), rows, cols, _p(q, _u8p), _p(s, _u8p))
        return q, s

    def mxfp8_quantize_padcrop(self, x: np.ndarray):
        x = _bits16(x)
        rows, cols = x.shape
        assert cols % 32 == 0
        q = np.empty((rows, cols), np.uint8)
        s = np.empty((rows, cols // 32), np.uint8)
        rc = self.L.orc_mxfp8_quantize_padcrop(_p(x, _u16p), rows, cols, _p(q, _u8p), _p(s, _u8p))
        assert rc == 0
        return q, s

    def mxfp8_quantize_colwise(self, x: np.ndarray):
        """-> (q [rows, cols] u8 in x's layout, scale [ceil(rows/32), cols] u8)."""
        x = _bits16(x)
        rows, cols = x.shape
        q = np.empty((rows, cols), np.uint8)
        s = np.empty(((rows + 31) // 32, cols), np.uint8)
        self.L.orc_mxfp8_quantize_colwise(_p(x, _u16p), rows, cols, _p(q, _u8p), _p(s, _u8p))
        return q, s

    def mxfp8_quantize_colwise_t(self, x: np.ndarray):
        """-> (qt [cols, rows] u8: codes of the column groups, transposed;
        st [cols, ceil(rows/32)] u8)."""
        x = _bits16(x)
        rows, cols = x.shape
        qt = np.empty((cols, rows), np.uint8)
        st = np.empty((cols, (rows + 31) // 32), np.uint8)
        rc = self.L.orc_mxfp8_quantize_colwise_t(_p(x, _u16p), rows, cols, _p(qt, _u8p),
                                                 _p(st, _u8p))
        assert rc == 0
        return qt, st

    def mxfp8_dequantize(self, q: np.ndarray, scale: np.ndarray, axis: int = 1) -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=np.uint8)
        scale = np.ascontiguousarray(scale, dtype=np.uint8)
        rows, cols = q.shape
        out = np.empty((rows, cols), np.uint16)
        self.L.orc_mxfp8_dequantize(_p(q, _u8p), _p(scale, _u8p), rows, cols, int(axis),
                                    _p(out, _u16p))
        return out

    def mxfp8_fake_quant(self, x: np.ndarray, axis: int = 1) -> np.ndarray:
        x = _bits16(x)
        rows, cols = x.shape
        out = np.empty((rows, cols), np.uint16)
        rc = self.L.orc_mxfp8_fake_quant(_p(x, _u16p), rows, cols, int(axis), _p(out, _u16p))
        assert rc == 0
        return out

    def mxfp8_quantize_rowwise_many(self, xs):
        """Independent row-wise quantization of each tensor, in order."""
        return [self.mxfp8_quantize_rowwise(x) for x in xs]

    # ---- MXFP4 ------------------------------------------------------------
    def mxfp4_quantize(self, x: np.ndarray):
        """x: uint16 bf16 bits [rows, cols], cols % 32 == 0 ->
        (q_packed [rows, cols/2] u8, scale [rows, cols/32] u8 E8M0)."""
        x = _bits16(x)
        rows, cols = x.shape
        assert cols % 32 == 0
        q = np.empty((rows, cols // 2), np.uint8)
        s = np.empty((rows, cols // 32), np.uint8)
        self.L.orc_mxfp4_quantize(_p(x, _u16p), rows, cols, _p(q, _u8p), _p(s, _u8p))
        return q, s

    def mxfp4_dequantize(self, q: np.ndarray, scale: np.ndarray) -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=np.uint8)
        scale = np.ascontiguousarray(scale, dtype=np.uint8)
        rows, cols = q.shape[0], 2 * q.shape[1]
        out = np.empty((rows, cols), np.uint16)
        self.L.orc_mxfp4_dequantize(_p(q, _u8p), _p(scale, _u8p), rows, cols, _p(out, _u16p))
        return out

    def mxfp4_fake_quant(self, x: np.ndarray) -> np.ndarray:
        x = _bits16(x)
        rows, cols = x.shape
        out = np.empty((rows, cols), np.uint16)
        rc = self.L.orc_mxfp4_fake_quant(_p(x, _u16p), rows, cols, _p(out, _u16p))
        assert rc == 0
        return out

    # ---- block-FP8 --------------------------------------------------------
    def blockfp8_quantize(self, x: np.ndarray, blk: int = 128):
        x = _bits16(x)
        rows, cols = x.shape
        q = np.empty((rows, cols), np.uint8)
        S = np.empty(((rows + blk - 1) // blk, (cols + blk - 1) // blk), np.float32)
        self.L.orc_blockfp8_quantize(_p(x, _u16p), rows, cols, int(blk), _p(q, _u8p), _p(S, _f32p))
        return q, S

    def blockfp8_dequantize(self, q: np.ndarray, S: np.ndarray, blk: int = 128) -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=np.uint8)
        S = np.ascontiguousarray(S, dtype=np.float32)
        rows, cols = q.shape
        out = np.empty((rows, cols), np.uint16)
        self.L.orc_blockfp8_dequantize(_p(q, _u8p), _p(S, _f32p), rows, cols, int(blk),
                                       _p(out, _u16p))
        return out

    def blockfp8_quantize_gkn(self, x: np.ndarray, blk: int = 128):
        """x: uint16 [G, K, N] -> (q [G, K, N] u8, S [G, ceil(K/blk), ceil(N/blk)] f32)."""
        x = np.ascontiguousarray(x)
        assert x.dtype == np.uint16 and x.ndim == 3
        G, K, N = x.shape
        q = np.empty((G, K, N), np.uint8)
        S = np.empty((G, (K + blk - 1) // blk, (N + blk - 1) // blk), np.float32)
        self.L.orc_blockfp8_quantize_gkn(_p(x, _u16p), G, K, N, int(blk), _p(q, _u8p),
                                         _p(S, _f32p))
        return q, S

    def blockfp8_dequantize_gkn(self, q: np.ndarray, S: np.ndarray, blk: int = 128):
        q = np.ascontiguousarray(q, dtype=np.uint8)
        S = np.ascontiguousarray(S, dtype=np.float32)
        G, K, N = q.shape
        out = np.empty((G, K, N), np.uint16)
        self.L.orc_blockfp8_dequantize_gkn(_p(q, _u8p), _p(S, _f32p), G, K, N, int(blk),
                                           _p(out, _u16p))
        return out

    def blockfp8_quantize_rect(self, x: np.ndarray, br: int, bc: int):
        """br x bc blocks: (q [rows, cols] u8, S [ceil(rows/br), ceil(cols/bc)] f32)."""
        x = _bits16(x)
        rows, cols = x.shape
        q = np.empty((rows, cols), np.uint8)
        S = np.empty(((rows + br - 1) // br, (cols + bc - 1) // bc), np.float32)
        self.L.orc_blockfp8_quantize_rect(_p(x, _u16p), rows, cols, int(br), int(bc),
                                          _p(q, _u8p), _p(S, _f32p))
        return q, S

    def blockfp8_dequantize_rect(self, q: np.ndarray, S: np.ndarray, br: int, bc: int):
        q = np.ascontiguousarray(q, dtype=np.uint8)
        S = np.ascontiguousarray(S, dtype=np.float32)
        rows, cols = q.shape
        out = np.empty((rows, cols), np.uint16)
        self.L.orc_blockfp8_dequantize_rect(_p(q, _u8p), _p(S, _f32p), rows, cols, int(br),
                                            int(bc), _p(out, _u16p))
        return out

    def blockfp8_fake_quant_1x128(self, x: np.ndarray) -> np.ndarray:
        x = _bits16(x)
        rows, cols = x.shape
        out = np.empty((rows, cols), np.uint16)
        rc = self.L.orc_blockfp8_fake_quant_1x128(_p(x, _u16p), rows, cols, _p(out, _u16p))
        assert rc == 0
        return out

    def blockfp8_to_mxfp8(self, q: np.ndarray, S: np.ndarray, blk: int = 128):
        """Block-FP8 (codes + fp32 tile scales) -> bf16 -> row-wise MXFP8:
        (q8 [rows, cols] u8, scale [rows, cols/32] u8)."""
        q = np.ascontiguousarray(q, dtype=np.uint8)
        S = np.ascontiguousarray(S, dtype=np.float32)
        rows, cols = q.shape
        assert cols % 32 == 0
        q8 = np.empty((rows, cols), np.uint8)
        s8 = np.empty((rows, cols // 32), np.uint8)
        rc = self.L.orc_blockfp8_to_mxfp8(_p(q, _u8p), _p(S, _f32p), rows, cols, int(blk),
                                          _p(q8, _u8p), _p(s8, _u8p))
        assert rc == 0
        return q8, s8

    # ---- NVFP4 ------------------------------------------------------------
    def nvfp4_quantize(self, x: np.ndarray):
        """-> (q_packed [rows, cols/2] u8, s [rows, cols/16] u8 E4M3, g float32 [1])."""
        x = _bits16(x)
        rows, cols = x.shape
        assert cols % 16 == 0
        q = np.empty((rows, cols // 2), np.uint8)
        s = np.empty((rows, cols // 16), np.uint8)
        g = np.empty((1,), np.float32)
        self.L.orc_nvfp4_quantize(_p(x, _u16p), rows, cols, _p(q, _u8p), _p(s, _u8p), _p(g, _f32p))
        return q, s, g

    def nvfp4_quantize_grouped(self, xs, groups, n_groups: int):
        """NVFP4 of each tensor in xs with the global scale shared within scale
        groups (groups[i] is tensor i's group) -> ([(q_packed, s)], g float32
        [n_groups])."""
        xs = [_bits16(x) for x in xs]
        n = len(xs)
        outs = [(np.empty((x.shape[0], x.shape[1] // 2), np.uint8),
                 np.empty((x.shape[0], x.shape[1] // 16), np.uint8)) for x in xs]
        gs = np.empty((max(n_groups, 1),), np.float32)
        arr = lambda ct, vals: (ct * n)(*vals)
        rc = self.L.orc_nvfp4_quantize_grouped(
            n, arr(_u16p, [_p(x, _u16p) for x in xs]), arr(_i64, [x.shape[0] for x in xs]),
            arr(_i64, [x.shape[1] for x in xs]), arr(ctypes.c_int32, [int(g) for g in groups]),
            int(n_groups), arr(_u8p, [_p(o[0], _u8p) for o in outs]),
            arr(_u8p, [_p(o[1], _u8p) for o in outs]), _p(gs, _f32p))
        assert rc == 0
        return outs, gs[:n_groups]

    def nvfp4_dequantize(self, q: np.ndarray, s: np.ndarray, g: np.ndarray) -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=np.uint8)
        s = np.ascontiguousarray(s, dtype=np.uint8)
        g = np.ascontiguousarray(g, dtype=np.float32).reshape(1)
        rows, half = q.shape
        cols = half * 2
        out = np.empty((rows, cols), np.uint16)
        self.L.orc_nvfp4_dequantize(_p(q, _u8p), _p(s, _u8p), _p(g, _f32p), rows, cols,
                                    _p(out, _u16p))
        return out


_default = None


def default() -> Oracle:
    """The oracle built from ``mxq_oracle.c`` (compiled on first use if needed)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _default = Oracle(_LIB)
    return _default


def build_variant(source_text: str, out_path: str) -> Oracle:
    """Compile an edited copy of the oracle source (used only by the tests that
    plant mistakes to check the pins) and wrap it."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(source_text)
    subprocess.run(["gcc", *CFLAGS, src, "-o", out_path, "-lm"], check=True)
    return Oracle(out_path)


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def __getattr__(name):
    # Module-level shortcuts: oracle.mxfp8_quantize_rowwise(x) etc.
    if not name.startswith("_") and hasattr(Oracle, name):
        return getattr(default(), name)
    raise AttributeError(name)
