"""The C ABI on the host (no GPU): the library loads, exports every function
include/mxq.h declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import block_scaled_precision_mxfp8_amd as mxq
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "mxq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b((?:mxq|blockfp8|nvfp4|mxfp4)_\w+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mxq.LIB_PATH):
        pytest.fail("libmxq.so is not built (run __graft_entry__.build())")
    return mxq.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ["mxq_quantize_rowwise", "mxq_quantize_colwise", "mxq_dequantize", "mxq_fake_quant",
                 "mxq_quantize_rowwise_grouped", "blockfp8_quantize", "blockfp8_dequantize",
                 "nvfp4_quantize", "nvfp4_dequantize", "mxq_status_string", "mxq_abi_version",
                 "mxq_grouped_workspace_size", "nvfp4_workspace_size", "mxfp4_quantize",
                 "mxfp4_dequantize", "mxfp4_fake_quant", "mxq_quantize_colwise_t",
                 "blockfp8_to_mxfp8", "blockfp8_quantize_1x128", "blockfp8_dequantize_1x128",
                 "blockfp8_fake_quant_1x128", "nvfp4_quantize_grouped",
                 "nvfp4_grouped_workspace_size", "blockfp8_quantize_gkn",
                 "blockfp8_dequantize_gkn"]:
        assert want in names
    assert set(names) == set(mxq.SIGNATURES), "binding and header disagree"


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", mxq.LIB_PATH], check=True,
                         capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_version_and_strings(lib):
    assert lib.mxq_abi_version() == 2
    for st in range(7):
        assert lib.mxq_status_string(st)
    assert b"unknown" in lib.mxq_status_string(99)
    assert b"captur" in lib.mxq_status_string(mxq.MXQ_ECAPTURE)


def test_build_id_matches_sources(lib):
    """The library in the tree was built from the sources beside it."""
    from block_scaled_precision_mxfp8_amd import build
    assert lib.mxq_build_id().decode() == build.source_hash()


def _load_copy(root):
    code = ("import block_scaled_precision_mxfp8_amd as m\n"
            "try:\n    m.load()\nexcept m.StaleLibraryError as e:\n"
            "    print('STALE', e)\nelse:\n    print('LOADED')\n")
    env = dict(os.environ, PYTHONPATH=str(root))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    return r.stdout


def test_stale_library_is_refused(tmp_path):
    """A copy of the package with its built library loads; after an edit to a
    kernel source, or to the public header, the same library is refused
    (StaleLibraryError names the rebuild), and nothing is rebuilt behind the
    caller's back."""
    import shutil
    pkg = tmp_path / "block_scaled_precision_mxfp8_amd"
    shutil.copytree(os.path.dirname(mxq.__file__), pkg,
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(os.path.join(ROOT, "include"), tmp_path / "include")
    lib_before = (pkg / "libmxq.so").read_bytes()
    assert "LOADED" in _load_copy(tmp_path)
    src = pkg / "csrc" / "mx_kernels.hip"
    text = src.read_text()
    src.write_text(text + "\n// an edit after the build\n")
    out = _load_copy(tmp_path)
    assert "STALE" in out and "rebuild" in out
    src.write_text(text)
    assert "LOADED" in _load_copy(tmp_path)
    hdr = tmp_path / "include" / "mxq.h"
    hdr.write_text(hdr.read_text().replace("MXQ_ABI_VERSION 2", "MXQ_ABI_VERSION 3"))
    assert "STALE" in _load_copy(tmp_path)
    assert (pkg / "libmxq.so").read_bytes() == lib_before


P16 = ctypes.c_void_p(0x10000)   # aligned fake device addresses: never dereferenced,
P8 = ctypes.c_void_p(0x10008)    # because every call below fails validation first
P4 = ctypes.c_void_p(0x10004)
P2 = ctypes.c_void_p(0x10002)
NULL = None


def test_rowwise_errors(lib):
    f = lib.mxq_quantize_rowwise
    assert f(P16, -1, 32, 32, P16, 32, P16, 1, NULL, 0, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 4, 33, 33, P16, 33, P16, 1, NULL, 0, NULL) == mxq.MXQ_ESHAPE
    assert f(NULL, 4, 32, 32, P16, 32, P16, 1, NULL, 0, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 4, 32, 32, NULL, 32, P16, 1, NULL, 0, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 4, 32, 32, P16, 32, NULL, 1, NULL, 0, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 4, 64, 32, P16, 64, P16, 2, NULL, 0, NULL) == mxq.MXQ_ESHAPE   # ldx < cols
    assert f(P16, 4, 64, 64, P16, 32, P16, 2, NULL, 0, NULL) == mxq.MXQ_ESHAPE   # ldq < cols
    assert f(P16, 4, 64, 64, P16, 64, P16, 1, NULL, 0, NULL) == mxq.MXQ_ESHAPE   # lds < cols/32
    assert f(P8, 4, 32, 32, P16, 32, P16, 1, NULL, 0, NULL) == mxq.MXQ_EALIGN    # x not 16-aligned
    assert f(P16, 4, 32, 36, P16, 32, P16, 1, NULL, 0, NULL) == mxq.MXQ_EALIGN   # ldx % 8
    assert f(P16, 4, 32, 32, P4, 32, P16, 1, NULL, 0, NULL) == mxq.MXQ_EALIGN    # q not 8-aligned
    assert f(P16, 4, 32, 32, P16, 36, P16, 1, NULL, 0, NULL) == mxq.MXQ_EALIGN   # ldq % 8
    assert f(P16, 4, 32, 32, P16, 32, P16, 1, P8, 32, NULL) == mxq.MXQ_EALIGN    # fq not 16-aligned
    assert f(P16, 4, 32, 32, P16, 32, P16, 1, P16, 16, NULL) == mxq.MXQ_ESHAPE   # ldf < cols
    assert f(P16, 2**62, 64, 64, P16, 64, P16, 2, NULL, 0, NULL) == mxq.MXQ_ESIZE  # overflow
    # empty problems are accepted and launch nothing, even with NULL pointers
    assert f(NULL, 0, 64, 64, NULL, 64, NULL, 2, NULL, 0, NULL) == mxq.MXQ_OK
    assert f(NULL, 5, 0, 0, NULL, 0, NULL, 0, NULL, 0, NULL) == mxq.MXQ_OK


def test_colwise_dequant_fakequant_errors(lib):
    c = lib.mxq_quantize_colwise
    assert c(P16, 4, 48, P16, P16, NULL, NULL, NULL, NULL) == mxq.MXQ_ESHAPE
    assert c(P16, 4, 32, NULL, P16, NULL, NULL, NULL, NULL) == mxq.MXQ_EINVAL
    assert c(P16, 4, 32, P16, P16, P16, NULL, NULL, NULL) == mxq.MXQ_EINVAL      # qr without sr
    assert c(P8, 4, 32, P16, P16, NULL, NULL, NULL, NULL) == mxq.MXQ_EALIGN
    assert c(P16, 4, 32, P16, P4, NULL, NULL, NULL, NULL) == mxq.MXQ_EALIGN      # sc 8-aligned
    assert c(P16, 4, 32, P16, P16, NULL, NULL, P8, NULL) == mxq.MXQ_EALIGN       # fq 16-aligned
    assert c(NULL, 0, 32, NULL, NULL, NULL, NULL, NULL, NULL) == mxq.MXQ_OK
    d = lib.mxq_dequantize
    assert d(P16, P16, 4, 32, 2, P16, NULL) == mxq.MXQ_EINVAL                     # bad axis
    assert d(P16, P16, 4, 40, 1, P16, NULL) == mxq.MXQ_ESHAPE
    assert d(P16, NULL, 4, 32, 1, P16, NULL) == mxq.MXQ_EINVAL
    assert d(P16, P16, 4, 32, 1, P8, NULL) == mxq.MXQ_EALIGN
    assert d(P16, P4, 4, 32, 0, P16, NULL) == mxq.MXQ_EALIGN
    fq = lib.mxq_fake_quant
    assert fq(P16, 4, 32, -1, P16, NULL) == mxq.MXQ_EINVAL
    assert fq(P16, 4, 31, 1, P16, NULL) == mxq.MXQ_ESHAPE
    assert fq(P16, 4, 32, 1, NULL, NULL) == mxq.MXQ_EINVAL
    assert fq(P2, 4, 32, 0, P16, NULL) == mxq.MXQ_EALIGN


def test_grouped_errors(lib):
    g = lib.mxq_quantize_rowwise_grouped
    assert lib.mxq_grouped_workspace_size(0) == 0
    ws = lib.mxq_grouped_workspace_size(3)
    assert ws >= 3 * 84 and ws % 16 == 0
    descs = (mxq.GroupDesc * 3)()
    for i in range(3):
        descs[i] = mxq.GroupDesc(0x10000, 0x20000, 0x30000, 8, 64, 64, 64, 2)
    assert g(descs, -1, P16, ws, NULL) == mxq.MXQ_EINVAL
    assert g(descs, 0, NULL, 0, NULL) == mxq.MXQ_OK
    assert g(NULL, 3, P16, ws, NULL) == mxq.MXQ_EINVAL
    assert g(descs, 3, P16, ws - 1, NULL) == mxq.MXQ_ESIZE
    assert g(descs, 3, P8, ws, NULL) == mxq.MXQ_EALIGN
    descs[2] = mxq.GroupDesc(0x10000, 0x20000, 0x30000, 8, 48, 48, 48, 2)      # cols % 32
    assert g(descs, 3, P16, ws, NULL) == mxq.MXQ_ESHAPE
    descs[2] = mxq.GroupDesc(0x10008, 0x20000, 0x30000, 8, 64, 64, 64, 2)      # x misaligned
    assert g(descs, 3, P16, ws, NULL) == mxq.MXQ_EALIGN
    descs[2] = mxq.GroupDesc(0x10000, 0, 0x30000, 8, 64, 64, 64, 2)            # NULL q
    assert g(descs, 3, P16, ws, NULL) == mxq.MXQ_EINVAL


def test_blockfp8_nvfp4_errors(lib):
    b = lib.blockfp8_quantize
    assert b(P16, 4, 64, 64, P16, P16, NULL) == mxq.MXQ_ESHAPE                   # blk != 128
    assert b(P16, 4, 60, 128, P16, P16, NULL) == mxq.MXQ_ESHAPE                  # cols % 8
    assert b(P16, -4, 64, 128, P16, P16, NULL) == mxq.MXQ_EINVAL
    assert b(P16, 4, 64, 128, NULL, P16, NULL) == mxq.MXQ_EINVAL
    assert b(P8, 4, 64, 128, P16, P16, NULL) == mxq.MXQ_EALIGN
    assert b(P16, 4, 64, 128, P16, P2, NULL) == mxq.MXQ_EALIGN
    bd = lib.blockfp8_dequantize
    assert bd(P16, P16, 4, 64, 128, P8, NULL) == mxq.MXQ_EALIGN
    assert bd(P16, NULL, 4, 64, 128, P16, NULL) == mxq.MXQ_EINVAL
    n = lib.nvfp4_quantize
    W = lib.nvfp4_workspace_size()
    assert W >= 4
    assert n(P16, 4, 24, P16, P16, P16, P16, W, NULL) == mxq.MXQ_ESHAPE          # cols % 16
    assert n(P16, 4, 32, P16, P16, P16, NULL, W, NULL) == mxq.MXQ_EINVAL         # no workspace
    assert n(P16, 4, 32, P16, P16, P16, P16, W - 1, NULL) == mxq.MXQ_ESIZE
    assert n(P8, 4, 32, P16, P16, P16, P16, W, NULL) == mxq.MXQ_EALIGN
    assert n(P16, 4, 32, P2, P16, P16, P16, W, NULL) == mxq.MXQ_EALIGN
    nd = lib.nvfp4_dequantize
    assert nd(P16, P16, NULL, 4, 32, P16, NULL) == mxq.MXQ_EINVAL
    assert nd(P16, P16, P16, 4, 32, P8, NULL) == mxq.MXQ_EALIGN
    assert nd(NULL, NULL, NULL, 0, 32, NULL, NULL) == mxq.MXQ_OK


def test_colwise_t_errors(lib):
    f = lib.mxq_quantize_colwise_t
    assert f(P16, -1, 32, P16, 16, P16, NULL, NULL, NULL, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 4, 48, P16, 16, P16, NULL, NULL, NULL, NULL) == mxq.MXQ_ESHAPE   # cols % 32
    assert f(NULL, 4, 32, P16, 16, P16, NULL, NULL, NULL, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 4, 32, NULL, 16, P16, NULL, NULL, NULL, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 4, 32, P16, 16, NULL, NULL, NULL, NULL, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 4, 32, P16, 16, P16, P16, NULL, NULL, NULL) == mxq.MXQ_EINVAL    # qr without sr
    assert f(P16, 40, 32, P16, 32, P16, NULL, NULL, NULL, NULL) == mxq.MXQ_ESHAPE  # ldt < rows
    assert f(P16, 4, 32, P16, 24, P16, NULL, NULL, NULL, NULL) == mxq.MXQ_EALIGN   # ldt % 16
    assert f(P16, 4, 32, P8, 16, P16, NULL, NULL, NULL, NULL) == mxq.MXQ_EALIGN    # qt 16-aligned
    assert f(P8, 4, 32, P16, 16, P16, NULL, NULL, NULL, NULL) == mxq.MXQ_EALIGN
    assert f(P16, 4, 32, P16, 16, P16, P4, P16, NULL, NULL) == mxq.MXQ_EALIGN      # qr 8-aligned
    assert f(P16, 4, 32, P16, 16, P16, NULL, NULL, P8, NULL) == mxq.MXQ_EALIGN     # fq 16-aligned
    assert f(P16, 4, 32, P16, 16, P2, NULL, NULL, NULL, NULL) == mxq.MXQ_EALIGN    # st 4-aligned
    assert f(NULL, 0, 32, NULL, 0, NULL, NULL, NULL, NULL, NULL) == mxq.MXQ_OK


def test_blockfp8_to_mxfp8_errors(lib):
    f = lib.blockfp8_to_mxfp8
    assert f(P16, P16, -1, 32, 128, P16, P16, NULL) == mxq.MXQ_EINVAL
    assert f(P16, P16, 4, 32, 64, P16, P16, NULL) == mxq.MXQ_ESHAPE     # blk != 128
    assert f(P16, P16, 4, 48, 128, P16, P16, NULL) == mxq.MXQ_ESHAPE    # cols % 32
    assert f(NULL, P16, 4, 32, 128, P16, P16, NULL) == mxq.MXQ_EINVAL
    assert f(P16, NULL, 4, 32, 128, P16, P16, NULL) == mxq.MXQ_EINVAL
    assert f(P16, P16, 4, 32, 128, NULL, P16, NULL) == mxq.MXQ_EINVAL
    assert f(P16, P16, 4, 32, 128, P16, NULL, NULL) == mxq.MXQ_EINVAL
    assert f(P4, P16, 4, 32, 128, P16, P16, NULL) == mxq.MXQ_EALIGN     # q 8-aligned
    assert f(P16, P2, 4, 32, 128, P16, P16, NULL) == mxq.MXQ_EALIGN     # scale 4-aligned
    assert f(P16, P16, 4, 32, 128, P4, P16, NULL) == mxq.MXQ_EALIGN     # q8 8-aligned
    assert f(NULL, NULL, 0, 32, 128, NULL, NULL, NULL) == mxq.MXQ_OK


def test_blockfp8_1x128_errors(lib):
    f = lib.blockfp8_quantize_1x128
    assert f(P16, -1, 32, P16, P16, NULL, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 4, 36, P16, P16, NULL, NULL) == mxq.MXQ_ESHAPE           # cols % 8
    assert f(NULL, 4, 32, P16, P16, NULL, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 4, 32, NULL, P16, NULL, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 4, 32, P16, NULL, NULL, NULL) == mxq.MXQ_EINVAL
    assert f(P8, 4, 32, P16, P16, NULL, NULL) == mxq.MXQ_EALIGN
    assert f(P16, 4, 32, P4, P16, NULL, NULL) == mxq.MXQ_EALIGN            # q 8-aligned
    assert f(P16, 4, 32, P16, P2, NULL, NULL) == mxq.MXQ_EALIGN            # scale 4-aligned
    assert f(P16, 4, 32, P16, P16, P8, NULL) == mxq.MXQ_EALIGN             # fq 16-aligned
    assert f(NULL, 0, 32, NULL, NULL, NULL, NULL) == mxq.MXQ_OK
    d = lib.blockfp8_dequantize_1x128
    assert d(P16, P16, 4, 36, P16, NULL) == mxq.MXQ_ESHAPE
    assert d(P16, NULL, 4, 32, P16, NULL) == mxq.MXQ_EINVAL
    assert d(P16, P16, 4, 32, P8, NULL) == mxq.MXQ_EALIGN
    fq = lib.blockfp8_fake_quant_1x128
    assert fq(P16, 4, 32, NULL, NULL) == mxq.MXQ_EINVAL
    assert fq(P2, 4, 32, P16, NULL) == mxq.MXQ_EALIGN
    assert fq(P16, 4, 12, P16, NULL) == mxq.MXQ_ESHAPE


def test_nvfp4_noalloc_errors(lib):
    """The allocation-free NVFP4 entry point validates like nvfp4_quantize
    (minus the workspace) before touching the GPU."""
    f = lib.nvfp4_quantize_noalloc
    assert f(P16, -1, 32, P16, P16, P16, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 4, 24, P16, P16, P16, NULL) == mxq.MXQ_ESHAPE          # cols % 16
    assert f(NULL, 4, 32, P16, P16, P16, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 4, 32, NULL, P16, P16, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 4, 32, P16, NULL, P16, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 4, 32, P16, P16, NULL, NULL) == mxq.MXQ_EINVAL          # no global scale
    assert f(P8, 4, 32, P16, P16, P16, NULL) == mxq.MXQ_EALIGN            # x 16-aligned
    assert f(P16, 4, 32, P2, P16, P16, NULL) == mxq.MXQ_EALIGN            # q 4-aligned
    assert f(P16, 4, 32, P16, P16, P2, NULL) == mxq.MXQ_EALIGN            # g 4-aligned
    assert f(P16, 1 << 62, 1 << 4, P16, P16, P16, NULL) == mxq.MXQ_ESIZE  # rows * cols overflows
    assert f(NULL, 0, 32, NULL, NULL, NULL, NULL) == mxq.MXQ_OK


def test_nvfp4_grouped_errors(lib):
    f = lib.nvfp4_quantize_grouped
    descs = (mxq.NvGroupDesc * 2)()
    descs[0] = mxq.NvGroupDesc(0x10000, 0x20000, 0x30000, 8, 64, 0, 0)
    descs[1] = mxq.NvGroupDesc(0x40000, 0x50000, 0x60000, 40, 32, 1, 0)
    ws = lib.nvfp4_grouped_workspace_size(descs, 2)
    assert ws >= 2 * 16 and ws % 16 == 0
    assert lib.nvfp4_grouped_workspace_size(descs, 0) == 0
    assert f(descs, -1, P16, 2, P16, ws, NULL) == mxq.MXQ_EINVAL
    assert f(descs, 2, P16, 0, P16, ws, NULL) == mxq.MXQ_EINVAL            # no groups
    assert f(NULL, 2, P16, 2, P16, ws, NULL) == mxq.MXQ_EINVAL
    assert f(descs, 2, NULL, 2, P16, ws, NULL) == mxq.MXQ_EINVAL           # no global scales
    assert f(descs, 2, P2, 2, P16, ws, NULL) == mxq.MXQ_EALIGN             # gs 4-aligned
    assert f(descs, 2, P16, 1, P16, ws, NULL) == mxq.MXQ_EINVAL            # group 1 out of range
    assert f(descs, 2, P16, 2, NULL, ws, NULL) == mxq.MXQ_EINVAL           # no workspace
    assert f(descs, 2, P16, 2, P8, ws, NULL) == mxq.MXQ_EALIGN             # workspace 16-aligned
    assert f(descs, 2, P16, 2, P16, ws - 1, NULL) == mxq.MXQ_ESIZE
    descs[1] = mxq.NvGroupDesc(0x40000, 0x50000, 0x60000, 40, 24, 1, 0)   # cols % 16
    assert f(descs, 2, P16, 2, P16, ws, NULL) == mxq.MXQ_ESHAPE
    descs[1] = mxq.NvGroupDesc(0x40008, 0x50000, 0x60000, 40, 32, 1, 0)   # x 16-aligned
    assert f(descs, 2, P16, 2, P16, ws, NULL) == mxq.MXQ_EALIGN
    descs[1] = mxq.NvGroupDesc(0x40000, 0x50002, 0x60000, 40, 32, 1, 0)   # q 4-aligned
    assert f(descs, 2, P16, 2, P16, ws, NULL) == mxq.MXQ_EALIGN
    descs[1] = mxq.NvGroupDesc(0x40000, 0, 0x60000, 40, 32, 1, 0)         # NULL q
    assert f(descs, 2, P16, 2, P16, ws, NULL) == mxq.MXQ_EINVAL
    assert f(descs, 0, P16, 0, NULL, 0, NULL) == mxq.MXQ_OK


def test_blockfp8_gkn_errors(lib):
    f = lib.blockfp8_quantize_gkn
    assert f(P16, -1, 4, 32, 128, P16, P16, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 2, 4, 32, 64, P16, P16, NULL) == mxq.MXQ_ESHAPE        # blk != 128
    assert f(P16, 2, 4, 36, 128, P16, P16, NULL) == mxq.MXQ_ESHAPE       # N % 8
    assert f(NULL, 2, 4, 32, 128, P16, P16, NULL) == mxq.MXQ_EINVAL
    assert f(P8, 2, 4, 32, 128, P16, P16, NULL) == mxq.MXQ_EALIGN
    assert f(P16, 2, 4, 32, 128, P4, P16, NULL) == mxq.MXQ_EALIGN        # q 8-aligned
    assert f(P16, 2, 4, 32, 128, P16, P2, NULL) == mxq.MXQ_EALIGN        # scale 4-aligned
    assert f(P16, 2**40, 2**20, 64, 128, P16, P16, NULL) == mxq.MXQ_ESIZE
    assert f(NULL, 0, 4, 32, 128, NULL, NULL, NULL) == mxq.MXQ_OK
    d = lib.blockfp8_dequantize_gkn
    assert d(P16, NULL, 2, 4, 32, 128, P16, NULL) == mxq.MXQ_EINVAL
    assert d(P16, P16, 2, 4, 32, 128, P8, NULL) == mxq.MXQ_EALIGN
    assert d(P16, P16, 2, 4, 33, 128, P16, NULL) == mxq.MXQ_ESHAPE


def test_mxfp4_errors(lib):
    f = lib.mxfp4_quantize
    assert f(P16, -1, 32, P16, P16, NULL, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 4, 48, P16, P16, NULL, NULL) == mxq.MXQ_ESHAPE                 # cols % 32
    assert f(NULL, 4, 32, P16, P16, NULL, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 4, 32, NULL, P16, NULL, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 4, 32, P16, NULL, NULL, NULL) == mxq.MXQ_EINVAL
    assert f(P8, 4, 32, P16, P16, NULL, NULL) == mxq.MXQ_EALIGN                  # x 16-aligned
    assert f(P16, 4, 32, P2, P16, NULL, NULL) == mxq.MXQ_EALIGN                  # q 4-aligned
    assert f(P16, 4, 32, P16, P16, P8, NULL) == mxq.MXQ_EALIGN                   # fq 16-aligned
    assert f(P16, 2**62, 64, P16, P16, NULL, NULL) == mxq.MXQ_ESIZE
    assert f(NULL, 0, 32, NULL, NULL, NULL, NULL) == mxq.MXQ_OK
    d = lib.mxfp4_dequantize
    assert d(P16, P16, 4, 40, P16, NULL) == mxq.MXQ_ESHAPE
    assert d(P16, NULL, 4, 32, P16, NULL) == mxq.MXQ_EINVAL
    assert d(P2, P16, 4, 32, P16, NULL) == mxq.MXQ_EALIGN
    assert d(P16, P16, 4, 32, P8, NULL) == mxq.MXQ_EALIGN
    assert d(NULL, NULL, 0, 32, NULL, NULL) == mxq.MXQ_OK
    fq = lib.mxfp4_fake_quant
    assert fq(P16, 4, 33, P16, NULL) == mxq.MXQ_ESHAPE
    assert fq(P16, 4, 32, NULL, NULL) == mxq.MXQ_EINVAL
    assert fq(P2, 4, 32, P16, NULL) == mxq.MXQ_EALIGN
    assert fq(P16, -4, 32, P16, NULL) == mxq.MXQ_EINVAL


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((4, 32), dtype=torch.bfloat16)
    for fn in (mxq.quantize_rowwise, mxq.fake_quant, mxq.blockfp8_quantize, mxq.nvfp4_quantize,
               mxq.mxfp8_quantize, mxq.mxfp4_quantize, mxq.mxfp4_simulate_qat,
               mxq.blockfp8_quantize_1x128, mxq.fp8_simulate_qat):
        with pytest.raises(ValueError):
            fn(x)
    with pytest.raises(TypeError):
        mxq.quantize_rowwise(x.float())


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "block_scaled_precision_mxfp8_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "oracle" not in text.replace("oracle-free", ""), f


C_CLIENT = r"""
#include <stdio.h>
#include "mxq.h"

#define EXPECT(call, want) do { mxq_status s_ = (call); if (s_ != (want)) { \
    printf("line %d: got %d (%s), want %d\n", __LINE__, (int)s_, mxq_status_string(s_), \
           (int)(want)); return 1; } } while (0)

int main(void)
{
    const uint16_t *x = (const uint16_t *)0x10000;   /* never dereferenced: every */
    uint8_t *q = (uint8_t *)0x10000;                 /* call fails validation     */
    uint16_t *o = (uint16_t *)0x10000;
    float *f = (float *)0x10000;
    int st;
    if (mxq_abi_version() != MXQ_ABI_VERSION) return 2;
    for (st = 0; st <= 5; ++st)
        if (!mxq_status_string(st)) return 3;
    EXPECT(mxq_quantize_rowwise(x, 4, 33, 33, q, 33, q, 1, NULL, 0, NULL), MXQ_ESHAPE);
    EXPECT(mxq_quantize_rowwise(x, 0, 32, 32, NULL, 32, NULL, 1, NULL, 0, NULL), MXQ_OK);
    EXPECT(mxq_quantize_colwise(NULL, 4, 32, q, q, NULL, NULL, NULL, NULL), MXQ_EINVAL);
    EXPECT(mxq_quantize_colwise_t(x, 4, 32, q, 2, q, NULL, NULL, NULL, NULL), MXQ_ESHAPE);
    EXPECT(mxq_dequantize(q, q, 4, 32, 2, o, NULL), MXQ_EINVAL);
    EXPECT(mxq_fake_quant(x, 4, 48, 1, o, NULL), MXQ_ESHAPE);
    EXPECT(mxq_quantize_rowwise_grouped(NULL, -1, NULL, 0, NULL), MXQ_EINVAL);
    EXPECT(blockfp8_quantize(x, 4, 32, 64, q, f, NULL), MXQ_ESHAPE);
    EXPECT(blockfp8_dequantize(q, f, -4, 32, 128, o, NULL), MXQ_EINVAL);
    EXPECT(blockfp8_quantize_1x128(x, 4, 12, q, f, NULL, NULL), MXQ_ESHAPE);
    EXPECT(blockfp8_to_mxfp8(q, f, 4, 48, 128, q, q, NULL), MXQ_ESHAPE);
    EXPECT(mxfp4_quantize(x, 4, 16, q, q, NULL, NULL), MXQ_ESHAPE);
    EXPECT(nvfp4_quantize(x, 4, 24, q, q, f, q, nvfp4_workspace_size(), NULL), MXQ_ESHAPE);
    EXPECT(nvfp4_quantize(x, 4, 32, q, q, f, q, 0, NULL), MXQ_ESIZE);
    EXPECT(nvfp4_dequantize(q, q, f, 4, 32, (uint16_t *)0x10002, NULL), MXQ_EALIGN);
    printf("c client ok\n");
    return 0;
}
"""


def test_c_client_builds_links_and_gets_errors(tmp_path):
    """A plain C99 program includes include/mxq.h, links libmxq.so and gets
    the documented status codes back (argument checks run before any HIP call,
    so this needs no GPU): the header is valid C and the symbols unmangled."""
    if not os.path.exists(mxq.LIB_PATH):
        pytest.fail("libmxq.so is not built (run __graft_entry__.build())")
    src = tmp_path / "client.c"
    src.write_text(C_CLIENT)
    exe = tmp_path / "client"
    libdir = os.path.dirname(mxq.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), str(src), "-L", libdir, "-lmxq",
                    f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c client ok" in r.stdout


def test_e8m0_to_fp32_errors(lib):
    f = lib.mxq_e8m0_to_fp32
    assert f(P16, -1, P16, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 0, NULL, NULL) == mxq.MXQ_OK
    assert f(NULL, 8, P16, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 8, NULL, NULL) == mxq.MXQ_EINVAL
    assert f(P16, 8, P2, NULL) == mxq.MXQ_EALIGN


def test_grouped_plan_build_and_refusals(lib):
    """Building a grouped plan runs on the host only: the table image holds
    every non-empty descriptor with its first tile (tiles are 512-column
    blocks of 16 rows for MXFP8 and 32 rows for NVFP4, numbered tensor by
    tensor), and a launch refuses a missing, foreign or altered plan before
    anything reaches the GPU."""
    import numpy as np
    b = lib.mxq_grouped_plan_build
    descs = (mxq.GroupDesc * 3)()
    descs[0] = mxq.GroupDesc(0x10000, 0x20000, 0x30000, 40, 1056, 1056, 1056, 33)
    descs[1] = mxq.GroupDesc(None, None, None, 0, 64, 64, 64, 2)           # empty: no entry
    descs[2] = mxq.GroupDesc(0x40000, 0x50000, 0x60000, 8, 64, 72, 64, 2)
    plan = mxq.GroupedPlan()
    assert b(descs, 3, NULL, NULL, 0) == mxq.MXQ_EINVAL
    assert b(descs, -1, ctypes.byref(plan), NULL, 0) == mxq.MXQ_EINVAL
    assert b(NULL, 3, ctypes.byref(plan), NULL, 0) == mxq.MXQ_EINVAL
    assert b(descs, 3, ctypes.byref(plan), NULL, 0) == mxq.MXQ_OK      # sizes only
    assert (plan.n_entries, plan.n_groups, plan.total_tiles) == (2, 0, 3 * 3 + 1)
    assert plan.table_bytes == 176 and plan.workspace_bytes == 176    # 2 x (80 + 4), to 16
    img = (ctypes.c_ubyte * 176)()
    assert b(descs, 3, ctypes.byref(plan), img, 175) == mxq.MXQ_ESIZE
    assert b(descs, 3, ctypes.byref(plan), img, 176) == mxq.MXQ_OK
    w = np.frombuffer(bytes(img), dtype=np.int64, count=20)
    assert list(w[:10]) == [0x10000, 0x20000, 0x30000, 40, 1056, 1056, 1056, 33, 0, 3]
    assert list(w[10:]) == [0x40000, 0x50000, 0x60000, 8, 64, 72, 64, 2, 9, 1]
    assert list(np.frombuffer(bytes(img), dtype=np.int32, offset=160, count=2)) == [0, 9]
    bad_desc = (mxq.GroupDesc * 1)(mxq.GroupDesc(0x10000, 0x20000, 0x30000, 8, 48, 48, 48, 2))
    assert b(bad_desc, 1, ctypes.byref(plan), NULL, 0) == mxq.MXQ_ESHAPE
    assert plan.n_entries == 2                                         # untouched on error
    empty = mxq.GroupedPlan()
    assert b(descs, 0, ctypes.byref(empty), NULL, 0) == mxq.MXQ_OK
    assert (empty.n_entries, empty.total_tiles, empty.table_bytes) == (0, 0, 0)

    go = lib.mxq_quantize_rowwise_grouped_plan
    assert go(NULL, P16, 176, NULL) == mxq.MXQ_EINVAL
    assert go(ctypes.byref(plan), NULL, 176, NULL) == mxq.MXQ_EINVAL
    assert go(ctypes.byref(plan), P8, 176, NULL) == mxq.MXQ_EALIGN
    assert go(ctypes.byref(plan), P16, 175, NULL) == mxq.MXQ_ESIZE
    for field, value in [("kind", 0), ("n_entries", 3), ("reserved", 1), ("total_tiles", -1),
                         ("table_bytes", 160), ("n_groups", 1)]:
        alt = mxq.GroupedPlan.from_buffer_copy(plan)
        setattr(alt, field, value)
        assert go(ctypes.byref(alt), P16, 176, NULL) == mxq.MXQ_EINVAL, field
    assert lib.nvfp4_quantize_grouped_plan(ctypes.byref(plan), P16, P16, 176, NULL) == mxq.MXQ_EINVAL

    nb = lib.nvfp4_grouped_plan_build
    nd = (mxq.NvGroupDesc * 3)()
    nd[0] = mxq.NvGroupDesc(0x10000, 0x20000, 0x30000, 40, 1056, 1, 0)
    nd[1] = mxq.NvGroupDesc(None, None, None, 0, 32, 0, 0)
    nd[2] = mxq.NvGroupDesc(0x40000, 0x50000, 0x60000, 8, 32, 0, 0)
    nplan = mxq.GroupedPlan()
    assert nb(nd, 3, 0, ctypes.byref(nplan), NULL, 0) == mxq.MXQ_EINVAL     # no groups
    assert nb(nd, 3, 1, ctypes.byref(nplan), NULL, 0) == mxq.MXQ_EINVAL     # group 1 out of range
    assert nb(nd, 3, 2, NULL, NULL, 0) == mxq.MXQ_EINVAL
    assert nb(nd, 3, 2, ctypes.byref(nplan), NULL, 0) == mxq.MXQ_OK
    assert (nplan.n_entries, nplan.n_groups, nplan.total_tiles) == (2, 2, 7)
    assert nplan.table_bytes == 128 and nplan.workspace_bytes == 128 + 32   # 7 partials, to 16
    nimg = (ctypes.c_ubyte * 128)()
    assert nb(nd, 3, 2, ctypes.byref(nplan), nimg, 128) == mxq.MXQ_OK
    raw = bytes(nimg)
    assert list(np.frombuffer(raw, np.int64, 6, 0)) == [0x10000, 0x20000, 0x30000, 40, 1056, 3]
    assert list(np.frombuffer(raw, np.int32, 2, 48)) == [0, 1]              # first tile, group
    assert list(np.frombuffer(raw, np.int64, 6, 56)) == [0x40000, 0x50000, 0x60000, 8, 32, 1]
    assert list(np.frombuffer(raw, np.int32, 2, 104)) == [6, 0]
    assert list(np.frombuffer(raw, np.int32, 4, 112)) == [0, 6, 1, 0]       # starts, groups
    nd[2] = mxq.NvGroupDesc(0x40000, 0x50000, 0x60000, 8, 24, 0, 0)
    assert nb(nd, 3, 2, ctypes.byref(nplan), NULL, 0) == mxq.MXQ_ESHAPE

    ngo = lib.nvfp4_quantize_grouped_plan
    assert ngo(ctypes.byref(nplan), NULL, P16, 160, NULL) == mxq.MXQ_EINVAL  # no global scales
    assert ngo(ctypes.byref(nplan), P2, P16, 160, NULL) == mxq.MXQ_EALIGN
    assert ngo(ctypes.byref(nplan), P16, NULL, 160, NULL) == mxq.MXQ_EINVAL
    assert ngo(ctypes.byref(nplan), P16, P8, 160, NULL) == mxq.MXQ_EALIGN
    assert ngo(ctypes.byref(nplan), P16, P16, 159, NULL) == mxq.MXQ_ESIZE
    for field, value in [("kind", 0), ("n_entries", 1), ("workspace_bytes", 128),
                         ("n_groups", 0)]:
        alt = mxq.GroupedPlan.from_buffer_copy(nplan)
        setattr(alt, field, value)
        assert ngo(ctypes.byref(alt), P16, P16, 160, NULL) == mxq.MXQ_EINVAL, field
    assert go(ctypes.byref(nplan), P16, 160, NULL) == mxq.MXQ_EINVAL
