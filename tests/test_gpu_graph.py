"""The entry points inside a captured HIP graph.

The single-tensor entry points launch kernels only (no allocation, no copy,
no memset), so a caller can capture them.  One graph holds the MXFP8 one-pass
(column-wise + row-wise + fake-quant), MXFP4 quantize, block-FP8 quantize and
NVFP4 quantize (three kernels: amax partials, finalize, encode) of a static
input.  The graph is replayed on three different inputs, written into the
static buffer by eager copies between replays; every replay's outputs must
equal, bit for bit, the same calls made eagerly, and the first replay's must
equal the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import block_scaled_precision_mxfp8_amd as mxq
import workloads
from gpu_util import announce, assert_same, bits16, f32bits, to_dev_bf16, u8

pytestmark = pytest.mark.gpu

ROWS, COLS = 200, 1056


def _alloc(dev):
    return dict(
        qc=torch.empty((ROWS, COLS), dtype=torch.uint8, device=dev),
        sc=torch.empty(((ROWS + 31) // 32, COLS), dtype=torch.uint8, device=dev),
        qr=torch.empty((ROWS, COLS), dtype=torch.uint8, device=dev),
        sr=torch.empty((ROWS, COLS // 32), dtype=torch.uint8, device=dev),
        fq=torch.empty((ROWS, COLS), dtype=torch.bfloat16, device=dev),
        q4=torch.empty((ROWS, COLS // 2), dtype=torch.uint8, device=dev),
        s4=torch.empty((ROWS, COLS // 32), dtype=torch.uint8, device=dev),
        bq=torch.empty((ROWS, COLS), dtype=torch.uint8, device=dev),
        bS=torch.empty(((ROWS + 127) // 128, (COLS + 127) // 128), dtype=torch.float32, device=dev),
        nq=torch.empty((ROWS, COLS // 2), dtype=torch.uint8, device=dev),
        ns=torch.empty((ROWS, COLS // 16), dtype=torch.uint8, device=dev),
        ng=torch.empty((1,), dtype=torch.float32, device=dev),
        ws=torch.empty((mxq.load().nvfp4_workspace_size(),), dtype=torch.uint8, device=dev),
    )


def _launch_all(lib, x, o):
    """Every call on torch's current stream (the capture stream inside a graph)."""
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.mxq_quantize_colwise(P(x), ROWS, COLS, P(o["qc"]), P(o["sc"]), P(o["qr"]), P(o["sr"]),
                                    P(o["fq"]), sp) == mxq.MXQ_OK
    assert lib.mxfp4_quantize(P(x), ROWS, COLS, P(o["q4"]), P(o["s4"]), None, sp) == mxq.MXQ_OK
    assert lib.blockfp8_quantize(P(x), ROWS, COLS, 128, P(o["bq"]), P(o["bS"]), sp) == mxq.MXQ_OK
    assert lib.nvfp4_quantize(P(x), ROWS, COLS, P(o["nq"]), P(o["ns"]), P(o["ng"]), P(o["ws"]),
                              o["ws"].numel(), sp) == mxq.MXQ_OK


def _host(o):
    return {k: (bits16(v) if v.dtype == torch.bfloat16 else
                f32bits(v) if v.dtype == torch.float32 else u8(v))
            for k, v in o.items() if k != "ws"}


def test_graph_replays_match_eager_and_oracle(gpu, orc):
    lib = gpu.load()
    dev = torch.device("cuda")
    inputs = [workloads.random_bf16((ROWS, COLS), 700 + k) for k in range(3)]
    inputs[1][3, 5] = 0x7FC0                      # a NaN group / tile / tensor in replay 2
    x = to_dev_bf16(inputs[0])                    # the graph's static input
    og, oe = _alloc(dev), _alloc(dev)             # graph outputs, eager outputs
    announce("graph capture: MXFP8 one-pass, MXFP4, block-FP8, NVFP4")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                 # warm-up outside the capture
        _launch_all(lib, x, og)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _launch_all(lib, x, og)
    torch.cuda.synchronize()
    for k, xb in enumerate(inputs):
        announce(f"graph replay {k}")
        x.copy_(to_dev_bf16(xb))                  # eager work between replays
        torch.cuda.synchronize()
        for t in og.values():
            if t.dtype == torch.uint8:
                t.fill_(0xA5)                     # stale bytes must be overwritten
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _launch_all(lib, x, oe)
        torch.cuda.synchronize()
        hg, he = _host(og), _host(oe)
        for name in hg:
            assert_same(f"replay {k} {name} vs eager", hg[name], he[name])
        if k == 0:
            oqc, osc = orc.mxfp8_quantize_colwise(xb)
            oqr, osr = orc.mxfp8_quantize_rowwise(xb)
            assert_same("graph qc", hg["qc"], oqc)
            assert_same("graph sc", hg["sc"], osc)
            assert_same("graph qr", hg["qr"], oqr)
            assert_same("graph sr", hg["sr"], osr)
            assert_same("graph fq", hg["fq"], orc.mxfp8_dequantize(oqr, osr, 1))
            oq4, os4 = orc.mxfp4_quantize(xb)
            assert_same("graph q4", hg["q4"], oq4)
            assert_same("graph s4", hg["s4"], os4)
            obq, obS = orc.blockfp8_quantize(xb, 128)
            assert_same("graph bq", hg["bq"], obq)
            assert_same("graph bS", hg["bS"], f32bits(obS))
            onq, ons, ong = orc.nvfp4_quantize(xb)
            assert_same("graph nq", hg["nq"], onq)
            assert_same("graph ns", hg["ns"], ons)
            assert_same("graph ng", hg["ng"], f32bits(ong))
        if k == 1:
            assert np.isnan(og["ng"].cpu().numpy()[0])   # the NaN made it into the replay
