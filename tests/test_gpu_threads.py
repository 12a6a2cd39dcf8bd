"""Host threads and streams: the library keeps no state, so calls from several
host threads, each on its own stream, run side by side and each returns
exactly the oracle's bytes."""
import threading

import numpy as np
import pytest
import torch

import workloads
from gpu_util import announce, assert_same, bits16, f32bits, to_dev_bf16, u8

pytestmark = pytest.mark.gpu


def test_concurrent_threads_on_their_own_streams(gpu, orc):
    shapes = [(96, 544), (130, 1056), (33, 7168), (256, 512)]
    inputs = [workloads.random_bf16(sh, 1300 + i) for i, sh in enumerate(shapes)]
    results, errors = [None] * len(shapes), []
    announce(f"{len(shapes)} host threads, one stream each")

    def work(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                x = to_dev_bf16(inputs[i])
                outs = []
                for _ in range(8):  # repeated calls, overlapping the other threads'
                    q, sc, fq = gpu.quantize_rowwise(x, fake_quant=True)
                    col = gpu.quantize_colwise(x, rowwise=False, fake_quant=False)
                    nq, ns, ng = gpu.nvfp4_quantize(x)
                    outs.append((q, sc, fq, col["q_col"], col["s_col"], nq, ns, ng))
            s.synchronize()
            results[i] = outs
        except Exception as exc:  # reported below, in the main thread
            errors.append(exc)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(shapes))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    assert all(not t.is_alive() for t in threads)
    for xb, outs in zip(inputs, results):
        oq, os_ = orc.mxfp8_quantize_rowwise(xb)
        ofq = orc.mxfp8_dequantize(oq, os_, 1)
        oqc, osc = orc.mxfp8_quantize_colwise(xb)
        onq, ons, ong = orc.nvfp4_quantize(xb)
        for k, (q, sc, fq, qc, scc, nq, ns, ng) in enumerate(outs):
            name = f"{xb.shape} call {k}"
            assert_same(f"{name} q", u8(q), oq)
            assert_same(f"{name} s", u8(sc), os_)
            assert_same(f"{name} fq", bits16(fq), ofq)
            assert_same(f"{name} q_col", u8(qc), oqc)
            assert_same(f"{name} s_col", u8(scc), osc)
            assert_same(f"{name} nvfp4 q", u8(nq), onq)
            assert_same(f"{name} nvfp4 s", u8(ns), ons)
            assert_same(f"{name} nvfp4 g", f32bits(ng), f32bits(ong))
    assert np.all([r is not None for r in results])
