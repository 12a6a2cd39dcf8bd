"""Grouped launches prepared once (the table built on the host and copied to
the device a single time) against the CPU oracle, bit for bit, and against the
one-call grouped forms.  The inputs are refilled in place between runs, as a
training step does; the last test captures both prepared launches in a HIP
graph and replays it."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import announce, assert_same, f32bits, to_dev_bf16, u8

pytestmark = pytest.mark.gpu

MX_SHAPES = [(64, 512), (1, 32), (33, 96), (0, 64), (97, 7168), (5, 544), (300, 2048)]


def _mx_inputs(seed):
    return [workloads.random_bf16(sh, seed + i, std=0.02 * (i + 1)) if sh[0] else
            np.zeros(sh, np.uint16) for i, sh in enumerate(MX_SHAPES)]


def _nv_inputs(seed):
    shapes = [(33, 48), (1, 16), (0, 32), (130, 528), (64, 1040), (5, 16)]
    return [workloads.random_bf16(sh, seed + k, std=0.02 + 0.01 * k) if sh[0] else
            np.zeros(sh, np.uint16) for k, sh in enumerate(shapes)]


NV_GROUPS, NV_N_GROUPS = [0, 0, 1, 2, 2, 3], 5   # group 4 unused, group 1 only empty


def _check_mx(orc, xs_b, outs, name):
    for i, (b, (q, s)) in enumerate(zip(xs_b, outs)):
        if b.shape[0] == 0:
            continue
        oq, os_ = orc.mxfp8_quantize_rowwise(b)
        assert_same(f"{name}[{i}] q", u8(q), oq)
        assert_same(f"{name}[{i}] s", u8(s), os_)


def _check_nv(orc, xs_b, outs, gs, name):
    oouts, ogs = orc.nvfp4_quantize_grouped(xs_b, NV_GROUPS, NV_N_GROUPS)
    assert_same(f"{name} g", f32bits(gs), f32bits(ogs))
    for i, ((q, s), (oq, os_)) in enumerate(zip(outs, oouts)):
        assert_same(f"{name} q[{i}]", u8(q), oq)
        assert_same(f"{name} s[{i}]", u8(s), os_)


def test_prepared_rowwise_grouped_runs_on_refilled_inputs(gpu, orc):
    xs_b = _mx_inputs(1400)
    xs = [to_dev_bf16(b) for b in xs_b]
    wide = torch.empty((40, 256), dtype=torch.bfloat16, device="cuda")
    xs.append(wide[:, :128])                          # row stride 256 > cols
    announce("prepared MXFP8 grouped: build once")
    prep = gpu.prepare_rowwise_grouped(xs)
    assert prep.plan.n_entries == len(xs) - 1         # the empty tensor has no entry
    for k in range(3):
        announce(f"prepared MXFP8 grouped run {k}")
        new_b = _mx_inputs(1500 + 20 * k)
        wb = workloads.random_bf16((40, 256), 1590 + k)
        for x, b in zip(xs, new_b):
            if b.size:
                x.copy_(to_dev_bf16(b))
        wide.copy_(to_dev_bf16(wb))
        outs = prep.run()
        torch.cuda.synchronize()
        _check_mx(orc, new_b + [np.ascontiguousarray(wb[:, :128])], outs, f"prepared run {k}")
        one = gpu.quantize_rowwise_grouped(xs)        # the one-call form: same bytes
        torch.cuda.synchronize()
        for (q, s), (q1, s1) in zip(outs, one):
            assert torch.equal(q, q1) and torch.equal(s, s1)


def test_prepared_nvfp4_grouped_runs_on_refilled_inputs(gpu, orc):
    xs_b = _nv_inputs(1600)
    xs = [to_dev_bf16(b) for b in xs_b]
    announce("prepared NVFP4 grouped: build once")
    prep = gpu.prepare_nvfp4_grouped(xs, NV_GROUPS, NV_N_GROUPS)
    for k in range(3):
        announce(f"prepared NVFP4 grouped run {k}")
        new_b = _nv_inputs(1700 + 20 * k)
        if k == 1:
            new_b[4][7, 9] = 0x7F80                   # +Inf: group 2 all-NaN in this run only
        for x, b in zip(xs, new_b):
            if b.size:
                x.copy_(to_dev_bf16(b))
        outs, gs = prep.run()
        torch.cuda.synchronize()
        _check_nv(orc, new_b, outs, gs, f"prepared run {k}")


def test_prepared_nvfp4_without_elements_writes_zero_scales(gpu):
    xs = [torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")]
    announce("prepared NVFP4 grouped: no elements, two groups")
    prep = gpu.prepare_nvfp4_grouped(xs, [1], 2)
    assert prep.plan.n_entries == 0 and prep.plan.workspace_bytes == 0
    prep.global_scales.fill_(-1.0)
    _, gs = prep.run()
    torch.cuda.synchronize()
    assert gs.cpu().tolist() == [0.0, 0.0]


def test_prepared_plans_refuse_the_other_kind(gpu):
    xs = [to_dev_bf16(workloads.random_bf16((32, 64), 1800))]
    mx_prep = gpu.prepare_rowwise_grouped(xs)
    nv_prep = gpu.prepare_nvfp4_grouped(xs, [0], 1)
    mx_prep.plan, nv_prep.plan = nv_prep.plan, mx_prep.plan
    for prep in (mx_prep, nv_prep):
        with pytest.raises(gpu.MXQError) as err:
            prep.run()
        assert err.value.status == gpu.MXQ_EINVAL


def test_prepared_grouped_in_a_graph(gpu, orc):
    mx_b, nv_b = _mx_inputs(1900), _nv_inputs(1950)
    mx_x = [to_dev_bf16(b) for b in mx_b]
    nv_x = [to_dev_bf16(b) for b in nv_b]
    announce("prepared grouped launches: graph capture")
    mx_prep = gpu.prepare_rowwise_grouped(mx_x)
    nv_prep = gpu.prepare_nvfp4_grouped(nv_x, NV_GROUPS, NV_N_GROUPS)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                     # warm-up outside the capture
        mx_prep.run()
        nv_prep.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mx_prep.run()
        nv_prep.run()
    torch.cuda.synchronize()
    for k in range(3):
        announce(f"prepared grouped graph replay {k}")
        mb, nb = _mx_inputs(2000 + 20 * k), _nv_inputs(2100 + 20 * k)
        for x, b in zip(mx_x + nv_x, mb + nb):
            if b.size:
                x.copy_(to_dev_bf16(b))               # eager work between replays
        for q, s in mx_prep.outputs + nv_prep.outputs:
            q.fill_(0xA5)                             # stale bytes must be overwritten
            s.fill_(0xA5)
        nv_prep.global_scales.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _check_mx(orc, mb, mx_prep.outputs, f"graph replay {k} MXFP8")
        _check_nv(orc, nb, nv_prep.outputs, nv_prep.global_scales, f"graph replay {k} NVFP4")


def test_one_call_grouped_forms_refuse_capture(gpu, orc):
    """The one-call grouped forms copy their launch table from a host buffer
    that is freed when they return, so under stream capture they refuse with
    MXQ_ECAPTURE and enqueue nothing; the capture ends cleanly, its (empty)
    graph is never replayed, and the same calls then run eagerly and match the
    oracle."""
    import block_scaled_precision_mxfp8_amd as mxq
    xs_b = _mx_inputs(1700)
    xs = [to_dev_bf16(b) for b in xs_b]
    nv_b = _nv_inputs(1800)
    nv = [to_dev_bf16(b) for b in nv_b]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    announce("one-call grouped forms under capture")
    with torch.cuda.stream(side):
        g.capture_begin()
        try:
            with pytest.raises(mxq.MXQError) as e1:
                gpu.quantize_rowwise_grouped(xs)
            with pytest.raises(mxq.MXQError) as e2:
                gpu.nvfp4_quantize_grouped(nv, NV_GROUPS, NV_N_GROUPS)
        finally:
            g.capture_end()
    assert e1.value.status == mxq.MXQ_ECAPTURE and "plan form" in str(e1.value)
    assert e2.value.status == mxq.MXQ_ECAPTURE
    torch.cuda.synchronize()
    announce("one-call grouped forms eagerly after the refused capture")
    _check_mx(orc, xs_b, gpu.quantize_rowwise_grouped(xs), "eager mx")
    outs, gs = gpu.nvfp4_quantize_grouped(nv, NV_GROUPS, NV_N_GROUPS)
    torch.cuda.synchronize()
    _check_nv(orc, nv_b, outs, gs, "eager nv")
