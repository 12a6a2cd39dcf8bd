"""GPU parity of grouped NVFP4 (global scales shared within scale groups)
against the CPU oracle, bit for bit: the per-half (QAT) and shared
weight_scale_2 (export) conventions for fused gated-MoE gate/up weights."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import announce, assert_same, bits16, f32bits, parallel_map, to_dev_bf16, u8

pytestmark = pytest.mark.gpu


def check_grouped(gpu, orc, xs_bits, groups, n_groups, name, workspace=None):
    announce(f"nvfp4 grouped {name}: {len(xs_bits)} tensors, {n_groups} groups")
    xs = [to_dev_bf16(x) for x in xs_bits]
    outs, gs = gpu.nvfp4_quantize_grouped(xs, groups, n_groups, workspace=workspace)
    torch.cuda.synchronize()
    oouts, ogs = orc.nvfp4_quantize_grouped(xs_bits, groups, n_groups)
    assert_same(f"{name} g", f32bits(gs), f32bits(ogs))
    for i, ((q, s), (oq, os_)) in enumerate(zip(outs, oouts)):
        assert_same(f"{name} q[{i}]", u8(q), oq)
        assert_same(f"{name} s[{i}]", u8(s), os_)


def experts(n, rows, cols, seed):
    mult = np.random.default_rng(seed).uniform(0.5, 2.0, n)
    xs = []
    for e in range(n):
        xs.append(workloads.random_bf16((rows, cols), seed + 2 * e, std=0.02 * mult[e]))       # gate
        xs.append(workloads.random_bf16((rows, cols), seed + 2 * e + 1, std=0.03 * mult[e]))   # up
    return xs


def test_grouped_per_half(gpu, orc):
    xs = experts(4, 64, 256, 100)
    check_grouped(gpu, orc, xs, list(range(len(xs))), len(xs), "per-half")


def test_grouped_shared_gate_up(gpu, orc):
    xs = experts(4, 64, 256, 200)
    check_grouped(gpu, orc, xs, [i // 2 for i in range(len(xs))], len(xs) // 2, "shared")


def test_grouped_mixed_shapes_empty_unused_nonfinite(gpu, orc):
    xs = [workloads.random_bf16(sh, 300 + k) for k, sh in
          enumerate([(33, 48), (1, 16), (0, 32), (130, 528), (64, 1040), (5, 16)])]
    xs[4][7, 9] = 0x7F80                      # +Inf: group 2 becomes all-NaN
    groups = [0, 0, 1, 2, 2, 3]
    check_grouped(gpu, orc, xs, groups, 5, "mixed")   # group 4 unused, group 1 only empty


def test_grouped_zero_group(gpu, orc):
    xs = [np.zeros((16, 64), np.uint16), workloads.random_bf16((16, 64), 5)]
    xs[0][3, 3] = 0x8000                      # -0 keeps its sign
    check_grouped(gpu, orc, xs, [0, 1], 2, "zero")


def test_grouped_full_size_experts(gpu, orc):
    """Four experts' gate and up at full size [2048, 7168], shared scales."""
    xs = experts(4, 2048, 7168, 400)
    check_grouped(gpu, orc, xs, [i // 2 for i in range(len(xs))], 4, "full-size")


@pytest.mark.timeout(900)
def test_grouped_moe_gate_up_full(gpu, orc):
    """The benchmarked launch: the gate and up weights of all 128 MoE experts
    ([2048, 7168] each, drawn as the moe_experts workload draws them) in one
    grouped call, gate and up of an expert sharing one global scale.  Every
    expert's g and every tensor's codes and scales against the oracle, which
    runs expert by expert (a scale group depends on its members only) over
    host threads."""
    shapes = workloads.moe_shapes()
    mult = workloads.moe_multipliers()
    gu = [i for i, (name, _, _) in enumerate(shapes)
          if name.endswith(("gate_proj.weight", "up_proj.weight"))]
    n_exp = len(shapes) // 3
    assert len(gu) == 2 * n_exp
    announce(f"nvfp4 grouped moe gate/up: {len(gu)} tensors, {n_exp} groups")
    xs = [workloads.moe_tensor(i, shapes[i][1], shapes[i][2], mult[i // 3], "cuda") for i in gu]
    outs, gs = gpu.nvfp4_quantize_grouped(xs, [i // 3 for i in gu], n_exp)
    torch.cuda.synchronize()
    g_got = f32bits(gs)
    announce("nvfp4 grouped moe gate/up: oracle per expert")

    def check(e):
        k0, k1 = 2 * e, 2 * e + 1            # gate and up of expert e in xs
        assert gu[k0] // 3 == e and gu[k1] // 3 == e
        oouts, og = orc.nvfp4_quantize_grouped([bits16(xs[k0]), bits16(xs[k1])], [0, 0], 1)
        assert_same(f"expert {e} g", g_got[e:e + 1], f32bits(og))
        for k, (oq, os_) in zip((k0, k1), oouts):
            assert_same(f"expert {e} q[{k}]", u8(outs[k][0]), oq)
            assert_same(f"expert {e} s[{k}]", u8(outs[k][1]), os_)
        return e

    assert parallel_map(check, range(n_exp)) == list(range(n_exp))


def test_grouped_workspace_needs_no_initial_contents(gpu, orc):
    xs = experts(2, 96, 512, 500)
    groups = [0, 0, 1, 1]
    from block_scaled_precision_mxfp8_amd import NvGroupDesc
    n = gpu.load().nvfp4_grouped_workspace_size((NvGroupDesc * 4)(*[
        NvGroupDesc(None, None, None, x.shape[0], x.shape[1], g, 0) for x, g in zip(xs, groups)]), 4)
    ws = torch.randint(0, 256, (int(n) + 64,), dtype=torch.uint8, device="cuda")
    check_grouped(gpu, orc, xs, groups, 2, "garbage-ws-1", workspace=ws)
    ws.fill_(0xFF)
    check_grouped(gpu, orc, xs, groups, 2, "garbage-ws-2", workspace=ws)
