"""The streaming-ceiling kernels bench.py times beside the quantizers
(bench_streams.hip): every tiled and flat variant launches with status 0 and
writes nothing outside the buffers it is given, on a ragged shape; bad
arguments are refused before any launch."""
import ctypes

import pytest
import torch

import bench
from gpu_util import announce

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes of 0xA5 after every buffer


def _buf(nbytes):
    return torch.full((nbytes + GUARD,), 0xA5, dtype=torch.uint8, device="cuda")


def _guard_intact(t, nbytes):
    return bool((t[nbytes:] == 0xA5).all().item())


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


@pytest.fixture(scope="module")
def streams():
    return bench.load_streams()


@pytest.fixture
def sp():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


ROWS, COLS = 37, 1024  # 37 rows: the last row block of every tile height is partial
E = ROWS * COLS


def test_every_tiled_variant_stays_in_its_buffers(streams, sp):
    kinds = streams.bench_streams_kinds()
    assert kinds == len(bench.MIXES)
    sizes = {"x": 2 * E, "o8a": E, "o8b": E, "o16": 2 * E, "sc": E // 32}
    for v in range(32 * kinds):  # 4 tile heights x kinds x 2 orders x 2 tile widths x 2 caps
        announce(f"bench_stream_tiled variant {v}")
        b = {k: _buf(n) for k, n in sizes.items()}
        sink = _buf(64)
        st = streams.bench_stream_tiled(v, _p(b["x"]), ROWS, COLS, _p(b["o8a"]), _p(b["o8b"]),
                                        _p(b["o16"]), _p(b["sc"]), _p(sink), sp)
        torch.cuda.synchronize()
        assert st == 0, v
        for k, n in sizes.items():
            assert _guard_intact(b[k], n), (v, k)
        assert _guard_intact(sink, 64), v


def test_every_flat_variant_stays_in_its_buffers(streams, sp):
    kinds = streams.bench_streams_kinds()
    nvec = E // 8
    sizes = {"x": 16 * nvec, "o8a": 8 * nvec, "o8b": 8 * nvec, "o16": 16 * nvec}
    for v in range(3 * kinds):  # 3 depths x kinds
        for grid in (1, 7, 1024):
            announce(f"bench_stream_flat variant {v} grid {grid}")
            b = {k: _buf(n) for k, n in sizes.items()}
            sink = _buf(64)
            st = streams.bench_stream_flat(v, _p(b["x"]), nvec, _p(b["o8a"]), _p(b["o8b"]),
                                           _p(b["o16"]), _p(sink), grid, sp)
            torch.cuda.synchronize()
            assert st == 0, (v, grid)
            for k, n in sizes.items():
                assert _guard_intact(b[k], n), (v, grid, k)
            assert _guard_intact(sink, 64), (v, grid)


def test_bad_arguments_are_refused_before_any_launch(streams, sp):
    kinds = streams.bench_streams_kinds()
    b = _buf(2 * E)
    sink = _buf(64)
    before = b.clone()
    null = ctypes.c_void_p(None)
    for v, rows, cols, o8a in ((-1, ROWS, COLS, b), (32 * kinds, ROWS, COLS, b),
                               (0, ROWS, 1000, b), (0, ROWS, 768, b), (8 * kinds, ROWS, 1000, b),
                               (0, 0, COLS, b), (0, ROWS, COLS, None)):
        st = streams.bench_stream_tiled(v, _p(b), rows, cols, null if o8a is None else _p(b),
                                        _p(b), _p(b), _p(b), _p(sink), sp)
        assert st == 1, (v, rows, cols)
    for v, nvec, grid in ((-1, 8, 1), (3 * kinds, 8, 1), (0, 0, 1), (0, 8, 0), (0, 8, 65537)):
        st = streams.bench_stream_flat(v, _p(b), nvec, _p(b), _p(b), _p(b), _p(sink), grid, sp)
        assert st == 1, (v, nvec, grid)
    torch.cuda.synchronize()
    assert torch.equal(b, before) and _guard_intact(sink, 64)
