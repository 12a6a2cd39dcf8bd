"""Helpers for the GPU parity tests: moving bf16 bit patterns between numpy
(oracle side) and torch device tensors (HIP side), and byte-exact compares."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

# Host threads for oracle work in the full-size tests.  The oracle's C calls
# release the GIL, so tensors run in parallel; 16 is the host CPU share a GPU
# box grants one GPU, whatever os.cpu_count() reports there.
HOST_THREADS = max(1, min(16, os.cpu_count() or 1))


def parallel_map(fn, items, workers: int = HOST_THREADS):
    """[fn(item) for item in items] over a thread pool, in order; the first
    exception raised by any call is re-raised."""
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))


def to_dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bits (numpy) -> bf16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bits16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> uint16 numpy bits."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def f32bits(t) -> np.ndarray:
    a = t.detach().cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def assert_same(name: str, got: np.ndarray, want: np.ndarray):
    """Bit-exact equality, reporting the first mismatches."""
    assert got.shape == want.shape, f"{name}: shape {got.shape} != {want.shape}"
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        n = len(bad)
        first = [(tuple(int(i) for i in b), int(got[tuple(b)]), int(want[tuple(b)])) for b in bad[:8]]
        raise AssertionError(f"{name}: {n} mismatches of {got.size}; first (index, got, want): {first}")


def announce(case: str):
    """Name the case on stdout before a GPU step (flushed, so it survives a crash)."""
    print(f"[gpu case] {case}", flush=True)
    sys.stdout.flush()
