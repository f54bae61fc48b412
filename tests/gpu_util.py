"""Helpers of the GPU parity tests: build inputs once, run the HIP path
through the C ABI binding, fetch results as numpy for the oracle."""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import torch

import workloads as W


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def bits16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).double().numpy()


@dataclasses.dataclass
class DispatchCase:
    w: W.Workload
    counts: np.ndarray
    ids: np.ndarray
    weights: np.ndarray
    payload: np.ndarray          # uint8 [P, T, row]
    scales: np.ndarray | None    # uint8 [P, T, srow]


def random_byte_case(w: W.Workload, seed: int, counts=None, oob=False, dup=False) -> DispatchCase:
    """Routing from the workload's generator; payload and scale rows are
    uniformly random bytes (every bf16/fp8 bit pattern: NaN, Inf, -0,
    subnormals), since dispatch must move bytes unchanged."""
    R = W.draw_routing(w, seed)
    rng = np.random.default_rng(seed + 99)
    ids = R.ids.copy()
    if dup and w.k > 1:
        m = rng.random(ids.shape[:2]) < 0.25
        ids[m, 1] = ids[m, 0]
    if oob:
        m = rng.random(ids.shape) < 0.05
        ids[m] = rng.choice([-1, -5, w.E, w.E + 11], size=int(m.sum()))
    row = W.payload_row_bytes(w.fmt, w.H)
    srow = W.scale_row_bytes(w.fmt, w.H)
    payload = rng.integers(0, 256, size=(w.P, w.T, row), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(w.P, w.T, srow), dtype=np.uint8) if srow else None
    c = R.counts if counts is None else np.asarray(counts, np.int32)
    return DispatchCase(w, c, ids.astype(np.int32), R.weights, payload, scales)


def gpu_inputs(c: DispatchCase, dev="cuda"):
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return t(c.payload), t(c.scales), t(c.ids), t(c.weights)
