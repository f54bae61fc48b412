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


# --------------------------------------------------------------------------
# combine bars
# --------------------------------------------------------------------------

def check_bf16_sum(y_bits: np.ndarray, ref32: np.ndarray, y_oracle: np.ndarray, what: str = ""):
    """The BF16 combine / reduce-scatterv bar, element by element: finite
    references satisfy |y - ref| <= 2^-7 |ref| + 1e-3 with ref the oracle's
    fp32 sum in ascending rank order (the bar as stated); both sides add
    the same fp32 terms in the same order from +0 and round once, so y must
    also equal the oracle's bf16 result bit for bit (NaN as a class)."""
    y = bf16_bits_to_f64(y_bits)
    r = np.asarray(ref32, np.float64)
    fin = np.isfinite(r)
    with np.errstate(invalid="ignore"):  # inf - inf where both are infinite
        err = np.abs(y - r)
    bad = fin & ~(err <= 2.0 ** -7 * np.abs(r) + 1e-3)
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside 2^-7|ref| + 1e-3, worst {err[fin].max()}"
    assert np.array_equal(y[~fin & ~np.isnan(r)], r[~fin & ~np.isnan(r)]), f"{what}: infinite sums differ"
    yo = np.asarray(y_oracle, np.uint16)
    nan_o = np.isnan(bf16_bits_to_f64(yo))
    assert np.array_equal(np.isnan(y), nan_o), f"{what}: NaN positions differ"
    diff = (np.asarray(y_bits, np.uint16) != yo) & ~nan_o
    assert not diff.any(), f"{what}: {int(diff.sum())} elements differ from the oracle's bf16 result"


def fp8_exact_bound(terms_abs_sum, floor):
    """Bound of |y - exact sum of the bf16 terms| for the FP8 combine.

    Each term is quantised to e4m3 with a power-of-two block scale 2^e:
    within 2^-4 of its value where the scaled value is an e4m3 normal, else
    within half a subnormal step, 2^(e-10) (floor = the sum of those over
    the token's ranks).  The dequantised terms are summed in fp32 ((m-1)
    2^-24 relative, m <= 64) and rounded once to bf16 (2^-8 relative, or
    2^-134 absolute among bf16 subnormals).  Together:
    (2^-4 + 2^-8 (1 + 2^-4) + 64 * 2^-24 * 1.07) sum|t| <= 0.0667 sum|t|,
    within the stated 0.07 sum|terms|, plus (1 + 2^-8 + 64 * 2^-24) floor,
    taken as (1 + 2^-7) floor, plus 2^-133."""
    return 0.07 * terms_abs_sum + (1.0 + 2.0 ** -7) * floor + 2.0 ** -133


def check_fp8_sum(y_bits, y_oracle, exact, terms_abs_sum, floor, what=""):
    """FP8 combine bars: y equals the oracle's bf16 result (fp32 sum of the
    same dequantised terms in the same order) bit for bit, NaN as a class;
    finite results lie within fp8_exact_bound of the exact sum of the bf16
    terms.  Returns the number of elements outside the literal
    0.07 * sum|terms| (the subnormal-scale floor is what lets them pass)."""
    yo = np.asarray(y_oracle, np.uint16)
    y = bf16_bits_to_f64(y_bits)
    nan_o = np.isnan(bf16_bits_to_f64(yo))
    assert np.array_equal(np.isnan(y), nan_o), f"{what}: NaN positions differ"
    diff = (np.asarray(y_bits, np.uint16) != yo) & ~nan_o
    assert not diff.any(), f"{what}: {int(diff.sum())} elements differ from the oracle's bf16 result"
    fin = np.isfinite(exact) & np.isfinite(y)
    with np.errstate(invalid="ignore"):
        err = np.abs(y - exact)
    bound = fp8_exact_bound(terms_abs_sum, floor)
    bad = fin & ~(err <= bound)
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside the FP8 bound, worst excess {(err - bound)[fin].max()}"
    return int((fin & (err > 0.07 * terms_abs_sum)).sum())


def fp8_terms_and_floor(ev, valid, land_scales_s, s, T, n, P):
    """sum|terms| and the e4m3-subnormal floor sum_r 2^(e_r,b - 10) of the
    first n tokens of source s: ev [P, P*T, H] float64 expert outputs,
    valid [P, P*T], land_scales_s [P*T, H/32] (the oracle's scale codes of
    source s's landing plane, slot r*T + t)."""
    H = ev.shape[-1]
    mag = np.zeros((n, H))
    floor = np.zeros((n, H))
    for r in range(P):
        vr = valid[r, s * T:s * T + n]
        mag += np.where(vr[:, None], np.abs(ev[r, s * T:s * T + n]), 0.0)
        e = land_scales_s[r * T:r * T + n].astype(np.int64) - 127
        floor += np.where(vr[:, None], np.repeat(2.0 ** (e - 10), 32, axis=1), 0.0)
    return mag, floor
