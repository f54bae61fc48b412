"""CPU oracle of the MoE expert-parallel exchange (test infrastructure).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  The product path (the
HIP library and its binding) never imports this package.

The arithmetic lives in ``moe_ep_oracle.c`` (plain single-threaded C);
this module compiles it with gcc on first use and wraps it with numpy
arrays.  See the C file's header for the definitions and the pages each
one follows.  Every sum over ranks comes back twice: ``ref``, the fp32 sum
in ascending rank order from +0 (the reference the combine tolerance is
stated against; ``y`` is ``ref`` rounded to bf16), and ``exact``, the same
sum in double (exact for sums of bf16 or e4m3 terms).

Parity status: every function here is pinned by the CPU tests
(brute force on tiny inputs, closed forms, invariants, library codecs and
hand-worked golden cases under ``tests/golden``); none is unpinned.
"""
from __future__ import annotations

import collections
import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_ep_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no threads, no vector intrinsics)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        # ISO C11 with SSE arithmetic: float operations round to single
        # precision one by one (no contraction, no excess precision)
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            _lib = _declare(C.CDLL(_LIB))
    return _lib


_p = C.c_void_p
_i = C.c_int
_i64 = C.c_int64


def _declare(L):
    L.orc_bf16_to_double.argtypes = [C.c_uint16]
    L.orc_bf16_to_double.restype = C.c_double
    L.orc_double_to_bf16.argtypes = [C.c_double]
    L.orc_double_to_bf16.restype = C.c_uint16
    L.orc_e4m3_to_double.argtypes = [C.c_uint8]
    L.orc_e4m3_to_double.restype = C.c_double
    L.orc_double_to_e4m3.argtypes = [C.c_double]
    L.orc_double_to_e4m3.restype = C.c_uint8
    L.orc_fp8_block_exponent.argtypes = [C.c_double]
    L.orc_fp8_block_exponent.restype = _i
    L.orc_fp8_quantize_row.argtypes = [_i, _p, _p, _p]
    L.orc_fp8_quantize_row.restype = None
    L.orc_fp8_dequant.argtypes = [C.c_uint8, C.c_uint8]
    L.orc_fp8_dequant.restype = C.c_double
    L.orc_owner.argtypes = [C.c_int32, _i, _i]
    L.orc_owner.restype = _i
    L.orc_token_goes_to.argtypes = [_p, _i, _i, _i, _i]
    L.orc_token_goes_to.restype = _i
    L.orc_dispatch.argtypes = [_i, _i, _i, _i, C.c_int32, C.c_uint64, _p, _p, _i64, _p, _i64,
                               _p, _i64, _p, _p, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p]
    L.orc_dispatch.restype = None
    L.orc_combine_token_bf16.argtypes = [_i, _i, _i, _i, C.c_uint64, _p, _p, _i64, _p, _p, _p]
    L.orc_combine_token_bf16.restype = None
    L.orc_combine_bf16.argtypes = [_i, _i, _i, _i, _i, C.c_uint64, _p, _p, _p, _i64, _i64, _i, _i,
                                   _p, _p, _p]
    L.orc_combine_bf16.restype = None
    L.orc_combine_token_fp8.argtypes = [_i, _i, _i, _i, C.c_uint64, _p, _p, _i64, _p, _p, _p, _p, _p]
    L.orc_combine_token_fp8.restype = None
    L.orc_combine_fp8.argtypes = [_i, _i, _i, _i, _i, C.c_uint64, _p, _p, _p, _i64, _i64, _i, _i,
                                  _p, _p, _p, _p, _p, _p, _p]
    L.orc_combine_fp8.restype = None
    L.orc_eplb_allgather.argtypes = [_i, _i, C.c_uint64, _p, _i, _p]
    L.orc_eplb_allgather.restype = None
    L.orc_allgatherv.argtypes = [_i, _p, _i64, _p, _i64, _p]
    L.orc_allgatherv.restype = None
    L.orc_reduce_scatterv.argtypes = [_i, _p, _i, _p, _i, _p, _p, _p]
    L.orc_reduce_scatterv.restype = None
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
# scalar codecs
# --------------------------------------------------------------------------

def bf16_to_double(bits: int) -> float:
    return lib().orc_bf16_to_double(int(bits))


def double_to_bf16(x: float) -> int:
    return int(lib().orc_double_to_bf16(float(x)))


def e4m3_to_double(code: int) -> float:
    return lib().orc_e4m3_to_double(int(code))


def double_to_e4m3(x: float) -> int:
    return int(lib().orc_double_to_e4m3(float(x)))


def fp8_block_exponent(amax: float) -> int:
    return int(lib().orc_fp8_block_exponent(float(amax)))


def fp8_dequant(code: int, scale: int) -> float:
    return lib().orc_fp8_dequant(int(code), int(scale))


def owner(expert_id: int, E: int, P: int) -> int:
    return int(lib().orc_owner(int(expert_id), E, P))


def fp8_quantize_row(x_bits: np.ndarray):
    """e4m3 codes and e8m0 scales of one bf16 row (uint16 bit patterns)."""
    x = _c(x_bits, np.uint16)
    H = x.shape[-1]
    codes = np.zeros(H, np.uint8)
    scales = np.zeros(H // 32, np.uint8)
    lib().orc_fp8_quantize_row(H, _ptr(x), _ptr(codes), _ptr(scales))
    return codes, scales


# --------------------------------------------------------------------------
# dispatch / combine
# --------------------------------------------------------------------------

def _active(active, P):
    return (1 << P) - 1 if active is None else int(active)


def dispatch(counts, payload, ids, weights=None, scales=None, *, E: int,
             invalid_id=None, r0: int = 0, r1=None, want_payload: bool = True, active=None,
             extra=None):
    """Receive planes of destinations r0..r1-1.

    payload: uint8 [P, T, row_bytes]; scales: uint8 [P, T, srow] or None;
    ids: int32 [P, T, k]; weights: float32 [P, T, k] or None;
    counts: int32 [P].  Returns a dict of numpy arrays (see the C doc)."""
    counts = _c(counts, np.int32)
    ids = _c(ids, np.int32)
    P, T, k = ids.shape
    payload = _c(payload, np.uint8)
    row = payload.shape[-1]
    scales = _c(scales, np.uint8)
    srow = 0 if scales is None else scales.shape[-1]
    weights = _c(weights, np.float32)
    extra = _c(extra, np.uint8)
    xrow = 0 if extra is None else extra.shape[-1]
    r1 = P if r1 is None else r1
    nr = r1 - r0
    inv = E if invalid_id is None else invalid_id
    out = {
        "ids": np.zeros((nr, P * T, k), np.int32),
        "valid": np.zeros((nr, P * T), np.uint8),
        "counts": np.zeros((nr, P), np.int32),
        "slots": np.zeros((nr, P * T), np.int32),
        "payload": np.zeros((nr, P * T, row), np.uint8) if want_payload else None,
        "scales": np.zeros((nr, P * T, srow), np.uint8) if (srow and want_payload) else None,
        "extra": np.zeros((nr, P * T, xrow), np.uint8) if (xrow and want_payload) else None,
        "weights": np.zeros((nr, P * T, k), np.float32) if weights is not None else None,
    }
    lib().orc_dispatch(P, T, k, E, inv, _active(active, P), _ptr(counts), _ptr(payload), row,
                       _ptr(scales), srow, _ptr(extra), xrow,
                       _ptr(ids), _ptr(weights), r0, r1, _ptr(out["payload"]),
                       _ptr(out["scales"]), _ptr(out["extra"]), _ptr(out["ids"]),
                       _ptr(out["weights"]), _ptr(out["valid"]), _ptr(out["counts"]),
                       _ptr(out["slots"]))
    return out


def eplb_allgather(stats, r: int, active=None, out=None):
    """Rank r's gathered [P, n] statistics from stats [P, n] int32 (rows of
    masked-off ranks keep out's previous contents)."""
    stats = _c(stats, np.int32)
    P, n = stats.shape
    out = np.zeros((P, n), np.int32) if out is None else np.ascontiguousarray(out, np.int32)
    lib().orc_eplb_allgather(P, n, _active(active, P), _ptr(stats), r, _ptr(out))
    return out


# Results of the sums over ranks: ref is the fp32 sum in ascending rank
# order from +0 (float32), y / out its bf16 rounding (uint16 bit patterns),
# exact the same sum in double.
BF16Combine = collections.namedtuple("BF16Combine", "ref y exact")
FP8Combine = collections.namedtuple("FP8Combine", "land_codes land_scales ref y exact")
TokenFP8 = collections.namedtuple("TokenFP8", "codes scales ref y exact")
ReduceScatter = collections.namedtuple("ReduceScatter", "ref out exact")


def combine_token_bf16(ids_row, eo_rows, *, E: int, active=None) -> BF16Combine:
    """One token: eo_rows uint16 [P, H] (its slot's row on every rank)."""
    ids_row = _c(ids_row, np.int32)
    eo_rows = _c(eo_rows, np.uint16)
    P, H = eo_rows.shape
    ref = np.zeros(H, np.float32)
    exact = np.zeros(H, np.float64)
    y = np.zeros(H, np.uint16)
    lib().orc_combine_token_bf16(P, H, ids_row.shape[0], E, _active(active, P), _ptr(ids_row),
                                 _ptr(eo_rows), H, _ptr(ref), _ptr(exact), _ptr(y))
    return BF16Combine(ref, y, exact)


def _eo_range(eo, P, T, s0, s1, slot0):
    """Checks that eo [P, nslot, H] (slots slot0 .. slot0 + nslot - 1)
    holds every slot of sources s0 .. s1-1."""
    assert eo.ndim == 3 and eo.shape[0] == P, "eo must be [P, slots, H]"
    nslot = eo.shape[1]
    assert slot0 <= s0 * T and s1 * T <= slot0 + nslot, "eo does not hold the sources' slots"
    return nslot


def combine_bf16(counts, ids, eo, *, E: int, s0: int = 0, s1=None, active=None,
                 slot0: int = 0) -> BF16Combine:
    """BF16 combine of source ranks s0..s1-1.  eo: uint16 [P, nslot, H],
    every rank's expert output for slots slot0 .. slot0 + nslot - 1 (the
    whole [P, P*T, H] tensor by default).  Returns ref float32, y uint16,
    exact float64, each [s1-s0, T, H]; rows t >= n_s stay zero."""
    counts = _c(counts, np.int32)
    ids = _c(ids, np.int32)
    eo = _c(eo, np.uint16)
    P, T, k = ids.shape
    H = eo.shape[-1]
    s1 = P if s1 is None else s1
    nslot = _eo_range(eo, P, T, s0, s1, slot0)
    ref = np.zeros((s1 - s0, T, H), np.float32)
    exact = np.zeros((s1 - s0, T, H), np.float64)
    y = np.zeros((s1 - s0, T, H), np.uint16)
    lib().orc_combine_bf16(P, T, H, k, E, _active(active, P), _ptr(counts), _ptr(ids), _ptr(eo),
                           slot0, nslot, s0, s1, _ptr(ref), _ptr(exact), _ptr(y))
    return BF16Combine(ref, y, exact)


def combine_token_fp8(ids_row, eo_rows, *, E: int, active=None) -> TokenFP8:
    """One token's FP8 combine: codes [P, H], scales [P, H/32] (rows of
    ranks the token went to), ref float32, y uint16, exact float64 [H]."""
    ids_row = _c(ids_row, np.int32)
    eo_rows = _c(eo_rows, np.uint16)
    P, H = eo_rows.shape
    codes = np.zeros((P, H), np.uint8)
    scales = np.zeros((P, H // 32), np.uint8)
    ref = np.zeros(H, np.float32)
    exact = np.zeros(H, np.float64)
    y = np.zeros(H, np.uint16)
    lib().orc_combine_token_fp8(P, H, ids_row.shape[0], E, _active(active, P), _ptr(ids_row),
                                _ptr(eo_rows), H, _ptr(codes), _ptr(scales), _ptr(ref),
                                _ptr(exact), _ptr(y))
    return TokenFP8(codes, scales, ref, y, exact)


def combine_fp8(counts, ids, eo, *, E: int, s0: int = 0, s1=None, active=None,
                slot0: int = 0) -> FP8Combine:
    """FP8 combine of source ranks s0..s1-1 (eo as for combine_bf16).
    Returns land_codes [n, P*T, H], land_scales [n, P*T, H/32] (uint8),
    ref float32, y uint16 and exact float64, each [n, T, H]."""
    counts = _c(counts, np.int32)
    ids = _c(ids, np.int32)
    eo = _c(eo, np.uint16)
    P, T, k = ids.shape
    H = eo.shape[-1]
    s1 = P if s1 is None else s1
    nslot = _eo_range(eo, P, T, s0, s1, slot0)
    n = s1 - s0
    land_codes = np.zeros((n, P * T, H), np.uint8)
    land_scales = np.zeros((n, P * T, H // 32), np.uint8)
    ref = np.zeros((n, T, H), np.float32)
    exact = np.zeros((n, T, H), np.float64)
    y = np.zeros((n, T, H), np.uint16)
    sc = np.zeros((P, H), np.uint8)
    ss = np.zeros((P, H // 32), np.uint8)
    lib().orc_combine_fp8(P, T, H, k, E, _active(active, P), _ptr(counts), _ptr(ids), _ptr(eo),
                          slot0, nslot, s0, s1, _ptr(land_codes), _ptr(land_scales), _ptr(ref),
                          _ptr(exact), _ptr(y), _ptr(sc), _ptr(ss))
    return FP8Combine(land_codes, land_scales, ref, y, exact)


def allgatherv(sizes, rows):
    """rows: [P, in_rows, row_bytes] uint8 (rank q uses its first sizes[q]
    rows).  Returns the [sum(sizes), row_bytes] concatenation."""
    sizes = _c(sizes, np.int32)
    rows = _c(rows, np.uint8)
    P, in_rows, rb = rows.shape
    out = np.zeros((int(sizes.sum()), rb), np.uint8)
    lib().orc_allgatherv(P, _ptr(sizes), rb, _ptr(rows), in_rows, _ptr(out))
    return out


def reduce_scatterv(sizes, partial, r: int) -> ReduceScatter:
    """partial: uint16 [P, sum(sizes), H].  Returns ref float32, out
    uint16 and exact float64, each [sizes[r], H]."""
    sizes = _c(sizes, np.int32)
    partial = _c(partial, np.uint16)
    P, total, H = partial.shape
    ref = np.zeros((int(sizes[r]), H), np.float32)
    exact = np.zeros((int(sizes[r]), H), np.float64)
    out = np.zeros((int(sizes[r]), H), np.uint16)
    lib().orc_reduce_scatterv(P, _ptr(sizes), H, _ptr(partial), r, _ptr(ref), _ptr(exact),
                              _ptr(out))
    return ReduceScatter(ref, out, exact)
