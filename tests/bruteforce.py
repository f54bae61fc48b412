"""Pure-Python brute force of the exchange, for tiny inputs only.

Written as a *push*: every source token is walked once and its row is
appended to a dictionary per destination rank, the way the pages describe
the transfer (FlashInfer ``NVLinkTwoSidedAlltoAll.dispatch``: a token is
delivered to every rank holding one of its chosen experts;
``NVLinkOneSidedConfig``, lamport paragraph: token t of rank src occupies
slot src * tokens_per_rank + t of a receiving rank).  The C oracle is
written as a pull over destination slots; the two share nothing.  Number
conversions use torch.
"""
from __future__ import annotations

import numpy as np
import torch


def _bf16_bits_to_float(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).double().numpy()


def dispatch(counts, payload, ids, weights, scales, E, alive=None):
    """alive: set of ranks taking part (all when None); others neither
    send nor receive (FlashInfer moe_a2a_dispatch, active_rank_mask)."""
    P, T, k = ids.shape
    epr = E // P
    alive = set(range(P)) if alive is None else set(alive)
    recv = [dict() for _ in range(P)]
    for s in range(P):
        if s not in alive:
            continue
        for t in range(int(counts[s])):
            dests = set()
            for e in ids[s][t]:
                if 0 <= int(e) < E and int(e) // epr in alive:
                    dests.add(int(e) // epr)
            for r in dests:
                recv[r][s * T + t] = (
                    bytes(payload[s][t]),
                    None if scales is None else bytes(scales[s][t]),
                    [int(v) for v in ids[s][t]],
                    None if weights is None else [float(v) for v in weights[s][t]],
                )
    return recv


def recv_ids_plane(recv, P, T, k, invalid):
    out = np.full((P, P * T, k), invalid, np.int32)
    for r in range(P):
        for q, rec in recv[r].items():
            out[r, q] = rec[2]
    return out


def counts_and_slots(recv, P, T):
    cnt = np.zeros((P, P), np.int32)
    slots = []
    for r in range(P):
        for q in recv[r]:
            cnt[r, q // T] += 1
        slots.append(sorted(recv[r]))
    return cnt, slots


def combine_bf16(counts, ids, eo_bits, E, alive=None):
    """Sum, per source token, the rows its destinations hold in its slot.
    Returns {(s, t): list of float sums} (Python floats, ascending r)."""
    P, T, k = ids.shape
    epr = E // P
    alive = set(range(P)) if alive is None else set(alive)
    out = {}
    for s in range(P):
        if s not in alive:
            continue
        for t in range(int(counts[s])):
            dests = sorted({int(e) // epr for e in ids[s][t] if 0 <= int(e) < E} & alive)
            acc = [0.0] * eo_bits.shape[-1]
            for r in dests:
                row = _bf16_bits_to_float(eo_bits[r, s * T + t])
                for h, v in enumerate(row):
                    acc[h] += float(v)
            out[(s, t)] = acc
    return out


def combine_bf16_fp32(counts, ids, eo_bits, E, alive=None):
    """The same push-style walk summing in single precision: numpy float32
    additions one rank at a time, ascending r, from +0.  Returns
    {(s, t): float32 array}."""
    P, T, k = ids.shape
    epr = E // P
    alive = set(range(P)) if alive is None else set(alive)
    out = {}
    for s in range(P):
        if s not in alive:
            continue
        for t in range(int(counts[s])):
            dests = sorted({int(e) // epr for e in ids[s][t] if 0 <= int(e) < E} & alive)
            acc = np.zeros(eo_bits.shape[-1], np.float32)
            for r in dests:
                acc = (acc + _bf16_bits_to_float(eo_bits[r, s * T + t]).astype(np.float32)).astype(np.float32)
            out[(s, t)] = acc
    return out


def fp8_dequantise(codes, scales):
    """Values of e4m3 codes [..., H] with one e8m0 scale per 32 elements
    [..., H/32] (torch's float8_e4m3fn decode times 2^(scale - 127); a
    scale of 0xFF is NaN), float64."""
    c = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).double()
    sc = np.asarray(scales, np.int64)
    mult = np.where(sc == 0xFF, np.nan, np.ldexp(1.0, sc - 127))
    return c.numpy() * np.repeat(mult, 32, axis=-1)


def reduce_scatterv_fp32(sizes, partial_bits, r):
    """Rank r's rows of the reduce-scatterv: float32 sums of every rank's
    partial row, ascending rank, from +0."""
    P = len(sizes)
    off = sum(int(sizes[q]) for q in range(r))
    acc = np.zeros((int(sizes[r]), partial_bits.shape[-1]), np.float32)
    for q in range(P):
        acc = (acc + _bf16_bits_to_float(partial_bits[q, off:off + int(sizes[r])]).astype(np.float32)).astype(np.float32)
    return acc
