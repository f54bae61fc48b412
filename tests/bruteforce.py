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
