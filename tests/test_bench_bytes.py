"""The bench's algorithmic byte counts against a count taken from the
oracle's own dispatch result: M is the number of valid receive slots the
oracle produces, and each byte term is rebuilt from what the exchange must
read and write (token rows read once, one row per valid slot written, k ids
+ k weights per token read, k ids + k weights per valid slot written, k
marker ids per empty slot; combine reads one row per valid slot and writes
one per token)."""
import dataclasses

import numpy as np
import pytest

import bench
import oracle
import workloads as W


CASES = [
    dataclasses.replace(W.TINY, name="tiny"),
    dataclasses.replace(W.EP8_BF16, name="ep8 small", T=40, H=256, n_lo=0, n_hi=40),
    dataclasses.replace(W.EP8_MXFP8, name="mxfp8 zipf", T=24, H=256, n_lo=24, n_hi=24),
    dataclasses.replace(W.EP64_NVFP4, name="nvfp4 P64", T=6, H=64, n_lo=0, n_hi=6),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_step_bytes_match_the_oracle_count(w):
    R = W.draw_routing(w)
    row = W.payload_row_bytes(w.fmt, w.H)
    srow = W.scale_row_bytes(w.fmt, w.H)
    payload = np.zeros((w.P, w.T, row), np.uint8)
    out = oracle.dispatch(R.counts, payload, R.ids, R.weights, None, E=w.E, want_payload=False)
    valid = out["valid"].astype(bool)
    M = int(valid.sum())
    N = int(R.counts.sum())
    assert bench.pair_count(w, R) == M
    slots = w.P * w.P * w.T
    k = w.k
    disp = (N * (row + srow) + N * k * 4 * 2          # token rows, ids and weights read
            + M * (row + srow) + M * k * 4 * 2        # rows, ids and weights of valid slots
            + (slots - M) * k * 4)                    # marker ids of empty slots
    b = bench.step_bytes(w, N, M)
    assert b["dispatch"] == disp
    if w.combine == "fp8":
        land = w.H + w.H // 32                        # e4m3 codes + e8m0 scales per row
        assert b["combine_quant"] == M * 2 * w.H + M * land
        assert b["combine_gather"] == M * land + N * 2 * w.H
    else:
        assert b["combine"] == M * 2 * w.H + N * 2 * w.H
