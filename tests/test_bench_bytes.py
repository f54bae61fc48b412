"""The bench's algorithmic byte counts against a count taken from the
oracle's own dispatch result: M is the number of valid receive slots the
oracle produces, and each byte term is rebuilt from what the exchange must
read and write (token rows with their extra bytes read once, one row per
valid slot written, k ids + k weights per token read, k ids + k weights per
valid slot written, k marker ids per empty slot of a rank that takes part;
each taking-part rank's EPLB statistics read once and written to every
taking-part region; combine reads one row per valid slot and writes one per
token).  Ranks outside the active mask neither send nor receive."""
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
    dataclasses.replace(W.EP64_DSFP8, name="deepseek_fp8 P64", T=6, H=128, n_lo=0, n_hi=6),
    dataclasses.replace(W.EP64_NVFP4_EXTRAS, name="nvfp4 extras P64", T=6, H=64, n_lo=0, n_hi=6,
                        extra_bytes=40, n_eplb=16),
    dataclasses.replace(W.EP64_MASK48, name="alive48 P64", T=6, H=64, n_lo=0, n_hi=6),
    dataclasses.replace(W.EP8_BF16, name="ep8 mask extras", T=20, H=256, n_lo=0, n_hi=20, extra_bytes=24,
                        n_eplb=8, alive=(0, 2, 3, 5, 6)),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_step_bytes_match_the_oracle_count(w):
    R = W.draw_routing(w)
    row = W.payload_row_bytes(w.fmt, w.H)
    srow = W.scale_row_bytes(w.fmt, w.H)
    xrow = w.extra_bytes
    payload = np.zeros((w.P, w.T, row), np.uint8)
    extra = np.zeros((w.P, w.T, xrow), np.uint8) if xrow else None
    live = [r for r in range(w.P) if w.alive is None or r in w.alive]
    active = None if w.alive is None else sum(1 << r for r in live)
    out = oracle.dispatch(R.counts, payload, R.ids, R.weights, None, E=w.E, want_payload=False,
                          active=active, extra=extra)
    valid = out["valid"].astype(bool)
    M = int(valid.sum())
    N = int(sum(R.counts[s] for s in live))
    assert bench.pair_count(w, R) == M
    assert bench.live_tokens(w, R) == N
    dead = [r for r in range(w.P) if r not in live]
    assert not valid[dead].any()                      # masked-off regions receive nothing
    L = len(live)
    slots = L * w.P * w.T                             # slots of the regions that take part
    k = w.k
    disp = (N * (row + xrow + srow) + N * k * 4 * 2   # token rows (+ extra bytes), ids and weights read
            + M * (row + xrow + srow) + M * k * 4 * 2  # rows, ids and weights of valid slots
            + (slots - M) * k * 4                     # marker ids of empty slots
            + L * w.n_eplb * 4                        # each live rank's statistics read
            + L * L * w.n_eplb * 4)                   # ... and written into every live region
    b = bench.step_bytes(w, N, M)
    assert b["dispatch"] == disp
    if w.combine == "fp8":
        land = w.H + w.H // 32                        # e4m3 codes + e8m0 scales per row
        assert b["combine_quant"] == M * 2 * w.H + M * land
        assert b["combine_gather"] == M * land + N * 2 * w.H
    else:
        assert b["combine"] == M * 2 * w.H + N * 2 * w.H
