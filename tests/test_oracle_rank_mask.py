"""Oracle pins of the active rank mask (FlashInfer moe_a2a_dispatch,
active_rank_mask: a token bound for a rank whose bit is clear never reaches it): the
push-style brute force with an alive set, and invariants -- an all-ones
mask changes nothing, dead destinations are left untouched, dead sources
send nothing, combine sums live ranks only."""
import numpy as np
import pytest

import oracle
from tests import bruteforce as bf
from tests.test_oracle_bruteforce import _bf16_bits, _case


def _mask(alive):
    m = 0
    for r in alive:
        m |= 1 << r
    return m


@pytest.mark.parametrize("P,T,k,E,alive", [
    (4, 6, 3, 8, [0, 2, 3]), (4, 5, 2, 16, [1]), (3, 4, 4, 12, [0, 1, 2]),
    (6, 3, 2, 12, [5, 0, 3]), (2, 7, 1, 4, []),
])
def test_masked_dispatch_matches_bruteforce(P, T, k, E, alive):
    rng = np.random.default_rng(100 + P + len(alive))
    counts, payload, ids, weights, scales = _case(rng, P, T, k, E)
    got = oracle.dispatch(counts, payload, ids, weights, scales, E=E, active=_mask(alive))
    recv = bf.dispatch(counts, payload, ids, weights, scales, E, alive=alive)
    for r in range(P):
        if r not in alive:
            # untouched: the wrapper's zero-filled outputs stay zero
            assert not got["ids"][r].any() and not got["valid"][r].any() and not got["counts"][r].any()
            continue
        want = bf.recv_ids_plane(recv, P, T, k, E)[r]
        assert np.array_equal(got["ids"][r], want)
        cnt, slots = bf.counts_and_slots(recv, P, T)
        assert np.array_equal(got["counts"][r], cnt[r])
        assert list(got["slots"][r, :len(slots[r])]) == slots[r]
        for q, (pl, _, _, w) in recv[r].items():
            assert bytes(got["payload"][r, q]) == pl


def test_all_ones_mask_is_no_mask():
    rng = np.random.default_rng(7)
    P, T, k, E = 4, 8, 3, 16
    counts, payload, ids, weights, scales = _case(rng, P, T, k, E)
    a = oracle.dispatch(counts, payload, ids, weights, scales, E=E)
    b = oracle.dispatch(counts, payload, ids, weights, scales, E=E, active=(1 << P) - 1)
    for key in ("ids", "valid", "counts", "slots", "payload", "weights"):
        assert np.array_equal(a[key], b[key])


@pytest.mark.parametrize("alive", [[0, 1, 3], [2], [0, 1, 2, 3]])
def test_masked_combine_sums_live_ranks(alive):
    rng = np.random.default_rng(8 + len(alive))
    P, T, k, E, H = 4, 6, 3, 8, 8
    counts, _, ids, _, _ = _case(rng, P, T, k, E, H=H)
    eo = _bf16_bits(rng.standard_normal((P, P * T, H)))
    got = oracle.combine_bf16(counts, ids, eo, E=E, active=_mask(alive))
    want = bf.combine_bf16(counts, ids, eo, E, alive=alive)
    want32 = bf.combine_bf16_fp32(counts, ids, eo, E, alive=alive)
    for s in range(P):
        for t in range(T):
            if (s, t) in want:
                assert list(got.exact[s, t]) == want[(s, t)]
                assert np.array_equal(got.ref[s, t].view(np.uint32), want32[(s, t)].view(np.uint32))
            else:
                assert not got.ref[s, t].any() and not got.y[s, t].any()
    # fp8 path: masked ranks contribute nothing either
    rq = oracle.combine_fp8(counts, ids, eo, E=E, active=_mask(alive)).exact
    for s in range(P):
        if s not in alive:
            assert not rq[s].any()
