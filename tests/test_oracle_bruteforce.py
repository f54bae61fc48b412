"""Oracle vs a push-style pure-Python brute force on tiny random inputs,
including duplicate ids, out-of-range / negative ids, ragged counts,
P = 1 and k = 1.  Dispatch must agree exactly; combine sums must agree
bit for bit: the fp32 sums with numpy float32 additions in the same
(ascending rank) order, the exact sums with Python float sums, and the
bf16 result with torch's round-to-nearest-even cast of the fp32 sum."""
import numpy as np
import pytest
import torch

import oracle
from tests import bruteforce as bf


def _case(rng, P, T, k, E, H=8, srow=0, with_w=True, dup=True, oob=True):
    counts = rng.integers(0, T + 1, size=P).astype(np.int32)
    ids = rng.integers(0, E, size=(P, T, k)).astype(np.int32)
    if dup and k > 1:
        m = rng.random((P, T)) < 0.3
        ids[m, 1] = ids[m, 0]
    if oob:
        m = rng.random((P, T, k)) < 0.1
        ids[m] = rng.choice([-1, -7, E, E + 3], size=int(m.sum()))
    payload = rng.integers(0, 256, size=(P, T, 2 * H)).astype(np.uint8)
    scales = rng.integers(0, 256, size=(P, T, srow)).astype(np.uint8) if srow else None
    weights = rng.standard_normal((P, T, k)).astype(np.float32) if with_w else None
    return counts, payload, ids, weights, scales


def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


SHAPES = [(1, 5, 3, 4), (2, 3, 2, 4), (3, 4, 1, 3), (4, 6, 3, 8), (4, 8, 4, 16), (3, 7, 2, 12)]


@pytest.mark.parametrize("P,T,k,E", SHAPES)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_dispatch_matches_bruteforce(P, T, k, E, seed):
    rng = np.random.default_rng(1000 * seed + 17 * P + T)
    srow = 4 if seed == 1 else 0
    counts, payload, ids, weights, scales = _case(rng, P, T, k, E, srow=srow, with_w=(seed != 2))
    got = oracle.dispatch(counts, payload, ids, weights, scales, E=E)
    recv = bf.dispatch(counts, payload, ids, weights, scales, E)
    assert np.array_equal(got["ids"], bf.recv_ids_plane(recv, P, T, k, E))
    cnt, slots = bf.counts_and_slots(recv, P, T)
    assert np.array_equal(got["counts"], cnt)
    for r in range(P):
        n = len(slots[r])
        assert list(got["slots"][r, :n]) == slots[r]
        assert np.all(got["slots"][r, n:] == -1)
        assert set(np.nonzero(got["valid"][r])[0]) == set(recv[r])
        for q, (pl, sc, idr, w) in recv[r].items():
            assert bytes(got["payload"][r, q]) == pl
            if sc is not None:
                assert bytes(got["scales"][r, q]) == sc
            if w is not None:
                assert list(got["weights"][r, q]) == pytest.approx(w, abs=0, rel=0)


@pytest.mark.parametrize("P,T,k,E", SHAPES)
def test_dispatch_custom_invalid_id(P, T, k, E):
    rng = np.random.default_rng(5 + P)
    counts, payload, ids, weights, scales = _case(rng, P, T, k, E)
    got = oracle.dispatch(counts, payload, ids, weights, scales, E=E, invalid_id=-1)
    recv = bf.dispatch(counts, payload, ids, weights, scales, E)
    assert np.array_equal(got["ids"], bf.recv_ids_plane(recv, P, T, k, -1))


def test_dispatch_destination_subset_matches_full():
    rng = np.random.default_rng(9)
    P, T, k, E = 4, 6, 3, 8
    counts, payload, ids, weights, scales = _case(rng, P, T, k, E)
    full = oracle.dispatch(counts, payload, ids, weights, scales, E=E)
    part = oracle.dispatch(counts, payload, ids, weights, scales, E=E, r0=1, r1=3)
    for key in ("ids", "valid", "counts", "slots", "payload"):
        assert np.array_equal(full[key][1:3], part[key])


def _torch_bf16_bits(f32):
    return torch.from_numpy(np.asarray(f32, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("P,T,k,E", SHAPES)
def test_combine_bf16_matches_bruteforce(P, T, k, E):
    rng = np.random.default_rng(77 + P * T)
    H = 8
    counts, payload, ids, weights, scales = _case(rng, P, T, k, E, H=H)
    # magnitudes spread over 2^-20 .. 2^20 so fp32 rounding shows in the sums
    eo = _bf16_bits(rng.standard_normal((P, P * T, H)) * 2.0 ** rng.integers(-20, 21, (P, P * T, 1)))
    got = oracle.combine_bf16(counts, ids, eo, E=E)
    want = bf.combine_bf16(counts, ids, eo, E)
    want32 = bf.combine_bf16_fp32(counts, ids, eo, E)
    for s in range(P):
        for t in range(T):
            if t < counts[s]:
                assert list(got.exact[s, t]) == want[(s, t)]
                assert np.array_equal(got.ref[s, t].view(np.uint32), want32[(s, t)].view(np.uint32))
                assert np.array_equal(got.y[s, t], _torch_bf16_bits(want32[(s, t)]))
            else:
                assert np.all(got.ref[s, t] == 0) and np.all(got.exact[s, t] == 0) and np.all(got.y[s, t] == 0)


def test_combine_fp32_sum_within_recursive_summation_bound():
    """|fl32(sum) - sum| <= gamma_(m-1) * sum|terms| for m terms added one
    by one (gamma_n = n u / (1 - n u), u = 2^-24): the fp32 reference is a
    sum of exactly the token's terms, each rounded once per addition."""
    rng = np.random.default_rng(78)
    P, T, k, E, H = 8, 6, 8, 32, 64
    counts, _, ids, _, _ = _case(rng, P, T, k, E, H=H, oob=False)
    eo = _bf16_bits(rng.standard_normal((P, P * T, H)) * 2.0 ** rng.integers(-24, 25, (P, P * T, 1)))
    got = oracle.combine_bf16(counts, ids, eo, E=E)
    ev = torch.from_numpy(eo.view(np.int16)).view(torch.bfloat16).double().numpy()
    u = 2.0 ** -24
    for s in range(P):
        for t in range(int(counts[s])):
            dests = sorted({int(e) // (E // P) for e in ids[s, t]})
            m = len(dests)
            mag = np.abs(ev[dests, s * T + t]).sum(axis=0)
            gamma = (m - 1) * u / (1 - (m - 1) * u)
            assert np.all(np.abs(got.ref[s, t].astype(np.float64) - got.exact[s, t]) <= gamma * mag)


def test_combine_token_agrees_with_array_form():
    rng = np.random.default_rng(3)
    P, T, k, E, H = 4, 5, 3, 8, 16
    counts, _, ids, _, _ = _case(rng, P, T, k, E, H=H)
    eo = _bf16_bits(rng.standard_normal((P, P * T, H)))
    full = oracle.combine_bf16(counts, ids, eo, E=E)
    for s in range(P):
        for t in range(int(counts[s])):
            one = oracle.combine_token_bf16(ids[s, t], eo[:, s * T + t], E=E)
            for a, b in zip(one, full):
                assert np.array_equal(a, b[s, t])
    part = oracle.combine_bf16(counts, ids, eo, E=E, s0=2, s1=4)
    for a, b in zip(part, full):
        assert np.array_equal(a, b[2:4])
    # the sources' slots alone ([P, 2T, H] slice holding slots 2T .. 4T-1)
    sl = oracle.combine_bf16(counts, ids, eo[:, 2 * T:4 * T], E=E, s0=2, s1=4, slot0=2 * T)
    for a, b in zip(sl, full):
        assert np.array_equal(a, b[2:4])
    f8 = oracle.combine_fp8(counts, ids, eo, E=E, s0=1, s1=3)
    f8s = oracle.combine_fp8(counts, ids, eo[:, T:3 * T], E=E, s0=1, s1=3, slot0=T)
    for a, b in zip(f8, f8s):
        assert np.array_equal(a, b)
    with pytest.raises(AssertionError):
        oracle.combine_bf16(counts, ids, eo[:, 2 * T:4 * T], E=E, s0=1, s1=4, slot0=2 * T)


def test_fp8_combine_matches_bruteforce():
    """The fp32 sum of the dequantised landing rows (torch's e4m3 decode
    times 2^(scale - 127)), added in ascending rank order with numpy
    float32, bit for bit; exact sums with Python floats."""
    rng = np.random.default_rng(79)
    P, T, k, E, H = 4, 5, 3, 8, 64
    counts, _, ids, _, _ = _case(rng, P, T, k, E, H=H)
    eo = _bf16_bits(rng.standard_normal((P, P * T, H)) * 2.0 ** rng.integers(-30, 31, (P, P * T, 1)))
    got = oracle.combine_fp8(counts, ids, eo, E=E)
    epr = E // P
    for s in range(P):
        for t in range(int(counts[s])):
            dests = sorted({int(e) // epr for e in ids[s, t] if 0 <= int(e) < E})
            acc = np.zeros(H, np.float32)
            ex = [0.0] * H
            for r in dests:
                v = bf.fp8_dequantise(got.land_codes[s, r * T + t], got.land_scales[s, r * T + t])
                acc = (acc + v.astype(np.float32)).astype(np.float32)
                ex = [a + float(b) for a, b in zip(ex, v)]
            assert np.array_equal(got.ref[s, t].view(np.uint32), acc.view(np.uint32))
            assert list(got.exact[s, t]) == ex
            assert np.array_equal(got.y[s, t], _torch_bf16_bits(acc))


def test_reduce_scatterv_matches_bruteforce():
    rng = np.random.default_rng(80)
    P, H = 6, 24
    sizes = np.array([2, 0, 5, 1, 3, 4], np.int32)
    part = _bf16_bits(rng.standard_normal((P, int(sizes.sum()), H)) * 2.0 ** rng.integers(-20, 21, (P, int(sizes.sum()), 1)))
    for r in range(P):
        got = oracle.reduce_scatterv(sizes, part, r)
        want = bf.reduce_scatterv_fp32(sizes, part, r)
        assert np.array_equal(got.ref.view(np.uint32), want.view(np.uint32))
        assert np.array_equal(got.out, _torch_bf16_bits(want))


@pytest.mark.parametrize("P,T,k,E", SHAPES[:4])
def test_extra_payload_travels_with_token(P, T, k, E):
    rng = np.random.default_rng(55 + P)
    counts, payload, ids, weights, scales = _case(rng, P, T, k, E, srow=4)
    extra = rng.integers(0, 256, size=(P, T, 12)).astype(np.uint8)
    got = oracle.dispatch(counts, payload, ids, weights, scales, E=E, extra=extra)
    # the extra plane is one more per-token row: brute force it as the payload
    recv = bf.dispatch(counts, extra, ids, weights, scales, E)
    for r in range(P):
        assert set(np.nonzero(got["valid"][r])[0]) == set(recv[r])
        for q, (xb, _, _, _) in recv[r].items():
            assert bytes(got["extra"][r, q]) == xb


def test_eplb_allgather_is_the_stacked_rows():
    rng = np.random.default_rng(66)
    P, n = 5, 7
    stats = rng.integers(-1000, 1000, size=(P, n)).astype(np.int32)
    for r in range(P):
        assert np.array_equal(oracle.eplb_allgather(stats, r), stats)  # row s = rank s's stats
    alive = [0, 2, 3]
    act = sum(1 << a for a in alive)
    poison = np.full((P, n), -7, np.int32)
    for r in range(P):
        got = oracle.eplb_allgather(stats, r, active=act, out=poison.copy())
        if r not in alive:
            assert np.all(got == -7)
        else:
            for s in range(P):
                assert np.array_equal(got[s], stats[s] if s in alive else poison[s])
