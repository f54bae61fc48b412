"""Oracle pins that do not retype its definitions: hand-worked golden
cases, closed forms and invariants.

- golden: tests/golden/*.json, worked on paper from the pages' rules;
- every (token, owning rank) pair appears exactly once (pair count from
  numpy's unique, not from the oracle's routing);
- identity expert: each rank returns the token row times the sum of its
  local experts' weights, so the combine returns the row times the sum of
  all top-k weights (closed form, needs no routing at all);
- P = 1 / k = 1 special cases (copy is the identity, combine has one term);
- FP8 combine stays within the e4m3 rounding bound of the exact sum and
  is exact on values the format holds;
- all-gatherv / reduce-scatterv reduce to numpy concatenate and an exact
  (math.fsum) sum;
- generator sanity: mean fan-out matches P*(1-C(E-E/P,k)/C(E,k)).
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bits_to_f(b):
    return torch.from_numpy(np.asarray(b, np.uint16).view(np.int16)).view(torch.bfloat16).double().numpy()


# ---------------------------------------------------------------- golden

def test_golden_dispatch(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "dispatch_combine_p2.json")))
    ids = np.array(g["ids"], np.int32)
    payload = np.array(g["payload"], np.uint8)
    weights = np.array(g["weights"], np.float32)
    out = oracle.dispatch(g["counts"], payload, ids, weights, E=g["E"])
    ex = g["expect"]
    assert out["valid"].tolist() == ex["valid"]
    assert out["ids"].tolist() == ex["recv_ids"]
    assert out["counts"].tolist() == ex["recv_counts"]
    for r, sl in enumerate(ex["recv_slots"]):
        assert out["slots"][r, :len(sl)].tolist() == sl
    for r, m in ex["recv_weights_valid"].items():
        for q, w in m.items():
            assert out["weights"][int(r), int(q)].tolist() == w
    for r, m in ex["recv_payload_valid"].items():
        for q, p in m.items():
            assert out["payload"][int(r), int(q)].tolist() == p


def test_golden_combine(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "dispatch_combine_p2.json")))
    P, T, H = g["P"], g["T"], g["combine"]["H"]
    eo = np.full((P, P * T, H), np.nan, np.float32)
    for r in range(P):
        for q, row in enumerate(g["combine"]["eo"][r]):
            if row is not None:
                eo[r, q] = row
    ref, y, exact = oracle.combine_bf16(g["counts"], np.array(g["ids"], np.int32), _bf16_bits(eo), E=g["E"])
    for s, rows in enumerate(g["combine"]["expect_y"]):
        for t, want in enumerate(rows):
            assert ref[s, t].tolist() == want
            assert exact[s, t].tolist() == want
            assert _bits_to_f(y[s, t]).tolist() == want
    # +0 for a token sent nowhere (rank 1 token 1)
    assert y[1, 1].tolist() == [0, 0]


def test_golden_agrs(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "agrs_p2.json")))
    sizes = np.array(g["sizes"], np.int32)
    rows = np.zeros((2, 2, 2), np.uint8)
    for q, rr in enumerate(g["rows"]):
        rows[q, :len(rr)] = rr
    assert oracle.allgatherv(sizes, rows).tolist() == g["expect_gather"]
    part = _bf16_bits(np.array(g["partial"], np.float32))
    for r in range(2):
        ref, out, exact = oracle.reduce_scatterv(sizes, part, r)
        assert ref.tolist() == g["expect_scatter"][r]
        assert exact.tolist() == g["expect_scatter"][r]
        assert _bits_to_f(out).tolist() == g["expect_scatter"][r]


def test_golden_fp32_order(golden_dir):
    """fp32 sums in ascending rank order from +0, rounded once to bf16
    (tests/golden/combine_fp32_order.json, worked by hand)."""
    g = json.load(open(os.path.join(golden_dir, "combine_fp32_order.json")))
    P, T, H = g["P"], g["T"], g["H"]
    eo = np.full((P, P * T, H), np.nan, np.float32)
    for r in range(P):
        for q, row in enumerate(g["eo"][r]):
            if row is not None:
                eo[r, q] = row
    eb = _bf16_bits(eo)
    assert np.array_equal(_bits_to_f(eb)[~np.isnan(eo)], eo[~np.isnan(eo)])  # every term is a bf16 value
    ref, y, exact = oracle.combine_bf16(g["counts"], np.array(g["ids"], np.int32), eb, E=g["E"])
    for s in range(P):
        if g["expect_ref"][s] is None:
            assert not y[s].any()
            continue
        assert ref[s].tolist() == g["expect_ref"][s]
        assert y[s].tolist() == g["expect_y_bits"][s]
        assert _bits_to_f(y[s]).tolist() == g["expect_y"][s]
        assert exact[s].tolist() == g["expect_exact"][s]
    assert not np.signbit(ref[0, 0, 2])  # +0, not -0
    rs = g["reduce_scatterv"]
    part = _bf16_bits(np.array(rs["partial"], np.float32))
    for r in range(P):
        ref, out, exact = oracle.reduce_scatterv(np.array(rs["sizes"], np.int32), part, r)
        assert ref.tolist() == rs["expect_ref"][r]
        assert out.tolist() == rs["expect_out_bits"][r]
        assert exact.tolist() == rs["expect_exact"][r]
    f8 = g["fp8"]
    H8 = f8["H"]
    eo8 = np.zeros((P, P * T, H8), np.float32)
    for col, terms in f8["terms"].items():
        for r, v in enumerate(terms):
            eo8[r, 0, int(col)] = v
    eb8 = _bf16_bits(eo8)
    codes, scales, ref, y, exact = oracle.combine_fp8(g["counts"], np.array(g["ids"], np.int32), eb8, E=g["E"],
                                                      s0=0, s1=1)
    for r in range(P):
        land = r * T + 0  # rank r's row of source 0's token 0
        assert scales[0, land].tolist() == f8["expect_scale_codes"][r]
        assert [int(codes[0, land, 0]), int(codes[0, land, 32])] == f8["expect_codes_0_32"][r]
        assert np.count_nonzero(codes[0, land]) == 2
    for col in f8["terms"]:
        h = int(col)
        assert float(ref[0, 0, h]) == f8["expect_ref"][col]
        assert float(exact[0, 0, h]) == f8["expect_exact"][col]
        assert int(y[0, 0, h]) == f8["expect_y_bits"][col]
    others = [h for h in range(H8) if str(h) not in f8["terms"]]
    assert not ref[0, 0, others].any() and not y[0, 0, others].any()


# ---------------------------------------------------------------- dispatch invariants

SMALL = [dataclasses.replace(W.TINY),
         dataclasses.replace(W.EP8_BF16, T=32, n_lo=5, n_hi=32, H=64),
         dataclasses.replace(W.EP8_MXFP8, T=24, n_lo=24, n_hi=24, H=64),
         dataclasses.replace(W.EP64_BF16, P=16, E=64, T=8, n_lo=0, n_hi=8, H=32)]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_every_pair_exactly_once(w):
    d = W.draw_dispatch_inputs(w)
    R = d.routing
    pl = d.payload.numpy()
    sc = None if d.scales is None else d.scales.numpy()
    out = oracle.dispatch(R.counts, pl, R.ids, R.weights, sc, E=w.E)
    P, T = w.P, w.T
    epr = w.E // P
    # pairs from numpy set semantics
    pairs = set()
    for s in range(P):
        for t in range(int(R.counts[s])):
            for r in np.unique(R.ids[s, t] // epr):
                pairs.add((s, t, int(r)))
    got = set()
    for r in range(P):
        for q in np.nonzero(out["valid"][r])[0]:
            got.add((int(q) // T, int(q) % T, r))
    assert got == pairs
    assert out["counts"].sum() == len(pairs)
    # per-source fan-out equals the row sums of counts^T
    for s in range(P):
        assert out["counts"][:, s].sum() == sum(1 for p in pairs if p[0] == s)
    # each valid slot holds its source row, ids and weights; others hold markers
    for r in range(P):
        v = out["valid"][r].astype(bool)
        src = np.arange(P * T)
        assert np.array_equal(out["payload"][r][v], pl.reshape(P * T, -1)[src[v]])
        assert np.array_equal(out["ids"][r][v], R.ids.reshape(P * T, -1)[src[v]])
        assert np.array_equal(out["weights"][r][v], R.weights.reshape(P * T, -1)[src[v]])
        if sc is not None:
            assert np.array_equal(out["scales"][r][v], sc.reshape(P * T, -1)[src[v]])
        assert np.all(out["ids"][r][~v] == w.E)
        # slots list ascending and equal to the valid set
        n = int(out["counts"][r].sum())
        assert np.array_equal(out["slots"][r, :n], np.nonzero(v)[0])


def test_p1_dispatch_is_identity():
    rng = np.random.default_rng(4)
    T, k, E, H = 9, 3, 4, 16
    ids = rng.integers(0, E, (1, T, k)).astype(np.int32)
    pl = rng.integers(0, 256, (1, T, 2 * H)).astype(np.uint8)
    out = oracle.dispatch([7], pl, ids, None, E=E)
    assert out["valid"][0].tolist() == [1] * 7 + [0] * 2
    assert np.array_equal(out["payload"][0, :7], pl[0, :7])
    assert out["slots"][0, :7].tolist() == list(range(7))


# ---------------------------------------------------------------- combine invariants

@pytest.mark.parametrize("w", SMALL[:2] + SMALL[3:], ids=lambda w: w.name)
def test_identity_expert_combine(w):
    """Each rank r returns bf16(x * sum of weights of r's experts); the
    combine must return x * sum of all k weights (within two bf16
    roundings: 2 * 2^-8 relative to sum |terms|)."""
    d = W.draw_dispatch_inputs(w)
    R = d.routing
    P, T, H = w.P, w.T, w.H
    x = d.hidden_bf16.double().numpy()
    epr = w.E // P
    eo = np.full((P, P * T, H), np.nan, np.float32)  # unsent slots poisoned
    for s in range(P):
        for t in range(int(R.counts[s])):
            owners = R.ids[s, t] // epr
            for r in np.unique(owners):
                wsum = float(R.weights[s, t][owners == r].sum(dtype=np.float64))
                eo[r, s * T + t] = (x[s, t] * wsum).astype(np.float32)
    y = oracle.combine_bf16(R.counts, R.ids, _bf16_bits(eo), E=w.E).y
    yv = _bits_to_f(y)
    for s in range(P):
        n = int(R.counts[s])
        want = x[s, :n] * R.weights[s, :n].sum(axis=1, dtype=np.float64)[:, None]
        mag = np.abs(x[s, :n]) * R.weights[s, :n].sum(axis=1, dtype=np.float64)[:, None]
        assert np.all(np.isfinite(yv[s, :n]))
        assert np.all(np.abs(yv[s, :n] - want) <= 2 * 2.0 ** -8 * mag + 1e-30)


def test_k1_and_p1_combine_single_term_is_exact():
    rng = np.random.default_rng(8)
    P, T, E, H = 4, 6, 8, 32
    ids = rng.integers(0, E, (P, T, 1)).astype(np.int32)
    eo = _bf16_bits(rng.standard_normal((P, P * T, H)))
    counts = np.array([6, 3, 0, 5], np.int32)
    y = oracle.combine_bf16(counts, ids, eo, E=E).y
    for s in range(P):
        for t in range(int(counts[s])):
            r = ids[s, t, 0] // (E // P)
            assert np.array_equal(y[s, t], eo[r, s * T + t])
    ids1 = rng.integers(0, E, (1, T, 3)).astype(np.int32)
    eo1 = _bf16_bits(rng.standard_normal((1, T, H)))
    y1 = oracle.combine_bf16([T], ids1, eo1, E=E).y
    assert np.array_equal(y1[0], eo1[0])


def test_fp8_combine_error_bound_and_exact_values():
    rng = np.random.default_rng(21)
    P, T, k, E, H = 4, 6, 4, 16, 64
    ids = np.stack([np.stack([rng.permutation(E)[:k] for _ in range(T)]) for _ in range(P)]).astype(np.int32)
    counts = np.array([6, 6, 2, 5], np.int32)
    eo_f = rng.standard_normal((P, P * T, H)) * 2.0 ** rng.integers(-6, 6, (P, P * T, 1))
    eo = _bf16_bits(eo_f)
    land_c, land_s, _, _, ref_q = oracle.combine_fp8(counts, ids, eo, E=E)
    ref = oracle.combine_bf16(counts, ids, eo, E=E).exact
    ev = _bits_to_f(eo)
    epr = E // P
    for s in range(P):
        for t in range(int(counts[s])):
            dests = np.unique(ids[s, t] // epr)
            bound = np.zeros(H)
            for r in dests:
                row = ev[r, s * T + t]
                e = np.array([oracle.fp8_block_exponent(float(np.abs(row[b * 32:(b + 1) * 32]).max()))
                              for b in range(H // 32)])
                # half an e4m3 ulp: 2^-4 relative for normals, 2^(e-10) floor
                bound += np.abs(row) * 2.0 ** -4 + np.repeat(2.0 ** (e - 10), 32)
                # the landing row is r's quantised row
                codes, sc = oracle.fp8_quantize_row(eo[r, s * T + t])
                assert np.array_equal(land_c[s, r * T + t], codes)
                assert np.array_equal(land_s[s, r * T + t], sc)
            assert np.all(np.abs(ref_q[s, t] - ref[s, t]) <= bound)
    # values e4m3 holds exactly (small integers times a common power of two)
    ints = rng.integers(-15, 16, (P, P * T, H)).astype(np.float32) / 8.0
    ints[..., 0] = 15.0 / 8.0  # fix the block maximum so the scale keeps 4 bits
    ints[..., 32] = 15.0 / 8.0
    eo2 = _bf16_bits(ints)
    ref_q2 = oracle.combine_fp8(counts, ids, eo2, E=E).exact
    ref2 = oracle.combine_bf16(counts, ids, eo2, E=E).exact
    assert np.array_equal(ref_q2, ref2)


# ---------------------------------------------------------------- AgRs

def test_allgatherv_is_concatenation():
    rng = np.random.default_rng(31)
    P, rb = 5, 24
    sizes = np.array([3, 0, 7, 1, 4], np.int32)
    rows = rng.integers(0, 256, (P, 8, rb)).astype(np.uint8)
    want = np.concatenate([rows[q, :sizes[q]] for q in range(P)])
    assert np.array_equal(oracle.allgatherv(sizes, rows), want)


def test_reduce_scatterv_matches_exact_sum():
    rng = np.random.default_rng(32)
    P, H = 6, 16
    sizes = np.array([2, 5, 0, 1, 3, 4], np.int32)
    total = int(sizes.sum())
    part = _bf16_bits(rng.standard_normal((P, total, H)) * 2.0 ** rng.integers(-10, 10, (P, total, 1)))
    pv = _bits_to_f(part)
    off = np.concatenate([[0], np.cumsum(sizes)])
    for r in range(P):
        ref, out, exact = oracle.reduce_scatterv(sizes, part, r)
        assert ref.shape == (sizes[r], H)
        u = 2.0 ** -24
        for i in range(sizes[r]):
            for h in range(H):
                fs = math.fsum(pv[:, off[r] + i, h])
                mag = np.abs(pv[:, off[r] + i, h]).sum()
                assert exact[i, h] == fs  # a handful of bf16 terms: the double sum is exact
                # the fp32 sum: within the recursive summation bound of P terms
                assert abs(float(ref[i, h]) - fs) <= (P - 1) * u / (1 - (P - 1) * u) * mag
    # P = 1: identity
    one = _bf16_bits(rng.standard_normal((1, 7, H)))
    o1 = oracle.reduce_scatterv(np.array([7], np.int32), one, 0).out
    assert np.array_equal(o1, one[0])


# ---------------------------------------------------------------- generator sanity

@pytest.mark.parametrize("P,E,k,want", [(4, 16, 2, 1.8), (8, 256, 8, 5.2947), (64, 256, 8, 7.6758)])
def test_uniform_fanout_closed_form(P, E, k, want):
    closed = P * (1.0 - math.comb(E - E // P, k) / math.comb(E, k))
    assert closed == pytest.approx(want, abs=1e-4)
    rng = np.random.default_rng(41)
    ids = W.draw_topk_ids(rng, 20000, E, k)
    assert all(len(set(r)) == k for r in ids[:200])
    fan = np.mean([len(np.unique(r // (E // P))) for r in ids])
    assert fan == pytest.approx(closed, rel=0.02)


def test_weights_are_softmax():
    rng = np.random.default_rng(42)
    w = W.draw_topk_weights(rng, 1000, 8)
    assert np.all(w > 0)
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)


def test_owner_contiguous_blocks_and_out_of_range():
    # contiguous blocks of E/P experts; ids outside [0, E) have no owner
    assert [oracle.owner(e, 16, 4) for e in range(16)] == [e // 4 for e in range(16)]
    for bad in (-1, -100, 16, 17, 1 << 30):
        assert oracle.owner(bad, 16, 4) == -1
