"""GPU combine parity against the CPU oracle.

BF16 combine: |y - ref| <= 2^-7 |ref| + 1e-3 element by element, ref being
the oracle's exact (double) sum of the bf16 terms.  FP8 combine: the
landing planes (e4m3 codes + e8m0 scales) are bit-exact with the
oracle's quantisation, y is within bf16 rounding of the oracle's sum of
the dequantised terms (|y - ref_q| <= 2^-8 |ref_q| + 2^-126), and within
0.07 * sum|terms| (+ half an e4m3 subnormal step per term) of the exact
sum.  Expert-output slots that received no token are NaN-poisoned: they
must never reach the result."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import bf16_bits_to_f64, bits16, gpu_inputs, log, random_byte_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from combine_route_mask_amd import moe_ep
    assert torch.cuda.is_available() and moe_ep.moe_ep_is_supported()
    yield
    torch.cuda.empty_cache()


def _exchange(w, combine=None, T_cap=None):
    from combine_route_mask_amd.moe_ep import MoeEpExchange
    return MoeEpExchange(w.P, w.E, w.k, T_cap or w.T, w.H, dispatch_format=w.fmt,
                         combine_format=combine or w.combine)


def _dispatch(w, seed, combine=None, counts=None):
    c = random_byte_case(w, seed, counts=counts)
    ex = _exchange(w, combine)
    pl, sc, ids, wt = gpu_inputs(c)
    ex.dispatch(pl, ids, wt, scales=sc, num_tokens=c.counts.tolist(), runtime_max_tokens_per_rank=w.T)
    valid = oracle.dispatch(c.counts, c.payload, c.ids, None, c.scales, E=w.E,
                            want_payload=False)["valid"].astype(bool)
    return c, ex, valid


def _poison(eo, valid):
    """NaN in every expert-output slot that received no token."""
    m = torch.from_numpy(~valid).to(eo.device)
    eo[m] = float("nan")
    return eo


def _check_bf16(y_bits, ref):
    y = bf16_bits_to_f64(y_bits)
    assert np.all(np.isfinite(ref))
    err = np.abs(y - ref)
    bad = ~(err <= 2.0 ** -7 * np.abs(ref) + 1e-3)
    assert not bad.any(), f"{bad.sum()} elements outside tolerance, worst err {err.max()}"


SMALL = [
    W.TINY,
    dataclasses.replace(W.TINY, name="ragged P5 T37 H136", P=5, E=20, k=3, T=37, H=136, n_lo=0, n_hi=37),
    dataclasses.replace(W.TINY, name="P64 E64", P=64, E=64, k=8, T=5, H=64, n_lo=0, n_hi=5),
    dataclasses.replace(W.TINY, name="long rows H8200", P=3, E=12, k=4, T=6, H=8200, n_lo=1, n_hi=6),
    dataclasses.replace(W.TINY, name="k1", k=1, T=70, H=512, n_lo=1, n_hi=70),
    dataclasses.replace(W.EP8_BF16, name="ep8 mid", T=40, H=1024, n_lo=0, n_hi=40),
    dataclasses.replace(W.TINY, name="k16", P=8, E=64, k=16, T=30, H=512, n_lo=0, n_hi=30),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_combine_bf16_small(w):
    log(f"combine bf16: {w.name}")
    c, ex, valid = _dispatch(w, 61)
    eo = _poison(W.draw_expert_output(w.P, w.T, w.H, 61, device="cuda"), valid)
    y = ex.combine(eo)
    ref, _ = oracle.combine_bf16(c.counts, c.ids, bits16(eo), E=w.E)
    yb = bits16(y)
    for s in range(w.P):
        n = int(c.counts[s])
        _check_bf16(yb[s, :n], ref[s, :n])
    if w.k == 1:  # one term per token: the output is that term, bit for bit
        _, yo = oracle.combine_bf16(c.counts, c.ids, bits16(eo), E=w.E)
        for s in range(w.P):
            assert np.array_equal(yb[s, :c.counts[s]], yo[s, :c.counts[s]])


def test_combine_bf16_rows_past_count_untouched():
    w = dataclasses.replace(W.TINY, name="untouched", T=20, H=128)
    c, ex, valid = _dispatch(w, 62, counts=[20, 3, 0, 11])
    eo = _poison(W.draw_expert_output(w.P, w.T, w.H, 62, device="cuda"), valid)
    out = torch.full((w.P, w.T, w.H), 7.0, dtype=torch.bfloat16, device="cuda")
    ex.combine(eo, out)
    o = out.float().cpu().numpy()
    for s in range(w.P):
        assert np.all(o[s, c.counts[s]:] == 7.0)


def test_combine_identity_expert():
    """Each rank returns its token row times the sum of its local experts'
    weights; combine must give the row times the sum of all k weights."""
    w = W.TINY
    d = W.draw_dispatch_inputs(w)
    R = d.routing
    ex = _exchange(w)
    ex.dispatch(d.payload.cuda(), torch.from_numpy(R.ids).cuda(), torch.from_numpy(R.weights).cuda(),
                num_tokens=R.counts.tolist())
    x = d.hidden_bf16.double().numpy()
    eo = np.full((w.P, w.P * w.T, w.H), np.nan, np.float32)
    for s in range(w.P):
        for t in range(int(R.counts[s])):
            owners = np.array([oracle.owner(e, w.E, w.P) for e in R.ids[s, t]])
            for r in np.unique(owners[owners >= 0]):
                eo[r, s * w.T + t] = x[s, t] * float(R.weights[s, t][owners == r].sum(dtype=np.float64))
    eo_t = torch.from_numpy(eo).to(torch.bfloat16).cuda()
    y = ex.combine(eo_t).double().cpu().numpy()
    for s in range(w.P):
        n = int(R.counts[s])
        tot = R.weights[s, :n].sum(1, dtype=np.float64)[:, None]
        want = x[s, :n] * tot
        assert np.all(np.abs(y[s, :n] - want) <= 2 * 2.0 ** -8 * np.abs(x[s, :n]) * tot + 1e-30)


def test_combine_bf16_special_values():
    w = dataclasses.replace(W.TINY, name="specials", T=8, H=64, n_lo=8, n_hi=8)
    c, ex, valid = _dispatch(w, 63)
    rng = np.random.default_rng(63)
    vals = np.array([0.0, -0.0, 3.0e37, -3.0e37, 1e-40, -1e-40, 9.2e-41, 65504.0,
                     1.0, -1.0, 2.0 ** -133, np.inf, -np.inf], np.float32)
    eo_np = rng.choice(vals, size=(w.P, w.P * w.T, w.H)).astype(np.float32)
    eo = _poison(torch.from_numpy(eo_np).to(torch.bfloat16).cuda(), valid)
    y = bits16(ex.combine(eo))
    ref, yo = oracle.combine_bf16(c.counts, c.ids, bits16(eo), E=w.E)
    yf, of = bf16_bits_to_f64(y), bf16_bits_to_f64(yo)
    for s in range(w.P):
        n = int(c.counts[s])
        a, b, r = yf[s, :n], of[s, :n], ref[s, :n]
        assert np.array_equal(np.isnan(a), np.isnan(b)), "NaN positions differ"
        fin = np.isfinite(r)
        assert np.array_equal(a[~fin & ~np.isnan(b)], b[~fin & ~np.isnan(b)])
        # finite sums: fp32 accumulation may overflow only where the double sum
        # is at the bf16 edge; both must agree on the class and be within tolerance
        f = fin & np.isfinite(a)
        assert np.all(np.abs(a[f] - r[f]) <= 2.0 ** -7 * np.abs(r[f]) + 1e-3)


def test_combine_full_ep8_bf16():
    w = W.EP8_BF16
    c, ex, valid = _dispatch(w, w.seed)
    eo = _poison(W.draw_expert_output(w.P, w.T, w.H, w.seed, device="cuda"), valid)
    y = bits16(ex.combine(eo))
    ref, _ = oracle.combine_bf16(c.counts, c.ids, bits16(eo), E=w.E)
    for s in range(w.P):
        _check_bf16(y[s, :c.counts[s]], ref[s, :c.counts[s]])


def test_combine_full_ep64_bf16_sampled():
    w = W.EP64_BF16
    c = random_byte_case(w, w.seed)
    ex = _exchange(w)
    pl, sc, ids, wt = gpu_inputs(c)
    ex.dispatch(pl, ids, wt, num_tokens=c.counts.tolist())
    del pl
    eo = W.draw_expert_output(w.P, w.T, w.H, w.seed, device="cuda")
    y = ex.combine(eo)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    qs = rng.choice(w.P * w.T, size=512, replace=False)
    for q in qs:
        s, t = divmod(int(q), w.T)
        if t >= c.counts[s]:
            continue
        rows = bits16(eo[:, q])
        ref, _ = oracle.combine_token_bf16(c.ids[s, t], rows, E=w.E)
        _check_bf16(bits16(y[s, t]), ref)
    ex.destroy()
    del eo, y, ex
    torch.cuda.empty_cache()


def _check_fp8(c, ex, eo, y, valid, s_range=None):
    w = c.w
    P, T, H = w.P, w.T, w.H
    eo_b = bits16(eo)
    land_c, land_s, ref_q, yq = oracle.combine_fp8(c.counts, c.ids, eo_b, E=w.E)
    ref, _ = oracle.combine_bf16(c.counts, c.ids, eo_b, E=w.E)
    gc, gs = ex.combine_landing()
    gc, gs = gc.cpu().numpy(), gs.cpu().numpy()
    yb = bits16(y)
    ev = bf16_bits_to_f64(eo_b)
    for s in range(P):
        n = int(c.counts[s])
        # landing slot r*T + t of source s is valid iff rank r got token (s, t)
        lv = np.zeros(P * T, bool)
        for r in range(P):
            lv[r * T:(r * T + n)] = valid[r, s * T:s * T + n]
        assert np.array_equal(gc[s][lv], land_c[s][lv]), f"landing codes of source {s} differ"
        assert np.array_equal(gs[s][lv], land_s[s][lv]), f"landing scales of source {s} differ"
        yv = bf16_bits_to_f64(yb[s, :n])
        rq = ref_q[s, :n]
        # bound against the exact sum
        mag = np.zeros((n, H))
        floor = np.zeros((n, H))
        nterms = np.zeros((n, 1))
        for r in range(P):
            vr = valid[r, s * T:s * T + n]
            rows = ev[r, s * T:s * T + n]
            mag += np.where(vr[:, None], np.abs(rows), 0.0)
            nterms += vr[:, None]
            e = land_s[s][r * T:r * T + n].astype(np.int64) - 127
            floor += np.where(vr[:, None], np.repeat(2.0 ** (e - 10), 32, axis=1), 0.0)
        # against the oracle's sum of the same dequantised terms: one bf16
        # rounding plus fp32 accumulation ((m-1) * 2^-24 * sum|terms|, the
        # dequantised terms being within 2^-4 of the exact ones)
        acc = np.maximum(nterms - 1, 0) * 2.0 ** -24 * (1 + 2.0 ** -4) * (mag + floor)
        assert np.all(np.abs(yv - rq) <= 2.0 ** -8 * np.abs(rq) + acc + 2.0 ** -126), \
            "y vs dequantised sum"
        err = np.abs(yv - ref[s, :n])
        assert np.all(err <= 0.07 * mag + floor + 2.0 ** -8 * np.abs(ref[s, :n])), "y vs exact sum"


FP8 = [
    dataclasses.replace(W.EP8_MXFP8, name="fp8 small", T=40, H=96, n_lo=0, n_hi=40),
    dataclasses.replace(W.EP8_MXFP8, name="fp8 bf16-dispatch", fmt="bf16", P=4, E=16, k=3, T=21,
                        H=1056, n_lo=1, n_hi=21, routing="uniform"),
    dataclasses.replace(W.EP8_MXFP8, name="fp8 long rows", P=2, E=8, k=2, T=3, H=8224, n_lo=3, n_hi=3,
                        routing="uniform"),
    # rows cut into whole workgroup chunks: 448 threads (H = 7168), 64 threads
    # (H = 5120), 256 threads (H = 4096 * 2)
    dataclasses.replace(W.EP8_MXFP8, name="fp8 H7168 448-thread chunks", P=3, E=12, k=4, T=9, H=7168,
                        n_lo=0, n_hi=9, routing="uniform"),
    dataclasses.replace(W.EP8_MXFP8, name="fp8 H5120 64-thread chunks", P=3, E=12, k=4, T=9, H=5120,
                        n_lo=0, n_hi=9, routing="uniform"),
    dataclasses.replace(W.EP8_MXFP8, name="fp8 H8192 256-thread chunks", P=2, E=8, k=3, T=5, H=8192,
                        n_lo=1, n_hi=5, routing="uniform"),
]


@pytest.mark.parametrize("w", FP8, ids=lambda w: w.name)
def test_combine_fp8_small(w):
    log(f"combine fp8: {w.name}")
    c, ex, valid = _dispatch(w, 71)
    g = W.torch_generator(71, "cuda")
    scale = torch.pow(2.0, torch.randint(-30, 30, (w.P, w.P * w.T, 1), generator=g, device="cuda").float())
    eo = (torch.randn(w.P, w.P * w.T, w.H, generator=g, device="cuda") * scale).to(torch.bfloat16)
    eo = _poison(eo, valid)
    y = ex.combine(eo)
    _check_fp8(c, ex, eo, y, valid)


def test_combine_fp8_special_blocks():
    """Blocks of zeros, bf16 subnormals, huge magnitudes and exact ties."""
    w = dataclasses.replace(W.EP8_MXFP8, name="fp8 specials", P=4, E=16, k=4, T=6, H=256,
                            n_lo=6, n_hi=6, fmt="bf16", routing="uniform")
    c, ex, valid = _dispatch(w, 72)
    rng = np.random.default_rng(72)
    vals = np.array([0.0, -0.0, 1e-40, -9.2e-41, 2.0 ** -133, 3.0e37, -1.0e37, 448.0, 1.0625,
                     1.1875, 2.0 ** -12, 3 * 2.0 ** -16, 2.0 ** -17, -3.0, 0.5], np.float32)
    eo_np = rng.choice(vals, size=(w.P, w.P * w.T, w.H)).astype(np.float32)
    eo_np[:, :, :32] = 0.0                 # an all-zero block
    eo_np[:, :, 32:64] = rng.choice([1e-40, -2e-40, 9.2e-41], size=(w.P, w.P * w.T, 32))
    eo = _poison(torch.from_numpy(eo_np).to(torch.bfloat16).cuda(), valid)
    y = ex.combine(eo)
    _check_fp8(c, ex, eo, y, valid)


def test_combine_fp8_full_ep8_mxfp8():
    w = W.EP8_MXFP8
    c, ex, valid = _dispatch(w, w.seed)
    eo = _poison(W.draw_expert_output(w.P, w.T, w.H, w.seed, device="cuda"), valid)
    y = ex.combine(eo)
    _check_fp8(c, ex, eo, y, valid)


def test_combine_fp8_landing_above_256mib_sampled():
    """The quantise pass writes its landing codes non-temporally when
    N * P * (H + H/32) exceeds 256 MiB (here 16 * 8192 * 2112 bytes), and
    through L2 below (every other FP8 case); sampled tokens against the
    oracle's per-token FP8 combine."""
    w = dataclasses.replace(W.EP8_MXFP8, name="fp8 landing 277 MB", fmt="bf16", P=16, E=64, k=8, T=512,
                            H=2048, n_lo=512, n_hi=512, routing="uniform")
    log(f"fp8 combine case: {w.name}")
    c = random_byte_case(w, w.seed)
    ex = _exchange(w)
    pl, sc, ids, wt = gpu_inputs(c)
    ex.dispatch(pl, ids, wt, num_tokens=c.counts.tolist())
    del pl
    eo = W.draw_expert_output(w.P, w.T, w.H, w.seed, device="cuda")
    y = ex.combine(eo)
    torch.cuda.synchronize()
    gc, gs = ex.combine_landing()
    rng = np.random.default_rng(5)
    for q in rng.choice(w.P * w.T, size=96, replace=False):
        s, t = divmod(int(q), w.T)
        rows = bits16(eo[:, q])
        codes, scales, ref_q, yq = oracle.combine_token_fp8(c.ids[s, t], rows, E=w.E)
        ref, _ = oracle.combine_token_bf16(c.ids[s, t], rows, E=w.E)
        owners = {oracle.owner(int(i), w.E, w.P) for i in c.ids[s, t]} - {-1}
        mag = np.zeros(w.H)
        floor = np.zeros(w.H)
        for r in sorted(owners):
            assert torch.equal(gc[s, r * w.T + t].cpu(), torch.from_numpy(codes[r])), f"codes {s},{t},{r}"
            assert torch.equal(gs[s, r * w.T + t].cpu(), torch.from_numpy(scales[r])), f"scales {s},{t},{r}"
            mag += np.abs(bf16_bits_to_f64(rows[r]))
            floor += np.repeat(2.0 ** (scales[r].astype(np.int64) - 127 - 10), 32)
        yv = bf16_bits_to_f64(bits16(y[s, t]))
        acc = max(len(owners) - 1, 0) * 2.0 ** -24 * (1 + 2.0 ** -4) * (mag + floor)
        assert np.all(np.abs(yv - ref_q) <= 2.0 ** -8 * np.abs(ref_q) + acc + 2.0 ** -126), (s, t)
        assert np.all(np.abs(yv - ref) <= 0.07 * mag + floor + 2.0 ** -8 * np.abs(ref)), (s, t)
    ex.destroy()
    del eo, y, ex, gc, gs
    torch.cuda.empty_cache()
