"""GPU combine parity against the CPU oracle, through the C ABI.

BF16 combine: every element satisfies |y - ref| <= 2^-7 |ref| + 1e-3, ref
being the oracle's fp32 sum over ranks (ascending rank order from +0), and
equals the oracle's bf16 result bit for bit (both sides add the same fp32
terms in the same order).  FP8 combine: the landing planes (e4m3 codes +
e8m0 scales) and y are bit-exact with the oracle's; y lies within
0.07 * sum|terms| of the exact sum of the bf16 terms, plus half an e4m3
subnormal step per term where a scaled term falls among the e4m3
subnormals (the elements that need it are counted and logged).  Expert
output slots that received no token are NaN-poisoned: they must never
reach the result.  The identity expert (each rank returns the token row
times the sum of its own experts' weights) must give the row times the sum
of all top-k weights, on the small, EP8 BF16 and MXFP8 workloads."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import bruteforce as bf
from tests.gpu_util import (bf16_bits_to_f64, bits16, check_bf16_sum, check_fp8_sum, fp8_exact_bound,
                            fp8_terms_and_floor, gpu_inputs, log, random_byte_case)

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


def _check_bf16_all(counts, y, o, what):
    yb = bits16(y)
    for s in range(len(counts)):
        n = int(counts[s])
        check_bf16_sum(yb[s, :n], o.ref[s, :n], o.y[s, :n], f"{what} source {s}")


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
    # magnitudes spread over 2^-20 .. 2^20 per row, so fp32 rounding shows
    g = W.torch_generator(61, "cuda")
    scale = torch.pow(2.0, torch.randint(-20, 21, (w.P, w.P * w.T, 1), generator=g, device="cuda").float())
    eo = (torch.randn(w.P, w.P * w.T, w.H, generator=g, device="cuda") * scale).to(torch.bfloat16)
    eo = _poison(eo, valid)
    y = ex.combine(eo)
    o = oracle.combine_bf16(c.counts, c.ids, bits16(eo), E=w.E)
    _check_bf16_all(c.counts, y, o, w.name)
    if w.k == 1:  # one term per token: the output is that term, bit for bit
        yb, eb = bits16(y), bits16(eo)
        for s in range(w.P):
            for t in range(int(c.counts[s])):
                r = int(c.ids[s, t, 0]) // (w.E // w.P)
                assert np.array_equal(yb[s, t], eb[r, s * w.T + t])


def test_combine_bf16_rows_past_count_untouched():
    w = dataclasses.replace(W.TINY, name="untouched", T=20, H=128)
    c, ex, valid = _dispatch(w, 62, counts=[20, 3, 0, 11])
    eo = _poison(W.draw_expert_output(w.P, w.T, w.H, 62, device="cuda"), valid)
    out = torch.full((w.P, w.T, w.H), 7.0, dtype=torch.bfloat16, device="cuda")
    ex.combine(eo, out)
    o = oracle.combine_bf16(c.counts, c.ids, bits16(eo), E=w.E)
    _check_bf16_all(c.counts, out, o, "untouched")
    v = out.float().cpu().numpy()
    for s in range(w.P):
        assert np.all(v[s, c.counts[s]:] == 7.0)


def test_combine_allocates_its_output_on_the_launch_stream():
    """combine(stream=s) with no output tensor, called while another stream
    is current: the output's zero fill is ordered before the kernel on s,
    so rows past each count are zero and the rest match the oracle."""
    w = dataclasses.replace(W.EP8_BF16, name="side stream", T=48, H=1024, n_lo=0, n_hi=48)
    c, ex, valid = _dispatch(w, 64)
    eo = _poison(W.draw_expert_output(w.P, w.T, w.H, 64, device="cuda"), valid)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    y = ex.combine(eo, stream=side)
    side.synchronize()
    o = oracle.combine_bf16(c.counts, c.ids, bits16(eo), E=w.E)
    _check_bf16_all(c.counts, y, o, "side stream")
    yb = bits16(y)
    for s in range(w.P):
        assert not yb[s, c.counts[s]:].any(), f"rows past the count of source {s} are not zero"


# --------------------------------------------------------------------------
# identity expert
# --------------------------------------------------------------------------

def identity_expert_output(w, R, x_f32, valid):
    """Expert outputs of the identity expert: rank r's row for token (s, t)
    is bf16(x[s, t] * W_r), W_r the sum of the token's weights of experts
    on rank r (double, then fp32); NaN where the token was not sent.
    x_f32: [P, T, H] float32 on the GPU."""
    P, T, H = w.P, w.T, w.H
    epr = w.E // P
    own = np.where((R.ids >= 0) & (R.ids < w.E), R.ids // epr, -1)
    wt = R.weights.astype(np.float64)
    xs = x_f32.reshape(P * T, H)
    eo = torch.empty((P, P * T, H), dtype=torch.bfloat16, device=x_f32.device)
    for r in range(P):
        wr = torch.from_numpy((wt * (own == r)).sum(-1).reshape(P * T).astype(np.float32)).to(x_f32.device)
        eo[r] = (xs * wr[:, None]).to(torch.bfloat16)
        eo[r][torch.from_numpy(~valid[r]).to(x_f32.device)] = float("nan")
    return eo


def check_identity(y_bits_s, x_s, wsum_s, extra=0.0, what=""):
    """y = x * sum(w) within (2^-7 + 2^-15) |x| sum(w) (+ extra): the terms
    bf16(x * W_r) carry one bf16 rounding and two fp32 roundings each and
    share the sign of x, their fp32 sum adds (m - 1) 2^-24, and y one more
    bf16 rounding; 2^-7 + 2^-15 covers all of them for m <= 64."""
    y = bf16_bits_to_f64(y_bits_s)
    want = x_s * wsum_s[:, None]
    mag = np.abs(x_s) * wsum_s[:, None]
    err = np.abs(y - want)
    bound = (2.0 ** -7 + 2.0 ** -15) * mag + extra + 2.0 ** -133
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    assert np.all(err <= bound), f"{what}: worst excess {(err - bound).max()}"


@pytest.mark.parametrize("w", [W.TINY, W.EP8_BF16], ids=lambda w: w.name)
def test_combine_identity_expert(w):
    """Each rank returns its token row times the sum of its local experts'
    weights; combine must give the row times the sum of all k weights, and
    match the oracle on the same expert outputs."""
    log(f"identity expert: {w.name}")
    d = W.draw_dispatch_inputs(w)
    R = d.routing
    ex = _exchange(w)
    ex.dispatch(d.payload.cuda(), torch.from_numpy(R.ids).cuda(), torch.from_numpy(R.weights).cuda(),
                num_tokens=R.counts.tolist())
    valid = oracle.dispatch(R.counts, d.payload.numpy(), R.ids, None, E=w.E, want_payload=False)["valid"].astype(bool)
    x = d.hidden_bf16.float()
    eo = identity_expert_output(w, R, x.cuda(), valid)
    y = ex.combine(eo)
    yb = bits16(y)
    xd = d.hidden_bf16.double().numpy()
    o = oracle.combine_bf16(R.counts, R.ids, bits16(eo), E=w.E)
    for s in range(w.P):
        n = int(R.counts[s])
        check_identity(yb[s, :n], xd[s, :n], R.weights[s, :n].sum(1, dtype=np.float64), what=f"source {s}")
        check_bf16_sum(yb[s, :n], o.ref[s, :n], o.y[s, :n], f"source {s}")


def test_combine_identity_expert_fp8_mxfp8():
    """The MXFP8 workload with FP8 combine: the identity expert works on the
    dequantised MXFP8 row x (e4m3 codes times 2^(scale - 127)), so y must be
    x * sum(w) within the identity bound plus the FP8 bound of the terms."""
    w = W.EP8_MXFP8
    log(f"identity expert, FP8 combine: {w.name}")
    d = W.draw_dispatch_inputs(w)
    R = d.routing
    ex = _exchange(w)
    ex.dispatch(d.payload.cuda(), torch.from_numpy(R.ids).cuda(), torch.from_numpy(R.weights).cuda(),
                scales=d.scales.cuda(), num_tokens=R.counts.tolist())
    valid = oracle.dispatch(R.counts, d.payload.numpy(), R.ids, None, d.scales.numpy(), E=w.E,
                            want_payload=False)["valid"].astype(bool)
    xd = bf.fp8_dequantise(d.payload.numpy(), d.scales.numpy())   # exact in fp32
    eo = identity_expert_output(w, R, torch.from_numpy(xd.astype(np.float32)).cuda(), valid)
    y = ex.combine(eo)
    eb = bits16(eo)
    o8 = oracle.combine_fp8(R.counts, R.ids, eb, E=w.E)
    exact = oracle.combine_bf16(R.counts, R.ids, eb, E=w.E).exact
    yb = bits16(y)
    ev = bf16_bits_to_f64(eb)
    viol = 0
    for s in range(w.P):
        n = int(R.counts[s])
        mag, floor = fp8_terms_and_floor(ev, valid, o8.land_scales[s], s, w.T, n, w.P)
        viol += check_fp8_sum(yb[s, :n], o8.y[s, :n], exact[s, :n], mag, floor, f"source {s}")
        # identity: the bf16 terms are within 2^-8 + 2^-22 of x * W_r
        wsum = R.weights[s, :n].sum(1, dtype=np.float64)
        extra = fp8_exact_bound(mag, floor) + (2.0 ** -8 + 2.0 ** -22) * np.abs(xd[s, :n]) * wsum[:, None]
        check_identity(yb[s, :n], xd[s, :n], wsum, extra=extra, what=f"source {s}")
    log(f"identity FP8: {viol} elements outside the literal 0.07 sum|terms| of "
        f"{int(R.counts.sum()) * w.H}")


def test_combine_bf16_special_values():
    w = dataclasses.replace(W.TINY, name="specials", T=8, H=64, n_lo=8, n_hi=8)
    c, ex, valid = _dispatch(w, 63)
    rng = np.random.default_rng(63)
    vals = np.array([0.0, -0.0, 3.0e37, -3.0e37, 1e-40, -1e-40, 9.2e-41, 65504.0,
                     1.0, -1.0, 2.0 ** -133, np.inf, -np.inf], np.float32)
    eo_np = rng.choice(vals, size=(w.P, w.P * w.T, w.H)).astype(np.float32)
    eo = _poison(torch.from_numpy(eo_np).to(torch.bfloat16).cuda(), valid)
    y = ex.combine(eo)
    o = oracle.combine_bf16(c.counts, c.ids, bits16(eo), E=w.E)
    _check_bf16_all(c.counts, y, o, "specials")


def test_combine_full_ep8_bf16():
    w = W.EP8_BF16
    c, ex, valid = _dispatch(w, w.seed)
    eo = _poison(W.draw_expert_output(w.P, w.T, w.H, w.seed, device="cuda"), valid)
    y = ex.combine(eo)
    o = oracle.combine_bf16(c.counts, c.ids, bits16(eo), E=w.E)
    _check_bf16_all(c.counts, y, o, w.name)


# --------------------------------------------------------------------------
# FP8 combine
# --------------------------------------------------------------------------

def _check_fp8(c, ex, eo, y, valid, what):
    w = c.w
    P, T = w.P, w.T
    eo_b = bits16(eo)
    o8 = oracle.combine_fp8(c.counts, c.ids, eo_b, E=w.E)
    exact = oracle.combine_bf16(c.counts, c.ids, eo_b, E=w.E).exact
    gc, gs = ex.combine_landing()
    gc, gs = gc.cpu().numpy(), gs.cpu().numpy()
    yb = bits16(y)
    ev = bf16_bits_to_f64(eo_b)
    viol, total = 0, 0
    for s in range(P):
        n = int(c.counts[s])
        # landing slot r*T + t of source s is valid iff rank r got token (s, t)
        lv = np.zeros(P * T, bool)
        for r in range(P):
            lv[r * T:(r * T + n)] = valid[r, s * T:s * T + n]
        assert np.array_equal(gc[s][lv], o8.land_codes[s][lv]), f"landing codes of source {s} differ"
        assert np.array_equal(gs[s][lv], o8.land_scales[s][lv]), f"landing scales of source {s} differ"
        mag, floor = fp8_terms_and_floor(ev, valid, o8.land_scales[s], s, T, n, P)
        viol += check_fp8_sum(yb[s, :n], o8.y[s, :n], exact[s, :n], mag, floor, f"{what} source {s}")
        total += n * w.H
    log(f"{what}: {viol} of {total} elements outside the literal 0.07 sum|terms| "
        f"(within it once the e4m3-subnormal floor is added)")
    return viol


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
    _check_fp8(c, ex, eo, y, valid, w.name)


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
    _check_fp8(c, ex, eo, y, valid, "fp8 specials")


def test_combine_fp8_full_ep8_mxfp8():
    w = W.EP8_MXFP8
    c, ex, valid = _dispatch(w, w.seed)
    eo = _poison(W.draw_expert_output(w.P, w.T, w.H, w.seed, device="cuda"), valid)
    y = ex.combine(eo)
    _check_fp8(c, ex, eo, y, valid, w.name)


def test_combine_fp8_landing_above_256mib():
    """The quantise pass writes its landing codes non-temporally when
    N * P * (H + H/32) exceeds 256 MiB (here 16 * 8192 * 2112 bytes), and
    through L2 below (every other FP8 case); every token against the
    oracle."""
    w = dataclasses.replace(W.EP8_MXFP8, name="fp8 landing 277 MB", fmt="bf16", P=16, E=64, k=8, T=512,
                            H=2048, n_lo=512, n_hi=512, routing="uniform")
    log(f"fp8 combine case: {w.name}")
    c, ex, valid = _dispatch(w, w.seed)
    eo = _poison(W.draw_expert_output(w.P, w.T, w.H, w.seed, device="cuda"), valid)
    y = ex.combine(eo)
    torch.cuda.synchronize()
    _check_fp8(c, ex, eo, y, valid, w.name)
    ex.destroy()
    del eo, y, ex
    torch.cuda.empty_cache()
