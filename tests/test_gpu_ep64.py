"""GPU parity at the EP64 workload's full size (P = 64 virtual ranks, 512
tokens per rank, hidden 7168, 256 experts, top-8), in the launch
configuration the bench times: every destination's receive planes
(payload, scale, id and weight planes, counts, source offsets, slot
lists) bit-exact for BF16, NVFP4 and DeepSeekFp8 dispatch and for NVFP4
with 1 KB of router logits per token, 256 EPLB statistics per rank and 48
of the 64 ranks taking part, every token of the BF16
combine against the oracle's fp32 sum (NaN in every expert-output slot
that received no token), and the identity-expert invariant over all 32768
tokens.  The oracle takes one destination, or one source rank's slots, at
a time, so host memory stays at one rank's share."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import bits16, check_bf16_sum, log, random_byte_case

pytestmark = pytest.mark.gpu


def _exchange(w):
    from combine_route_mask_amd.moe_ep import MoeEpExchange
    return MoeEpExchange(w.P, w.E, w.k, w.T, w.H, dispatch_format=w.fmt, combine_format=w.combine)


class Step:
    """One EP64 dispatch on the GPU with its inputs and the oracle's valid
    mask (every destination, no payload)."""

    def __init__(self, w):
        self.w = w
        log(f"ep64 setup: {w.name}")
        self.c = random_byte_case(w, w.seed)
        self.ex = _exchange(w)
        c = self.c
        self.pl = torch.from_numpy(c.payload).cuda()
        self.sc = None if c.scales is None else torch.from_numpy(c.scales).cuda()
        self.ids = torch.from_numpy(c.ids).cuda()
        self.wt = torch.from_numpy(c.weights).cuda()
        self.out = self.ex.dispatch(self.pl, self.ids, self.wt, scales=self.sc, num_tokens=c.counts.tolist(),
                                    runtime_max_tokens_per_rank=w.T)
        torch.cuda.synchronize()
        self.ids_only = oracle.dispatch(c.counts, c.payload, c.ids, None, None, E=w.E, want_payload=False)
        self.valid = self.ids_only["valid"].astype(bool)

    def free(self):
        self.ex.destroy()
        del self.pl, self.sc, self.out, self.ex
        torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def ep64_bf16():
    st = Step(W.EP64_BF16)
    yield st
    st.free()


def _check_bookkeeping(st):
    w, out, full = st.w, st.out, st.ids_only
    P = w.P
    assert np.array_equal(out["ids"].cpu().numpy(), full["ids"]), "ids plane / markers differ"
    cnt = full["counts"]
    assert np.array_equal(out["counts"].cpu().numpy(), cnt), "counts differ"
    offs = out["src_offsets"].cpu().numpy()
    assert np.array_equal(offs[:, :P], np.cumsum(cnt, axis=1) - cnt), "source offsets differ"
    assert np.array_equal(offs[:, P], cnt.sum(1)), "totals differ"
    slots = out["slots"].cpu().numpy()
    for r in range(P):
        n = int(cnt[r].sum())
        assert np.array_equal(slots[r, :n], full["slots"][r, :n]), f"slot list of rank {r} differs"
    log(f"{w.name}: id planes, counts, offsets and slot lists of all {P} ranks equal; "
        f"M = {int(cnt.sum())} pairs")


def _check_destinations(st, r0, r1):
    """Payload, scale and weight bytes of every valid slot of ranks r0..r1-1
    (only valid rows leave the GPU)."""
    w, c, out = st.w, st.c, st.out
    for r in range(r0, r1):
        one = oracle.dispatch(c.counts, c.payload, c.ids, c.weights, c.scales, E=w.E, r0=r, r1=r + 1)
        v = one["valid"][0].astype(bool)
        assert np.array_equal(v, st.valid[r])
        idx = torch.from_numpy(np.nonzero(v)[0]).cuda()
        assert np.array_equal(out["payload"][r].index_select(0, idx).cpu().numpy(), one["payload"][0][v]), \
            f"payload of rank {r} differs"
        if c.scales is not None:
            assert np.array_equal(out["scales"][r].index_select(0, idx).cpu().numpy(), one["scales"][0][v]), \
                f"scales of rank {r} differ"
        wt = out["weights"][r].index_select(0, idx).cpu().numpy()
        assert np.array_equal(wt.view(np.uint32), one["weights"][0][v].view(np.uint32)), \
            f"weights of rank {r} differ"
    log(f"{w.name}: payload / scale / weight rows of ranks {r0}..{r1 - 1} equal")


def test_ep64_bf16_dispatch_bookkeeping(ep64_bf16):
    _check_bookkeeping(ep64_bf16)


@pytest.mark.parametrize("group", range(4))
def test_ep64_bf16_dispatch_rows(ep64_bf16, group):
    _check_destinations(ep64_bf16, 16 * group, 16 * group + 16)


@pytest.fixture(scope="module")
def ep64_combined(ep64_bf16):
    """The BF16 combine of the fixture's dispatch on N(0,1) expert outputs
    with NaN in every slot that received no token."""
    st = ep64_bf16
    w = st.w
    eo = W.draw_expert_output(w.P, w.T, w.H, w.seed, device="cuda")
    eo[torch.from_numpy(~st.valid).cuda()] = float("nan")
    y = st.ex.combine(eo)
    torch.cuda.synchronize()
    yield eo, bits16(y)
    del eo, y
    torch.cuda.empty_cache()


@pytest.mark.parametrize("group", range(4))
def test_ep64_bf16_combine_every_token(ep64_bf16, ep64_combined, group):
    """Sources 16*group .. 16*group + 15: every token of the BF16 combine,
    each source rank's slots copied to the host and summed by the oracle."""
    st = ep64_bf16
    w, c = st.w, st.c
    T = w.T
    eo, yb = ep64_combined
    for s in range(16 * group, 16 * group + 16):
        eo_s = bits16(eo[:, s * T:(s + 1) * T])
        o = oracle.combine_bf16(c.counts, c.ids, eo_s, E=w.E, s0=s, s1=s + 1, slot0=s * T)
        n = int(c.counts[s])
        check_bf16_sum(yb[s, :n], o.ref[0, :n], o.y[0, :n], f"source {s}")
    log(f"{w.name}: combine of sources {16 * group}..{16 * group + 15} within the bar and bit-exact")


def test_ep64_identity_expert(ep64_bf16):
    """Identity expert over every token, on the fixture's routing (the
    workload's seeded routing, which the dispatch inputs' generator draws
    again here): y = x * sum(w) within (2^-7 + 2^-15) |x| sum(w) (see
    test_gpu_combine.check_identity), x being the workload's N(0,1) bf16
    token rows."""
    from tests.test_gpu_combine import check_identity, identity_expert_output
    st = ep64_bf16
    w = st.w
    d = W.draw_dispatch_inputs(w, device="cuda")
    R = d.routing
    assert np.array_equal(R.ids, st.c.ids) and np.array_equal(R.counts, st.c.counts)
    eo = identity_expert_output(w, R, d.hidden_bf16.float(), st.valid)
    y = bits16(st.ex.combine(eo))
    del eo
    torch.cuda.empty_cache()
    x = d.hidden_bf16
    for s in range(w.P):
        n = int(R.counts[s])
        check_identity(y[s, :n], x[s, :n].double().cpu().numpy(), R.weights[s, :n].sum(1, dtype=np.float64),
                       what=f"source {s}")
    log(f"{w.name}: identity expert holds on all {int(R.counts.sum())} tokens")


def test_ep64_nvfp4_dispatch_every_destination():
    st = Step(W.EP64_NVFP4)
    try:
        _check_bookkeeping(st)
        _check_destinations(st, 0, st.w.P)
    finally:
        st.free()


def test_ep64_deepseek_fp8_dispatch_every_destination():
    """7 KB DeepSeekFp8 rows in a launch too large to prefetch: two vectors
    per lane, one workgroup per row (the EP64 DeepSeekFp8 workload)."""
    st = Step(W.EP64_DSFP8)
    try:
        _check_bookkeeping(st)
        _check_destinations(st, 0, st.w.P)
    finally:
        st.free()


def test_ep64_nvfp4_extras_alive48_every_destination():
    """The bench's EP64 NVFP4 workload with each token's 1 KB of router
    logits (extra payload, loaded with the row), 256 EPLB statistics per
    rank, and 48 of the 64 ranks taking part: every live destination's
    payload, scale, extra, id and weight rows and gathered statistics
    bit-exact; the 16 masked-off regions untouched (poisoned workspace)."""
    import dataclasses
    from combine_route_mask_amd.moe_ep import MoeEpExchange
    w = dataclasses.replace(W.EP64_NVFP4_EXTRAS, alive=W.EP64_MASK48.alive)
    log(f"ep64 setup: {w.name} alive48")
    c = random_byte_case(w, w.seed)
    rng = np.random.default_rng(w.seed + 17)
    extra = rng.integers(0, 256, size=(w.P, w.T, w.extra_bytes)).astype(np.uint8)
    stats = rng.integers(-(1 << 30), 1 << 30, size=(w.P, w.n_eplb)).astype(np.int32)
    live = list(w.alive)
    active = sum(1 << r for r in live)
    ex = MoeEpExchange(w.P, w.E, w.k, w.T, w.H, dispatch_format=w.fmt, combine_format=w.combine,
                       extra_payload_bytes_per_token=w.extra_bytes, eplb_stats_num_experts=w.n_eplb)
    try:
        ex.workspace.fill_(0x5A)
        pl = torch.from_numpy(c.payload).cuda()
        sc = torch.from_numpy(c.scales).cuda()
        out = ex.dispatch(pl, torch.from_numpy(c.ids).cuda(), torch.from_numpy(c.weights).cuda(), scales=sc,
                          num_tokens=c.counts.tolist(), runtime_max_tokens_per_rank=w.T, active_rank_mask=active,
                          extra_payload=torch.from_numpy(extra).cuda(), eplb_local_stats=torch.from_numpy(stats).cuda())
        torch.cuda.synchronize()
        for r in range(w.P):
            if r not in live:
                assert bool((ex.workspace[r] == 0x5A).all()), f"masked-off rank {r} was written"
        g = out["eplb_gathered_stats"].cpu().numpy()
        poison = np.full((w.P, w.n_eplb), 0x5A5A5A5A, np.int32)
        ids_g = out["ids"]
        for r in live:
            one = oracle.dispatch(c.counts, c.payload, c.ids, c.weights, c.scales, E=w.E, r0=r, r1=r + 1,
                                  active=active, extra=extra)
            v = one["valid"][0].astype(bool)
            assert np.array_equal(ids_g[r].cpu().numpy(), one["ids"][0]), f"ids plane of rank {r}"
            idx = torch.from_numpy(np.nonzero(v)[0]).cuda()
            for key in ("payload", "scales", "extra"):
                assert np.array_equal(out[key][r].index_select(0, idx).cpu().numpy(), one[key][0][v]), \
                    f"{key} of rank {r} differs"
            wt = out["weights"][r].index_select(0, idx).cpu().numpy()
            assert np.array_equal(wt.view(np.uint32), one["weights"][0][v].view(np.uint32)), f"weights of rank {r}"
            expect = oracle.eplb_allgather(stats, r, active=active, out=poison.copy())
            assert np.array_equal(g[r], expect), f"gathered statistics of rank {r}"
        log(f"{w.name}: 48 live destinations bit-exact, 16 masked-off regions untouched")
    finally:
        ex.destroy()
        del ex
        torch.cuda.empty_cache()
