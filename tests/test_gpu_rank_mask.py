"""GPU parity of the active rank mask (FlashInfer moe_a2a_dispatch,
active_rank_mask: a token bound for a rank whose bit is clear never reaches it).  With
every virtual rank in one call, a masked-off rank neither sends nor
receives: its workspace region must stay byte-for-byte untouched, live
regions must match the oracle run with the same mask bit for bit, and the
combine sums live ranks only and writes no row of a masked-off source."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import (bf16_bits_to_f64, bits16, check_bf16_sum, check_fp8_sum, fp8_terms_and_floor, gpu_inputs,
                            log, random_byte_case)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from combine_route_mask_amd import moe_ep
    assert torch.cuda.is_available() and moe_ep.moe_ep_is_supported()
    yield
    torch.cuda.empty_cache()


def _mask(alive):
    m = 0
    for r in alive:
        m |= 1 << r
    return m


CASES = [
    (dataclasses.replace(W.TINY, name="tiny"), [0, 2, 3]),
    (dataclasses.replace(W.EP8_BF16, name="ep8 H1024", H=1024, T=64, n_lo=10, n_hi=64), [1, 2, 5, 7]),
    (dataclasses.replace(W.TINY, name="P64 E128", P=64, E=128, k=8, T=6, H=64, n_lo=0, n_hi=6),
     sorted(np.random.default_rng(3).choice(64, size=41, replace=False).tolist())),
    (dataclasses.replace(W.EP8_MXFP8, name="mxfp8 fp8-combine", T=24, H=256, n_lo=5, n_hi=24), [0, 3, 4, 6]),
    (dataclasses.replace(W.TINY, name="one live rank", k=3), [2]),
]


@pytest.mark.parametrize("w,alive", CASES, ids=lambda x: getattr(x, "name", "mask"))
def test_rank_mask_dispatch_and_combine(w, alive):
    from combine_route_mask_amd.moe_ep import MoeEpExchange
    log(f"rank mask: {w.name} alive={alive}")
    active = _mask(alive)
    c = random_byte_case(w, 81)
    ex = MoeEpExchange(w.P, w.E, w.k, w.T, w.H, dispatch_format=w.fmt, combine_format=w.combine)
    ex.workspace.fill_(0xA5)
    pl, sc, ids, wt = gpu_inputs(c)
    out = ex.dispatch(pl, ids, wt, scales=sc, num_tokens=c.counts.tolist(),
                      runtime_max_tokens_per_rank=w.T, active_rank_mask=active)
    torch.cuda.synchronize()
    for r in range(w.P):
        if r not in alive:
            assert bool((ex.workspace[r] == 0xA5).all()), f"masked-off rank {r} was written"
    want = oracle.dispatch(c.counts, c.payload, c.ids, c.weights, c.scales, E=w.E, active=active)
    ids_g = out["ids"].cpu().numpy()
    cnt_g = out["counts"].cpu().numpy()
    slots_g = out["slots"].cpu().numpy()
    pl_g = out["payload"].cpu().numpy()
    for r in alive:
        assert np.array_equal(ids_g[r], want["ids"][r]), f"ids of rank {r}"
        assert np.array_equal(cnt_g[r], want["counts"][r]), f"counts of rank {r}"
        n = int(want["counts"][r].sum())
        assert np.array_equal(slots_g[r, :n], want["slots"][r, :n])
        v = want["valid"][r].astype(bool)
        assert np.array_equal(pl_g[r][v], want["payload"][r][v]), f"payload of rank {r}"
    # combine over live ranks only; NaN in every slot that holds no token
    valid = want["valid"].astype(bool)
    eo = W.draw_expert_output(w.P, w.T, w.H, 81, device="cuda")
    eo[torch.from_numpy(~valid).cuda()] = float("nan")
    y = torch.full((w.P, w.T, w.H), 7.0, dtype=torch.bfloat16, device="cuda")
    ex.combine(eo, y)
    yb = bits16(y)
    eb = bits16(eo)
    if w.combine == "fp8":
        o8 = oracle.combine_fp8(c.counts, c.ids, eb, E=w.E, active=active)
        exact = oracle.combine_bf16(c.counts, c.ids, eb, E=w.E, active=active).exact
        ev = bf16_bits_to_f64(eb)
    else:
        o = oracle.combine_bf16(c.counts, c.ids, eb, E=w.E, active=active)
    for s in range(w.P):
        rows = bf16_bits_to_f64(yb[s])
        if s not in alive:
            assert np.all(rows == 7.0), f"rows of masked-off source {s} were written"
            continue
        n = int(c.counts[s])
        if w.combine == "fp8":
            # valid is False on masked-off ranks: they receive nothing
            mag, floor = fp8_terms_and_floor(ev, valid, o8.land_scales[s], s, w.T, n, w.P)
            check_fp8_sum(yb[s, :n], o8.y[s, :n], exact[s, :n], mag, floor, f"source {s}")
        else:
            check_bf16_sum(yb[s, :n], o.ref[s, :n], o.y[s, :n], f"source {s}")
        assert np.all(rows[n:] == 7.0)


def test_rank_mask_all_ones_equals_no_mask():
    from combine_route_mask_amd.moe_ep import MoeEpExchange
    w = dataclasses.replace(W.EP8_BF16, name="ones", H=512, T=32, n_lo=0, n_hi=32)
    c = random_byte_case(w, 82)
    pl, sc, ids, wt = gpu_inputs(c)
    ex = MoeEpExchange(w.P, w.E, w.k, w.T, w.H)
    a = ex.dispatch(pl, ids, wt, num_tokens=c.counts.tolist())
    snap = {k: v.clone() for k, v in a.items() if isinstance(v, torch.Tensor)}
    b = ex.dispatch(pl, ids, wt, num_tokens=c.counts.tolist(), active_rank_mask=(1 << w.P) - 1)
    for k, v in snap.items():
        assert torch.equal(v.view(torch.uint8), b[k].view(torch.uint8)), k


def test_rank_mask_rejects_bits_beyond_ep_size():
    from combine_route_mask_amd import moe_ep
    w = W.TINY
    c = random_byte_case(w, 83)
    pl, sc, ids, wt = gpu_inputs(c)
    ex = moe_ep.MoeEpExchange(w.P, w.E, w.k, w.T, w.H)
    with pytest.raises(moe_ep.MoeEpArgError):
        ex.dispatch(pl, ids, wt, num_tokens=c.counts.tolist(), active_rank_mask=1 << w.P)
