"""GPU parity of the dispatch extras, bit-exact against the oracle:
DeepSeekFp8 rows (e4m3 + one fp32 scale per 128 elements), extra
per-token payload bytes (NVLinkOneSidedConfig, extra_payload_bytes_per_token)
and the EPLB statistics all-gather (moe_a2a_dispatch, eplb_local_stats ->
eplb_gathered_stats, row r = rank r's statistics), alone and under an
active rank mask; plus the router-logits all-gatherv (vLLM
AgRsAll2AllManager.dispatch_router_logits: hidden, router_logits and extra
tensors gathered in one call)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import gpu_inputs, log, random_byte_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from combine_route_mask_amd import moe_ep
    assert torch.cuda.is_available() and moe_ep.moe_ep_is_supported()
    yield
    torch.cuda.empty_cache()


CASES = [
    (dataclasses.replace(W.EP8_BF16, name="deepseek fp8", fmt="deepseek_fp8", T=40, H=512,
                         n_lo=0, n_hi=40), 0, 0, None),
    (dataclasses.replace(W.TINY, name="extra 48B + eplb 16"), 48, 16, None),
    (dataclasses.replace(W.EP8_MXFP8, name="mxfp8 extra 7B eplb 256", T=20, H=256, n_lo=3,
                         n_hi=20), 7, 256, None),
    (dataclasses.replace(W.EP8_BF16, name="masked extra + eplb", T=24, H=256, n_lo=0,
                         n_hi=24), 32, 64, [0, 2, 3, 6]),
    (dataclasses.replace(W.EP64_BF16, name="P64 eplb E", T=4, H=64, n_lo=0, n_hi=4), 16, 256, None),
    # extra rows of at most 256 aligned 16-byte words travel with the payload
    # loads (long and short rows, small and large steps); longer or unaligned
    # ones are copied after the payload
    (dataclasses.replace(W.EP8_BF16, name="router logits 1 KB, long rows", T=64, H=4096, n_lo=0,
                         n_hi=64), 1024, 0, None),
    (dataclasses.replace(W.TINY, name="extra 4096B, long rows", P=4, E=16, k=4, T=8, H=8192, n_lo=1,
                         n_hi=8), 4096, 0, None),
    (dataclasses.replace(W.TINY, name="extra 4112B copied, long rows", P=4, E=16, k=4, T=8, H=8192,
                         n_lo=1, n_hi=8), 4112, 0, None),
    (dataclasses.replace(W.EP64_BF16, name="extra 64B, 16640 slots", T=260, H=64, n_lo=0, n_hi=3),
     64, 0, None),
    # 7 KB rows in steps too large to prefetch (two vectors per lane, one
    # workgroup per row), with the extra row loaded beside the payload or
    # copied after it
    (dataclasses.replace(W.EP8_BF16, name="deepseek fp8 7 KB rows, 17600 slots, extra 1 KB + eplb 64", P=16,
                         fmt="deepseek_fp8", T=1100, H=7168, n_lo=900, n_hi=1100), 1024, 64, None),
    (dataclasses.replace(W.EP8_BF16, name="mxfp8 7 KB rows, 17600 slots, extra 4100B copied, masked", P=16,
                         fmt="mxfp8", T=1100, H=7168, n_lo=900, n_hi=1100), 4100, 0,
     [0, 3, 5, 6, 9, 12, 15]),
]


@pytest.mark.parametrize("w,xb,neplb,alive", CASES, ids=lambda x: getattr(x, "name", str(x)))
def test_dispatch_extras(w, xb, neplb, alive):
    from combine_route_mask_amd.moe_ep import MoeEpExchange
    log(f"extras: {w.name} extra={xb} eplb={neplb} alive={alive}")
    c = random_byte_case(w, 91)
    rng = np.random.default_rng(91)
    extra = rng.integers(0, 256, size=(w.P, w.T, xb)).astype(np.uint8) if xb else None
    stats = rng.integers(-(1 << 30), 1 << 30, size=(w.P, neplb)).astype(np.int32) if neplb else None
    active = None if alive is None else sum(1 << r for r in alive)
    ex = MoeEpExchange(w.P, w.E, w.k, w.T, w.H, dispatch_format=w.fmt, combine_format=w.combine,
                       extra_payload_bytes_per_token=xb, eplb_stats_num_experts=neplb)
    ex.workspace.fill_(0x5A)
    pl, sc, ids, wt = gpu_inputs(c)
    out = ex.dispatch(pl, ids, wt, scales=sc, num_tokens=c.counts.tolist(),
                      active_rank_mask=active,
                      extra_payload=None if extra is None else torch.from_numpy(extra).cuda(),
                      eplb_local_stats=None if stats is None else torch.from_numpy(stats).cuda())
    want = oracle.dispatch(c.counts, c.payload, c.ids, c.weights, c.scales, E=w.E, active=active,
                           extra=extra)
    live = range(w.P) if alive is None else alive
    ids_g = out["ids"].cpu().numpy()
    for r in live:
        v = want["valid"][r].astype(bool)
        assert np.array_equal(ids_g[r], want["ids"][r])
        assert np.array_equal(out["payload"][r].cpu().numpy()[v], want["payload"][r][v])
        if c.scales is not None:
            assert np.array_equal(out["scales"][r].cpu().numpy()[v], want["scales"][r][v])
        if xb:
            assert np.array_equal(out["extra"][r].cpu().numpy()[v], want["extra"][r][v])
    if neplb:
        g = out["eplb_gathered_stats"].cpu().numpy()
        poison = np.full((w.P, neplb), 0x5A5A5A5A, np.int32)
        for r in range(w.P):
            expect = oracle.eplb_allgather(stats, r, active=active, out=poison.copy())
            assert np.array_equal(g[r], expect), f"gathered statistics of rank {r}"
    else:
        assert out["eplb_gathered_stats"] is None
    if alive is not None:
        for r in range(w.P):
            if r not in alive:
                assert bool((ex.workspace[r] == 0x5A).all()), f"masked-off rank {r} was written"


def test_extras_argument_checks():
    from combine_route_mask_amd import moe_ep
    w = W.TINY
    c = random_byte_case(w, 92)
    pl, sc, ids, wt = gpu_inputs(c)
    ex = moe_ep.MoeEpExchange(w.P, w.E, w.k, w.T, w.H)
    x = torch.zeros((w.P, w.T, 16), dtype=torch.uint8, device="cuda")
    st = torch.zeros((w.P, 8), dtype=torch.int32, device="cuda")
    with pytest.raises(moe_ep.MoeEpArgError):  # no extra bytes reserved
        moe_ep.moe_ep_dispatch(ex.handle, pl, None, ids, wt, c.counts.tolist(), w.T, extra_payload=x)
    with pytest.raises(moe_ep.MoeEpArgError):  # no statistics configured
        moe_ep.moe_ep_dispatch(ex.handle, pl, None, ids, wt, c.counts.tolist(), w.T, eplb_local_stats=st)


def test_allgatherv_router_logits_and_extras():
    from combine_route_mask_amd import moe_ep
    P, H, E = 6, 512, 64
    sizes = [5, 0, 17, 3, 9, 1]
    total, smax = sum(sizes), max(sizes)
    g = torch.Generator(device="cuda").manual_seed(93)
    hidden = torch.randn(P, smax, H, generator=g, device="cuda").to(torch.bfloat16)
    logits = torch.randn(P, smax, E, generator=g, device="cuda")
    extra1 = torch.randint(0, 1 << 30, (P, smax, 3), generator=g, device="cuda", dtype=torch.int32)
    extra2 = torch.randint(0, 255, (P, smax, 5), generator=g, device="cuda", dtype=torch.int64).to(torch.uint8)
    ins = [hidden, logits, extra1, extra2]
    outs = [torch.empty((P, total) + tuple(x.shape[2:]), dtype=x.dtype, device="cuda") for x in ins]
    moe_ep.allgatherv(sizes, ins, outs)
    for x, o in zip(ins, outs):
        rows = x.contiguous().view(torch.uint8).cpu().numpy().reshape(P, smax, -1)
        want = oracle.allgatherv(np.array(sizes, np.int32), rows)
        got = o.view(torch.uint8).cpu().numpy().reshape(P, total, -1)
        for r in range(P):
            assert np.array_equal(got[r], want)
