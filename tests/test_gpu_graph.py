"""Captured HIP graphs of the exchange: a dispatch + combine step (and an
all-gatherv + reduce-scatterv step) captured once, replayed several times
with eager work and synchronisations in between; every replay must equal
the eager result bit for bit.  The kernels write no memset nodes, so the
graphs hold kernel nodes only."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_util import gpu_inputs, log, random_byte_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from combine_route_mask_amd import moe_ep
    assert torch.cuda.is_available() and moe_ep.moe_ep_is_supported()
    yield
    torch.cuda.empty_cache()


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("w", [
    dataclasses.replace(W.EP8_BF16, name="ep8 bf16 graph", H=1024),
    dataclasses.replace(W.EP8_BF16, name="ep8 bf16 long rows graph (write-through stores)", H=7168),
    dataclasses.replace(W.EP8_MXFP8, name="mxfp8 fp8 graph", T=64, H=512, n_lo=10, n_hi=64),
    dataclasses.replace(W.EP8_MXFP8, name="mxfp8 fp8 graph, 448-thread rows", T=32, H=7168, n_lo=5,
                        n_hi=32),
], ids=lambda w: w.name)
def test_exchange_graph_replays(w):
    from combine_route_mask_amd.moe_ep import MoeEpExchange
    log(f"graph: {w.name}")
    c = random_byte_case(w, 101)
    pl, sc, ids, wt = gpu_inputs(c)
    ex = MoeEpExchange(w.P, w.E, w.k, w.T, w.H, dispatch_format=w.fmt, combine_format=w.combine)
    eo = W.draw_expert_output(w.P, w.T, w.H, 101, device="cuda")
    out = torch.zeros((w.P, w.T, w.H), dtype=torch.bfloat16, device="cuda")

    def step():
        ex.dispatch(pl, ids, wt, scales=sc, num_tokens=c.counts.tolist())
        ex.combine(eo, out)

    step()
    torch.cuda.synchronize()
    views = ex.dispatch(pl, ids, wt, scales=sc, num_tokens=c.counts.tolist())
    ex.combine(eo, out)
    ref_out = out.clone()
    ref_ids = views["ids"].clone()
    ref_pl = views["payload"].clone()
    g = _capture(step)
    for i in range(4):
        out.zero_()                       # eager work between replays
        views["ids"].view(torch.uint8).fill_(0x33)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"replay {i}: output"
        assert torch.equal(views["ids"], ref_ids), f"replay {i}: ids"
        valid = (ref_ids[..., 0] != w.E)
        assert torch.equal(views["payload"][valid], ref_pl[valid]), f"replay {i}: payload"


def test_agrs_graph_replays():
    from combine_route_mask_amd import moe_ep
    w = dataclasses.replace(W.AGRS16, name="agrs graph", P=6, H=512)
    d = W.draw_agrs_inputs(w, device="cuda", sizes=np.array([3, 0, 9, 4, 1, 7], np.int32))
    sizes = d.sizes.tolist()
    total = sum(sizes)
    x = [d.hidden, torch.from_numpy(d.weights).cuda(), torch.from_numpy(d.ids).cuda()]
    outs = [torch.zeros((w.P, total) + tuple(t.shape[2:]), dtype=t.dtype, device="cuda") for t in x]
    part = d.partial.contiguous()
    rs = torch.zeros((w.P, max(sizes), w.H), dtype=torch.bfloat16, device="cuda")

    def step():
        moe_ep.allgatherv(sizes, x, outs)
        moe_ep.reduce_scatterv(sizes, part, rs)

    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs] + [rs.clone()]
    g = _capture(step)
    for i in range(3):
        for o in outs + [rs]:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs + [rs], ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {i}"
