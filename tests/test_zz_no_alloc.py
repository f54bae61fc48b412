"""The combine entry point that allocates nothing (moe_ep_combine_noalloc)
against moe_ep_combine, through the C ABI: on an FP8-combine handle it
stages the landing planes in the library's static array instead of the
workspace, and its output must equal moe_ep_combine's bit for bit (and the
oracle's bf16 result), on two calls in a row, the second with a smaller
step; a BF16 handle gives the same result as moe_ep_combine; a step whose
landing planes exceed the array is rejected before any launch."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import bits16, gpu_inputs, log, random_byte_case

pytestmark = pytest.mark.gpu

BASE = dataclasses.replace(W.EP8_BF16, name="noalloc", combine="fp8")  # P=8, E=256, k=8, H=7168


def _step(ex, w, seed):
    c = random_byte_case(w, seed)
    pl, sc, ids, wt = gpu_inputs(c)
    ex.dispatch(pl, ids, wt, num_tokens=c.counts.tolist(), runtime_max_tokens_per_rank=w.T)
    valid = oracle.dispatch(c.counts, c.payload, c.ids, None, E=w.E, want_payload=False)["valid"].astype(bool)
    eo = W.draw_expert_output(w.P, w.T, w.H, seed, device="cuda")
    eo[torch.from_numpy(~valid).cuda()] = float("nan")
    return c, eo


@pytest.mark.parametrize("combine", ["fp8", "bf16"])
def test_noalloc_combine_matches_combine(combine):
    from combine_route_mask_amd import moe_ep
    from combine_route_mask_amd.moe_ep import MoeEpExchange
    w0 = dataclasses.replace(BASE, combine=combine)
    ex = MoeEpExchange(w0.P, w0.E, w0.k, w0.T, w0.H, combine_format=combine)
    # a 128-token step (60.6 MB of FP8 landing planes), then a 40-token one
    for T, lo, seed in ((128, 64, 91), (40, 0, 92)):
        w = dataclasses.replace(w0, T=T, n_lo=lo, n_hi=T)
        log(f"noalloc combine: {combine}, T={T}")
        c, eo = _step(ex, w, seed)
        if combine == "fp8":
            codes, scales = ex.combine_landing()
            codes.fill_(0x7F)   # NaN codes and scales: reading the workspace's
            scales.fill_(0xFF)  # landing planes would poison the result
        y_na = torch.full((w.P, w.T, w.H), 3.0, dtype=torch.bfloat16, device="cuda")
        moe_ep.moe_ep_combine_noalloc(ex.handle, eo, y_na)
        if combine == "fp8":
            assert bool((codes == 0x7F).all()) and bool((scales == 0xFF).all()), \
                "the workspace landing planes were written"
        y = torch.full((w.P, w.T, w.H), 3.0, dtype=torch.bfloat16, device="cuda")
        moe_ep.moe_ep_combine(ex.handle, eo, y)
        torch.cuda.synchronize()
        a, b = bits16(y_na), bits16(y)
        assert np.array_equal(a, b), f"T={T}: {int((a != b).sum())} elements differ from moe_ep_combine"
        eb = bits16(eo)
        o = (oracle.combine_fp8 if combine == "fp8" else oracle.combine_bf16)(c.counts, c.ids, eb, E=w.E)
        for s in range(w.P):
            n = int(c.counts[s])
            assert np.array_equal(a[s, :n], o.y[s, :n]), f"T={T}: source {s} differs from the oracle"
            assert np.all(a[s, n:] == b[s, n:]), f"T={T}: rows past the count of source {s}"
    ex.destroy()


def test_noalloc_combine_rejects_steps_beyond_the_array():
    """160 tokens per rank at P = 8, H = 7168: 8 * 1280 * 7392 bytes of
    landing planes, above 64 MiB; rejected with nothing launched, while
    the ordinary combine of the same step works."""
    from combine_route_mask_amd import moe_ep
    from combine_route_mask_amd.moe_ep import MoeEpExchange
    w = dataclasses.replace(BASE, T=160, n_lo=150, n_hi=160)
    assert w.P * -(-(w.P * w.T * (w.H + w.H // 32)) // 256) * 256 > moe_ep.STATIC_SCRATCH_BYTES
    ex = MoeEpExchange(w.P, w.E, w.k, w.T, w.H, combine_format="fp8")
    c, eo = _step(ex, w, 93)
    y = torch.full((w.P, w.T, w.H), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe_ep.MoeEpError) as e:
        moe_ep.moe_ep_combine_noalloc(ex.handle, eo, y)
    assert e.value.code == moe_ep.ERR_CAPACITY and "static staging array" in str(e.value)
    torch.cuda.synchronize()
    assert bool((y == 3.0).all()), "a rejected call wrote the output"
    moe_ep.moe_ep_combine(ex.handle, eo, y)
    o = oracle.combine_fp8(c.counts, c.ids, bits16(eo), E=w.E)
    yb = bits16(y)
    for s in range(w.P):
        n = int(c.counts[s])
        assert np.array_equal(yb[s, :n], o.y[s, :n])
    ex.destroy()


def test_noalloc_combine_replays_from_a_captured_graph():
    """Captured into a HIP graph (a caller that cannot allocate inside the
    capture), replayed three times with eager work between the replays that
    rewrites the shared static array (a combine of another step through the
    same entry point): every replay equals the eager call bit for bit."""
    from combine_route_mask_amd import moe_ep
    from combine_route_mask_amd.moe_ep import MoeEpExchange
    w = dataclasses.replace(BASE, T=64, n_lo=20, n_hi=64)
    ex = MoeEpExchange(w.P, w.E, w.k, w.T, w.H, combine_format="fp8")
    c, eo = _step(ex, w, 94)
    other = MoeEpExchange(w.P, w.E, w.k, w.T, w.H, combine_format="fp8")
    c2, eo2 = _step(other, w, 95)
    y_ref = torch.zeros((w.P, w.T, w.H), dtype=torch.bfloat16, device="cuda")
    moe_ep.moe_ep_combine_noalloc(ex.handle, eo, y_ref)
    y = torch.zeros_like(y_ref)
    y2 = torch.zeros_like(y_ref)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe_ep.moe_ep_combine_noalloc(ex.handle, eo, y)
    torch.cuda.synchronize()
    for i in range(3):
        y.fill_(0)
        moe_ep.moe_ep_combine_noalloc(other.handle, eo2, y2)  # overwrites the static array
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"replay {i} differs from the eager call"
    o = oracle.combine_fp8(c.counts, c.ids, bits16(eo), E=w.E)
    yb = bits16(y)
    for s in range(w.P):
        n = int(c.counts[s])
        assert np.array_equal(yb[s, :n], o.y[s, :n])
    del g
    ex.destroy()
    other.destroy()
