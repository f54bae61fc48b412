"""GPU dispatch parity: the HIP path (through the C ABI) against the CPU
oracle, bit-exact -- receive payload / scale / ids / weights planes of
every valid slot, invalid-id markers on every other slot, per-source
counts, source offsets and the ascending valid-slot list.

Sizes: the small cases span several 256-thread tiles and ragged tails;
the EP8 workloads run at their real shapes here, the EP64 ones in
test_gpu_ep64.py."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import DispatchCase, bits16, check_bf16_sum, gpu_inputs, log, random_byte_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from combine_route_mask_amd import moe_ep
    assert torch.cuda.is_available() and moe_ep.moe_ep_is_supported()
    yield
    torch.cuda.empty_cache()


def _exchange(w, T_cap=None, **kw):
    from combine_route_mask_amd.moe_ep import MoeEpExchange
    return MoeEpExchange(w.P, w.E, w.k, T_cap or w.T, w.H, dispatch_format=w.fmt,
                         combine_format=w.combine, **kw)


def _check(c: DispatchCase, out, dests=None, invalid_id=None, with_weights=True):
    w = c.w
    P, T, k = w.P, w.T, w.k
    inv = w.E if invalid_id is None else invalid_id
    full = oracle.dispatch(c.counts, c.payload, c.ids, c.weights if with_weights else None,
                           c.scales, E=w.E, invalid_id=inv, want_payload=False)
    torch.cuda.synchronize()
    ids = out["ids"].cpu().numpy()
    assert np.array_equal(ids, full["ids"]), "ids plane / markers differ"
    assert np.array_equal(out["counts"].cpu().numpy(), full["counts"]), "counts differ"
    offs = out["src_offsets"].cpu().numpy()
    cnt = full["counts"]
    assert np.array_equal(offs[:, :P], np.cumsum(cnt, axis=1) - cnt), "source offsets differ"
    assert np.array_equal(offs[:, P], cnt.sum(1)), "totals differ"
    slots = out["slots"].cpu().numpy()
    for r in range(P):
        n = int(cnt[r].sum())
        assert np.array_equal(slots[r, :n], full["slots"][r, :n]), f"slot list of rank {r} differs"
    for r in (range(P) if dests is None else dests):
        one = oracle.dispatch(c.counts, c.payload, c.ids, c.weights if with_weights else None,
                              c.scales, E=w.E, invalid_id=inv, r0=r, r1=r + 1)
        v = one["valid"][0].astype(bool)
        pl = out["payload"][r].cpu().numpy()
        assert np.array_equal(pl[v], one["payload"][0][v]), f"payload of rank {r} differs"
        if c.scales is not None:
            sc = out["scales"][r].cpu().numpy()
            assert np.array_equal(sc[v], one["scales"][0][v]), f"scales of rank {r} differ"
        if with_weights:
            wt = out["weights"][r].cpu().numpy()
            assert np.array_equal(wt[v].view(np.uint32), one["weights"][0][v].view(np.uint32)), \
                f"weights of rank {r} differ"


def _run(c: DispatchCase, ex=None, T_cap=None, dests=None, invalid_id=None, with_weights=True):
    w = c.w
    log(f"dispatch case: {w.name} P={w.P} T={w.T} H={w.H} k={w.k} E={w.E} fmt={w.fmt} "
        f"counts[:8]={c.counts[:8].tolist()}")
    ex = ex or _exchange(w, T_cap, has_weights=with_weights, invalid_expert_id=invalid_id)
    pl, sc, ids, wt = gpu_inputs(c)
    out = ex.dispatch(pl, ids, wt if with_weights else None, scales=sc,
                      num_tokens=c.counts.tolist(), runtime_max_tokens_per_rank=w.T)
    _check(c, out, dests, invalid_id, with_weights)
    return ex


SMALL = [
    W.TINY,
    dataclasses.replace(W.TINY, name="p1", P=1, E=4, T=300, n_lo=0, n_hi=300, H=64),
    dataclasses.replace(W.TINY, name="k1", k=1, T=70, n_lo=1, n_hi=70),
    dataclasses.replace(W.TINY, name="ragged P5 T37 H136", P=5, E=20, k=3, T=37, H=136,
                        n_lo=0, n_hi=37),
    dataclasses.replace(W.TINY, name="P64 E64 epr1", P=64, E=64, k=8, T=9, H=64, n_lo=0, n_hi=9),
    dataclasses.replace(W.TINY, name="two-pass rows H8200", P=3, E=12, k=4, T=5, H=8200,
                        n_lo=1, n_hi=5),
    dataclasses.replace(W.EP8_MXFP8, name="mxfp8 small", T=33, H=96, n_lo=0, n_hi=33),
    dataclasses.replace(W.EP64_NVFP4, name="nvfp4 small", P=16, E=64, T=20, H=64, n_lo=3, n_hi=20),
    dataclasses.replace(W.TINY, name="many slots P16 T1500", P=16, E=64, k=4, T=1500, H=32,
                        n_lo=700, n_hi=1500),
    dataclasses.replace(W.TINY, name="k16", P=8, E=64, k=16, T=50, H=256, n_lo=0, n_hi=50),
    dataclasses.replace(W.TINY, name="k64 all experts", P=4, E=64, k=64, T=20, H=128, n_lo=0, n_hi=20),
    dataclasses.replace(W.TINY, name="bf16 H16384 two long chunks", P=4, E=16, k=3, T=6, H=16384,
                        n_lo=0, n_hi=6),
    dataclasses.replace(W.EP8_MXFP8, name="mxfp8 H8192 long rows", P=4, E=32, T=7, H=8192, n_lo=2, n_hi=7),
    dataclasses.replace(W.EP8_MXFP8, name="mxfp8 H16384 scale row 512B", P=3, E=12, k=4, T=5, H=16384,
                        n_lo=1, n_hi=5, routing="uniform"),
    dataclasses.replace(W.EP64_NVFP4, name="nvfp4 H4096 scale row 256B", P=8, E=32, T=9, H=4096,
                        n_lo=0, n_hi=9),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("seed", [11, 12])
def test_dispatch_small(w, seed):
    c = random_byte_case(w, seed, oob=(seed == 12), dup=(seed == 12))
    _run(c)


@pytest.mark.parametrize("k", [4, 8, 16])
def test_dispatch_ids_not_16_byte_aligned(k):
    # id / weight planes that start 4 bytes past a 16-byte boundary take the
    # word-wise id path; results must not change
    w = dataclasses.replace(W.TINY, name=f"unaligned k{k}", P=8, E=64, k=k, T=30, H=128, n_lo=0, n_hi=30)
    c = random_byte_case(w, 21, oob=True, dup=True)
    log(f"dispatch case: {w.name} with 4-byte-offset id and weight planes")
    pl, sc, ids, wt = gpu_inputs(c)
    n = ids.numel()
    ids_buf = torch.empty(n + 1, dtype=torch.int32, device=ids.device)
    wt_buf = torch.empty(n + 1, dtype=torch.float32, device=wt.device)
    ids_u = ids_buf[1:].view(ids.shape)
    wt_u = wt_buf[1:].view(wt.shape)
    ids_u.copy_(ids)
    wt_u.copy_(wt)
    assert ids_u.data_ptr() % 16 != 0 and wt_u.data_ptr() % 16 != 0
    ex = _exchange(w)
    out = ex.dispatch(pl, ids_u, wt_u, num_tokens=c.counts.tolist(), runtime_max_tokens_per_rank=w.T)
    _check(c, out)


def test_dispatch_without_weights_and_custom_marker():
    w = dataclasses.replace(W.TINY, name="noweights", T=40, n_lo=0, n_hi=40)
    c = random_byte_case(w, 5, oob=True)
    _run(c, invalid_id=-1, with_weights=False)


def test_dispatch_empty_ranks_and_T1():
    w = dataclasses.replace(W.TINY, name="empty", T=24, H=128)
    c = random_byte_case(w, 6, counts=[0, 24, 0, 3])
    _run(c)
    w1 = dataclasses.replace(W.TINY, name="T1", T=1, H=128)
    _run(random_byte_case(w1, 7, counts=[1, 0, 1, 1]))


def test_dispatch_and_combine_with_no_tokens():
    """Every rank sends nothing: every slot carries the marker, counts and
    offsets are zero, and combine writes no output row; a step after a
    full one must also clear that step's slots."""
    w = dataclasses.replace(W.TINY, name="no tokens", P=6, E=24, k=3, T=40, H=1024, n_lo=20, n_hi=40)
    ex = _run(random_byte_case(w, 31))
    _run(random_byte_case(w, 32, counts=[0] * w.P), ex=ex)
    out = torch.full((w.P, w.T, w.H), 3.0, dtype=torch.bfloat16, device="cuda")
    eo = W.draw_expert_output(w.P, w.T, w.H, 32, device="cuda")
    ex.combine(eo, out)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()), "combine wrote rows although no rank has tokens"


def test_dispatch_with_no_live_rank():
    """active_rank_mask = 0: nothing is sent or received, no region is
    written, and combine writes no output row."""
    w = dataclasses.replace(W.TINY, name="mask 0", T=16, H=256)
    c = random_byte_case(w, 33)
    ex = _exchange(w)
    pl, sc, ids, wt = gpu_inputs(c)
    ex.workspace.fill_(0x5A)
    before = ex.workspace.clone()
    ex.dispatch(pl, ids, wt, scales=sc, num_tokens=c.counts.tolist(), active_rank_mask=0)
    torch.cuda.synchronize()
    assert torch.equal(ex.workspace, before), "a masked-off region was written"
    out = torch.full((w.P, w.T, w.H), 3.0, dtype=torch.bfloat16, device="cuda")
    ex.combine(W.draw_expert_output(w.P, w.T, w.H, 33, device="cuda"), out)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()), "combine wrote rows of masked-off ranks"


def test_dispatch_stale_slots_are_remarked():
    """Two steps on one handle: the second has a smaller T, other counts
    and other routing; every slot of step 2 must reflect step 2 only."""
    w = dataclasses.replace(W.TINY, name="stale", T=64, H=256, n_lo=30, n_hi=64)
    ex = _run(random_byte_case(w, 21), T_cap=64)
    w2 = dataclasses.replace(w, T=48)
    _run(random_byte_case(w2, 22, counts=[48, 5, 0, 17]), ex=ex)
    # and a third step back at full size, mostly empty
    _run(random_byte_case(w, 23, counts=[1, 0, 2, 0]), ex=ex)


def test_dispatch_runtime_T_below_capacity():
    w = dataclasses.replace(W.EP8_BF16, name="T below cap", T=100, n_lo=10, n_hi=100, H=512)
    _run(random_byte_case(w, 31), T_cap=128)


def test_dispatch_full_ep8_bf16():
    _run(random_byte_case(W.EP8_BF16, W.EP8_BF16.seed))


def test_dispatch_full_ep8_mxfp8_zipf():
    _run(random_byte_case(W.EP8_MXFP8, W.EP8_MXFP8.seed))


# Long rows (8 KB and more) are stored write-through when the launch's
# payload writes are bounded by 256 MiB (N * min(P, k) * row) and
# non-temporally above; the row loads go before the mask in steps of at
# most 16384 (token, chunk) items.  These two cases take the combinations
# the other tests miss: a small step above the byte bound, and a large step
# (many slots) below it.
STORE_PATHS = [
    dataclasses.replace(W.TINY, name="long rows, small step, 315 MB of rows", P=8, E=64, k=8, T=300,
                        H=8192, n_lo=300, n_hi=300),
    dataclasses.replace(W.TINY, name="long rows, 16640 slots, few tokens", P=64, E=256, k=8, T=260,
                        H=4096, n_lo=0, n_hi=2),
]


@pytest.mark.parametrize("w", STORE_PATHS, ids=lambda w: w.name)
def test_dispatch_store_paths(w):
    c = random_byte_case(w, 41)
    ex = _run(c)
    ex.destroy()
    del ex
    torch.cuda.empty_cache()


def test_dispatch_is_deterministic():
    w = dataclasses.replace(W.EP8_BF16, name="determinism", H=1024)
    c = random_byte_case(w, 41)
    ex = _exchange(w)
    pl, sc, ids, wt = gpu_inputs(c)
    a = ex.dispatch(pl, ids, wt, num_tokens=c.counts.tolist())
    snap = {k: v.clone() for k, v in a.items() if isinstance(v, torch.Tensor)}
    b = ex.dispatch(pl, ids, wt, num_tokens=c.counts.tolist())
    for k, v in snap.items():
        # bit patterns: never-written slots may hold NaN bytes from earlier use
        assert torch.equal(v.view(torch.uint8), b[k].view(torch.uint8)), k


def test_dispatch_rejects_bad_steps():
    from combine_route_mask_amd import moe_ep
    w = dataclasses.replace(W.TINY, name="errors")
    c = random_byte_case(w, 51)
    ex = _exchange(w)
    pl, sc, ids, wt = gpu_inputs(c)
    with pytest.raises(moe_ep.MoeEpError) as e:
        moe_ep.moe_ep_dispatch(ex.handle, pl, None, ids, wt, c.counts.tolist(), w.T + 1)
    assert e.value.code == moe_ep.ERR_CAPACITY
    with pytest.raises(moe_ep.MoeEpArgError):
        moe_ep.moe_ep_dispatch(ex.handle, pl, None, ids, wt, [w.T + 1] + [0] * (w.P - 1), w.T)
    with pytest.raises(moe_ep.MoeEpArgError):
        moe_ep.moe_ep_dispatch(ex.handle, pl, None, ids, None, c.counts.tolist(), w.T)
    with pytest.raises(moe_ep.MoeEpArgError):
        moe_ep.moe_ep_dispatch(ex.handle, pl, pl, ids, wt, c.counts.tolist(), w.T)
    with pytest.raises(moe_ep.MoeEpError) as e:
        moe_ep.moe_ep_combine(ex.handle, pl, pl)
    assert e.value.code == moe_ep.ERR_BAD_STATE


def test_two_handles_on_two_streams():
    """Two exchanges with their own workspaces run concurrently on two side
    streams (one passed explicitly, one taken from the current stream);
    both match the oracle."""
    from combine_route_mask_amd.moe_ep import MoeEpExchange
    ws = [dataclasses.replace(W.EP8_BF16, name="stream a", T=48, H=1024, n_lo=0, n_hi=48),
          dataclasses.replace(W.TINY, name="stream b", P=6, E=24, k=5, T=33, H=520, n_lo=0, n_hi=33)]
    cases = [random_byte_case(w, 31 + i, oob=True, dup=True) for i, w in enumerate(ws)]
    log("two handles on two side streams")
    exs = [_exchange(w) for w in ws]
    ins = [gpu_inputs(c) for c in cases]
    eos = [W.draw_expert_output(w.P, w.T, w.H, 31 + i, device="cuda") for i, w in enumerate(ws)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    cur = torch.cuda.current_stream()
    outs, ys = [], []
    for i, (w, c, ex, (pl, sc, ids, wt), eo, st) in enumerate(zip(ws, cases, exs, ins, eos, streams)):
        st.wait_stream(cur)
        with torch.cuda.stream(st):
            if i == 0:
                outs.append(ex.dispatch(pl, ids, wt, scales=sc, num_tokens=c.counts.tolist(),
                                        runtime_max_tokens_per_rank=w.T, stream=st))
                ys.append(ex.combine(eo, stream=st))
            else:
                outs.append(ex.dispatch(pl, ids, wt, scales=sc, num_tokens=c.counts.tolist(),
                                        runtime_max_tokens_per_rank=w.T))
                ys.append(ex.combine(eo))
    torch.cuda.synchronize()
    for c, out in zip(cases, outs):
        _check(c, out)
    for w, c, eo, y in zip(ws, cases, eos, ys):
        o = oracle.combine_bf16(c.counts, c.ids, bits16(eo), E=w.E)
        yb = bits16(y)
        for s in range(w.P):
            n = int(c.counts[s])
            check_bf16_sum(yb[s, :n], o.ref[s, :n], o.y[s, :n], f"{w.name} source {s}")
