"""The benchmark's plain reference kernels (libmoe_ep_ceilings.so) compute
what the bench says they do, on the EP8 workload (P = 8, T = 128, H = 7168
bf16, top-8): the row scatter leaves exactly the dispatch's payload planes
(every token row at its slot of every destination in its mask, nothing
elsewhere), the gather-sum gives the oracle's fp32 ascending-rank sums
truncated to bf16 and leaves rows with an empty mask alone, the gather
without stores leaves the output alone, the fill writes its pattern.  Their
times are only meaningful if they move those bytes."""
import numpy as np
import pytest
import torch

import bench
import oracle
import workloads as W
from tests.gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ep8():
    from combine_route_mask_amd import moe_ep
    assert torch.cuda.is_available() and moe_ep.moe_ep_is_supported()
    w = bench.WORKLOADS["ep8"]
    st = bench.Setup(w)
    lib = bench.load_ceilings()
    yield w, st, lib
    st.free()
    torch.cuda.empty_cache()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def test_scatter_matches_the_dispatch_payload_planes(ep8):
    w, st, lib = ep8
    P, S, row = w.P, w.P * w.T, 2 * w.H
    masks = bench.destination_masks(w, st.R)
    mk = torch.from_numpy(masks.view(np.int64)).cuda()
    spr = st.ex.size_per_rank
    pay = st.views["payload"]
    off = pay.data_ptr() - st.ex.workspace.data_ptr()
    base = torch.zeros((P, spr), dtype=torch.uint8, device="cuda")
    rc = lib.ceil_scatter(st.payload.data_ptr(), st.payload.numel() * 2, row, mk.data_ptr(), S, P,
                          base.data_ptr() + off, spr, base.numel() - off, _stream())
    assert rc == 0
    torch.cuda.synchronize()
    got = base[:, off:off + S * row].view(P, S, row)
    bits = ((mk.view(torch.int64)[None, :] >> torch.arange(P, device="cuda")[:, None]) & 1).bool()  # [P, S]
    src = st.payload.view(torch.uint8).view(1, S, row)
    want = torch.where(bits[..., None], src, torch.zeros((), dtype=torch.uint8, device="cuda"))
    assert torch.equal(got, want)
    # the same bytes as the exchange's own receive planes on every sent slot
    assert torch.equal(got[bits], pay[bits])
    log(f"reference scatter: {int(bits.sum())} rows placed, {P * S - int(bits.sum())} slots untouched")


def test_gather_is_the_truncated_fp32_oracle_sum(ep8):
    w, st, lib = ep8
    P, T, S, row = w.P, w.T, w.P * w.T, 2 * w.H
    masks = bench.destination_masks(w, st.R)
    mk = torch.from_numpy(masks.view(np.int64)).cuda()
    out = torch.full((P, T, w.H), -1, dtype=torch.int16, device="cuda")  # 0xFFFF: a NaN pattern
    rc = lib.ceil_gather(st.eo.data_ptr(), S * row, P, mk.data_ptr(), S, row, out.data_ptr(),
                         out.numel() * 2, 1, _stream())
    assert rc == 0
    torch.cuda.synchronize()
    eo = st.eo.view(torch.int16).cpu().numpy().view(np.uint16)
    o = oracle.combine_bf16(st.R.counts, st.R.ids, eo, E=w.E)
    want = (o.ref.view(np.uint32) >> 16).astype(np.uint16)
    got = out.cpu().numpy().view(np.uint16)
    live = masks.reshape(P, T) != 0
    assert np.array_equal(got[live], want[live])
    assert (got[~live] == 0xFFFF).all()
    # without stores the output stays as it was
    out.fill_(-1)
    rc = lib.ceil_gather(st.eo.data_ptr(), S * row, P, mk.data_ptr(), S, row, out.data_ptr(),
                         out.numel() * 2, 0, _stream())
    assert rc == 0
    torch.cuda.synchronize()
    assert (out.cpu().numpy().view(np.uint16) == 0xFFFF).all()
    log(f"reference gather: {int(live.sum())} rows equal the truncated oracle sums")


def test_fill_and_read(ep8):
    _, _, lib = ep8
    buf = torch.zeros((1 << 20) + 16, dtype=torch.uint8, device="cuda")
    assert lib.ceil_fill(buf.data_ptr(), buf.numel(), _stream()) == 0
    sink = torch.zeros(256 * 8 * 8, dtype=torch.int32, device="cuda")
    assert lib.ceil_read(buf.data_ptr(), buf.numel(), sink.data_ptr(), sink.numel(), _stream()) == 0
    torch.cuda.synchronize()
    assert (buf.view(torch.int16) == 0x3F80).all()
    assert int(sink.abs().sum()) == 0  # the fill's words xor to 0, never the sink pattern


def test_bench_reference_kernels_report(ep8):
    w, st, _ = ep8
    m = {"dispatch_ms": 0.02, "combine_ms": 0.02}
    r = bench.reference_kernels(st, m, reps=2)
    for k in ("scatter", "gather", "gather_reads_only", "fill_workspace", "read_expert_output"):
        assert r[k]["us"] > 0 and r[k]["bytes"] > 0 and r[k]["GBps"] > 0, k
    assert r["scatter"]["bytes"] == (st.N + st.M) * 2 * w.H
    assert r["gather_reads_only"]["bytes"] == st.M * 2 * w.H
    log("reference kernels (EP8, warm): " + ", ".join(f"{k} {r[k]['us']:.1f} us" for k in
                                                      ("scatter", "gather", "gather_reads_only")))
