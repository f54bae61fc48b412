"""The bench's profile post-processing on small synthetic rocprofv3 CSVs:
the kernel-trace table (workload phases, cold launches, launch context,
warm-up launch left out) and the counter summary (scaled by the calibration
copy)."""
import csv
import json

import bench

TRACE_COLS = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id",
              "Kernel_Name", "Correlation_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size",
              "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X",
              "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]

DISPATCH = "void moe_ep::(anonymous namespace)::dispatch_kernel<2, 4, true>(moe_ep::DispatchArgs, long, long, long)"
COMBINE = "void moe_ep::(anonymous namespace)::combine_bf16_kernel<1, 8, true>(moe_ep::CombineArgs, long)"
NORMAL = "void at::native::distribution_elementwise_grid_stride_kernel<float, 4, normal_kernel>(int)"
FLUSH = "void at::native::vectorized_elementwise_kernel<16, at::native::FillFunctor<unsigned char>, x>(int)"


def _trace(path, kernels):
    t = 0
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=TRACE_COLS)
        w.writeheader()
        for name, grid, dur in kernels:
            row = {c: 0 for c in TRACE_COLS}
            row.update(Kernel_Name=name, Start_Timestamp=t, End_Timestamp=t + dur,
                       Workgroup_Size_X=256, Grid_Size_X=grid)
            w.writerow(row)
            t += dur + 1000


def test_trace_summary_phases_and_cold(tmp_path):
    p = tmp_path / "trace.csv"
    _trace(p, [
        (NORMAL, 2048 * 256, 500),
        (DISPATCH, 1036 * 256, 99000),      # first launch of the phase: left out
        (DISPATCH, 1036 * 256, 12000),
        (DISPATCH, 1036 * 256, 14000),
        (COMBINE, 4096 * 256, 13000),
        (NORMAL, 2048 * 256, 500),          # second workload starts
        (DISPATCH, 1036 * 256, 50000),      # warm-up, left out
        (FLUSH, 1 << 26, 100000),
        (DISPATCH, 1036 * 256, 20000),      # after a flush: cold
        (DISPATCH, 1036 * 256, 12000),
    ])
    lines = bench.trace_summary(str(p), ["first", "second"]).splitlines()
    rows = [l.split("|")[1:-1] for l in lines[2:]]
    rows = [[c.strip() for c in r] for r in rows]
    assert ["first", "`dispatch_kernel<2, 4, true>`", "1036", "warm", "alone", "2", "13.0", "13.0", "12.0"] in rows
    assert ["second", "`dispatch_kernel<2, 4, true>`", "1036", "cold", "alone", "1", "20.0", "20.0", "20.0"] in rows
    assert ["second", "`dispatch_kernel<2, 4, true>`", "1036", "warm", "alone", "1", "12.0", "12.0", "12.0"] in rows
    assert not any(r[1].startswith("`combine") and r[0] == "first" for r in rows)


def test_trace_summary_context(tmp_path):
    """Launches alternating with the other side of the exchange are "step",
    back-to-back launches of one kernel "alone"."""
    p = tmp_path / "trace.csv"
    D, C = (DISPATCH, 1036 * 256), (COMBINE, 4096 * 256)
    _trace(p, [(NORMAL, 2048 * 256, 500), (*D, 90000), (*C, 90000),   # warm-up launches
               (*D, 10000), (*C, 20000), (*D, 11000), (*C, 21000),     # step graph
               (*D, 30000), (*D, 31000), (*C, 40000), (*C, 41000)])    # per-kernel graphs
    lines = bench.trace_summary(str(p), ["wl"]).splitlines()
    rows = [[c.strip() for c in l.split("|")[1:-1]] for l in lines[2:]]
    got = {(r[1].split("<")[0].strip("`"), r[4]): (r[5], r[6]) for r in rows}
    assert got == {("dispatch_kernel", "step"): ("3", "17.0"), ("dispatch_kernel", "alone"): ("1", "31.0"),
                   ("combine_bf16_kernel", "step"): ("3", "27.0"),
                   ("combine_bf16_kernel", "alone"): ("1", "41.0")}


def test_trace_summary_reference_kernels(tmp_path):
    """The plain reference kernels get their own "reference" rows and do not
    change the exchange kernels' contexts."""
    p = tmp_path / "trace.csv"
    D, C = (DISPATCH, 1036 * 256), (COMBINE, 4096 * 256)
    SC = ("void (anonymous namespace)::scatter_kernel(unsigned char const*, long, unsigned long const*, "
          "unsigned long, long, unsigned char*, long)", 32768 * 256)
    GA = ("void (anonymous namespace)::gather_kernel<true>(unsigned char const*, long, unsigned long const*, "
          "unsigned long, long, long, unsigned char*)", 229376 * 256)
    _trace(p, [(NORMAL, 2048 * 256, 500), (*D, 90000), (*D, 10000), (*D, 12000),
               (*SC, 99000), (FLUSH, 1 << 26, 100000), (*SC, 30000),
               (FLUSH, 1 << 26, 100000), (*SC, 32000), (*GA, 99000), (*GA, 25000),
               (*D, 14000)])
    lines = bench.trace_summary(str(p), ["wl"]).splitlines()
    rows = [[c.strip() for c in l.split("|")[1:-1]] for l in lines[2:]]
    got = {(r[1].strip("`"), r[3], r[4]): (r[2], r[5], r[6]) for r in rows}
    assert got == {("dispatch_kernel<2, 4, true>", "warm", "alone"): ("1036", "3", "12.0"),
                   ("scatter_kernel", "cold", "reference"): ("32768", "2", "31.0"),
                   ("gather_kernel<true>", "warm", "reference"): ("229376", "1", "25.0")}


def _pmc(path, entries):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Value"])
        w.writeheader()
        for name, grid, val in entries:
            w.writerow({"Kernel_Name": name, "Grid_Size": grid, "Counter_Value": val})


def test_pmc_summary_scales_by_the_copy(tmp_path):
    copy_kib = (2 << 30) / 1024
    fetch, write, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "out.txt"
    # the counters read half the copy's fetched bytes and all of its written bytes
    _pmc(fetch, [("__amd_rocclr_copyBuffer", 256, copy_kib / 2), (COMBINE, 1048576, 1000.0),
                 (COMBINE, 1048576, 1200.0)])
    _pmc(write, [("__amd_rocclr_copyBuffer", 256, copy_kib), (COMBINE, 1048576, 300.0),
                 (COMBINE, 1048576, 300.0)])
    lines = bench.pmc_summary(str(fetch), str(write), str(out), "wl")
    assert len(lines) == 1
    r = json.loads(lines[0])
    assert r["kernel"] == "combine_bf16_kernel" and r["fetch_scale"] == 2.0 and r["write_scale"] == 1.0
    assert r["hbm_bytes_per_launch"] == int(round((1100.0 * 2 + 300.0) * 1024))
    assert r["source_digest"] == bench.source_digest()
    assert open(out).read().count("\n{") == 1


def test_pmc_summary_reference_kernels(tmp_path, monkeypatch):
    """Reference-kernel rows carry their own source digest and are found by
    kernel instance; an exchange row with the same grid is not confused with
    them."""
    copy_kib = (2 << 30) / 1024
    fetch, write, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "out.txt"
    SC = ("void (anonymous namespace)::scatter_kernel(unsigned char const*, long, unsigned long const*, "
          "unsigned long, long, unsigned char*, long)")
    GT = ("void (anonymous namespace)::gather_kernel<true>(unsigned char const*, long, unsigned long const*, "
          "unsigned long, long, long, unsigned char*)")
    _pmc(fetch, [("__amd_rocclr_copyBuffer", 256, copy_kib / 2), (SC, 8388608, 100.0), (GT, 8388608, 400.0),
                 (COMBINE, 8388608, 500.0)])
    _pmc(write, [("__amd_rocclr_copyBuffer", 256, copy_kib), (SC, 8388608, 800.0), (GT, 8388608, 50.0),
                 (COMBINE, 8388608, 60.0)])
    lines = [json.loads(l) for l in bench.pmc_summary(str(fetch), str(write), str(out), "wl")]
    by = {r["instance"]: r for r in lines}
    assert set(by) == {"scatter_kernel", "gather_kernel<true>", "combine_bf16_kernel<1, 8, true>"}
    assert by["scatter_kernel"]["reference"] and by["gather_kernel<true>"]["reference"]
    assert "reference" not in by["combine_bf16_kernel<1, 8, true>"]
    assert by["scatter_kernel"]["source_digest"] == bench.source_digest(bench.REFERENCE_SOURCES)
    assert by["combine_bf16_kernel<1, 8, true>"]["source_digest"] == bench.source_digest()
    assert by["scatter_kernel"]["hbm_bytes_per_launch"] == int(round((100.0 * 2 + 800.0) * 1024))
    monkeypatch.setattr(bench, "traffic_summary_path", lambda config: str(out))
    assert bench.measured_traffic("gather_kernel", "wl", "x", instance="gather_kernel<true>") == \
        int(round((400.0 * 2 + 50.0) * 1024))
    assert bench.measured_traffic("gather_kernel", "wl", "x", instance="gather_kernel<false>") is None
    assert bench.measured_traffic("combine_bf16_kernel", "wl", "x") == int(round((500.0 * 2 + 60.0) * 1024))


def test_pmc_table_phases_and_ratios(tmp_path):
    """Counter rows of one dispatch are merged; workloads split at the first
    random-input kernel after exchange kernels; the reference kernels do not
    start a workload; cold after a flush; ratios to the write requests."""
    p = tmp_path / "ctr.csv"
    cols = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"]
    SC = ("void (anonymous namespace)::scatter_kernel(unsigned char const*, long, unsigned long const*, "
          "unsigned long, long, unsigned char*, long)")
    seq = [(NORMAL, 1), (DISPATCH, 1), (FLUSH, 1 << 26), (DISPATCH, 1), (FLUSH, 1 << 26), (DISPATCH, 1),
           (SC, 1), (SC, 1), (NORMAL, 1), (DISPATCH, 1), (DISPATCH, 1)]
    vals = {1: (10, 5, 40), 3: (100, 50, 400), 5: (100, 150, 600), 6: (7, 7, 7), 7: (80, 8, 160),
            9: (1, 1, 1), 10: (20, 10, 60)}
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for i, (name, grid) in enumerate(seq):
            wr, st, lv = vals.get(i, (0, 0, 0))
            for cn, cv in (("TCC_EA0_WRREQ_sum", wr), ("TCC_EA0_WRREQ_STALL_sum", st),
                           ("TCC_EA0_WRREQ_LEVEL_sum", lv)):
                w.writerow({"Dispatch_Id": i + 1, "Grid_Size": grid * 256, "Kernel_Name": name,
                            "Counter_Name": cn, "Counter_Value": cv})
    lines = bench.pmc_table(str(p), ["first", "second"]).splitlines()
    head = [c.strip() for c in lines[0].split("|")[1:-1]]
    assert head[-2:] == ["TCC_EA0_WRREQ_STALL_sum / TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_LEVEL_sum / TCC_EA0_WRREQ_sum"]
    rows = {(r[0], r[1].strip("`"), r[2]): r for r in
            ([c.strip() for c in l.split("|")[1:-1]] for l in lines[2:])}
    # first workload: dispatches 3 and 5 (cold; 1 is its warm-up), scatter 7 (warm; 6 is its warm-up);
    # second: dispatch 10 (9 is its warm-up)
    d = rows[("first", "dispatch_kernel<2, 4, true>", "cold")]
    assert d[3] == "2" and d[-2] == "1" and d[-1] == "5" and d[4] == "0.0"
    sc = rows[("first", "scatter_kernel", "warm")]
    assert sc[3] == "1" and sc[-2] == "0.1" and sc[-1] == "2"
    d2 = rows[("second", "dispatch_kernel<2, 4, true>", "warm")]
    assert d2[3] == "1" and d2[-2] == "0.5" and d2[-1] == "3"


def test_step_traffic_per_kernel(tmp_path, monkeypatch):
    """Each kernel of a step gets its counted bytes from the workload's
    summary; a kernel without a row (or with a stale digest) gets None."""
    out = tmp_path / "s.txt"
    rows = [{"kernel": "dispatch_kernel", "instance": "dispatch_kernel<2, 4, false, false, false>", "workload": "wl",
             "hbm_bytes_per_launch": 11, "source_digest": bench.source_digest()},
            {"kernel": "combine_bf16_kernel", "instance": "combine_bf16_kernel<128, 1, 4, false, true>",
             "workload": "wl", "hbm_bytes_per_launch": 22, "source_digest": "stale"},
            {"kernel": "combine_fp8_quant_kernel", "instance": "q", "workload": "wl", "hbm_bytes_per_launch": 33,
             "source_digest": bench.source_digest()}]
    out.write_text("# header\n" + "\n".join(json.dumps(r) for r in rows) + "\n")
    monkeypatch.setattr(bench, "traffic_summary_path", lambda config: str(out))
    import dataclasses
    w = dataclasses.replace(bench.WORKLOADS["ep8"], name="wl")
    assert bench.step_traffic(w, "x") == {"dispatch": 11, "combine": None}
    wf = dataclasses.replace(bench.WORKLOADS["ep8-mxfp8"], name="wl")
    assert bench.step_traffic(wf, "x") == {"dispatch": 11, "combine_quant": 33, "combine_gather": None}
    assert set(bench.step_traffic(bench.WORKLOADS["agrs"], "agrs")) == {"allgatherv", "reduce_scatterv"}


def test_also_plan_cache_states():
    """--also entries are warm unless suffixed '-cold'; the headline in its own
    cache state is not repeated; warm and cold runs of one workload share one
    entry (one set of buffers)."""
    import argparse
    a = argparse.Namespace(config="ep64", cache="cold", also="ep64,ep64-cold,ep8,ep8-cold,agrs,ep8")
    assert bench.also_plan(a) == {"ep64": [False], "ep8": [False, True], "agrs": [False]}
    a = argparse.Namespace(config="ep8", cache="warm", also="ep8,ep8-cold,ep64-cold")
    assert bench.also_plan(a) == {"ep8": [True], "ep64": [True]}
    assert bench.also_plan(argparse.Namespace(config="ep64", cache="cold", also="")) == {}


def test_step_bytes_of_the_headline_workload():
    """The EP64 headline's algorithmic bytes (the dispatch formula with N
    tokens, M pairs, 14336-byte rows, k = 8): the roofline's bytes per launch."""
    import workloads as W
    w = W.EP64_BF16
    N, M = 32768, 251630
    b = bench.step_bytes(w, N, M)
    row, k, P, T = 14336, 8, 64, 512
    assert b["dispatch"] == N * k * 8 + N * row + M * (row + 8 * k) + (P * P * T - M) * 4 * k == 4154387904
    assert b["combine"] == M * 2 * 7168 + N * 2 * 7168


def test_destination_masks_count_the_pairs():
    """One bit per (token, destination rank) pair: popcounts add up to the
    host pair count M, inactive rows and out-of-range ids set no bit."""
    import numpy as np
    import workloads as W
    w = bench.WORKLOADS["ep64"]
    R = W.draw_routing(w)
    m = bench.destination_masks(w, R)
    assert m.shape == (w.P * w.T,) and m.dtype == np.uint64
    assert sum(bin(int(x)).count("1") for x in m) == bench.pair_count(w, R) == 251630
    rows = m.reshape(w.P, w.T)
    for s in (0, 17, 63):
        assert not rows[s, R.counts[s]:].any()
    # hand case: P = 4 ranks of 2 experts, k = 3
    import dataclasses
    w4 = dataclasses.replace(bench.WORKLOADS["ep8"], P=4, T=2, E=8, k=3)
    R4 = W.Routing(np.array([2, 1, 1, 0], dtype=np.int32),
                   np.array([[[0, 1, 7], [2, 9, -1]], [[3, 2, 4], [5, 5, 5]],
                             [[6, 7, 0], [1, 1, 1]], [[8, 8, 8], [0, 0, 0]]], dtype=np.int32),
                   np.zeros((4, 2, 3), np.float32))
    got = bench.destination_masks(w4, R4).tolist()
    assert got == [0b1001, 0b0010, 0b0110, 0, 0b1001, 0, 0, 0]


def test_reference_kernels_reject_bad_sizes():
    """The plain reference kernels check sizes on the host and return -1
    before any launch (no GPU needed)."""
    import ctypes as C
    import os
    if not os.path.exists(bench.CEILINGS_LIB):
        from combine_route_mask_amd import build
        build.build()
    lib = bench.load_ceilings()
    p = 4096  # never dereferenced: every call below fails its host checks
    row = 14336
    # source smaller than ntok rows
    assert lib.ceil_scatter(p, row * 3, row, p, 4, 2, p, row * 4, row * 8, None) == -1
    # destination: (nregions - 1) * region + ntok * row beyond the base
    assert lib.ceil_scatter(p, row * 4, row, p, 4, 2, p, row * 4, row * 8 - 1, None) == -1
    # rows the scatter cannot hold in its four vectors per lane, or ragged
    assert lib.ceil_scatter(p, 1 << 30, 16400, p, 4, 2, p, 1 << 30, 1 << 31, None) == -1
    assert lib.ceil_scatter(p, 1 << 30, row + 8, p, 4, 2, p, 1 << 30, 1 << 31, None) == -1
    assert lib.ceil_scatter(p, row * 4, row, p, 4, 65, p, row * 4, 1 << 31, None) == -1
    assert lib.ceil_scatter(None, row * 4, row, p, 4, 2, p, row * 4, row * 8, None) == -1
    # gather: plane or output smaller than ntok rows, too many planes
    assert lib.ceil_gather(p, row * 3, 2, p, 4, row, p, row * 4, 1, None) == -1
    assert lib.ceil_gather(p, row * 4, 2, p, 4, row, p, row * 4 - 16, 1, None) == -1
    assert lib.ceil_gather(p, row * 4, 65, p, 4, row, p, row * 4, 1, None) == -1
    assert lib.ceil_gather(p, row * 4, 2, None, 4, row, p, row * 4, 1, None) == -1
    # sweeps: too small, or a sink with fewer words than workgroups
    assert lib.ceil_fill(p, 8, None) == -1
    assert lib.ceil_read(p, 1 << 20, p, 16383, None) == -1
    assert lib.ceil_read(p, 1 << 20, None, 16384, None) == -1
