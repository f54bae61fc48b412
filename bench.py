"""Benchmark of the MoE expert-parallel exchange on one MI355X.

One step = one dispatch + one combine over all P virtual EP ranks of the
workload, inputs (token rows, ids, weights, expert outputs) resident in
HBM.  Prints one JSON line:

  value        tokens/s = N / step time (N = sum of local token counts)
  roofline     the dominant kernel's algorithmic bytes per launch / its
               average launch time (HIP events on the launch stream),
               against the MI355X HBM peak (8 TB/s)
  cpu_baseline the CPU oracle on a bounded sample of the same workload

Algorithmic bytes (per launch; N tokens, M (token, destination) pairs,
row / srow payload and scale row bytes, k, P ranks, T tokens per rank):
  dispatch  N*k*8 + N*(row+srow) + M*(row+srow+8k) + (P*P*T - M)*4k
  combine   bf16: M*2H + N*2H
            fp8:  quantise M*(2H + H + H/32), gather M*(H + H/32) + N*2H
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0

WORKLOADS = {
    "ep8": W.EP8_BF16,
    "ep8-mxfp8": W.EP8_MXFP8,
    "ep64": W.EP64_BF16,
    "ep64-nvfp4": W.EP64_NVFP4,
}


def pair_count(w, R) -> int:
    """M: distinct (token, destination rank) pairs, from the routing on the
    host (numpy; ids outside [0, E) route nowhere)."""
    M = 0
    epr = w.E // w.P
    for s in range(w.P):
        ids = R.ids[s, :R.counts[s]]
        own = np.where((ids >= 0) & (ids < w.E), ids // epr, -1)
        own = np.sort(own, axis=1)
        distinct = (own[:, 1:] != own[:, :-1]) & (own[:, 1:] >= 0)
        M += int(distinct.sum() + (own[:, 0] >= 0).sum())
    return M


def step_bytes(w, N, M):
    row = W.payload_row_bytes(w.fmt, w.H)
    srow = W.scale_row_bytes(w.fmt, w.H)
    k, P, T, H = w.k, w.P, w.T, w.H
    disp = N * k * 8 + N * (row + srow) + M * (row + srow + 8 * k) + (P * P * T - M) * 4 * k
    if w.combine == "fp8":
        quant = M * (2 * H + H + H // 32)
        gather = M * (H + H // 32) + N * 2 * H
        return {"dispatch": disp, "combine_quant": quant, "combine_gather": gather,
                "combine": quant + gather}
    return {"dispatch": disp, "combine": M * 2 * H + N * 2 * H}


class Setup:
    def __init__(self, w, seed=None):
        import torch
        from combine_route_mask_amd.moe_ep import MoeEpExchange
        self.w = w
        dev = torch.device("cuda")
        d = W.draw_dispatch_inputs(w, device=dev, seed=seed)
        self.R = d.routing
        self.payload = d.payload
        self.scales = d.scales
        self.ids = torch.from_numpy(self.R.ids).to(dev)
        self.weights = torch.from_numpy(self.R.weights).to(dev)
        del d
        self.eo = W.draw_expert_output(w.P, w.T, w.H, w.seed, device=dev)
        self.ex = MoeEpExchange(w.P, w.E, w.k, w.T, w.H, dispatch_format=w.fmt,
                                combine_format=w.combine, device=dev)
        self.out = torch.empty((w.P, w.T, w.H), dtype=torch.bfloat16, device=dev)
        self.counts = self.R.counts.tolist()
        self.N = int(self.R.counts.sum())
        self.M = pair_count(w, self.R)

    def dispatch(self):
        self.ex.dispatch(self.payload, self.ids, self.weights, scales=self.scales,
                         num_tokens=self.counts, runtime_max_tokens_per_rank=self.w.T)

    def combine(self):
        self.ex.combine(self.eo, self.out)

    def free(self):
        self.ex.destroy()
        del self.eo, self.payload, self.ex


def measure(setup, steps, warmup, flush_bytes=0):
    """Time `steps` dispatch+combine steps after `warmup` untimed ones.
    Events on the current stream (the one the kernels are launched on)
    bracket the whole timed region and every single launch."""
    import torch
    stream = torch.cuda.current_stream()
    flush = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda") if flush_bytes else None
    for _ in range(warmup):
        setup.dispatch()
        setup.combine()
    torch.cuda.synchronize()
    # the recv counts of the step must match the host-side pair count
    got_M = int(setup.ex.dispatch(setup.payload, setup.ids, setup.weights, scales=setup.scales,
                                  num_tokens=setup.counts,
                                  runtime_max_tokens_per_rank=setup.w.T)["counts"].sum().item())
    assert got_M == setup.M, (got_M, setup.M)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        if flush is not None:
            flush.fill_(i & 0xFF)  # untimed: evicts the 256 MB last-level cache
        ev[i][0].record(stream)
        setup.dispatch()
        ev[i][1].record(stream)
        setup.combine()
        ev[i][2].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_disp = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(steps)])
    t_comb = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in range(steps)])
    total_ms = start.elapsed_time(stop)
    step_ms = float((t_disp + t_comb).mean()) if flush is not None else total_ms / steps
    return {"ms_per_step": step_ms, "dispatch_ms": float(t_disp.mean()),
            "combine_ms": float(t_comb.mean()), "dispatch_ms_median": float(np.median(t_disp)),
            "combine_ms_median": float(np.median(t_comb)), "wall_s": wall}


def summarize(setup, m):
    w, N, M = setup.w, setup.N, setup.M
    b = step_bytes(w, N, M)
    step_s = m["ms_per_step"] / 1e3
    gbs = lambda nbytes, ms: nbytes / (ms / 1e3) / 1e9
    res = {
        "workload": w.name, "N_tokens": N, "M_pairs": M,
        "tokens_per_s": N / step_s,
        "ms_per_step": m["ms_per_step"],
        "step_bytes": b["dispatch"] + b["combine"],
        "step_GBps": (b["dispatch"] + b["combine"]) / step_s / 1e9,
        "dispatch_ms": m["dispatch_ms"], "combine_ms": m["combine_ms"],
        "dispatch_GBps": gbs(b["dispatch"], m["dispatch_ms"]),
        "combine_GBps": gbs(b["combine"], m["combine_ms"]),
    }
    res["step_frac_of_peak"] = res["step_GBps"] / HBM_PEAK_GBS
    return res, b


def cpu_baseline(w, budget_s=12.0):
    """The oracle (single-threaded C) on the same workload: whole dispatch
    + combine steps over every rank, repeated until ~budget_s of CPU work."""
    import torch
    import oracle
    d = W.draw_dispatch_inputs(w, device="cpu")
    R = d.routing
    payload = d.payload.numpy()
    scales = None if d.scales is None else d.scales.numpy()
    eo = W.draw_expert_output(w.P, w.T, w.H, w.seed, device="cpu").view(torch.int16).numpy().view(np.uint16)
    N = int(R.counts.sum())
    steps = 0
    t0 = time.perf_counter()
    while True:
        oracle.dispatch(R.counts, payload, R.ids, R.weights, scales, E=w.E)
        if w.combine == "fp8":
            oracle.combine_fp8(R.counts, R.ids, eo, E=w.E)
        else:
            oracle.combine_bf16(R.counts, R.ids, eo, E=w.E)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": N * steps / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} full dispatch+combine steps of '{w.name}' ({N} tokens each), "
                      f"single-threaded C oracle, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="ep8", choices=sorted(WORKLOADS))
    ap.add_argument("--also", default="ep64", help="comma list of extra workloads ('' for none)")
    ap.add_argument("--cold", action="store_true", help="flush the last-level cache between steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this exchange runs P virtual EP ranks on one GPU; "
                                   "--gpus above 1 is not supported"}))
        sys.exit(2)

    import torch
    from combine_route_mask_amd import moe_ep
    if not torch.cuda.is_available() or not moe_ep.moe_ep_is_supported():
        print(json.dumps({"error": "no gfx950 GPU visible"}))
        sys.exit(1)
    w = WORKLOADS[args.config]
    print(f"[bench] setting up {w.name}", file=sys.stderr, flush=True)
    setup = Setup(w)
    m = measure(setup, args.steps, args.warmup, flush_bytes=(1 << 30) if args.cold else 0)
    res, b = summarize(setup, m)
    setup.free()
    torch.cuda.empty_cache()
    print(f"[bench] {w.name}: {res['ms_per_step']*1e3:.1f} us/step", file=sys.stderr, flush=True)

    # dominant kernel: the longer of the two launches of a step
    if w.combine == "fp8":
        dom_name, dom_ms, dom_bytes = ("dispatch", m["dispatch_ms"], b["dispatch"]) \
            if m["dispatch_ms"] >= m["combine_ms"] else ("combine (quantise + gather)", m["combine_ms"], b["combine"])
    else:
        dom_name, dom_ms, dom_bytes = ("dispatch_kernel", m["dispatch_ms"], b["dispatch"]) \
            if m["dispatch_ms"] >= m["combine_ms"] else ("combine_bf16_kernel", m["combine_ms"], b["combine"])
    achieved = dom_bytes / (dom_ms / 1e3) / 1e9
    roofline = {"bound": "hbm", "kernel": dom_name, "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                "bytes_per_launch": dom_bytes, "launch_ms": dom_ms}

    also = []
    for name in [a for a in args.also.split(",") if a]:
        if name == args.config:
            continue
        wa = WORKLOADS[name]
        print(f"[bench] setting up {wa.name}", file=sys.stderr, flush=True)
        sa = Setup(wa)
        ma = measure(sa, max(10, args.steps // 2), max(3, args.warmup // 2))
        ra, _ = summarize(sa, ma)
        sa.free()
        del sa
        torch.cuda.empty_cache()
        print(f"[bench] {wa.name}: {ra['ms_per_step']*1e3:.1f} us/step", file=sys.stderr, flush=True)
        also.append(ra)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, args.cpu_budget)

    line = {
        "metric": "dispatch+combine tokens/s and achieved HBM GB/s (% peak), H=7168 bf16 top_k=8",
        "value": res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.fmt == "bf16" else w.fmt,
        "data": "synthetic (seeded routing and N(0,1) rows, see workloads/)",
        "config": {"workload": w.name, "P_virtual_ranks": w.P, "tokens_per_rank": w.T,
                   "hidden": w.H, "experts": w.E, "top_k": w.k, "dispatch_format": w.fmt,
                   "combine_format": w.combine, "cache": "cold" if args.cold else "warm"},
        "achieved_GBps": res["step_GBps"], "frac_of_peak": res["step_frac_of_peak"],
        "detail": res,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "also": also,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
