"""Benchmark of the MoE expert-parallel exchange on one MI355X.

One step = one dispatch + one combine over all P virtual EP ranks of the
workload, inputs (token rows, ids, weights, expert outputs) resident in
HBM.  The headline workload (default: P = 64, 512 tokens per rank, hidden
7168 bf16, 256 experts, top-8) runs cache-cold by default: every timed step
and every timed launch follows a 1 GiB write and a 1 GiB read of unrelated
buffers, so the 256 MB last-level cache holds none of its data, and each
step is timed alone with HIP events on the launch stream.  Warm runs replay
HIP graphs of ten consecutive steps (and one more for the remainder, so
that exactly the requested number of steps is timed).  Prints one JSON
line:

  value        tokens/s = N / step time (N = sum of local token counts)
  gate         the headline step's fraction of the HBM peak against 0.70
  roofline     the dominant kernel's algorithmic bytes per launch / its
               average launch time (HIP events on the launch stream: around
               each eager launch after the flush when cold, around graphs of
               20 back-to-back launches when warm), against the MI355X HBM
               peak (8 TB/s); traffic: HBM bytes per launch from the
               committed rocprofv3 counter summary, null when the kernel
               sources have changed since it was taken
  cpu_baseline the CPU oracle on a bounded sample of the same workload
  reference_kernels
               plain kernels moving the headline step's payload bytes in its
               patterns on its own buffers (scatter, gather-sum, the gather
               without stores, whole-buffer fill and read), timed like the
               step's launches: what its routing work costs over them
  also         the other workloads (--also), warm, or cold with a '-cold'
               suffix, each with its kernels' counted bytes per launch
               ("traffic", from the committed counter summaries, null where
               none matches the current source); by default EP64 warm, EP8 warm and cold, EP64 NVFP4,
               the MXFP8 workload with FP8 combine, EP64 DeepSeekFp8, EP64
               NVFP4 with 1 KB router logits per token and 256 EPLB
               statistics per rank, EP64 with 48 of 64 ranks taking part,
               and AgRs

Algorithmic bytes (per launch; N tokens of the ranks taking part, M
(token, destination) pairs between them, row / srow payload (with its extra
bytes) and scale row bytes, k, P ranks of which L take part, T tokens per
rank, n EPLB statistics per rank):
  dispatch  N*k*8 + N*(row+srow) + M*(row+srow+8k) + (L*P*T - M)*4k
            + L*n*4 + L*L*n*4
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


def traffic_summary_path(config: str) -> str:
    """Committed counter summary of a bench workload (profiles/)."""
    name = "ep8_bf16" if config == "ep8" else config.replace("-", "_")
    return os.path.join(ROOT, "profiles", f"pmc_traffic_{name}.txt")
# device sources of the kernels the counter summaries describe
SOURCE_NAMES = ("exchange.hip", "agrs.hip", "formats.h", "memory_ops.h", "moe_ep_internal.h")
KERNEL_SOURCES = [os.path.join(ROOT, "combine_route_mask_amd", "csrc", f) for f in SOURCE_NAMES]


# the benchmark's plain reference kernels (their own digest)
REFERENCE_SOURCES = [os.path.join(ROOT, "combine_route_mask_amd", "csrc", "ceilings.hip")]
REFERENCE_KERNELS = ("scatter_kernel", "gather_kernel", "fill_kernel", "read_kernel")


def source_digest(paths=None) -> str:
    """Digest of the device sources (default: the exchange's) with comments
    and blank space removed, so that editing a comment does not retire the
    counter summaries."""
    import hashlib
    import re
    h = hashlib.sha256()
    for path in (KERNEL_SOURCES if paths is None else paths):
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, config: str, instance=None):
    """HBM bytes per launch of `kernel` (or of one `instance`) on `workload`
    from the committed counter summary, or None when there is none or the
    kernel source has changed since the counters were taken."""
    try:
        rows = [json.loads(l) for l in open(traffic_summary_path(config)) if l.startswith("{")]
    except OSError:
        return None
    for r in rows:
        digest = source_digest(REFERENCE_SOURCES) if r.get("reference") else source_digest()
        if r.get("kernel") == kernel and r.get("workload") == workload and \
                (instance is None or r.get("instance") == instance) and r.get("source_digest") == digest:
            return r["hbm_bytes_per_launch"]
    return None


def step_traffic(w, config: str) -> dict:
    """Counted HBM bytes per launch of each kernel of a step of workload w
    from its committed counter summary (None where there is none or the
    source has changed since)."""
    if config == "agrs":
        kernels = {"allgatherv": "allgatherv_kernel", "reduce_scatterv": "reduce_scatterv_kernel"}
    elif w.combine == "fp8":
        kernels = {"dispatch": "dispatch_kernel", "combine_quant": "combine_fp8_quant_kernel",
                   "combine_gather": "combine_fp8_gather_kernel"}
    else:
        kernels = {"dispatch": "dispatch_kernel", "combine": "combine_bf16_kernel"}
    return {k: measured_traffic(kern, w.name, config) for k, kern in kernels.items()}


def pmc_summary(fetch_csv: str, write_csv: str, out_path: str, workload: str, config: str = "ep8"):
    """Per-launch HBM traffic from two counter runs (FETCH_SIZE, WRITE_SIZE;
    KiB per dispatch).  Each counter is scaled by what it reads for the
    calibration copy kernel of known size (2 GiB read + 2 GiB written)."""
    import csv
    import collections

    def load(path):
        per = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            key = name.split("(anonymous namespace)::")[-1].split("(")[0] \
                if "(anonymous namespace)::" in name else name
            per[(key, int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
        return per

    fetch, write = load(fetch_csv), load(write_csv)
    copy_kib = (2 << 30) / 1024
    cf = [v for (k, g), vs in fetch.items() if "copyBuffer" in k for v in vs if v > copy_kib / 4]
    cw = [v for (k, g), vs in write.items() if "copyBuffer" in k for v in vs if v > copy_kib / 2]
    f_scale = copy_kib / (sum(cf) / len(cf))
    w_scale = copy_kib / (sum(cw) / len(cw))
    lines = []
    family = ("allgatherv_kernel", "reduce_scatterv_kernel") if config == "agrs" else \
        ("dispatch_kernel", "combine_")
    for (k, g), vs in sorted(fetch.items()):
        # the reference kernels run on the headline workload's buffers; the
        # AgRs counter runs time AgRs as an extra workload of another headline
        ref = k.split("<")[0] in REFERENCE_KERNELS and config != "agrs"
        if not (k.startswith(family) or ref):
            continue
        wv = write.get((k, g), [0.0])
        fk, wk = sum(vs) / len(vs), sum(wv) / len(wv)
        row = {"kernel": k.split("<")[0], "instance": k, "workload": workload, "grid_threads": g,
               "fetch_KiB": round(fk, 1), "write_KiB": round(wk, 1),
               "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
               "hbm_bytes_per_launch": int(round((fk * f_scale + wk * w_scale) * 1024)),
               "launches": len(vs)}
        if ref:
            row["reference"] = True
        row["source_digest"] = source_digest(REFERENCE_SOURCES) if ref else source_digest()
        lines.append(json.dumps(row))
    cfg = f" --config {config}"
    if config == "agrs":  # the AgRs step runs as an extra workload of another one
        run = ("python3 <repo>/bench.py --config ep8 --cache warm --also agrs --no-cpu-baseline --no-graph "
               "--steps 3 --warmup 2")
    else:
        run = (f"python3 <repo>/bench.py{cfg} --also '' --no-cpu-baseline --no-graph "
               f"--steps {6 if config == 'ep8' else 3} --warmup 2")
    with open(out_path, "w") as f:
        f.write("# HBM traffic per launch from rocprofv3 counters (FETCH_SIZE, WRITE_SIZE in KiB per\n"
                "# dispatch), each scaled by its reading for a plain 2 GiB device copy\n"
                "# (calibration copy in bench.py: 2 GiB read, 2 GiB written).  Commands, run from /tmp\n"
                "# with TMPDIR=/tmp (<repo>: this repository, <out>: any output directory):\n"
                "#   rocprofv3 --pmc FETCH_SIZE -d <out>/pmc_fetch -o pmc --output-format csv -- \\\n"
                f"#       {run}\n"
                "#   rocprofv3 --pmc WRITE_SIZE -d <out>/pmc_write -o pmc --output-format csv -- \\\n"
                f"#       {run}\n"
                f"#   python3 <repo>/bench.py{cfg} --pmc-summary <out>/pmc_fetch/pmc_counter_collection.csv \\\n"
                "#       <out>/pmc_write/pmc_counter_collection.csv\n"
                "# source_digest: first 16 hex digits of the sha256 of combine_route_mask_amd/csrc/\n"
                f"# {', '.join(SOURCE_NAMES[:-1])} and {SOURCE_NAMES[-1]}, concatenated, with\n"
                "# comments and white space removed; rows marked \"reference\" are the bench's plain\n"
                "# reference kernels (run on the headline workload's buffers), digest of csrc/ceilings.hip\n")
        for l in lines:
            f.write(l + "\n")
    return lines

WORKLOADS = {
    "ep8": W.EP8_BF16,
    "ep8-mxfp8": W.EP8_MXFP8,
    "ep64": W.EP64_BF16,
    "ep64-nvfp4": W.EP64_NVFP4,
    "ep64-dsfp8": W.EP64_DSFP8,
    "ep64-nvfp4-extras": W.EP64_NVFP4_EXTRAS,
    "ep64-alive48": W.EP64_MASK48,
    "agrs": W.AGRS16,
}


def live_ranks(w) -> np.ndarray:
    """[P] bool: the ranks that take part in the step (all unless w.alive)."""
    live = np.zeros(w.P, bool)
    live[list(range(w.P)) if w.alive is None else list(w.alive)] = True
    return live


def live_tokens(w, R) -> int:
    """N: tokens of the ranks that take part (masked-off ranks send nothing)."""
    return int(np.asarray(R.counts)[live_ranks(w)].sum())


def pair_count(w, R) -> int:
    """M: distinct (token, destination rank) pairs, from the routing on the
    host (numpy; ids outside [0, E) route nowhere; only ranks that take part
    send and receive)."""
    M = 0
    epr = w.E // w.P
    live = live_ranks(w)
    for s in range(w.P):
        if not live[s]:
            continue
        ids = R.ids[s, :R.counts[s]]
        own = np.where((ids >= 0) & (ids < w.E), ids // epr, -1)
        own = np.where(live[np.clip(own, 0, w.P - 1)], own, -1)
        own = np.sort(own, axis=1)
        distinct = (own[:, 1:] != own[:, :-1]) & (own[:, 1:] >= 0)
        M += int(distinct.sum() + (own[:, 0] >= 0).sum())
    return M


def step_bytes(w, N, M):
    row = W.payload_row_bytes(w.fmt, w.H) + w.extra_bytes  # extra bytes travel with the row
    srow = W.scale_row_bytes(w.fmt, w.H)
    k, P, T, H = w.k, w.P, w.T, w.H
    L = int(live_ranks(w).sum())
    disp = N * k * 8 + N * (row + srow) + M * (row + srow + 8 * k) + (L * P * T - M) * 4 * k
    # EPLB statistics: each live rank's row read once, the live rows written to every live region
    disp += L * w.n_eplb * 4 + L * L * w.n_eplb * 4
    if w.combine == "fp8":
        quant = M * (2 * H + H + H // 32)
        gather = M * (H + H // 32) + N * 2 * H
        return {"dispatch": disp, "combine_quant": quant, "combine_gather": gather,
                "combine": quant + gather}
    return {"dispatch": disp, "combine": M * 2 * H + N * 2 * H}


class Setup:
    """Inputs of one workload resident on the GPU, a handle, and the two
    launches of a step through the raw C ABI (pointers precomputed, so the
    host adds only a ctypes call per launch)."""

    def __init__(self, w, seed=None):
        import ctypes as C
        import torch
        from combine_route_mask_amd import moe_ep
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
        self.extra, self.stats = W.draw_extras(w, device=dev, seed=seed)
        self.ex = MoeEpExchange(w.P, w.E, w.k, w.T, w.H, dispatch_format=w.fmt,
                                combine_format=w.combine, extra_payload_bytes_per_token=w.extra_bytes,
                                eplb_stats_num_experts=w.n_eplb, device=dev)
        self.out = torch.empty((w.P, w.T, w.H), dtype=torch.bfloat16, device=dev)
        self.counts = self.R.counts.tolist()
        self.N = live_tokens(w, self.R)
        self.M = pair_count(w, self.R)
        mask = None if w.alive is None else sum(1 << r for r in w.alive)
        # first step through the checked binding (sets up the views)
        self.views = self.ex.dispatch(self.payload, self.ids, self.weights, scales=self.scales,
                                      num_tokens=self.counts, runtime_max_tokens_per_rank=w.T,
                                      active_rank_mask=mask, extra_payload=self.extra,
                                      eplb_local_stats=self.stats)
        self.ex.combine(self.eo, self.out)
        self._lib = moe_ep.lib
        self._h = self.ex.handle
        ptr = lambda t: C.c_void_p(t.data_ptr()) if t is not None else None
        self._mask = None if mask is None else (C.c_uint64 * 1)(mask)
        self._args = (ptr(self.payload), ptr(self.scales), ptr(self.extra), ptr(self.stats),
                      ptr(self.ids), ptr(self.weights),
                      (C.c_int32 * w.P)(*self.counts), C.c_int32(w.T), self._mask)
        self._eo = C.c_void_p(self.eo.data_ptr())
        self._out = C.c_void_p(self.out.data_ptr())

    def dispatch(self):
        import torch
        st = torch.cuda.current_stream().cuda_stream
        rc = self._lib.moe_ep_dispatch(self._h, *self._args, st, None)
        if rc:
            raise RuntimeError(self._lib.moe_ep_last_error().decode())

    def combine(self):
        import torch
        st = torch.cuda.current_stream().cuda_stream
        rc = self._lib.moe_ep_combine(self._h, self._eo, self._out, st)
        if rc:
            raise RuntimeError(self._lib.moe_ep_last_error().decode())

    def free(self):
        self.ex.destroy()
        del self.eo, self.payload, self.ex, self.views, self.extra, self.stats


class AgRsSetup:
    """All-gatherv of [hidden, topk_weights, topk_ids] then reduce-scatterv of
    the hidden partials over P virtual ranks, through the raw C ABI."""

    def __init__(self, w):
        import ctypes as C
        import torch
        from combine_route_mask_amd import moe_ep
        self.w = w
        d = W.draw_agrs_inputs(w, device="cuda")
        self.sizes = d.sizes
        total = int(d.sizes.sum())
        self.N = total
        self.hidden = d.hidden
        self.wts = torch.from_numpy(d.weights).cuda()
        self.ids_t = torch.from_numpy(d.ids).cuda()
        self.outs = [torch.empty((w.P, total, w.H), dtype=torch.bfloat16, device="cuda"),
                     torch.empty((w.P, total, w.k), dtype=torch.float32, device="cuda"),
                     torch.empty((w.P, total, w.k), dtype=torch.int32, device="cuda")]
        self.part = d.partial.contiguous()
        self.rs_out = torch.empty((w.P, int(d.sizes.max()), w.H), dtype=torch.bfloat16, device="cuda")
        # one checked call of each through the binding, then raw pointers
        moe_ep.allgatherv(self.sizes.tolist(), [self.hidden, self.wts, self.ids_t], self.outs)
        moe_ep.reduce_scatterv(self.sizes.tolist(), self.part, self.rs_out)
        planes = []
        for x, o in zip([self.hidden, self.wts, self.ids_t], self.outs):
            planes.append(moe_ep.Plane(x.data_ptr(), x.stride(0) * x.element_size(), o.data_ptr(),
                                       o.stride(0) * o.element_size(), x[0, 0].numel() * x.element_size()))
        self._lib = moe_ep.lib
        self._planes = (moe_ep.Plane * 3)(*planes)
        self._sizes = (C.c_int32 * w.P)(*self.sizes.tolist())
        self._rs = (C.c_void_p(self.part.data_ptr()), C.c_int64(self.part.stride(0) * 2),
                    C.c_void_p(self.rs_out.data_ptr()), C.c_int64(self.rs_out.stride(0) * 2))
        rowb = w.H * 2 + 8 * w.k
        self.bytes = {"allgatherv": total * rowb * (1 + w.P), "reduce_scatterv": total * 2 * w.H * (w.P + 1)}

    def dispatch(self):
        import torch
        st = torch.cuda.current_stream().cuda_stream
        if self._lib.moe_ep_allgatherv(self.w.P, self._sizes, 3, self._planes, st):
            raise RuntimeError(self._lib.moe_ep_last_error().decode())

    def combine(self):
        import torch
        st = torch.cuda.current_stream().cuda_stream
        if self._lib.moe_ep_reduce_scatterv(self.w.P, self._sizes, self.w.H, *self._rs, st):
            raise RuntimeError(self._lib.moe_ep_last_error().decode())

    def free(self):
        del self.hidden, self.outs, self.part, self.rs_out


def _graph(fn, reps=1):
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm the stream once outside capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for _ in range(reps):
                fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def _time(fn, iters):
    import torch
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(iters):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b)


class _Flush:
    """Evicts the last-level cache: writes nbytes of one scratch buffer,
    then reads nbytes of another, so the cache ends up holding clean lines
    of unrelated data (no dirty write-backs land in the timed region)."""

    def __init__(self, nbytes):
        import torch
        self.w = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.r = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
        self.i = 0

    def __call__(self):
        self.i += 1
        self.w.fill_(self.i & 0xFF)
        self.sink = self.r.max()


def measure(setup, steps, warmup, flush_bytes=0, graphs=True, check=True):
    """Step time of `steps` dispatch+combine steps after `warmup` untimed
    ones, eager (two C-ABI launches per step) and from HIP-graph replays of
    10 steps each (plus one graph of the remaining steps when `steps` is not
    a multiple of 10, so exactly `steps` steps are timed); per-launch kernel
    times from graphs of 20 back-to-back
    launches of one kernel.  With flush_bytes, every timed step and every
    timed single launch follows a write and a read of that many bytes
    (last-level cache cold and clean) and is timed alone.  All events sit on the launch stream."""
    import torch

    def step():
        setup.dispatch()
        setup.combine()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    exchange = isinstance(setup, Setup) and check
    if exchange:
        # the step's receive counts (regions that take part; the others are
        # never written) must match the host-side pair count
        live = torch.from_numpy(live_ranks(setup.w)).to(setup.views["counts"].device)
        got_M = int(setup.views["counts"][live].sum().item())
        assert got_M == setup.M, (got_M, setup.M)
        ref_out = setup.out.clone()
        ref_ids = setup.views["ids"].clone()

    eager_ms = _time(step, steps) / steps
    if not graphs:
        return {"ms_per_step": eager_ms, "eager_ms_per_step": eager_ms,
                "dispatch_ms": _time(setup.dispatch, steps) / steps,
                "combine_ms": _time(setup.combine, steps) / steps, "wall_s": 0.0}
    # one graph holds `per` consecutive steps, so a small step is not bound
    # by the host's graph-launch rate; a second graph holds the remainder
    per = min(10, steps)
    full, rem = divmod(steps, per)
    g_step = _graph(step, per)
    g_rem = _graph(step, rem) if rem else None

    def timed_steps():
        for _ in range(full):
            g_step.replay()
        if g_rem is not None:
            g_rem.replay()

    for _ in range(max(1, warmup // per)):
        g_step.replay()
    wall0 = time.perf_counter()
    if flush_bytes:
        # cold: a 1 GiB write, then a 1 GiB read of another buffer, between
        # steps (untimed) evicts the last-level cache
        flush = _Flush(flush_bytes)
        stream = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        # eager launches: the host enqueues them while the flush still runs
        for i in range(steps):
            flush()
            ev[i][0].record(stream)
            step()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        graph_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        del flush
    else:
        graph_ms = _time(timed_steps, 1) / steps
    wall = time.perf_counter() - wall0
    # graph replays must reproduce the eager step bit for bit
    if exchange:
        assert torch.equal(setup.out.view(torch.int16), ref_out.view(torch.int16))
        assert torch.equal(setup.views["ids"], ref_ids)

    if flush_bytes:
        # cold per-kernel times: the same fill before each single launch
        flush = _Flush(flush_bytes)
        stream = torch.cuda.current_stream()
        per_kernel = []
        for fn in (setup.dispatch, setup.combine):
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
            for i in range(steps):
                flush()
                ev[i][0].record(stream)
                fn()
                ev[i][1].record(stream)
            torch.cuda.synchronize()
            per_kernel.append(float(np.mean([a.elapsed_time(b) for a, b in ev])))
        del flush, g_step, g_rem
        return {"ms_per_step": graph_ms, "eager_ms_per_step": eager_ms, "dispatch_ms": per_kernel[0],
                "combine_ms": per_kernel[1], "wall_s": wall}
    reps = 20
    g_d = _graph(setup.dispatch, reps)
    g_c = _graph(setup.combine, reps)
    g_d.replay()
    g_c.replay()
    it = max(2, steps // reps)
    disp_ms = _time(g_d.replay, it) / (it * reps)
    comb_ms = _time(g_c.replay, it) / (it * reps)
    del g_step, g_rem, g_d, g_c
    return {"ms_per_step": graph_ms, "eager_ms_per_step": eager_ms, "dispatch_ms": disp_ms,
            "combine_ms": comb_ms, "wall_s": wall}


CEILINGS_LIB = os.path.join(ROOT, "combine_route_mask_amd", "libmoe_ep_ceilings.so")


def destination_masks(w, R) -> np.ndarray:
    """[P*T] uint64, entry s*T + t: bit r set when token t of rank s has an
    expert on rank r (contiguous ownership, E/P experts per rank; ids outside
    [0, E) route nowhere) and both ranks take part; 0 for rows t >= n_s.
    Popcounts sum to M."""
    assert w.P <= 64
    epr = w.E // w.P
    live = live_ranks(w)
    ids = R.ids.astype(np.int64)
    owner = np.where((ids >= 0) & (ids < w.E), ids, 0) // epr
    valid = (ids >= 0) & (ids < w.E) & live[owner]
    bits = np.where(valid, np.left_shift(np.uint64(1), owner.astype(np.uint64)), np.uint64(0))
    m = np.bitwise_or.reduce(bits, axis=2)
    m[np.arange(w.T)[None, :] >= np.asarray(R.counts)[:, None]] = 0
    m[~live] = 0
    return m.reshape(-1)


def load_ceilings(path: str = CEILINGS_LIB):
    import ctypes as C
    lib = C.CDLL(path)
    vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int32
    lib.ceil_scatter.argtypes = [vp, i64, i64, vp, i64, i32, vp, i64, i64, vp]
    lib.ceil_gather.argtypes = [vp, i64, i32, vp, i64, i64, vp, i64, i32, vp]
    lib.ceil_fill.argtypes = [vp, i64, vp]
    lib.ceil_read.argtypes = [vp, i64, vp, i64, vp]
    for f in (lib.ceil_scatter, lib.ceil_gather, lib.ceil_fill, lib.ceil_read):
        f.restype = C.c_int
    return lib


def reference_kernels(setup, m, reps=5, flush_bytes=0, config=None):
    """Plain reference kernels (libmoe_ep_ceilings.so) on the step's own
    buffers, each launch timed alone with HIP events on the launch stream
    (after the cache flush when flush_bytes): the dispatch's payload scatter
    into the workspace's receive planes, the BF16 combine's gather-sum from
    the expert outputs into the output (and the same with no output stores),
    a fill of the whole workspace and a read of the whole expert-output
    buffer.  They move the exchange's bytes in its patterns with none of its
    routing work, so exchange / reference time is what that work costs on
    these allocations.  BF16 dispatch and combine only; run after the step's
    own checks (the gather leaves truncated sums in the output).  With
    config, each kernel's HBM bytes per launch from that workload's counter
    summary ("traffic", null when none matches the current source)."""
    import ctypes as C
    import torch
    w = setup.w
    if w.fmt != "bf16" or w.combine != "bf16" or w.P > 64 or w.extra_bytes or w.n_eplb:
        return None
    try:
        lib = load_ceilings()
    except OSError as e:
        return {"error": f"reference kernels not built: {e}"}
    st = torch.cuda.current_stream()
    sp = C.c_void_p(st.cuda_stream)
    masks = torch.from_numpy(destination_masks(w, setup.R).view(np.int64)).cuda()
    row = 2 * w.H
    ntok = w.P * w.T
    ex = setup.ex
    ws, spr = ex.workspace, ex.size_per_rank
    pay = setup.views["payload"]
    pay_off = pay.data_ptr() - ws.data_ptr()
    sink = torch.empty(256 * 8 * 8, dtype=torch.int32, device="cuda")
    N, M = setup.N, setup.M
    eo_bytes = setup.eo.numel() * 2
    runs = {
        "scatter": (lambda: lib.ceil_scatter(setup.payload.data_ptr(), setup.payload.numel() * 2, row,
                                             masks.data_ptr(), ntok, w.P, pay.data_ptr(), spr,
                                             ws.numel() - pay_off, sp), (N + M) * row),
        "gather": (lambda: lib.ceil_gather(setup.eo.data_ptr(), ntok * row, w.P, masks.data_ptr(), ntok,
                                           row, setup.out.data_ptr(), setup.out.numel() * 2, 1, sp),
                   (M + N) * row),
        "gather_reads_only": (lambda: lib.ceil_gather(setup.eo.data_ptr(), ntok * row, w.P, masks.data_ptr(),
                                                      ntok, row, setup.out.data_ptr(), setup.out.numel() * 2,
                                                      0, sp), M * row),
        "fill_workspace": (lambda: lib.ceil_fill(ws.data_ptr(), ws.numel(), sp), ws.numel()),
        "read_expert_output": (lambda: lib.ceil_read(setup.eo.data_ptr(), eo_bytes, sink.data_ptr(),
                                                     sink.numel(), sp), eo_bytes),
    }
    assert setup.eo.shape == (w.P, ntok, w.H) and setup.out.shape == (w.P, w.T, w.H)
    assert setup.payload.is_contiguous() and setup.eo.is_contiguous() and setup.out.is_contiguous()
    assert pay.stride(0) == spr and pay.stride(1) == row and pay_off + ntok * row <= spr
    flush = _Flush(flush_bytes) if flush_bytes else None
    res = {}
    for name, (fn, nbytes) in runs.items():
        if fn():  # untimed first launch (checks the arguments)
            raise RuntimeError(f"reference kernel {name}: bad arguments")
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            if flush is not None:
                flush()
            a.record(st)
            fn()
            b.record(st)
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        res[name] = {"us": ms * 1e3, "bytes": int(nbytes), "GBps": nbytes / (ms / 1e3) / 1e9}
        inst = {"scatter": "scatter_kernel", "gather": "gather_kernel<true>",
                "gather_reads_only": "gather_kernel<false>", "fill_workspace": "fill_kernel",
                "read_expert_output": "read_kernel"}[name]
        if config:
            res[name]["traffic"] = measured_traffic(inst.split("<")[0], w.name, config, instance=inst)
    del flush
    res["dispatch_over_scatter"] = m["dispatch_ms"] * 1e3 / res["scatter"]["us"]
    res["combine_over_gather"] = m["combine_ms"] * 1e3 / res["gather"]["us"]
    res["what"] = ("plain kernels on the step's own buffers, each launch timed alone"
                   + (" after the cache flush" if flush_bytes else "") +
                   ": scatter = payload rows read once and stored at their slot of every destination "
                   "rank's receive plane (N + M rows), gather = per-token sum of its M rows of "
                   "expert output plus the N output rows, gather_reads_only = the same with the sum "
                   "kept only on a pattern match (no output stores)")
    return res


def trace_summary(trace_csv: str, workloads: list) -> str:
    """Markdown table of per-launch exchange-kernel durations from a
    rocprofv3 kernel-trace CSV of a bench run, grouped by workload (a new
    workload starts at the first random-input kernel after exchange
    kernels have run), kernel instance, grid, cache state and context.  A
    launch that follows a 1 GiB cache flush counts as cold.  Context "step":
    a kernel of the other side of the exchange (dispatch side: dispatch,
    all-gatherv; combine side: the combine kernels, reduce-scatterv) ran
    since this instance's previous launch, as in the step graphs; "alone":
    none did, as in the per-kernel graphs whose launch times the bench
    reports.  The plain reference kernels (scatter_kernel, gather_kernel,
    fill_kernel, read_kernel) get context "reference" and leave the others'
    contexts alone.  The first launch of an instance in a workload is left
    out (warm-up)."""
    import collections
    import csv
    import re
    import statistics
    ours = ("dispatch_kernel", "combine_bf16_kernel", "combine_fp8_quant_kernel",
            "combine_fp8_gather_kernel", "allgatherv_kernel", "reduce_scatterv_kernel")
    dispatch_side = ("dispatch_kernel", "allgatherv_kernel")
    reference = ("scatter_kernel", "gather_kernel", "fill_kernel", "read_kernel")
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    phase, ran, after_flush, seen = 0, False, False, set()
    sides_since = collections.defaultdict(set)  # instance -> sides launched since its last launch
    groups = collections.defaultdict(list)
    for r in rows:
        name = r["Kernel_Name"]
        if "normal_kernel" in name and ran:
            phase, ran = phase + 1, False
            continue
        if "FillFunctor<unsigned char>" in name and int(r["Grid_Size_X"]) >= (1 << 26):
            after_flush = True
            continue
        m = re.search(r"(\w+_kernel(<[^(]*>)?)\(", name)
        if not m or m.group(1).split("<")[0] not in ours + reference:
            continue
        inst, cold, after_flush = m.group(1), after_flush, False
        if inst.split("<")[0] in reference:
            if (phase, inst) not in seen:
                seen.add((phase, inst))
                continue
            wg = int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"])
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            groups[(phase, inst, wg, "cold" if cold else "warm", "reference")].append(dur)
            continue
        ran = True
        side = "dispatch" if inst.startswith(dispatch_side) else "combine"
        ctx = "step" if (sides_since[inst] - {side}) else "alone"
        sides_since[inst] = set()
        for other in sides_since:
            if other != inst:
                sides_since[other].add(side)
        if (phase, inst) not in seen:
            seen.add((phase, inst))
            continue
        wg = int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"])
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups[(phase, inst, wg, "cold" if cold else "warm", ctx)].append(dur)
    out = ["| workload | kernel | workgroups | cache | context | launches | mean us | median us | min us |",
           "|---|---|---|---|---|---|---|---|---|"]
    for (ph, inst, wg, c, ctx), d in sorted(groups.items()):
        label = workloads[ph] if ph < len(workloads) else str(ph)
        out.append(f"| {label} | `{inst}` | {wg} | {c} | {ctx} | {len(d)} | {statistics.mean(d):.1f} | "
                   f"{statistics.median(d):.1f} | {min(d):.1f} |")
    return "\n".join(out) + "\n"


def pmc_table(counter_csv: str, workloads: list) -> str:
    """Markdown table of per-launch counter means from a rocprofv3 counter
    run of the bench (any counters), grouped like trace_summary: workload
    phase, exchange or reference kernel instance, cache state (a launch
    after a 1 GiB flush is cold); the first launch of an instance in a
    workload is left out; "mean us" from the dispatches' timestamps.  With
    TCC_EA0_WRREQ_sum, the ratios of TCC_EA0_WRREQ_STALL_sum (stalled cycles
    per write request) and of TCC_EA0_WRREQ_LEVEL_sum (requests in flight
    summed per cycle: the mean write latency in cycles) to it are added; with
    TCP_TCC_WRITE_REQ_sum, the mean L1-to-L2 write latency
    (TCP_TCC_WRITE_REQ_LATENCY_sum / TCP_TCC_WRITE_REQ_sum); with
    GRBM_GUI_ACTIVE, the busy fraction of the second-level translation cache
    (GRBM_UTCL2_BUSY / GRBM_GUI_ACTIVE)."""
    import collections
    import csv
    import re
    ours = ("dispatch_kernel", "combine_bf16_kernel", "combine_fp8_quant_kernel",
            "combine_fp8_gather_kernel", "allgatherv_kernel", "reduce_scatterv_kernel") + REFERENCE_KERNELS
    disp = collections.OrderedDict()
    for r in csv.DictReader(open(counter_csv)):
        d = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "grid": int(r["Grid_Size"]),
                                                    "c": {}})
        if r.get("End_Timestamp") and r.get("Start_Timestamp"):
            d["us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    counters = sorted({k for d in disp.values() for k in d["c"]})
    phase, ran, after_flush, seen = 0, False, False, set()
    groups = collections.defaultdict(list)
    for _, d in sorted(disp.items()):
        name = d["name"]
        if "normal_kernel" in name and ran:
            phase, ran = phase + 1, False
            continue
        if "FillFunctor<unsigned char>" in name and d["grid"] >= (1 << 26):
            after_flush = True
            continue
        m = re.search(r"(\w+_kernel(<[^(]*>)?)\(", name)
        if not m or m.group(1).split("<")[0] not in ours:
            continue
        inst, cold, after_flush = m.group(1), after_flush, False
        if inst.split("<")[0] not in REFERENCE_KERNELS:
            ran = True
        if (phase, inst) not in seen:
            seen.add((phase, inst))
            continue
        groups[(phase, inst, "cold" if cold else "warm")].append(dict(d["c"], _us=d.get("us", 0.0)))
    extra = []
    if "TCC_EA0_WRREQ_sum" in counters:
        extra = [x for x in ("TCC_EA0_WRREQ_STALL_sum", "TCC_EA0_WRREQ_LEVEL_sum") if x in counters]
    if "TCP_TCC_WRITE_REQ_sum" in counters and "TCP_TCC_WRITE_REQ_LATENCY_sum" in counters:
        extra.append("TCP_TCC_WRITE_REQ_LATENCY_sum")
    ratio_to = {x: ("TCP_TCC_WRITE_REQ_sum" if x.startswith("TCP_") else "TCC_EA0_WRREQ_sum") for x in extra}
    if "GRBM_UTCL2_BUSY" in counters and "GRBM_GUI_ACTIVE" in counters:
        extra.append("GRBM_UTCL2_BUSY")
        ratio_to["GRBM_UTCL2_BUSY"] = "GRBM_GUI_ACTIVE"
    head = ["workload", "kernel", "cache", "launches", "mean us"] + counters + \
        [f"{x} / {ratio_to[x]}" for x in extra]
    out = ["| " + " | ".join(head) + " |", "|" + "---|" * len(head)]
    for (ph, inst, c), ds in sorted(groups.items()):
        label = workloads[ph] if ph < len(workloads) else str(ph)
        mean = {k: sum(d.get(k, 0.0) for d in ds) / len(ds) for k in counters + ["_us"]}
        cells = [label, f"`{inst}`", c, str(len(ds)), f"{mean['_us']:.1f}"] + [f"{mean[k]:.4g}" for k in counters]
        cells += [f"{mean[x] / mean[ratio_to[x]]:.3g}" if mean[ratio_to[x]] else "-" for x in extra]
        out.append("| " + " | ".join(cells) + " |")
    return "\n".join(out) + "\n"


def calibrate(nbytes=2 << 30, iters=10):
    """Achievable HBM bandwidth on this GPU: a plain device copy (read +
    write, torch copy_) and a fill (write only) of nbytes."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    ms_copy = _time(lambda: dst.copy_(src), iters) / iters
    ms_fill = _time(lambda: dst.fill_(3), iters) / iters
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_GBps": 2 * nbytes / (ms_copy / 1e3) / 1e9,
            "fill_GBps": nbytes / (ms_fill / 1e3) / 1e9, "bytes": nbytes}


def summarize(setup, m):
    if isinstance(setup, AgRsSetup):
        b = setup.bytes
        tot = b["allgatherv"] + b["reduce_scatterv"]
        step_s = m["ms_per_step"] / 1e3
        res = {"workload": setup.w.name, "rows": setup.N, "rows_per_s": setup.N / step_s,
               "ms_per_step": m["ms_per_step"], "eager_ms_per_step": m["eager_ms_per_step"],
               "step_bytes": tot, "step_GBps": tot / step_s / 1e9,
               "allgatherv_ms": m["dispatch_ms"], "reduce_scatterv_ms": m["combine_ms"],
               "allgatherv_GBps": b["allgatherv"] / (m["dispatch_ms"] / 1e3) / 1e9,
               "reduce_scatterv_GBps": b["reduce_scatterv"] / (m["combine_ms"] / 1e3) / 1e9}
        res["step_frac_of_peak"] = res["step_GBps"] / HBM_PEAK_GBS
        return res, b
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
        "eager_ms_per_step": m["eager_ms_per_step"],
        "dispatch_ms": m["dispatch_ms"], "combine_ms": m["combine_ms"],
        "dispatch_GBps": gbs(b["dispatch"], m["dispatch_ms"]),
        "combine_GBps": gbs(b["combine"], m["combine_ms"]),
    }
    res["step_frac_of_peak"] = res["step_GBps"] / HBM_PEAK_GBS
    return res, b


def cpu_baseline(w, budget_s=12.0):
    """The oracle (single-threaded C) on the same workload.  A whole step of
    the large workloads is minutes of CPU time (and its receive planes tens
    of GB of host memory), so the oracle takes the step in its own units:
    one destination rank's dispatch (every receive plane of that rank) and
    one source rank's combine (every token of that rank), alternating over
    ranks until ~budget_s of CPU work; the step time is P times the mean
    of each, and tokens/s = N / step time.  The combine of a source reads
    that source's slots of every rank's expert output (one N(0,1) slice,
    reused: the oracle's speed does not depend on the values)."""
    import torch
    import oracle
    d = W.draw_dispatch_inputs(w, device="cpu")
    R = d.routing
    payload = d.payload.numpy()
    scales = None if d.scales is None else d.scales.numpy()
    N = live_tokens(w, R)
    P, T = w.P, w.T
    active = None if w.alive is None else sum(1 << r for r in w.alive)
    extra, _ = W.draw_extras(w, device="cpu")
    extra = None if extra is None else extra.numpy()
    g = W.torch_generator(w.seed + 7, "cpu")
    eo_s = W.normal_bf16((P, T, w.H), g, "cpu").view(torch.int16).numpy().view(np.uint16)
    t_disp, t_comb = [], []
    i = 0
    while sum(t_disp) + sum(t_comb) < budget_s or not (t_disp and t_comb):
        r = (i * 37) % P  # spread the sampled ranks
        a = time.perf_counter()
        oracle.dispatch(R.counts, payload, R.ids, R.weights, scales, E=w.E, r0=r, r1=r + 1, active=active,
                        extra=extra)
        t_disp.append(time.perf_counter() - a)
        a = time.perf_counter()
        if w.combine == "fp8":
            oracle.combine_fp8(R.counts, R.ids, eo_s, E=w.E, s0=r, s1=r + 1, slot0=r * T, active=active)
        else:
            oracle.combine_bf16(R.counts, R.ids, eo_s, E=w.E, s0=r, s1=r + 1, slot0=r * T, active=active)
        t_comb.append(time.perf_counter() - a)
        i += 1
    el = sum(t_disp) + sum(t_comb)
    step_s = P * (float(np.mean(t_disp)) + float(np.mean(t_comb)))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
    except OSError:
        pass
    b = step_bytes(w, N, pair_count(w, R))
    return {"value": N / step_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "GBps": (b["dispatch"] + b["combine"]) / step_s / 1e9,
            "step_s": step_s,
            "sample": f"'{w.name}': {len(t_disp)} one-destination dispatches (every receive plane of "
                      f"that rank) and {len(t_comb)} one-source combines (every token of that rank) of "
                      f"the single-threaded C oracle, {el:.1f} s of CPU time; step = {P} x (mean "
                      f"dispatch + mean combine) = {step_s:.1f} s for {N} tokens",
            "host": {"cpu": model, "nproc": os.cpu_count(),
                     "usable_cpus": len(os.sched_getaffinity(0))}}


def also_plan(args) -> dict:
    """Workloads of --also in first-mention order, each with the cache
    states (False warm, True cold: a '-cold' suffix) to run on its one set
    of buffers; the primary workload in its own state is left out."""
    plan = {}
    primary_cold = args.cache == "cold"
    for name in [a for a in args.also.split(",") if a]:
        cold = name.endswith("-cold")
        base = name[:-5] if cold else name
        if base == args.config and cold == primary_cold:
            continue
        if cold not in plan.setdefault(base, []):
            plan[base].append(cold)
    return plan


# Fraction of the HBM peak the path is held to (dispatch + combine step time).
GATE_FRAC = 0.70


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="ep64", choices=sorted(WORKLOADS),
                    help="workload of the headline line (default: P=64, T=512, H=7168 bf16, top-8)")
    ap.add_argument("--cache", default="cold", choices=("cold", "warm"),
                    help="cold (default): write 1 GiB and read another 1 GiB before every timed step and "
                         "launch of the headline workload, so the last-level cache holds none of its data")
    ap.add_argument("--also", default="ep64,ep8,ep8-cold,ep64-nvfp4,ep8-mxfp8,ep64-dsfp8,ep64-nvfp4-extras,"
                                      "ep64-alive48,agrs",
                    help="comma list of extra workloads ('' for none), warm unless suffixed '-cold'")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (for counter-collection runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-reference-kernels", action="store_true",
                    help="skip the plain reference kernels on the headline buffers")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="print the per-workload kernel-duration table of a rocprofv3 kernel trace "
                         "of this bench (same --config / --cache / --also) and exit")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the counter traffic summary under profiles/ and exit")
    ap.add_argument("--pmc-table", metavar="COUNTER_CSV",
                    help="print the per-workload counter table of a rocprofv3 counter run of this bench "
                         "(same --config / --cache / --also) and exit")
    args = ap.parse_args()
    cold = args.cache == "cold"
    if args.trace_summary:
        labels = [args.config + ("-cold" if cold else "")]
        for base, colds in also_plan(args).items():
            labels.append(base if False in colds else base + "-cold")
        print(trace_summary(args.trace_summary, labels), end="")
        return
    if args.pmc_table:
        labels = [args.config + ("-cold" if cold else "")]
        for base, colds in also_plan(args).items():
            labels.append(base if False in colds else base + "-cold")
        print(pmc_table(args.pmc_table, labels), end="")
        return
    if args.pmc_summary:
        for l in pmc_summary(*args.pmc_summary, traffic_summary_path(args.config),
                             WORKLOADS[args.config].name, args.config):
            print(l)
        return
    if args.steps < 1 or args.warmup < 0:
        print(json.dumps({"error": "--steps must be >= 1 and --warmup >= 0"}))
        sys.exit(2)
    if args.gpus != 1:
        print(json.dumps({"error": "this exchange runs P virtual EP ranks on one GPU; "
                                   "--gpus above 1 is not supported"}))
        sys.exit(2)
    if args.config == "agrs":
        print(json.dumps({"error": "the AgRs step runs as an extra workload: --also agrs"}))
        sys.exit(2)

    import torch
    from combine_route_mask_amd import moe_ep
    if not torch.cuda.is_available() or not moe_ep.moe_ep_is_supported():
        print(json.dumps({"error": "no gfx950 GPU visible"}))
        sys.exit(1)
    w = WORKLOADS[args.config]
    print("[bench] device copy / fill bandwidth (context only)", file=sys.stderr, flush=True)
    calib = calibrate()
    print(f"[bench] setting up {w.name} ({args.cache})", file=sys.stderr, flush=True)
    setup = Setup(w)
    m = measure(setup, args.steps, args.warmup, flush_bytes=(1 << 30) if cold else 0,
                graphs=not args.no_graph)
    res, b = summarize(setup, m)
    res["traffic"] = step_traffic(w, args.config)
    ref_kernels = None
    if not args.no_reference_kernels:
        print(f"[bench] reference kernels on the {w.name} buffers", file=sys.stderr, flush=True)
        ref_kernels = reference_kernels(setup, m, flush_bytes=(1 << 30) if cold else 0, config=args.config)
    setup.free()
    torch.cuda.empty_cache()
    print(f"[bench] {w.name} ({args.cache}): {res['ms_per_step']*1e3:.1f} us/step", file=sys.stderr, flush=True)

    # dominant kernel: the longer of the two launches of a step
    if w.combine == "fp8":
        dom_name, dom_ms, dom_bytes = ("dispatch_kernel", m["dispatch_ms"], b["dispatch"]) \
            if m["dispatch_ms"] >= m["combine_ms"] else ("combine (quantise + gather)", m["combine_ms"], b["combine"])
    else:
        dom_name, dom_ms, dom_bytes = ("dispatch_kernel", m["dispatch_ms"], b["dispatch"]) \
            if m["dispatch_ms"] >= m["combine_ms"] else ("combine_bf16_kernel", m["combine_ms"], b["combine"])
    achieved = dom_bytes / (dom_ms / 1e3) / 1e9
    traffic = measured_traffic(dom_name, w.name, args.config)
    roofline = {"bound": "hbm", "kernel": dom_name, "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                "bytes_per_launch": dom_bytes, "launch_ms": dom_ms,
                "launch_timing": ("HIP events on the launch stream around each eager launch, each after a "
                                  "1 GiB write + 1 GiB read (cache cold)") if cold else
                                 ("HIP events on the launch stream around graphs of 20 back-to-back launches")}

    # the other workloads; warm and cold runs of one workload share its
    # buffers, so the two differ only in what the cache holds
    also = []
    for base, colds in also_plan(args).items():
        wa = WORKLOADS[base]
        print(f"[bench] setting up {wa.name}", file=sys.stderr, flush=True)
        sa = AgRsSetup(wa) if base == "agrs" else Setup(wa)
        for c in colds:
            ma = measure(sa, max(10, args.steps // 2), max(3, args.warmup // 2),
                         flush_bytes=(1 << 30) if c else 0, graphs=not args.no_graph)
            ra, _ = summarize(sa, ma)
            ra["cache"] = "cold" if c else "warm"
            ra["traffic"] = step_traffic(wa, base)
            if not c and base in ("ep8", "ep8-mxfp8"):
                ra["note"] = ("warm: the step's inputs partly stay in the 256 MB last-level cache "
                              "between steps, so this is not an HBM-bound figure")
            print(f"[bench] {wa.name} ({ra['cache']}): {ra['ms_per_step']*1e3:.1f} us/step",
                  file=sys.stderr, flush=True)
            also.append(ra)
        sa.free()
        del sa
        torch.cuda.empty_cache()

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
                   "combine_format": w.combine, "cache": args.cache},
        "achieved_GBps": res["step_GBps"], "frac_of_peak": res["step_frac_of_peak"],
        "gate": {"workload": w.name, "cache": args.cache, "target_frac_of_peak": GATE_FRAC,
                 "frac_of_peak": res["step_frac_of_peak"], "met": res["step_frac_of_peak"] >= GATE_FRAC},
        "detail": res,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "reference_kernels": ref_kernels,
        "device_copy_context": {"torch_copy_GBps": calib["copy_GBps"], "torch_fill_GBps": calib["fill_GBps"],
                                "bytes": calib["bytes"],
                                "what": "torch copy_ (read + write counted) and fill_ of 2 GiB on this GPU"},
        "also": also,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
