"""GPU parity on seeded random configurations: every combination of the
options the exchange takes, each case small, checked against the oracle
to the same bars as the targeted tests: dispatch bit-exact; BF16 combine
within 2^-7 |ref| + 1e-3 of the oracle's fp32 sum over ranks and equal to
its bf16 result bit for bit (row magnitudes span 2^-20..2^20, so fp32
rounding shows); FP8 landing planes and result bit-exact, and the result
within 0.07 sum|terms| (plus half an e4m3 subnormal step per term) of the
exact sum of the bf16 terms, the elements outside the literal bound being
counted and logged.

Drawn per case: P in 1..64, experts per rank 1..8 (E % 4 == 0), top_k up
to 16 with duplicate and out-of-range ids, T and per-rank counts, the
dispatch format (BF16 / MXFP8 / NVFP4 / DeepSeekFp8) and combine format,
hidden sizes that leave ragged 256-lane chunks (and, in 24 more cases,
rows of 1024..14336 elements for every combine workgroup shape), weights
present or not,
the invalid expert id, an active rank mask, extra payload bytes and EPLB
statistics.  Masked-off regions and output rows must stay untouched."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import (bf16_bits_to_f64, bits16, check_bf16_sum, check_fp8_sum, fp8_terms_and_floor, gpu_inputs,
                            log, random_byte_case)

pytestmark = pytest.mark.gpu


@dataclasses.dataclass(frozen=True)
class Case:
    w: W.Workload
    has_weights: bool
    invalid_id: int
    alive: tuple
    extra_bytes: int
    n_eplb: int

    @property
    def name(self):
        w = self.w
        return (f"P{w.P}-E{w.E}-k{w.k}-T{w.T}-H{w.H}-{w.fmt}-{w.combine}"
                f"{'' if self.has_weights else '-noweights'}"
                f"{'-mask' if len(self.alive) < w.P else ''}"
                f"{f'-x{self.extra_bytes}' if self.extra_bytes else ''}"
                f"{f'-eplb{self.n_eplb}' if self.n_eplb else ''}-s{w.seed}")


def _cases(n=120, seed=20261202, wide=False):
    """wide: few ranks and tokens but rows of 1024..14336 elements, so the
    combine kernels take every workgroup shape they choose by row width."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        P = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 24, 32, 48, 64] if not wide else [1, 2, 3, 4, 6, 8]))
        E = P * int(rng.choice([1, 2, 3, 4, 5, 8]))
        if E % 4:
            continue
        k = int(rng.integers(1, min(E, 12) + 1)) if rng.random() < 0.85 else min(E, 16)
        T = int(rng.integers(1, 41)) if P <= 16 and not wide else int(rng.integers(1, 9))
        fmt = str(rng.choice(["bf16", "bf16", "mxfp8", "nvfp4", "deepseek_fp8"]))
        comb = "fp8" if rng.random() < (0.3 if not wide else 0.6) else "bf16"
        quantum = {"bf16": 8, "mxfp8": 32, "nvfp4": 32, "deepseek_fp8": 128}[fmt]
        if comb == "fp8":
            quantum = max(quantum, 32)
        if wide:
            H = int(rng.choice([1024, 2048, 3072, 5120, 7168, 8192, 14336, 7168 + 1024]))
        else:
            H = quantum * int(rng.integers(1, max(2, 720 // quantum) + 1))
        alive = tuple(range(P))
        if P > 1 and rng.random() < 0.3:
            alive = tuple(sorted(rng.choice(P, size=int(rng.integers(1, P + 1)), replace=False).tolist()))
        w = W.Workload(name="random", P=P, T=T, H=H, E=E, k=k, n_lo=0, n_hi=T, fmt=fmt, combine=comb,
                       routing="uniform", seed=int(rng.integers(1 << 30)))
        out.append(Case(w, has_weights=bool(rng.random() < 0.85),
                        invalid_id=int(rng.choice([E, -1, 12345])), alive=alive,
                        extra_bytes=int(rng.integers(1, 41)) if rng.random() < 0.3 else 0,
                        n_eplb=min(E, int(rng.integers(1, 300))) if rng.random() < 0.3 else 0))
    return out


CASES = _cases() + _cases(n=24, seed=20261203, wide=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from combine_route_mask_amd import moe_ep
    assert torch.cuda.is_available() and moe_ep.moe_ep_is_supported()
    yield
    torch.cuda.empty_cache()


def _check_dispatch(cs, c, out, ex, want, extra, stats, active):
    w = cs.w
    P = w.P
    ids_g = out["ids"].cpu().numpy()
    cnt_g = out["counts"].cpu().numpy()
    offs_g = out["src_offsets"].cpu().numpy()
    slots_g = out["slots"].cpu().numpy()
    pl_g = out["payload"].cpu().numpy()
    for r in range(P):
        if r not in cs.alive:
            assert bool((ex.workspace[r] == 0x5A).all()), f"masked-off rank {r} was written"
            continue
        assert np.array_equal(ids_g[r], want["ids"][r]), f"ids plane of rank {r}"
        cnt = want["counts"][r]
        assert np.array_equal(cnt_g[r], cnt), f"counts of rank {r}"
        assert np.array_equal(offs_g[r, :P], np.cumsum(cnt) - cnt), f"source offsets of rank {r}"
        assert offs_g[r, P] == cnt.sum()
        n = int(cnt.sum())
        assert np.array_equal(slots_g[r, :n], want["slots"][r, :n]), f"slot list of rank {r}"
        v = want["valid"][r].astype(bool)
        assert np.array_equal(pl_g[r][v], want["payload"][r][v]), f"payload of rank {r}"
        if c.scales is not None:
            assert np.array_equal(out["scales"][r].cpu().numpy()[v], want["scales"][r][v]), f"scales of rank {r}"
        if cs.has_weights:
            wt = out["weights"][r].cpu().numpy()
            assert np.array_equal(wt[v].view(np.uint32), want["weights"][r][v].view(np.uint32)), \
                f"weights of rank {r}"
        if extra is not None:
            assert np.array_equal(out["extra"][r].cpu().numpy()[v], want["extra"][r][v]), f"extra of rank {r}"
    if stats is not None:
        g = out["eplb_gathered_stats"].cpu().numpy()
        poison = np.full((P, cs.n_eplb), 0x5A5A5A5A, np.int32)
        for r in cs.alive:
            expect = oracle.eplb_allgather(stats, r, active=active, out=poison.copy())
            assert np.array_equal(g[r], expect), f"gathered statistics of rank {r}"


def _check_combine_bf16(cs, c, y, eb, valid, active):
    w = cs.w
    o = oracle.combine_bf16(c.counts, c.ids, eb, E=w.E, active=active)
    yb = bits16(y)
    for s in range(w.P):
        rows = bf16_bits_to_f64(yb[s])
        if s not in cs.alive:
            assert np.all(rows == 7.0), f"rows of masked-off source {s} were written"
            continue
        n = int(c.counts[s])
        check_bf16_sum(yb[s, :n], o.ref[s, :n], o.y[s, :n], f"source {s}")
        assert np.all(rows[n:] == 7.0), f"rows past the count of source {s} were written"


def _check_combine_fp8(cs, c, ex, y, eb, valid, active):
    w = cs.w
    P, T, H = w.P, w.T, w.H
    o8 = oracle.combine_fp8(c.counts, c.ids, eb, E=w.E, active=active)
    exact = oracle.combine_bf16(c.counts, c.ids, eb, E=w.E, active=active).exact
    gc, gs = ex.combine_landing()
    gc, gs = gc.cpu().numpy(), gs.cpu().numpy()
    yb = bits16(y)
    ev = bf16_bits_to_f64(eb)
    viol, total = 0, 0
    for s in range(P):
        rows = bf16_bits_to_f64(yb[s])
        if s not in cs.alive:
            assert np.all(rows == 7.0), f"rows of masked-off source {s} were written"
            continue
        n = int(c.counts[s])
        lv = np.zeros(P * T, bool)
        for r in range(P):
            lv[r * T:r * T + n] = valid[r, s * T:s * T + n]
        assert np.array_equal(gc[s][lv], o8.land_codes[s][lv]), f"landing codes of source {s}"
        assert np.array_equal(gs[s][lv], o8.land_scales[s][lv]), f"landing scales of source {s}"
        mag, floor = fp8_terms_and_floor(ev, valid, o8.land_scales[s], s, T, n, P)
        viol += check_fp8_sum(yb[s, :n], o8.y[s, :n], exact[s, :n], mag, floor, f"source {s}")
        total += n * H
        assert np.all(rows[n:] == 7.0), f"rows past the count of source {s} were written"
    log(f"FP8 literal bound: {viol} of {total} elements outside 0.07 sum|terms|")


@pytest.mark.parametrize("cs", CASES, ids=lambda cs: cs.name)
def test_random_exchange(cs):
    from combine_route_mask_amd.moe_ep import MoeEpExchange
    w = cs.w
    log(f"random case {cs.name} alive={list(cs.alive)}")
    c = random_byte_case(w, w.seed, oob=True, dup=True)
    rng = np.random.default_rng(w.seed + 1)
    extra = rng.integers(0, 256, size=(w.P, w.T, cs.extra_bytes)).astype(np.uint8) if cs.extra_bytes else None
    stats = rng.integers(-(1 << 30), 1 << 30, size=(w.P, cs.n_eplb)).astype(np.int32) if cs.n_eplb else None
    active = sum(1 << r for r in cs.alive)
    ex = MoeEpExchange(w.P, w.E, w.k, w.T, w.H, dispatch_format=w.fmt, combine_format=w.combine,
                       has_weights=cs.has_weights, invalid_expert_id=cs.invalid_id,
                       extra_payload_bytes_per_token=cs.extra_bytes, eplb_stats_num_experts=cs.n_eplb)
    ex.workspace.fill_(0x5A)
    pl, sc, ids, wt = gpu_inputs(c)
    out = ex.dispatch(pl, ids, wt if cs.has_weights else None, scales=sc, num_tokens=c.counts.tolist(),
                      runtime_max_tokens_per_rank=w.T, active_rank_mask=active,
                      extra_payload=None if extra is None else torch.from_numpy(extra).cuda(),
                      eplb_local_stats=None if stats is None else torch.from_numpy(stats).cuda())
    torch.cuda.synchronize()
    want = oracle.dispatch(c.counts, c.payload, c.ids, c.weights if cs.has_weights else None, c.scales,
                           E=w.E, invalid_id=cs.invalid_id, active=active, extra=extra)
    _check_dispatch(cs, c, out, ex, want, extra, stats, active)

    # combine: random magnitudes per row, NaN in every slot that got no token
    valid = want["valid"].astype(bool)
    g = W.torch_generator(w.seed, "cuda")
    scale = torch.pow(2.0, torch.randint(-20, 20, (w.P, w.P * w.T, 1), generator=g, device="cuda").float())
    eo = (torch.randn(w.P, w.P * w.T, w.H, generator=g, device="cuda") * scale).to(torch.bfloat16)
    eo[torch.from_numpy(~valid).cuda()] = float("nan")
    y = torch.full((w.P, w.T, w.H), 7.0, dtype=torch.bfloat16, device="cuda")
    ex.combine(eo, y)
    torch.cuda.synchronize()
    eb = bits16(eo)
    if w.combine == "fp8":
        _check_combine_fp8(cs, c, ex, y, eb, valid, active)
    else:
        _check_combine_bf16(cs, c, y, eb, valid, active)
    ex.destroy()
