"""Seeded synthetic workloads for MoE expert-parallel dispatch / combine.

This module only *draws inputs*: routing (per-rank token counts, top-k
expert ids, top-k weights), token payloads and expert outputs.  It holds
none of the exchange's arithmetic (no routing masks, no slot rule, no
reduction), so the CPU oracle and the GPU path can both be fed from it
without sharing any code.

Workload shapes follow the five workloads the exchange is measured on:
the expert-parallel dispatch / combine contract of FlashInfer's
``NVLinkTwoSidedAlltoAll.dispatch`` / ``combine`` pages (token rows
``[local_num_tokens, *]``, ``topk_ids`` / ``topk_weights``
``[local_num_tokens, top_k]``) and the all-gatherv / reduce-scatterv
workload of vLLM's ``AgRsAll2AllManager``.

Draw order per workload (one ``numpy.random.default_rng(seed)``):
counts/sizes -> ids -> logits -> (bulk data from a torch generator seeded
with ``seed``).  Bulk tensors (token rows, expert outputs) come from a
``torch.Generator`` on the requested device so the large workloads can be
drawn on the GPU without a host round trip; small parity cases draw them
on the CPU and upload.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

FMT_BF16 = "bf16"
FMT_MXFP8 = "mxfp8"
FMT_NVFP4 = "nvfp4"
FMT_DEEPSEEK_FP8 = "deepseek_fp8"


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic exchange workload.

    ``P`` virtual EP ranks, capacity ``T`` tokens per rank (the step's
    ``runtime_max_tokens_per_rank``), ``H`` hidden size, ``E`` experts,
    ``k`` experts per token.  ``n_lo``..``n_hi`` bounds the per-rank
    token counts (inclusive, uniform).  ``routing`` is ``"uniform"``
    (k distinct experts uniformly) or ``"zipf"`` (k distinct experts,
    popularity p_e proportional to (e+1)^-zipf_s, drawn by Gumbel-top-k).
    ``extra_bytes`` more bytes per token travel with the payload (router
    logits: E fp32 values), ``n_eplb`` per-expert int32 statistics per rank
    are all-gathered, and only the ranks in ``alive`` take part (None: all).
    """

    name: str
    P: int
    T: int
    H: int
    E: int
    k: int
    n_lo: int
    n_hi: int
    fmt: str = FMT_BF16
    combine: str = "bf16"  # "bf16" or "fp8"
    routing: str = "uniform"
    zipf_s: float = 1.2
    seed: int = 0
    extra_bytes: int = 0
    n_eplb: int = 0
    alive: Optional[tuple] = None

    @property
    def epr(self) -> int:
        return self.E // self.P


# The five measured workloads.  Sizes are the ones the exchange is quoted on.
TINY = Workload("tiny P4 T16 H256 E16 k2", P=4, T=16, H=256, E=16, k=2,
                n_lo=16, n_hi=16, seed=1)
EP8_BF16 = Workload("ep8 T128 H7168 bf16 E256 k8", P=8, T=128, H=7168,
                    E=256, k=8, n_lo=64, n_hi=128, seed=2)
EP8_MXFP8 = Workload("ep8 T512 H7168 mxfp8 zipf E256 k8 fp8-combine", P=8,
                     T=512, H=7168, E=256, k=8, n_lo=512, n_hi=512,
                     fmt=FMT_MXFP8, combine="fp8", routing="zipf", seed=3)
EP64_BF16 = Workload("ep64 T512 H7168 bf16 E256 k8", P=64, T=512, H=7168,
                     E=256, k=8, n_lo=512, n_hi=512, seed=4)
EP64_NVFP4 = dataclasses.replace(EP64_BF16, name="ep64 T512 H7168 nvfp4 E256 k8",
                                 fmt=FMT_NVFP4)
# The next rows on the EP64 shape: DeepSeekFp8 payloads; NVFP4 with each
# token's 256 fp32 router logits as extra payload and 256 per-expert
# statistics all-gathered; BF16 with 48 of the 64 ranks taking part.
EP64_DSFP8 = dataclasses.replace(EP64_BF16, name="ep64 T512 H7168 deepseek_fp8 E256 k8",
                                 fmt=FMT_DEEPSEEK_FP8)
EP64_NVFP4_EXTRAS = dataclasses.replace(EP64_NVFP4, name="ep64 T512 H7168 nvfp4 E256 k8 logits1024 eplb256",
                                        extra_bytes=1024, n_eplb=256)
EP64_MASK48 = dataclasses.replace(EP64_BF16, name="ep64 T512 H7168 bf16 E256 k8 alive48",
                                  alive=tuple(r for r in range(64) if r % 4 != 3))


@dataclasses.dataclass(frozen=True)
class AgRsWorkload:
    """All-gatherv / reduce-scatterv workload: ``P`` ranks with row counts
    uniform in ``[s_lo, s_hi]``, hidden ``H`` bf16, ``k`` ids/weights per
    row over ``E`` experts."""

    name: str
    P: int
    H: int
    E: int
    k: int
    s_lo: int
    s_hi: int
    seed: int = 5


AGRS16 = AgRsWorkload("agrs P16 sizes U[1,1024] H4096", P=16, H=4096, E=128,
                      k=4, s_lo=1, s_hi=1024)


def payload_row_bytes(fmt: str, H: int) -> int:
    """Bytes of one token's payload row in the given dispatch format."""
    if fmt == FMT_BF16:
        return 2 * H
    if fmt == FMT_MXFP8:
        return H
    if fmt == FMT_NVFP4:
        return H // 2
    if fmt == FMT_DEEPSEEK_FP8:
        return H
    raise ValueError(fmt)


def scale_row_bytes(fmt: str, H: int) -> int:
    """Bytes of one token's scale row (0 when the format has none)."""
    if fmt == FMT_BF16:
        return 0
    if fmt == FMT_MXFP8:
        return H // 32
    if fmt == FMT_NVFP4:
        return H // 16
    if fmt == FMT_DEEPSEEK_FP8:
        return H // 128 * 4
    raise ValueError(fmt)


# ---------------------------------------------------------------------------
# routing draws (numpy, host)
# ---------------------------------------------------------------------------

def draw_counts(rng: np.random.Generator, P: int, lo: int, hi: int) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=P, dtype=np.int64).astype(np.int32)


def draw_topk_ids(rng: np.random.Generator, rows: int, E: int, k: int,
                  routing: str = "uniform", zipf_s: float = 1.2) -> np.ndarray:
    """``[rows, k]`` int32 distinct expert ids per row.

    uniform: the first k of a uniform random permutation key;
    zipf: Gumbel-top-k over log p_e with p_e ~ (e+1)^-s (k distinct draws
    without replacement, proportional to popularity)."""
    if routing == "uniform":
        key = rng.random((rows, E))
    elif routing == "zipf":
        logp = -zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
        u = rng.random((rows, E))
        gumbel = -np.log(-np.log(np.clip(u, 1e-300, 1.0)))
        key = -(logp[None, :] + gumbel)
    else:
        raise ValueError(routing)
    ids = np.argpartition(key, k - 1, axis=1)[:, :k]
    # order the k ids by their key so the draw is independent of argpartition
    order = np.take_along_axis(key, ids, axis=1).argsort(axis=1, kind="stable")
    return np.take_along_axis(ids, order, axis=1).astype(np.int32)


def draw_topk_weights(rng: np.random.Generator, rows: int, k: int) -> np.ndarray:
    """``[rows, k]`` fp32 weights: softmax (in fp32) of N(0,1) logits."""
    logits = rng.standard_normal((rows, k)).astype(np.float32)
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m, dtype=np.float32)
    return (e / e.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)


@dataclasses.dataclass
class Routing:
    counts: np.ndarray   # [P] int32 local token counts n_s
    ids: np.ndarray      # [P, T, k] int32 (rows t >= n_s hold decoy ids)
    weights: np.ndarray  # [P, T, k] float32


def draw_routing(w: Workload, seed: Optional[int] = None) -> Routing:
    """Counts, ids and weights of workload ``w``.

    Rows ``t >= n_s`` of ``ids`` / ``weights`` are filled with ordinary
    looking decoys: the exchange must never read them."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    counts = draw_counts(rng, w.P, w.n_lo, w.n_hi)
    ids = draw_topk_ids(rng, w.P * w.T, w.E, w.k, w.routing, w.zipf_s)
    weights = draw_topk_weights(rng, w.P * w.T, w.k)
    return Routing(counts, ids.reshape(w.P, w.T, w.k),
                   weights.reshape(w.P, w.T, w.k))


# ---------------------------------------------------------------------------
# bulk draws (torch, any device)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def torch_generator(seed: int, device):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal_bf16(shape, gen, device, chunk_rows: int = 1 << 15):
    """bf16 tensor of N(0,1) draws (fp32 draw, round-to-nearest-even to
    bf16), drawn in row chunks so huge tensors need no fp32 copy."""
    torch = _torch()
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1, shape[-1])
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(flat.shape[0], r0 + chunk_rows)
        flat[r0:r1] = torch.randn((r1 - r0, shape[-1]), generator=gen,
                                  device=device, dtype=torch.float32).to(torch.bfloat16)
    return out


def encode_mxfp8(x_bf16):
    """MXFP8 payload of bf16 rows ``[..., H]``: e4m3 codes ``[..., H]`` and
    one e8m0 scale per 32 elements ``[..., H/32]`` (uint8).

    Shared exponent floor(log2 amax) - 8 per block (the e4m3 largest
    power of two is 2^8), elements cast with saturation to +-448."""
    torch = _torch()
    H = x_bf16.shape[-1]
    xb = x_bf16.float().reshape(*x_bf16.shape[:-1], H // 32, 32)
    amax = xb.abs().amax(dim=-1, keepdim=True)
    _, ex = torch.frexp(amax)                      # amax = m * 2^ex, m in [0.5,1)
    e = torch.where(amax > 0, ex - 1 - 8, torch.full_like(ex, -127))
    e = e.clamp(-127, 127)
    scaled = (xb * torch.pow(2.0, -e.float())).clamp(-448.0, 448.0)
    codes = scaled.to(torch.float8_e4m3fn).view(torch.uint8).reshape(x_bf16.shape)
    scales = (e + 127).to(torch.uint8).reshape(*x_bf16.shape[:-1], H // 32)
    return codes, scales


_E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def encode_nvfp4(x_bf16):
    """NVFP4 payload of bf16 rows ``[..., H]``: packed e2m1 nibbles
    ``[..., H/2]`` (low nibble = even element) and one e4m3 scale per 16
    elements ``[..., H/16]`` (uint8).  Scale s = e4m3(amax / 6), element
    = nearest e2m1 magnitude of x / s (ties to the even code), saturating
    at 6.  No second-level global scale."""
    torch = _torch()
    H = x_bf16.shape[-1]
    xb = x_bf16.float().reshape(*x_bf16.shape[:-1], H // 16, 16)
    amax = xb.abs().amax(dim=-1, keepdim=True)
    s8 = (amax / 6.0).clamp(max=448.0).to(torch.float8_e4m3fn)
    s = s8.float()
    safe = torch.where(s > 0, s, torch.ones_like(s))
    y = torch.where(s > 0, xb / safe, torch.zeros_like(xb))
    a = y.abs()
    code = torch.zeros_like(a, dtype=torch.int32)
    for i in range(7):
        mid = 0.5 * (_E2M1_GRID[i] + _E2M1_GRID[i + 1])
        up = (a > mid) | ((a == mid) & (i % 2 == 1))
        code += up.to(torch.int32)
    code = code | (((y < 0) & (code != 0)).to(torch.int32) << 3)
    code = code.to(torch.uint8).reshape(*x_bf16.shape[:-1], H)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    scales = s8.view(torch.uint8).reshape(*x_bf16.shape[:-1], H // 16)
    return packed.contiguous(), scales.contiguous()


def encode_deepseek_fp8(x_bf16):
    """DeepSeekFp8 payload of bf16 rows ``[..., H]``: e4m3 codes ``[..., H]``
    and one fp32 scale per 128 elements ``[..., H/128]`` as bytes
    ``[..., H/32]``: scale = amax / 448, element = e4m3(x / scale)."""
    torch = _torch()
    H = x_bf16.shape[-1]
    xb = x_bf16.float().reshape(*x_bf16.shape[:-1], H // 128, 128)
    amax = xb.abs().amax(dim=-1, keepdim=True)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    codes = (xb / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    scales = scale.reshape(*x_bf16.shape[:-1], H // 128).contiguous().view(torch.uint8)
    return codes.reshape(x_bf16.shape).contiguous(), scales


@dataclasses.dataclass
class DispatchInputs:
    routing: Routing
    payload: object        # torch uint8/bf16 tensor [P, T, row_bytes] (as bytes view)
    scales: object         # torch uint8 [P, T, scale_row_bytes] or None
    hidden_bf16: object    # the bf16 rows the payload was encoded from [P, T, H]


def draw_extras(w: Workload, device="cpu", seed: Optional[int] = None):
    """(extra payload uint8 [P, T, extra_bytes] or None, EPLB statistics
    int32 [P, n_eplb] or None).  The extra rows are the bytes of N(0,1)
    fp32 values (router logits); the statistics are per-expert token
    counts drawn uniformly in [0, 4T]."""
    torch = _torch()
    seed = w.seed if seed is None else seed
    extra = stats = None
    if w.extra_bytes:
        g = torch_generator(seed + 7919, device)
        nf = (w.extra_bytes + 3) // 4
        x = torch.randn((w.P, w.T, nf), generator=g, device=device, dtype=torch.float32)
        extra = x.view(torch.uint8)[..., :w.extra_bytes].contiguous()
    if w.n_eplb:
        rng = np.random.default_rng(seed + 104729)
        stats = torch.from_numpy(rng.integers(0, 4 * w.T + 1, size=(w.P, w.n_eplb)).astype(np.int32)).to(device)
    return extra, stats


def draw_dispatch_inputs(w: Workload, device="cpu", seed: Optional[int] = None,
                         routing: Optional[Routing] = None) -> DispatchInputs:
    torch = _torch()
    seed = w.seed if seed is None else seed
    if routing is None:
        routing = draw_routing(w, seed)
    g = torch_generator(seed, device)
    hidden = normal_bf16((w.P, w.T, w.H), g, device)
    if w.fmt == FMT_BF16:
        payload = hidden.view(torch.uint8).view(w.P, w.T, 2 * w.H)
        scales = None
    elif w.fmt == FMT_MXFP8:
        payload, scales = encode_mxfp8(hidden)
    elif w.fmt == FMT_NVFP4:
        payload, scales = encode_nvfp4(hidden)
    elif w.fmt == FMT_DEEPSEEK_FP8:
        payload, scales = encode_deepseek_fp8(hidden)
    else:
        raise ValueError(w.fmt)
    return DispatchInputs(routing, payload, scales, hidden)


def draw_expert_output(P: int, T: int, H: int, seed: int, device="cpu"):
    """``[P, P*T, H]`` bf16 N(0,1) per-slot expert outputs (every slot of
    every rank, valid or not)."""
    g = torch_generator(seed + 1000003, device)
    return normal_bf16((P, P * T, H), g, device)


# ---------------------------------------------------------------------------
# all-gatherv / reduce-scatterv draws
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class AgRsInputs:
    sizes: np.ndarray       # [P] int32
    hidden: object          # [P, max_size, H] bf16 (rank r uses rows < sizes[r])
    weights: np.ndarray     # [P, max_size, k] float32
    ids: np.ndarray         # [P, max_size, k] int32
    partial: object         # [P, sum(sizes), H] bf16 per-rank partial outputs


def draw_agrs_inputs(w: AgRsWorkload, device="cpu", seed: Optional[int] = None,
                     sizes: Optional[np.ndarray] = None) -> AgRsInputs:
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    if sizes is None:
        sizes = draw_counts(rng, w.P, w.s_lo, w.s_hi)
    sizes = np.asarray(sizes, dtype=np.int32)
    smax = max(int(sizes.max()), 1)
    ids = draw_topk_ids(rng, w.P * smax, w.E, w.k).reshape(w.P, smax, w.k)
    weights = draw_topk_weights(rng, w.P * smax, w.k).reshape(w.P, smax, w.k)
    g = torch_generator(seed, device)
    hidden = normal_bf16((w.P, smax, w.H), g, device)
    total = int(sizes.sum())
    partial = normal_bf16((w.P, max(total, 1), w.H), g, device)[:, :total]
    return AgRsInputs(sizes, hidden, weights, ids, partial)

