"""Python binding of the C ABI in ``include/moe_ep.h`` (ctypes).

Argument marshalling only: every step of the exchange runs in the gfx950
kernels of ``libmoe_ep.so``.  torch supplies device memory and the current
HIP stream.  The functions carry the C names; ``MoeEpExchange`` bundles a
handle with its torch-allocated workspace and exposes the receive planes as
tensor views.

There is no fallback: if ``libmoe_ep.so`` is missing, importing this module
raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_ep.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_BAD_STATE = -3
ERR_CAPACITY = -4
ERR_HIP = -5

FMT_BF16, FMT_MXFP8, FMT_NVFP4, FMT_DEEPSEEK_FP8 = 0, 1, 2, 3
COMBINE_BF16, COMBINE_FP8 = 0, 1
MAX_RANKS = 64

_FMT_NAMES = {"bf16": FMT_BF16, "mxfp8": FMT_MXFP8, "nvfp4": FMT_NVFP4,
              "deepseek_fp8": FMT_DEEPSEEK_FP8}
_COMBINE_NAMES = {"bf16": COMBINE_BF16, "fp8": COMBINE_FP8}

# Every symbol include/moe_ep.h declares.
EXPORTS = ("moe_ep_is_supported", "moe_ep_workspace_bytes", "moe_ep_create", "moe_ep_dispatch",
           "moe_ep_combine", "moe_ep_combine_noalloc", "moe_ep_destroy", "moe_ep_allgatherv",
           "moe_ep_reduce_scatterv", "moe_ep_last_error")
STATIC_SCRATCH_BYTES = 64 << 20  # MOE_EP_STATIC_SCRATCH_BYTES


class MoeEpError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"moe_ep error {code}: {msg}")
        self.code = code


class MoeEpArgError(MoeEpError, ValueError):
    pass


class Params(C.Structure):
    _fields_ = [("ep_size", C.c_int32), ("num_experts", C.c_int32), ("top_k", C.c_int32),
                ("max_tokens_per_rank", C.c_int32), ("hidden_size", C.c_int32),
                ("dispatch_format", C.c_int32), ("combine_format", C.c_int32),
                ("has_weights", C.c_int32), ("invalid_expert_id", C.c_int32),
                ("extra_payload_bytes_per_token", C.c_int32), ("eplb_stats_num_experts", C.c_int32)]


class DispatchViews(C.Structure):
    _fields_ = [("tokens_per_rank", C.c_int32), ("ep_size", C.c_int32),
                ("region_bytes", C.c_int64), ("payload_offset", C.c_int64),
                ("payload_row_bytes", C.c_int64), ("scales_offset", C.c_int64),
                ("scale_row_bytes", C.c_int64), ("ids_offset", C.c_int64),
                ("weights_offset", C.c_int64), ("slots_offset", C.c_int64),
                ("counts_offset", C.c_int64), ("src_offsets_offset", C.c_int64),
                ("combine_payload_offset", C.c_int64), ("combine_scales_offset", C.c_int64),
                ("extra_offset", C.c_int64), ("extra_row_bytes", C.c_int64),
                ("eplb_offset", C.c_int64), ("eplb_num_experts", C.c_int64)]


class Plane(C.Structure):
    _fields_ = [("in_", C.c_void_p), ("in_rank_stride", C.c_int64), ("out", C.c_void_p),
                ("out_rank_stride", C.c_int64), ("row_bytes", C.c_int64)]


def _load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run combine_route_mask_amd.build.build() "
                          "(or __graft_entry__.build())")
    L = C.CDLL(path)
    vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
    L.moe_ep_is_supported.argtypes = []
    L.moe_ep_is_supported.restype = C.c_int
    L.moe_ep_workspace_bytes.argtypes = [C.POINTER(Params)]
    L.moe_ep_workspace_bytes.restype = C.c_size_t
    L.moe_ep_create.argtypes = [C.POINTER(Params), vp, C.c_size_t, C.POINTER(vp)]
    L.moe_ep_create.restype = C.c_int
    L.moe_ep_dispatch.argtypes = [vp, vp, vp, vp, vp, vp, vp, C.POINTER(i32), i32,
                                  C.POINTER(C.c_uint64), vp, C.POINTER(DispatchViews)]
    L.moe_ep_dispatch.restype = C.c_int
    L.moe_ep_combine.argtypes = [vp, vp, vp, vp]
    L.moe_ep_combine.restype = C.c_int
    L.moe_ep_combine_noalloc.argtypes = [vp, vp, vp, vp]
    L.moe_ep_combine_noalloc.restype = C.c_int
    L.moe_ep_destroy.argtypes = [vp]
    L.moe_ep_destroy.restype = C.c_int
    L.moe_ep_allgatherv.argtypes = [i32, C.POINTER(i32), i32, C.POINTER(Plane), vp]
    L.moe_ep_allgatherv.restype = C.c_int
    L.moe_ep_reduce_scatterv.argtypes = [i32, C.POINTER(i32), i32, vp, i64, vp, i64, vp]
    L.moe_ep_reduce_scatterv.restype = C.c_int
    L.moe_ep_last_error.argtypes = []
    L.moe_ep_last_error.restype = C.c_char_p
    return L


lib = _load()


def _check(rc: int):
    if rc != OK:
        msg = lib.moe_ep_last_error().decode()
        cls = MoeEpArgError if rc == ERR_INVALID_ARG else MoeEpError
        raise cls(rc, msg)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _torch_stream(stream):
    """The torch stream object of a stream argument (None: the current
    stream; a raw hipStream_t handle is wrapped)."""
    import torch
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream)
    return stream


def _i32_array(vals: Sequence[int]):
    a = np.ascontiguousarray(np.asarray(vals, dtype=np.int32))
    return a, a.ctypes.data_as(C.POINTER(C.c_int32))


# ----------------------------------------------------------------------------
# C-named entry points
# ----------------------------------------------------------------------------

def make_params(ep_size: int, num_experts: int, top_k: int, max_tokens_per_rank: int,
                hidden_size: int, dispatch_format="bf16", combine_format="bf16",
                has_weights: bool = True, invalid_expert_id: Optional[int] = None,
                extra_payload_bytes_per_token: int = 0, eplb_stats_num_experts: int = 0) -> Params:
    df = _FMT_NAMES.get(dispatch_format, dispatch_format)
    cf = _COMBINE_NAMES.get(combine_format, combine_format)
    return Params(ep_size, num_experts, top_k, max_tokens_per_rank, hidden_size, int(df), int(cf),
                  1 if has_weights else 0,
                  num_experts if invalid_expert_id is None else invalid_expert_id,
                  int(extra_payload_bytes_per_token), int(eplb_stats_num_experts))


def moe_ep_is_supported() -> bool:
    return bool(lib.moe_ep_is_supported())


def moe_ep_workspace_bytes(params: Params) -> int:
    n = lib.moe_ep_workspace_bytes(C.byref(params))
    if n == 0:
        raise MoeEpArgError(ERR_INVALID_ARG, lib.moe_ep_last_error().decode())
    return int(n)


def moe_ep_create(params: Params, workspace_ptr: int, size_per_rank: int) -> C.c_void_p:
    h = C.c_void_p()
    _check(lib.moe_ep_create(C.byref(params), C.c_void_p(workspace_ptr), size_per_rank,
                             C.byref(h)))
    return h


def moe_ep_dispatch(handle, hidden, scales, topk_ids, topk_weights, num_tokens,
                    runtime_max_tokens_per_rank: int = 0, stream=None,
                    active_rank_mask: Optional[int] = None, extra_payload=None,
                    eplb_local_stats=None) -> DispatchViews:
    counts, cptr = _i32_array(num_tokens)
    views = DispatchViews()
    mask = None if active_rank_mask is None else C.byref(C.c_uint64(int(active_rank_mask)))
    _check(lib.moe_ep_dispatch(handle, _ptr(hidden), _ptr(scales), _ptr(extra_payload),
                               _ptr(eplb_local_stats), _ptr(topk_ids),
                               _ptr(topk_weights), cptr, int(runtime_max_tokens_per_rank), mask,
                               _stream(stream), C.byref(views)))
    del counts
    return views


def moe_ep_combine(handle, expert_output, output, stream=None) -> None:
    _check(lib.moe_ep_combine(handle, _ptr(expert_output), _ptr(output), _stream(stream)))


def moe_ep_combine_noalloc(handle, expert_output, output, stream=None) -> None:
    """moe_ep_combine staging the FP8 landing planes in the library's static
    array (no allocation anywhere; output must be given)."""
    _check(lib.moe_ep_combine_noalloc(handle, _ptr(expert_output), _ptr(output), _stream(stream)))


def moe_ep_destroy(handle) -> None:
    _check(lib.moe_ep_destroy(handle))


def moe_ep_allgatherv(sizes: Sequence[int], planes: Sequence[Plane], stream=None) -> None:
    s, sptr = _i32_array(sizes)
    arr = (Plane * len(planes))(*planes)
    _check(lib.moe_ep_allgatherv(len(s), sptr, len(planes), arr, _stream(stream)))


def moe_ep_reduce_scatterv(sizes: Sequence[int], hidden_size: int, in_ptr: int,
                           in_rank_stride: int, out_ptr: int, out_rank_stride: int,
                           stream=None) -> None:
    s, sptr = _i32_array(sizes)
    _check(lib.moe_ep_reduce_scatterv(len(s), sptr, hidden_size, C.c_void_p(in_ptr),
                                      in_rank_stride, C.c_void_p(out_ptr), out_rank_stride,
                                      _stream(stream)))


# ----------------------------------------------------------------------------
# torch-facing convenience wrappers (shape checks and views only)
# ----------------------------------------------------------------------------

def _need(cond: bool, msg: str):
    if not cond:
        raise MoeEpArgError(ERR_INVALID_ARG, msg)


def _dev_contig(t, name, device=None):
    _need(t.is_cuda, f"{name} must be a GPU tensor")
    _need(device is None or t.device == device, f"{name} must be on {device}, got {t.device}")
    _need(t.is_contiguous(), f"{name} must be contiguous")


class MoeEpExchange:
    """A handle plus its ``[P, size_per_rank]`` uint8 workspace tensor.

    ``dispatch`` takes stacked per-rank tensors ``[P, T, ...]`` and returns
    a dict of receive-plane views ``[P, P*T, ...]`` (rank r's region first),
    valid until the next dispatch.  ``combine`` takes the stacked expert
    outputs ``[P, P*T, H]`` bf16 and writes ``[P, T, H]`` bf16."""

    def __init__(self, ep_size: int, num_experts: int, top_k: int, max_tokens_per_rank: int,
                 hidden_size: int, dispatch_format="bf16", combine_format="bf16",
                 has_weights: bool = True, invalid_expert_id: Optional[int] = None,
                 extra_payload_bytes_per_token: int = 0, eplb_stats_num_experts: int = 0,
                 device="cuda"):
        import torch
        self.params = make_params(ep_size, num_experts, top_k, max_tokens_per_rank, hidden_size,
                                  dispatch_format, combine_format, has_weights, invalid_expert_id,
                                  extra_payload_bytes_per_token, eplb_stats_num_experts)
        self.size_per_rank = moe_ep_workspace_bytes(self.params)
        self.workspace = torch.empty((ep_size, self.size_per_rank), dtype=torch.uint8,
                                     device=device)
        self.handle = moe_ep_create(self.params, self.workspace.data_ptr(), self.size_per_rank)
        self.views: Optional[DispatchViews] = None

    @property
    def P(self):
        return self.params.ep_size

    def row_bytes(self):
        """(payload row bytes, scale row bytes) of the dispatch format."""
        H, f = self.params.hidden_size, self.params.dispatch_format
        return {FMT_BF16: (2 * H, 0), FMT_MXFP8: (H, H // 32), FMT_NVFP4: (H // 2, H // 16),
                FMT_DEEPSEEK_FP8: (H, H // 128 * 4)}[f]

    def destroy(self):
        if self.handle is not None:
            moe_ep_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    def _plane(self, offset: int, row_bytes: int, T: int, dtype=None):
        import torch
        P = self.P
        S = P * T
        if row_bytes == 0:
            return None
        base = self.workspace.view(-1)
        v = base.as_strided((P, S, row_bytes), (self.size_per_rank, row_bytes, 1), offset)
        return v if dtype is None else v.view(dtype)

    def dispatch(self, hidden, topk_ids, topk_weights=None, scales=None, num_tokens=None,
                 runtime_max_tokens_per_rank: Optional[int] = None, stream=None,
                 active_rank_mask: Optional[int] = None, extra_payload=None,
                 eplb_local_stats=None):
        import torch
        P = self.P
        T = runtime_max_tokens_per_rank or self.params.max_tokens_per_rank
        _need(1 <= T <= self.params.max_tokens_per_rank, "T must be in [1, max_tokens_per_rank]")
        _dev_contig(hidden, "hidden", self.workspace.device)
        _dev_contig(topk_ids, "topk_ids", self.workspace.device)
        _need(hidden.dim() >= 2 and hidden.shape[0] == P and hidden.shape[1] == T,
              f"hidden must be [P={P}, T={T}, row], got {tuple(hidden.shape)}")
        row, srow = self.row_bytes()
        _need(hidden.numel() * hidden.element_size() == P * T * row,
              f"hidden rows must be {row} bytes")
        _need(topk_ids.dtype == torch.int32 and tuple(topk_ids.shape) == (P, T, self.params.top_k),
              "topk_ids must be int32 [P, T, top_k]")
        if topk_weights is not None:
            _dev_contig(topk_weights, "topk_weights", self.workspace.device)
            _need(topk_weights.dtype == torch.float32 and topk_weights.shape == topk_ids.shape,
                  "topk_weights must be float32 [P, T, top_k]")
        if scales is not None:
            _dev_contig(scales, "scales", self.workspace.device)
            _need(scales.dim() >= 2 and scales.shape[0] == P and scales.shape[1] == T and
                  scales.numel() * scales.element_size() == P * T * srow,
                  f"scales must be [P, T] rows of {srow} bytes")
        if extra_payload is not None:
            xb = self.params.extra_payload_bytes_per_token
            _dev_contig(extra_payload, "extra_payload", self.workspace.device)
            _need(extra_payload.dim() >= 2 and extra_payload.shape[0] == P and
                  extra_payload.shape[1] == T and
                  extra_payload.numel() * extra_payload.element_size() == P * T * xb,
                  f"extra_payload must be [P, T] rows of {xb} bytes")
        if eplb_local_stats is not None:
            n = self.params.eplb_stats_num_experts
            _dev_contig(eplb_local_stats, "eplb_local_stats", self.workspace.device)
            _need(eplb_local_stats.dtype == torch.int32 and
                  tuple(eplb_local_stats.shape) == (P, n),
                  f"eplb_local_stats must be int32 [P, {n}]")
        if num_tokens is None:
            num_tokens = [T] * P
        _need(len(num_tokens) == P, "num_tokens needs one entry per rank")
        v = moe_ep_dispatch(self.handle, hidden, scales, topk_ids, topk_weights, num_tokens,
                            T, stream, active_rank_mask, extra_payload, eplb_local_stats)
        self.views = v
        k = self.params.top_k
        out = {
            "tokens_per_rank": v.tokens_per_rank,
            "payload": self._plane(v.payload_offset, v.payload_row_bytes, T),
            "scales": self._plane(v.scales_offset, v.scale_row_bytes, T),
            "ids": self._plane(v.ids_offset, 4 * k, T, torch.int32),
            "weights": (self._plane(v.weights_offset, 4 * k, T, torch.float32)
                        if self.params.has_weights else None),
        }
        base = self.workspace.view(-1)
        out["slots"] = base.as_strided((P, P * T * 4), (self.size_per_rank, 1),
                                       v.slots_offset).view(torch.int32)
        out["counts"] = base.as_strided((P, P * 4), (self.size_per_rank, 1),
                                        v.counts_offset).view(torch.int32)
        out["src_offsets"] = base.as_strided((P, (P + 1) * 4), (self.size_per_rank, 1),
                                             v.src_offsets_offset).view(torch.int32)
        out["extra"] = self._plane(v.extra_offset, v.extra_row_bytes, T)
        out["eplb_gathered_stats"] = None
        if v.eplb_offset >= 0:
            n = v.eplb_num_experts
            out["eplb_gathered_stats"] = base.as_strided((P, P * n * 4), (self.size_per_rank, 1),
                                                         v.eplb_offset).view(torch.int32).view(P, P, n)
        return out

    def combine_landing(self):
        """FP8 combine landing planes of the last step: codes
        ``[P, P*T, H]`` and scales ``[P, P*T, H/32]`` (uint8); slot r*T + t
        of source rank s holds rank r's quantised row of token (s, t)."""
        v = self.views
        _need(v is not None and v.combine_payload_offset >= 0, "no FP8 combine landing plane")
        H, T = self.params.hidden_size, v.tokens_per_rank
        return (self._plane(v.combine_payload_offset, H, T),
                self._plane(v.combine_scales_offset, H // 32, T))

    def combine(self, expert_output, output=None, stream=None):
        import torch
        P, H = self.P, self.params.hidden_size
        _need(self.views is not None, "combine before any dispatch")
        T = self.views.tokens_per_rank
        _dev_contig(expert_output, "expert_output", self.workspace.device)
        _need(expert_output.dtype == torch.bfloat16 and tuple(expert_output.shape) == (P, P * T, H),
              f"expert_output must be bf16 [P, P*T, H] = [{P}, {P * T}, {H}]")
        if output is None:
            # zero-filled on the launch stream, so the fill is ordered before
            # the combine's writes whatever the current stream is
            with torch.cuda.stream(_torch_stream(stream)):
                output = torch.zeros((P, T, H), dtype=torch.bfloat16, device=expert_output.device)
        _dev_contig(output, "output", self.workspace.device)
        _need(output.dtype == torch.bfloat16 and tuple(output.shape) == (P, T, H),
              "output must be bf16 [P, T, H]")
        moe_ep_combine(self.handle, expert_output, output, stream)
        return output


def allgatherv(sizes: Sequence[int], tensors, outs, stream=None):
    """All-gatherv of stacked per-rank tensors ``[P, max_rows, ...]`` into
    stacked outputs ``[P, sum(sizes), ...]`` (one launch for all planes)."""
    planes = []
    P, total = len(sizes), int(sum(sizes))
    _need(P >= 1 and len(tensors) == len(outs) >= 1, "need sizes for P >= 1 ranks and one output per input")
    dev = tensors[0].device
    for x, o in zip(tensors, outs):
        _dev_contig(x, "input", dev)
        _dev_contig(o, "output", dev)
        _need(x.shape[0] == P and o.shape[0] == P, "inputs and outputs are stacked [P, rows, ...]")
        _need(max(sizes) <= x.shape[1], "an input holds fewer rows than its size")
        _need(o.shape[1] >= total and o.shape[2:] == x.shape[2:] and o.dtype == x.dtype,
              "outputs must be [P, >= sum(sizes), ...] of the input's row type")
        rb = x[0, 0].numel() * x.element_size() if x.dim() > 2 else x.element_size()
        planes.append(Plane(x.data_ptr(), x.stride(0) * x.element_size(), o.data_ptr(),
                            o.stride(0) * o.element_size(), rb))
    moe_ep_allgatherv(sizes, planes, stream)
    return outs


def reduce_scatterv(sizes: Sequence[int], partial, out, stream=None):
    """Reduce-scatterv of stacked bf16 partials ``[P, sum(sizes), H]`` into
    ``out`` ``[P, max(sizes), H]`` (rank r's first sizes[r] rows)."""
    _dev_contig(partial, "partial")
    _dev_contig(out, "out", partial.device)
    import torch
    P, total = len(sizes), int(sum(sizes))
    _need(P >= 1, "need sizes for P >= 1 ranks")
    _need(partial.dtype == torch.bfloat16 and out.dtype == torch.bfloat16, "bf16 tensors only")
    _need(partial.dim() == 3 and partial.shape[0] == P and partial.shape[1] >= total,
          "partial must be [P, >= sum(sizes), H]")
    _need(out.dim() == 3 and out.shape[0] == P and out.shape[1] >= max(sizes) and
          out.shape[2] == partial.shape[2], "out must be [P, >= max(sizes), H]")
    H = partial.shape[-1]
    moe_ep_reduce_scatterv(sizes, H, partial.data_ptr(), partial.stride(0) * 2, out.data_ptr(),
                           out.stride(0) * 2, stream)
    return out
