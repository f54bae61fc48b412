"""The C-ABI library loads, exports every entry point include/moe_ep.h
declares, and rejects bad arguments before touching a GPU.  No kernel is
launched here."""
import ctypes as C
import os
import re

import pytest

from tests.conftest import ROOT


@pytest.fixture(scope="module")
def m():
    lib = os.path.join(ROOT, "combine_route_mask_amd", "libmoe_ep.so")
    if not os.path.exists(lib):
        from combine_route_mask_amd import build
        build.build()
    from combine_route_mask_amd import moe_ep
    return moe_ep


def _declared():
    hdr = open(os.path.join(ROOT, "include", "moe_ep.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_ep_[a-z_]+)\s*\(", hdr)))


def test_exports_every_declared_symbol(m):
    names = _declared()
    assert set(names) == set(m.EXPORTS)
    lib = C.CDLL(m.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_unsupported_without_gpu(m):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert m.moe_ep_is_supported() is False
    p = m.make_params(8, 256, 8, 128, 7168)
    with pytest.raises(m.MoeEpError) as e:
        m.moe_ep_create(p, 256, m.moe_ep_workspace_bytes(p))
    assert e.value.code == m.ERR_UNSUPPORTED


def test_workspace_bytes_layout(m):
    p = m.make_params(8, 256, 8, 128, 7168)
    n = m.moe_ep_workspace_bytes(p)
    S = 8 * 128
    # payload + ids + weights + slots + counts + offsets + masks, each 256-aligned
    want = 0
    for b in (S * 14336, 0, S * 32, S * 32, S * 4, 32, 36, 128 * 8):
        want = (want + b + 255) // 256 * 256
    assert n == want
    p8 = m.make_params(8, 256, 8, 512, 7168, "mxfp8", "fp8")
    n8 = m.moe_ep_workspace_bytes(p8)
    assert n8 > 4096 * (7168 + 224 + 64 + 4 + 7168 + 224)
    # no weights plane when has_weights = 0
    assert m.moe_ep_workspace_bytes(m.make_params(8, 256, 8, 128, 7168, has_weights=False)) == n - S * 32
    # extra bytes and EPLB statistics add their planes
    nx = m.moe_ep_workspace_bytes(m.make_params(8, 256, 8, 128, 7168, extra_payload_bytes_per_token=48,
                                                eplb_stats_num_experts=256))
    assert nx == n + S * 48 + 8 * 256 * 4
    # DeepSeekFp8: H e4m3 bytes + H/128 fp32 scales per row
    nd = m.moe_ep_workspace_bytes(m.make_params(8, 256, 8, 128, 7168, "deepseek_fp8"))
    assert nd == n - S * 7168 + S * 56 * 4


@pytest.mark.parametrize("kw,code", [
    (dict(ep_size=0), -1), (dict(ep_size=65), -1),
    (dict(num_experts=254), -1),                 # E % 4
    (dict(ep_size=3, num_experts=8), -1),        # E % P
    (dict(top_k=0), -1), (dict(top_k=65), -1),
    (dict(max_tokens_per_rank=0), -1),
    (dict(hidden_size=7164), -1),                # BF16 row not a multiple of 16 B
    (dict(hidden_size=7176, dispatch_format="mxfp8"), -1),
    (dict(hidden_size=7176, combine_format="fp8"), -1),
    (dict(dispatch_format=7), -2), (dict(combine_format=5), -2),
    (dict(hidden_size=7200, dispatch_format="deepseek_fp8"), -1),  # H % 128
    (dict(extra_payload_bytes_per_token=-1), -1), (dict(eplb_stats_num_experts=-4), -1),
    (dict(eplb_stats_num_experts=257), -1),      # statistics of more experts than exist
    (dict(eplb_stats_num_experts=(1 << 31) - 1), -1),
    (dict(max_tokens_per_rank=1 << 30, ep_size=64), -4),
    (dict(max_tokens_per_rank=1 << 24, ep_size=64, hidden_size=1 << 20), -4),   # region above 2^46 B
])
def test_param_validation(m, kw, code):
    base = dict(ep_size=8, num_experts=256, top_k=8, max_tokens_per_rank=128, hidden_size=7168)
    base.update(kw)
    p = m.make_params(**base)
    assert m.lib.moe_ep_workspace_bytes(C.byref(p)) == 0
    h = C.c_void_p()
    assert m.lib.moe_ep_create(C.byref(p), C.c_void_p(256), 1 << 30, C.byref(h)) == code
    assert m.lib.moe_ep_last_error().decode() != ""


def test_create_checks_workspace_before_device(m):
    p = m.make_params(8, 256, 8, 128, 7168)
    n = m.moe_ep_workspace_bytes(p)
    h = C.c_void_p()
    assert m.lib.moe_ep_create(C.byref(p), None, n, C.byref(h)) == m.ERR_INVALID_ARG
    assert m.lib.moe_ep_create(C.byref(p), C.c_void_p(4096 + 16), n, C.byref(h)) == m.ERR_INVALID_ARG
    assert m.lib.moe_ep_create(C.byref(p), C.c_void_p(4096), n + 8, C.byref(h)) == m.ERR_INVALID_ARG
    assert m.lib.moe_ep_create(C.byref(p), C.c_void_p(4096), n - 256, C.byref(h)) == m.ERR_CAPACITY
    assert m.lib.moe_ep_create(C.byref(p), C.c_void_p(4096), n, None) == m.ERR_INVALID_ARG


def test_calls_on_bad_handles(m):
    counts = (C.c_int32 * 8)(*([1] * 8))
    assert m.lib.moe_ep_dispatch(None, C.c_void_p(256), None, None, None, C.c_void_p(256), None,
                                 counts, 0, None, None, None) == m.ERR_INVALID_ARG
    assert m.lib.moe_ep_combine(None, C.c_void_p(256), C.c_void_p(256), None) == m.ERR_INVALID_ARG
    assert m.lib.moe_ep_combine_noalloc(None, C.c_void_p(256), C.c_void_p(256), None) == m.ERR_INVALID_ARG
    bogus = C.c_void_p(0x1234560)
    assert m.lib.moe_ep_dispatch(bogus, C.c_void_p(256), None, None, None, C.c_void_p(256), None,
                                 counts, 0, None, None, None) == m.ERR_INVALID_ARG
    assert m.lib.moe_ep_combine_noalloc(bogus, C.c_void_p(256), C.c_void_p(256), None) == m.ERR_INVALID_ARG
    assert m.lib.moe_ep_destroy(None) == 0
    assert m.lib.moe_ep_destroy(bogus) == 0  # unknown handles are ignored


def test_agrs_argument_checks(m):
    sizes = (C.c_int32 * 4)(1, 2, 3, 4)
    plane = (m.Plane * 1)(m.Plane(256, 1024, 512, 4096, 16))
    assert m.lib.moe_ep_allgatherv(0, sizes, 1, plane, None) == m.ERR_INVALID_ARG
    assert m.lib.moe_ep_allgatherv(65, sizes, 1, plane, None) == m.ERR_INVALID_ARG
    assert m.lib.moe_ep_allgatherv(4, None, 1, plane, None) == m.ERR_INVALID_ARG
    assert m.lib.moe_ep_allgatherv(4, sizes, 0, plane, None) == m.ERR_INVALID_ARG
    assert m.lib.moe_ep_allgatherv(4, sizes, 9, plane, None) == m.ERR_INVALID_ARG
    bad = (m.Plane * 1)(m.Plane(256, 1024, 512, 4096, 0))
    assert m.lib.moe_ep_allgatherv(4, sizes, 1, bad, None) == m.ERR_INVALID_ARG
    neg = (C.c_int32 * 4)(1, -2, 3, 4)
    assert m.lib.moe_ep_allgatherv(4, neg, 1, plane, None) == m.ERR_INVALID_ARG
    zero = (C.c_int32 * 4)(0, 0, 0, 0)
    assert m.lib.moe_ep_allgatherv(4, zero, 1, plane, None) == 0  # nothing to move, no launch
    rs = m.lib.moe_ep_reduce_scatterv
    assert rs(4, sizes, 4092, C.c_void_p(256), 4096, C.c_void_p(512), 4096, None) == m.ERR_INVALID_ARG
    assert rs(4, sizes, 4096, C.c_void_p(264), 4096, C.c_void_p(512), 4096, None) == m.ERR_INVALID_ARG
    assert rs(4, sizes, 4096, C.c_void_p(256), 4104, C.c_void_p(512), 4096, None) == m.ERR_INVALID_ARG
    assert rs(4, neg, 4096, C.c_void_p(256), 4096, C.c_void_p(512), 4096, None) == m.ERR_INVALID_ARG
    assert rs(4, zero, 4096, C.c_void_p(256), 4096, C.c_void_p(512), 4096, None) == 0
