"""moe_ep_workspace_bytes on random parameter sets against the contract in
include/moe_ep.h, restated here on its own: every invalid set gives 0 (and
moe_ep_create rejects it before touching a device), every valid one the sum
of its planes, each starting 256-byte aligned, in the documented order
(payload, scales, extra bytes, ids, weights, slot list, counts, source
offsets, token masks, EPLB statistics, then, for an FP8 combine, the
landing codes and scales).  No kernel runs."""
import ctypes as C
import os

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from tests.conftest import ROOT

INT32_MAX = (1 << 31) - 1


@pytest.fixture(scope="module")
def m():
    lib = os.path.join(ROOT, "combine_route_mask_amd", "libmoe_ep.so")
    if not os.path.exists(lib):
        from combine_route_mask_amd import build
        build.build()
    from combine_route_mask_amd import moe_ep
    return moe_ep


def _row_bytes(fmt, H):
    """(payload row, scale row) bytes of a dispatch format, or None."""
    return {0: (2 * H, 0), 1: (H, H // 32), 2: (H // 2, H // 16), 3: (H, H // 128 * 4)}.get(fmt)


def expected_bytes(P, E, k, T, H, fmt, comb, hw, xb, n):
    """0 when the header's rules reject the set, else the region size."""
    if not (1 <= P <= 64) or E < 1 or E % 4 or E % P or not (1 <= k <= 64) or T < 1 or H < 1:
        return 0
    if P * T > INT32_MAX or hw not in (0, 1) or comb not in (0, 1) or _row_bytes(fmt, H) is None:
        return 0
    if H % 8 or (fmt != 0 and H % 32) or (fmt == 3 and H % 128) or (comb == 1 and H % 32):
        return 0
    if xb < 0 or not (0 <= n <= E):
        return 0
    row, srow = _row_bytes(fmt, H)
    S = P * T
    per_slot = row + srow + xb + 8 * k + 4 + (H + H // 32 if comb == 1 else 0)
    if per_slot > (1 << 46) // S:
        return 0
    off = 0
    for b in (S * row, S * srow, S * xb, S * k * 4, S * k * 4 if hw else 0, S * 4, P * 4, (P + 1) * 4,
              T * 8, P * n * 4) + ((S * H, S * (H // 32)) if comb == 1 else ()):
        off = (off + b + 255) // 256 * 256
    return off


params = st.fixed_dictionaries({
    "P": st.one_of(st.integers(-1, 70), st.sampled_from([1, 8, 16, 64])),
    "E": st.one_of(st.integers(-4, 300), st.sampled_from([4, 16, 64, 128, 256, 512])),
    "k": st.one_of(st.integers(-1, 70), st.sampled_from([1, 2, 4, 8])),
    "T": st.one_of(st.integers(-1, 5000), st.sampled_from([1, 128, 512, 1 << 25, 1 << 26])),
    "H": st.one_of(st.integers(-8, 20000), st.sampled_from([8, 64, 128, 256, 4096, 7168, 7176, 7200])),
    "fmt": st.integers(-1, 4),
    "comb": st.integers(-1, 2),
    "hw": st.integers(-1, 2),
    "xb": st.one_of(st.integers(-3, 5000), st.just(0)),
    "n": st.one_of(st.integers(-2, 600), st.just(0)),
})


@settings(max_examples=400, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(params)
def test_workspace_bytes_follow_the_contract(m, p):
    cp = m.Params(p["P"], p["E"], p["k"], p["T"], p["H"], p["fmt"], p["comb"], p["hw"], p["E"], p["xb"], p["n"])
    got = m.lib.moe_ep_workspace_bytes(C.byref(cp))
    want = expected_bytes(p["P"], p["E"], p["k"], p["T"], p["H"], p["fmt"], p["comb"], p["hw"], p["xb"], p["n"])
    assert got == want, (p, got, want)
    if want == 0:
        assert m.lib.moe_ep_last_error().decode() != ""
        h = C.c_void_p()
        # rejected on the parameters, before the workspace or a device is looked at
        assert m.lib.moe_ep_create(C.byref(cp), C.c_void_p(4096), 1 << 40, C.byref(h)) in \
            (m.ERR_INVALID_ARG, m.ERR_UNSUPPORTED, m.ERR_CAPACITY)
        assert not h.value
