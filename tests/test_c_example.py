"""The plain C example (combine_route_mask_amd/examples/moe_ep_example.c)
uses the exchange through include/moe_ep.h alone: it compiles as strict
C99 with every warning an error, links only libmoe_ep.so and the HIP
runtime, and refuses to run without a gfx950 device.  On the GPU it runs a
small dispatch, plays identity experts on the host from the returned id
and weight planes, combines, and checks that every token comes back as its
row times the sum of its top-k weights (the combine's contract) with the
rows past each rank's token count untouched; then it all-gathers the token
rows and ids (every rank gets every rank's rows, byte for byte) and
reduce-scatters (q + 1)-scaled copies of them (each result row equal, bit
for bit, to the fp32 ascending-rank sum rounded to bf16)."""
import os
import subprocess

import pytest

from combine_route_mask_amd import build


def _lib():
    if not os.path.exists(build.LIB):
        build.build()
    return build.LIB


def test_example_compiles_as_c99_and_needs_a_gfx950_device(tmp_path):
    _lib()
    exe = build.build_example(out=str(tmp_path / "moe_ep_example"))
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    # 0 with "ok" where a gfx950 device is present, else exit code 2
    if res.returncode == 0:
        assert res.stdout.startswith("ok")
    else:
        assert res.returncode == 2, res.stdout + res.stderr
        assert "no gfx950 device" in res.stderr


@pytest.mark.gpu
def test_example_runs_a_step_through_the_c_abi():
    _lib()
    exe = build.EXAMPLE if os.path.exists(build.EXAMPLE) else build.build_example()
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok:") and "reduce-scattered bit-exact" in res.stdout, res.stdout
    print(res.stdout.strip(), flush=True)
