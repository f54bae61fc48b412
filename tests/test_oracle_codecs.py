"""Pins of the oracle's number formats against library routines and
closed forms: bf16 (torch), OCP e4m3fn (torch.float8_e4m3fn), the
power-of-two block-scale rule (its defining inequality) and a hand-worked
block (tests/golden/fp8_block.json)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

import oracle


def test_bf16_decode_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_to_double(b) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_bf16_encode_matches_torch_on_float32_values():
    # every fp32 value is exact in double, so RNE(double) must equal
    # torch's fp32 -> bf16 conversion (round to nearest even)
    rng = np.random.default_rng(11)
    u = rng.integers(0, 1 << 32, size=20000, dtype=np.uint64).astype(np.uint32)
    # add ties: patterns whose low 16 bits are exactly 0x8000
    ties = (rng.integers(0, 1 << 16, size=2000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    u = np.concatenate([u, ties, np.array([0, 0x80000000, 0x7F800000, 0xFF800000,
                                           0x7F7FFFFF, 0x00000001, 0x007FFFFF], np.uint32)])
    f = u.view(np.float32)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.double_to_bf16(float(x)) for x in f], dtype=np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], want[~nan])
    # NaN stays NaN (any payload)
    assert all((g & 0x7F80) == 0x7F80 and (g & 0x7F) for g in got[nan])


def _exact_rne_bf16(x: float) -> int:
    """bf16 RNE of a double by exact rational arithmetic (normal range)."""
    sign = 0x8000 if x < 0 else 0
    a = Fraction(abs(x))
    E = math.floor(math.log2(abs(x)))
    while Fraction(2) ** E > a:
        E -= 1
    while Fraction(2) ** (E + 1) <= a:
        E += 1
    q = a / Fraction(2) ** (E - 7)
    r = math.floor(q)
    rem = q - r
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and r % 2 == 1):
        r += 1
    if r == 256:
        E, r = E + 1, 128
    return sign | ((E + 127) << 7) | (r - 128)


def test_bf16_encode_single_rounding_of_doubles():
    # doubles just beside a bf16 midpoint: a double -> float -> bf16 chain
    # would round twice; the oracle must round once
    rng = np.random.default_rng(12)
    for _ in range(3000):
        base = float(rng.standard_normal() * 2.0 ** rng.integers(-20, 20))
        b = oracle.double_to_bf16(base)
        lo = oracle.bf16_to_double(b)
        step = math.ldexp(1.0, math.frexp(lo)[1] - 8) if lo != 0 else 1e-30
        for x in (lo + step / 2, lo + step / 2 + step * 2 ** -30, lo + step / 2 - step * 2 ** -30):
            if x == 0:
                continue
            assert oracle.double_to_bf16(x) == _exact_rne_bf16(x), x


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_to_double(c) for c in codes])
    nan = np.isnan(want)
    assert nan.sum() == 2  # S.1111.111
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(13)
    vals = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 8, 20000),
        # exact midpoints between neighbouring codes (ties to even)
        [(torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).double().item() +
          torch.tensor([c + 1], dtype=torch.uint8).view(torch.float8_e4m3fn).double().item()) / 2
         for c in range(0, 125)],
        [0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 2.0 ** -6],
    ]).astype(np.float32)  # float32 so torch's cast sees the same value
    want = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.double_to_e4m3(float(v)) for v in vals], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_fp8_block_exponent_is_smallest_power_that_fits():
    rng = np.random.default_rng(14)
    amaxes = np.concatenate([np.abs(rng.standard_normal(3000)) * 2.0 ** rng.integers(-60, 60, 3000),
                             [448.0 * 2.0 ** e for e in range(-20, 20)],
                             [np.nextafter(448.0 * 2.0 ** e, np.inf) for e in range(-20, 20)]])
    for a in amaxes:
        a = float(a)
        e = oracle.fp8_block_exponent(a)
        assert a <= 448.0 * 2.0 ** e
        assert a > 448.0 * 2.0 ** (e - 1)
        # closed form where log2 is unambiguous
        assert e == math.ceil(math.log2(a / 448.0)) or abs(math.log2(a / 448.0) - round(math.log2(a / 448.0))) < 1e-12
    assert oracle.fp8_block_exponent(0.0) == -127
    assert oracle.fp8_block_exponent(1e-40) == -127


def test_fp8_codes_match_torch_scaled_cast():
    # quantise_row's codes are e4m3(x * 2^-e): check against torch's cast
    rng = np.random.default_rng(15)
    x = torch.from_numpy(rng.standard_normal(32 * 64).astype(np.float32)
                         * 2.0 ** rng.integers(-8, 8, 32 * 64)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    codes, scales = oracle.fp8_quantize_row(bits)
    xb = x.float().reshape(64, 32)
    for b in range(64):
        e = int(scales[b]) - 127
        assert e == oracle.fp8_block_exponent(float(xb[b].abs().max()))
        want = (xb[b] * 2.0 ** -e).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes[b * 32:(b + 1) * 32], want)


def test_fp8_nonfinite_block():
    x = np.zeros(64, np.uint16)
    x[3] = 0x7FC0  # NaN in block 0
    x[40] = 0x3F80  # 1.0 in block 1
    codes, scales = oracle.fp8_quantize_row(x)
    assert scales[0] == 0xFF and np.all(codes[:32] == 0x7F)
    assert math.isnan(oracle.fp8_dequant(codes[0], scales[0]))
    assert oracle.fp8_dequant(codes[40], scales[1]) == 1.0


def test_fp8_golden_block(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "fp8_block.json")))
    x = np.zeros(32, np.float32)
    x[:len(g["x"])] = g["x"]
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy(), x)
    codes, scales = oracle.fp8_quantize_row(bits)
    assert scales[0] == g["expect_scale"]
    n = len(g["expect_codes_head"])
    assert list(codes[:n]) == g["expect_codes_head"]
    assert all(c == 0 for c in codes[n:])
    deq = [oracle.fp8_dequant(c, scales[0]) for c in codes[:n]]
    assert deq == g["expect_dequant_head"]
