"""The payload encoders of the input generator against the formats'
definitions (dispatch moves these bytes unread, so they matter only for
realistic inputs, but a wrong encoder would make the MXFP8 / NVFP4 /
DeepSeekFp8 workloads something else).

- e2m1 (OCP MX, FP4): sign bit 3, exponent bits 2..1, mantissa bit 0;
  exponent 0 is subnormal (m * 0.5), else 2^(e-1) * (1 + m/2).
- e8m0 scale codes: 2^(code - 127).
- e4m3fn decode is torch's float8_e4m3fn (pinned against its definition
  in test_oracle_codecs.py); nearest-value checks here are brute force
  over every code."""
import numpy as np
import pytest
import torch

import workloads as W


def e2m1_value(code: int) -> float:
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
    return -mag if s else mag


E2M1 = np.array([e2m1_value(c) for c in range(16)])
E4M3 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
E4M3_FINITE = np.where(np.isfinite(E4M3), E4M3, np.nan)


def _rows(seed, shape):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(*shape, generator=g)
    x = x * torch.pow(2.0, torch.randint(-12, 12, shape[:-1] + (1,), generator=g).float())
    return x.to(torch.bfloat16)


def test_e2m1_table_is_the_encoder_grid():
    assert list(E2M1[:8]) == list(W._E2M1_GRID)
    assert list(E2M1[8:]) == [-v for v in W._E2M1_GRID]


def test_nvfp4_nearest_code_ties_to_even():
    x = _rows(1, (6, 64))
    packed, scales = W.encode_nvfp4(x)
    codes = np.stack([packed.numpy() & 0xF, packed.numpy() >> 4], axis=-1).reshape(6, 64)
    s = scales.view(torch.float8_e4m3fn).float().numpy().repeat(16, axis=1)
    xf = x.float().numpy()
    amax = np.abs(xf.reshape(6, 4, 16)).max(-1).repeat(16, axis=1)
    # scale: e4m3 rounding of amax / 6 (nearest e4m3 value, brute force)
    want_s = np.array([[E4M3_FINITE[np.nanargmin(np.abs(E4M3_FINITE - a / 6.0))] for a in row] for row in amax])
    assert np.array_equal(s, np.abs(want_s))
    for i in range(6):
        for j in range(64):
            y = xf[i, j] / s[i, j] if s[i, j] > 0 else 0.0
            d = np.abs(E2M1[:8] - min(abs(y), 6.0))
            best = np.flatnonzero(d == d.min())
            mag = best[best % 2 == 0][0] if len(best) > 1 else best[0]  # ties to the even code
            got = codes[i, j]
            assert (got & 7) == mag, (i, j, y, got)
            if mag != 0:
                assert (got >> 3) == (1 if y < 0 else 0)


def test_mxfp8_shared_exponent_and_elements():
    x = _rows(2, (5, 96))
    codes, scales = W.encode_mxfp8(x)
    xf = x.float().numpy().reshape(5, 3, 32)
    e = scales.numpy().astype(np.int64).reshape(5, 3) - 127
    amax = np.abs(xf).max(-1)
    # shared exponent: floor(log2 amax) - 8 (the largest e4m3 power of two is 2^8)
    assert np.array_equal(e, np.floor(np.log2(amax)).astype(np.int64) - 8)
    dec = E4M3[codes.numpy().astype(np.int64)].reshape(5, 3, 32)
    scaled = np.clip(xf * 2.0 ** (-e[..., None]), -448, 448)
    err = np.abs(dec - scaled)
    # nearest: no finite e4m3 value is strictly closer
    best = np.nanmin(np.abs(E4M3_FINITE[None, :] - scaled.reshape(-1, 1)), axis=1).reshape(scaled.shape)
    assert np.all(err <= best)


def test_deepseek_fp8_scale_and_elements():
    x = _rows(3, (4, 256))
    codes, scales = W.encode_deepseek_fp8(x)
    xf = x.float().numpy().reshape(4, 2, 128)
    sc = scales.contiguous().view(torch.float32).numpy().reshape(4, 2)
    amax = np.abs(xf).max(-1)
    assert np.allclose(sc, (torch.from_numpy(amax).float() / 448.0).numpy(), rtol=0, atol=0)
    dec = E4M3[codes.numpy().astype(np.int64)].reshape(4, 2, 128)
    y = (torch.from_numpy(xf) / torch.from_numpy(sc)[..., None]).numpy()
    best = np.nanmin(np.abs(E4M3_FINITE[None, :] - y.reshape(-1, 1)), axis=1).reshape(y.shape)
    assert np.all(np.abs(dec - y) <= best)


def test_zipf_routing_is_popularity_sampling_without_replacement():
    """The MXFP8 workload's routing (k = 8 distinct of E = 256 experts,
    p_e proportional to (e+1)^-1.2, drawn by Gumbel-top-k) against an
    independent sampler: numpy's sequential weighted draws without
    replacement.  Checks distinct ids, the first draw's distribution
    (categorical in p), every expert's inclusion rate and the mean number
    of destination ranks per token at P = 8 (about 2.90 in identity order,
    against 5.29 for uniform routing), which sets the workload's bytes."""
    E, k, P, s = 256, 8, 8, 1.2
    n_g, n_c = 60000, 20000
    ids = W.draw_topk_ids(np.random.default_rng(123), n_g, E, k, "zipf", s)
    assert all(len(set(r)) == k for r in ids[:2000])
    assert ids.min() >= 0 and ids.max() < E
    p = np.arange(1, E + 1, dtype=np.float64) ** -s
    p /= p.sum()
    rng = np.random.default_rng(7)
    ref = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(n_c)])
    # first draw (the ids come ordered by their key): categorical in p
    f = np.bincount(ids[:, 0], minlength=E) / n_g
    assert np.all(np.abs(f - p) <= 5 * np.sqrt(p * (1 - p) / n_g) + 1e-4)
    # inclusion rates of every expert agree with the sequential sampler
    inc_g = np.bincount(ids.ravel(), minlength=E) / n_g
    inc_c = np.bincount(ref.ravel(), minlength=E) / n_c
    se = np.sqrt(inc_g * (1 - inc_g) / n_g + inc_c * (1 - inc_c) / n_c)
    assert np.all(np.abs(inc_g - inc_c) <= 5 * se + 1e-4)
    # mean fan-out over P = 8 ranks of 32 contiguous experts
    fan_g = np.array([len(np.unique(r // (E // P))) for r in ids])
    fan_c = np.array([len(np.unique(r // (E // P))) for r in ref])
    se_f = np.sqrt(fan_g.var() / n_g + fan_c.var() / n_c)
    assert abs(fan_g.mean() - fan_c.mean()) <= 5 * se_f
    assert fan_g.mean() == pytest.approx(2.90, abs=0.02)
