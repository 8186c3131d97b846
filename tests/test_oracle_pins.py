"""Pins of the CPU oracle against facts fixed outside it: library routines
(numpy / scipy / torch), closed forms, invariants and brute force.  These run
without a GPU.  Each test names the page passage (or the plain mathematics)
that fixes the expected value."""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import ref

RNG = np.random.default_rng(20260)


# ---------------------------------------------------------------- number formats

def test_f32_to_f16_matches_numpy_rne():
    # IEEE binary16 round-to-nearest-even, as numpy's float32 -> float16 cast
    x = np.concatenate([
        RNG.standard_normal(200000).astype(np.float32) * np.float32(10.0) ** RNG.integers(-9, 6, 200000),
        np.float32([0.0, -0.0, 65504, 65519.996, 65520, 1e9, -1e9, np.inf, -np.inf, 2.0 ** -24, 2.0 ** -25,
                    2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 6.1035156e-05, 6.097555e-05]),
        # exact ties between adjacent halves
        (np.arange(1, 2000, dtype=np.float32) + np.float32(0.5)) * np.float32(2.0 ** -10),
    ]).astype(np.float32)
    got = ref.f32_to_f16(x)
    want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_f16_bf16_widening():
    for h in list(range(0, 65536, 7)) + [0x7bff, 0x0001, 0x03ff, 0x8001]:
        want = float(np.uint16(h).view(np.float16))
        got = ref.f16_to_f64(h)
        assert (math.isnan(got) and math.isnan(want)) or got == want
    for b in range(0, 65536, 13):
        want = torch.tensor([b], dtype=torch.int32).to(torch.int16).view(torch.bfloat16).double().item()
        got = ref.bf16_to_f64(b)
        assert (math.isnan(got) and math.isnan(want)) or got == want


# ---------------------------------------------------------------- INT4 quantizer

def _deq(s, z, q):
    s64 = s.view(np.float16).astype(np.float64)
    z64 = z.view(np.float16).astype(np.float64)
    return q.astype(np.float64) * s64[:, None] + z64[:, None]


def test_int4_worked_example_form_on_exact_grids():
    # BellowsKV "Worked Example": s = (max - min) / (2^bits - 1), q = round((v - min) / s) with Python's
    # round (half to even).  On groups whose min and scale are exact fp16 values the stored-fp16 step is
    # the identity, so the oracle must give exactly the page's codes -- ties included.
    for trial in range(300):
        lo = RNG.integers(-64, 64) / 64.0
        s = RNG.integers(1, 64) / 1024.0
        k = RNG.integers(0, 16, 32)
        v = lo + (k + RNG.choice([0.0, 0.5, 0.25, -0.25], 32)) * s
        v = np.clip(v, lo, lo + 15 * s)
        v[0], v[1] = lo, lo + 15 * s
        v32 = v.astype(np.float32)
        assert np.array_equal(v32.astype(np.float64), v)
        S, Z, Q = ref.quant_int4(v32[None])
        assert S[0] == np.float16(s).view(np.uint16) and Z[0] == np.float16(lo).view(np.uint16)
        page_codes = [round((float(x) - lo) / s) for x in v]
        assert Q[0].tolist() == page_codes, trial


def test_int4_brute_force_nearest_level_and_bounds():
    x = (RNG.standard_normal((20000, 32)) * RNG.uniform(0.01, 3.0, (20000, 1))).astype(np.float32)
    S, Z, Q = ref.quant_int4(x)
    s64 = S.view(np.float16).astype(np.float64)
    z64 = Z.view(np.float16).astype(np.float64)
    levels = np.arange(16)[None, None, :] * s64[:, None, None] + z64[:, None, None]
    dist = np.abs(x.astype(np.float64)[:, :, None] - levels)
    best = dist.argmin(-1)
    mism = best != Q
    if mism.any():
        # only near-ties may differ (the code is taken in fp32): the two distances agree to rounding
        d_code = np.take_along_axis(dist, Q[..., None].astype(np.int64), -1)[..., 0]
        d_best = dist.min(-1)
        assert np.all((d_code - d_best)[mism] <= 1e-6 * s64[:, None].repeat(32, 1)[mism])
    assert Q.max() <= 15
    # endpoints: the group minimum maps to 0, the maximum to 15
    assert np.all(Q[np.arange(len(x)), x.argmin(1)] == 0)
    assert np.all(Q[np.arange(len(x)), x.argmax(1)] == 15)
    # reconstruction error is at most half a step, plus the fp16 rounding of the endpoints
    err = np.abs(_deq(S, Z, Q) - x)
    lo, hi = x.min(1).astype(np.float64), x.max(1).astype(np.float64)
    slack = np.maximum(np.abs(lo - z64), np.abs(hi - (z64 + 15 * s64)))
    assert np.all(err <= 0.5 * s64[:, None] + slack[:, None] + 1e-12)


@pytest.mark.parametrize("bits", [2, 3])
def test_low_bit_brute_force_nearest_level_and_bounds(bits):
    # the INT3 and 2-bit variants of the same min/max quantizer ("BellowsKV Architecture ...", "Reading the
    # Retention Table"): 2^bits - 1 steps over the group's range
    L = (1 << bits) - 1
    x = (RNG.standard_normal((20000, 32)) * RNG.uniform(0.01, 3.0, (20000, 1))).astype(np.float32)
    S, Z, Q = ref.quant_intb(x, bits)
    s64 = S.view(np.float16).astype(np.float64)
    z64 = Z.view(np.float16).astype(np.float64)
    levels = np.arange(L + 1)[None, None, :] * s64[:, None, None] + z64[:, None, None]
    dist = np.abs(x.astype(np.float64)[:, :, None] - levels)
    mism = dist.argmin(-1) != Q
    if mism.any():
        d_code = np.take_along_axis(dist, Q[..., None].astype(np.int64), -1)[..., 0]
        assert np.all((d_code - dist.min(-1))[mism] <= 1e-6 * s64[:, None].repeat(32, 1)[mism])
    assert Q.max() <= L
    assert np.all(Q[np.arange(len(x)), x.argmin(1)] == 0)
    assert np.all(Q[np.arange(len(x)), x.argmax(1)] == L)
    # the scale is the fp16 of range / (2^bits - 1)
    rng = x.max(1) - x.min(1)
    assert np.array_equal(S, ref.f32_to_f16(rng / np.float32(L)))
    # 4 bits through the general form is the INT4 quantizer
    assert all(np.array_equal(a, b) for a, b in zip(ref.quant_intb(x[:500], 4), ref.quant_int4(x[:500])))


def test_int4_requantize_round_trip():
    # quantizing the dequantized group again returns the same codes and the same fp16 scale/zero
    x = (RNG.standard_normal((50000, 32)) * (np.arange(1, 33) ** -0.7)).astype(np.float32)
    S, Z, Q = ref.quant_int4(x)
    y = _deq(S, Z, Q).astype(np.float32)
    S2, Z2, Q2 = ref.quant_int4(y)
    assert np.array_equal(S, S2) and np.array_equal(Z, Z2) and np.array_equal(Q, Q2)


def test_int4_degenerate_group():
    S, Z, Q = ref.quant_int4(np.full((1, 32), 0.3, np.float32))
    assert S[0] == 0 and Z[0] == np.float16(0.3).view(np.uint16) and not Q.any()


# ---------------------------------------------------------------- 2-bit residual quantizer

def test_res2_brute_force_nearest_level():
    y = (RNG.standard_normal((20000, 128)) * 0.05).astype(np.float32)
    S, Q = ref.quant_res2(y)
    s64 = S.view(np.float16).astype(np.float64)
    levels = (np.arange(4) - 1.5)[None, None, :] * s64[:, None, None]
    dist = np.abs(y.astype(np.float64)[:, :, None] - levels)
    best = dist.argmin(-1)
    mism = best != Q
    d_code = np.take_along_axis(dist, Q[..., None].astype(np.int64), -1)[..., 0]
    assert np.all((d_code - dist.min(-1))[mism] <= 1e-6 * np.broadcast_to(s64[:, None], mism.shape)[mism])
    # scale = max |y| / 1.5 (stored fp16): the largest magnitude sits on an outer level
    amax = np.abs(y).max(1)
    assert np.allclose(s64, amax / 1.5, rtol=2 ** -11)
    idx = np.abs(y).argmax(1)
    assert np.all(np.isin(Q[np.arange(len(y)), idx], [0, 3]))


def test_res2_zero_vector():
    S, Q = ref.quant_res2(np.zeros((1, 128), np.float32))
    assert S[0] == 0 and np.all(Q == 2)


# ---------------------------------------------------------------- Hadamard

@pytest.mark.parametrize("n", [2, 16, 64, 128])
def test_hadamard_is_sylvester_orthonormal(n):
    H = ref.hadamard(n)
    assert np.array_equal(H * math.sqrt(n), scipy.linalg.hadamard(n).astype(np.float64))
    assert np.allclose(H @ H, np.eye(n), atol=1e-14)
    assert np.array_equal(H, H.T)
    v = RNG.standard_normal(n)
    assert np.isclose(np.linalg.norm(H @ v), np.linalg.norm(v))


# ---------------------------------------------------------------- RoPE

def test_rope_closed_forms():
    # d = 2: one pair at frequency theta^0 = 1, so the pair turns by pos radians
    assert np.allclose(ref.rope([1.0, 0.0], math.pi / 2, 10000.0), [0.0, 1.0], atol=1e-15)
    assert np.allclose(ref.rope([0.0, 1.0], math.pi / 2, 10000.0), [-1.0, 0.0], atol=1e-15)
    x = RNG.standard_normal(128)
    assert np.array_equal(ref.rope(x, 12345, 0.0), x)          # theta 0 switches it off
    assert np.array_equal(ref.rope(x, 0, 500000.0), x)          # position 0 is the identity


def test_rope_rotate_half_as_complex_multiplication():
    # rotate-half pairs (x_j, x_{j+d/2}) behave as z_j = x_j + i x_{j+d/2} times exp(i pos theta^(-2j/d))
    d, theta, pos = 128, 500000.0, 98765.0
    x = RNG.standard_normal(d)
    z = (x[: d // 2] + 1j * x[d // 2:]) * np.exp(1j * pos * theta ** (-2.0 * np.arange(d // 2) / d))
    assert np.allclose(ref.rope(x, pos, theta), np.concatenate([z.real, z.imag]), atol=1e-12)


def test_rope_relative_position_and_norm():
    d, theta = 128, 500000.0
    q, k = RNG.standard_normal(d), RNG.standard_normal(d)
    a = ref.rope(q, 131072, theta) @ ref.rope(k, 70000, theta)
    b = ref.rope(q, 131072 - 70000, theta) @ ref.rope(k, 0, theta)
    assert abs(a - b) < 1e-9 * np.linalg.norm(q) * np.linalg.norm(k)
    assert np.isclose(np.linalg.norm(ref.rope(q, 5555, theta)), np.linalg.norm(q))
