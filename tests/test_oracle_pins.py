"""Pins of the CPU oracle against facts that do not come from the oracle itself.

The pages print no worked input/output pair, so each step of the oracle is
pinned by a closed form, an invariant, a library routine (torch's bf16 and
float8_e4m3fn conversions, numpy complex arithmetic) or a hand-written
fixture under tests/golden/.  The checks are chosen so that a dropped term,
a wrong sign, a swapped pair index or a wrong rounding rule fails one of
them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# bf16 RNE converter
# ----------------------------------------------------------------------------

def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_known_values():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins (1.0);
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6.
    assert oracle.f32_to_bf16(np.array([1 + 2**-8], np.float32))[0] == 0x3F80
    assert oracle.f32_to_bf16(np.array([1 + 3 * 2**-8], np.float32))[0] == 0x3F82
    assert oracle.f32_to_bf16(np.array([-0.0], np.float32))[0] == 0x8000
    # largest finite float rounds to +inf in bf16 under RNE
    assert oracle.f32_to_bf16(np.array([np.finfo(np.float32).max], np.float32))[0] == 0x7F80


def test_bf16_matches_torch_on_random_and_structured_patterns():
    rng = np.random.default_rng(7)
    pats = [rng.integers(0, 2**32, size=1 << 22, dtype=np.uint64).astype(np.uint32)]
    # every exponent with the mantissa patterns around the rounding point
    exps = np.arange(0, 255, dtype=np.uint32) << 23
    low = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x17FFF, 0x18000, 0x18001],
                   dtype=np.uint32)
    hi = np.array([0, 1 << 16, 0x7F0000], dtype=np.uint32)
    grid = (exps[:, None, None] | hi[None, :, None] | low[None, None, :]).ravel()
    pats.append(grid)
    pats.append(grid | 0x80000000)
    u = np.concatenate(pats)
    x = u.view(np.float32)
    finite = np.isfinite(x)
    x = x[finite]
    got = oracle.f32_to_bf16(x)
    ref = _torch_bf16_bits(x)
    assert np.array_equal(got, ref)


# ----------------------------------------------------------------------------
# E4M3 RN-satfinite converter
# ----------------------------------------------------------------------------

def _golden_codes():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_codes.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            rows.append((int(c, 16), float(v)))
    return rows


def test_e4m3_decode_matches_hand_written_codes():
    for code, value in _golden_codes():
        got = oracle.e4m3_to_f64(code)
        assert got == value and math.copysign(1, got) == math.copysign(1, value), hex(code)


def test_e4m3_encode_matches_hand_written_codes():
    for code, value in _golden_codes():
        assert oracle.f64_to_e4m3(np.array([value]))[0] == code, hex(code)


def test_e4m3_all_finite_codes_round_trip():
    codes = [c for c in range(256) if (c & 0x7F) != 0x7F]
    assert len(codes) == 254
    vals = np.array([oracle.e4m3_to_f64(c) for c in codes])
    assert np.array_equal(oracle.f64_to_e4m3(vals), np.array(codes, np.uint8))
    # the decoded finite codes agree with torch's float8_e4m3fn decoding
    tv = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(vals, tv)


def test_e4m3_matches_torch_below_overflow():
    # every finite |x| <= 464 that torch converts without producing NaN:
    # random fp32 values, exact midpoints between neighbouring codes (ties)
    # and the midpoints nudged by one fp32 ulp either way.
    codes = np.arange(0, 127)
    vals = np.array([oracle.e4m3_to_f64(c) for c in codes])
    mids = (vals[:-1] + vals[1:]) / 2
    mids = np.concatenate([mids, [464.0]])
    m32 = mids.astype(np.float32)
    near = np.concatenate([m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9))])
    rng = np.random.default_rng(3)
    rand = (rng.standard_normal(1 << 20) * np.exp2(rng.integers(-12, 9, 1 << 20))).astype(np.float32)
    x = np.concatenate([near, -near, rand, vals.astype(np.float32)])
    x = x[np.abs(x) <= 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.f64_to_e4m3(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_e4m3_saturates_finite_overflow():
    x = np.array([448.0, 455.9, 464.0, 464.0001, 1000.0, 1e30, -500.0, -1e30])
    got = oracle.f64_to_e4m3(x)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_e4m3_subnormal_ties():
    # 2^-10 is halfway between 0 and 2^-9: even (0) wins; 3*2^-10 is between
    # 2^-9 (code 1, odd) and 2^-8 (code 2, even): code 2.
    got = oracle.f64_to_e4m3(np.array([2**-10, 3 * 2**-10, 2**-10 * 1.0001, -2**-11]))
    assert list(got) == [0x00, 0x02, 0x01, 0x80]


# ----------------------------------------------------------------------------
# RMSNorm
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("D", [128, 256])
def test_rmsnorm_unit_weight_gives_unit_rms(D):
    rng = np.random.default_rng(D)
    for trial in range(50):
        x = rng.standard_normal(D) * rng.uniform(1.0, 5.0)
        ms = float(np.mean(x * x))
        assert ms >= 0.5
        y = oracle.rmsnorm(x, np.ones(D, np.float32), 1, 1e-6)
        rms = math.sqrt(float(np.mean(y * y)))
        assert abs(rms - 1.0) <= 1e-6
        # and the exact value including eps
        assert abs(rms - math.sqrt(ms / (ms + 1e-6))) <= 1e-13


def test_rmsnorm_constant_vector_closed_form():
    D = 128
    w = np.linspace(0.5, 1.5, D).astype(np.float32)
    for c in [1e-3, 0.25, 3.0, -7.0]:
        x = np.full(D, c)
        y = oracle.rmsnorm(x, w, 1, 1e-6)
        expect = c / math.sqrt(c * c + 1e-6) * w.astype(np.float64)
        assert np.allclose(y, expect, rtol=1e-14, atol=0)
        yg = oracle.rmsnorm(x, w, 2, 1e-6)
        expect_g = c / math.sqrt(c * c + 1e-6) * (1.0 + w.astype(np.float64))
        assert np.allclose(yg, expect_g, rtol=1e-14, atol=0)


def test_rmsnorm_zero_row_and_policies():
    D = 128
    rng = np.random.default_rng(1)
    w = rng.standard_normal(D).astype(np.float32)
    assert np.array_equal(oracle.rmsnorm(np.zeros(D), w, 1, 1e-6), np.zeros(D))
    x = rng.standard_normal(D)
    # norm 0 is the identity
    assert np.array_equal(oracle.rmsnorm(x, w, 0, 1e-6), x)
    # Gemma with w = 0 equals plain RMSNorm with w = 1
    g = oracle.rmsnorm(x, np.zeros(D, np.float32), 2, 1e-6)
    r = oracle.rmsnorm(x, np.ones(D, np.float32), 1, 1e-6)
    assert np.array_equal(g, r)
    # the norm is per element in w: scaling one weight scales one output
    w2 = w.copy()
    w2[5] *= 2
    a = oracle.rmsnorm(x, w, 1, 1e-6)
    b = oracle.rmsnorm(x, w2, 1, 1e-6)
    assert b[5] == 2 * a[5] and np.array_equal(np.delete(a, 5), np.delete(b, 5))


# ----------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------

def _angles(D, theta, pos):
    half = D // 2
    f = theta ** (-(2.0 * np.arange(half)) / D)
    return pos * f


@pytest.mark.parametrize("style", [0, 1])
def test_rope_position_zero_is_identity(style):
    D = 128
    y = np.random.default_rng(0).standard_normal(D)
    o = oracle.rope(y, style, np.ones(D // 2), np.zeros(D // 2))
    assert np.array_equal(o, y)


@pytest.mark.parametrize("style", [0, 1])
def test_rope_is_complex_multiplication(style):
    # pair (a, b) -> (a + ib) * exp(i angle), computed by numpy's complex type
    D = 128
    rng = np.random.default_rng(11 + style)
    y = rng.standard_normal(D)
    ang = _angles(D, 1e4, 1234.0)
    o = oracle.rope(y, style, np.cos(ang), np.sin(ang))
    half = D // 2
    if style == 0:
        ia, ib = np.arange(half), np.arange(half) + half
    else:
        ia, ib = 2 * np.arange(half), 2 * np.arange(half) + 1
    z = (y[ia] + 1j * y[ib]) * np.exp(1j * ang)
    assert np.allclose(o[ia], z.real, rtol=0, atol=1e-14)
    assert np.allclose(o[ib], z.imag, rtol=0, atol=1e-14)


@pytest.mark.parametrize("style", [0, 1])
def test_rope_preserves_pair_norm_and_composes(style):
    D = 256
    rng = np.random.default_rng(5)
    y = rng.standard_normal(D)
    a, b = _angles(D, 1e6, 321.0), _angles(D, 1e6, 4567.0)
    ya = oracle.rope(y, style, np.cos(a), np.sin(a))
    yab = oracle.rope(ya, style, np.cos(b), np.sin(b))
    direct = oracle.rope(y, style, np.cos(a + b), np.sin(a + b))
    assert np.max(np.abs(yab - direct)) <= 1e-12
    half = D // 2
    idx = (np.arange(half), np.arange(half) + half) if style == 0 else (2 * np.arange(half), 2 * np.arange(half) + 1)
    n0 = y[idx[0]] ** 2 + y[idx[1]] ** 2
    n1 = ya[idx[0]] ** 2 + ya[idx[1]] ** 2
    assert np.max(np.abs(n1 - n0) / n0) <= 1e-13


def test_rope_one_hot_and_interleaved_is_permuted_neox():
    D = 128
    half = D // 2
    ang = _angles(D, 1e6, 77.0)
    c, s = np.cos(ang), np.sin(ang)
    for i in [0, 5, 63]:
        e = np.zeros(D)
        e[i] = 1.0
        o = oracle.rope(e, 0, c, s)
        assert o[i] == c[i] and o[i + half] == s[i]
        e = np.zeros(D)
        e[i + half] = 1.0
        o = oracle.rope(e, 0, c, s)
        assert o[i] == -s[i] and o[i + half] == c[i]
    # interleaved = P^-1 NeoX P with P gathering even then odd elements
    y = np.random.default_rng(2).standard_normal(D)
    perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])
    neox = oracle.rope(y[perm], 0, c, s)
    inter = oracle.rope(y, 1, c, s)
    back = np.empty(D)
    back[perm] = neox
    assert np.array_equal(inter, back)


@pytest.mark.parametrize("style", [0, 1])
@pytest.mark.parametrize("D,R", [(128, 64), (128, 32), (128, 96), (256, 128), (64, 64), (64, 16), (128, 0)])
def test_partial_rope_rotates_the_first_R_dims_only(style, D, R):
    """Partial rotary (vLLM issue, model table: RoPE on part of the head,
    NoPE on the rest): the first R dims are paired with half R/2 (NeoX) or
    as (2i, 2i+1) and multiplied by exp(i angle) as complex numbers; the
    remaining D - R dims are returned bit for bit."""
    rng = np.random.default_rng(100 + D + R + style)
    y = rng.standard_normal(D)
    half = R // 2
    ang = _angles(R, 1e4, 987.0) if R else np.zeros(0)
    o = oracle.rope(y, style, np.cos(ang), np.sin(ang), rot=R)
    assert np.array_equal(o[R:], y[R:])
    if R:
        if style == 0:
            ia, ib = np.arange(half), np.arange(half) + half
        else:
            ia, ib = 2 * np.arange(half), 2 * np.arange(half) + 1
        z = (y[ia] + 1j * y[ib]) * np.exp(1j * ang)
        assert np.allclose(o[ia], z.real, rtol=0, atol=1e-14)
        assert np.allclose(o[ib], z.imag, rtol=0, atol=1e-14)


def test_partial_rope_one_hot_pairs_use_half_of_R():
    # with D = 128 and R = 64, dim i < 32 pairs with i + 32 (not i + 64)
    D, R = 128, 64
    ang = _angles(R, 1e6, 77.0)
    c, s = np.cos(ang), np.sin(ang)
    for i in [0, 7, 31]:
        e = np.zeros(D)
        e[i] = 1.0
        o = oracle.rope(e, 0, c, s, rot=R)
        expect = np.zeros(D)
        expect[i], expect[i + R // 2] = c[i], s[i]
        assert np.array_equal(o, expect)
    for d in [64, 100, 127]:
        e = np.zeros(D)
        e[d] = 1.0
        assert np.array_equal(oracle.rope(e, 0, c, s, rot=R), e)
        assert np.array_equal(oracle.rope(e, 1, c, s, rot=R), e)


# ----------------------------------------------------------------------------
# dynamic Q scale
# ----------------------------------------------------------------------------

def test_q_scale_closed_forms():
    v = np.zeros(128, np.float32)
    assert oracle.q_scale(v, 448.0) == np.float32(1e-6 / 448.0)
    v[3], v[77] = 3.0, -5.0
    assert oracle.q_scale(v, 448.0) == np.float32(5.0 / 448.0)
    assert oracle.q_scale(v, 240.0) == np.float32(5.0 / 240.0)
    v[:] = 1e-9
    assert oracle.q_scale(v, 448.0) == np.float32(1e-6 / 448.0)
