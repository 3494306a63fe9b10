"""Pins of the GEMM oracle against closed forms, exact sums and invariants (CPU only).

The oracle's definition follows the ninfer page (issue "t-dependent kernel
dispatch"), table "Where t selects arithmetic", row "ops::linear W8G32": int8
codes, one scale per 32 consecutive K elements, 16-bit activations, and the
"Proposal" section's per-column result.  Each test below would fail on a
plausible slip in it: a wrong scale index, a dropped or shifted group, a
transposed operand, a wrong sign, a rounding in the wrong place.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import bf16_bits_to_f64, bf16_round_by_search

F16_ONE = 0x3C00


def exact_y(q, s, x):
    """Exact rational y[j, n] = sum_k q[n,k] * s[n,k//32] * x[j,k], via integer scaling."""
    N, K = q.shape
    t = x.shape[0]
    sv = [[Fraction(oracle.f16_value(int(h))) for h in row] for row in s]
    xv = [[Fraction(float(v)) for v in bf16_bits_to_f64(row)] for row in x]
    y = [[Fraction(0)] * N for _ in range(t)]
    for n in range(N):
        for j in range(t):
            acc = Fraction(0)
            for g in range(K // 32):
                part = sum(int(q[n, k]) * xv[j][k] for k in range(32 * g, 32 * g + 32))
                acc += sv[n][g] * part
            y[j][n] = acc
    return y


def test_f16_decoding_matches_numpy_for_every_pattern():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_value(int(p)) for p in pats])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    assert np.all(np.signbit(ref[~both_nan]) == np.signbit(got[~both_nan]))


def test_bf16_decoding_matches_torch_for_every_pattern():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_value(int(p)) for p in pats])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))


def test_bf16_rounding_matches_table_search():
    rng = np.random.default_rng(11)
    vals = list(rng.standard_normal(3000) * np.exp2(rng.integers(-140, 130, 3000)))
    # exact midpoints between neighbouring bf16 values (ties go to even), and their neighbours
    for p in rng.integers(1, 0x7F7F, 800):
        a, b = bf16_bits_to_f64(np.array([p, p + 1], dtype=np.uint16))
        mid = (a + b) / 2
        vals += [mid, -mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf)]
    vals += [0.0, -0.0, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 2.0 ** -126, 3.3895313892515355e38,
             3.4e38, 1e39, float("inf"), -float("inf")]
    for v in vals:
        assert oracle.bf16_round(float(v)) == bf16_round_by_search(float(v)), v


def test_identity_block_reproduces_x_exactly():
    K = N = 256
    q = np.eye(N, K, dtype=np.int8)
    rng = np.random.default_rng(0)
    x = synth.draw_acts(rng, 5, K)
    for scale_bits, factor in ((F16_ONE, 1.0), (0x3000, 0.125), (0x4800, 8.0)):
        s = np.full((N, K // 32), scale_bits, dtype=np.uint16)
        y = oracle.w8_linear(q, s, x)
        assert np.array_equal(y, bf16_bits_to_f64(x) * factor)


def test_all_ones_gives_exact_integer_column_sums():
    N, K, t = 8, 5120, 4
    q = np.ones((N, K), dtype=np.int8)
    s = np.full((N, K // 32), F16_ONE, dtype=np.uint16)
    rng = np.random.default_rng(1)
    xi = rng.integers(-8, 9, size=(t, K))
    x = synth.f32_to_bf16_bits(xi.astype(np.float32))
    y = oracle.w8_linear(q, s, x)
    sums = xi.sum(axis=1)
    assert np.array_equal(y, np.repeat(sums[:, None], N, axis=1).astype(np.float64))


def test_all_ones_general_x_matches_fsum():
    N, K, t = 4, 5120, 3
    q = np.ones((N, K), dtype=np.int8)
    s = np.full((N, K // 32), F16_ONE, dtype=np.uint16)
    x = synth.draw_acts(np.random.default_rng(2), t, K)
    y = oracle.w8_linear(q, s, x)
    xv = bf16_bits_to_f64(x)
    for j in range(t):
        exact = math.fsum(xv[j])
        bound = K * 2.0 ** -53 * np.abs(xv[j]).sum()
        assert np.all(np.abs(y[j] - exact) <= bound)


def test_single_group_probe_pins_scale_indexing():
    """q[n, k] = 1 only inside group g(n): y = s[n, g(n)] * (sum of x over that group)."""
    N, K, t = 40, 512, 3
    G = K // 32
    rng = np.random.default_rng(3)
    gsel = rng.integers(0, G, size=N)
    q = np.zeros((N, K), dtype=np.int8)
    for n in range(N):
        q[n, 32 * gsel[n]:32 * gsel[n] + 32] = 1
    # scales include fp16 subnormals and zero
    s = synth.f64_to_f16_bits(np.abs(rng.normal(0, 0.02, size=(N, G))))
    s[::7, :] = rng.integers(1, 0x3FF, size=s[::7, :].shape)  # subnormal patterns
    s[5, gsel[5]] = 0
    x = synth.draw_acts(rng, t, K)
    y = oracle.w8_linear(q, s, x)
    xv = bf16_bits_to_f64(x)
    for n in range(N):
        g = gsel[n]
        sc = Fraction(oracle.f16_value(int(s[n, g])))
        for j in range(t):
            exact = sc * sum(Fraction(float(v)) for v in xv[j, 32 * g:32 * g + 32])
            assert abs(Fraction(float(y[j, n])) - exact) <= Fraction(2.0 ** -50) * abs(exact) + Fraction(2.0 ** -1070)


@pytest.mark.parametrize("N,K,t", [(16, 32, 1), (32, 64, 3), (64, 256, 16), (17, 96, 5)])
def test_brute_force_exact_rational(N, K, t):
    q, s, x = synth.small_linear(100 + N + K + t, N, K, t)
    y = oracle.w8_linear(q, s, x)
    ex = exact_y(q, s, x)
    sv = np.array([[oracle.f16_value(int(h)) for h in row] for row in s])
    xv = bf16_bits_to_f64(x)
    for j in range(t):
        for n in range(N):
            mag = float(np.sum(np.abs(q[n].astype(np.float64) * np.repeat(sv[n], 32) * xv[j])))
            err = abs(Fraction(float(y[j, n])) - ex[j][n])
            assert err <= Fraction(K * 2.0 ** -53 * mag + 2.0 ** -1070)


def test_rows_subset_and_column_independence():
    q, s, x = synth.small_linear(7, 96, 256, 9)
    full = oracle.w8_linear(q, s, x)
    rows = np.array([95, 0, 13, 13, 64], dtype=np.int64)
    sub = oracle.w8_linear(q, s, x, rows=rows)
    assert np.array_equal(sub, full[:, rows])
    one = oracle.w8_linear(q, s, x[4:5])
    assert np.array_equal(one[0], full[4])


def test_bitwise_algebraic_invariants():
    q, s, x = synth.small_linear(9, 64, 1024, 6, scale_eps=1e-4)
    y = oracle.w8_linear(q, s, x)
    neg_x = x ^ np.uint16(0x8000)
    assert np.array_equal(oracle.w8_linear(q, s, neg_x), -y)
    two_x = synth.f32_to_bf16_bits(bf16_bits_to_f64(x).astype(np.float32) * 2)
    assert np.array_equal(oracle.w8_linear(q, s, two_x), 2 * y)
    two_s = synth.f64_to_f16_bits(np.array([[oracle.f16_value(int(h)) * 2 for h in r] for r in s]))
    assert np.array_equal(oracle.w8_linear(q, two_s, x), 2 * y)
    assert np.array_equal(oracle.w8_linear(-q, s, x), -y)


def test_linearity_within_rounding():
    """y(x1 + x2) = y(x1) + y(x2) up to fp64 rounding, with x1 + x2 exact in bf16."""
    N, K, t = 32, 2048, 4
    rng = np.random.default_rng(12)
    q = synth.draw_codes(rng, N, K)
    s = synth.draw_scales(rng, N, K, 1e-4)
    a = rng.integers(-64, 65, size=(t, K)).astype(np.float32) / 16
    b = rng.integers(-64, 65, size=(t, K)).astype(np.float32) / 16
    x1, x2, x12 = (synth.f32_to_bf16_bits(v) for v in (a, b, a + b))
    assert np.array_equal(bf16_bits_to_f64(x12), (a + b).astype(np.float64))
    y1, y2, y12 = (oracle.w8_linear(q, s, v) for v in (x1, x2, x12))
    mag = oracle.w8_linear(np.abs(q), s, synth.f32_to_bf16_bits(np.abs(a) + np.abs(b)))
    assert np.all(np.abs(y12 - (y1 + y2)) <= 3 * K * 2.0 ** -53 * mag)


def test_mistakes_are_detected_by_the_pins():
    """A shifted scale index or a transposed operand changes the probe's result."""
    N, K, t = 8, 128, 2
    rng = np.random.default_rng(5)
    q = np.zeros((N, K), dtype=np.int8)
    q[:, 32:64] = 1  # group 1 only
    s = synth.f64_to_f16_bits(rng.uniform(0.5, 2.0, size=(N, K // 32)))
    x = synth.draw_acts(rng, t, K)
    y = oracle.w8_linear(q, s, x)
    xv = bf16_bits_to_f64(x)
    right = np.array([[oracle.f16_value(int(s[n, 1])) * xv[j, 32:64].sum() for n in range(N)] for j in range(t)])
    wrong = np.array([[oracle.f16_value(int(s[n, 2])) * xv[j, 32:64].sum() for n in range(N)] for j in range(t)])
    assert np.allclose(y, right, rtol=1e-12)
    assert not np.allclose(y, wrong, rtol=1e-6)


def test_absolute_mass_is_the_sum_of_absolute_terms():
    """The oracle's second output, sum_k |q s x| (the fp32 accumulation floor's scale): for all-ones
    weights with unit scales and x on a 1/16 grid it is the exact sum of |x| (math.fsum); for random
    signed codes and activations it equals, bit for bit, the plain projection of |q| and |x| (every term
    is the same exact fp64 product, summed in the same order); it is never below |y|."""
    K, t = 5120, 6
    rng = np.random.default_rng(21)
    xi = rng.integers(-64, 65, size=(t, K)).astype(np.float32) / 16
    x = synth.f32_to_bf16_bits(xi)
    q1 = np.ones((8, K), dtype=np.int8)
    s1 = np.full((8, K // 32), F16_ONE, dtype=np.uint16)
    _, m1 = oracle.w8_linear(q1, s1, x, mass=True)
    for j in range(t):
        assert np.all(m1[j] == math.fsum(abs(float(v)) for v in xi[j]))
    q, s, x2 = synth.small_linear(22, 64, 1024, 5, 0.0)
    y, m = oracle.w8_linear(q, s, x2, mass=True)
    y_abs = oracle.w8_linear(np.abs(q.astype(np.int16)).astype(np.int8), s, x2 & np.uint16(0x7FFF))
    assert np.array_equal(m, y_abs)
    assert np.all(m >= np.abs(y))
    assert np.array_equal(oracle.w8_linear(q, s, x2), y)

