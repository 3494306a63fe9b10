"""Pins of the column-local glue references (RMSNorm, SwiGLU, residual add) used between the
projections of one decode layer (the ninfer page's note that norms and other per-lane ops are
invariant).  Checked against closed forms and 60-digit decimal arithmetic (CPU only)."""
from decimal import Decimal

import numpy as np

import oracle
import synth
from tests.helpers import bf16_bits_to_f64


def test_rmsnorm_constant_column_is_sign_without_eps():
    x = synth.f32_to_bf16_bits(np.array([[3.5] * 64, [-0.25] * 64], dtype=np.float32))
    y = oracle.rmsnorm(x, 0.0)
    assert np.array_equal(y[0], np.ones(64)) and np.array_equal(y[1], -np.ones(64))


def test_rmsnorm_against_decimal():
    rng = np.random.default_rng(0)
    x = synth.draw_acts(rng, 3, 96)
    w = synth.f32_to_bf16_bits(rng.uniform(0.5, 1.5, 96).astype(np.float32))
    eps = 1e-6
    y = oracle.rmsnorm(x, eps, weight=w)
    xv, wv = bf16_bits_to_f64(x), bf16_bits_to_f64(w[None])[0]
    for j in range(3):
        ms = sum(Decimal(float(v)) ** 2 for v in xv[j]) / 96 + Decimal(eps)
        r = ms.sqrt()
        for h in range(0, 96, 7):
            want = Decimal(float(xv[j, h])) * Decimal(float(wv[h])) / r
            assert abs(Decimal(float(y[j, h])) - want) <= abs(want) * Decimal("1e-15")


def test_swiglu_closed_forms_and_decimal():
    g = np.array([0.0, 30.0, -30.0, 1.0, -2.5, 0.125], dtype=np.float32)
    u = np.array([5.0, 2.0, 7.0, 3.0, 1.0, -4.0], dtype=np.float32)
    gu = synth.f32_to_bf16_bits(np.concatenate([g, u])[None])
    y = oracle.swiglu(gu)[0]
    assert y[0] == 0.0
    for i in range(6):
        G, U = Decimal(float(g[i])), Decimal(float(u[i]))
        want = G / (1 + (-G).exp()) * U
        assert abs(Decimal(float(y[i])) - want) <= abs(want) * Decimal("1e-15") + Decimal("1e-300")


def test_add_is_exact():
    rng = np.random.default_rng(2)
    a, b = synth.draw_acts(rng, 2, 50), synth.draw_acts(rng, 2, 50)
    y = oracle.add(a, b)
    assert np.array_equal(y, bf16_bits_to_f64(a) + bf16_bits_to_f64(b))
