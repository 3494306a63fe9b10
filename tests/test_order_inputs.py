"""CPU pins for the order-sensitive projection inputs and the numpy model of the documented schedule
(tests/order_model.py), which the GPU schedule checks and the GPU mutant tier rely on.

The model is pinned to the oracle: with one slice holding every group, its fold adds the same exact
terms in the oracle's ascending-k order (the zero products the oracle also adds change nothing), so
the two fp64 sums must be equal bit for bit.  The slice table is pinned to values worked out by hand
from the header's formula.  The inputs are pinned to their purpose: the documented plan, an equal
plan, the reversed slice fold and the one-slice order give different bf16 results for most outputs.
"""
import numpy as np

import oracle
import synth
from tests import order_model


def test_slice_table_worked_by_hand():
    # G = 160: P = 80, 2*floor(80*c/16) = 10c
    assert order_model.slice_bounds(160) == [0, 30, 60, 90, 120, 130, 140, 150, 160]
    # G = 33 (odd): P = 16, 2c; slice 7 also takes group 32
    assert order_model.slice_bounds(33) == [0, 6, 12, 18, 24, 26, 28, 30, 33]
    # G = 1: every slice but the last is empty
    assert order_model.slice_bounds(1) == [0] * 8 + [1]
    # G = 32: P = 16
    assert order_model.slice_bounds(32) == [0, 6, 12, 18, 24, 26, 28, 30, 32]
    assert order_model.equal_bounds(32) == [0, 4, 8, 12, 16, 20, 24, 28, 32]


def test_inputs_have_one_product_per_group_and_an_exactly_cancelling_pair():
    q, s, x = synth.order_sensitive_linear(3, 200, 1024, 4)
    G = 1024 // 32
    assert np.all(np.count_nonzero(q.reshape(200, G, 32), axis=2) <= 1)
    terms = order_model.scaled_terms(q, s, x, np.arange(200))
    big = np.abs(terms) > 2.0 ** 40
    assert np.all(big.sum(axis=2) == 2)
    assert np.all(np.where(big, terms, 0.0).sum(axis=2) == 0.0)
    assert np.all(np.abs(terms[~big]) < 2.0 ** 16)


def test_one_slice_model_equals_the_oracle_sum_exactly():
    for seed, N, K, t in ((4, 300, 5120, 3), (5, 97, 5152, 2), (6, 64, 32, 2)):
        q, s, x = synth.order_sensitive_linear(seed, N, K, t) if K > 32 else _one_group(seed, N, t)
        G = K // 32
        y = order_model.fold(order_model.scaled_terms(q, s, x, np.arange(N)), [0] + [G] * 8)
        assert np.array_equal(y, oracle.w8_linear(q, s, x))


def _one_group(seed, N, t):
    rng = np.random.default_rng(seed)
    q = np.zeros((N, 32), np.int8)
    q[:, 5] = rng.integers(-127, 128, size=N, dtype=np.int8)
    s = synth.draw_scales(rng, N, 32, 0.0)
    x = synth.draw_acts(rng, t, 32)
    return q, s, x


def test_orders_give_different_results_on_most_outputs():
    for seed, N, K in ((7, 512, 5120), (8, 2048, 1024)):
        q, s, x = synth.order_sensitive_linear(seed, N, K, 4)
        G = K // 32
        terms = order_model.scaled_terms(q, s, x, np.arange(N))
        doc = oracle.bf16_round_array(order_model.fold(terms, order_model.slice_bounds(G)))
        others = {
            "equal plan": order_model.fold(terms, order_model.equal_bounds(G)),
            "reversed fold": order_model.fold(terms, order_model.slice_bounds(G), reverse_slices=True),
            "one slice": order_model.fold(terms, [0] + [G] * 8),
        }
        for name, y in others.items():
            frac = float(np.mean(oracle.bf16_round_array(y) != doc))
            assert frac > 0.5, (name, K, frac)
