"""Pins of the fixed-order fp32 logprob oracle (CPU only).

The algorithm is the tokenspeed "Numerics envelopes" page's blockwise logprob:
alignment.trainer table, row "--logprob-order blockwise" (row max, shift,
target gather, sum_exp over fixed vocabulary blocks with an in-block tree and a
left fp32 fold across blocks, negative cross-entropy); the "Logprobs" section
(exact bf16 -> fp32 widening, -0.0 for a certain token); and the block_sumexp
leaf contract paragraph.  EXP32 / LOG32 are read as the correctly rounded fp32
exponential and logarithm; they are pinned here against 60-digit decimal
arithmetic.
"""
import math
from decimal import Decimal

import numpy as np
import pytest

import oracle
import synth
from tests.helpers import exp_rn32, ln_rn32, rn32


def bf16(v):
    """bf16 bit pattern (int) of one value."""
    return int(synth.f32_to_bf16_bits(np.array([v], dtype=np.float32))[0])


def f32_bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


# ------------------------------------------------------------ EXP32 / LOG32
def test_exp32_correctly_rounded_against_decimal():
    rng = np.random.default_rng(0)
    xs = [np.float32(v) for v in rng.uniform(-104, 89, 3000)]
    xs += [np.float32(v) for v in rng.uniform(-104, -87, 1500)]  # subnormal and near-underflow results
    xs += [np.float32(v) for v in rng.uniform(-1e-3, 1e-3, 500)]
    lo = np.float32(-150 * math.log(2))  # e^x = 2^-150 is the last rounding boundary before 0
    for d in range(-40, 41):
        xs.append(np.float32(lo + np.float32(d) * np.float32(7.62939453125e-06)))
    xs += [np.float32(v) for v in (0.0, -0.0, 1e-45, -1e-45, 88.72283, 88.72284, -103.97208, -103.9721, -104.0)]
    x = np.array(xs, dtype=np.float32)
    got = oracle.exp32(x)
    want = np.array([exp_rn32(float(v)) for v in x], dtype=np.float32)
    assert np.array_equal(f32_bits(got), f32_bits(want))


def test_exp32_special_values():
    x = np.array([np.nan, -np.inf, np.inf, -200.0, 100.0], dtype=np.float32)
    got = oracle.exp32(x)
    assert np.isnan(got[0]) and got[1] == 0 and np.isinf(got[2]) and got[3] == 0 and np.isinf(got[4])


def test_log32_correctly_rounded_against_decimal():
    rng = np.random.default_rng(1)
    xs = list(rng.uniform(1, 2, 1500).astype(np.float32))
    xs += list(np.exp2(rng.uniform(0, 18, 1500)).astype(np.float32))
    one = np.float32(1.0)
    for k in range(1, 200):
        xs.append(np.float32(1 + k * 2.0 ** -23))
    xs += [np.float32(v) for v in (1.0, 2.0, 248320.0, 61.0, 0.5, 3.0)]
    x = np.array(xs, dtype=np.float32)
    got = oracle.log32(x)
    want = np.array([ln_rn32(float(v)) if v != one else np.float32(0) for v in x], dtype=np.float32)
    assert np.array_equal(f32_bits(got), f32_bits(want))


# ---------------------------------------------------------------- closed forms
def test_uniform_logits_give_minus_ln_V():
    V, block = 248320, 4096
    logits = np.full((2, V), bf16(3.0), dtype=np.uint16)
    targets = np.array([0, V - 1], dtype=np.int64)
    out, part = oracle.block_logprob(logits, targets, block, return_partials=True)
    # every e_v is exactly 1, so each full block sums to 4096 and the last (1536 real) to 1536
    assert np.all(part[:, :-1] == 4096.0) and np.all(part[:, -1] == V - 60 * 4096)
    want = -ln_rn32(V)
    assert np.array_equal(f32_bits(out), f32_bits(np.array([want, want])))


def test_dominant_logit_gives_minus_zero_and_exact_shift():
    V, block = 10000, 256
    row = np.full(V, bf16(-150.0), dtype=np.uint16)
    row[4321] = bf16(2.5)
    row[17] = bf16(-90.0)   # 92.5 below the max: e^-92.5 is subnormal, too small to move S off 1
    logits = np.stack([row, row, row])
    out = oracle.block_logprob(logits, np.array([4321, 17, 9999], dtype=np.int64), block)
    assert out[0] == 0 and math.copysign(1.0, out[0]) < 0   # certain token: -0.0
    assert out[1] == np.float32(-92.5)                       # s_t exactly, log(S) = 0
    assert out[2] == np.float32(-152.5)


@pytest.mark.parametrize("k", [2, 3, 7, 100])
def test_k_way_tie_gives_minus_ln_k(k):
    V, block = 5000, 512
    rng = np.random.default_rng(k)
    row = np.full(V, bf16(-120.0), dtype=np.uint16)
    idx = rng.choice(V, size=k, replace=False)
    row[idx] = bf16(1.0)
    out = oracle.block_logprob(row[None], np.array([idx[0]], dtype=np.int64), block)
    assert np.float32(out[0]) == -ln_rn32(k)


def test_fold_is_left_to_right_over_blocks():
    """Block 0 holds the max (e = 1); each of the 60 other blocks holds one e = EXP32(-16.75),
    which is below half an ulp of 1.  A left fold keeps S == 1 exactly, so out = s_t = -16.75;
    any other association (e.g. the tiny partials first) would leave S > 1."""
    block, nb = 256, 61
    V = block * nb
    row = np.full(V, bf16(-200.0), dtype=np.uint16)
    row[0] = bf16(0.0)
    for b in range(1, nb):
        row[b * block + 5] = bf16(-16.75)
    e = oracle.exp32(np.array([-16.75], dtype=np.float32))[0]
    assert e < 2.0 ** -24
    out, part = oracle.block_logprob(row[None], np.array([block + 5], dtype=np.int64), block, return_partials=True)
    assert part[0, 0] == 1.0 and np.all(part[0, 1:] == e)
    assert out[0] == np.float32(-16.75)
    assert np.float32(1.0) + np.float32(60 * e) > 1.0   # the reversed association differs


def test_in_block_tree_is_pairwise_not_sequential():
    """e_0 = 1 and 255 copies of eps = EXP32(-16.75) < 2^-24.  A sequential sum from the left
    stays at 1; the balanced pairwise tree adds the eps in exact power-of-two subtrees and
    lands within 8 half-ulps (one per level) of 1 + 255 eps."""
    block = 256
    row = np.full(block, bf16(-16.75), dtype=np.uint16)
    row[0] = bf16(0.0)
    _, part = oracle.block_logprob(row[None], np.array([0], dtype=np.int64), block, return_partials=True)
    eps = float(oracle.exp32(np.array([-16.75], dtype=np.float32))[0])
    P = float(part[0, 0])
    assert P != 1.0
    assert abs(P - (1 + 255 * eps)) <= 8 * 2.0 ** -24
    # mirrored: the max at the last index gives the same partial (the tree is symmetric here)
    row2 = row[::-1].copy()
    _, part2 = oracle.block_logprob(row2[None], np.array([0], dtype=np.int64), block, return_partials=True)
    assert part2[0, 0] == part[0, 0]


def test_in_block_tree_pairs_neighbours_not_strided_halves():
    """A 256-wide block with the row max at indices 0 and 128 (e = 1 each), d = EXP32(-15.75) at index 1
    and every other entry far below the max (e = +0).  d lies strictly between 2^-23 and 1.5 * 2^-23
    (checked against a decimal exp), which fixes every rounding:
      * index-order pairwise tree: T(0,2) = RN(1 + d) = 1 + 2^-23 and zeros keep it up to T(0,128);
        T(128,128) = 1; P = RN(2 + 2^-23) = 2, a tie resolved to even;
      * strided pairing (i with i + 128, then i with i + 64, ...): 1 + 1 = 2 first, and d joins last:
        RN(2 + d) = 2 + 2^-22.
    So the partial is exactly 2 and the logprob of the target at index 0 is -RN32(ln 2); the strided
    tree would give -RN32(ln(2 + 2^-22)), two ulps away."""
    block = 256
    d = exp_rn32(-15.75)
    assert 2.0 ** -23 < float(d) < 1.5 * 2.0 ** -23
    assert float(np.float32(2.0) + d) == 2.0 + 2.0 ** -22      # the strided order's last add
    row = np.full(block, bf16(-200.0), dtype=np.uint16)
    row[0] = row[128] = bf16(0.0)
    row[1] = bf16(-15.75)
    out, part = oracle.block_logprob(row[None], np.array([0], dtype=np.int64), block, return_partials=True)
    assert part[0, 0] == 2.0
    assert out[0] == -ln_rn32(2.0)
    assert ln_rn32(2.0) != ln_rn32(2.0 + 2.0 ** -22)


def test_virtual_padding_equals_materialised_minus_inf():
    rng = np.random.default_rng(4)
    V, block = 3 * 256 + 17, 256
    logits, targets = synth.random_logits(5, 6, V, std=3.0)
    padded = np.concatenate([logits, np.full((6, 4 * 256 - V), 0xFF80, dtype=np.uint16)], axis=1)
    a, pa = oracle.block_logprob(logits, targets, block, return_partials=True)
    b, pb = oracle.block_logprob(padded, targets, block, return_partials=True)
    assert np.array_equal(f32_bits(a), f32_bits(b)) and np.array_equal(pa, pb)


# ------------------------------------------------------------ brute force
def test_fp32_oracle_close_to_extended_reference():
    V, block = 3 * 256 + 17, 256
    for std in (1.0, 8.0, 105.0):
        logits, targets = synth.random_logits(int(std), 16, V, std=std)
        out = oracle.block_logprob(logits, targets, block)
        ref = oracle.logprob_ref(logits, targets)
        tol = 8 * np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) + 1e-6
        assert np.all(np.abs(out.astype(np.float64) - ref) <= tol)


def test_extended_reference_against_decimal():
    logits, targets = synth.random_logits(9, 4, 40, std=4.0)
    ref = oracle.logprob_ref(logits, targets)
    lv = synth.bf16_bits_to_f32(logits).astype(np.float64)
    for j in range(4):
        m = max(Decimal(float(v)) for v in lv[j])
        se = sum((Decimal(float(v)) - m).exp() for v in lv[j])
        want = Decimal(float(lv[j, targets[j]])) - m - se.ln()
        assert abs(Decimal(float(ref[j])) - want) < Decimal("1e-14")


def test_logprob_at_head_scale_is_about_minus_480():
    logits, targets = synth.random_logits(3, 4, 248320)
    out = oracle.block_logprob(logits, targets, 4096)
    ref = oracle.logprob_ref(logits, targets)
    assert np.all(out < -100) and np.all(np.abs(out - ref) <= 4 * np.spacing(np.abs(out)))


# ---------------------------------------------------------------- error cases
def test_nan_inf_and_bad_targets_give_nan():
    V, block = 600, 256
    logits, _ = synth.random_logits(2, 5, V, std=2.0)
    logits[0, 13] = 0x7FC0          # NaN
    logits[1, 7] = 0x7F80           # +inf
    targets = np.array([0, 0, -1, V, 3], dtype=np.int64)
    out = oracle.block_logprob(logits, targets, block)
    assert np.all(np.isnan(out[:4])) and np.isfinite(out[4])


def test_padding_contributes_exact_zeros():
    """V = 257 with block 256: the last block has one real logit 95 below the max, whose e is a
    subnormal; the 255 virtual entries must add exactly nothing to that block's partial."""
    V, block = 257, 256
    row = np.full(V, bf16(-300.0), dtype=np.uint16)
    row[3] = bf16(5.0)
    row[256] = bf16(-90.0)
    _, part = oracle.block_logprob(row[None], np.array([3], dtype=np.int64), block, return_partials=True)
    e = oracle.exp32(np.array([-95.0], dtype=np.float32))[0]
    assert 0 < e < np.finfo(np.float32).tiny
    assert part[0, 1] == e and part[0, 0] == 1.0


def test_shift_uses_the_global_row_max():
    """Block 1 holds the row max; block 0's values are shifted by it too (not by their own block max)."""
    V, block = 512, 256
    row = np.full(V, bf16(-300.0), dtype=np.uint16)
    row[10] = bf16(-2.0)
    row[300] = bf16(1.0)
    out, part = oracle.block_logprob(row[None], np.array([10], dtype=np.int64), block, return_partials=True)
    assert part[0, 0] == exp_rn32(-3.0) and part[0, 1] == 1.0
    S = np.float32(part[0, 0]) + np.float32(1.0)
    assert out[0] == -(ln_rn32(float(S)) - np.float32(-3.0))


# ------------------------------------------------------------- blockwise-direct
def test_direct_form_gives_plus_zero_and_the_same_nonzero_values():
    """tokenspeed numerics, "Logprobs": blockwise-direct is target - log(sum_exp) over the same
    reduction.  A certain token gives +0.0 (blockwise: -0.0); any other result equals the
    blockwise value, because IEEE subtraction is exactly sign-symmetric (a - b = -(b - a))."""
    V, block = 10000, 256
    row = np.full(V, bf16(-150.0), dtype=np.uint16)
    row[4321] = bf16(2.5)
    row[17] = bf16(-90.0)
    logits = np.stack([row, row, row])
    tg = np.array([4321, 17, 9999], dtype=np.int64)
    d = oracle.block_logprob(logits, tg, block, direct=True)
    assert d[0] == 0 and math.copysign(1.0, d[0]) > 0        # certain token: +0.0
    assert d[1] == np.float32(-92.5) and d[2] == np.float32(-152.5)
    rng = np.random.default_rng(3)
    lg = synth.f32_to_bf16_bits((rng.standard_normal((4, 3000)) * 8).astype(np.float32))
    tg = rng.integers(0, 3000, 4)
    a = oracle.block_logprob(lg, tg, 512)
    b = oracle.block_logprob(lg, tg, 512, direct=True)
    assert np.all(a != 0) and np.array_equal(f32_bits(b), f32_bits(a))
    u = oracle.block_logprob(np.full((1, 248320), bf16(3.0), dtype=np.uint16), np.array([7]), 4096, direct=True)
    assert u[0] == -ln_rn32(248320)


# ---------------------------------------------------------------- greedy argmax
def _argmax_by_hand(row_bits):
    """The rule written out: scan in index order; a NaN is larger than any number and the first
    NaN wins; otherwise move only to a strictly larger value (ties keep the lowest index;
    -0 == +0)."""
    vals = [float(synth.bf16_bits_to_f32(np.array([b], dtype=np.uint16))[0]) for b in row_bits]
    best = 0
    for i, v in enumerate(vals):
        if math.isnan(vals[best]):
            break
        if math.isnan(v) or v > vals[best]:
            best = i
    return best


def test_argmax_hand_cases():
    rows = [
        [bf16(1.0), bf16(2.0), bf16(2.0), bf16(-3.0)],                # tie: lowest index
        [0x8000, 0x0000, 0x8000, bf16(-1.0)],                        # -0 / +0 tie: index 0
        [bf16(-1.0), 0x0000, 0x8000, bf16(-2.0)],                     # +0 before -0: index 1
        [bf16(5.0), 0x7FC0, bf16(9.0), 0xFFC1],                       # first NaN wins (even over larger numbers)
        [0xFF80, 0xFF80, 0xFF80, 0xFF80],                             # all -inf: index 0
        [bf16(1.0), 0x7F80, bf16(3.0), 0x7F80],                       # +inf, first one
    ]
    want = [1, 0, 1, 1, 0, 1]
    got = oracle.argmax(np.array(rows, dtype=np.uint16))
    assert got.tolist() == want


def test_argmax_matches_the_rule_and_numpy():
    """Brute force of the written-out rule on rows full of exact ties, signed zeros, infinities
    and NaNs; on rows without NaN it is numpy's argmax of the fp32 values (first maximum)."""
    rng = np.random.default_rng(11)
    pool = np.array([bf16(v) for v in (-2.0, -1.0, -0.5, 0.5, 1.0, 3.0)] + [0x0000, 0x8000, 0x7F80, 0xFF80],
                    dtype=np.uint16)
    rows = pool[rng.integers(0, len(pool), (300, 37))]
    rows[::7, rng.integers(0, 37)] = 0x7FC1   # NaN in some rows
    got = oracle.argmax(rows)
    assert got.tolist() == [_argmax_by_hand(r) for r in rows]
    clean = ~np.isnan(synth.bf16_bits_to_f32(rows)).any(axis=1)
    assert np.array_equal(got[clean], np.argmax(synth.bf16_bits_to_f32(rows[clean]), axis=1))
