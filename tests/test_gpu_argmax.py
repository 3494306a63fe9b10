"""LM-head epilogue variants on the GPU, through the C ABI: the canonical greedy argmax and the
blockwise-direct logprob (tokenspeed "Numerics envelopes", "Logprobs" section).

The argmax is integer work (order keys, MAX), so the bar is exact: every index equals the oracle's
(lowest index among equal maxima, +-0 equal, the first NaN).  The direct logprob runs the same
fp32 reduction as the blockwise one, so it is expected to equal the fixed-order oracle bit for bit
(bar 1e-5 absolute), with +0.0 for a certain token.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import invariant_quantized_decode_amd as w8  # noqa: E402
from tests.gpu_util import DEV, bf16, host, say  # noqa: E402


def gpu_argmax(bits, offset=0, pad=0):
    """Rows at `offset` elements into a buffer of width V + pad (unaligned or strided rows)."""
    t, V = bits.shape
    if offset == 0 and pad == 0:
        return host(w8.vocab_argmax(bf16(bits)))
    buf = torch.zeros((t, offset + V + pad), dtype=torch.bfloat16, device=DEV)
    buf[:, offset:offset + V] = bf16(bits)
    return host(w8.vocab_argmax(buf[:, offset:offset + V]))


def tie_heavy(rng, t, V):
    """Logits from a handful of values, so exact ties (and +-0) are everywhere."""
    pool = synth.f32_to_bf16_bits(np.array([-3.0, -1.0, 0.0, 0.5, 2.0, 7.0], dtype=np.float32))
    pool = np.concatenate([pool, np.array([0x8000], dtype=np.uint16)])
    return pool[rng.integers(0, len(pool), (t, V))]


@pytest.mark.parametrize("V,t", [(248320, 32), (248320, 1), (4096, 3), (4097, 5), (5, 7), (1, 2), (100003, 4)])
def test_argmax_matches_oracle(V, t):
    say(f"case argmax V={V} t={t}")
    rng = np.random.default_rng(V + t)
    logits, _ = synth.random_logits(V + t, t, V, std=105.0)
    ties = tie_heavy(rng, t, V)
    for name, bits in (("random", logits), ("ties", ties)):
        got = gpu_argmax(bits)
        assert np.array_equal(got, oracle.argmax(bits)), name


def test_argmax_special_rows_and_layouts():
    rng = np.random.default_rng(5)
    V = 9000
    rows = tie_heavy(rng, 8, V)
    rows[1, 7000] = 0x7FC0                     # a NaN wins over every number
    rows[2, [100, 5000]] = 0xFFC1              # negative-signed NaNs count as NaN too: the first
    rows[3, :] = 0xFF80                        # all -inf: index 0
    rows[4, :] = 0x8000                        # all -0: index 0
    rows[5, 8999] = 0x7F80                     # +inf at the end
    rows[6, :] = 0x0000
    rows[6, 4096] = 0x8000                     # -0 among +0: still index 0
    rows[7, 4095:4097] = synth.f32_to_bf16_bits(np.array([9.0, 9.0], dtype=np.float32))  # tie across a block edge
    want = oracle.argmax(rows)
    assert want[1] == 7000 and want[2] == 100 and want[3] == 0 and want[4] == 0 and want[5] == 8999
    assert want[6] == 0 and want[7] == 4095
    for off, pad in ((0, 0), (1, 0), (3, 40), (8, 8)):
        say(f"case argmax layout offset={off} pad={pad}")
        assert np.array_equal(gpu_argmax(rows, off, pad), want)


def test_argmax_columns_are_independent():
    rng = np.random.default_rng(9)
    bits = tie_heavy(rng, 32, 248320)
    full = gpu_argmax(bits)
    for t in (1, 7, 31):
        perm = rng.permutation(32)[:t]
        assert np.array_equal(gpu_argmax(bits[perm]), full[perm])


def test_direct_logprob_matches_oracle_and_gives_plus_zero():
    V, block = 248320, 4096
    logits, targets = synth.random_logits(21, 16, V, std=105.0)
    Ld, Td = bf16(logits), torch.from_numpy(targets).to(DEV)
    got = host(w8.vocab_block_logprob_direct(Ld, Td, block))
    want = oracle.block_logprob(logits, targets, block, direct=True)
    say(f"direct: max |diff| {float(np.max(np.abs(got.astype(np.float64) - want))):.3g}")
    assert np.all(np.abs(got.astype(np.float64) - want) <= 1e-5)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # a certain token: +0.0 here, -0.0 from the blockwise form
    row = np.full((1, V), synth.f32_to_bf16_bits(np.array([-200.0], np.float32))[0], dtype=np.uint16)
    row[0, 777] = synth.f32_to_bf16_bits(np.array([3.0], np.float32))[0]
    T = torch.tensor([777], dtype=torch.int64, device=DEV)
    d = float(host(w8.vocab_block_logprob_direct(bf16(row), T, block))[0])
    b = float(host(w8.vocab_block_logprob(bf16(row), T, block))[0])
    assert d == 0 and math.copysign(1.0, d) > 0
    assert b == 0 and math.copysign(1.0, b) < 0
