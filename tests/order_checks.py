"""GPU checks of the library's fixed reduction orders, on inputs where another order changes the bits.

Random inputs barely exercise an fp64 accumulation order: a different K plan or slice fold moves the
fp64 sum by about 1e-16 relative, which decides a bf16 rounding for no output in 200k random ones.  The
projection checks therefore run on synth.order_sensitive_linear, where most outputs change with the
order, and compare with tests/order_model.py's model of the documented schedule and across t.  The
logprob checks use random logits and two constructed rows on which one fp32 rounding tells two orders
apart; the fused-maxima check, a ragged vocabulary of negative logits.

Each check returns a list of failure descriptions (empty: passed).  They call the binding's current
library, so the mutant tier runs them unchanged on each mutated build.  Test infrastructure only.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
import invariant_quantized_decode_amd as w8
from tests import order_model
from tests.gpu_util import DEV, bf16, bits, f16, host, i8

INVARIANCE_T = (1, 9, 16, 17, 24, 33, 48)


class OrderSensitiveProjection:
    """One order-sensitive problem, resident on the device in both layouts (packed by the product
    library), with the documented schedule's bits for a sample of rows at t = T_pad."""

    def __init__(self, seed: int, N: int, K: int, T_pad: int, model_rows: int):
        q, s, x = synth.order_sensitive_linear(seed, N, K, T_pad)
        self.name = f"N={N} K={K} T_pad={T_pad}"
        self.N, self.K, self.T_pad, self.x, self.seed = N, K, T_pad, x, seed
        self.W, self.S, self.X = i8(q), f16(s), bf16(x)
        self.Wp, self.Sp = w8.w8_pack(self.W, self.S)
        rng = np.random.default_rng(seed)
        self.rows = np.arange(N) if N <= model_rows else np.unique(
            np.concatenate([np.arange(64), rng.choice(N, model_rows - 128, replace=False), np.arange(N - 64, N)]))
        self.want = order_model.documented_schedule(q, s, x, self.rows)

    def call(self, packed: bool, xd, t: int, workspace="auto"):
        if packed:
            return w8.w8_linear_invariant_packed(self.Wp, self.Sp, xd, t, self.T_pad, self.N, workspace=workspace)
        return w8.w8_linear_invariant(self.W, self.S, xd, t, self.T_pad, workspace=workspace)


def check_projection(P: OrderSensitiveProjection) -> list:
    """The t = T_pad call gives the documented schedule's bits on the model rows, and every column
    computed at t < T_pad (a random subset of the columns, in random order) gives its t = T_pad bits;
    both weight layouts, with the workspace the size query asks for (small N: the K-slice kernels) and
    without one (the one-launch kernels)."""
    fails = []
    for packed in (False, True):
        for ws in ("auto", None):
            tag = f"{P.name} {'packed' if packed else 'plain'}{'' if ws else ' no workspace'}"
            full = bits(P.call(packed, P.X, P.T_pad, ws))
            bad = int(np.sum(full[:, P.rows] != P.want))
            if bad:
                fails.append(f"{tag}: t={P.T_pad} differs from the documented schedule in {bad} of {P.want.size}")
            rng = np.random.default_rng(P.seed + 1)
            for t in (t for t in INVARIANCE_T if t < P.T_pad):
                perm = rng.permutation(P.T_pad)[:t]
                bad = int(np.sum(bits(P.call(packed, bf16(P.x[perm]), t, ws)) != full[perm]))
                if bad:
                    fails.append(f"{tag}: t={t} columns differ from their t={P.T_pad} bits in {bad} of {t * P.N}")
    return fails


def _logprob_bits(logits, targets, block):
    out = w8.vocab_block_logprob(bf16(logits), torch.from_numpy(np.asarray(targets, np.int64)).to(DEV), block)
    return host(out).view(np.uint32)


def _compare_logprob(tag, logits, targets, block) -> list:
    got = _logprob_bits(logits, targets, block)
    want = oracle.block_logprob(logits, targets, block).view(np.uint32)
    bad = int(np.sum(got != want))
    return [f"{tag}: {bad} of {len(want)} logprobs differ from the oracle's bits"] if bad else []


def check_logprob_random() -> list:
    """Random logits (a spread one at V = 70000, block 1024; a flat one at the head's V = 248320,
    block 4096, where many blocks contribute): bitwise the oracle's fixed-order fp32 result."""
    fails = []
    for seed, t, V, std, block in ((5, 4, 70000, 20.0, 1024), (6, 3, 248320, 2.0, 4096)):
        logits, targets = synth.random_logits(seed, t, V, std)
        fails += _compare_logprob(f"random V={V} block={block}", logits, targets, block)
    return fails


def _bf16(v: float) -> int:
    return int(synth.f32_to_bf16_bits(np.array([v], np.float32))[0])


def fold_order_row():
    """Block 256, 64 blocks.  Block 0 holds the row maximum 0 (partial exactly 1: its other logits are
    -200, whose exp is +0 in fp32); blocks 1..60 each hold one logit -16.75 (partial e^-16.75 ~ 5.3e-8,
    under half an fp32 ulp of 1), the rest -200.  Folded left to right, every small partial rounds away
    and the sum stays 1, so the target-0 logprob is -(ln 1 - 0) = -0.0; adding any two small partials
    together first leaves a sum above 1."""
    V = 64 * 256
    row = np.full(V, _bf16(-200.0), dtype=np.uint16)
    row[0] = _bf16(0.0)
    for b in range(1, 61):
        row[256 * b + 17] = _bf16(-16.75)
    return row[None], np.array([0], np.int64), 256


def strided_tree_row():
    """Block 256 (one logit per thread), 4 blocks.  Logits 0 at indices 0 and 1 (the maximum), -15.75
    at index 32 (d = e^-15.75 ~ 1.21 u, u = 2^-23), -200 elsewhere.  The pairwise tree in index order
    adds 1 + 1 first and then 2 + d, which rounds to 2 + 2u; a tree that pairs index 0 with index 32
    first forms 1 + d -> 1 + u, then (1 + u) + 1, a tie that rounds to 2."""
    V = 4 * 256
    row = np.full(V, _bf16(-200.0), dtype=np.uint16)
    row[0] = row[1] = _bf16(0.0)
    row[32] = _bf16(-15.75)
    return row[None], np.array([0], np.int64), 256


def check_logprob_fold_order() -> list:
    logits, targets, block = fold_order_row()
    return _compare_logprob("fold order row", logits, targets, block)


def check_logprob_in_block_tree() -> list:
    logits, targets, block = strided_tree_row()
    return _compare_logprob("in-block tree row", logits, targets, block)


def check_fused_maxima() -> list:
    """The fused head's row maxima on a vocabulary that is not a multiple of the 32-row strip, every
    logit below -104 (positive codes and scales, negative activations): the last strip's rows past V
    compute zeros, and a maximum that counted them would be 0, under which every exp underflows
    (a maximum of 0 over logits near -60 can still give the same bits).  Both layouts' fused calls
    must give the unfused calls' logprob bits."""
    rng = np.random.default_rng(31)
    V, K, t, block = 4013, 256, 5, 256
    q = rng.integers(1, 128, size=(V, K), dtype=np.int8)
    s = synth.draw_scales(rng, V, K, 0.08)
    x = synth.draw_acts(rng, t, K) | np.uint16(0x8000)
    targets = rng.integers(0, V, size=t, dtype=np.int64)
    Wd, Sd, Xd, Td = i8(q), f16(s), bf16(x), torch.from_numpy(targets).to(DEV)
    logits = w8.w8_linear_invariant(Wd, Sd, Xd, t, 32)
    want = host(w8.vocab_block_logprob(logits, Td, block)).view(np.uint32)
    assert float(logits.float().max()) < -104.0, "every logit below -104"
    Wp, Sp = w8.w8_pack(Wd, Sd)
    fails = []
    for name, out in (("plain", w8.w8_head_logprob_invariant(Wd, Sd, Xd, Td, t, 32, block)[1]),
                      ("packed", w8.w8_head_logprob_invariant_packed(Wp, Sp, Xd, Td, t, 32, block, V)[1])):
        bad = int(np.count_nonzero(host(out).view(np.uint32) != want))
        if bad:
            fails.append(f"fused maxima ({name}): {bad} of {t} logprobs differ from the unfused calls'")
    return fails
