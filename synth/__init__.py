"""Seeded synthetic inputs for the W8A16 decode projection and the block logprob.

This module only draws random data and packs it into the storage formats the
library and the oracle read (int8 weights, fp16 scale bit patterns, bf16
activation bit patterns, int64 target ids).  It contains none of the method's
arithmetic; both the GPU path and the CPU oracle take their inputs from here.

The shapes follow the decode projections measured on the ninfer page
("Measured (RTX 5090 ...)" table: W8 [N x K] rows such as [1024x5120],
[6144x5120], [34816x5120], [5120x17408], [248320x5120]).  Value distributions:
int8 codes uniform in [-127, 127], one fp16 scale per 32 consecutive K elements
drawn as |N(0, 0.02)| (plus 1e-4 for the two plain linear workloads), bf16
activations N(0, 1).  Every generator is numpy PCG64 with a fixed seed and a
fixed draw order (codes, scales, activation pool, then targets/permutations).
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

GROUP = 32  # K elements per fp16 scale ("W8G32")


# --------------------------------------------------------------------------
# storage-format packing (data preparation, not part of the method)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = r.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f64_to_f16_bits(a: np.ndarray) -> np.ndarray:
    """Round to IEEE fp16 with numpy's conversion; return uint16 bit patterns."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


# --------------------------------------------------------------------------
# primitive draws
# --------------------------------------------------------------------------
def draw_codes(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    """int8 weight codes uniform in [-127, 127] (-128 is never drawn)."""
    return rng.integers(-127, 128, size=(n, k), dtype=np.int8)


def draw_scales(rng: np.random.Generator, n: int, k: int, eps: float) -> np.ndarray:
    """fp16 group scales |N(0, 0.02)| + eps, one per (row, 32 consecutive K); uint16 bits [n, k/32]."""
    assert k % GROUP == 0
    s = np.abs(rng.normal(0.0, 0.02, size=(n, k // GROUP))) + eps
    return f64_to_f16_bits(s)


def draw_acts(rng: np.random.Generator, t: int, k: int) -> np.ndarray:
    """bf16 activations N(0, 1); uint16 bits [t, k] (token j's features are contiguous)."""
    return f32_to_bf16_bits(rng.standard_normal(size=(t, k), dtype=np.float32))


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Linear:
    name: str
    N: int
    K: int
    T_pad: int
    seed: int
    scale_eps: float

    @property
    def weight_bytes(self) -> int:
        return self.N * self.K + 2 * self.N * (self.K // GROUP)


LINEAR_1024 = Linear("w8a16 linear 1024x5120", 1024, 5120, 16, 0, 1e-4)
LINEAR_6144 = Linear("w8a16 linear 6144x5120", 6144, 5120, 32, 1, 1e-4)
MLP_GATE_UP = Linear("w8a16 mlp gate/up 34816x5120", 34816, 5120, 64, 2, 0.0)
MLP_DOWN = Linear("w8a16 mlp down 5120x17408", 5120, 17408, 64, 2, 0.0)
HEAD = Linear("w8a16 vocab head 248320x5120", 248320, 5120, 32, 3, 0.0)
HEAD_BLOCK = 4096
MLP_T_VALUES = (1, 5, 17, 24, 32, 48, 64)

CHAIN_HIDDEN = 5120
CHAIN_QKV = 7168
CHAIN_Q = 6144
CHAIN_FFN = 17408
CHAIN_T_PAD = 32
CHAIN_LANES = 32
CHAIN_STEPS = 200


def linear_1024_col0_fixed():
    """1024x5120, T_pad 16, seed 0: column 0 drawn once, the other t-1 columns fresh for every t."""
    c = LINEAR_1024
    rng = np.random.default_rng(c.seed)
    q = draw_codes(rng, c.N, c.K)
    s = draw_scales(rng, c.N, c.K, c.scale_eps)
    col0 = draw_acts(rng, 1, c.K)
    xs = {}
    for t in range(1, c.T_pad + 1):
        fresh = draw_acts(rng, t - 1, c.K)
        xs[t] = np.concatenate([col0, fresh], axis=0)
    return dict(case=c, q=q, s=s, xs=xs)


def linear_6144_permuted():
    """6144x5120, T_pad 32, seed 1: a pool of 32 columns; for each t a random ordered subset of t of them."""
    c = LINEAR_6144
    rng = np.random.default_rng(c.seed)
    q = draw_codes(rng, c.N, c.K)
    s = draw_scales(rng, c.N, c.K, c.scale_eps)
    pool = draw_acts(rng, c.T_pad, c.K)
    perms = {t: rng.permutation(c.T_pad)[:t] for t in range(1, c.T_pad + 1)}
    return dict(case=c, q=q, s=s, pool=pool, perms=perms)


def mlp_pair():
    """gate/up 34816x5120 and down 5120x17408, T_pad 64, seed 2, each with its own activation pool."""
    gu, dn = MLP_GATE_UP, MLP_DOWN
    rng = np.random.default_rng(gu.seed)
    gu_q = draw_codes(rng, gu.N, gu.K)
    gu_s = draw_scales(rng, gu.N, gu.K, gu.scale_eps)
    dn_q = draw_codes(rng, dn.N, dn.K)
    dn_s = draw_scales(rng, dn.N, dn.K, dn.scale_eps)
    gu_pool = draw_acts(rng, gu.T_pad, gu.K)
    dn_pool = draw_acts(rng, dn.T_pad, dn.K)
    perms = {t: rng.permutation(gu.T_pad)[:t] for t in MLP_T_VALUES}
    return dict(gate_up=dict(case=gu, q=gu_q, s=gu_s, pool=gu_pool),
                down=dict(case=dn, q=dn_q, s=dn_s, pool=dn_pool), perms=perms)


def head_logprob():
    """248320x5120 head, T_pad 32, seed 3, plus a uniform target id per pool column."""
    c = HEAD
    rng = np.random.default_rng(c.seed)
    q = draw_codes(rng, c.N, c.K)
    s = draw_scales(rng, c.N, c.K, c.scale_eps)
    pool = draw_acts(rng, c.T_pad, c.K)
    targets = rng.integers(0, c.N, size=c.T_pad, dtype=np.int64)
    perms = {t: rng.permutation(c.T_pad)[:t] for t in range(1, c.T_pad + 1)}
    return dict(case=c, q=q, s=s, pool=pool, targets=targets, perms=perms, block=HEAD_BLOCK)


def chain_layer():
    """One 5120-hidden W8 layer (QKV 7168, O 5120x6144, gate+up 34816, down 5120x17408), seed 4.

    Scales are |N(0, 0.02)| without the 1e-4 floor.  32 lanes of N(0, 1) bf16 hidden
    state, then 200 steps, each with t uniform in 1..32 and a random choice of t
    distinct lanes placed in that order in the padded batch.
    """
    rng = np.random.default_rng(4)
    H, F = CHAIN_HIDDEN, CHAIN_FFN
    w = {}
    for name, n, k in (("qkv", CHAIN_QKV, H), ("o", H, CHAIN_Q), ("gate_up", 2 * F, H), ("down", H, F)):
        q = draw_codes(rng, n, k)
        s = draw_scales(rng, n, k, 0.0)
        w[name] = (q, s)
    lanes = draw_acts(rng, CHAIN_LANES, H)
    steps = []
    for _ in range(CHAIN_STEPS):
        t = int(rng.integers(1, CHAIN_LANES + 1))
        steps.append(rng.choice(CHAIN_LANES, size=t, replace=False))
    return dict(weights=w, lanes=lanes, steps=steps)


def small_linear(seed: int, N: int, K: int, t: int, scale_eps: float = 0.0):
    """A small random problem with the same distributions (for oracle-sized parity cases)."""
    rng = np.random.default_rng(seed)
    q = draw_codes(rng, N, K)
    s = draw_scales(rng, N, K, scale_eps)
    x = draw_acts(rng, t, K)
    return q, s, x


def random_logits(seed: int, t: int, V: int, std: float = 105.0):
    """bf16 logits N(0, std^2) of the head's scale (|lp| ~ 480 at V = 248320) and uniform targets."""
    rng = np.random.default_rng(seed)
    l = f32_to_bf16_bits((rng.standard_normal(size=(t, V), dtype=np.float32) * np.float32(std)))
    tg = rng.integers(0, V, size=t, dtype=np.int64)
    return l, tg


def order_sensitive_linear(seed: int, N: int, K: int, t: int):
    """A projection problem whose result depends on the order of its fp64 sums.

    Every 32-group of a weight row has at most one nonzero code, so each group's dot product is a
    single exact product.  Each row holds a pair of codes +100 / -100, both with scale 1024, at two
    distinct random groups; their positions see activations of 2^40 (offset 0 of every group), so
    the pair's terms are +-100 * 1024 * 2^40 and cancel exactly.  Every other group contributes one
    term of order 10^2 (a code at offset 1, scale |N(0, 1)| + 0.01, activation N(0, 1)), which a
    running sum that holds one term of the pair keeps only to a multiple of 16.  Which of those terms
    are added while the pair is half summed depends on the order of the additions, so different
    orders give different bf16 results for most rows.
    """
    rng = np.random.default_rng(seed)
    G = K // GROUP
    q = np.zeros((N, K), dtype=np.int8)
    q[:, 1::GROUP] = rng.integers(-127, 128, size=(N, G), dtype=np.int8)
    s = f64_to_f16_bits(np.abs(rng.normal(0.0, 1.0, size=(N, G))) + 0.01)
    a = rng.integers(0, G, size=N)
    b = rng.integers(0, G - 1, size=N)
    b = b + (b >= a)
    r = np.arange(N)
    q[r, GROUP * a + 1] = 0
    q[r, GROUP * b + 1] = 0
    q[r, GROUP * a] = 100
    q[r, GROUP * b] = -100
    s[r, a] = s[r, b] = f64_to_f16_bits(np.array(1024.0))
    x = f32_to_bf16_bits(rng.standard_normal(size=(t, K), dtype=np.float32))
    x[:, 0::GROUP] = f32_to_bf16_bits(np.full((t, G), 2.0 ** 40, dtype=np.float32))
    return q, s, x
