"""The projection's documented reduction schedule, written out in numpy for inputs on which it is exact.

The C header (include/w8inv.h, w8_linear_invariant's "Arithmetic, fixed for every (t, T_pad, N,
device)" paragraph) fixes the order of every
rounded addition of the projection: per 32-group a fp32 dot product, scaled exactly into fp64; K cut
into 8 slices of whole pairs of groups (c = 0, 3, 6, 9, 12, 13, 14, 15, 16; slice i covers groups
[2*floor(P*c_i/16), 2*floor(P*c_{i+1}/16)) with P = floor(G/2), the last slice also taking an odd
last group); each slice summed in fp64 in ascending group order from +0; the slice sums folded left
to right; one fp64 -> bf16 rounding.

The fp32 dot product of a group is only exact when at most one of its 32 products is nonzero, so the
model accepts only such inputs (synth.order_sensitive_linear draws them) and then reproduces every
rounding step.  `slice_bounds` and `fold` take the plan and the fold order as arguments so that the
CPU tests can show the inputs tell plans apart.  Test infrastructure only; nothing here is shared with
the HIP library (the final rounding is the oracle's).
"""
from __future__ import annotations

import numpy as np

import oracle
import synth

DOCUMENTED_C = (0, 3, 6, 9, 12, 13, 14, 15, 16)


def slice_bounds(G: int, c=DOCUMENTED_C) -> list:
    """First group of each of the 8 slices, and G: the header's formula with the 17-point c table."""
    P = G // 2
    b = [2 * ((P * ci) // c[-1]) for ci in c]
    b[-1] = G
    return b


def equal_bounds(G: int) -> list:
    """An 8-slice plan of equal pair counts (not the library's; for showing that plans differ)."""
    return slice_bounds(G, tuple(2 * i for i in range(9)))


def scaled_terms(q, s, x, rows):
    """fp64 terms s[n, g] * (sum_k q[n, 32g+k] x[j, 32g+k]), shape [t, len(rows), G].  Exact here:
    every group has at most one nonzero code, whose product with a bf16 value fits fp32, and the
    fp16 scale times that product fits fp64."""
    K = q.shape[1]
    G = K // synth.GROUP
    qr = q[rows].astype(np.float64).reshape(len(rows), G, synth.GROUP)
    if np.any(np.count_nonzero(qr, axis=2) > 1):
        raise ValueError("the model is exact only with at most one nonzero code per group")
    xv = synth.bf16_bits_to_f32(x).astype(np.float64).reshape(x.shape[0], G, synth.GROUP)
    D = np.einsum("ngk,tgk->tng", qr, xv)
    sv = np.asarray(s)[rows].view(np.float16).astype(np.float64)
    return sv[None] * D


def fold(terms, bounds, reverse_slices: bool = False):
    """Slice sums in ascending group order from +0, then the left fold (or, to show a different order,
    the fold from the last slice); fp64 [t, rows]."""
    parts = []
    for i in range(8):
        acc = np.zeros(terms.shape[:2])
        for g in range(bounds[i], bounds[i + 1]):
            acc = acc + terms[:, :, g]
        parts.append(acc)
    if reverse_slices:
        parts = parts[::-1]
    y = parts[0]
    for p in parts[1:]:
        y = y + p
    return y


def documented_schedule(q, s, x, rows) -> np.ndarray:
    """bf16 bit patterns [t, len(rows)] of the documented schedule."""
    terms = scaled_terms(q, s, x, rows)
    return oracle.bf16_round_array(fold(terms, slice_bounds(q.shape[1] // synth.GROUP)))
