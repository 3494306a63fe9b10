"""The two-projection launch (linear_pair) and the attention input projection (attn_input_proj) on the
GPU, through the C ABI.

The ninfer issue's table "Where t selects arithmetic" lists linear_pair and attn_input_proj among the
fused W8 decode ops without defining them.  The readings implemented, and pinned here bit for bit:

  w8_linear_pair_invariant(Wa, Wb, x)        == (w8_linear_invariant(Wa, x), w8_linear_invariant(Wb, x))
  w8_attn_input_proj_invariant(h, w, W)      == w8_linear_invariant(W, w8i_rmsnorm(h, w))

on both weight layouts, with each projection within the parity bar of the fp64 oracle (on its own GPU
inputs) and every column's bits independent of t.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import parity_bar, within_bf16_ulps

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import invariant_quantized_decode_amd as w8  # noqa: E402
from tests.gpu_util import DEV, bf16, bits, f16, i8, say  # noqa: E402


def check_bar(y_bits, q, s, x_bits, label):
    ref, mass = oracle.w8_linear(q, s, x_bits, mass=True)
    ok, err, misses = parity_bar(y_bits, ref, mass)
    say(f"{label}: {ok.size} outputs, {misses} beyond 2 ulps within the fp32 floor")
    assert ok.all(), f"{label}: {int((~ok).sum())} outputs outside the parity bar"


PAIRS = [  # Na, Nb, K, T_pad: q / kv of the chain's QKV, gate / up as two matrices, ragged rows, odd K/32
    (6144, 1024, 5120, 32),
    (17408, 17408, 5120, 64),
    (100, 37, 1056, 16),
    (257, 1000, 4096, 48),
]


@pytest.mark.parametrize("Na,Nb,K,T_pad", PAIRS)
def test_linear_pair_gives_the_single_projections_bits(Na, Nb, K, T_pad):
    rng = np.random.default_rng(Na + 3 * Nb + K)
    qa, qb = synth.draw_codes(rng, Na, K), synth.draw_codes(rng, Nb, K)
    sa, sb = synth.draw_scales(rng, Na, K, 0.0), synth.draw_scales(rng, Nb, K, 0.0)
    x = synth.draw_acts(rng, T_pad, K)
    Wa, Sa, Wb, Sb, Xd = i8(qa), f16(sa), i8(qb), f16(sb), bf16(x)
    Pa, Pb = w8.w8_pack(Wa, Sa), w8.w8_pack(Wb, Sb)
    full_a = bits(w8.w8_linear_invariant(Wa, Sa, Xd, T_pad, T_pad))
    full_b = bits(w8.w8_linear_invariant(Wb, Sb, Xd, T_pad, T_pad))
    for t in sorted({1, 9, T_pad // 2 + 1, T_pad}):
        perm = rng.permutation(T_pad)[:t]
        xp = bf16(x[perm])
        say(f"case linear_pair Na={Na} Nb={Nb} K={K} T_pad={T_pad} t={t}")
        ya, yb = w8.w8_linear_pair_invariant(Wa, Sa, Wb, Sb, xp, t, T_pad)
        assert np.array_equal(bits(ya), full_a[perm]) and np.array_equal(bits(yb), full_b[perm]), f"plain t={t}"
        ya, yb = w8.w8_linear_pair_invariant_packed(*Pa, *Pb, xp, t, T_pad, Na, Nb)
        assert np.array_equal(bits(ya), full_a[perm]) and np.array_equal(bits(yb), full_b[perm]), f"packed t={t}"
    check_bar(full_a, qa, sa, x, f"pair first Na={Na}")
    check_bar(full_b, qb, sb, x, f"pair second Nb={Nb}")


def test_linear_pair_writes_only_its_outputs():
    """Strided outputs inside wider buffers: nothing outside either window is written."""
    Na, Nb, K, T_pad, t = 96, 40, 1024, 32, 7
    rng = np.random.default_rng(5)
    qa, qb = synth.draw_codes(rng, Na, K), synth.draw_codes(rng, Nb, K)
    sa, sb = synth.draw_scales(rng, Na, K, 0.0), synth.draw_scales(rng, Nb, K, 0.0)
    x = synth.draw_acts(rng, t, K)
    Wa, Sa, Wb, Sb, Xd = i8(qa), f16(sa), i8(qb), f16(sb), bf16(x)
    wa = w8.w8_linear_invariant(Wa, Sa, Xd, t, T_pad)
    wb = w8.w8_linear_invariant(Wb, Sb, Xd, t, T_pad)
    say("case linear_pair strided outputs")
    ba = torch.full((t + 2, Na + 9), -5.0, dtype=torch.bfloat16, device=DEV)
    bb = torch.full((t + 2, Nb + 13), -5.0, dtype=torch.bfloat16, device=DEV)
    w8.w8_linear_pair_invariant(Wa, Sa, Wb, Sb, Xd, t, T_pad, ya=ba[1:1 + t, 2:2 + Na], yb=bb[:t, 5:5 + Nb])
    assert np.array_equal(bits(ba[1:1 + t, 2:2 + Na]), bits(wa)) and np.array_equal(bits(bb[:t, 5:5 + Nb]), bits(wb))
    ma = torch.ones_like(ba, dtype=torch.bool)
    ma[1:1 + t, 2:2 + Na] = False
    mb = torch.ones_like(bb, dtype=torch.bool)
    mb[:t, 5:5 + Nb] = False
    assert bool((ba[ma] == -5.0).all()) and bool((bb[mb] == -5.0).all())


ATTN = [  # N, H, T_pad, with a norm weight: the chain's QKV, a ragged projection, T_pad 64
    (7168, 5120, 32, False),
    (7168, 5120, 32, True),
    (300, 1056, 16, True),
    (1000, 4096, 64, False),
]


@pytest.mark.parametrize("N,H,T_pad,weighted", ATTN)
def test_attn_input_proj_is_rmsnorm_then_projection(N, H, T_pad, weighted):
    rng = np.random.default_rng(N + H + T_pad + weighted)
    q = synth.draw_codes(rng, N, H)
    s = synth.draw_scales(rng, N, H, 0.0)
    h = synth.draw_acts(rng, T_pad, H)
    nw = synth.f32_to_bf16_bits(rng.uniform(0.5, 1.5, H).astype(np.float32)) if weighted else None
    Wd, Sd, Hd = i8(q), f16(s), bf16(h)
    Nw = bf16(nw) if weighted else None
    Wp, Sp = w8.w8_pack(Wd, Sd)
    xn = w8.w8i_rmsnorm(Hd, 1e-6, Nw)
    full = bits(w8.w8_linear_invariant(Wd, Sd, xn, T_pad, T_pad))
    xn_bits = bits(xn)
    for t in sorted({1, 5, T_pad // 2 + 1, T_pad}):
        perm = rng.permutation(T_pad)[:t]
        hp = bf16(h[perm])
        say(f"case attn_input_proj N={N} H={H} T_pad={T_pad} weighted={weighted} t={t}")
        y = bits(w8.w8_attn_input_proj_invariant(hp, Nw, 1e-6, Wd, Sd, t, T_pad))
        assert np.array_equal(y, full[perm]), f"plain t={t}"
        y = bits(w8.w8_attn_input_proj_invariant_packed(hp, Nw, 1e-6, Wp, Sp, t, T_pad, N))
        assert np.array_equal(y, full[perm]), f"packed t={t}"
    # the two halves against the oracle: the norm within 1 bf16 ulp, the projection of its output
    # within the parity bar
    ok, err = within_bf16_ulps(xn_bits, oracle.rmsnorm(h, 1e-6, nw), 1.0)
    assert ok.all(), f"rmsnorm: max {float(err.max()):.2f} ulp"
    check_bar(full, q, s, xn_bits, f"attn_input_proj N={N} H={H}")
