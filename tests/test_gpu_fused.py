"""Fused W8 projection epilogues on the GPU, through the C ABI.

The ninfer issue's table "Where t selects arithmetic" lists the fused W8 decode ops (row
"attn_input_proj, linear_swiglu, linear_pair, linear_add (W8)") beside the plain linear.  Here
they run the plain projection's K plan and then the glue's arithmetic, so the contract is exact:

  w8_linear_add_invariant(x, r)  == w8i_residual_add(w8_linear_invariant(x), r)   bit for bit
  w8_linear_swiglu_invariant(x)  == w8i_swiglu(w8_linear_invariant(x))            bit for bit

Parity with the oracle follows from the two halves, each pinned on its own: the projection is
checked against the fp64 oracle within 2 bf16 ulps here (and in test_gpu_linear.py), the glue
within 1 ulp in test_gpu_glue.py.  The fused ops are also t-invariant column by column.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import within_bf16_ulps

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import invariant_quantized_decode_amd as w8  # noqa: E402
from tests.gpu_util import DEV, bf16, bits, f16, i8, say  # noqa: E402


def draw(seed, N, K, T_pad, eps=0.0):
    rng = np.random.default_rng(seed)
    q = synth.draw_codes(rng, N, K)
    s = synth.draw_scales(rng, N, K, eps)
    x = synth.draw_acts(rng, T_pad, K)
    return rng, q, s, x


def unaligned_scales(s):
    """The same scales 2 bytes past a 16-byte boundary (the per-stage scale-load variant)."""
    flat = torch.zeros(s.size + 8, dtype=torch.int16, device=DEV)
    flat[1:1 + s.size] = f16(s.reshape(-1))
    return flat[1:1 + s.size].view(s.shape)


ADD = [  # N, K, t, T_pad: chain O and down shapes, ragged rows, odd group count, every T_pad
    (5120, 6144, 17, 32),
    (5120, 17408, 32, 32),
    (100, 1056, 5, 16),
    (257, 4096, 48, 48),
    (33, 160, 64, 64),
]


@pytest.mark.parametrize("N,K,t,T_pad", ADD)
@pytest.mark.parametrize("aligned", [True, False])
def test_linear_add_equals_linear_then_residual_add(N, K, t, T_pad, aligned):
    say(f"case linear_add N={N} K={K} t={t} T_pad={T_pad} aligned={aligned}")
    rng, q, s, x = draw(N + K + t, N, K, T_pad)
    res = synth.draw_acts(rng, T_pad, N)
    Wd, Xd, Rd = i8(q), bf16(x), bf16(res)
    Sd = f16(s) if aligned else unaligned_scales(s)
    lin = w8.w8_linear_invariant(Wd, Sd, Xd, t, T_pad)
    ok, err = within_bf16_ulps(bits(lin), oracle.w8_linear(q, s, x[:t]), 2.0)
    assert ok.all(), f"projection: {int((~ok).sum())} outputs beyond 2 ulps"
    want = bits(w8.w8i_residual_add(lin, Rd[:t]))
    got = bits(w8.w8_linear_add_invariant(Wd, Sd, Xd, Rd, t, T_pad))
    assert np.array_equal(got, want)
    # in place: y is the residual buffer itself
    Rw = Rd.clone()
    w8.w8_linear_add_invariant(Wd, Sd, Xd, Rw, t, T_pad, y=Rw)
    assert np.array_equal(bits(Rw[:t]), want)
    assert np.array_equal(bits(Rw[t:]), bits(Rd[t:]))  # rows past t untouched


SWIGLU = [  # F, K, t, T_pad: chain gate+up (F = 17408), odd group count, ragged F, every T_pad
    (17408, 5120, 32, 32),
    (40, 1056, 3, 16),
    (37, 160, 48, 48),       # F * K/32 not a multiple of 8: scales loaded per stage
    (300, 2048, 64, 64),
    (16, 64, 1, 32),
]


@pytest.mark.parametrize("F,K,t,T_pad", SWIGLU)
@pytest.mark.parametrize("aligned", [True, False])
def test_linear_swiglu_equals_linear_then_swiglu(F, K, t, T_pad, aligned):
    say(f"case linear_swiglu F={F} K={K} t={t} T_pad={T_pad} aligned={aligned}")
    rng, q, s, x = draw(F + K + t, 2 * F, K, T_pad)
    Wd, Xd = i8(q), bf16(x)
    Sd = f16(s) if aligned else unaligned_scales(s)
    gu = w8.w8_linear_invariant(Wd, Sd, Xd, t, T_pad)
    if F * K <= 17408 * 5120 // 8:  # the oracle on the smaller shapes; the large one is spot-checked below
        ok, err = within_bf16_ulps(bits(gu), oracle.w8_linear(q, s, x[:t]), 2.0)
        assert ok.all(), f"projection: {int((~ok).sum())} outputs beyond 2 ulps"
    else:
        rows = np.sort(rng.choice(2 * F, 64, replace=False))
        ok, err = within_bf16_ulps(bits(gu)[:, rows], oracle.w8_linear(q[rows], s[rows], x[:t]), 2.0)
        assert ok.all()
    want = bits(w8.w8i_swiglu(gu))
    got = bits(w8.w8_linear_swiglu_invariant(Wd, Sd, Xd, t, T_pad))
    assert got.shape == (t, F)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("T_pad", [16, 32, 48, 64])
def test_fused_columns_are_t_invariant(T_pad):
    """A column's bits do not depend on t or on the other columns (the pages' fixed-width contract),
    on both layouts; at T_pad 48 and 64 the t <= 32 cases run the one-tile kernel (the second
    32-column tile would hold no live column), and the t values reach every count of live 8-column
    groups (1..8) the epilogue kernels have a loop copy for."""
    rng, q, s, x = draw(9 + T_pad, 2 * 96, 1024, T_pad)
    res = synth.draw_acts(rng, T_pad, 2 * 96)
    Wd, Sd, Xd, Rd = i8(q), f16(s), bf16(x), bf16(res)
    Wp, Sp = w8.w8_pack(Wd, Sd)
    full_sw = bits(w8.w8_linear_swiglu_invariant(Wd, Sd, Xd, T_pad, T_pad))
    full_add = bits(w8.w8_linear_add_invariant(Wd, Sd, Xd, Rd, T_pad, T_pad))
    for t in (t for t in (1, 5, 9, 17, 31, 33, 41, 49, 63) if t < T_pad):
        perm = rng.permutation(T_pad)[:t]
        say(f"case fused T_pad={T_pad} t={t}")
        xp, rp = bf16(x[perm]), bf16(res[perm])
        assert np.array_equal(bits(w8.w8_linear_swiglu_invariant(Wd, Sd, xp, t, T_pad)), full_sw[perm])
        assert np.array_equal(bits(w8.w8_linear_add_invariant(Wd, Sd, xp, rp, t, T_pad)), full_add[perm])
        assert np.array_equal(bits(w8.w8_linear_swiglu_invariant_packed(Wp, Sp, xp, t, T_pad, 96)), full_sw[perm])
        assert np.array_equal(bits(w8.w8_linear_add_invariant_packed(Wp, Sp, xp, rp, t, T_pad, 2 * 96)),
                              full_add[perm])


@pytest.mark.parametrize("N,K,t,T_pad", ADD)
def test_packed_linear_add_gives_the_plain_bits(N, K, t, T_pad):
    say(f"case packed linear_add N={N} K={K} t={t} T_pad={T_pad}")
    rng, q, s, x = draw(N + K + t, N, K, T_pad)
    res = synth.draw_acts(rng, T_pad, N)
    Wd, Sd, Xd, Rd = i8(q), f16(s), bf16(x), bf16(res)
    Wp, Sp = w8.w8_pack(Wd, Sd)
    want = bits(w8.w8_linear_add_invariant(Wd, Sd, Xd, Rd, t, T_pad))
    assert np.array_equal(bits(w8.w8_linear_add_invariant_packed(Wp, Sp, Xd, Rd, t, T_pad, N)), want)
    Rw = Rd.clone()
    w8.w8_linear_add_invariant_packed(Wp, Sp, Xd, Rw, t, T_pad, N, y=Rw)
    assert np.array_equal(bits(Rw[:t]), want)


@pytest.mark.parametrize("F,K,t,T_pad", SWIGLU + [(37, 1056, 5, 32)])  # F not a multiple of 16: strips straddled
def test_packed_linear_swiglu_gives_the_plain_bits(F, K, t, T_pad):
    say(f"case packed linear_swiglu F={F} K={K} t={t} T_pad={T_pad}")
    rng, q, s, x = draw(F + K + t, 2 * F, K, T_pad)
    Wd, Sd, Xd = i8(q), f16(s), bf16(x)
    Wp, Sp = w8.w8_pack(Wd, Sd)
    want = bits(w8.w8_linear_swiglu_invariant(Wd, Sd, Xd, t, T_pad))
    assert np.array_equal(bits(w8.w8_linear_swiglu_invariant_packed(Wp, Sp, Xd, t, T_pad, F)), want)
