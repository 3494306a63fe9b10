"""Column-local glue kernels on the GPU (RMSNorm, SwiGLU, residual add), through the C ABI.

These sit between the projections of one decode layer; the ninfer issue's "Where t selects
arithmetic" notes that norms and other per-lane ops are invariant.  Parity: every output within
1 bf16 ulp of the oracle's (long double) value -- the kernels compute in fp32 and round once to
bf16, and their fp32 error is far below half a bf16 ulp, so only the final rounding can move an
output, by at most one ulp.  Invariance: a column's bits do not depend on the other columns, on
their number or on the leading dimensions.
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
from tests.gpu_util import DEV, bf16, bits, say  # noqa: E402


def check(y_bits, ref, label, ulps=1.0):
    ok, err = within_bf16_ulps(y_bits, ref, ulps)
    say(f"{label}: max err {float(err.max()):.3f} bf16 ulp, {int((~ok).sum())} of {ok.size} outside {ulps} ulp")
    assert ok.all(), f"{label}: {int((~ok).sum())} outputs beyond {ulps} bf16 ulp (max {float(err.max()):.2f})"


@pytest.mark.parametrize("t,H,weighted", [(7, 5120, False), (32, 5120, True), (3, 1000, True), (2, 65536, False),
                                          (5, 1, False), (1, 17, True), (4, 4100, True), (3, 12288, True)])
def test_rmsnorm_matches_oracle(t, H, weighted):
    say(f"case rmsnorm t={t} H={H} weighted={weighted}")
    rng = np.random.default_rng(t * 1000 + H)
    x = synth.draw_acts(rng, t, H)
    w = synth.f32_to_bf16_bits(rng.uniform(0.25, 2.0, H).astype(np.float32)) if weighted else None
    y = bits(w8.w8i_rmsnorm(bf16(x), 1e-6, weight=bf16(w) if weighted else None))
    check(y, oracle.rmsnorm(x, 1e-6, weight=w), f"rmsnorm t={t} H={H}")


def test_rmsnorm_columns_are_independent_and_strided_rows_identical():
    rng = np.random.default_rng(11)
    t, H = 32, 5120
    x = synth.draw_acts(rng, t, H)
    base = bits(w8.w8i_rmsnorm(bf16(x), 1e-6))
    perm = rng.permutation(t)
    say("case rmsnorm permutation / subset / strided")
    assert np.array_equal(bits(w8.w8i_rmsnorm(bf16(x[perm]), 1e-6)), base[perm])
    assert np.array_equal(bits(w8.w8i_rmsnorm(bf16(x[5:6]), 1e-6)), base[5:6])
    wide = torch.zeros((t, H + 40), dtype=torch.bfloat16, device=DEV)
    wide[:, 8:8 + H] = bf16(x)
    out = torch.zeros((t, H + 24), dtype=torch.bfloat16, device=DEV)
    w8.w8i_rmsnorm(wide[:, 8:8 + H], 1e-6, y=out[:, :H])
    assert np.array_equal(bits(out[:, :H]), base)
    # rows and outputs off 16-byte alignment take the 2-byte loads and stores
    for xo, yo in ((1, 0), (8, 3), (3, 5)):
        say(f"case rmsnorm offsets x+{xo} y+{yo}")
        wide.zero_()
        wide[:, xo:xo + H] = bf16(x)
        out.zero_()
        w8.w8i_rmsnorm(wide[:, xo:xo + H], 1e-6, y=out[:, yo:yo + H])
        assert np.array_equal(bits(out[:, yo:yo + H]), base)


def test_rmsnorm_zero_column_and_large_values():
    """A zero column gives zeros (0 / sqrt(eps)); a column of large equal magnitudes gives +-1
    exactly.  (The fp32 sum of squares must stay finite: |x| <= 2^50 over 512 features.)"""
    H = 512
    x = np.zeros((3, H), dtype=np.float32)
    x[1] = 3.0e12
    x[2, ::2], x[2, 1::2] = 2.0 ** 50, -(2.0 ** 50)
    xb = synth.f32_to_bf16_bits(x)
    y = bits(w8.w8i_rmsnorm(bf16(xb), 1e-6))
    check(y, oracle.rmsnorm(xb, 1e-6), "rmsnorm special columns")
    assert np.all(y[0] == 0)
    assert np.all(synth.bf16_bits_to_f32(y[2]) == np.where(np.arange(H) % 2 == 0, 1.0, -1.0))


@pytest.mark.parametrize("t,F", [(32, 17408), (5, 1000), (1, 3)])
def test_swiglu_matches_oracle(t, F):
    say(f"case swiglu t={t} F={F}")
    rng = np.random.default_rng(t + F)
    gu = synth.f32_to_bf16_bits((rng.standard_normal((t, 2 * F)) * 30).astype(np.float32))
    y = bits(w8.w8i_swiglu(bf16(gu)))
    check(y, oracle.swiglu(gu), f"swiglu t={t} F={F}")


def test_swiglu_extremes():
    """Gates far into both tails (exp overflow and underflow) and zeros."""
    g = np.array([0.0, -0.0, 88.0, 89.5, 104.0, 300.0, -88.0, -104.0, -300.0, 1e-30, -3.0e38], dtype=np.float32)
    u = np.array([1.0, 2.0, -3.0, 0.5, 1.0, 2.0, 1.0, 3.0, 5.0, 7.0, 1.0], dtype=np.float32)
    gu = synth.f32_to_bf16_bits(np.concatenate([g, u])[None])
    y = bits(w8.w8i_swiglu(bf16(gu)))
    check(y, oracle.swiglu(gu), "swiglu extremes")


@pytest.mark.parametrize("t,H", [(32, 5120), (3, 77)])
def test_residual_add_matches_oracle_and_may_alias(t, H):
    say(f"case residual add t={t} H={H}")
    rng = np.random.default_rng(t * 7 + H)
    a = synth.f32_to_bf16_bits((rng.standard_normal((t, H)) * 1e4).astype(np.float32))
    b = synth.draw_acts(rng, t, H)
    y = bits(w8.w8i_residual_add(bf16(a), bf16(b)))
    check(y, oracle.add(a, b), f"residual add t={t} H={H}")
    ad = bf16(a)
    w8.w8i_residual_add(ad, bf16(b), y=ad)
    assert np.array_equal(bits(ad), y), "in-place result differs"
