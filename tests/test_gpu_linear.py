"""W8A16 fixed-width projection on the GPU, through the C ABI.

Parity: every output within 2 bf16 ulps of the fp64 oracle (the project's
tolerance; the ninfer page, "Reading" paragraph under "Measured", puts
schedule-to-schedule differences at 1-2 bf16 ulps).  Invariance: every column's
bits are identical for every t <= T_pad, under column permutations, across
repeats, across T_pad and across row slices (the page's "Proposal: opt-in
fixed decode width": no column's arithmetic involves another, one schedule for every t).
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
from tests.gpu_util import bf16, bits, f16, i8, say  # noqa: E402


def run(Wd, Sd, Xd, t, T_pad):
    return bits(w8.w8_linear_invariant(Wd, Sd, Xd, t, T_pad))


def check_parity(y_bits, ref, label):
    ok, err = within_bf16_ulps(y_bits, ref, 2.0)
    say(f"{label}: max err {float(err.max()):.3f} bf16 ulp, {int((~ok).sum())} of {ok.size} outside 2 ulps")
    assert ok.all(), f"{label}: {int((~ok).sum())} outputs beyond 2 bf16 ulps (max {float(err.max()):.2f})"


def check_bar(y_bits, ref, mass, label):
    """Full-size parity: within 2 bf16 ulps, or -- where the exact value has cancelled below the fp32
    accumulation floor -- within one fp32 rounding of sum |q s x|; the misses of 2 ulps are counted."""
    ok, err, misses = parity_bar(y_bits, ref, mass)
    say(f"{label}: {ok.size} outputs, {misses} beyond 2 bf16 ulps (all within the fp32 floor: "
        f"{bool(ok.all())}), max err {float(err[err <= 2].max()) if (err <= 2).any() else 0:.3f} ulp elsewhere")
    assert ok.all(), f"{label}: {int((~ok).sum())} outputs beyond 2 bf16 ulps and the fp32 floor"


SMALL = [  # N, K, t, T_pad, scale_eps: ragged rows, uneven slices, empty slices, several tiles
    (100, 512, 7, 16, 1e-4),
    (257, 1056, 33, 48, 0.0),
    (64, 32, 1, 16, 0.0),
    (1, 64, 64, 64, 1e-4),
    (1000, 4096, 64, 64, 0.0),
    (96, 8192, 32, 32, 1e-4),
    (33, 160, 16, 16, 0.0),
]


@pytest.mark.parametrize("N,K,t,T_pad,eps", SMALL)
def test_small_shapes_match_oracle(N, K, t, T_pad, eps):
    say(f"case small N={N} K={K} t={t} T_pad={T_pad}")
    q, s, x = synth.small_linear(N * 7 + K + t, N, K, t, eps)
    y = run(i8(q), f16(s), bf16(x), t, T_pad)
    check_parity(y, oracle.w8_linear(q, s, x), f"N={N} K={K} t={t}")


def test_subnormal_and_zero_scales_and_extreme_codes():
    N, K, t = 64, 1024, 32
    rng = np.random.default_rng(5)
    q = synth.draw_codes(rng, N, K)
    q[::5] = -127
    q[3, :] = -128  # accepted by the format
    s = rng.integers(0, 0x0400, size=(N, K // 32)).astype(np.uint16)  # all subnormal (or zero)
    s[0] = 0
    s[1] = 0x7BFF  # fp16 max
    x = synth.draw_acts(rng, t, K)
    say("case subnormal scales")
    y = run(i8(q), f16(s), bf16(x), t, 32)
    check_parity(y, oracle.w8_linear(q, s, x), "subnormal scales")


def test_identity_and_integer_sums_are_bitwise_exact():
    K = N = 512
    q = np.eye(N, K, dtype=np.int8)
    s = np.full((N, K // 32), 0x3C00, dtype=np.uint16)
    x = synth.draw_acts(np.random.default_rng(1), 16, K)
    say("case identity")
    y = run(i8(q), f16(s), bf16(x), 16, 16)
    assert np.array_equal(y, x[:, :N])
    q1 = np.ones((64, 5120), dtype=np.int8)
    s1 = np.full((64, 160), 0x3C00, dtype=np.uint16)
    xi = np.random.default_rng(2).integers(-8, 9, size=(32, 5120))
    x1 = synth.f32_to_bf16_bits(xi.astype(np.float32))
    say("case all-ones integer sums")
    y1 = run(i8(q1), f16(s1), bf16(x1), 32, 32)
    want = np.array([oracle.bf16_round(float(v)) for v in xi.sum(axis=1)], dtype=np.uint16)
    assert np.array_equal(y1, np.repeat(want[:, None], 64, axis=1))


def test_padding_is_never_read_or_written():
    """A T_pad-wide activation buffer with NaN rows beyond t, and a NaN-filled output buffer:
    the real columns equal the clean run and the output rows beyond t keep their NaN."""
    N, K, t, T_pad = 128, 2048, 5, 32
    q, s, x = synth.small_linear(77, N, K, T_pad, 0.0)
    Wd, Sd = i8(q), f16(s)
    clean = run(Wd, Sd, bf16(x[:t]), t, T_pad)
    poisoned = x.copy()
    poisoned[t:] = 0x7FC1
    ybuf = torch.full((T_pad, N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    w8.w8_linear_invariant(Wd, Sd, bf16(poisoned), t, T_pad, y=ybuf)
    yb = bits(ybuf)
    assert np.array_equal(yb[:t], clean)
    assert np.all(np.isnan(synth.bf16_bits_to_f32(yb[t:])))


def test_linearity_within_rounding():
    N, K, t = 256, 4096, 16
    rng = np.random.default_rng(12)
    q = synth.draw_codes(rng, N, K)
    s = synth.draw_scales(rng, N, K, 1e-4)
    a = rng.integers(-64, 65, size=(t, K)).astype(np.float32) / 16
    b = rng.integers(-64, 65, size=(t, K)).astype(np.float32) / 16
    x1, x2, x12 = (synth.f32_to_bf16_bits(v) for v in (a, b, a + b))
    Wd, Sd = i8(q), f16(s)
    say("case linearity")
    y1, y2, y12 = (synth.bf16_bits_to_f32(run(Wd, Sd, bf16(v), t, 16)).astype(np.float64) for v in (x1, x2, x12))
    # each side within 2 ulps of its exact value, plus one rounding of the sum
    from tests.helpers import ulp_bf16
    bound = 2 * (ulp_bf16(y1) + ulp_bf16(y2) + ulp_bf16(y12)) + ulp_bf16(y1 + y2)
    assert np.all(np.abs(y12 - (y1 + y2)) <= bound)


def test_bitwise_sign_and_scale_invariants():
    N, K, t = 256, 2048, 32
    q, s, x = synth.small_linear(31, N, K, t, 1e-4)
    Wd, Sd = i8(q), f16(s)
    say("case sign/scale invariants")
    y = run(Wd, Sd, bf16(x), t, 32)
    assert np.array_equal(run(Wd, Sd, bf16(x ^ np.uint16(0x8000)), t, 32), y ^ np.uint16(0x8000))
    assert np.array_equal(run(i8(-q), Sd, bf16(x), t, 32), y ^ np.uint16(0x8000))
    two_x = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(x) * 2)
    y2 = run(Wd, Sd, bf16(two_x), t, 32)
    assert np.array_equal(synth.bf16_bits_to_f32(y2), synth.bf16_bits_to_f32(y) * 2)


# --------------------------------------------------------------- workloads
def test_linear_1024x5120_t_sweep_column0_fixed():
    """T_pad 16, t = 1..16, column 0 fixed and the others fresh for each t: y[:, 0] is
    bitwise identical for every t, and every column is within 2 ulps of the oracle."""
    d = synth.linear_1024_col0_fixed()
    q, s = d["q"], d["s"]
    Wd, Sd = i8(q), f16(s)
    col0 = None
    xs_all, ys_all = [], []
    for t in range(1, 17):
        say(f"case 1024x5120 t={t}")
        y = run(Wd, Sd, bf16(d["xs"][t]), t, 16)
        if col0 is None:
            col0 = y[0].copy()
        assert np.array_equal(y[0], col0), f"column 0 changed bits at t={t}"
        xs_all.append(d["xs"][t])
        ys_all.append(y)
    X = np.concatenate(xs_all)
    Y = np.concatenate(ys_all)
    check_parity(Y, oracle.w8_linear(q, s, X), "1024x5120 all t")


def test_linear_6144x5120_permuted_columns():
    """T_pad 32, t = 1..32, each t a random ordered subset of a 32-column pool: every pool
    column's bits equal its bits in the identity-order t = 32 run; that run matches the oracle."""
    d = synth.linear_6144_permuted()
    q, s, pool = d["q"], d["s"], d["pool"]
    Wd, Sd = i8(q), f16(s)
    say("case 6144x5120 identity t=32")
    base = run(Wd, Sd, bf16(pool), 32, 32)
    check_parity(base, oracle.w8_linear(q, s, pool), "6144x5120 t=32")
    for t in range(1, 33):
        cols = d["perms"][t]
        y = run(Wd, Sd, bf16(pool[cols]), t, 32)
        assert np.array_equal(y, base[cols]), f"bits changed at t={t}"
    again = run(Wd, Sd, bf16(pool), 32, 32)
    assert np.array_equal(again, base), "repeat run differs"


def test_t_pad_and_row_slice_independence():
    """The same columns at T_pad 32 and 64 give the same bits; so does a slice of rows run as
    its own problem (the row-sharded layout), since the K plan depends on K alone."""
    N, K, t = 4096, 5120, 32
    q, s, x = synth.small_linear(44, N, K, t, 0.0)
    Wd, Sd, Xd = i8(q), f16(s), bf16(x)
    say("case T_pad / row-slice independence")
    a = run(Wd, Sd, Xd, t, 32)
    b = run(Wd, Sd, Xd, t, 64)
    c = run(Wd, Sd, Xd, 16, 16)
    assert np.array_equal(a, b) and np.array_equal(a[:16], c)
    r0, r1 = 1000, 1000 + 544
    sl = run(Wd[r0:r1], Sd[r0:r1], Xd, t, 32)
    assert np.array_equal(sl, a[:, r0:r1])


# --------------------------------- the LDS-staged split-K variants (T_pad <= 32)
STAGING = [  # N, K, t, T_pad: LDS ring depth 3 / 2 by the strip's scale bytes, then per-stage scales
    (257, 1056, 32, 32),   # K/32 = 33 (odd), depth 3
    (40, 17408, 5, 32),    # K/32 = 544, depth 3
    (24, 36896, 3, 16),    # K/32 = 1153 (odd), depth 2
    (16, 64000, 16, 16),   # K/32 = 2000: scales too large for LDS, loaded per stage
    (70, 15872, 48, 48),   # two column tiles, depth 2, K/32 = 496 (the largest that fits)
    (40, 16000, 64, 64),   # two column tiles, K/32 = 500 > 496: scales loaded per stage
    (33, 16032, 64, 64),   # the same with K/32 = 501 (odd)
]


@pytest.mark.parametrize("N,K,t,T_pad", STAGING)
def test_staging_variants_match_oracle_and_row_slices(N, K, t, T_pad):
    say(f"case staging N={N} K={K} t={t} T_pad={T_pad}")
    q, s, x = synth.small_linear(N + K + T_pad, N, K, t, 0.0)
    Wd, Sd, Xd = i8(q), f16(s), bf16(x)
    y = run(Wd, Sd, Xd, t, T_pad)
    check_parity(y, oracle.w8_linear(q, s, x), f"staging N={N} K={K} t={t}")
    part = run(Wd[3:], Sd[3:], Xd, t, T_pad)
    assert np.array_equal(part, y[:, 3:]), "row slice differs"


@pytest.mark.parametrize("T_pad", [16, 32, 48, 64])
def test_unaligned_scales_give_the_same_bits(T_pad):
    """Scales that are not 16-byte aligned cannot be copied to LDS in 16-byte pieces and are
    loaded per stage instead; the arithmetic, and so every bit, is the same."""
    N, K = 300, 5120
    q, s, x = synth.small_linear(77 + T_pad, N, K, T_pad, 0.0)
    Wd, Sd, Xd = i8(q), f16(s), bf16(x)
    G = K // 32
    flat = torch.zeros(N * G + 8, dtype=torch.int16, device=Sd.device)
    Smis = flat[1:1 + N * G].view(N, G)
    Smis.copy_(Sd)
    assert Smis.data_ptr() % 16 == 2
    for t in (1, T_pad):
        say(f"case unaligned scales T_pad={T_pad} t={t}")
        a = run(Wd, Sd, Xd[:t], t, T_pad)
        b = run(Wd, Smis, Xd[:t], t, T_pad)
        assert np.array_equal(a, b), f"aligned and unaligned scales differ at t={t}"
    check_parity(a, oracle.w8_linear(q, s, x), f"unaligned-scales case T_pad={T_pad}")


@pytest.mark.slow
def test_mlp_projections_t_values():
    """gate/up 34816x5120 and down 5120x17408 at T_pad 64 (plain layout), t in {1,5,17,24,32,48,64}:
    every output at t = 64 and at t = 1 within the parity bar (2 ulps; the fp32 floor where the
    exact value has cancelled), every column t-invariant."""
    d = synth.mlp_pair()
    for key in ("gate_up", "down"):
        p = d[key]
        q, s, pool = p["q"], p["s"], p["pool"]
        Wd, Sd = i8(q), f16(s)
        say(f"case mlp {key} t=64")
        base = run(Wd, Sd, bf16(pool), 64, 64)
        ref, mass = oracle.w8_linear(q, s, pool, mass=True)
        check_bar(base, ref, mass, f"mlp {key} t=64 (all outputs)")
        one = run(Wd, Sd, bf16(pool[:1]), 1, 64)
        check_bar(one, ref[:1], mass[:1], f"mlp {key} t=1 (all outputs)")
        for t in synth.MLP_T_VALUES:
            cols = d["perms"][t]
            y = run(Wd, Sd, bf16(pool[cols]), t, 64)
            assert np.array_equal(y, base[cols]), f"{key}: bits changed at t={t}"


# ------------------------------------------------- large N (persistent tile kernel)
LARGE = [  # N, K, T_pad: N >= 131072 selects the persistent kernel for T_pad <= 32
    (131072 + 100, 1024, 32),
    (131072 + 33, 96, 16),      # K/32 = 3: odd group count, seven empty slices
    (131072 + 256, 5120, 32),   # K/32 = 160: scales loaded 8 groups at a time
    (131072 + 77, 5088, 32),    # K/32 = 159: scales loaded per stage, odd group count
]


@pytest.mark.parametrize("N,K,T_pad", LARGE)
def test_large_n_matches_row_slices_and_oracle(N, K, T_pad):
    """The persistent mapping and the split-K mapping (row slices run as their own, smaller
    problems) give the same bits; every output is within the parity bar of the oracle."""
    rng = np.random.default_rng(N + K)
    q = synth.draw_codes(rng, N, K)
    s = synth.draw_scales(rng, N, K, 0.0)
    x = synth.draw_acts(rng, T_pad, K)
    Wd, Sd, Xd = i8(q), f16(s), bf16(x)
    for t in (1, 7, T_pad):
        say(f"case large N={N} K={K} T_pad={T_pad} t={t}")
        full = run(Wd, Sd, Xd[:t], t, T_pad)
        for r0, r1 in ((0, 544), (N - 300, N), (65536 + 17, 65536 + 17 + 1000)):
            part = run(Wd[r0:r1], Sd[r0:r1], Xd[:t], t, T_pad)
            assert np.array_equal(part, full[:, r0:r1]), f"rows {r0}:{r1} differ at t={t}"
        check_bar(full, *oracle.w8_linear(q, s, x[:t], mass=True), f"large N={N} K={K} t={t} (all outputs)")
