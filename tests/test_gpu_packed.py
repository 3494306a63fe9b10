"""The packed weight layout on the GPU, through the C ABI.

w8_pack is byte work: its output must equal the layout the header defines, element for element
(checked against a numpy construction of that layout).  The projection over the packed layout
runs the same K plan, so it must give the bits of w8_linear_invariant on the original layout
for every argument; parity with the oracle (2 bf16 ulps) then carries over, and is checked
directly on one shape as well.
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


def layout(q, s):
    """The packed layout, built from its definition with numpy indexing."""
    N, K = q.shape
    G = K // 32
    P = (G + 1) // 2
    strips = (N + 31) // 32
    qp = np.zeros((strips * 32, P * 64), dtype=np.int8)
    qp[:N, :K] = q
    sp = np.zeros((strips * 32, P * 2), dtype=np.uint16)
    sp[:N, :G] = s
    # [s, r, p, gs, c, b] -> [s, p, gs, c, r, b]
    codes = qp.reshape(strips, 32, P, 2, 2, 16).transpose(0, 2, 3, 4, 1, 5).reshape(-1)
    # [s, r, p, gs] -> [s, p, r, gs]
    scales = sp.reshape(strips, 32, P, 2).transpose(0, 2, 1, 3).reshape(-1)
    return codes, scales


@pytest.mark.parametrize("N,K", [(64, 256), (33, 160), (100, 1056), (1, 32), (6144, 5120)])
def test_pack_matches_the_defined_layout(N, K):
    say(f"case pack N={N} K={K}")
    rng = np.random.default_rng(N + K)
    q = synth.draw_codes(rng, N, K)
    s = synth.draw_scales(rng, N, K, 0.0)
    Wp, Sp = w8.w8_pack(i8(q), f16(s))
    codes, scales = layout(q, s)
    torch.cuda.synchronize()
    assert np.array_equal(Wp.cpu().numpy(), codes)
    assert np.array_equal(Sp.cpu().numpy().view(np.uint16), scales)


CASES = [  # N, K, T_pad: headline shape, ragged rows, odd K/32, empty slices, every T_pad, long K
    (6144, 5120, 32),
    (257, 1056, 48),
    (33, 160, 16),
    (64, 32, 16),
    (1000, 4096, 64),
    (40, 17408, 64),
    (24, 36896, 16),
    (5120, 6144, 32),
    (16400, 1056, 32),   # >= 16384 rows: two workgroups per CU (ring of two stages)
    (16384, 2080, 16),
]


@pytest.mark.parametrize("N,K,T_pad", CASES)
def test_packed_projection_gives_the_plain_bits(N, K, T_pad):
    say(f"case packed N={N} K={K} T_pad={T_pad}")
    rng = np.random.default_rng(3 * N + K)
    q = synth.draw_codes(rng, N, K)
    s = synth.draw_scales(rng, N, K, 0.0)
    x = synth.draw_acts(rng, T_pad, K)
    Wd, Sd, Xd = i8(q), f16(s), bf16(x)
    Wp, Sp = w8.w8_pack(Wd, Sd)
    full = bits(w8.w8_linear_invariant(Wd, Sd, Xd, T_pad, T_pad))
    assert np.array_equal(bits(w8.w8_linear_invariant_packed(Wp, Sp, Xd, T_pad, T_pad, N)), full)
    for t in (1, T_pad // 2 + 1):
        perm = rng.permutation(T_pad)[:t]
        got = bits(w8.w8_linear_invariant_packed(Wp, Sp, bf16(x[perm]), t, T_pad, N))
        assert np.array_equal(got, full[perm])


@pytest.mark.parametrize("N,K,T_pad", [(131172, 1024, 32), (131149, 5088, 32), (131105, 96, 16)])
def test_packed_persistent_kernel_gives_the_plain_bits(N, K, T_pad):
    """N >= 131072 at T_pad <= 32 runs the persistent kernel on both layouts (ragged tiles, odd K/32)."""
    say(f"case packed persistent N={N} K={K} T_pad={T_pad}")
    assert w8.w8_linear_invariant_packed_kernel(N, K, T_pad).startswith("gemm_w8g32_tiles")
    rng = np.random.default_rng(N + K)
    q = synth.draw_codes(rng, N, K)
    s = synth.draw_scales(rng, N, K, 0.0)
    x = synth.draw_acts(rng, T_pad, K)
    Wd, Sd, Xd = i8(q), f16(s), bf16(x)
    Wp, Sp = w8.w8_pack(Wd, Sd)
    for t in (1, T_pad):
        plain = bits(w8.w8_linear_invariant(Wd, Sd, Xd, t, T_pad))
        assert np.array_equal(bits(w8.w8_linear_invariant_packed(Wp, Sp, Xd, t, T_pad, N)), plain)


@pytest.mark.parametrize("N,K,T_pad", [(1000, 1056, 64), (300, 2080, 32), (70, 544, 16), (131172, 1024, 32),
                                       (257, 1056, 48), (131172, 1056, 64)])
def test_skipped_padding_loads_keep_the_bits(N, K, T_pad):
    """Activation loads whose 8 columns are all padding are not issued, nor are those columns'
    products formed (a tile with no live column skips its MFMAs, and at T_pad 48 or 64 a call with
    t <= 32 runs the one-tile kernel of T_pad 32); the kernels issue the loads of the
    ceil(t/8) live column groups.  On both sides of every such boundary (t = 8, 9, 16, 17, 32, 33,
    41, 48, 49) each column keeps the bits it has at full width, on both layouts.  The fourth case
    runs the persistent kernel throughout; in the last one (odd K/32, scales per stage) the kernel
    family itself changes at t = 32 / 33: the persistent one-tile kernel up to 32 columns, the
    two-tile split kernel above."""
    say(f"case padding loads N={N} K={K} T_pad={T_pad}")
    rng = np.random.default_rng(N * 7 + K)
    q = synth.draw_codes(rng, N, K)
    s = synth.draw_scales(rng, N, K, 0.0)
    x = synth.draw_acts(rng, T_pad, K)
    Wd, Sd, Xd = i8(q), f16(s), bf16(x)
    Wp, Sp = w8.w8_pack(Wd, Sd)
    full = bits(w8.w8_linear_invariant(Wd, Sd, Xd, T_pad, T_pad))
    assert np.array_equal(bits(w8.w8_linear_invariant_packed(Wp, Sp, Xd, T_pad, T_pad, N)), full)
    for t in (t for t in (8, 9, 16, 17, 32, 33, 41, 48, 49) if t < T_pad):
        perm = rng.permutation(T_pad)[:t]
        xp = bf16(x[perm])
        assert np.array_equal(bits(w8.w8_linear_invariant(Wd, Sd, xp, t, T_pad)), full[perm]), t
        assert np.array_equal(bits(w8.w8_linear_invariant_packed(Wp, Sp, xp, t, T_pad, N)), full[perm]), t


def test_packed_projection_matches_oracle():
    N, K, t, T_pad = 300, 2080, 20, 32
    rng = np.random.default_rng(77)
    q = synth.draw_codes(rng, N, K)
    s = synth.draw_scales(rng, N, K, 0.0)
    x = synth.draw_acts(rng, t, K)
    Wp, Sp = w8.w8_pack(i8(q), f16(s))
    y = bits(w8.w8_linear_invariant_packed(Wp, Sp, bf16(x), t, T_pad, N))
    ok, err = within_bf16_ulps(y, oracle.w8_linear(q, s, x), 2.0)
    say(f"packed vs oracle: max err {float(err.max()):.3f} ulp")
    assert ok.all()


@pytest.mark.parametrize("N,K,T_pad", [(1000, 2080, 32), (257, 544, 64), (131172, 1024, 32)])
def test_strided_activations_and_outputs(N, K, T_pad):
    """x read from inside a wider buffer (ldx > K, rows offset by 16 bytes) and y written into a wider
    one (ldy > N, an odd element offset): the contiguous call's bits, and nothing written outside y's
    window.  Plain and packed layouts; the last shape runs the persistent kernel."""
    say(f"case strided N={N} K={K} T_pad={T_pad}")
    rng = np.random.default_rng(N + 5 * K)
    q = synth.draw_codes(rng, N, K)
    s = synth.draw_scales(rng, N, K, 0.0)
    x = synth.draw_acts(rng, T_pad, K)
    Wd, Sd = i8(q), f16(s)
    Wp, Sp = w8.w8_pack(Wd, Sd)
    t = T_pad - 3
    want = bits(w8.w8_linear_invariant(Wd, Sd, bf16(x[:t]), t, T_pad))
    xw = torch.zeros((t, K + 72), dtype=torch.bfloat16, device=DEV)
    xw[:, 8:8 + K] = bf16(x[:t])
    xs = xw[:, 8:8 + K]
    for packed in (False, True):
        yw = torch.full((t + 1, N + 41), -7.0, dtype=torch.bfloat16, device=DEV)
        ys = yw[:t, 3:3 + N]
        if packed:
            w8.w8_linear_invariant_packed(Wp, Sp, xs, t, T_pad, N, y=ys)
        else:
            w8.w8_linear_invariant(Wd, Sd, xs, t, T_pad, y=ys)
        assert np.array_equal(bits(ys), want), f"packed={packed}"
        outside = torch.ones_like(yw, dtype=torch.bool)
        outside[:t, 3:3 + N] = False
        assert bool((yw[outside] == -7.0).all()), f"packed={packed}: written outside y"


def test_concurrent_streams_give_the_sequential_bits():
    """The library keeps no state between calls: two projections issued on two streams at once,
    four times each, give the bits each gives alone."""
    say("case concurrent streams")
    rng = np.random.default_rng(99)
    cases = []
    for N, K in ((6144, 5120), (1000, 2080)):
        q = synth.draw_codes(rng, N, K)
        s = synth.draw_scales(rng, N, K, 0.0)
        x = synth.draw_acts(rng, 32, K)
        Wp, Sp = w8.w8_pack(i8(q), f16(s))
        Xd = bf16(x)
        alone = bits(w8.w8_linear_invariant_packed(Wp, Sp, Xd, 32, 32, N))
        cases.append((Wp, Sp, Xd, N, alone))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = []
    for rep in range(4):
        for (Wp, Sp, Xd, N, _), st in zip(cases, streams):
            with torch.cuda.stream(st):
                outs.append((w8.w8_linear_invariant_packed(Wp, Sp, Xd, 32, 32, N), N))
    torch.cuda.synchronize()
    for k, (y, N) in enumerate(outs):
        assert np.array_equal(bits(y), cases[k % 2][4]), f"call {k} on stream {k % 2}"
