"""The K-slice path for small N, through the C ABI: each strip's 8 K-slices on separate workgroups, the
fp64 slice sums in the caller's (optional) workspace, folded by a second launch.

It runs the same slices, MFMA chain, fp64 operations in the same order, left fold and rounding as the
one-launch kernels, so every output must carry the one-launch bits: with and without the workspace
(workspace=None runs the one-launch kernel), on both weight layouts, ragged rows, odd and tiny K (empty
slices), long K (slices of several chunks), T_pad 16 / 32 and T_pad 48 / 64 called with t <= 32.  Also:
every output of 1024x5120 within the parity bar of the oracle, t-invariance, a workspace poisoned with
NaN before the call (every slice sum is written before the fold reads it), a workspace one byte short
(the one-launch kernel runs), and HIP-graph replays.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import parity_bar

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import invariant_quantized_decode_amd as w8  # noqa: E402
from tests.gpu_util import DEV, bf16, bits, f16, i8, say  # noqa: E402


def problem(seed, N, K, T):
    rng = np.random.default_rng(seed)
    q = synth.draw_codes(rng, N, K)
    s = synth.draw_scales(rng, N, K, 0.0)
    x = synth.draw_acts(rng, T, K)
    return q, s, x


def run(packed, dev, x, t, T_pad, N, workspace="auto"):
    if packed:
        return w8.w8_linear_invariant_packed(dev["Wp"], dev["Sp"], x, t, T_pad, N, workspace=workspace)
    return w8.w8_linear_invariant(dev["W"], dev["S"], x, t, T_pad, workspace=workspace)


def upload(q, s):
    W, S = i8(q), f16(s)
    Wp, Sp = w8.w8_pack(W, S)
    return dict(W=W, S=S, Wp=Wp, Sp=Sp)


SHAPES = [  # N, K, T_pad, t values
    (1024, 5120, 16, (1, 7, 8, 9, 16)),
    (1024, 5120, 32, (1, 17, 24, 32)),
    (1000, 5120, 32, (3, 32)),          # ragged last strip
    (2048, 1056, 32, (1, 9, 32)),       # 64 strips, odd K/32 (slice 7 takes the last group)
    (33, 160, 16, (1, 16)),             # 5 groups: empty slices
    (64, 32, 16, (2, 16)),              # one group: only slice 7 is not empty
    (500, 17408, 32, (1, 32)),          # long slices: several chunks per workgroup
    (257, 5152, 64, (1, 20, 32)),       # T_pad 64 with t <= 32 runs at width 32
    (96, 2080, 48, (5, 32)),
]


@pytest.mark.parametrize("N,K,T_pad,ts", SHAPES)
def test_kslice_gives_the_one_launch_bits(N, K, T_pad, ts):
    say(f"case kslice N={N} K={K} T_pad={T_pad}")
    assert w8.w8_linear_invariant_workspace_bytes(N, K, T_pad) > 0
    q, s, x = problem(N + 3 * K, N, K, T_pad)
    dev = upload(q, s)
    rng = np.random.default_rng(N)
    for packed in (False, True):
        for t in ts:
            perm = rng.permutation(T_pad)[:t]
            xd = bf16(x[perm])
            one = bits(run(packed, dev, xd, t, T_pad, N, workspace=None))
            ks = bits(run(packed, dev, xd, t, T_pad, N))
            assert np.array_equal(ks, one), f"packed={packed} t={t}: {int(np.sum(ks != one))} outputs differ"


def test_kslice_parity_with_the_oracle_on_every_output():
    N, K = 1024, 5120
    q, s, x = problem(1, N, K, 16)
    ref, mass = oracle.w8_linear(q, s, x, mass=True)
    dev = upload(q, s)
    for packed in (False, True):
        for t, T_pad in ((16, 16), (1, 16), (16, 32)):
            say(f"case kslice parity packed={packed} t={t} T_pad={T_pad}")
            y = bits(run(packed, dev, bf16(x[:t]), t, T_pad, N))
            ok, err, misses = parity_bar(y, ref[:t], mass[:t])
            say(f"  {ok.size} outputs, {misses} beyond 2 ulps within the fp32 floor")
            assert ok.all(), f"{int((~ok).sum())} outputs beyond the bar"


def test_kslice_columns_keep_their_bits_for_every_t():
    N, K, T_pad = 1024, 5120, 32
    q, s, x = problem(2, N, K, T_pad)
    dev = upload(q, s)
    rng = np.random.default_rng(5)
    for packed in (False, True):
        full = bits(run(packed, dev, bf16(x), T_pad, T_pad, N))
        for t in (1, 2, 8, 9, 16, 17, 31):
            perm = rng.permutation(T_pad)[:t]
            got = bits(run(packed, dev, bf16(x[perm]), t, T_pad, N))
            assert np.array_equal(got, full[perm]), f"packed={packed} t={t}"


def test_poisoned_and_short_workspaces():
    """Every slice sum is written before the fold reads it (a NaN-filled workspace changes nothing); a
    workspace one byte short of 8 * t * N doubles makes the call run the one-launch kernel."""
    N, K, T_pad, t = 1000, 5120, 16, 13
    q, s, x = problem(3, N, K, T_pad)
    dev = upload(q, s)
    xd = bf16(x[:t])
    need = w8.w8_linear_invariant_workspace_bytes(N, K, T_pad)
    for packed in (False, True):
        want = bits(run(packed, dev, xd, t, T_pad, N, workspace=None))
        ws = torch.full((need // 8,), float("nan"), dtype=torch.float64, device=DEV).view(torch.uint8)
        assert np.array_equal(bits(run(packed, dev, xd, t, T_pad, N, workspace=ws)), want)
        short = torch.empty(8 * 8 * t * N - 1, dtype=torch.uint8, device=DEV)
        assert np.array_equal(bits(run(packed, dev, xd, t, T_pad, N, workspace=short)), want)


def test_kslice_in_a_graph():
    """Captured with its workspace (allocated inside the capture), replayed three times with eager calls
    of the same entry point between the replays: every replay gives the eager bits."""
    N, K, T_pad = 1024, 5120, 16
    q, s, x = problem(4, N, K, T_pad)
    dev = upload(q, s)
    Xd = bf16(x)
    for packed in (False, True):
        eager = bits(run(packed, dev, Xd, 16, T_pad, N))
        y = torch.empty((16, N), dtype=torch.bfloat16, device=DEV)
        call = (lambda: w8.w8_linear_invariant_packed(dev["Wp"], dev["Sp"], Xd, 16, T_pad, N, y=y,
                                                      workspace="auto")) if packed else \
            (lambda: w8.w8_linear_invariant(dev["W"], dev["S"], Xd, 16, T_pad, y=y, workspace="auto"))
        call()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call()
        for rep in range(3):
            y.fill_(0)
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(bits(y), eager), f"packed={packed} replay {rep}"
            run(packed, dev, bf16(x[:3]), 3, T_pad, N)
            torch.cuda.synchronize()
