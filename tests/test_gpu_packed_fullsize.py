"""The packed projection at the decode workloads' full sizes, in the launch configuration the
benchmark times: weights packed once by w8_pack, calls captured in a HIP graph and replayed.

For each workload (1024x5120 T_pad 16, 6144x5120 T_pad 32, gate/up 34816x5120 and down
5120x17408 T_pad 64, the 248320x5120 head T_pad 32) and t in {1, T_pad}:
  * every output is within 2 bf16 ulps of the fp64 oracle, or -- where the exact value has cancelled
    below what fp32 accumulation can resolve -- within one fp32 rounding of sum |q s x| (counted);
  * every graph replay gives the eager call's bits, with eager work and synchronisation between
    the replays;
  * columns of a permuted subset keep their full-width bits (t-invariance on this path).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import parity_bar, within_bf16_ulps

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import invariant_quantized_decode_amd as w8  # noqa: E402
from tests.gpu_util import DEV, bf16, bits, f16, i8, say  # noqa: E402


def workload(index):
    """(label, codes, scales, activations [T_pad, K], T_pad) of the decode projections, by index."""
    if index == 0:
        d = synth.linear_1024_col0_fixed()
        return "1024x5120", d["q"], d["s"], d["xs"][16], 16
    if index == 1:
        d = synth.linear_6144_permuted()
        return "6144x5120", d["q"], d["s"], d["pool"], 32
    key = ("gate_up", "down")[index - 2]
    d = synth.mlp_pair()[key]
    return f"mlp {key}", d["q"], d["s"], d["pool"], 64


def check(label, q, s, x, T_pad, rng):
    N, K = q.shape
    Wp, Sp = w8.w8_pack(i8(q), f16(s))
    Xd = bf16(x)
    kernel = w8.w8_linear_invariant_packed_kernel(N, K, T_pad)
    full = None
    ref, mass = oracle.w8_linear(q, s, x, mass=True)  # x[:t] is a prefix of x: rows [:t] are the oracle at t
    for t in (T_pad, 1):
        say(f"case packed full size {label} t={t} ({kernel})")
        eager = w8.w8_linear_invariant_packed(Wp, Sp, Xd[:t], t, T_pad, N)
        want = bits(eager)
        ok, err, misses = parity_bar(want, ref[:t], mass[:t])
        say(f"{label} t={t}: all {ok.size} outputs, {misses} beyond 2 ulps within the fp32 floor")
        assert ok.all(), f"{label} t={t}: {int((~ok).sum())} outputs outside the parity bar"
        if full is None:
            full = want
        else:
            assert np.array_equal(want, full[:t]), f"{label}: column 0 changed bits at t={t}"
        # graph replay: the benchmark's launch path
        y = torch.zeros((t, N), dtype=torch.bfloat16, device=DEV)
        stream = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            w8.w8_linear_invariant_packed(Wp, Sp, Xd[:t], t, T_pad, N, y=y)  # warm-up outside the capture
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=stream):
                w8.w8_linear_invariant_packed(Wp, Sp, Xd[:t], t, T_pad, N, y=y)
        for rep in range(3):
            y.fill_(0.0)
            w8.w8_linear_invariant_packed(Wp, Sp, Xd[:1], 1, T_pad, N)  # eager work between replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert np.array_equal(bits(y), want), f"{label} t={t}: graph replay {rep} differs from eager"
    # a permuted subset of the columns keeps their full-width bits
    tp = max(1, T_pad // 2 + 1)
    perm = rng.permutation(T_pad)[:tp]
    got = bits(w8.w8_linear_invariant_packed(Wp, Sp, bf16(x[perm]), tp, T_pad, N))
    assert np.array_equal(got, full[perm]), f"{label}: permuted columns changed bits at t={tp}"


@pytest.mark.parametrize("index", range(4))
def test_packed_full_size_linear(index):
    label, q, s, x, T_pad = workload(index)
    check(label, q, s, x, T_pad, np.random.default_rng(100 + index))


def test_packed_full_size_head():
    d = synth.head_logprob()
    check("head 248320x5120", d["q"], d["s"], d["pool"], 32, np.random.default_rng(7))


def test_largest_accepted_shape():
    """The largest weights either layout accepts (codes just below 2^32 bytes: the buffer ranges and
    32-bit offsets the kernels use): 524287 x 8192 on the plain layout (one row short of 2^32
    bytes, a ragged last strip) and its first 524256 rows (16383 strips) packed.  Sampled rows --
    the last ones, whose offsets come within 8 KB of 2^32, among them -- are within 2 bf16 ulps of
    the oracle at T_pad 32 (the persistent kernel) and 64 (the split kernel), the packed rows give
    the plain bits, and a column keeps its bits at t = 1."""
    N, K, Np = 524287, 8192, 524256
    assert N * K < 1 << 32 <= (N + 1) * K and Np // 32 * (K // 64) * 2048 < 1 << 32
    rng = np.random.default_rng(4242)
    q = synth.draw_codes(rng, N, K)
    s = synth.draw_scales(rng, N, K, 0.0)
    x = synth.draw_acts(rng, 64, K)
    Wd, Sd, Xd = i8(q), f16(s), bf16(x)
    Wp, Sp = w8.w8_pack(Wd[:Np], Sd[:Np])
    rows = np.unique(np.concatenate([[0, Np - 1, Np], np.arange(N - 8, N), rng.choice(N, size=24, replace=False)]))
    for T_pad in (32, 64):
        t = T_pad
        say(f"case largest shape {N}x{K} T_pad={T_pad} ({w8.w8_linear_invariant_kernel(N, K, T_pad)}, "
            f"packed {w8.w8_linear_invariant_packed_kernel(Np, K, T_pad)})")
        y = bits(w8.w8_linear_invariant(Wd, Sd, Xd[:t], t, T_pad))
        ok, err = within_bf16_ulps(y[:, rows], oracle.w8_linear(q, s, x[:t], rows=rows), 2.0)
        say(f"largest shape T_pad={T_pad}: max err {float(err.max()):.3f} ulp over {ok.size} sampled outputs")
        assert ok.all()
        yp = bits(w8.w8_linear_invariant_packed(Wp, Sp, Xd[:t], t, T_pad, Np))
        assert np.array_equal(yp, y[:, :Np]), f"T_pad={T_pad}: packed rows differ from the plain bits"
        y1 = bits(w8.w8_linear_invariant(Wd, Sd, Xd[:1], 1, T_pad))
        assert np.array_equal(y1, y[:1]), f"T_pad={T_pad}: column 0 changed bits at t=1"
    del Wd, Sd, Wp, Sp
    torch.cuda.empty_cache()
