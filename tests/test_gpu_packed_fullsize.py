"""The packed projection at the decode workloads' full sizes, in the launch configuration the
benchmark times: weights packed once by w8_pack, calls captured in a HIP graph and replayed.

For each workload (1024x5120 T_pad 16, 6144x5120 T_pad 32, gate/up 34816x5120 and down
5120x17408 T_pad 64, the 248320x5120 head T_pad 32) and t in {1, T_pad}:
  * sampled rows are within 2 bf16 ulps of the fp64 oracle (computed row by row);
  * every graph replay gives the eager call's bits, with eager work and synchronisation between
    the replays;
  * columns of a permuted subset keep their full-width bits (t-invariance on this path).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import within_bf16_ulps

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
    for t in (T_pad, 1):
        say(f"case packed full size {label} t={t} ({kernel})")
        eager = w8.w8_linear_invariant_packed(Wp, Sp, Xd[:t], t, T_pad, N)
        want = bits(eager)
        rows = np.sort(np.concatenate([rng.choice(N, size=384, replace=False), [0, N - 1]]))
        ok, err = within_bf16_ulps(want[:, rows], oracle.w8_linear(q, s, x[:t], rows=rows), 2.0)
        say(f"{label} t={t}: max err {float(err.max()):.3f} ulp over {ok.size} sampled outputs")
        assert ok.all(), f"{label} t={t}: {int((~ok).sum())} sampled outputs beyond 2 ulps"
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
