"""Decode-step chain of one 5120-hidden W8 layer on the GPU, with random lane compositions.

Layer (T_pad 32, every projection through w8_linear_invariant, glue through the column-local
kernels): RMSNorm -> QKV 7168x5120 -> the q slice [0, 6144) (a column-local stand-in for
attention, which is outside this library) -> O 5120x6144 -> + residual -> RMSNorm -> gate+up
34816x5120 -> SwiGLU -> down 5120x17408 -> + residual.

32 lanes of hidden state run 200 steps; each step takes t random distinct lanes (t uniform in
1..32) in random slot order.  The invariance pin (the ninfer issue's "Proposal: opt-in fixed
decode width": one schedule at the padded width, no column's arithmetic touching another's):
every lane replayed alone (t = 1, slot 0) reproduces bit for bit every state it had inside the
compositions.  The values are checked against the oracle on the chain's own inputs at two steps
(the first, with N(0, 1) states, and a late one, where the residual stream has grown to ~1e7):
every output of each projection within the parity bar (2 bf16 ulps; the fp32 accumulation floor
where the exact value cancels), each glue op within 1 bf16 ulp.
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

EPS = 1e-6
T_PAD = synth.CHAIN_T_PAD
Q = synth.CHAIN_Q


def layer(h, W, trace=None):
    """One decode layer on the lanes h (bf16 [t, H]); `trace` collects the intermediates."""
    t = h.shape[0]
    x = w8.w8i_rmsnorm(h, EPS)
    qkv = w8.w8_linear_invariant(*W["qkv"], x, t, T_PAD)
    o = w8.w8_linear_invariant(*W["o"], qkv[:, :Q], t, T_PAD)
    h1 = w8.w8i_residual_add(h, o)
    x2 = w8.w8i_rmsnorm(h1, EPS)
    gu = w8.w8_linear_invariant(*W["gate_up"], x2, t, T_PAD)
    a = w8.w8i_swiglu(gu)
    d = w8.w8_linear_invariant(*W["down"], a, t, T_PAD)
    out = w8.w8i_residual_add(h1, d)
    if trace is not None:
        trace.update(h=h, x=x, qkv=qkv, o=o, h1=h1, x2=x2, gu=gu, a=a, d=d, out=out)
    return out


def spot_check(trace, Wh, rng, label):
    """Oracle parity of every op of one step, on that step's own GPU inputs."""
    hb = {k: bits(v) for k, v in trace.items()}

    def glue(y, ref, name):
        ok, err = within_bf16_ulps(y, ref, 1.0)
        say(f"{label} {name}: max err {float(err.max()):.3f} bf16 ulp")
        assert ok.all(), f"{label} {name}: {int((~ok).sum())} outputs beyond 1 bf16 ulp"

    def proj(name, x_bits, y_bits):
        q, s = Wh[name]
        ref, mass = oracle.w8_linear(q, s, x_bits, mass=True)
        ok, err, misses = parity_bar(y_bits, ref, mass)
        say(f"{label} {name}: all {ok.size} outputs, {misses} beyond 2 bf16 ulps within the fp32 floor")
        assert ok.all(), f"{label} {name}: {int((~ok).sum())} outputs beyond 2 bf16 ulps"

    glue(hb["x"], oracle.rmsnorm(hb["h"], EPS), "rmsnorm 1")
    proj("qkv", hb["x"], hb["qkv"])
    proj("o", np.ascontiguousarray(hb["qkv"][:, :Q]), hb["o"])
    glue(hb["h1"], oracle.add(hb["h"], hb["o"]), "residual 1")
    glue(hb["x2"], oracle.rmsnorm(hb["h1"], EPS), "rmsnorm 2")
    proj("gate_up", hb["x2"], hb["gu"])
    glue(hb["a"], oracle.swiglu(hb["gu"]), "swiglu")
    proj("down", hb["a"], hb["d"])
    glue(hb["out"], oracle.add(hb["h1"], hb["d"]), "residual 2")


def test_decode_chain_lanes_are_composition_independent():
    say("case chain: drawing the layer (seed 4)")
    c = synth.chain_layer()
    Wh = c["weights"]
    W = {name: (i8(q), f16(s)) for name, (q, s) in Wh.items()}
    states = bf16(c["lanes"]).clone()
    init = states.clone()
    steps = c["steps"]
    rng = np.random.default_rng(40)
    check_at = {0, 150}
    history = {lane: [] for lane in range(synth.CHAIN_LANES)}
    for i, lanes in enumerate(steps):
        idx = torch.as_tensor(lanes, dtype=torch.int64, device=states.device)
        trace = {} if i in check_at else None
        out = layer(states.index_select(0, idx).contiguous(), W, trace)
        states.index_copy_(0, idx, out)
        for slot, lane in enumerate(lanes):
            history[int(lane)].append(out[slot])
        if trace is not None:
            say(f"case chain step {i}: t={len(lanes)}, oracle spot checks")
            spot_check(trace, Wh, rng, f"step {i} (t={len(lanes)})")
    torch.cuda.synchronize()
    say(f"case chain: {len(steps)} composed steps done, replaying {synth.CHAIN_LANES} lanes alone")
    for lane in range(synth.CHAIN_LANES):
        h = init[lane:lane + 1].contiguous()
        replay = []
        for _ in history[lane]:
            h = layer(h, W)
            replay.append(h[0])
        if not replay:
            continue
        got, want = bits(torch.stack(replay)), bits(torch.stack(history[lane]))
        bad = np.flatnonzero(np.any(got != want, axis=1))
        assert bad.size == 0, f"lane {lane}: replay differs from the composed run at its step(s) {bad[:8].tolist()}"
    final = synth.bf16_bits_to_f32(bits(states))
    say(f"case chain: all lanes bitwise identical alone; final |h| max {float(np.abs(final).max()):.3g}")
    assert np.isfinite(final).all()


def fast_layer(h, P):
    """The same layer on the fast path: packed weights (w8_pack) and the fused epilogues
    (O + residual, gate+up + SwiGLU, down + residual)."""
    t = h.shape[0]
    x = w8.w8i_rmsnorm(h, EPS)
    qkv = w8.w8_linear_invariant_packed(*P["qkv"], x, t, T_PAD, P["n"]["qkv"])
    h1 = w8.w8_linear_add_invariant_packed(*P["o"], qkv[:, :Q], h, t, T_PAD, P["n"]["o"])
    x2 = w8.w8i_rmsnorm(h1, EPS)
    a = w8.w8_linear_swiglu_invariant_packed(*P["gate_up"], x2, t, T_PAD, P["n"]["gate_up"] // 2)
    return w8.w8_linear_add_invariant_packed(*P["down"], a, h1, t, T_PAD, P["n"]["down"])


def test_fast_path_chain_gives_the_plain_bits():
    """Thirty steps of random compositions through both paths: every lane state is bitwise the
    same (packed = plain layout and fused = unfused composition, step after step)."""
    say("case chain fast path: drawing the layer (seed 4)")
    c = synth.chain_layer()
    Wh = c["weights"]
    W = {name: (i8(q), f16(s)) for name, (q, s) in Wh.items()}
    P = {name: w8.w8_pack(*W[name]) for name in W}
    P["n"] = {name: Wh[name][0].shape[0] for name in Wh}
    plain = bf16(c["lanes"]).clone()
    fast = plain.clone()
    for i, lanes in enumerate(c["steps"][:30]):
        idx = torch.as_tensor(lanes, dtype=torch.int64, device=plain.device)
        a = layer(plain.index_select(0, idx).contiguous(), W)
        b = fast_layer(fast.index_select(0, idx).contiguous(), P)
        plain.index_copy_(0, idx, a)
        fast.index_copy_(0, idx, b)
        assert np.array_equal(bits(a), bits(b)), f"step {i} (t={len(lanes)}): fast path differs"
    say("case chain fast path: 30 steps bitwise identical")
