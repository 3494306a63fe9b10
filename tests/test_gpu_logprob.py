"""Block logprob and the EXP32 / LOG32 device functions on the GPU, through the C ABI.

The fp32 arithmetic is fixed step by step (tokenspeed "Numerics envelopes",
alignment.trainer "--logprob-order blockwise"; "Logprobs" section; block_sumexp
leaf contract), and EXP32/LOG32 are correctly rounded, so the GPU is expected to
equal the fixed-order fp32 oracle bit for bit; the pass bar is 1e-5 absolute.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import ln_rn32

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import invariant_quantized_decode_amd as w8  # noqa: E402
from tests.gpu_util import DEV, bf16, bits, f16, f32, host, i8, say  # noqa: E402


def f32bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def gpu_logprob(logits_bits, targets, block, pad_to=None):
    Ld = bf16(logits_bits)
    if pad_to is not None:  # a strided (ldl > V) view, unaligned rows
        t, V = logits_bits.shape
        buf = torch.zeros((t, pad_to), dtype=torch.bfloat16, device=DEV)
        buf[:, :V] = Ld
        Ld = buf[:, :V]
    return host(w8.vocab_block_logprob(Ld, torch.from_numpy(np.asarray(targets, np.int64)).to(DEV), block))


def compare(out, want, label):
    diff = np.abs(out.astype(np.float64) - want.astype(np.float64))
    both_nan = np.isnan(out) & np.isnan(want)
    diff[both_nan] = 0
    nbits = int(np.sum(f32bits(out) != f32bits(want)) - np.sum(both_nan & (f32bits(out) != f32bits(want))))
    say(f"{label}: max |diff| {float(np.nanmax(diff)) if diff.size else 0:.3g}, {nbits} not bitwise equal")
    assert not np.any(np.isnan(diff)) and np.all(diff <= 1e-5), label
    return nbits


@pytest.mark.parametrize("V,block,std,t", [
    (785, 256, 3.0, 9), (5000, 1024, 8.0, 7), (248320, 4096, 105.0, 32), (100000, 32768, 20.0, 3),
    (4096, 4096, 1.0, 5), (70000, 2048, 0.5, 4), (248320, 512, 105.0, 2)])
def test_random_logits_match_fixed_order_oracle(V, block, std, t):
    say(f"case logprob V={V} block={block} std={std}")
    logits, targets = synth.random_logits(V + block, t, V, std=std)
    out = gpu_logprob(logits, targets, block)
    want = oracle.block_logprob(logits, targets, block)
    assert compare(out, want, f"V={V} block={block}") == 0


def test_unaligned_rows_give_identical_bits():
    logits, targets = synth.random_logits(3, 6, 9000, std=4.0)
    say("case logprob strided rows")
    a = gpu_logprob(logits, targets, 4096)
    b = gpu_logprob(logits, targets, 4096, pad_to=9003)
    assert np.array_equal(f32bits(a), f32bits(b))


def test_closed_forms():
    V = 248320
    say("case logprob closed forms")
    uni = np.full((2, V), 0x4040, dtype=np.uint16)  # 3.0
    out = gpu_logprob(uni, [0, V - 1], 4096)
    assert np.all(out == -ln_rn32(V))
    row = np.full(V, synth.f32_to_bf16_bits(np.array([-150.0], np.float32))[0], dtype=np.uint16)
    row[4321] = synth.f32_to_bf16_bits(np.array([2.5], np.float32))[0]
    out = gpu_logprob(np.stack([row, row]), [4321, 17], 4096)
    assert out[0] == 0 and math.copysign(1.0, out[0]) < 0 and out[1] == np.float32(-152.5)
    k = 7
    tie = np.full(V, synth.f32_to_bf16_bits(np.array([-120.0], np.float32))[0], dtype=np.uint16)
    idx = np.random.default_rng(0).choice(V, size=k, replace=False)
    tie[idx] = 0x3F80
    out = gpu_logprob(tie[None], [idx[0]], 4096)
    assert out[0] == -ln_rn32(k)


def test_nan_inf_and_bad_targets():
    logits, _ = synth.random_logits(2, 5, 3000, std=2.0)
    logits[0, 13] = 0x7FC0
    logits[1, 7] = 0x7F80
    say("case logprob NaN/inf/targets")
    out = gpu_logprob(logits, [0, 0, -1, 3000, 3], 1024)
    assert np.all(np.isnan(out[:4])) and np.isfinite(out[4])


# ---------------------------------------------------------------- EXP32 / LOG32
def test_exp32_matches_correctly_rounded_oracle_on_samples():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-104, 89, 2_000_000), rng.uniform(-110, -85, 500_000),
                        rng.uniform(-1e-3, 1e-3, 100_000), rng.uniform(88.5, 89.5, 10_000)]).astype(np.float32)
    x = np.concatenate([x, np.array([0, -0.0, np.nan, np.inf, -np.inf, 1e-45, -1e-45, 88.72283, -103.97208],
                                    np.float32)])
    say("case exp32 samples")
    got = host(w8.w8i_exp32(f32(x)))
    want = oracle.exp32(x)
    same = (f32bits(got) == f32bits(want)) | (np.isnan(got) & np.isnan(want))
    assert same.all(), f"{int((~same).sum())} mismatches, e.g. x={x[~same][:5]}"


def test_log32_matches_correctly_rounded_oracle_on_samples():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.uniform(1, 2, 500_000), np.exp2(rng.uniform(-149, 128, 1_000_000)),
                        1 + np.arange(1, 20000) * 2.0 ** -23]).astype(np.float32)
    x = np.concatenate([x, np.array([1.0, 0.0, -1.0, np.inf, np.nan, 248320.0, 1e-45], np.float32)])
    say("case log32 samples")
    got = host(w8.w8i_log32(f32(x)))
    want = oracle.log32(x)
    same = (f32bits(got) == f32bits(want)) | (np.isnan(got) & np.isnan(want))
    assert same.all(), f"{int((~same).sum())} mismatches, e.g. x={x[~same][:5]}"


@pytest.mark.slow
def test_exp32_exhaustive_over_the_used_range():
    """Every binary32 x in [-104, 89]: the device EXP32 equals the correctly rounded value."""
    ranges = [(0x80000000, 0xC2D00000 - 0x80000000 + 1), (0x00000000, 0x42B20000 + 1)]  # [-104,-0], [0,89]
    chunk = 1 << 26
    total = bad = 0
    for start, count in ranges:
        for off in range(0, count, chunk):
            n = min(chunk, count - off)
            xb = (np.arange(n, dtype=np.uint64) + start + off).astype(np.uint32)
            x = xb.view(np.float32)
            got = host(w8.w8i_exp32(f32(x)))
            want = oracle.exp32_bits(start + off, n)
            bad += int(np.sum(f32bits(got) != f32bits(want)))
            total += n
    say(f"exp32 exhaustive: {total} inputs, {bad} mismatches")
    assert bad == 0


@pytest.mark.slow
def test_log32_exhaustive_over_the_fold_domain():
    """Every binary32 x in [1, 2^31] -- every value the fold's sum S can take (the row max contributes
    exactly 1, no term exceeds 1, V <= 2^31): the device LOG32 equals the oracle's, which is the
    correctly rounded ln on that domain (checked on the CPU against a decimal reference)."""
    lo, hi = 0x3F800000, 0x4F000000
    chunk = 1 << 26
    total = bad = 0
    for start in range(lo, hi + 1, chunk):
        n = min(chunk, hi + 1 - start)
        x = (np.arange(n, dtype=np.uint64) + start).astype(np.uint32).view(np.float32)
        got = host(w8.w8i_log32(f32(x)))
        want = oracle.log32_bits(start, n)
        bad += int(np.sum(f32bits(got) != f32bits(want)))
        total += n
    say(f"log32 exhaustive on [1, 2^31]: {total} inputs, {bad} mismatches")
    assert total == hi - lo + 1 and bad == 0


# ---------------------------------------------------------------- head workload
@pytest.mark.slow
def test_vocab_head_and_logprob_workload():
    """248320x5120 head at T_pad 32 on the plain layout (the persistent kernel), t = 1..32 permuted:
    logits bits are t-invariant, every logit at t = 32 and at t = 1 is within the parity bar of the
    fp64 oracle (2 ulps; the fp32 floor where the exact value has cancelled), and the block-4096 logprob of every column equals the fixed-order fp32 oracle on the
    GPU's own logits."""
    from tests.helpers import parity_bar
    d = synth.head_logprob()
    q, s, pool, targets = d["q"], d["s"], d["pool"], d["targets"]
    Wd, Sd = i8(q), f16(s)
    say(f"case head t=32 identity ({w8.w8_linear_invariant_kernel(q.shape[0], q.shape[1], 32, Sd)})")
    base_d = w8.w8_linear_invariant(Wd, Sd, bf16(pool), 32, 32)
    base = bits(base_d)
    ref, mass = oracle.w8_linear(q, s, pool, mass=True)
    ok, err, misses = parity_bar(base, ref, mass)
    say(f"head t=32, all {ok.size} outputs: {misses} beyond 2 ulps within the fp32 floor, "
        f"{int((~ok).sum())} outside the bar")
    assert ok.all()
    one = bits(w8.w8_linear_invariant(Wd, Sd, bf16(pool[:1]), 1, 32))
    ok1, err1, misses1 = parity_bar(one, ref[:1], mass[:1])
    say(f"head t=1, all {ok1.size} outputs: {misses1} beyond 2 ulps within the fp32 floor")
    assert ok1.all() and np.array_equal(one, base[:1])
    lp_base = host(w8.vocab_block_logprob(base_d, torch.from_numpy(targets).to(DEV), 4096))
    want = oracle.block_logprob(base, targets, 4096)
    assert compare(lp_base, want, "head logprob t=32") == 0
    for t in range(1, 33):
        cols = d["perms"][t]
        yd = w8.w8_linear_invariant(Wd, Sd, bf16(pool[cols]), t, 32)
        y = bits(yd)
        assert np.array_equal(y, base[cols]), f"logits changed bits at t={t}"
        lp = host(w8.vocab_block_logprob(yd, torch.from_numpy(targets[cols]).to(DEV), 4096))
        assert np.array_equal(f32bits(lp), f32bits(lp_base[cols])), f"logprob changed bits at t={t}"


def test_degenerate_and_largest_vocabularies():
    """A one-entry vocabulary, a last block of one entry, and the largest vocabulary the ABI accepts
    (V = 2^31, two rows: 8 GiB of logits, indices and row offsets past 2^31) -- against the oracle
    where it can run and otherwise against closed forms that hold bit for bit: 2^31 equal logits
    sum to exactly 2^31 in any fp32 order (every partial sum is a multiple of the block width below
    2^31), so every target's logprob is -RN32(ln 2^31); one dominant logit gives -0.0 for itself and
    the exact shift for the others.  The greedy argmax takes the lowest index among equal maxima."""
    say("case logprob V=1 and V=257 (block 256)")
    for V, block in ((1, 256), (257, 256), (4097, 4096)):
        logits, targets = synth.random_logits(V + 11, 3, V, std=5.0)
        compare(gpu_logprob(logits, targets, block), oracle.block_logprob(logits, targets, block), f"V={V}")
        got = host(w8.vocab_argmax(bf16(logits)))
        assert np.array_equal(got, oracle.argmax(logits)), f"argmax V={V}"
    V = 1 << 31
    say(f"case logprob and argmax V=2^31 (two rows, {2 * V * 2 >> 30} GiB)")
    L = torch.empty((2, V), dtype=torch.bfloat16, device=DEV)
    L[0].fill_(3.0)
    L[1].fill_(-150.0)
    L[1, V - 1] = 2.5
    tg = torch.tensor([V - 1, V - 1], dtype=torch.int64, device=DEV)
    out = host(w8.vocab_block_logprob(L, tg, 4096))
    assert out[0] == -ln_rn32(V), out[0]
    assert out[1] == 0 and math.copysign(1.0, out[1]) < 0, out[1]
    out = host(w8.vocab_block_logprob(L, torch.tensor([0, 17], dtype=torch.int64, device=DEV), 4096))
    assert out[0] == -ln_rn32(V) and out[1] == np.float32(-152.5), out
    assert list(host(w8.vocab_argmax(L))) == [0, V - 1]
    L[0, V - 1] = 4.0
    L[0, V - 2] = 4.0
    assert list(host(w8.vocab_argmax(L))) == [V - 2, V - 1]
    del L
    torch.cuda.empty_cache()
