"""The LM head fused with the blockwise logprob's row maximum, on the GPU through the C ABI.

tokenspeed numerics ("Logprobs", block_sumexp leaf contract) fixes the logprob's arithmetic: the row
maximum first, then block partials of exps shifted by it, folded left to right.  The fused call moves
only the first pass into the head projection (per-workgroup column maxima written with the logits; a maximum
is exact in any order), so both of its results must equal the unfused calls bit for bit:

  logits == w8_linear_invariant(W, S, x)           out == vocab_block_logprob(logits, targets, block)
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import invariant_quantized_decode_amd as w8  # noqa: E402
from tests.gpu_util import DEV, bf16, bits, f16, host, i8, say  # noqa: E402


def f32bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def run_both(Wd, Sd, Pk, Xd, Td, t, T_pad, block, V):
    """(unfused logits, unfused logprob) and the fused calls' results on both layouts."""
    ref_l = w8.w8_linear_invariant(Wd, Sd, Xd[:t], t, T_pad)
    ref_o = w8.vocab_block_logprob(ref_l, Td[:t].contiguous(), block)
    fl, fo = w8.w8_head_logprob_invariant(Wd, Sd, Xd[:t], Td[:t].contiguous(), t, T_pad, block)
    pl, po = w8.w8_head_logprob_invariant_packed(Pk[0], Pk[1], Xd[:t], Td[:t].contiguous(), t, T_pad, block, V)
    return bits(ref_l), host(ref_o), (bits(fl), host(fo)), (bits(pl), host(po))


CASES = [  # V, K, T_pad, block, t values: the head, ragged vocabularies on the same kernel, T_pad 16 / 64
    (248320, 5120, 32, 4096, (1, 7, 32)),
    (70001, 1056, 32, 256, (1, 32)),
    (40000, 2048, 16, 32768, (3, 16)),
    (131172, 5088, 64, 4096, (1, 32)),
]


@pytest.mark.parametrize("V,K,T_pad,block,ts", CASES)
def test_fused_head_logprob_gives_the_unfused_bits(V, K, T_pad, block, ts):
    rng = np.random.default_rng(V + K + block)
    q = synth.draw_codes(rng, V, K)
    s = synth.draw_scales(rng, V, K, 0.0)
    x = synth.draw_acts(rng, T_pad, K)
    targets = rng.integers(0, V, size=T_pad, dtype=np.int64)
    Wd, Sd, Xd, Td = i8(q), f16(s), bf16(x), torch.from_numpy(targets).to(DEV)
    Pk = w8.w8_pack(Wd, Sd)
    for t in ts:
        say(f"case fused head V={V} K={K} T_pad={T_pad} block={block} t={t}")
        ref_l, ref_o, plain, packed = run_both(Wd, Sd, Pk, Xd, Td, t, T_pad, block, V)
        for name, (lg, o) in (("plain", plain), ("packed", packed)):
            assert np.array_equal(lg, ref_l), f"{name} t={t}: logits differ"
            assert np.array_equal(f32bits(o), f32bits(ref_o)), f"{name} t={t}: logprob differs"
    want = oracle.block_logprob(ref_l, targets[:t], block)
    assert np.all(np.abs(ref_o.astype(np.float64) - want) <= 1e-5)


def test_fused_head_nan_inf_and_bad_targets():
    """A NaN activation column makes its logits NaN (the fused maxima say NaN too), a column of large
    activations overflows logits to +-inf, and targets outside [0, V) give NaN -- as unfused."""
    V, K, T_pad = 131072 + 96, 1024, 32
    rng = np.random.default_rng(9)
    q = synth.draw_codes(rng, V, K)
    s = synth.draw_scales(rng, V, K, 0.0)
    x = synth.draw_acts(rng, 6, K)
    x[1, 17] = 0x7FC0                                      # NaN
    x[2, :] = synth.f32_to_bf16_bits(np.full(K, 3e38, np.float32))  # overflows to inf
    targets = np.array([0, 5, 7, -1, V, V - 1], dtype=np.int64)
    Wd, Sd, Xd, Td = i8(q), f16(s), bf16(x), torch.from_numpy(targets).to(DEV)
    say("case fused head NaN / inf / bad targets")
    ref_l, ref_o, plain, packed = run_both(Wd, Sd, w8.w8_pack(Wd, Sd), Xd, Td, 6, T_pad, 4096, V)
    for lg, o in (plain, packed):
        assert np.array_equal(lg, ref_l)
        same = (f32bits(o) == f32bits(ref_o)) | (np.isnan(o) & np.isnan(ref_o))
        assert same.all()
    assert np.isnan(ref_o[[1, 2, 3, 4]]).all() and np.isfinite(ref_o[[0, 5]]).all()


def test_fused_head_refuses_two_tiles_and_small_workspace():
    V, K = 1024, 256
    rng = np.random.default_rng(3)
    Wd, Sd = i8(synth.draw_codes(rng, V, K)), f16(synth.draw_scales(rng, V, K, 0.0))
    Xd = bf16(synth.draw_acts(rng, 40, K))
    Td = torch.zeros(40, dtype=torch.int64, device=DEV)
    say("case fused head refusals")
    with pytest.raises(ValueError):
        w8.w8_head_logprob_invariant(Wd, Sd, Xd, Td, 40, 64, 4096)   # t > 32: two-tile width
    with pytest.raises(ValueError):
        w8.w8_head_logprob_invariant(Wd, Sd, Xd[:4], Td, 4, 32, 4096,
                                     workspace=torch.empty(64, dtype=torch.uint8, device=DEV))
    assert math.isfinite(float(host(w8.w8_head_logprob_invariant(Wd, Sd, Xd[:4], Td, 4, 64, 4096)[1])[0]))


@pytest.mark.parametrize("V,K", [(131149, 1024), (70001, 2048)])
def test_fused_head_maxima_skip_rows_past_the_vocabulary(V, K):
    """Every logit below -104 (positive codes and scales, negative activations), V not a multiple of
    the 32-row strip: the rows past V that the last strip computes (zeros) must not enter the fused
    row maxima -- if they did, the row maximum would be 0, every exp would underflow and every
    logprob would differ from the unfused call's."""
    rng = np.random.default_rng(V + 7)
    q = rng.integers(1, 128, size=(V, K), dtype=np.int8)
    s = synth.draw_scales(rng, V, K, 0.08)
    x = synth.draw_acts(rng, 32, K)
    x = x | np.uint16(0x8000)                       # every activation negative (or -0)
    targets = rng.integers(0, V, size=32, dtype=np.int64)
    Wd, Sd, Xd, Td = i8(q), f16(s), bf16(x), torch.from_numpy(targets).to(DEV)
    Pk = w8.w8_pack(Wd, Sd)
    for t in (1, 32):
        say(f"case fused head negative logits V={V} K={K} t={t}")
        ref_l, ref_o, plain, packed = run_both(Wd, Sd, Pk, Xd, Td, t, 32, 4096, V)
        assert np.all((ref_l & 0x8000) != 0) and np.all((ref_l & 0x7FFF) > 0x42D0), "every logit below -104"
        for name, (lg, o) in (("plain", plain), ("packed", packed)):
            assert np.array_equal(lg, ref_l), f"{name} t={t}: logits differ"
            assert np.array_equal(f32bits(o), f32bits(ref_o)), f"{name} t={t}: logprob differs"
