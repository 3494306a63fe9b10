"""The entry point that allocates nothing, vocab_block_logprob_noalloc, on the GPU through the C ABI.

It runs the kernels of vocab_block_logprob with the block maxima and partials in the library's fixed
device scratch instead of a caller's workspace, so for the same inputs it must give the same bits.
Two calls in a row, the second with a smaller input (fewer columns, a shorter vocabulary, another
block width), each checked bit for bit against vocab_block_logprob with a workspace and within 1e-5
of the fixed-order fp32 oracle; then a call that does not fit the scratch is refused and writes
nothing.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import invariant_quantized_decode_amd as w8  # noqa: E402
from tests.gpu_util import DEV, bf16, host, say  # noqa: E402

L = w8.lib()


def noalloc(logits, targets, block, out, t):
    """vocab_block_logprob_noalloc called directly through the C ABI (ctypes), on torch's current stream."""
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    V = logits.size(1)
    return L.vocab_block_logprob_noalloc(ctypes.c_void_p(logits.data_ptr()), ctypes.c_void_p(targets.data_ptr()),
                                         block, ctypes.c_void_p(out.data_ptr()), t, V, logits.stride(0), stream)


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    for t, V, block, std, seed in ((32, 248320, 4096, 105.0, 11), (5, 70001, 1024, 6.0, 12)):
        say(f"case noalloc logprob t={t} V={V} block={block}")
        logits, targets = synth.random_logits(seed, t, V, std=std)
        Ld = bf16(logits)
        Td = torch.from_numpy(targets).to(DEV)
        ws_out = w8.vocab_block_logprob(Ld, Td, block)
        out = torch.full((t,), float("nan"), dtype=torch.float32, device=DEV)
        assert noalloc(Ld, Td, block, out, t) == 0
        got, want = host(out), host(ws_out)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"t={t} V={V}: bits differ"
        ref = oracle.block_logprob(logits, targets, block)
        assert np.all(np.abs(got.astype(np.float64) - ref) <= 1e-5), f"t={t} V={V}: beyond 1e-5 of the oracle"


def test_noalloc_refuses_what_does_not_fit_and_writes_nothing():
    t, V, block = 64, 1 << 22, 256  # block maxima and partials: 2 x 4 MiB > 1 MiB
    say(f"case noalloc refusal t={t} V={V} block={block}")
    Ld = torch.zeros((t, V), dtype=torch.bfloat16, device=DEV)
    Td = torch.zeros(t, dtype=torch.int64, device=DEV)
    out = torch.full((t,), -3.0, dtype=torch.float32, device=DEV)
    assert noalloc(Ld, Td, block, out, t) == -8
    torch.cuda.synchronize()
    assert bool((out == -3.0).all())
    del Ld
    torch.cuda.empty_cache()
