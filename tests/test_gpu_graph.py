"""Every kind of call on the decode path captured in one HIP graph replays to its eager bits.

Projections (plain and packed, with the residual-add and SwiGLU epilogues), the column-local glue
and the vocabulary epilogues (block logprob, its blockwise-direct form, greedy argmax) are first run
eagerly, then captured together with preallocated outputs and workspaces.  The graph is replayed
several times; before each replay the outputs are overwritten, unrelated eager work runs and the
device is synchronised, and after it every output must equal the eager one bit for bit.  (The
library records no memset and allocates nothing, so a captured call is exactly its kernels.)
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import invariant_quantized_decode_amd as w8  # noqa: E402
from tests.gpu_util import DEV, bf16, f16, i8, say  # noqa: E402


def test_one_graph_of_every_call_replays_to_the_eager_bits():
    rng = np.random.default_rng(31)
    t, T_pad, N, F, K, V = 9, 32, 600, 200, 1024, 70000
    Wd, Sd = i8(synth.draw_codes(rng, N, K)), f16(synth.draw_scales(rng, N, K, 0.0))
    Gd, Gs = i8(synth.draw_codes(rng, 2 * F, K)), f16(synth.draw_scales(rng, 2 * F, K, 0.0))
    Xd = bf16(synth.draw_acts(rng, t, K))
    Rd = bf16(synth.draw_acts(rng, t, N))
    Hd = bf16(synth.draw_acts(rng, t, 2 * F))
    wn = bf16(synth.draw_acts(rng, 1, K))[0].contiguous()
    logits, targets = synth.random_logits(5, t, V, std=6.0)
    Ld, Td = bf16(logits), torch.from_numpy(targets).to(DEV)
    Wp, Sp = w8.w8_pack(Wd, Sd)
    Gp, Gq = w8.w8_pack(Gd, Gs)

    outs = {
        "linear": torch.empty((t, N), dtype=torch.bfloat16, device=DEV),
        "packed": torch.empty((t, N), dtype=torch.bfloat16, device=DEV),
        "add": torch.empty((t, N), dtype=torch.bfloat16, device=DEV),
        "add_packed": torch.empty((t, N), dtype=torch.bfloat16, device=DEV),
        "swiglu_packed": torch.empty((t, F), dtype=torch.bfloat16, device=DEV),
        "rmsnorm": torch.empty((t, K), dtype=torch.bfloat16, device=DEV),
        "swiglu": torch.empty((t, F), dtype=torch.bfloat16, device=DEV),
        "residual_add": torch.empty((t, N), dtype=torch.bfloat16, device=DEV),
        "logprob": torch.empty(t, dtype=torch.float32, device=DEV),
        "direct": torch.empty(t, dtype=torch.float32, device=DEV),
        "argmax": torch.empty(t, dtype=torch.int64, device=DEV),
    }
    ws_lp = torch.empty(max(16, w8.vocab_block_logprob_workspace_bytes(t, V, 4096)), dtype=torch.uint8, device=DEV)
    ws_lpd = torch.empty_like(ws_lp)
    ws_am = torch.empty(max(16, w8.vocab_argmax_workspace_bytes(t, V)), dtype=torch.uint8, device=DEV)

    def run():
        w8.w8_linear_invariant(Wd, Sd, Xd, t, T_pad, y=outs["linear"])
        w8.w8_linear_invariant_packed(Wp, Sp, Xd, t, T_pad, N, y=outs["packed"])
        w8.w8_linear_add_invariant(Wd, Sd, Xd, Rd, t, T_pad, y=outs["add"])
        w8.w8_linear_add_invariant_packed(Wp, Sp, Xd, Rd, t, T_pad, N, y=outs["add_packed"])
        w8.w8_linear_swiglu_invariant_packed(Gp, Gq, Xd, t, T_pad, F, y=outs["swiglu_packed"])
        w8.w8i_rmsnorm(Xd, 1e-6, wn, y=outs["rmsnorm"])
        w8.w8i_swiglu(Hd, y=outs["swiglu"])
        w8.w8i_residual_add(outs["linear"], Rd, y=outs["residual_add"])
        w8.vocab_block_logprob(Ld, Td, 4096, out=outs["logprob"], workspace=ws_lp)
        w8.vocab_block_logprob_direct(Ld, Td, 4096, out=outs["direct"], workspace=ws_lpd)
        w8.vocab_argmax(Ld, out=outs["argmax"], workspace=ws_am)

    def snapshot():
        return {k: v.view(torch.int16 if v.dtype == torch.bfloat16 else
                          torch.int32 if v.dtype == torch.float32 else torch.int64).cpu().numpy().copy()
                for k, v in outs.items()}

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        run()
    torch.cuda.synchronize()
    want = snapshot()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            run()
    other = torch.empty((t, N), dtype=torch.bfloat16, device=DEV)
    for rep in range(4):
        for v in outs.values():
            v.fill_(-1)
        w8.w8_linear_invariant(Wd, Sd, Xd[:1], 1, T_pad, y=other)  # eager work between replays
        w8.vocab_argmax(Ld[:2])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for k in want:
            assert np.array_equal(got[k], want[k]), f"replay {rep}: {k} differs from the eager call"
        say(f"graph replay {rep}: all {len(want)} outputs equal the eager bits")
