"""The library's reduction orders are the documented ones, on inputs where another order changes the bits.

Random inputs cannot show an fp64 accumulation order (another K plan changes no bf16 output of 200k
random ones), so the projection runs on synth.order_sensitive_linear: every group sum and scaled term
is exact there, the fp64 additions are the only roundings, and most outputs change with their order.
The t = T_pad call must give, bit for bit, the header's schedule written out in numpy
(tests/order_model.py, itself pinned to the oracle), and every column computed at t < T_pad its
t = T_pad bits: the K-slice kernels of small N and the one-launch split kernel at T_pad 32 and 64 (an
odd group count, so the last slice takes the extra group; at t <= 32 the K-slice kernels or the
one-tile kernel serve the T_pad-64 call), the split kernel at 6144 rows and the persistent kernel, both
weight layouts, with and without the workspace.  The logprob's left fold of block partials and its
pairwise in-block tree are checked on rows where one fp32 rounding tells them from the nearest
alternative orders.
"""
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import invariant_quantized_decode_amd as w8  # noqa: E402
from tests import order_checks  # noqa: E402
from tests.gpu_util import say  # noqa: E402

PROBLEMS = [  # seed, N, K, T_pad, rows modelled, one-launch kernel family
    (11, 512, 5120, 32, 512, "gemm_w8g32_split"),
    (12, 517, 5152, 64, 517, "gemm_w8g32_split"),
    (13, 131172, 1024, 32, 4096, "gemm_w8g32_tiles"),
    (14, 6144, 5120, 32, 1024, "gemm_w8g32_split"),
]


@pytest.mark.parametrize("seed,N,K,T_pad,rows,family", PROBLEMS)
def test_projection_follows_the_documented_schedule(seed, N, K, T_pad, rows, family):
    say(f"case schedule N={N} K={K} T_pad={T_pad}")
    assert w8.w8_linear_invariant_packed_kernel(N, K, T_pad).startswith(family)
    problem = order_checks.OrderSensitiveProjection(seed, N, K, T_pad, rows)
    fails = order_checks.check_projection(problem)
    assert not fails, "\n".join(fails)


def test_logprob_block_partials_fold_left_to_right():
    say("case logprob fold order row")
    fails = order_checks.check_logprob_fold_order()
    assert not fails, fails


def test_logprob_in_block_tree_is_pairwise_in_index_order():
    say("case logprob in-block tree row")
    fails = order_checks.check_logprob_in_block_tree()
    assert not fails, fails
