"""GPU mutant tier: the GPU checks catch plausible mistakes in the library's reduction orders.

tests/gpu_mutants.py builds seven copies of the library, each with one mistake planted in one
translation unit (built beside the product by __graft_entry__.build()).  The same process loads each
copy in turn in place of the product library and runs the order checks of tests/order_checks.py: the
product must pass them all, and each mutant must fail at least the checks named for it below.  The
checks are the ones the product's own GPU tests run (tests/test_gpu_schedule.py and the oracle
comparisons of tests/test_gpu_logprob.py), so a mutant that passed here would pass those too.

  k_plan_from_t               8 equal K slices when t > 16 (the split and persistent kernels)
  slice_fold_reversed_from_t  the split kernel folds its slice sums from the last when t > 16
  kslice_fold_reversed_from_t the small-N fold launch folds the slice sums from the last when t > 16
  block_fold_regrouped        the logprob fold adds four partials together before the running sum
  block_local_max             each block's exps are shifted by the block's own maximum
  in_block_tree_strided       the in-wave tree pairs lanes 32 apart first
  max_epilogue_counts_padding_rows  the fused head's row maxima count the last strip's rows past V

Every mutation keeps the memory accesses and loop bounds of the code it replaces.
"""
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from tests import gpu_mutants, order_checks  # noqa: E402
from tests.gpu_util import say  # noqa: E402

EXPECTED = {
    "k_plan_from_t": {"512 rows", "131172 rows"},
    "slice_fold_reversed_from_t": {"512 rows"},
    "kslice_fold_reversed_from_t": {"512 rows"},
    "block_fold_regrouped": {"fold order"},
    "block_local_max": {"random logits"},
    "in_block_tree_strided": {"in-block tree"},
    "max_epilogue_counts_padding_rows": {"fused maxima"},
}


@pytest.fixture(scope="module")
def problems():
    say("mutant tier: building the order-sensitive problems")
    # 512 rows: the K-slice kernels (with the queried workspace) and the split kernel (without);
    # 131172 rows: the persistent kernel
    return (order_checks.OrderSensitiveProjection(21, 512, 5120, 32, 512),
            order_checks.OrderSensitiveProjection(22, 131172, 1024, 32, 2048))


def run_checks(problems) -> dict:
    split, persistent = problems
    return {
        "512 rows": order_checks.check_projection(split),
        "131172 rows": order_checks.check_projection(persistent),
        "random logits": order_checks.check_logprob_random(),
        "fold order": order_checks.check_logprob_fold_order(),
        "in-block tree": order_checks.check_logprob_in_block_tree(),
        "fused maxima": order_checks.check_fused_maxima(),
    }


def test_mutant_table_covers_every_mutant():
    assert set(EXPECTED) == set(gpu_mutants.MUTANTS)


def test_product_library_passes_every_check(problems):
    say("mutant tier: product library")
    results = run_checks(problems)
    assert not any(results.values()), results


@pytest.mark.parametrize("name", sorted(gpu_mutants.MUTANTS))
def test_mutant_is_caught(name, problems):
    path = gpu_mutants.lib_path(name)
    if not os.path.exists(path):
        pytest.skip(f"{path} is not built (__graft_entry__.build() builds it)")
    say(f"mutant tier: {name}")
    with gpu_mutants.library(path):
        results = run_checks(problems)
    caught = {check for check, fails in results.items() if fails}
    for check in sorted(caught):
        say(f"  {check}: {results[check][0]}")
    assert EXPECTED[name] <= caught, f"{name} escaped {sorted(EXPECTED[name] - caught)}"
