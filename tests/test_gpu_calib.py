"""The calibration kernels on the GPU (include/w8calib.h): their rates are finite and physically
plausible -- a read no faster than the 8 TB/s HBM peak, a matrix-core rate no faster than the
dense bf16 peak -- so the context bench.py prints beside the projection can be trusted."""
import math

import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from invariant_quantized_decode_amd import calib  # noqa: E402
from tests.gpu_util import say  # noqa: E402


def test_stream_read_rate_is_plausible():
    rates = calib.stream_read_gbs(33423360, workgroups=(192, 1024), replays=2)
    say(f"stream read GB/s: {rates}")
    for wg, gbs in rates.items():
        assert math.isfinite(gbs) and 500.0 < gbs < 8000.0, (wg, gbs)


def test_strip_read_rate_is_plausible():
    gbs = calib.strip_read_gbs(6144, 5120, workgroups=256, replays=2)
    say(f"strip read GB/s: {gbs:.1f}")
    assert math.isfinite(gbs) and 500.0 < gbs < 8000.0


def test_mfma_rate_is_plausible():
    tf = calib.mfma_bf16_tflops(workgroups=1024, iters=512, launches=2)
    say(f"mfma bf16 TFLOP/s: {tf:.1f}")
    assert math.isfinite(tf) and 200.0 < tf < 2600.0
