"""The MFMA-rate measurement behind bench.py --mfma-ceiling runs and gives
plausible rates (GPU)."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

pytestmark = pytest.mark.gpu


def test_mfma_ceiling_runs():
    out = bench.mfma_ceiling(0.2)
    for kind in ("constant", "random"):
        r = out[kind]
        assert r["launches"] >= 4
        # a dense bf16 rate between a tenth of the peak and the peak (with
        # timing slack)
        assert 0.1 * bench.PEAK_BF16_TFLOPS < r["tflops"] < 1.05 * bench.PEAK_BF16_TFLOPS, r
