"""The library's peak kernels on the device (needs an MI355X): the measured
achievable rates are positive and below the part's published peaks (8 TB/s
HBM, 2.5 PFLOP/s dense bf16), and a copy really copies."""
from __future__ import annotations

import pytest
import torch

from recurrent_decode_step_amd import binding

pytestmark = pytest.mark.gpu


def test_peak_bandwidth_is_plausible_and_copy_copies():
    n = 256 << 20
    src = torch.arange(n // 4, dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    read = binding.peak_bandwidth(src, dst, copy=False, reps=3)
    copy = binding.peak_bandwidth(src, dst, copy=True, reps=3)
    torch.cuda.synchronize()
    print(f"read {read:.0f} GB/s, copy {copy:.0f} GB/s", flush=True)
    assert 500.0 < read < 8200.0
    assert 500.0 < copy < 8200.0
    assert torch.equal(dst, src)


@pytest.mark.parametrize("shape", [0, 1])
def test_peak_mfma_is_plausible(shape):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(2 * cus * 256, dtype=torch.float32, device="cuda")
    tf = binding.peak_mfma(shape, 1024, sink, reps=3)
    torch.cuda.synchronize()
    print(f"shape {shape}: {tf:.0f} TFLOP/s", flush=True)
    assert 50.0 < tf < 2600.0
    assert torch.isfinite(sink).all() and bool((sink != 0).any())
