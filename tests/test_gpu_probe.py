"""The dense bf16 MFMA rate probe that bench.py reports beside the published peak:
its FLOP count follows its launch shape, and the rate it measures is positive and
no higher than the 2.5 PFLOP/s the matrix cores reach at their 2.4 GHz peak clock."""
import pytest
import torch

from test_weight_layers_amd import ttt

pytestmark = pytest.mark.gpu


def test_mfma_rate_probe_flops_and_rate():
    torch.cuda.set_device(0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 4096
    f = ttt.mfma_rate_probe(iters)
    # every compute unit: 8 waves x 8 chains x iters MFMAs of 16 x 16 x 32 multiply-adds
    assert f == cus * 8 * 8 * iters * 16 * 16 * 32 * 2
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    f = ttt.mfma_rate_probe(iters)
    e1.record()
    e1.synchronize()
    tflops = f / (e0.elapsed_time(e1) * 1e-3) / 1e12
    print(f"mfma probe: {cus} CUs, {tflops:.0f} TFLOP/s", flush=True)
    assert 100.0 < tflops < 2600.0
