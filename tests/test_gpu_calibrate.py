"""The MFMA-only calibration call that the benchmark prices the fused kernel against: it
runs on every CU, reports the flop count of its launch, rejects a sink that is too small,
and its sustained rate lies between a quarter of the published dense bf16 peak and the
peak itself (the kernel issues nothing but MFMAs; the power limit lowers the clock)."""
import pytest
import torch

import ff_input_projection_amd as fpa

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def test_mfma_ceiling_rate_and_flop_count():
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    sink = torch.full((cus * 256,), float("nan"), dtype=torch.float32, device=DEV)
    stream = torch.cuda.current_stream(DEV)
    iters = 500
    flops = fpa.mfma_ceiling_launch(iters, sink, stream)
    assert flops == cus * 4 * iters * 16 * 32768
    for i in range(20):   # warm the clocks
        fpa.mfma_ceiling_launch(iters, sink, stream, seed=i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(10):
        fpa.mfma_ceiling_launch(iters, sink, stream, seed=100 + i)
    e1.record(stream)
    torch.cuda.synchronize()
    tflops = flops * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    print(f"[calibrate] sustained bf16 MFMA rate {tflops:.0f} TFLOP/s on {cus} CUs", flush=True)
    assert 625.0 < tflops < 2600.0, tflops
    # every thread wrote its accumulators' sum (finite: operands in [-1, 1))
    assert torch.isfinite(sink).all()


def test_mfma_ceiling_rejects_a_small_sink():
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    sink = torch.empty(cus * 256 - 1, dtype=torch.float32, device=DEV)
    with pytest.raises(fpa.FusedProjError) as e:
        fpa.mfma_ceiling_launch(10, sink)
    assert e.value.code == fpa.EINVAL
