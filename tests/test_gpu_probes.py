"""The measurement references of the library on the GPU: the read probe and
the matrix-core probe run through the C ABI, leave their sinks untouched for
ordinary data and report the operation count the header states. They are not
part of the method; the benchmark times the history kernels against them."""

import pytest
import torch

from long_context_speculative_amd import ssverify as ss

pytestmark = pytest.mark.gpu


def test_read_probe_runs():
    src = torch.randn(1 << 20, dtype=torch.bfloat16, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    for wgs in (1, 7, 256, 2048):
        ss.ss_read_probe(src, wgs, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0


@pytest.mark.parametrize("n_ops, wgs", [(8192, 1), (8192 * 3 + 17, 5), (1 << 20, 512)])
def test_mfma_probe_runs(n_ops, wgs):
    ops = torch.randn(n_ops, dtype=torch.bfloat16, device="cuda")
    sink = torch.zeros(256, dtype=torch.float32, device="cuda")
    flops = ss.ss_mfma_probe(ops, 64, wgs, sink)
    torch.cuda.synchronize()
    assert flops == wgs * 4 * 64 * 8 * 16384
    assert float(sink.abs().sum()) == 0.0
