"""The matrix-core throughput probe (measurement support for bench.py, not part of the method) runs
through the C ABI, reports the FLOP it executes and leaves finite values in its sink."""
import pytest

torch = pytest.importorskip("torch")

from block_sparse_causal_lcsa_amd import lcsa


@pytest.mark.gpu
def test_mfma_probe_runs_and_reports_its_flop():
    sink = torch.full((64 * 256,), float("nan"), dtype=torch.float32, device="cuda:0")
    flop = lcsa.lcsa_mfma_probe(64, 50, sink)
    torch.cuda.synchronize()
    assert flop == 64 * 4 * 50 * 8 * 2 * 32 * 32 * 16
    assert bool(torch.isfinite(sink).all())
