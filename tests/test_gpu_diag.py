"""GPU check of the diagnostic fp32 matrix-core issue loop (convfuse_measure_mfma), whose
rate bench.py --ceilings reports as the practical MFMA ceiling: every MFMA of the loop ran
(its accumulators end at an exact value)."""
import pytest

from test_gpu_parity import _torch, cf

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("iters,workgroups", [(1, 1), (37, 3), (2048, 64)])
def test_mfma_loop_exact(iters, workgroups):
    torch = _torch()
    out = torch.full((1,), -1.0, device="cuda")
    cf().measure_mfma(iters, workgroups, out)
    assert out.item() == iters * 2.0 ** -14
