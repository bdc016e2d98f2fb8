"""The matrix-core calibration stream on the GPU: both operand kinds run
through the C ABI and report a rate between zero and the bf16 peak (2.5
PFLOP/s, with 5% allowance for the clock the events see)."""

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("operands", ["random", "constant"])
def test_mfma_calibration_reports_a_rate_below_peak(operands):
    from coalesced_attention_amd import zl
    tflops = zl.calibrate_mfma(operands, iters=20_000)
    assert 50.0 < tflops <= 2500.0 * 1.05, tflops
