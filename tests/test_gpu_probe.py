"""The matrix-core rate probe the benchmark uses as a second roofline
denominator: it runs, reports the work of its launch, and leaves its sink
alone."""
import pytest

torch = pytest.importorskip("torch")

from _util import say  # noqa: E402
from log_mel_conformer_amd import ae  # noqa: E402


@pytest.mark.gpu
def test_probe_reports_its_flops():
    say("[gpu] matrix-core rate probe")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    flops = ae.probe_mfma(10, sink)
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert flops == 4 * cus * 4 * 10 * 8 * (2 * 32 * 32 * 16)
    assert sink.item() == 0.0
    with pytest.raises(ae.AeError):
        ae.probe_mfma(0, sink)
