"""The dense-MFMA measurement probe runs and reports the FLOP of its launch."""
import pytest
import torch

import block_sparse_attention_svg_amd as svg
from parity_utils import banner

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fp8", [False, True])
def test_mfma_peak_probe_runs(fp8):
    banner("mfma probe", "fp8" if fp8 else "bf16")
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.full((n_cu * 512,), float("nan"), dtype=torch.float32, device="cuda")
    flop = svg.svg_mfma_peak_probe(fp8, 3, sink)
    torch.cuda.synchronize()
    assert flop == n_cu * 8 * 3 * 16 * 2 * 32 * 32 * (64 if fp8 else 16)
    assert torch.isfinite(sink).all()          # every thread stored its sum
    with pytest.raises(svg.SvgError):
        svg.svg_mfma_peak_probe(fp8, 3, sink[: n_cu * 512 - 1])
