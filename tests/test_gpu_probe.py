"""The read-rate probe (moe_fetch_probe) runs on every compute unit and
reports plausible rates: positive cycle counts on every CU, and a rate below
what one CU's 64-byte-per-clock request path could move."""
import pytest
import torch

import mixture_experts_layer_06_amd as moe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", [0, 1], ids=["lds_dma", "vector"])
@pytest.mark.parametrize("shared,nbytes", [(True, 2 << 20), (False, 256 << 20)], ids=["l2", "hbm"])
def test_fetch_probe_runs_on_every_cu(mode, shared, nbytes):
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    cycles, per_cu = moe.fetch_probe(buf, mode, shared, 64)
    torch.cuda.synchronize()
    c = cycles.cpu()
    assert c.numel() == torch.cuda.get_device_properties(0).multi_processor_count
    assert (c > 0).all()
    rate = per_cu / c.double()
    assert (rate > 0.5).all() and (rate < 64.0).all(), (rate.min().item(), rate.max().item())
