"""moe_layer_noalloc (the allocation-free form of moe_layer, scratch in the
library's static device buffer) against moe_layer on the same inputs: y,
indices, gates and counts equal bit for bit, over consecutive calls whose
later ones are smaller (the buffer keeps the previous call's contents), on
the streaming GEMM (decode, skewed and small batches), the bounds-checked
tiled GEMM (unaligned widths) and the fp32 path: the shapes whose scratch
fits the buffer (the 256x256-tile GEMM's split-K scratch alone takes 75 MiB,
so prefill-sized calls are refused). A call that
needs more than the buffer is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_06_amd as moe
from synth import configs
from tests.helpers import to_dev, to_host

pytestmark = pytest.mark.gpu


def _both(d):
    T, E, K = d["T"], d["E"], d["K"]
    x, wr, w1, w2 = (to_dev(d[k]) for k in ("x", "wr", "w1", "w2"))
    bias = to_dev(d["bias"]) if d["bias"] is not None else None
    outs = []
    for fn in (moe.layer, moe.layer_noalloc):
        idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
        gate = torch.empty((T, K), dtype=torch.float32, device="cuda")
        counts = torch.empty((E,), dtype=torch.int32, device="cuda")
        y = fn(x, wr, w1, w2, K, bias=bias, topk_idx=idx, topk_gate=gate, counts=counts)
        torch.cuda.synchronize()
        outs.append([to_host(t) for t in (y, idx, gate, counts)])
    return outs


@pytest.mark.parametrize("calls", [
    [dict(name="decode", T=256), dict(name="decode", T=16)],
    [dict(name="skewed", T=300), dict(name="prefill", T=100, H=1024, F=2048)],
    [dict(name="tiny", T=300, H=1000, E=16, K=4, F=1500, dtype="bf16", wid=70), dict(name="tiny", T=64)],
], ids=["decode", "skewed_then_prefill_small", "unaligned_then_tiny_f32"])
def test_noalloc_equals_layer_on_consecutive_calls(calls):
    for kw in calls:
        d = configs.layer_inputs(**kw)
        need = moe.layer_workspace_size(d["T"], d["H"], d["E"], d["K"], d["F"], moe.F32 if d["dtype"] == "f32"
                                        else moe.BF16)
        assert need <= moe.NOALLOC_SCRATCH_BYTES
        print(f"{kw}: scratch {need / 2**20:.2f} MiB", flush=True)
        (y0, i0, g0, c0), (y1, i1, g1, c1) = _both(d)
        assert np.array_equal(y0.view(np.uint8), y1.view(np.uint8))
        assert np.array_equal(i0, i1) and np.array_equal(c0, c1)
        assert np.array_equal(g0.view(np.uint32), g1.view(np.uint32))


def test_noalloc_refuses_calls_beyond_the_buffer():
    d = configs.layer_inputs("decode", T=16)
    x, wr, w1, w2 = (to_dev(d[k]) for k in ("x", "wr", "w1", "w2"))
    big = torch.empty((1024, d["H"]), dtype=torch.bfloat16, device="cuda")
    y = torch.full((1024, d["H"]), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.layer_noalloc(big, wr, w1, w2, d["K"], y=y)
    assert ei.value.status == moe.ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())  # nothing was enqueued
