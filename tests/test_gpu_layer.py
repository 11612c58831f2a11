"""End-to-end moe_layer parity against the fp64 oracle at reduced sizes that
keep every path (route, both permute paths, tiled / streaming / fp32 GEMM,
combine) in play, plus invariants: identity experts, determinism, forced
empty experts. Every token is checked: where the oracle's k-th and (k+1)-th
scores are more than 1e-3 apart the GPU's experts must be the oracle's; where
they nearly tie, the GPU's experts must be a valid top-k within 1e-3 and the
gates and y are compared with the oracle evaluated on the GPU's own
selection. On integer-valued inputs the indices are bit-exact, ties included."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_06_amd as moe
import oracle
import synth
from synth import configs
from tests.helpers import TOL, layer_check, normwise_err, to_dev, to_host

pytestmark = pytest.mark.gpu


def run_layer(d):
    T, E, K = d["T"], d["E"], d["K"]
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, K), dtype=torch.float32, device="cuda")
    counts = torch.empty((E,), dtype=torch.int32, device="cuda")
    bias = to_dev(d["bias"]) if d["bias"] is not None else None
    y = moe.layer(to_dev(d["x"]), to_dev(d["wr"]), to_dev(d["w1"]), to_dev(d["w2"]), K, bias=bias,
                  topk_idx=idx, topk_gate=gate, counts=counts)
    torch.cuda.synchronize()
    return to_host(y), to_host(idx), to_host(gate), to_host(counts)


LAYER_CASES = [
    # (name, kwargs for configs.layer_inputs)
    ("tiny_f32", dict(name="tiny")),
    ("tiny_bf16", dict(name="tiny", dtype="bf16")),
    ("mid_bf16", dict(name="tiny", T=512, H=256, E=16, K=4, F=384, dtype="bf16", wid=60)),
    ("skewed_small", dict(name="skewed", T=256)),
    ("decode_t16", dict(name="decode", T=16, H=1024, F=512, wid=61)),
    ("prefill_small", dict(name="prefill", T=128, H=512, F=1024, wid=62)),
    # more than 4096 pairs and at most 16 experts: the router's per-block
    # counts feed a one-launch dispatch (ragged last block, chunks of 21 or
    # 64 blocks, K = E)
    ("counted_e8_k3", dict(name="tiny", T=4100, H=256, E=8, K=3, F=256, dtype="bf16", wid=63)),
    ("counted_e16_k1_bias", dict(name="tiny", T=5000, H=128, E=16, K=1, F=128, dtype="bf16", bias=True,
                                 wid=64)),
    ("counted_e4_k4", dict(name="tiny", T=4097, H=64, E=4, K=4, F=128, dtype="bf16", wid=65)),
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_layer_parity(case):
    name, kw = case
    d = configs.layer_inputs(**kw)
    y, idx, gate, counts = run_layer(d)
    ref = oracle.layer(d["x"], d["wr"], d["w1"], d["w2"], d["K"], bias=d["bias"], nthreads=8)
    tol = TOL[d["dtype"]]
    err, n_alt = layer_check(y, idx, gate, d, ref, tol=tol, gate_tol=1e-5 if d["dtype"] == "f32" else 2e-3)
    assert counts.sum() == d["T"] * d["K"]
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=d["E"]))
    if n_alt == 0:
        assert np.array_equal(counts, ref["counts"])


def test_layer_integer_variant_exact_routing():
    d = configs.layer_inputs("tiny", integer=True)
    y, idx, gate, counts = run_layer(d)
    ref = oracle.layer(d["x"], d["wr"], d["w1"], d["w2"], d["K"])
    assert np.array_equal(idx, ref["idx"])
    assert np.array_equal(counts, ref["counts"])
    assert normwise_err(y, ref["y"]) <= TOL["f32"]


def test_layer_dense_masked_sum_agrees():
    d = configs.layer_inputs("tiny")
    y, idx, gate, _ = run_layer(d)
    dense = oracle.layer_dense(d["x"], d["wr"], d["w1"], d["w2"], d["K"])
    ref = oracle.layer(d["x"], d["wr"], d["w1"], d["w2"], d["K"])
    assert normwise_err(dense, ref["y"]) <= 1e-12
    layer_check(y, idx, gate, d, dict(ref, y=dense), tol=TOL["f32"], gate_tol=1e-5)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_layer_identity_experts_return_x(dt):
    d = configs.layer_inputs("tiny", dtype=dt)
    d["w1"], d["w2"] = configs.identity_ffn(d["H"], d["E"], dt)
    d["F"] = 2 * d["H"]
    y, _, _, _ = run_layer(d)
    x = d["x"].astype(np.float64) if dt == "f32" else to_host(to_dev(d["x"]).float()).astype(np.float64)
    tol = 1e-6 if dt == "f32" else 2 ** -8
    assert normwise_err(y, x) <= tol


def test_layer_forced_empty_experts():
    d = configs.layer_inputs("tiny", dtype="bf16")
    b = np.zeros(d["E"], np.float32)
    b[5:] = -1e4
    d["bias"] = b
    y, idx, gate, counts = run_layer(d)
    assert counts[5:].sum() == 0
    ref = oracle.layer(d["x"], d["wr"], d["w1"], d["w2"], d["K"], bias=b)
    layer_check(y, idx, gate, d, ref, tol=TOL["bf16"])


def test_layer_deterministic():
    d = configs.layer_inputs("skewed", T=300)
    y1 = run_layer(d)[0]
    y2 = run_layer(d)[0]
    assert np.array_equal(y1, y2)


# ---------------------------------------------------------------- E4M3 layer

def _run_layer_fp8(d):
    T, E, K = d["T"], d["E"], d["K"]
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, K), dtype=torch.float32, device="cuda")
    counts = torch.empty((E,), dtype=torch.int32, device="cuda")
    sc = lambda v: torch.tensor([float(v)], dtype=torch.float32, device="cuda")
    y = moe.layer_fp8(to_dev(d["x"]), to_dev(d["wr"]), to_dev(d["w1"]), sc(d["w1_scale"]), to_dev(d["w2"]),
                      sc(d["w2_scale"]), K, bias=None if d["bias"] is None else to_dev(d["bias"]),
                      topk_idx=idx, topk_gate=gate, counts=counts)
    torch.cuda.synchronize()
    return to_host(y), to_host(idx), to_host(gate), to_host(counts)


@pytest.mark.parametrize("name,shape", [("tiny", dict(T=64)), ("prefill", dict(T=300, H=512, F=1024)),
                                        ("skewed", dict(T=400, H=256, F=384)),
                                        ("decode", dict(T=16, H=512, F=256))])
def test_layer_fp8_parity(name, shape):
    """E4M3 experts with per-token dynamic quantisation: routing checked on
    every token, y against the oracle's E4M3 layer (fp64 hidden rows) within
    the fp8 bar, against the unquantised layer on the same weights within the
    fp8 bar, and, as a tighter diagnostic, within 2e-2 of the oracle with its
    hidden rows rounded to bf16 before quantisation (the layer stores them in
    bf16; that one rounding moves about a thirtieth of the hidden codes by one
    E4M3 step, which alone accounts for up to 2.1e-2 between the two oracles
    on these shapes)."""
    d = configs.layer_fp8_inputs(name, **shape)
    y, idx, gate, counts = _run_layer_fp8(d)
    ref = oracle.layer_fp8(d["x"], d["wr"], d["w1"], d["w1_scale"], d["w2"], d["w2_scale"], d["K"],
                           bias=d["bias"], nthreads=8)
    err, _ = layer_check(y, idx, gate, d, ref, tol=TOL["fp8"], fp8=True)
    mirror = oracle.layer_fp8(d["x"], d["wr"], d["w1"], d["w1_scale"], d["w2"], d["w2_scale"], d["K"],
                              bias=d["bias"], hidden="bf16", nthreads=8)
    err_m, _ = layer_check(y, idx, gate, d, mirror, tol=2e-2, fp8=True, fp8_hidden="bf16")
    w1f = (oracle.decode(d["w1"]) * float(d["w1_scale"])).astype(np.float32)
    w2f = (oracle.decode(d["w2"]) * float(d["w2_scale"])).astype(np.float32)
    dp = dict(d, x=synth.bf16_to_f32(d["x"]), wr=synth.bf16_to_f32(d["wr"]), w1=w1f, w2=w2f)
    plain = oracle.layer(dp["x"], dp["wr"], w1f, w2f, d["K"], bias=d["bias"], nthreads=8)
    err_plain, _ = layer_check(y, idx, gate, dp, plain, tol=TOL["fp8"])
    print(f"{name}: E4M3 layer vs oracle {err:.2e} (bf16-hidden mirror {err_m:.2e}), "
          f"vs unquantised layer {err_plain:.2e}")



def test_layer_fp8_forced_empty_experts_odd_batch_and_determinism():
    """E4M3 layer with experts 5.. forced empty by the bias, a batch that is not
    a multiple of the 16-token tiles, and two runs bit-identical."""
    d = configs.layer_fp8_inputs("tiny", T=37)
    b = np.zeros(d["E"], np.float32)
    b[5:] = -1e4
    d["bias"] = b
    y1, idx, gate, counts = _run_layer_fp8(d)
    y2, _, _, _ = _run_layer_fp8(d)
    assert counts[5:].sum() == 0 and counts.sum() == d["T"] * d["K"]
    assert np.array_equal(y1, y2)
    ref = oracle.layer_fp8(d["x"], d["wr"], d["w1"], d["w1_scale"], d["w2"], d["w2_scale"], d["K"], bias=b,
                           nthreads=8)
    layer_check(y1, idx, gate, d, ref, tol=TOL["fp8"], fp8=True)


@pytest.mark.parametrize("name,T", [("decode", 16), ("prefill", 300)])
def test_layer_graph_replays_match_eager(name, T):
    """moe_layer and moe_layer_fp8 captured in a HIP graph: every replay, with
    eager work and synchronisations between replays, equals the eager result
    bit for bit (the library enqueues kernels only: no memsets, copies or
    allocations)."""
    d = configs.layer_inputs(name, T=T, dtype="bf16", H=512, F=768)
    x, wr, w1, w2 = to_dev(d["x"]), to_dev(d["wr"]), to_dev(d["w1"]), to_dev(d["w2"])
    K = d["K"]
    ws = torch.empty((moe.layer_workspace_size(T, d["H"], d["E"], K, d["F"], moe.BF16),), dtype=torch.uint8,
                     device="cuda")
    y = torch.empty((T, d["H"]), dtype=torch.bfloat16, device="cuda")
    f = configs.layer_fp8_inputs(name, T=T, H=512, F=768)
    sc = lambda v: torch.tensor([float(v)], dtype=torch.float32, device="cuda")
    xf, wrf, w1f, w2f, s1, s2 = (to_dev(f["x"]), to_dev(f["wr"]), to_dev(f["w1"]), to_dev(f["w2"]),
                                 sc(f["w1_scale"]), sc(f["w2_scale"]))
    wsf = torch.empty((moe.layer_fp8_workspace_size(T, 512, f["E"], K, 768),), dtype=torch.uint8, device="cuda")
    yf = torch.empty((T, 512), dtype=torch.bfloat16, device="cuda")

    def both():
        moe.layer(x, wr, w1, w2, K, y=y, ws=ws)
        moe.layer_fp8(xf, wrf, w1f, s1, w2f, s2, K, y=yf, ws=wsf)

    both()
    torch.cuda.synchronize()
    ref, reff = to_host(y).copy(), to_host(yf).copy()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        both()  # warm the side stream before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        both()
    for _ in range(3):
        y.zero_()
        yf.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(y), ref) and np.array_equal(to_host(yf), reff)
        both()  # eager work between replays
        torch.cuda.synchronize()
