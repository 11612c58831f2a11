"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (moe_layer / moe_route / moe_permute / moe_gmm / moe_combine
on the same shapes). The oracle computes sampled outputs one by one (the
per-token form of the layer, single rows of the grouped GEMM); properties that
hold at any size cover the rest. Inputs come from synth only.
"""
import functools

import numpy as np
import pytest
import torch

import mixture_experts_layer_06_amd as moe
import oracle
import synth
from synth import configs
from tests.helpers import TOL, as_f64, check_selection, layer_check, normwise_err, to_dev, to_host

pytestmark = pytest.mark.gpu

NTH = synth.threads()


@functools.lru_cache(maxsize=4)
def _inputs(name, T):
    return configs.layer_inputs(name, T=T)


def _layer_on_gpu(d):
    T, E, K = d["T"], d["E"], d["K"]
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, K), dtype=torch.float32, device="cuda")
    counts = torch.empty((E,), dtype=torch.int32, device="cuda")
    bias = to_dev(d["bias"]) if d["bias"] is not None else None
    x, wr, w1, w2 = (to_dev(d[k]) for k in ("x", "wr", "w1", "w2"))
    y = moe.layer(x, wr, w1, w2, K, bias=bias, topk_idx=idx, topk_gate=gate, counts=counts)
    torch.cuda.synchronize()
    del x, wr, w1, w2
    return to_host(y), to_host(idx), to_host(gate), to_host(counts)


def _sample_tokens(T, n, seed):
    rng = np.random.default_rng(seed)
    s = set([0, T - 1]) | set(rng.choice(T, size=min(n, T), replace=False).tolist())
    return np.array(sorted(s), np.int32)


@pytest.mark.parametrize("name,T,nsample", [
    ("prefill", 4096, 24),
    ("skewed", 16384, 48),
    ("decode", 16, 16),
    ("decode", 64, 24),
    ("decode", 256, 32),
])
def test_layer_full_size_sampled_tokens(name, T, nsample):
    d = _inputs(name, T)
    y, idx, gate, counts = _layer_on_gpu(d)
    K, E = d["K"], d["E"]
    assert counts.sum() == T * K
    assert np.array_equal(np.bincount(idx.ravel(), minlength=E), counts)
    toks = _sample_tokens(T, nsample, seed=T)
    ref = oracle.layer_tokens(d["x"], d["wr"], d["w1"], d["w2"], K, toks, bias=d["bias"],
                              nthreads=NTH)
    err, n_alt = layer_check(y, idx, gate, d, ref, tokens=toks, tol=TOL["bf16"], nthreads=NTH)
    print(f"{name} T={T}: {len(toks)} sampled tokens, normwise error {err:.2e}, {n_alt} near ties")
    if name == "skewed":
        # the router bias gives expert 0 the largest share and a long tail
        assert counts.argmax() == 0 and counts[0] > 8 * np.median(counts)


def test_route_full_size_all_tokens_decode_and_prefill():
    for name, T in (("decode", 256), ("prefill", 4096)):
        d = _inputs(name, T)
        K = d["K"]
        idx, gate = moe.route(to_dev(d["x"]), to_dev(d["wr"]), K)
        torch.cuda.synchronize()
        idx, gate = to_host(idx), to_host(gate)
        ridx, rgate, logits, gap = oracle.route(d["x"], d["wr"], T, d["H"], d["E"], K)
        diff = check_selection(idx, ridx, logits, K)
        if diff.any():
            _, g2, _, _ = oracle.route_given(d["x"][diff], d["wr"], int(diff.sum()), d["H"], d["E"], K,
                                             idx[diff])
            rgate = rgate.copy()
            rgate[diff] = g2
        assert np.abs(gate - rgate).max() <= 2e-3
        print(f"{name} T={T}: every token checked, {int((gap <= 1e-3).sum())} near ties, "
              f"{int(diff.sum())} selections differ from the oracle's")


@pytest.mark.parametrize("T,E,K,H", [(4096, 8, 2, 4096), (16384, 64, 6, 2048), (8192, 32, 8, 7168)])
def test_permute_full_size_bit_exact(T, E, K, H):
    idx = synth.random_routing(600 + E, T, E, K)
    x = synth.normal(601, (T, H), dtype="bf16") if H <= 4096 else None
    r = moe.permute(to_dev(idx), E, x=to_dev(x) if x is not None else None)
    torch.cuda.synchronize()
    counts, offsets, psrc, pdst = oracle.permute(idx, E)
    assert np.array_equal(to_host(r["counts"]), counts)
    assert np.array_equal(to_host(r["offsets"]), offsets)
    assert np.array_equal(to_host(r["perm_src"]), psrc)
    assert np.array_equal(to_host(r["perm_dst"]), pdst)
    if x is not None:
        xp = to_host(r["x_perm"])
        rows = np.random.default_rng(1).choice(T * K, 512, replace=False)
        assert np.array_equal(xp[rows], x[psrc[rows] // K])


def _boundary_rows(offsets, extra, seed):
    rows = set()
    for e in range(len(offsets) - 1):
        if offsets[e + 1] > offsets[e]:
            rows |= {int(offsets[e]), int(offsets[e + 1] - 1)}
    rng = np.random.default_rng(seed)
    rows |= set(rng.choice(int(offsets[-1]), extra, replace=False).tolist())
    return np.array(sorted(rows), np.int32)


@pytest.mark.parametrize("which", ["w1", "w2"])
def test_gmm_full_size_prefill_sampled_rows(which):
    """moe_gmm on the prefill GEMM shapes (8192 rows, 8 experts) against
    single-row oracle results, first/last row of every expert included."""
    T, E, K, H, F = 4096, 8, 2, 4096, 14336
    idx = synth.random_routing(610, T, E, K)
    counts, offsets, _, _ = oracle.permute(idx, E)
    Hin, N = (H, F) if which == "w1" else (F, H)
    a = synth.normal(611, (T * K, Hin), dtype="bf16")
    w = synth.normal(612, (E, Hin, N), (1.0 / Hin) ** 0.5, dtype="bf16")
    act = moe.ACT_RELU if which == "w1" else moe.ACT_NONE
    out = to_host(moe.gmm(to_dev(a), to_dev(w), to_dev(offsets), act=act))
    rows = _boundary_rows(offsets, 16, 613)
    ref = oracle.gmm(a, w, offsets, act=act, rows=rows, nthreads=NTH)
    assert normwise_err(out[rows], ref) <= 8e-3


def test_fp8_gmm_unpermute_and_shared_expert_full_size():
    """The page-2 workload: E4M3 grouped GEMM (65536 x 7168 x 2048, 32 experts,
    per-tensor scales) + Unpermute, separate and fused, and the bf16
    shared-expert GEMM."""
    d = configs.fp8_inputs()
    T, e, K, A, H1, N1 = (d[k] for k in ("T", "e", "K", "A", "H1", "N1"))
    counts, offsets, psrc, pdst = oracle.permute(d["topk_idx"], e)
    perm = moe.permute(to_dev(d["topk_idx"]), e)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(perm["offsets"]), offsets)
    sx = torch.tensor([float(d["gmm_x_scale"])], device="cuda")
    sw = torch.tensor([float(d["gmm_w_scale"])], device="cuda")
    gy = moe.gmm(to_dev(d["gmm_x"]), to_dev(d["gmm_w"]), perm["offsets"], a_scale=sx, w_scale=sw)
    un = moe.combine(gy, perm["perm_dst"], None, T, K)
    torch.cuda.synchronize()
    gy_h, un_h = to_host(gy), to_host(un)
    rows = _boundary_rows(offsets, 24, 620)
    ref = oracle.gmm(d["gmm_x"], d["gmm_w"], offsets, a_scale=float(d["gmm_x_scale"]),
                     w_scale=float(d["gmm_w_scale"]), rows=rows, nthreads=NTH)
    assert normwise_err(gy_h[rows], ref) <= TOL["fp8"]
    assert normwise_err(gy_h[rows], ref) <= 8e-3  # one bf16 rounding of an exact-input sum
    # Unpermute: slot psrc[r] of the output holds row r (bit copy), at every sampled row
    assert np.array_equal(un_h[psrc[rows]], gy_h[rows])
    assert normwise_err(un_h[psrc[rows]], ref) <= 8e-3
    # the whole unpermute is a bijection of rows
    assert np.array_equal(un_h[psrc], gy_h)
    # Unpermute fused into the GEMM's stores (the launch the benchmark times) is
    # the same bytes
    fu = moe.gmm(to_dev(d["gmm_x"]), to_dev(d["gmm_w"]), perm["offsets"], a_scale=sx, w_scale=sw,
                 dst=perm["perm_src"])
    torch.cuda.synchronize()
    assert np.array_equal(to_host(fu), un_h)
    # shared expert: e = 1 grouped GEMM == plain GEMM
    mo = moe.gmm(to_dev(d["mm_x"]), to_dev(d["mm_w"]).view(1, d["H2"], d["N2"]),
                 to_dev(np.array([0, T], np.int32)))
    torch.cuda.synchronize()
    srows = np.random.default_rng(621).choice(T, 12, replace=False).astype(np.int32)
    sref = oracle.gmm(d["mm_x"], d["mm_w"].reshape(1, d["H2"], d["N2"]), np.array([0, T], np.int32),
                      rows=srows, nthreads=NTH)
    assert normwise_err(to_host(mo)[srows], sref) <= 8e-3


def test_fp8_mx_gmm_full_size_sampled_rows():
    """The fp8 workload with MX block scales (65536 x 7168 x 2048, 32 experts):
    sampled rows, the first and last of every expert, against the oracle."""
    d = configs.fp8_mx_inputs(with_shared=False)
    e = d["e"]
    counts, offsets, _, _ = oracle.permute(d["topk_idx"], e)
    perm = moe.permute(to_dev(d["topk_idx"]), e)
    gy = moe.gmm_mx(to_dev(d["gmm_x"]), to_dev(synth.mx_scales_slice_major(d["gmm_x_scale"], 4)), to_dev(d["gmm_w"]),
                    to_dev(synth.mx_weight_scales_interleaved(d["gmm_w_scale"])), perm["offsets"])
    torch.cuda.synchronize()
    rows = _boundary_rows(offsets, 24, 640)
    ref = oracle.gmm_mx(d["gmm_x"], d["gmm_x_scale"], d["gmm_w"], d["gmm_w_scale"], offsets, rows=rows,
                        nthreads=NTH)
    assert normwise_err(to_host(gy)[rows], ref) <= 8e-3


def test_fp8_dynamic_per_token_full_size_sampled_rows():
    """The fp8 workload with gmmX in bf16, quantised per row on the device
    (65536 x 7168), then the per-token-scaled GEMM with the Unpermute fused
    into its stores, as the benchmark runs it: codes and scales of sampled rows
    bit-exact, outputs of sampled rows against the oracle."""
    d = configs.fp8_dyn_inputs(with_shared=False)
    e, A = d["e"], d["A"]
    counts, offsets, psrc, _ = oracle.permute(d["topk_idx"], e)
    perm = moe.permute(to_dev(d["topk_idx"]), e)
    q, sc = moe.quant_rows(to_dev(d["gmm_x"]))
    sw = float(d["gmm_w_scale"])
    un = moe.gmm(q, to_dev(d["gmm_w"]), perm["offsets"], a_scale=sc, per_token=True,
                 w_scale=torch.tensor([sw], dtype=torch.float32, device="cuda"), dst=perm["perm_src"])
    torch.cuda.synchronize()
    rows = _boundary_rows(offsets, 24, 650)
    rq, rs = oracle.quant_rows(d["gmm_x"][rows])
    q_h, sc_h = to_host(q), to_host(sc)
    assert np.array_equal(q_h[rows], rq) and np.array_equal(sc_h[rows], rs)
    ref = oracle.gmm(q_h, d["gmm_w"], offsets, a_scale=sc_h.astype(np.float64), w_scale=sw, rows=rows,
                     nthreads=NTH)
    assert normwise_err(to_host(un)[psrc[rows]], ref) <= 8e-3


def test_fp4_mx_gmm_full_size_sampled_rows():
    """The fp8 workload's shapes with MXFP4 operands (65536 x 7168 x 2048, 32
    experts): sampled rows, the first and last of every expert, against the oracle."""
    d = configs.fp4_mx_inputs(with_shared=False)
    e = d["e"]
    counts, offsets, _, _ = oracle.permute(d["topk_idx"], e)
    perm = moe.permute(to_dev(d["topk_idx"]), e)
    gy = moe.gmm_mxfp4(to_dev(d["gmm_x"]), to_dev(synth.mx_scales_slice_major(d["gmm_x_scale"], 8)),
                       to_dev(d["gmm_w"]),
                       to_dev(synth.mx_weight_scales_interleaved(d["gmm_w_scale"])), perm["offsets"])
    torch.cuda.synchronize()
    rows = _boundary_rows(offsets, 24, 660)
    ref = oracle.gmm_mx4(d["gmm_x"], d["gmm_x_scale"], d["gmm_w"], d["gmm_w_scale"], offsets, rows=rows,
                         nthreads=NTH)
    assert normwise_err(to_host(gy)[rows], ref) <= 8e-3


def test_layer_fp8_full_size_prefill_sampled_tokens():
    """The E4M3 layer on the prefill shapes (T=4096, H=4096, E=8, K=2, F=14336):
    sampled tokens against the oracle's E4M3 layer on those tokens."""
    d = configs.layer_fp8_inputs("prefill")
    T, K = d["T"], d["K"]
    sc = lambda v: torch.tensor([float(v)], dtype=torch.float32, device="cuda")
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, K), dtype=torch.float32, device="cuda")
    y = moe.layer_fp8(to_dev(d["x"]), to_dev(d["wr"]), to_dev(d["w1"]), sc(d["w1_scale"]), to_dev(d["w2"]),
                      sc(d["w2_scale"]), K, topk_idx=idx, topk_gate=gate)
    torch.cuda.synchronize()
    tokens = np.random.default_rng(670).choice(T, 12, replace=False)
    ref = oracle.layer_fp8(d["x"], d["wr"], d["w1"], d["w1_scale"], d["w2"], d["w2_scale"], K, tokens=tokens,
                           nthreads=NTH)
    err, _ = layer_check(to_host(y), to_host(idx), to_host(gate), d, ref, tokens=tokens, tol=TOL["fp8"], fp8=True,
                         nthreads=NTH)
    print(f"E4M3 layer, prefill shapes, 12 sampled tokens: normwise error {err:.2e} against the oracle")


def test_combine_full_size_prefill():
    T, E, K, H = 4096, 8, 2, 4096
    idx = synth.random_routing(630, T, E, K)
    _, _, psrc, pdst = oracle.permute(idx, E)
    yp = synth.normal(631, (T * K, H), dtype="bf16")
    g = np.abs(synth.normal(632, (T, K))).astype(np.float32)
    g /= g.sum(1, keepdims=True)
    out = to_host(moe.combine(to_dev(yp), to_dev(pdst), to_dev(g), T, K))
    ref = oracle.combine(as_f64(yp), pdst, g.astype(np.float64), T, K)
    assert normwise_err(out, ref) <= 4e-3
