"""moe_gmm_routed_shared: the routed experts' E4M3 grouped GEMM and the shared
expert's bf16 GEMM in one launch ("aclnnQuantGroupedMatMulAlltoAllv": the
gmmY and mmY formulas of section 计算公式, run side by side as its interface
description has them). Each output must equal the separate entry point's
result bit for bit (the same tile code runs in the fused launch) and the
oracle's within one bf16 rounding."""
import math

import numpy as np
import pytest
import torch

import mixture_experts_layer_06_amd as moe
import oracle
import synth
from synth import configs
from tests.helpers import TOL, normwise_err, to_dev, to_host

pytestmark = pytest.mark.gpu


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


# (name, routed expert counts, Hin, N, shared T, Hs, Ns, mode). Both parts take
# the DMA kernels (one launch) unless the name says which part does not.
CASES = [
    ("ragged", [300, 0, 17, 513, 256, 1, 95, 600], 384, 272, 700, 384, 400, "pt"),
    ("per_token_gated_relu", [129, 640, 0, 255, 77], 256, 400, 513, 256, 256, "tok"),
    ("unscattered", [512, 512, 3], 128, 128, 257, 128, 512, "plain"),
    ("shared_streams", [200, 0, 333, 129], 256, 384, 40, 256, 256, "pt"),      # T <= 48: streaming kernel
    ("shared_unaligned", [200, 0, 333, 129], 256, 384, 300, 200, 200, "pt"),   # Ns % 16: register-staged kernel
    ("routed_unaligned", [100, 77], 200, 100, 300, 256, 256, "pt"),            # Hin % 16: register-staged kernel
    ("routed_empty", [0, 0, 0], 256, 256, 600, 256, 256, "pt"),
    ("shared_empty", [300, 11, 0, 450], 256, 256, 0, 256, 256, "pt"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_routed_shared_equals_separate_calls_and_oracle(case):
    name, counts, Hin, N, T, Hs, Ns, mode = case
    e = len(counts)
    off = _offsets(counts)
    A = int(off[-1])
    seed = 1100 + 13 * len(name) + A
    rng = np.random.default_rng(seed)
    xf = synth.normal(seed, (max(A, 1), Hin))[:A]
    w, sw = synth.quantize_e4m3(synth.normal(seed + 1, (e, Hin, N), math.sqrt(1.0 / Hin)))
    swd = torch.tensor([sw], dtype=torch.float32, device="cuda")
    if mode == "tok":  # per-row scales amax/448, codes of x / scale
        rs = (np.abs(xf).max(axis=1) / 448.0).astype(np.float32)
        x = np.stack([synth.to_e4m3(xf[r:r + 1], float(rs[r]))[0] for r in range(A)])
        asd, o_as = to_dev(rs), rs.astype(np.float64)
    else:
        x, sa = synth.quantize_e4m3(xf) if A else (np.zeros((0, Hin), np.uint8), 1.0)
        asd, o_as = torch.tensor([sa], dtype=torch.float32, device="cuda"), float(sa)
    xs = synth.normal(seed + 2, (max(T, 1), Hs), dtype="bf16")[:T]
    wsw = synth.normal(seed + 3, (1, Hs, Ns), math.sqrt(1.0 / Hs), dtype="bf16")
    dst = rng.permutation(A).astype(np.int32) if mode != "plain" else None
    gate = rng.uniform(0.05, 1.0, A).astype(np.float32) if mode == "tok" else None
    act = moe.ACT_RELU if mode == "tok" else moe.ACT_NONE
    act_s = moe.ACT_RELU if mode != "tok" else moe.ACT_NONE
    xd, wd, od = to_dev(x), to_dev(w), to_dev(off)
    xsd, wswd, osd = to_dev(xs), to_dev(wsw), to_dev(np.array([0, T], np.int32))
    dd = to_dev(dst) if dst is not None else None
    gd = to_dev(gate) if gate is not None else None
    print(f"case {name}: A={A} Hin={Hin} N={N} T={T} Hs={Hs} Ns={Ns} mode={mode}", flush=True)

    out, ys = moe.gmm_routed_shared(xd, wd, od, asd, swd, xsd, wswd, osd, act=act, act_s=act_s, dst=dd, gate=gd,
                                    per_token=mode == "tok")
    torch.cuda.synchronize()
    out_h, ys_h = to_host(out), to_host(ys)
    if A:
        sep = moe.gmm(xd, wd, od, act=act, a_scale=asd, w_scale=swd, per_token=mode == "tok", dst=dd, gate=gd)
        assert np.array_equal(out_h, to_host(sep)), name
        ref = oracle.gmm(x, w, off, act=act, a_scale=o_as, w_scale=float(sw), nthreads=8)
        if dst is not None:
            if gate is not None:
                ref = ref * gate[dst][:, None]
            full = np.zeros_like(ref)
            full[dst] = ref
            ref = full
        assert normwise_err(out_h, ref) <= 8e-3, name
    if T:
        sep_s = moe.gmm(xsd, wswd, osd, act=act_s)
        assert np.array_equal(ys_h, to_host(sep_s)), name
        sref = oracle.gmm(xs, wsw, np.array([0, T], np.int32), act=act_s, nthreads=8)
        assert normwise_err(ys_h, sref) <= 8e-3, name


def test_routed_shared_repeated_calls_are_bitwise_stable():
    """Two calls in a row, the second with fewer routed and shared rows, give
    the separate calls' bytes each time (no state is carried between calls)."""
    for counts, T in (([400, 123, 0, 700], 900), ([64, 0, 5, 30], 260)):
        e, Hin, N, Hs, Ns = len(counts), 256, 256, 256, 512
        off = _offsets(counts)
        A = int(off[-1])
        x, sa = synth.quantize_e4m3(synth.normal(1200 + A, (A, Hin)))
        w, sw = synth.quantize_e4m3(synth.normal(1201, (e, Hin, N), math.sqrt(1.0 / Hin)))
        xs = synth.normal(1202 + T, (T, Hs), dtype="bf16")
        wsw = synth.normal(1203, (1, Hs, Ns), math.sqrt(1.0 / Hs), dtype="bf16")
        asd = torch.tensor([sa], dtype=torch.float32, device="cuda")
        swd = torch.tensor([sw], dtype=torch.float32, device="cuda")
        osd = to_dev(np.array([0, T], np.int32))
        out, ys = moe.gmm_routed_shared(to_dev(x), to_dev(w), to_dev(off), asd, swd, to_dev(xs), to_dev(wsw), osd)
        sep = moe.gmm(to_dev(x), to_dev(w), to_dev(off), a_scale=asd, w_scale=swd)
        sep_s = moe.gmm(to_dev(xs), to_dev(wsw), osd)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(out), to_host(sep))
        assert np.array_equal(to_host(ys), to_host(sep_s))


def test_routed_shared_full_size_fp8_workload():
    """The E4M3 workload at full size (65536 routed rows x 7168 x 2048 over 32
    experts, Unpermute fused into the stores; shared expert 8192 x 7168 x 2048
    in bf16) in one launch: both outputs equal the separate launches bit for
    bit (the shared GEMM's 256 tiles fill one round, so the separate call does
    not split either), and sampled rows match the oracle."""
    d = configs.fp8_inputs()
    T, e, K, A, H1, N1, H2, N2 = (d[k] for k in ("T", "e", "K", "A", "H1", "N1", "H2", "N2"))
    counts, offsets, psrc, _ = oracle.permute(d["topk_idx"], e)
    perm = moe.permute(to_dev(d["topk_idx"]), e)
    sx = torch.tensor([float(d["gmm_x_scale"])], device="cuda")
    sw = torch.tensor([float(d["gmm_w_scale"])], device="cuda")
    gx, gw = to_dev(d["gmm_x"]), to_dev(d["gmm_w"])
    mx, mw = to_dev(d["mm_x"]), to_dev(d["mm_w"]).view(1, H2, N2)
    moff = to_dev(np.array([0, T], np.int32))
    print(f"full size: A={A} H1={H1} N1={N1} T={T} H2={H2} N2={N2}", flush=True)
    un, my = moe.gmm_routed_shared(gx, gw, perm["offsets"], sx, sw, mx, mw, moff, dst=perm["perm_src"])
    sep = moe.gmm(gx, gw, perm["offsets"], a_scale=sx, w_scale=sw, dst=perm["perm_src"])
    sep_s = moe.gmm(mx, mw, moff)
    torch.cuda.synchronize()
    un_h, my_h = to_host(un), to_host(my)
    assert np.array_equal(un_h, to_host(sep))
    assert np.array_equal(my_h, to_host(sep_s))
    rng = np.random.default_rng(1210)
    rows = np.unique(np.concatenate([offsets[:-1][counts > 0], offsets[1:][counts > 0] - 1,
                                     rng.choice(A, 16, replace=False)])).astype(np.int32)
    ref = oracle.gmm(d["gmm_x"], d["gmm_w"], offsets, a_scale=float(d["gmm_x_scale"]),
                     w_scale=float(d["gmm_w_scale"]), rows=rows, nthreads=16)
    assert normwise_err(un_h[psrc[rows]], ref) <= min(TOL["fp8"], 8e-3)
    srows = rng.choice(T, 12, replace=False).astype(np.int32)
    sref = oracle.gmm(d["mm_x"], d["mm_w"].reshape(1, H2, N2), np.array([0, T], np.int32), rows=srows,
                      nthreads=16)
    assert normwise_err(my_h[srows], sref) <= 8e-3


# (name, routed expert counts, Hin, N, shared T, Hs, Ns, fp4)
MX_CASES = [
    ("mx_e4m3", [300, 0, 17, 513, 256, 95], 384, 272, 700, 384, 400, False),
    ("mx_e2m1", [129, 640, 0, 255, 77], 512, 400, 513, 256, 256, True),
    ("mx_e2m1_shared_streams", [200, 0, 333], 256, 128, 40, 256, 256, True),   # T <= 48: two launches
    ("mx_e4m3_routed_empty", [0, 0], 256, 128, 300, 256, 256, False),
]


@pytest.mark.parametrize("case", MX_CASES, ids=[c[0] for c in MX_CASES])
def test_mx_routed_shared_equals_separate_calls_and_oracle(case):
    """The MX variant: the routed part equals moe_gmm_mx / moe_gmm_mxfp4 and the
    shared part moe_gmm, bit for bit, and both match the oracle."""
    name, counts, Hin, N, T, Hs, Ns, fp4 = case
    e = len(counts)
    off = _offsets(counts)
    A = int(off[-1])
    seed = 1300 + 7 * len(name) + A
    quant = synth.quantize_mx4 if fp4 else synth.quantize_mx
    if A:
        a, sa = quant(synth.normal(seed, (A, Hin)), axis=1)
    else:
        a, sa = np.zeros((0, Hin // 2 if fp4 else Hin), np.uint8), np.zeros((0, Hin // 32), np.uint8)
    w, sw = quant(synth.normal(seed + 1, (e, Hin, N), math.sqrt(1.0 / Hin)), axis=1)
    xs = synth.normal(seed + 2, (T, Hs), dtype="bf16")
    wsw = synth.normal(seed + 3, (1, Hs, Ns), math.sqrt(1.0 / Hs), dtype="bf16")
    ad, sad = to_dev(a), to_dev(synth.mx_scales_slice_major(sa, 8 if fp4 else 4))
    wd, swd, od = to_dev(w), to_dev(synth.mx_weight_scales_interleaved(sw)), to_dev(off)
    xsd, wswd, osd = to_dev(xs), to_dev(wsw), to_dev(np.array([0, T], np.int32))
    print(f"case {name}: A={A} Hin={Hin} N={N} T={T} Hs={Hs} Ns={Ns} fp4={fp4}", flush=True)
    out, ys = moe.gmm_mx_routed_shared(ad, sad, wd, swd, od, xsd, wswd, osd, fp4=fp4, act=moe.ACT_RELU,
                                       act_s=moe.ACT_RELU)
    torch.cuda.synchronize()
    out_h, ys_h = to_host(out), to_host(ys)
    if A:
        sep = (moe.gmm_mxfp4 if fp4 else moe.gmm_mx)(ad, sad, wd, swd, od, act=moe.ACT_RELU)
        assert np.array_equal(out_h, to_host(sep)), name
        ref = (oracle.gmm_mx4 if fp4 else oracle.gmm_mx)(a, sa, w, sw, off, act=moe.ACT_RELU, nthreads=8)
        assert normwise_err(out_h, ref) <= 8e-3, name
    sep_s = moe.gmm(xsd, wswd, osd, act=moe.ACT_RELU)
    assert np.array_equal(ys_h, to_host(sep_s)), name
    sref = oracle.gmm(xs, wsw, np.array([0, T], np.int32), act=moe.ACT_RELU, nthreads=8)
    assert normwise_err(ys_h, sref) <= 8e-3, name
