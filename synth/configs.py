"""Input recipes for the five MoE workloads.

Every tensor comes from the counter-based stream with
seed = 0x4D6F45000000 + 256 * workload + tensor id, so element i of a tensor
depends only on (seed, i): a smaller token count gives a prefix of the
larger one's rows. Weights are N(0, 1/fan_in).

  tiny   T=64 H=128 E=8 K=2 F=256 fp32 (+ "int": every entry in {-2..2})
  prefill T=4096 H=4096 E=8 K=2 F=14336 bf16
  fp8gmm  e=32 K=8 T=8192 (A=65536) H1=7168 N1=2048 E4M3 per-tensor scales,
          plus the bf16 shared expert (8192,7168)x(7168,2048)
  skewed  T=16384 H=2048 E=64 K=6 F=1408 bf16, router bias -1.2*ln(e+1)
  decode  T in {16,64,256} H=4096 E=128 K=8 F=1536 bf16
"""
from __future__ import annotations

import math

import numpy as np

from . import (amax, bf16_to_f32, ints, normal, quantize_e4m3, quantize_mx, quantize_mx4, random_routing, seed_for,
               to_bf16, to_e4m3)

LAYER_SHAPES = {
    # name: (workload id, T, H, E, K, F, dtype)
    "tiny": (0, 64, 128, 8, 2, 256, "f32"),
    "prefill": (1, 4096, 4096, 8, 2, 14336, "bf16"),
    "skewed": (3, 16384, 2048, 64, 6, 1408, "bf16"),
    "decode": (4, 256, 4096, 128, 8, 1536, "bf16"),
}

FP8_SHAPE = dict(e=32, K=8, T=8192, H1=7168, N1=2048, H2=7168, N2=2048)


def skew_bias(E: int) -> np.ndarray:
    """b_e = -1.2 * ln(e + 1), as binary32."""
    return np.array([-1.2 * math.log(e + 1.0) for e in range(E)], np.float32)


def layer_inputs(name: str, T: int | None = None, integer: bool = False, H=None, E=None, K=None,
                 F=None, dtype=None, bias: bool | None = None, wid: int | None = None) -> dict:
    """Inputs of a whole-layer workload. Overrides give reduced or edge shapes
    drawn with the same recipe."""
    w0, T0, H0, E0, K0, F0, dt0 = LAYER_SHAPES[name]
    wid = w0 if wid is None else wid
    T = T0 if T is None else T
    H = H0 if H is None else H
    E = E0 if E is None else E
    K = K0 if K is None else K
    F = F0 if F is None else F
    dt = dt0 if dtype is None else dtype
    use_bias = (name == "skewed") if bias is None else bias
    if integer:
        s = lambda i: seed_for(wid, 10 + i)
        x = ints(s(0), (T, H), -2, 2, dt)
        wr = ints(s(1), (H, E), -2, 2, dt)
        w1 = ints(s(2), (E, H, F), -2, 2, dt)
        w2 = ints(s(3), (E, F, H), -2, 2, dt)
    else:
        s = lambda i: seed_for(wid, i)
        x = normal(s(0), (T, H), 1.0, dtype=dt)
        wr = normal(s(1), (H, E), math.sqrt(1.0 / H), dtype=dt)
        w1 = normal(s(2), (E, H, F), math.sqrt(1.0 / H), dtype=dt)
        w2 = normal(s(3), (E, F, H), math.sqrt(1.0 / F), dtype=dt)
    b = skew_bias(E) if use_bias else None
    return dict(name=name, T=T, H=H, E=E, K=K, F=F, dtype=dt, x=x, wr=wr, w1=w1, w2=w2, bias=b)


def layer_fp8_inputs(name: str, **shape) -> dict:
    """Inputs of the E4M3 layer on a whole-layer workload's shapes: the same
    seeds, tokens and router in bf16, expert weights drawn in fp32 and
    quantised per tensor to E4M3 (scale = amax / 448)."""
    d = layer_inputs(name, dtype="f32", **shape)
    d["x"], d["wr"] = to_bf16(d["x"]), to_bf16(d["wr"])
    d["w1"], d["w1_scale"] = quantize_e4m3(d["w1"])
    d["w2"], d["w2_scale"] = quantize_e4m3(d["w2"])
    d["dtype"] = "fp8"
    return d


def identity_ffn(H: int, E: int, dtype: str = "f32"):
    """W1 = [I | -I] (H, 2H) and W2 = [I ; -I] (2H, H) for every expert, so
    relu(x) - relu(-x) = x: each expert returns its input."""
    I = np.eye(H, dtype=np.float32)
    w1 = np.concatenate([I, -I], axis=1)
    w2 = np.concatenate([I, -I], axis=0)
    w1 = np.broadcast_to(w1, (E, H, 2 * H)).copy()
    w2 = np.broadcast_to(w2, (E, 2 * H, H)).copy()
    if dtype == "bf16":
        return to_bf16(w1), to_bf16(w2)
    return w1, w2


def fp8_inputs(T: int | None = None, e: int | None = None, K: int | None = None, H1=None, N1=None,
               H2=None, N2=None, wid: int = 2, with_shared: bool = True) -> dict:
    """Page-2 form: routing assignment, E4M3 gmmX (already in expert-grouped
    row order) and gmmWeight with per-tensor scales, bf16 shared expert."""
    d = dict(FP8_SHAPE)
    for k, v in dict(T=T, e=e, K=K, H1=H1, N1=N1, H2=H2, N2=N2).items():
        if v is not None:
            d[k] = v
    T, e, K, H1, N1, H2, N2 = d["T"], d["e"], d["K"], d["H1"], d["N1"], d["H2"], d["N2"]
    A = T * K
    idx = random_routing(seed_for(wid, 0), T, e, K)
    gx = normal(seed_for(wid, 1), (A, H1), 1.0)
    gx_q, sx = quantize_e4m3(gx)
    del gx
    gw = normal(seed_for(wid, 2), (e, H1, N1), math.sqrt(1.0 / H1))
    gw_q, sw = quantize_e4m3(gw)
    del gw
    out = dict(T=T, e=e, K=K, A=A, H1=H1, N1=N1, H2=H2, N2=N2, topk_idx=idx, gmm_x=gx_q,
               gmm_x_scale=sx, gmm_w=gw_q, gmm_w_scale=sw)
    if with_shared:
        out["mm_x"] = normal(seed_for(wid, 3), (T, H2), 1.0, dtype="bf16")
        out["mm_w"] = normal(seed_for(wid, 4), (H2, N2), math.sqrt(1.0 / H2), dtype="bf16")
    return out


def fp8_mx_inputs(wid: int = 2, with_shared: bool = True, **shape) -> dict:
    """The fp8 workload with MX operands instead of per-tensor scales: the same
    fp32 sources (same seeds), gmmX quantised in 32-element blocks along H1 per
    row, gmmWeight in 32-element blocks along H1 per output column; scales as
    E8M0 bytes (gmm_x_scale (A, H1/32), gmm_w_scale (e, H1/32, N1))."""
    d = dict(FP8_SHAPE)
    d.update({k: v for k, v in shape.items() if v is not None})
    T, e, K, H1, N1, H2, N2 = d["T"], d["e"], d["K"], d["H1"], d["N1"], d["H2"], d["N2"]
    A = T * K
    idx = random_routing(seed_for(wid, 0), T, e, K)
    gx_q, sx = quantize_mx(normal(seed_for(wid, 1), (A, H1), 1.0), axis=1)
    gw_q, sw = quantize_mx(normal(seed_for(wid, 2), (e, H1, N1), math.sqrt(1.0 / H1)), axis=1)
    out = dict(T=T, e=e, K=K, A=A, H1=H1, N1=N1, H2=H2, N2=N2, topk_idx=idx, gmm_x=gx_q,
               gmm_x_scale=sx, gmm_w=gw_q, gmm_w_scale=sw)
    if with_shared:
        out["mm_x"] = normal(seed_for(wid, 3), (T, H2), 1.0, dtype="bf16")
        out["mm_w"] = normal(seed_for(wid, 4), (H2, N2), math.sqrt(1.0 / H2), dtype="bf16")
    return out


def fp4_mx_inputs(wid: int = 2, with_shared: bool = True, **shape) -> dict:
    """The fp8 workload with MXFP4 operands: the same fp32 sources (same seeds)
    quantised to E2M1 in 32-element blocks along H1 (per row of gmmX, per
    column of gmmWeight), packed two per byte along H1: gmm_x (A, H1/2),
    gmm_w (e, H1/2, N1); E8M0 scales gmm_x_scale (A, H1/32), gmm_w_scale
    (e, H1/32, N1)."""
    d = dict(FP8_SHAPE)
    d.update({k: v for k, v in shape.items() if v is not None})
    T, e, K, H1, N1, H2, N2 = d["T"], d["e"], d["K"], d["H1"], d["N1"], d["H2"], d["N2"]
    A = T * K
    idx = random_routing(seed_for(wid, 0), T, e, K)
    gx_q, sx = quantize_mx4(normal(seed_for(wid, 1), (A, H1), 1.0), axis=1)
    gw_q, sw = quantize_mx4(normal(seed_for(wid, 2), (e, H1, N1), math.sqrt(1.0 / H1)), axis=1)
    out = dict(T=T, e=e, K=K, A=A, H1=H1, N1=N1, H2=H2, N2=N2, topk_idx=idx, gmm_x=gx_q,
               gmm_x_scale=sx, gmm_w=gw_q, gmm_w_scale=sw)
    if with_shared:
        out["mm_x"] = normal(seed_for(wid, 3), (T, H2), 1.0, dtype="bf16")
        out["mm_w"] = normal(seed_for(wid, 4), (H2, N2), math.sqrt(1.0 / H2), dtype="bf16")
    return out


def fp8_dyn_inputs(wid: int = 2, with_shared: bool = True, **shape) -> dict:
    """The fp8 workload for per-token dynamic quantisation: the same sources
    (same seeds) with gmmX left in bf16 (A, H1), to be quantised per row on the
    device; gmmWeight E4M3 with a per-tensor scale as in fp8_inputs."""
    d = dict(FP8_SHAPE)
    d.update({k: v for k, v in shape.items() if v is not None})
    T, e, K, H1, N1, H2, N2 = d["T"], d["e"], d["K"], d["H1"], d["N1"], d["H2"], d["N2"]
    A = T * K
    idx = random_routing(seed_for(wid, 0), T, e, K)
    gx = normal(seed_for(wid, 1), (A, H1), 1.0, dtype="bf16")
    gw_q, sw = quantize_e4m3(normal(seed_for(wid, 2), (e, H1, N1), math.sqrt(1.0 / H1)))
    out = dict(T=T, e=e, K=K, A=A, H1=H1, N1=N1, H2=H2, N2=N2, topk_idx=idx, gmm_x=gx,
               gmm_w=gw_q, gmm_w_scale=sw)
    if with_shared:
        out["mm_x"] = normal(seed_for(wid, 3), (T, H2), 1.0, dtype="bf16")
        out["mm_w"] = normal(seed_for(wid, 4), (H2, N2), math.sqrt(1.0 / H2), dtype="bf16")
    return out


__all__ = ["LAYER_SHAPES", "FP8_SHAPE", "skew_bias", "layer_inputs", "identity_ffn", "fp8_inputs", "fp8_mx_inputs",
           "fp8_dyn_inputs", "fp4_mx_inputs", "layer_fp8_inputs",
           "bf16_to_f32", "amax", "to_e4m3"]
