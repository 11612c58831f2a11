"""fp64 CPU oracle of the mixture-of-experts layer (ctypes over moe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product package. It shares no code
with the HIP library.

Encodings are taken from the numpy dtype of each array:
float32 -> binary32, uint16 -> bfloat16 bit patterns, uint8 -> OCP E4M3
bytes, float64 -> binary64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

F32, BF16, E4M3, F64 = 0, 1, 2, 3
ACT_NONE, ACT_RELU = 0, 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
             "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.orc_decode.argtypes = [vp, i32, i64]
        L.orc_decode.restype = dbl
        L.orc_decode_array.argtypes = [vp, i32, i64, vp]
        L.orc_round_bf16.argtypes = [dbl]
        L.orc_round_bf16.restype = dbl
        L.orc_bf16_bits.argtypes = [dbl]
        L.orc_bf16_bits.restype = ctypes.c_uint16
        L.orc_route.argtypes = [vp, vp, i32, vp, i32, i32, i32, i32, vp, vp, vp, vp]
        L.orc_route_given.argtypes = [vp, vp, i32, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp]
        L.orc_permute.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
        L.orc_gather_rows.argtypes = [vp, i64, vp, i32, i32, vp]
        L.orc_gmm.argtypes = [vp, i32, dbl, vp, i32, dbl, vp, i32, i32, i32, i32, vp, i32, vp, i32]
        L.orc_gmm_mx.argtypes = [vp, i32, vp, vp, i32, vp, vp, i32, i32, i32, i32, vp, i32, vp, i32]
        L.orc_gmm_row_scaled.argtypes = [vp, i32, vp, vp, i32, dbl, vp, i32, i32, i32, i32, vp, i32, vp,
                                         i32]
        L.orc_e4m3_nearest.argtypes = [ctypes.c_float]
        L.orc_e4m3_nearest.restype = ctypes.c_uint8
        L.orc_e4m3_nearest_ratio.argtypes = [dbl, dbl]
        L.orc_e4m3_nearest_ratio.restype = ctypes.c_uint8
        L.orc_div448_f32.argtypes = [dbl]
        L.orc_div448_f32.restype = ctypes.c_float
        L.orc_e4m3_nearest_array.argtypes = [vp, i64, vp]
        L.orc_quant_rows.argtypes = [vp, i32, i32, i32, vp, i32, i32, vp, vp]
        L.orc_gmm_mx4.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, i32, vp, i32]
        L.orc_e2m1.argtypes = [i32]
        L.orc_e2m1.restype = dbl
        L.orc_e8m0.argtypes = [i32]
        L.orc_e8m0.restype = dbl
        L.orc_combine.argtypes = [vp, vp, vp, i32, i32, i32, vp]
        L.orc_expert_ffn.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp]
        L.orc_layer.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp,
                                vp, i32]
        L.orc_layer_tokens.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, i32,
                                       vp, vp, vp, vp, i32]
        L.orc_layer_tokens_given.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, i32,
                                             vp, vp, vp, vp, vp, i32]
        L.orc_layer_dense.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp]
        for name in ("orc_decode_array", "orc_route", "orc_route_given", "orc_layer_tokens_given",
                     "orc_permute", "orc_gather_rows", "orc_gmm", "orc_gmm_mx",
                     "orc_gmm_row_scaled", "orc_e4m3_nearest_array", "orc_quant_rows", "orc_gmm_mx4",
                     "orc_combine", "orc_expert_ffn", "orc_layer", "orc_layer_tokens",
                     "orc_layer_dense"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def _code(a: np.ndarray) -> int:
    m = {np.dtype(np.float32): F32, np.dtype(np.uint16): BF16, np.dtype(np.uint8): E4M3,
         np.dtype(np.float64): F64}
    if a.dtype not in m:
        raise TypeError(f"oracle: unsupported array dtype {a.dtype}")
    return m[a.dtype]


def _c(a):
    a = np.ascontiguousarray(a)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def decode(a: np.ndarray) -> np.ndarray:
    a, pa = _c(a)
    out = np.empty(a.size, np.float64)
    _check(lib().orc_decode_array(pa, _code(a), a.size, _p(out)), "decode")
    return out.reshape(a.shape)


def round_bf16(v: float) -> float:
    return lib().orc_round_bf16(float(v))


def bf16_bits(values) -> np.ndarray:
    v = np.asarray(values, np.float64)
    f = lib().orc_bf16_bits
    return np.array([f(float(x)) for x in v.ravel()], np.uint16).reshape(v.shape)


def route(x, wr, T, H, E, K, bias=None):
    """Router scores, top-k and sparse softmax. Returns (idx, gate, logits, gap)."""
    x, px = _c(x)
    wr, pw = _c(wr)
    if _code(x) != _code(wr):
        raise TypeError("x and wr must share an encoding")
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    idx = np.empty((T, K), np.int32)
    gate = np.empty((T, K), np.float64)
    logits = np.empty((T, E), np.float64)
    gap = np.empty(T, np.float64)
    _check(lib().orc_route(px, pw, _code(x), _p(b), T, H, E, K, _p(idx), _p(gate), _p(logits),
                           _p(gap)), "route")
    return idx, gate, logits, gap


def route_given(x, wr, T, H, E, K, given, bias=None):
    """Router scores with the K experts of each token given ((T,K), e.g. a
    selection made elsewhere): gates over the given experts' scores in the
    given slot order. Returns (idx, gate, logits, gap); gap is the full sort's."""
    x, px = _c(x)
    wr, pw = _c(wr)
    gv, pg = _c(np.asarray(given, np.int32).reshape(T, K))
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    idx = np.empty((T, K), np.int32)
    gate = np.empty((T, K), np.float64)
    logits = np.empty((T, E), np.float64)
    gap = np.empty(T, np.float64)
    _check(lib().orc_route_given(px, pw, _code(x), _p(b), T, H, E, K, pg, _p(idx), _p(gate), _p(logits),
                                 _p(gap)), "route_given")
    return idx, gate, logits, gap


def permute(topk_idx, E):
    idx, pidx = _c(np.asarray(topk_idx, np.int32))
    T, K = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    psrc = np.empty(T * K, np.int32)
    pdst = np.empty(T * K, np.int32)
    _check(lib().orc_permute(pidx, T, E, K, _p(counts), _p(offsets), _p(psrc), _p(pdst)), "permute")
    return counts, offsets, psrc, pdst


def gather_rows(x, perm_src, K):
    x, px = _c(x)
    ps, pps = _c(np.asarray(perm_src, np.int32))
    A = ps.size
    out = np.empty((A,) + x.shape[1:], x.dtype)
    row_bytes = x[0].nbytes if x.shape[0] else 1
    _check(lib().orc_gather_rows(px, row_bytes, pps, A, K, _p(out)), "gather_rows")
    return out


def gmm(a, w, offsets, act=ACT_NONE, a_scale=1.0, w_scale=1.0, rows=None, nthreads=1):
    """Grouped GEMM: a (A,Hin), w (e,Hin,N), offsets (e+1). fp64 result.
    a_scale: one number, or one per grouped row (an array of A values: the
    per-token scale of gmmX)."""
    if np.ndim(a_scale) > 0:
        return _gmm_row_scaled(a, w, offsets, act, a_scale, w_scale, rows, nthreads)
    a, pa = _c(a)
    w, pw = _c(w)
    off, poff = _c(np.asarray(offsets, np.int32))
    e, Hin, N = w.shape
    if a.shape[1] != Hin:
        raise ValueError("a and w disagree on Hin")
    if rows is None:
        out = np.empty((int(off[e]), N), np.float64)
        prow, nrows = None, 0
    else:
        rows = np.ascontiguousarray(rows, np.int32)
        out = np.empty((rows.size, N), np.float64)
        prow, nrows = _p(rows), rows.size
    _check(lib().orc_gmm(pa, _code(a), float(a_scale), pw, _code(w), float(w_scale), poff, e, Hin,
                         N, act, prow, nrows, _p(out), int(nthreads)), "gmm")
    return out


def _gmm_row_scaled(a, w, offsets, act, a_scale, w_scale, rows, nthreads):
    a, pa = _c(a)
    w, pw = _c(w)
    rs, prs = _c(np.asarray(a_scale, np.float64).reshape(-1))
    off, poff = _c(np.asarray(offsets, np.int32))
    e, Hin, N = w.shape
    if a.shape[1] != Hin or rs.size != a.shape[0]:
        raise ValueError("gmm: a, w and the row scales disagree")
    if rows is None:
        out = np.empty((int(off[e]), N), np.float64)
        prow, nrows = None, 0
    else:
        rows = np.ascontiguousarray(rows, np.int32)
        out = np.empty((rows.size, N), np.float64)
        prow, nrows = _p(rows), rows.size
    _check(lib().orc_gmm_row_scaled(pa, _code(a), prs, pw, _code(w), float(w_scale), poff, e, Hin, N, act,
                                    prow, nrows, _p(out), int(nthreads)), "gmm (per-row scales)")
    return out


def e4m3_nearest(v) -> np.ndarray:
    """E4M3 codes (uint8) of the finite E4M3 values nearest to the binary32
    values v, ties to the even code, +-448 beyond the range."""
    v, pv = _c(np.asarray(v, np.float32))
    out = np.empty(v.shape, np.uint8)
    _check(lib().orc_e4m3_nearest_array(pv, v.size, _p(out)), "e4m3_nearest")
    return out


def e4m3_nearest_ratio(num: float, den: float) -> int:
    """E4M3 code of the value nearest to the exact quotient num / den (den a
    positive binary32 number), by exact comparisons; ties to the even code."""
    return int(lib().orc_e4m3_nearest_ratio(float(num), float(den)))


def div448_f32(amax: float) -> np.float32:
    """amax / 448 rounded to the nearest binary32 number (ties to even)."""
    return np.float32(lib().orc_div448_f32(float(amax)))


def quant_rows(x, rows=None, div=1):
    """Per-token dynamic E4M3 quantisation: for each output row, the source row
    t = rows[r] // div (or r), scale = max|x[t]| / 448 rounded to binary32,
    codes = the E4M3 values nearest to the exact quotients x[t] / scale (ties
    to even). x in binary32, bfloat16 (uint16) or binary64. Returns (codes
    (R,H) uint8, scales (R,) float32)."""
    x, px = _c(x)
    n, H = x.shape
    if rows is None:
        R, pr = n, None
    else:
        rows = np.ascontiguousarray(rows, np.int32)
        R, pr = rows.size, _p(rows)
    q = np.empty((R, H), np.uint8)
    sc = np.empty(R, np.float32)
    _check(lib().orc_quant_rows(px, _code(x), n, H, pr, int(div), R, _p(q), _p(sc)), "quant_rows")
    return q, sc


def e8m0(s: int) -> float:
    """Value of one E8M0 scale byte: 2**(s - 127); 255 is NaN."""
    return lib().orc_e8m0(int(s))


def gmm_mx(a, a_scale, w, w_scale, offsets, act=ACT_NONE, rows=None, nthreads=1):
    """Grouped GEMM on MX block-scaled operands: a (A,Hin) and w (e,Hin,N) E4M3
    (or any oracle encoding), a_scale (A, Hin/32) and w_scale (e, Hin/32, N)
    E8M0 bytes (uint8); every 32-element reduction block is scaled by both of
    its scales. fp64 result."""
    a, pa = _c(a)
    w, pw = _c(w)
    sa, psa = _c(np.asarray(a_scale, np.uint8))
    sw, psw = _c(np.asarray(w_scale, np.uint8))
    off, poff = _c(np.asarray(offsets, np.int32))
    e, Hin, N = w.shape
    if a.shape[1] != Hin or Hin % 32 or sa.shape != (a.shape[0], Hin // 32) or sw.shape != (e, Hin // 32, N):
        raise ValueError("gmm_mx: shapes disagree")
    if rows is None:
        out = np.empty((int(off[e]), N), np.float64)
        prow, nrows = None, 0
    else:
        rows = np.ascontiguousarray(rows, np.int32)
        out = np.empty((rows.size, N), np.float64)
        prow, nrows = _p(rows), rows.size
    _check(lib().orc_gmm_mx(pa, _code(a), psa, pw, _code(w), psw, poff, e, Hin, N, act, prow, nrows, _p(out),
                            int(nthreads)), "gmm_mx")
    return out


def e2m1(code: int) -> float:
    """Value of one E2M1 (OCP FP4) code 0..15."""
    return lib().orc_e2m1(int(code))


def gmm_mx4(a, a_scale, w, w_scale, offsets, act=ACT_NONE, rows=None, nthreads=1):
    """Grouped GEMM on MX operands with E2M1 elements: a (A, Hin/2) and w
    (e, Hin/2, N) packed bytes (two elements per byte along Hin, the even one
    in the low nibble), a_scale (A, Hin/32) and w_scale (e, Hin/32, N) E8M0
    bytes. fp64 result."""
    a, pa = _c(np.asarray(a, np.uint8))
    w, pw = _c(np.asarray(w, np.uint8))
    sa, psa = _c(np.asarray(a_scale, np.uint8))
    sw, psw = _c(np.asarray(w_scale, np.uint8))
    off, poff = _c(np.asarray(offsets, np.int32))
    e, Hh, N = w.shape
    Hin = 2 * Hh
    if a.shape[1] != Hh or Hin % 32 or sa.shape != (a.shape[0], Hin // 32) or sw.shape != (e, Hin // 32, N):
        raise ValueError("gmm_mx4: shapes disagree")
    if rows is None:
        out = np.empty((int(off[e]), N), np.float64)
        prow, nrows = None, 0
    else:
        rows = np.ascontiguousarray(rows, np.int32)
        out = np.empty((rows.size, N), np.float64)
        prow, nrows = _p(rows), rows.size
    _check(lib().orc_gmm_mx4(pa, psa, pw, psw, poff, e, Hin, N, act, prow, nrows, _p(out), int(nthreads)),
           "gmm_mx4")
    return out


def combine(yp, perm_dst, gate, T, K):
    yp, pyp = _c(np.asarray(yp, np.float64))
    pd, ppd = _c(np.asarray(perm_dst, np.int32))
    N = yp.shape[1]
    g = None if gate is None else np.ascontiguousarray(gate, np.float64)
    out = np.empty((T, N) if g is not None else (T * K, N), np.float64)
    _check(lib().orc_combine(pyp, ppd, _p(g), T, K, N, _p(out)), "combine")
    return out


def expert_ffn(xrow, w1, w2, ex, act=ACT_RELU):
    xv, pxv = _c(np.asarray(xrow, np.float64))
    w1, p1 = _c(w1)
    w2, p2 = _c(w2)
    _, H, F = w1.shape
    out = np.empty(H, np.float64)
    _check(lib().orc_expert_ffn(pxv, p1, p2, _code(w1), ex, H, F, act, _p(out)), "expert_ffn")
    return out


def layer(x, wr, w1, w2, K, bias=None, act=ACT_RELU, nthreads=1):
    """Whole layer, sparse form. Returns dict with y, idx, gate, gap, counts."""
    x, px = _c(x)
    wr, pwr = _c(wr)
    w1, p1 = _c(w1)
    w2, p2 = _c(w2)
    T, H = x.shape
    E, _, F = w1.shape
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    y = np.empty((T, H), np.float64)
    idx = np.empty((T, K), np.int32)
    gate = np.empty((T, K), np.float64)
    gap = np.empty(T, np.float64)
    counts = np.empty(E, np.int32)
    _check(lib().orc_layer(px, pwr, _p(b), p1, p2, _code(x), T, H, E, K, F, act, _p(y), _p(idx),
                           _p(gate), _p(gap), _p(counts), int(nthreads)), "layer")
    return {"y": y, "idx": idx, "gate": gate, "gap": gap, "counts": counts}


def layer_fp8(x, wr, w1, w1_scale, w2, w2_scale, K, bias=None, act=ACT_RELU, tokens=None, given=None,
              hidden="f64", nthreads=1):
    """The layer with E4M3 experts and per-token dynamic quantisation
    ("aclnnQuantGroupedMatMulAlltoAllv": quant mode 7 for the activations,
    per-tensor weight scales, gmmY = (gmmX @ W) * gmmXScale * wScale), composed
    from the functions above: route the bf16 tokens, permute, quantise each
    token, GEMM 1 on the dispatched codes with their tokens' scales, the fp64
    hidden rows quantised per row, GEMM 2, the weighted combine. Every token is
    independent, so `tokens` (indices) computes just those tokens. `given`
    ((T,K), or (len(tokens),K)) replaces the router's selection by the given
    experts (gates over their scores). hidden="bf16" rounds the hidden rows to
    bfloat16 before quantising them, as a layer that stores them in bf16 does
    (a diagnostic mirror of that storage step; the default keeps them in
    fp64). Returns dict with y, idx, gate, gap, counts."""
    x = np.asarray(x)
    if tokens is not None:
        x = x[np.asarray(tokens)]
    T, H = x.shape
    E = w1.shape[0]
    if given is None:
        idx, gate, _, gap = route(x, wr, T, H, E, K, bias=bias)
    else:
        idx, gate, _, gap = route_given(x, wr, T, H, E, K, given, bias=bias)
    counts, off, psrc, pdst = permute(idx, E)
    xq, xs = quant_rows(x)
    tok = psrc // K
    hm = gmm(xq[tok], w1, off, act=act, a_scale=xs[tok].astype(np.float64), w_scale=float(w1_scale),
             nthreads=nthreads)
    if hidden not in ("f64", "bf16"):
        raise ValueError("hidden must be 'f64' or 'bf16'")
    hq, hs = quant_rows(hm if hidden == "f64" else bf16_bits(hm))
    yp = gmm(hq, w2, off, a_scale=hs.astype(np.float64), w_scale=float(w2_scale), nthreads=nthreads)
    y = combine(yp, pdst, gate, T, K)
    return {"y": y, "idx": idx, "gate": gate, "gap": gap, "counts": counts}


def layer_tokens(x, wr, w1, w2, K, tokens, bias=None, act=ACT_RELU, given=None, nthreads=1):
    """Per-token form on a subset of tokens. `given` ((len(tokens),K))
    replaces the router's selection by the given experts (gates over their
    scores). Returns dict with y, idx, gate, gap."""
    x, px = _c(x)
    wr, pwr = _c(wr)
    w1, p1 = _c(w1)
    w2, p2 = _c(w2)
    T, H = x.shape
    E, _, F = w1.shape
    tok, ptok = _c(np.asarray(tokens, np.int32))
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    n = tok.size
    gv = None if given is None else np.ascontiguousarray(np.asarray(given, np.int32).reshape(n, K))
    y = np.empty((n, H), np.float64)
    idx = np.empty((n, K), np.int32)
    gate = np.empty((n, K), np.float64)
    gap = np.empty(n, np.float64)
    _check(lib().orc_layer_tokens_given(px, pwr, _p(b), p1, p2, _code(x), T, H, E, K, F, act, ptok, n, _p(gv),
                                        _p(y), _p(idx), _p(gate), _p(gap), int(nthreads)), "layer_tokens")
    return {"y": y, "idx": idx, "gate": gate, "gap": gap}


def layer_dense(x, wr, w1, w2, K, bias=None, act=ACT_RELU):
    x, px = _c(x)
    wr, pwr = _c(wr)
    w1, p1 = _c(w1)
    w2, p2 = _c(w2)
    T, H = x.shape
    E, _, F = w1.shape
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    y = np.empty((T, H), np.float64)
    _check(lib().orc_layer_dense(px, pwr, _p(b), p1, p2, _code(x), T, H, E, K, F, act, _p(y)),
           "layer_dense")
    return y
