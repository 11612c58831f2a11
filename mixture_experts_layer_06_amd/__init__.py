"""Python binding of the gfx950 MoE C-ABI library (libmoe.so).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind include/moe.h. torch supplies device memory (tensors) and the stream
(torch.cuda.current_stream()). There is no CPU fallback: if libmoe.so is
missing the import of any entry point raises.

Tensor element types: torch.float32 -> MOE_F32, torch.bfloat16 -> MOE_BF16,
torch.uint8 or torch.float8_e4m3fn -> MOE_FP8_E4M3 (OCP E4M3 bytes).
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime libmoe.so binds to)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

# moe.h enums
OK, ERR_NULL_POINTER, ERR_BAD_SHAPE, ERR_BAD_DTYPE, ERR_UNSUPPORTED = 0, 1, 2, 3, 4
ERR_WORKSPACE_TOO_SMALL, ERR_MISALIGNED, ERR_DEVICE, ERR_SCRATCH_LIMIT = 5, 6, 7, 8
NOALLOC_SCRATCH_BYTES = 32 << 20  # MOE_NOALLOC_SCRATCH_BYTES
F32, BF16, FP8_E4M3 = 0, 1, 2
QUANT_NONE, QUANT_PER_TENSOR, QUANT_PER_TOKEN = 0, 1, 3
ACT_NONE, ACT_RELU = 0, 1

EXPORTS = ("moe_status_string", "moe_version", "moe_route_workspace_size", "moe_route",
           "moe_permute_workspace_size", "moe_permute", "moe_gmm_workspace_size", "moe_gmm",
           "moe_gmm_gather", "moe_gmm_scatter", "moe_gmm_routed_shared", "moe_gmm_mx_routed_shared", "moe_gmm_mx", "moe_gmm_mxfp4", "moe_combine", "moe_sum_slots",
           "moe_quant_rows", "moe_layer_workspace_size", "moe_layer", "moe_layer_fp8_workspace_size",
           "moe_layer_fp8", "moe_layer_noalloc", "moe_fetch_probe", "moe_mfma_probe")


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (built in-tree by build()); raise if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libmoe.so not built at {LIB_PATH}; run __graft_entry__.build() "
                              "or python -m mixture_experts_layer_06_amd._build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.moe_status_string.argtypes = [i32]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_version.argtypes = []
        L.moe_version.restype = i32
        L.moe_route_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
        L.moe_route.argtypes = [vp, vp, i32, vp, i32, i32, i32, i32, vp, vp, vp, sz, vp]
        L.moe_permute_workspace_size.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
        L.moe_permute.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_gmm_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
        L.moe_gmm.argtypes = [vp, i32, i32, vp, vp, i32, i32, vp, vp, i32, i32, i32, i32, i32, vp,
                              i32, vp, sz, vp]
        L.moe_gmm_gather.argtypes = [vp, i32, vp, i32, i32, i32, vp, vp, i32, i32, vp, vp, i32, i32,
                                     i32, i32, i32, vp, i32, vp, sz, vp]
        L.moe_gmm_scatter.argtypes = [vp, i32, i32, vp, vp, i32, i32, vp, vp, i32, i32, i32, i32, i32,
                                      vp, vp, vp, i32, vp, sz, vp]
        L.moe_gmm_routed_shared.argtypes = [vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp,
                                            vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]
        L.moe_gmm_mx_routed_shared.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp,
                                               vp, i32, i32, i32, i32, i32, vp, vp]
        L.moe_gmm_mx.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]
        L.moe_gmm_mxfp4.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]
        L.moe_combine.argtypes = [vp, i32, vp, vp, i32, i32, i32, vp, i32, vp]
        L.moe_sum_slots.argtypes = [vp, i32, i32, i32, i32, vp, vp]
        L.moe_quant_rows.argtypes = [vp, i32, i32, i32, vp, i32, i32, vp, vp, vp]
        L.moe_layer_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
        L.moe_layer.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp,
                                vp, vp, sz, vp]
        L.moe_layer_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp,
                                        vp, vp]
        L.moe_layer_fp8_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
        L.moe_layer_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp,
                                    vp, sz, vp]
        L.moe_fetch_probe.argtypes = [vp, sz, i32, i32, i32, vp, vp]
        L.moe_mfma_probe.argtypes = [i32, i32, vp, vp, vp]
        for n in EXPORTS[2:]:
            getattr(L, n).restype = i32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != OK:
        raise MoeError(status, where)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else None


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


# ---------------------------------------------------------------- entry points

def route_workspace_size(T, H, E, K, dt) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_route_workspace_size(T, H, E, K, dt, ctypes.byref(n)), "moe_route_workspace_size")
    return n.value


def route(x, w_router, K, bias=None, topk_idx=None, topk_gate=None, ws=None, stream=None):
    """moe_route. Returns (topk_idx int32 (T,K), topk_gate fp32 (T,K)). ws: a device
    buffer of at least route_workspace_size() bytes, allocated here when None."""
    T, H = x.shape
    E = w_router.shape[1]
    dt = dtype_code(x)
    if topk_idx is None:
        topk_idx = _empty((T, K), torch.int32, x)
    if topk_gate is None:
        topk_gate = _empty((T, K), torch.float32, x)
    if ws is None:
        n = route_workspace_size(T, H, E, K, dt)
        ws = _empty((n,), torch.uint8, x) if n else None
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    st = lib().moe_route(_ptr(x), _ptr(w_router), dt, _ptr(bias), T, H, E, K,
                         _ptr(topk_idx), _ptr(topk_gate), _ptr(ws), nbytes, _stream(stream))
    _check(st, "moe_route")
    return topk_idx, topk_gate


def permute_workspace_size(T, E, K) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_permute_workspace_size(T, E, K, ctypes.byref(n)), "moe_permute_workspace_size")
    return n.value


def permute(topk_idx, E, x=None, ws=None, stream=None, out=None):
    """moe_permute. Returns dict counts, offsets, perm_src, perm_dst, x_perm (or None)."""
    T, K = topk_idx.shape
    A = T * K
    dev = topk_idx
    o = dict(out or {})
    counts = o.get("counts", _empty((E,), torch.int32, dev))
    offsets = o.get("offsets", _empty((E + 1,), torch.int32, dev))
    psrc = o.get("perm_src", _empty((A,), torch.int32, dev))
    pdst = o.get("perm_dst", _empty((A,), torch.int32, dev))
    xp = None
    H, dt = 1, F32
    if x is not None:
        H = x.shape[1]
        dt = dtype_code(x)
        xp = o.get("x_perm", _empty((A, H), x.dtype, dev))
    need = permute_workspace_size(T, E, K)
    if ws is None and need:
        ws = _empty((need,), torch.uint8, dev)
    st = lib().moe_permute(_ptr(topk_idx), _ptr(x), dt, T, H, E, K, _ptr(counts), _ptr(offsets),
                           _ptr(psrc), _ptr(pdst), _ptr(xp), _ptr(ws) if need else None,
                           ws.numel() if (ws is not None and need) else 0, _stream(stream))
    _check(st, "moe_permute")
    return {"counts": counts, "offsets": offsets, "perm_src": psrc, "perm_dst": pdst, "x_perm": xp}


def gmm_workspace_size(a_dt, e, A, Hin, N) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_gmm_workspace_size(a_dt, e, A, Hin, N, ctypes.byref(n)), "moe_gmm_workspace_size")
    return n.value


def gmm(a, w, offsets, act=ACT_NONE, a_scale=None, w_scale=None, out=None, ws=None, stream=None,
        rows=None, row_div=1, dst=None, gate=None, per_token=False):
    """moe_gmm over w (e,Hin,N). Scales (1-element fp32 device tensors) select
    MOE_QUANT_PER_TENSOR. Output: fp32 for fp32 inputs, else bf16. ws: a device
    buffer of at least gmm_workspace_size() bytes, allocated here when None.
    rows (int32 device tensor, one entry per grouped row): moe_gmm_gather, grouped
    row r is row rows[r] // row_div of a. dst (int32, one entry per grouped row):
    moe_gmm_scatter, grouped row r is stored as out row dst[r], times gate[dst[r]]
    when gate (fp32) is given. per_token: a_scale holds one fp32 per row of a
    (MOE_QUANT_PER_TOKEN, E4M3 activations)."""
    if dst is not None and rows is not None:
        raise ValueError("gather (rows) and scatter (dst) are separate entry points")
    A, Hin = a.shape
    if rows is not None:
        A = rows.numel()
    e, Hw, N = w.shape
    if Hw != Hin:
        raise ValueError("a and w disagree on Hin")
    adt, wdt = dtype_code(a), dtype_code(w)
    odt = F32 if adt == F32 else BF16
    if out is None:
        out = _empty((A, N), torch.float32 if odt == F32 else torch.bfloat16, a)
    if ws is None:
        n = gmm_workspace_size(adt, e, A, Hin, N)
        ws = _empty((n,), torch.uint8, a) if n else None
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    aq = QUANT_PER_TENSOR if a_scale is not None else QUANT_NONE
    if per_token:
        aq = QUANT_PER_TOKEN
    wq = QUANT_PER_TENSOR if w_scale is not None else QUANT_NONE
    if dst is not None:
        st = lib().moe_gmm_scatter(_ptr(a), adt, aq, _ptr(a_scale), _ptr(w), wdt, wq, _ptr(w_scale),
                                   _ptr(offsets), e, A, Hin, N, act, _ptr(dst), _ptr(gate), _ptr(out),
                                   odt, _ptr(ws), nbytes, _stream(stream))
        _check(st, "moe_gmm_scatter")
        return out
    if rows is not None:
        st = lib().moe_gmm_gather(_ptr(a), a.shape[0], _ptr(rows), row_div, adt, aq, _ptr(a_scale),
                                  _ptr(w), wdt, wq, _ptr(w_scale), _ptr(offsets), e, A, Hin, N, act,
                                  _ptr(out), odt, _ptr(ws), nbytes, _stream(stream))
        _check(st, "moe_gmm_gather")
        return out
    st = lib().moe_gmm(_ptr(a), adt, aq, _ptr(a_scale), _ptr(w), wdt, wq, _ptr(w_scale),
                       _ptr(offsets), e, A, Hin, N, act, _ptr(out), odt, _ptr(ws), nbytes,
                       _stream(stream))
    _check(st, "moe_gmm")
    return out


def gmm_routed_shared(a, w, offsets, a_scale, w_scale, xs, ws_w, offsets_s, act=ACT_NONE, act_s=ACT_NONE,
                      dst=None, gate=None, per_token=False, out=None, ys=None, stream=None):
    """moe_gmm_routed_shared: the E4M3 grouped GEMM over w (e,Hin,N) (per-tensor
    scales, or per_token: one a_scale per row of a; stored through dst, times
    gate, when dst is given) and the bf16 grouped GEMM xs @ ws_w (e_s,Hs,Ns)
    over offsets_s in one launch. Returns (out, ys), both bf16."""
    A, Hin = a.shape
    e, Hw, N = w.shape
    T, Hs = xs.shape
    e_s, Hw2, Ns = ws_w.shape
    if Hw != Hin or Hw2 != Hs:
        raise ValueError("activations and weights disagree on the reduction size")
    if out is None:
        out = _empty((A, N), torch.bfloat16, a)
    if ys is None:
        ys = _empty((T, Ns), torch.bfloat16, xs)
    aq = QUANT_PER_TOKEN if per_token else QUANT_PER_TENSOR
    st = lib().moe_gmm_routed_shared(_ptr(a), aq, _ptr(a_scale), _ptr(w), _ptr(w_scale), _ptr(offsets), e, A,
                                     Hin, N, act, _ptr(dst), _ptr(gate), _ptr(out), _ptr(xs), _ptr(ws_w),
                                     _ptr(offsets_s), e_s, T, Hs, Ns, act_s, _ptr(ys), _stream(stream))
    _check(st, "moe_gmm_routed_shared")
    return out, ys


def gmm_mx_routed_shared(a, a_scale, w, w_scale, offsets, xs, ws_w, offsets_s, fp4=False, act=ACT_NONE,
                         act_s=ACT_NONE, out=None, ys=None, stream=None):
    """moe_gmm_mx_routed_shared: gmm_mx (fp4 False) or gmm_mxfp4 (fp4 True)
    and the bf16 grouped GEMM xs @ ws_w (e_s,Hs,Ns) over offsets_s in one
    launch. Returns (out, ys), both bf16."""
    A, Hb = a.shape
    Hin = 2 * Hb if fp4 else Hb
    e, Hw, N = w.shape
    T, Hs = xs.shape
    e_s, Hw2, Ns = ws_w.shape
    if Hw != Hb or Hw2 != Hs:
        raise ValueError("activations and weights disagree on the reduction size")
    if out is None:
        out = _empty((A, N), torch.bfloat16, a)
    if ys is None:
        ys = _empty((T, Ns), torch.bfloat16, xs)
    st = lib().moe_gmm_mx_routed_shared(_ptr(a), _ptr(a_scale), _ptr(w), _ptr(w_scale), _ptr(offsets), e, A, Hin,
                                        N, act, int(bool(fp4)), _ptr(out), _ptr(xs), _ptr(ws_w), _ptr(offsets_s),
                                        e_s, T, Hs, Ns, act_s, _ptr(ys), _stream(stream))
    _check(st, "moe_gmm_mx_routed_shared")
    return out, ys


def gmm_mx(a, a_scale, w, w_scale, offsets, act=ACT_NONE, out=None, stream=None):
    """moe_gmm_mx: E4M3 a (A,Hin) and w (e,Hin,N) with E8M0 block scales a_scale
    (slice-major, (Hin/128, A, 4)) and w_scale (e,Hin/32,N) (uint8 device
    tensors); bf16 output."""
    A, Hin = a.shape
    e, Hw, N = w.shape
    if Hw != Hin:
        raise ValueError("a and w disagree on Hin")
    if out is None:
        out = _empty((A, N), torch.bfloat16, a)
    st = lib().moe_gmm_mx(_ptr(a), _ptr(a_scale), _ptr(w), _ptr(w_scale), _ptr(offsets), e, A, Hin, N,
                          act, _ptr(out), _stream(stream))
    _check(st, "moe_gmm_mx")
    return out


def gmm_mxfp4(a, a_scale, w, w_scale, offsets, act=ACT_NONE, out=None, stream=None):
    """moe_gmm_mxfp4: E2M1 a (A, Hin/2) and w (e, Hin/2, N) packed bytes (two
    values per byte along Hin), E8M0 scales a_scale (slice-major, (Hin/256, A,
    8)) and w_scale (e, Hin/32, N) (uint8 device tensors); bf16 output."""
    A, Hh = a.shape
    e, Hw, N = w.shape
    if Hw != Hh:
        raise ValueError("a and w disagree on Hin")
    if out is None:
        out = _empty((A, N), torch.bfloat16, a)
    st = lib().moe_gmm_mxfp4(_ptr(a), _ptr(a_scale), _ptr(w), _ptr(w_scale), _ptr(offsets), e, A, 2 * Hh, N,
                             act, _ptr(out), _stream(stream))
    _check(st, "moe_gmm_mxfp4")
    return out


def combine(y_perm, perm_dst, topk_gate, T, K, out=None, stream=None):
    """moe_combine: weighted sum (gate given) -> (T,N); Unpermute (gate None) -> (T*K,N)."""
    N = y_perm.shape[1]
    dt = dtype_code(y_perm)
    if out is None:
        shape = (T, N) if topk_gate is not None else (T * K, N)
        out = _empty(shape, y_perm.dtype, y_perm)
    st = lib().moe_combine(_ptr(y_perm), dt, _ptr(perm_dst), _ptr(topk_gate), T, K, N, _ptr(out),
                           dt, _stream(stream))
    _check(st, "moe_combine")
    return out


def quant_rows(x, rows=None, row_div=1, n_out=None, q=None, scale=None, stream=None):
    """moe_quant_rows: per-token dynamic E4M3 quantisation of x (f32/bf16,
    (x_rows,H)); output row r quantises x[rows[r] // row_div] (or x[r]).
    Returns (codes (R,H) float8_e4m3fn, scales (R,) fp32)."""
    x_rows, H = x.shape
    R = (rows.numel() if rows is not None else x_rows) if n_out is None else n_out
    if q is None:
        q = _empty((R, H), torch.float8_e4m3fn, x)
    if scale is None:
        scale = _empty((R,), torch.float32, x)
    st = lib().moe_quant_rows(_ptr(x), dtype_code(x), x_rows, H, _ptr(rows), row_div, R, _ptr(q), _ptr(scale),
                              _stream(stream))
    _check(st, "moe_quant_rows")
    return q, scale


def sum_slots(z, T, K, out=None, stream=None):
    """moe_sum_slots: y[t] = sum_k z[t*K+k] for z (T*K,N) -> (T,N)."""
    N = z.shape[1]
    dt = dtype_code(z)
    if out is None:
        out = _empty((T, N), z.dtype, z)
    _check(lib().moe_sum_slots(_ptr(z), dt, T, K, N, _ptr(out), _stream(stream)), "moe_sum_slots")
    return out


def layer_workspace_size(T, H, E, K, F, dtype_code_) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_layer_workspace_size(T, H, E, K, F, dtype_code_, ctypes.byref(n)),
           "moe_layer_workspace_size")
    return n.value


def layer(x, w_router, w1, w2, K, bias=None, act=ACT_RELU, y=None, ws=None, topk_idx=None,
          topk_gate=None, counts=None, stream=None):
    """moe_layer: route -> permute -> GEMM1(act) -> GEMM2 -> weighted combine. Returns y."""
    T, H = x.shape
    E, _, F = w1.shape
    dt = dtype_code(x)
    if y is None:
        y = torch.empty_like(x)
    need = layer_workspace_size(T, H, E, K, F, dt)
    if ws is None:
        ws = _empty((max(need, 1),), torch.uint8, x)
    st = lib().moe_layer(_ptr(x), _ptr(w_router), _ptr(bias), _ptr(w1), _ptr(w2), dt, T, H, E, K, F,
                         act, _ptr(y), _ptr(topk_idx), _ptr(topk_gate), _ptr(counts), _ptr(ws),
                         ws.numel(), _stream(stream))
    _check(st, "moe_layer")
    return y


def layer_noalloc(x, w_router, w1, w2, K, bias=None, act=ACT_RELU, y=None, topk_idx=None, topk_gate=None,
                  counts=None, stream=None):
    """moe_layer_noalloc: moe_layer with its scratch in the library's static
    device buffer (no workspace argument, nothing allocated by the call
    itself beyond y when y is None). Returns y."""
    T, H = x.shape
    E, _, F = w1.shape
    dt = dtype_code(x)
    if y is None:
        y = torch.empty_like(x)
    st = lib().moe_layer_noalloc(_ptr(x), _ptr(w_router), _ptr(bias), _ptr(w1), _ptr(w2), dt, T, H, E, K, F,
                                 act, _ptr(y), _ptr(topk_idx), _ptr(topk_gate), _ptr(counts), _stream(stream))
    _check(st, "moe_layer_noalloc")
    return y


def layer_fp8_workspace_size(T, H, E, K, F) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_layer_fp8_workspace_size(T, H, E, K, F, ctypes.byref(n)), "moe_layer_fp8_workspace_size")
    return n.value


def layer_fp8(x, w_router, w1, w1_scale, w2, w2_scale, K, bias=None, act=ACT_RELU, y=None, ws=None,
              topk_idx=None, topk_gate=None, counts=None, stream=None):
    """moe_layer_fp8: bf16 tokens x (T,H) and router (H,E); E4M3 experts w1
    (E,H,F), w2 (E,F,H) with one fp32 device scale each; bf16 y (T,H)."""
    T, H = x.shape
    E = w_router.shape[1]
    F = w1.shape[2]
    if y is None:
        y = _empty((T, H), torch.bfloat16, x)
    if ws is None:
        ws = _empty((layer_fp8_workspace_size(T, H, E, K, F),), torch.uint8, x)
    st = lib().moe_layer_fp8(_ptr(x), _ptr(w_router), _ptr(bias), _ptr(w1), _ptr(w1_scale), _ptr(w2),
                             _ptr(w2_scale), T, H, E, K, F, act, _ptr(y), _ptr(topk_idx), _ptr(topk_gate),
                             _ptr(counts), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "moe_layer_fp8")
    return y


def fetch_probe(buf, mode, shared_window, kb_per_wave, stream=None, cycles=None):
    """moe_fetch_probe over the uint8 device tensor buf (mode 0: LDS DMA, 1:
    vector loads). Returns the per-compute-unit s_memtime ticks (int64
    device tensor, one entry per CU; pass `cycles` to reuse one, so that a
    timed call launches nothing else) and the bytes each CU read; time the
    call with stream events for a rate."""
    ncu = torch.cuda.get_device_properties(buf.device).multi_processor_count
    if cycles is None:
        cycles = torch.zeros((ncu,), dtype=torch.int64, device=buf.device)
    elif cycles.numel() != ncu or cycles.dtype != torch.int64 or cycles.device != buf.device:
        raise ValueError("cycles must be an int64 tensor of one entry per compute unit on buf's device")
    _check(lib().moe_fetch_probe(_ptr(buf), buf.numel(), mode, 1 if shared_window else 0, kb_per_wave,
                                 _ptr(cycles), _stream(stream)), "moe_fetch_probe")
    return cycles, 8 * kb_per_wave * 1024


def mfma_probe(fp8, iters, device="cuda", stream=None, cycles=None, sink=None):
    """moe_mfma_probe: per-CU s_memtime ticks (int64 device tensor) and the
    flops each CU issued; pass `cycles` (int64, one per CU) and `sink`
    (float32, 512 per CU) to reuse them, so that a timed call launches
    nothing else; time the call with stream events for a rate."""
    ncu = torch.cuda.get_device_properties(torch.device(device)).multi_processor_count
    if cycles is None:
        cycles = torch.zeros((ncu,), dtype=torch.int64, device=device)
    if sink is None:
        sink = torch.empty((ncu * 512,), dtype=torch.float32, device=device)
    if cycles.numel() != ncu or cycles.dtype != torch.int64 or sink.numel() < ncu * 512 or sink.dtype != torch.float32:
        raise ValueError("cycles: int64, one per compute unit; sink: float32, 512 per compute unit")
    _check(lib().moe_mfma_probe(FP8_E4M3 if fp8 else BF16, iters, _ptr(sink), _ptr(cycles), _stream(stream)),
           "moe_mfma_probe")
    return cycles, 8 * 8 * iters * (131072 if fp8 else 16384)
