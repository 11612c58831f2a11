"""Shared test utilities: host <-> device moves and error metrics."""
import numpy as np
import torch

import synth


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy host array -> device tensor. uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev())


def to_host(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy; bf16 comes back as uint16 bit patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return synth.bf16_to_f32(a).astype(np.float64)
    return np.asarray(a, np.float64)


def normwise_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max_i |got_i - ref_i| / max_i |ref_i| (0 when both are all zero)."""
    got = as_f64(got)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(got - ref).max() if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}
GAP = 1e-3


def check_selection(idx, ref_idx, logits, K, gap_tol=GAP):
    """Check a top-K selection made on the GPU against the oracle's fp64
    scores (T,E), on every token:
      - K distinct experts in [0, E);
      - every chosen expert scores at least the K-th largest score - gap_tol
        (a valid top-K up to the tolerance), so where the K-th and (K+1)-th
        scores are more than gap_tol apart the set is the oracle's;
      - slots in descending score order up to gap_tol, and exactly the
        oracle's order on tokens whose selected scores are all more than
        gap_tol apart.
    Returns the mask of tokens whose selection differs from the oracle's (in
    set or order): those are compared against the oracle evaluated with the
    GPU's own selection."""
    idx = np.asarray(idx)
    T, E = logits.shape
    assert idx.shape == (T, K)
    assert ((idx >= 0) & (idx < E)).all()
    if K > 1:
        assert (np.diff(np.sort(idx, axis=1), axis=1) != 0).all()
    chosen = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
    desc = -np.sort(-logits, axis=1)
    kth = desc[:, K - 1]
    assert (chosen >= kth[:, None] - gap_tol).all()
    if K > 1:
        assert (chosen[:, :-1] >= chosen[:, 1:] - gap_tol).all()
    gap = kth - desc[:, K] if K < E else np.full(T, np.inf)
    clear = gap > gap_tol
    assert np.array_equal(np.sort(idx[clear], axis=1), np.sort(ref_idx[clear], axis=1))
    ref_chosen = np.take_along_axis(logits, np.asarray(ref_idx).astype(np.int64), axis=1)
    ordered = clear & ((np.diff(-ref_chosen, axis=1) > gap_tol).all(axis=1) if K > 1 else True)
    assert np.array_equal(idx[ordered], ref_idx[ordered])
    return (idx != ref_idx).any(axis=1)


def layer_check(y, idx, gate, d, ref, tokens=None, tol=None, gate_tol=2e-3, nthreads=8, fp8=False,
                fp8_hidden="f64"):
    """Whole-layer check on every listed token (all tokens when tokens is None):
    the selection by check_selection against the oracle's scores; the gates and
    y against the oracle evaluated with the GPU's own selection wherever it
    differs from the oracle's (near ties), else against ref. Returns the
    normwise error of y and the number of tokens evaluated with the GPU's
    selection."""
    import oracle
    T = d["x"].shape[0]
    K = d["K"]
    E = d["w1"].shape[0]
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    xs = d["x"][toks]
    _, _, logits, _ = oracle.route(xs, d["wr"], len(toks), d["H"], E, K, bias=d["bias"])
    g_idx, g_gate, g_y = np.asarray(idx)[toks], np.asarray(gate)[toks], np.asarray(y)[toks]
    diff = check_selection(g_idx, ref["idx"], logits, K)
    ref_y = np.array(ref["y"], np.float64, copy=True)
    ref_gate = np.array(ref["gate"], np.float64, copy=True)
    if diff.any():
        sel = np.nonzero(diff)[0]
        if fp8:
            alt = oracle.layer_fp8(d["x"], d["wr"], d["w1"], d["w1_scale"], d["w2"], d["w2_scale"], K,
                                   bias=d["bias"], tokens=toks[sel], given=g_idx[sel], hidden=fp8_hidden,
                                   nthreads=nthreads)
        else:
            alt = oracle.layer_tokens(d["x"], d["wr"], d["w1"], d["w2"], K, toks[sel], bias=d["bias"],
                                      given=g_idx[sel], nthreads=nthreads)
        assert np.array_equal(alt["idx"], g_idx[sel])
        ref_y[sel] = alt["y"]
        ref_gate[sel] = alt["gate"]
    assert np.abs(g_gate - ref_gate).max() <= gate_tol
    np.testing.assert_allclose(g_gate.sum(axis=1), 1.0, atol=1e-5)
    err = normwise_err(g_y, ref_y)
    if tol is not None:
        assert err <= tol, f"normwise error {err:.3e} > {tol:.1e}"
    return err, int(diff.sum())
