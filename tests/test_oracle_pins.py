"""Pins of the fp64 oracle against things other than itself.

Each check below ties one oracle function to a library routine, a closed
form, an invariant, a special case with a textbook answer, or brute force on
tiny inputs, so that a dropped term, a wrong sign or index, or a transposed
operand in the oracle fails at least one of them. CPU only.
"""
import math

import numpy as np
import pytest
import scipy.sparse
import scipy.special
import torch

import oracle
import synth
from synth import configs


def _dec(a):
    """Independent decode for pins: numpy/torch views, not the oracle's decoder."""
    if a.dtype == np.uint16:
        return synth.bf16_to_f32(a).astype(np.float64)
    return np.asarray(a, np.float64)


# ---------------------------------------------------------------- decoding

def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.decode(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode(codes)
    nan = np.isnan(ref)
    assert nan.sum() == 2  # 0x7f and 0xff
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9


def test_round_bf16_matches_torch_on_binary32_values():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 1e3,
                        rng.standard_normal(2000).astype(np.float32) * 1e-39,  # subnormals
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3.0e38, 0.0],
                                 np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_bits(v.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_bf16_ties_to_even_direct_from_fp64():
    # 1 + 2^-8 is exactly half-way between bf16 neighbours 1 and 1 + 2^-7: even is 1.
    assert oracle.round_bf16(1 + 2 ** -8) == 1.0
    assert oracle.round_bf16(1 + 3 * 2 ** -8) == 1 + 2 * 2 ** -7
    # just above the half-way point must round up (no double rounding through binary32)
    assert oracle.round_bf16(1 + 2 ** -8 + 2 ** -40) == 1 + 2 ** -7


# ---------------------------------------------------------------- generator encoders

def test_synth_bf16_encoder_matches_torch():
    x = synth.normal(123, (50000,), 3.0)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.to_bf16(x), ref)


def test_synth_e4m3_encoder_matches_torch_in_range():
    x = synth.normal(7, (50000,), 100.0)
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(synth.to_e4m3(x, 1.0), ref)


def test_synth_counter_based_prefix_property():
    a = synth.normal(99, (1000,))
    b = synth.normal(99, (300,))
    assert np.array_equal(a[:300], b)
    assert abs(float(a.mean())) < 0.15 and abs(float(a.std()) - 1) < 0.1


def test_random_routing_distinct_and_in_range():
    idx = synth.random_routing(5, 500, 32, 8)
    assert idx.min() >= 0 and idx.max() < 32
    assert all(len(set(r)) == 8 for r in idx.tolist())


# ---------------------------------------------------------------- router

def _tiny(integer=False, **kw):
    return configs.layer_inputs("tiny", integer=integer, **kw)


@pytest.mark.parametrize("integer", [False, True])
def test_route_logits_match_numpy_matmul(integer):
    d = _tiny(integer)
    idx, gate, logits, gap = oracle.route(d["x"], d["wr"], d["T"], d["H"], d["E"], d["K"])
    ref = _dec(d["x"]) @ _dec(d["wr"])
    np.testing.assert_allclose(logits, ref, rtol=1e-12, atol=1e-12)


def test_route_bias_added_before_selection():
    d = _tiny(bias=True)
    _, _, logits_b, _ = oracle.route(d["x"], d["wr"], d["T"], d["H"], d["E"], d["K"], bias=d["bias"])
    _, _, logits, _ = oracle.route(d["x"], d["wr"], d["T"], d["H"], d["E"], d["K"])
    np.testing.assert_allclose(logits_b - logits, np.broadcast_to(d["bias"].astype(np.float64),
                                                                  logits.shape), atol=1e-12)


@pytest.mark.parametrize("integer", [False, True])
@pytest.mark.parametrize("K", [1, 2, 3, 8])
def test_topk_matches_bruteforce_lexsort(integer, K):
    d = _tiny(integer)
    idx, gate, logits, gap = oracle.route(d["x"], d["wr"], d["T"], d["H"], d["E"], K)
    for t in range(d["T"]):
        order = np.lexsort((np.arange(d["E"]), -logits[t]))  # by -score, then index
        assert list(idx[t]) == list(order[:K])
        srt = logits[t][order]
        want_gap = srt[K - 1] - srt[K] if K < d["E"] else math.inf
        assert gap[t] == want_gap


def test_integer_inputs_exercise_ties_lower_index_wins():
    d = _tiny(True)
    idx, _, logits, gap = oracle.route(d["x"], d["wr"], d["T"], d["H"], d["E"], d["K"])
    ties = 0
    for t in range(d["T"]):
        for a in range(d["K"] - 1):
            if logits[t, idx[t, a]] == logits[t, idx[t, a + 1]]:
                assert idx[t, a] < idx[t, a + 1]
                ties += 1
        ties += int(gap[t] == 0)
    assert ties > 0  # the integer variant does contain ties


def test_explicit_tie_goes_to_lower_index():
    H, E, K = 4, 6, 3
    x = np.ones((1, H), np.float32)
    wr = np.zeros((H, E), np.float32)
    wr[:, 4] = 1.0
    wr[:, 1] = 1.0  # experts 1 and 4 tie for first
    wr[:, 5] = 0.5
    idx, gate, _, gap = oracle.route(x, wr, 1, H, E, K)
    assert list(idx[0]) == [1, 4, 5]
    assert gate[0, 0] == gate[0, 1]


def test_gates_sum_to_one_and_k2_closed_form():
    d = _tiny()
    idx, gate, logits, _ = oracle.route(d["x"], d["wr"], d["T"], d["H"], d["E"], 2)
    np.testing.assert_allclose(gate.sum(1), 1.0, atol=1e-15)
    l0 = logits[np.arange(d["T"]), idx[:, 0]]
    l1 = logits[np.arange(d["T"]), idx[:, 1]]
    np.testing.assert_allclose(gate[:, 0], scipy.special.expit(l0 - l1), rtol=1e-14)


def test_gates_k_equals_e_is_full_softmax():
    d = _tiny()
    E = d["E"]
    idx, gate, logits, gap = oracle.route(d["x"], d["wr"], d["T"], d["H"], E, E)
    full = scipy.special.softmax(logits, axis=1)
    for t in range(d["T"]):
        np.testing.assert_allclose(gate[t], full[t][idx[t]], rtol=1e-13)
    assert np.all(np.isinf(gap))


def test_gates_k1_is_one():
    d = _tiny()
    _, gate, _, _ = oracle.route(d["x"], d["wr"], d["T"], d["H"], d["E"], 1)
    assert np.all(gate == 1.0)


# ---------------------------------------------------------------- dispatch

def _check_perm(idx, E, counts, offsets, psrc, pdst):
    T, K = idx.shape
    A = T * K
    assert counts.sum() == A
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(np.sort(psrc), np.arange(A))
    assert np.array_equal(psrc[pdst], np.arange(A))
    assert np.array_equal(pdst[psrc], np.arange(A))
    for e in range(E):
        seg = psrc[offsets[e]:offsets[e + 1]]
        assert np.all(idx.ravel()[seg] == e)
        assert np.all(np.diff(seg) > 0)  # stable: ascending (token, slot)


@pytest.mark.parametrize("integer", [False, True])
def test_permute_invariants_and_csc_of_mask(integer):
    d = _tiny(integer)
    idx, _, _, _ = oracle.route(d["x"], d["wr"], d["T"], d["H"], d["E"], d["K"])
    counts, offsets, psrc, pdst = oracle.permute(idx, d["E"])
    _check_perm(idx, d["E"], counts, offsets, psrc, pdst)
    # the per-expert row blocks are the CSC form of the (T,E) binary activation mask
    T, K = idx.shape
    mask = np.zeros((T, d["E"]))
    mask[np.repeat(np.arange(T), K), idx.ravel()] = 1
    csc = scipy.sparse.csc_matrix(mask)
    csc.sort_indices()
    assert np.array_equal(csc.indptr, offsets)
    assert np.array_equal(csc.indices, psrc // K)


def test_permute_empty_experts_and_skew():
    idx = synth.random_routing(11, 300, 5, 3)
    idx[idx == 2] = 0  # expert 2 now empty
    idx2 = idx.copy()
    counts, offsets, psrc, pdst = oracle.permute(idx2, 7)  # experts 5 and 6 empty too
    assert counts[2] == 0 and counts[5] == 0 and counts[6] == 0
    # duplicates of expert 0 inside a token are still placed stably
    _check_perm(idx2, 7, counts, offsets, psrc, pdst)


def test_permute_rejects_out_of_range_index():
    idx = np.array([[0, 9]], np.int32)
    with pytest.raises(ValueError):
        oracle.permute(idx, 4)


def test_gather_rows_is_bitwise_copy():
    d = _tiny()
    idx, _, _, _ = oracle.route(d["x"], d["wr"], d["T"], d["H"], d["E"], d["K"])
    _, _, psrc, pdst = oracle.permute(idx, d["E"])
    xp = oracle.gather_rows(d["x"], psrc, d["K"])
    for t in range(d["T"]):
        for k in range(d["K"]):
            assert np.array_equal(xp[pdst[t * d["K"] + k]].view(np.uint32),
                                  d["x"][t].view(np.uint32))


# ---------------------------------------------------------------- grouped GEMM

def _offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gmm_single_expert_is_plain_matmul(dt):
    a = synth.normal(1, (37, 50), dtype=dt)
    w = synth.normal(2, (1, 50, 23), dtype=dt)
    out = oracle.gmm(a, w, _offsets([37]))
    np.testing.assert_allclose(out, _dec(a) @ _dec(w)[0], rtol=1e-12, atol=1e-12)


def test_gmm_grouped_matches_per_segment_matmul_with_empty_groups():
    counts = [5, 0, 17, 1, 0, 9]
    off = _offsets(counts)
    a = synth.normal(3, (off[-1], 33), dtype="bf16")
    w = synth.normal(4, (6, 33, 19), dtype="bf16")
    out = oracle.gmm(a, w, off)
    A, W = _dec(a), _dec(w)
    for e in range(6):
        np.testing.assert_allclose(out[off[e]:off[e + 1]], A[off[e]:off[e + 1]] @ W[e], rtol=1e-12,
                                   atol=1e-12)


def test_gmm_transposed_operand_would_fail():
    # square weights whose transpose differs: the wrong orientation is caught
    a = synth.normal(5, (8, 16))
    w = synth.normal(6, (1, 16, 16))
    out = oracle.gmm(a, w, _offsets([8]))
    assert not np.allclose(out, _dec(a) @ _dec(w)[0].T)
    np.testing.assert_allclose(out, _dec(a) @ _dec(w)[0], rtol=1e-12, atol=1e-12)


def test_gmm_relu_and_scales():
    a = synth.normal(7, (12, 20))
    w = synth.normal(8, (2, 20, 9))
    off = _offsets([7, 5])
    plain = oracle.gmm(a, w, off)
    both = oracle.gmm(a, w, off, act=oracle.ACT_RELU, a_scale=0.25, w_scale=3.0)
    np.testing.assert_allclose(both, np.maximum(plain * 0.75, 0), rtol=1e-14, atol=0)


def test_gmm_identity_weights_return_input_exactly():
    a = synth.normal(9, (30, 24), dtype="bf16")
    w = synth.to_bf16(np.broadcast_to(np.eye(24, dtype=np.float32), (3, 24, 24)).copy())
    out = oracle.gmm(a, w, _offsets([10, 0, 20]))
    assert np.array_equal(out, _dec(a))


def test_gmm_e4m3_integer_inputs_exact_with_power_of_two_scales():
    a_f = synth.ints(10, (40, 64), -4, 4)
    w_f = synth.ints(11, (2, 64, 32), -4, 4)
    a_q = synth.to_e4m3(a_f, 1.0)
    w_q = synth.to_e4m3(w_f, 1.0)
    out = oracle.gmm(a_q, w_q, _offsets([25, 15]), a_scale=0.5, w_scale=4.0)
    ref = np.concatenate([a_f[:25].astype(np.float64) @ w_f[0], a_f[25:].astype(np.float64) @ w_f[1]])
    assert np.array_equal(out, ref * 2.0)


# ---- MX (block-scaled) grouped GEMM: quant mode 6 of the CANN interface, read
# as OCP MX: 32-element reduction blocks, E8M0 scale bytes 2^(s-127).

def test_e8m0_decoding():
    for s in range(255):
        assert oracle.e8m0(s) == math.ldexp(1.0, s - 127)
    assert math.isnan(oracle.e8m0(255))


def _mx_ints(seed, counts, Hin, N):
    e = len(counts)
    A = int(sum(counts))
    a_f = synth.ints(seed, (A, Hin), -4, 4)
    w_f = synth.ints(seed + 1, (e, Hin, N), -4, 4)
    return a_f, w_f, synth.to_e4m3(a_f, 1.0), synth.to_e4m3(w_f, 1.0)


def test_gmm_mx_unit_scales_equal_plain_grouped_gemm():
    counts = [25, 0, 15]
    a_f, w_f, a_q, w_q = _mx_ints(20, counts, 64, 24)
    off = _offsets(counts)
    sa = np.full((40, 2), 127, np.uint8)
    sw = np.full((3, 2, 24), 127, np.uint8)
    assert np.array_equal(oracle.gmm_mx(a_q, sa, w_q, sw, off), oracle.gmm(a_q, w_q, off))


def test_gmm_mx_is_the_sum_of_scaled_block_products():
    """Each 32-deep block enters with the scale of its activation row and of its
    weight column: the result equals the sum over blocks of plain grouped GEMMs
    on that block's slice, times 2^(sa-127) 2^(sw-127), exactly (integer
    inputs, power-of-two scales)."""
    counts = [20, 13]
    Hin, N = 96, 10
    a_f, w_f, a_q, w_q = _mx_ints(22, counts, Hin, N)
    off = _offsets(counts)
    rng = np.random.default_rng(23)
    sa = rng.integers(121, 134, size=(33, Hin // 32)).astype(np.uint8)
    sw = rng.integers(121, 134, size=(2, Hin // 32, N)).astype(np.uint8)
    out = oracle.gmm_mx(a_q, sa, w_q, sw, off)
    ref = np.zeros((33, N))
    for ex in range(2):
        r0, r1 = off[ex], off[ex + 1]
        for b in range(Hin // 32):
            blk = a_f[r0:r1, 32 * b:32 * b + 32].astype(np.float64) @ w_f[ex, 32 * b:32 * b + 32]
            ref[r0:r1] += blk * np.exp2(sa[r0:r1, b].astype(np.float64) - 127)[:, None] \
                * np.exp2(sw[ex, b].astype(np.float64) - 127)[None, :]
    assert np.array_equal(out, ref)


def test_gmm_mx_one_scale_moves_one_block_of_one_column():
    counts = [12]
    a_f, w_f, a_q, w_q = _mx_ints(24, counts, 64, 6)
    off = _offsets(counts)
    sa = np.full((12, 2), 127, np.uint8)
    sw = np.full((1, 2, 6), 127, np.uint8)
    base = oracle.gmm_mx(a_q, sa, w_q, sw, off)
    sw2 = sw.copy()
    sw2[0, 1, 4] = 129  # x4 on block 1 of column 4
    out = oracle.gmm_mx(a_q, sa, w_q, sw2, off)
    blk1 = a_f[:, 32:].astype(np.float64) @ w_f[0, 32:, 4]
    assert np.array_equal(np.delete(out, 4, axis=1), np.delete(base, 4, axis=1))
    assert np.array_equal(out[:, 4], base[:, 4] + 3 * blk1)
    sa2 = sa.copy()
    sa2[7, 0] = 255  # NaN scale poisons that row only
    nan_out = oracle.gmm_mx(a_q, sa2, w_q, sw, off)
    assert np.isnan(nan_out[7]).all() and not np.isnan(np.delete(nan_out, 7, axis=0)).any()


def test_gmm_mx_recipe_roundtrip_close_to_source():
    """The MX input recipe reproduces the fp32 source to within 2^-3 of the
    largest magnitude: half an E4M3 step (2^-4 relative) below 1.75 * 2^8 times
    the block scale, and saturation at 448 (at most 1/8 of a block maximum in
    [1.75, 2) * 2^(e+8)) above it."""
    x = synth.normal(25, (16, 128))
    q, sc = synth.quantize_mx(x, axis=1)
    qv = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()  # torch's E4M3 decoder
    deq = qv.reshape(16, 4, 32) * np.exp2(sc.astype(np.float64) - 127)[..., None]
    err = np.abs(deq.reshape(16, 128) - x).max() / np.abs(x).max()
    assert err <= 2.0 ** -3


def test_gmm_row_subset_equals_full():
    a = synth.normal(12, (50, 16), dtype="bf16")
    w = synth.normal(13, (3, 16, 8), dtype="bf16")
    off = _offsets([20, 10, 20])
    full = oracle.gmm(a, w, off, nthreads=4)
    rows = np.array([49, 0, 19, 20, 29, 30], np.int32)
    sub = oracle.gmm(a, w, off, rows=rows)
    assert np.array_equal(sub, full[rows])


# ---------------------------------------------------------------- combine

def test_combine_constant_expert_rows_is_dense_gate_matmul():
    """SpMM page: with each expert a constant row B_e, y = G @ B (G the gates in (T,E))."""
    d = _tiny()
    T, E, K, N = d["T"], d["E"], d["K"], 40
    idx, gate, _, _ = oracle.route(d["x"], d["wr"], T, d["H"], E, K)
    counts, offsets, psrc, pdst = oracle.permute(idx, E)
    B = synth.normal(14, (E, N)).astype(np.float64)
    expert_of_row = np.repeat(np.arange(E), counts)
    yp = B[expert_of_row]
    y = oracle.combine(yp, pdst, gate, T, K)
    G = np.zeros((T, E))
    G[np.repeat(np.arange(T), K), idx.ravel()] = gate.ravel()
    np.testing.assert_allclose(y, G @ B, rtol=1e-14, atol=1e-14)


def test_combine_one_hot_gates_is_gather_and_unpermute_is_inverse():
    d = _tiny()
    T, E, K = d["T"], d["E"], d["K"]
    idx, _, _, _ = oracle.route(d["x"], d["wr"], T, d["H"], E, K)
    _, _, psrc, pdst = oracle.permute(idx, E)
    yp = synth.normal(15, (T * K, 12)).astype(np.float64)
    onehot = np.zeros((T, K))
    onehot[:, 1] = 1.0
    y = oracle.combine(yp, pdst, onehot, T, K)
    assert np.array_equal(y, yp[pdst.reshape(T, K)[:, 1]])
    un = oracle.combine(yp, pdst, None, T, K)
    assert np.array_equal(un, yp[pdst])
    # unpermute after the gather of the permuted rows gives back token-major rows
    assert np.array_equal(un[psrc], yp)


# ---------------------------------------------------------------- experts and layer

def test_expert_ffn_matches_numpy():
    d = _tiny()
    xv = d["x"][3].astype(np.float64)
    out = oracle.expert_ffn(xv, d["w1"], d["w2"], 5)
    ref = np.maximum(xv @ d["w1"][5].astype(np.float64), 0) @ d["w2"][5].astype(np.float64)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("integer", [False, True])
def test_layer_sparse_equals_dense_masked_sum(integer):
    d = _tiny(integer)
    res = oracle.layer(d["x"], d["wr"], d["w1"], d["w2"], d["K"], nthreads=2)
    dense = oracle.layer_dense(d["x"], d["wr"], d["w1"], d["w2"], d["K"])
    scale = max(1.0, np.abs(dense).max())
    assert np.abs(res["y"] - dense).max() <= 1e-12 * scale
    toks = np.arange(d["T"], dtype=np.int32)
    pt = oracle.layer_tokens(d["x"], d["wr"], d["w1"], d["w2"], d["K"], toks)
    assert np.abs(pt["y"] - dense).max() <= 1e-12 * scale
    assert np.array_equal(pt["idx"], res["idx"])


def test_layer_identity_experts_return_x():
    d = _tiny()
    w1, w2 = configs.identity_ffn(d["H"], d["E"])
    res = oracle.layer(d["x"], d["wr"], w1, w2, d["K"])
    np.testing.assert_allclose(res["y"], d["x"].astype(np.float64), rtol=0, atol=4e-16 * 8)


def test_layer_integer_variant_hidden_values_are_integers():
    d = _tiny(True)
    res = oracle.layer(d["x"], d["wr"], d["w1"], d["w2"], d["K"])
    counts, offsets, psrc, pdst = oracle.permute(res["idx"], d["E"])
    xp = oracle.gather_rows(d["x"], psrc, d["K"])
    hm = oracle.gmm(xp, d["w1"], offsets, act=oracle.ACT_RELU)
    yp = oracle.gmm(hm, d["w2"], offsets)
    assert np.all(hm == np.round(hm)) and np.abs(yp).max() < 2 ** 24
    np.testing.assert_allclose(oracle.combine(yp, pdst, res["gate"], d["T"], d["K"]), res["y"],
                               rtol=0, atol=0)


def test_layer_skew_bias_forced_empty_experts():
    d = _tiny(bias=True)
    b = np.zeros(d["E"], np.float32)
    b[6:] = -1e4
    res = oracle.layer(d["x"], d["wr"], d["w1"], d["w2"], d["K"], bias=b)
    assert res["counts"][6] == 0 and res["counts"][7] == 0
    assert res["counts"].sum() == d["T"] * d["K"]


# ---- Per-token E4M3 quantisation (quant modes 3 / 7 of the CANN interface):
# nearest E4M3 value with ties to the even code, scale = row amax / 448, all in
# binary32.

def _all_e4m3_values():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.decode(codes)
    finite = ~np.isnan(vals)
    return codes[finite], vals[finite]


def test_e4m3_nearest_matches_torch_in_range():
    """torch's float -> float8_e4m3fn conversion rounds to nearest even; inside
    the finite range the oracle's codes must be the same, also on every exact
    value and on every midpoint between neighbours (the ties)."""
    rng = np.random.default_rng(40)
    mag = np.exp2(rng.uniform(-12, math.log2(448.0), 20000))
    v = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    _, vals = _all_e4m3_values()
    pos = np.unique(vals[vals >= 0])
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[1:] + pos[:-1]) / 2)  # midpoints are exact in binary32
    v = np.concatenate([v, pos.astype(np.float32), mids, -mids])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_nearest(v), ref)


def test_e4m3_nearest_is_the_nearest_value_by_brute_force():
    rng = np.random.default_rng(41)
    v = (rng.standard_normal(3000) * np.exp2(rng.integers(-10, 9, 3000))).astype(np.float32)
    v = v[np.abs(v) < 448]
    codes, vals = _all_e4m3_values()
    got = oracle.decode(oracle.e4m3_nearest(v))
    dist = np.abs(v.astype(np.float64)[:, None] - vals[None, :])
    best = dist.min(axis=1)
    assert np.array_equal(np.abs(got - v.astype(np.float64)), best)
    # ties go to the even code: exactly half-way between 1 and 1.125 (codes 0x38, 0x39)
    assert oracle.e4m3_nearest(np.float32(1.0625)) == 0x38
    assert oracle.e4m3_nearest(np.float32(1.1875)) == 0x3A


def test_e4m3_nearest_saturates_and_keeps_sign():
    v = np.array([448.0, 449.0, 464.0, 1e30, -1e30, -448.0, np.nan, -0.0, -1e-10, 2 ** -10],
                 np.float32)
    got = oracle.e4m3_nearest(v)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x80, 0x80, 0x00]


def test_quant_rows_scale_and_error_bound():
    rng = np.random.default_rng(42)
    x = (rng.standard_normal((64, 300)) * np.exp2(rng.integers(-6, 6, (64, 1)))).astype(np.float32)
    q, s = oracle.quant_rows(x)
    amax = np.abs(x).max(axis=1)
    assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))
    # the largest element of each row lands on +-448
    arg = np.abs(x).argmax(axis=1)
    assert np.all((q[np.arange(64), arg] & 0x7F) == 0x7E)
    # within half a step of the value grid: 2^-4 relative (normal), 2^-10 * scale (subnormal)
    deq = oracle.decode(q) * s[:, None].astype(np.float64)
    ratio = np.abs(x) / s[:, None]
    bound = np.where(ratio >= 2 ** -6, np.abs(x) * 2 ** -4, s[:, None] * 2 ** -10) * (1 + 1e-6)
    assert np.all(np.abs(deq - x) <= bound)


def test_quant_rows_special_cases():
    rng = np.random.default_rng(43)
    x = rng.standard_normal((10, 64)).astype(np.float32)
    x[3] = 0.0
    q, s = oracle.quant_rows(x)
    assert s[3] == 0 and not q[3].any()
    # scaling a row by a power of two scales its scale and keeps its codes
    q2, s2 = oracle.quant_rows(x * np.float32(8.0))
    assert np.array_equal(q2, q) and np.array_equal(s2, s * np.float32(8.0))
    # gathering: output row r quantises source row rows[r] // div; out of range -> zero row
    rows = np.array([5, 0, 19, -1, 40, 7], np.int32)
    qg, sg = oracle.quant_rows(x, rows=rows, div=2)
    src = rows // 2
    for r, t in enumerate(src):
        if 0 <= rows[r] and t < 10:
            assert np.array_equal(qg[r], q[t]) and sg[r] == s[t]
        else:
            assert not qg[r].any() and sg[r] == 0
    # bf16 input: the same as its binary32 values
    xb = synth.to_bf16(x)
    qb, sb = oracle.quant_rows(xb)
    qf, sf = oracle.quant_rows(synth.bf16_to_f32(xb))
    assert np.array_equal(qb, qf) and np.array_equal(sb, sf)


def test_gmm_row_scales():
    """Per-row activation scales: unit scales are the scale-free product, a
    constant is the per-tensor scale, and each row's scale moves only its row."""
    rng = np.random.default_rng(44)
    counts = [5, 0, 9, 3]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    A = int(off[-1])
    a = rng.integers(-3, 4, (A, 48)).astype(np.float32)
    w = rng.integers(-2, 3, (4, 48, 20)).astype(np.float32)
    base = oracle.gmm(a, w, off)
    assert np.array_equal(oracle.gmm(a, w, off, a_scale=np.ones(A)), base)
    assert np.array_equal(oracle.gmm(a, w, off, a_scale=np.full(A, 0.375), w_scale=2.0),
                          oracle.gmm(a, w, off, a_scale=0.375, w_scale=2.0))
    rs = np.ones(A)
    rs[7] = 4.0
    got = oracle.gmm(a, w, off, a_scale=rs, act=oracle.ACT_RELU)
    ref = oracle.gmm(a, w, off, act=oracle.ACT_RELU)
    assert np.array_equal(np.delete(got, 7, axis=0), np.delete(ref, 7, axis=0))
    assert np.array_equal(got[7], 4.0 * ref[7])


# ---- MX with E2M1 (OCP FP4) elements, packed two per byte along the reduction.

def test_e2m1_format_properties():
    vals = np.array([oracle.e2m1(c) for c in range(16)])
    assert np.array_equal(vals[8:], -vals[:8]) and vals[0] == 0.0
    assert np.all(np.diff(vals[:8]) > 0)
    # one mantissa bit per binade above the subnormal code: value(e+1, m) = 2 value(e, m)
    for e in range(1, 3):
        for m in range(2):
            assert vals[2 * (e + 1) + m] == 2 * vals[2 * e + m]
    assert vals[1] == vals[2] / 2  # the subnormal code is half the smallest normal value
    # the input encoder picks the nearest value, ties to the even code, saturating
    rng = np.random.default_rng(50)
    v = rng.uniform(-8, 8, 5000)
    got = np.array([oracle.e2m1(c) for c in synth.to_e2m1(v)])
    dist = np.abs(v[:, None] - vals[None, :])
    assert np.allclose(np.abs(got - v), dist.min(axis=1))


def _e2m1_grid_case(seed, counts, Hin, N):
    rng = np.random.default_rng(seed)
    e = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    A = int(off[-1])
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    af = rng.choice(grid, (A, Hin)) * rng.choice([-1, 1], (A, Hin))
    wf = rng.choice(grid, (e, Hin, N)) * rng.choice([-1, 1], (e, Hin, N))
    a = synth.pack_e2m1(synth.to_e2m1(af), 1)
    w = synth.pack_e2m1(synth.to_e2m1(wf), 1)
    return off, af, wf, a, w


def test_gmm_mx4_unit_scales_equal_numpy_matmul():
    """Grid values with unit scales: the packed FP4 GEMM equals numpy's matmul
    of the unpacked values exactly (this pins the decoding and both packings)."""
    counts = [7, 0, 12, 5]
    off, af, wf, a, w = _e2m1_grid_case(51, counts, 64, 24)
    A, e = af.shape[0], len(counts)
    sa = np.full((A, 2), 127, np.uint8)
    sw = np.full((e, 2, 24), 127, np.uint8)
    out = oracle.gmm_mx4(a, sa, w, sw, off)
    ref = np.concatenate([af[off[i]:off[i + 1]] @ wf[i] for i in range(e)])
    assert np.array_equal(out, ref)


def test_gmm_mx4_block_scales_by_brute_force():
    counts = [5, 9]
    off, af, wf, a, w = _e2m1_grid_case(52, counts, 96, 10)
    A, e, nb = af.shape[0], len(counts), 3
    rng = np.random.default_rng(53)
    sa = rng.integers(120, 135, (A, nb)).astype(np.uint8)
    sw = rng.integers(120, 135, (e, nb, 10)).astype(np.uint8)
    out = oracle.gmm_mx4(a, sa, w, sw, off, act=oracle.ACT_RELU)
    ref = np.zeros((A, 10))
    for r in range(A):
        ex = int(np.searchsorted(off, r, side="right") - 1)
        for b in range(nb):
            dot = af[r, 32 * b:32 * b + 32] @ wf[ex, 32 * b:32 * b + 32]
            ref[r] += 2.0 ** (int(sa[r, b]) - 127) * 2.0 ** (sw[ex, b].astype(int) - 127) * dot
    assert np.allclose(out, np.maximum(ref, 0), rtol=1e-15, atol=0)


def test_quantize_mx4_recipe_roundtrip():
    rng = np.random.default_rng(54)
    x = (rng.standard_normal((16, 128)) * np.exp2(rng.integers(-5, 5, (16, 1)))).astype(np.float32)
    q, sc = synth.quantize_mx4(x, axis=1)
    lo, hi = q & 15, q >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(16, 128)
    vals = np.array([oracle.e2m1(c) for c in range(16)])[codes]
    step = np.repeat(np.exp2(sc.astype(np.float64) - 127), 32, axis=1)
    deq = vals * step
    assert np.all(np.abs(deq - x) <= 0.25 * np.abs(x) + 0.25 * step + 1e-30)


def test_layer_fp8_composition():
    """The E4M3 layer: token subsets give the same rows as the whole batch
    (every step is per token), and the result stays within the fp8 bar of the
    unquantised layer on the same (dequantised) weights."""
    d = configs.layer_fp8_inputs("tiny", T=48)
    full = oracle.layer_fp8(d["x"], d["wr"], d["w1"], d["w1_scale"], d["w2"], d["w2_scale"], d["K"])
    sub = np.array([3, 17, 40, 0])
    part = oracle.layer_fp8(d["x"], d["wr"], d["w1"], d["w1_scale"], d["w2"], d["w2_scale"], d["K"], tokens=sub)
    assert np.array_equal(part["y"], full["y"][sub]) and np.array_equal(part["idx"], full["idx"][sub])
    w1f = (oracle.decode(d["w1"]) * float(d["w1_scale"])).astype(np.float32)
    w2f = (oracle.decode(d["w2"]) * float(d["w2_scale"])).astype(np.float32)
    plain = oracle.layer(synth.bf16_to_f32(d["x"]), synth.bf16_to_f32(d["wr"]), w1f, w2f, d["K"])
    err = np.abs(full["y"] - plain["y"]).max() / np.abs(plain["y"]).max()
    assert err <= 6e-2


def test_gmm_row_scales_on_sampled_rows():
    """Per-row scales follow the grouped row, also when only listed rows are computed."""
    rng = np.random.default_rng(45)
    counts = [6, 3, 9]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    A = int(off[-1])
    a = rng.integers(-3, 4, (A, 32)).astype(np.float32)
    w = rng.integers(-2, 3, (3, 32, 8)).astype(np.float32)
    rs = np.exp2(rng.integers(-2, 3, A)).astype(np.float64)
    full = oracle.gmm(a, w, off, a_scale=rs)
    rows = np.array([17, 2, 9, 0, 11], np.int32)
    assert np.array_equal(oracle.gmm(a, w, off, a_scale=rs, rows=rows), full[rows])


# ---------------------------------------------------------------- per-token quantisation, exact quotient
# The pins below hold the quantiser to its plain definition, scale =
# binary32(amax / 448) and codes = nearest E4M3 value of the exact quotient
# x / scale, by means other than the oracle's own comparisons: exact rational
# arithmetic (fractions), and torch's E4M3 conversion where the quotient is a
# binary32 number.

from fractions import Fraction


def _e4m3_table():
    codes = np.arange(0x7F, dtype=np.uint8)  # 0x00 .. 0x7e: the non-negative finite values
    return codes, [Fraction(float(v)) for v in oracle.decode(codes)]


def _nearest_code_exact(q: Fraction, table) -> int:
    """Code (sign bit clear) of the non-negative finite E4M3 value nearest to
    |q|, by exact distances to all of them; ties to the even code."""
    codes, vals = table
    a = abs(q)
    best, bestd = None, None
    for c, v in zip(codes, vals):
        d = abs(a - v)
        if bestd is None or d < bestd or (d == bestd and int(c) % 2 == 0):
            best, bestd = int(c), d
    return best


def _f32_nearest_exact(q: Fraction) -> np.float32:
    """binary32 number nearest to the rational q (q >= 0), ties to even, from
    exact distances to the binary32 neighbours of a first guess."""
    g = np.float32(float(q))
    cands = [np.nextafter(g, np.float32(-np.inf)), g, np.nextafter(g, np.float32(np.inf))]
    cands = [c for c in cands if c >= 0]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - q), int(np.float32(c).view(np.uint32)) & 1))
    return np.float32(best)


def test_div448_is_correctly_rounded():
    rng = np.random.default_rng(50)
    vals = list(np.abs(rng.standard_normal(300)) * np.exp2(rng.integers(-140, 120, 300)))
    vals += [float(np.float32(v)) for v in vals[:100]]                 # binary32 amax
    vals += [448.0 * float(np.float32(v)) for v in vals[:50]]          # exact quotients
    # amax exactly half-way between 448 s and 448 next(s): ties to even
    for s in np.float32([1.0, 1.5, 3.0e-5, 2.0 ** -130]):
        up = np.nextafter(s, np.float32(np.inf))
        vals.append(float((Fraction(float(s)) + Fraction(float(up))) / 2 * 448))
    # binary64 amax one or two ulps from such a tie (the fp64 hidden rows of
    # the E4M3 layer are binary64)
    for s in np.float32(rng.uniform(1, 2, 200) * np.exp2(rng.integers(-60, 60, 200))):
        up = np.nextafter(s, np.float32(np.inf))
        tie = float((Fraction(float(s)) + Fraction(float(up))) / 2 * 448)
        for step in (-2, -1, 1, 2):
            v = tie
            for _ in range(abs(step)):
                v = np.nextafter(v, np.inf if step > 0 else -np.inf)
            vals.append(float(v))
    for v in vals:
        assert oracle.div448_f32(v) == _f32_nearest_exact(Fraction(v) / 448), v


def test_quant_rows_codes_are_nearest_to_the_exact_quotient():
    """Random rows, rows with a subnormal or vanishing scale, and elements
    placed on and next to every E4M3 midpoint times the row's scale (where a
    quotient formed in binary32 arithmetic can round to the wrong side): each
    code is the E4M3 value nearest to x / scale in exact rational arithmetic."""
    rng = np.random.default_rng(51)
    table = _e4m3_table()
    pos = np.unique(oracle.decode(np.arange(0x7F, dtype=np.uint8)))
    mids = (pos[1:] + pos[:-1]) / 2
    rows = []
    for k in range(6):
        r = (rng.standard_normal(64) * np.exp2(rng.integers(-20, 20))).astype(np.float32)
        s = np.float32(oracle.div448_f32(float(np.abs(r).max())))
        # the binary32 numbers nearest to midpoint * scale, and their neighbours
        m = rng.choice(mids, 20)
        sign = rng.choice([-1.0, 1.0], 20)
        near = np.float32(m * float(s) * sign)
        extra = np.concatenate([near, np.nextafter(near, np.float32(np.inf)),
                                np.nextafter(near, np.float32(-np.inf))])
        rows.append(np.concatenate([r, extra[np.abs(extra) < np.abs(r).max()]]))
    tiny = (rng.standard_normal(40) * 1e-37).astype(np.float32)        # subnormal scale
    rows.append(tiny)
    rows.append(np.float32([1e-45, -1e-45, 0.0] + [0.0] * 5))          # amax / 448 rounds to 0
    rows.append(np.float32([448.0 * 2.0 ** -140, 3.0 * 2.0 ** -149, -2.0 ** -145] + [0.0] * 5))
    Hmax = max(r.size for r in rows)
    x = np.zeros((len(rows), Hmax), np.float32)
    for i, r in enumerate(rows):
        x[i, :r.size] = r
    q, s = oracle.quant_rows(x)
    for i in range(x.shape[0]):
        amax = np.abs(x[i]).max()
        assert s[i] == _f32_nearest_exact(Fraction(float(amax)) / 448)
        if s[i] == 0:
            assert not q[i].any()
            continue
        for h in range(Hmax):
            want = _nearest_code_exact(Fraction(float(x[i, h])) / Fraction(float(s[i])), table)
            if x[i, h] < 0 or (x[i, h] == 0 and np.signbit(x[i, h])):
                want |= 0x80
            assert q[i, h] == want, (i, h, x[i, h], s[i])
    assert s[-2] == 0 and s[-1] > 0 and not np.isnan(oracle.decode(q)).any()


def test_quant_rows_codes_equal_torch_where_the_quotient_is_binary32():
    """Rows whose scale is a power of two (amax = 448 * 2^k): the quotient
    x / scale is a binary32 number, so torch's binary32 -> float8_e4m3fn
    conversion (round to nearest even) gives the exact answer; elsewhere
    torch's conversion of the binary32-rounded quotient agrees except where a
    midpoint lies within one binary32 rounding, where the oracle's code is one
    of the two neighbours."""
    rng = np.random.default_rng(52)
    x = rng.standard_normal((40, 256)).astype(np.float32)
    k = rng.integers(-30, 30, 40)
    x /= np.abs(x).max(axis=1, keepdims=True)
    x = (x * np.float32(448.0) * np.exp2(k)[:, None]).astype(np.float32)
    pw = np.abs(x).max(axis=1) == np.float32(448.0) * np.exp2(k).astype(np.float32)
    q, s = oracle.quant_rows(x)
    assert pw.sum() >= 30
    exact = (x[pw] / s[pw, None]).astype(np.float32)
    assert np.array_equal(exact.astype(np.float64) * s[pw, None].astype(np.float64), x[pw].astype(np.float64))
    ref = torch.from_numpy(exact).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q[pw], ref)
    # general scales: binary32 quotients, compared away from the midpoints
    y = (rng.standard_normal((30, 512)) * np.exp2(rng.integers(-10, 10, (30, 1)))).astype(np.float32)
    qy, sy = oracle.quant_rows(y)
    quo = (y.astype(np.float64) / sy[:, None].astype(np.float64)).astype(np.float32)
    ref = torch.from_numpy(quo).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    differ = qy != ref
    if differ.any():
        lo = np.minimum(oracle.decode(qy[differ]), oracle.decode(ref[differ]))
        hi = np.maximum(oracle.decode(qy[differ]), oracle.decode(ref[differ]))
        mid = (lo + hi) / 2
        assert np.all(np.abs(np.abs(quo[differ]) - np.abs(mid)) <= np.abs(mid) * 2.0 ** -23)
    assert differ.mean() < 1e-3


def test_quant_rows_binary64_input():
    """Binary64 rows (the fp64 hidden activation of the E4M3 layer): the scale
    is amax / 448 rounded once to binary32 and the codes follow the exact
    quotient, also where a binary32 copy of the row would round differently."""
    table = _e4m3_table()
    rng = np.random.default_rng(53)
    x = rng.standard_normal((4, 48))
    x[1, 5] = 448.0 * (1 + 2.0 ** -30)          # amax not a binary32 value
    x[2, :3] = [1.0625 * (1 + 2.0 ** -40), -1.0625 * (1 + 2.0 ** -40), 448.0]   # just past a tie
    q, s = oracle.quant_rows(x)
    for i in range(4):
        amax = Fraction(float(np.abs(x[i]).max()))
        assert s[i] == _f32_nearest_exact(amax / 448)
        for h in range(48):
            want = _nearest_code_exact(Fraction(float(x[i, h])) / Fraction(float(s[i])), table)
            if x[i, h] < 0:
                want |= 0x80
            assert q[i, h] == want
    assert s[2] == 1.0 and q[2, 0] == 0x39 and q[2, 1] == 0xB9  # binary32 would give the tie's even code 0x38
