/*
 * moe_oracle.h — plain, slow, fp64 CPU oracle of the single-GPU
 * mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link,
 * load or call this code: only tests/, the smoke check and the CPU baseline
 * leg of the benchmark do. It shares no source, header, table or helper with
 * the HIP library; the two only ever see the same input bytes.
 *
 * What it computes, and where the pages define it:
 *   - MoE output  y = sum_i g_i(x) * E_i(x)
 *       ("稀疏矩阵乘法（SpMM）在大模型中的复兴", section "MoE 模型与专家选择的挑战").
 *   - Router: one score per expert from the token embedding and the router
 *     weights, keep the top-k, softmax over the kept scores only
 *       ("Advanced GPU Optimization ... Part 5", section 1.1 "The Router
 *        Kernel (Top-k Gating)"; top-K index matrix (N,K) and binary
 *        activation mask (N,E) from the SpMM page, section "专家选择的计算过程").
 *   - Dispatch into per-expert contiguous blocks ("Part 5", section 1.2,
 *     "Token dispatch"); per-expert counts as in the counts arrays of
 *     "aclnnQuantGroupedMatMulAlltoAllv" (parameter constraints).
 *   - Grouped GEMM with per-tensor scales  gmmY = (gmmX @ gmmWeight) *
 *     gmmXScale * gmmWeightScale, and Unpermute
 *       ("aclnnQuantGroupedMatMulAlltoAllv", section 计算公式), and with MX
 *     (block-scaled) operands, the page's other supported quantisation.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - ties in top-k go to the lower expert index; the k slots are ordered by
 *     descending score;
 *   - the softmax is max-subtracted, no temperature;
 *   - the optional router bias is added before both selection and softmax;
 *   - the expert FFN is act(x . W1[e]) . W2[e] with no biases;
 *   - the hidden activation is kept in fp64 here (also where it is
 *     quantised per row before the second GEMM);
 *   - the scaled GEMM applies the activation after the scales:
 *     act(acc * xScale * wScale);
 *   - rows are placed stably: inside one expert's block, rows appear in
 *     ascending (token, slot) order.
 *
 * All arithmetic is fp64 on values decoded exactly from the input bytes.
 * Every function returns 0 on success and a negative value on bad arguments.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element encodings the oracle can read. */
#define ORC_F32 0  /* IEEE binary32 */
#define ORC_BF16 1 /* bfloat16: the top 16 bits of a binary32 */
#define ORC_E4M3 2 /* OCP 8-bit float E4M3 "fn": bias 7, no inf, 0x7f/0xff NaN */
#define ORC_F64 3  /* IEEE binary64 (oracle-internal intermediates) */

#define ORC_ACT_NONE 0
#define ORC_ACT_RELU 1

/* Exact value of element i of a buffer of encoding dt. */
double orc_decode(const void* buf, int dt, int64_t i);
/* Decode n elements into fp64. */
int orc_decode_array(const void* buf, int dt, int64_t n, double* out);
/* Nearest bfloat16 value to v, ties to even (as fp64), and its bit pattern. */
double orc_round_bf16(double v);
uint16_t orc_bf16_bits(double v);

/* O1-O3: router scores, top-k by a full sort, softmax over the kept k.
 *   x (T,H) and wr (H,E) row-major in encoding dt; bias (E) fp32 or NULL.
 *   topk_idx (T,K): descending score, ties -> lower index.
 *   topk_gate (T,K): g_k = exp(l_k - l_0) / sum_j exp(l_j - l_0).
 *   logits (T,E) and gap (T) are optional outputs; gap[t] is the k-th minus
 *   the (k+1)-th largest score (+inf when K == E). */
int orc_route(const void* x, const void* wr, int dt, const float* bias, int T, int H, int E, int K,
              int32_t* topk_idx, double* topk_gate, double* logits, double* gap);
/* The same scores, with the K experts of each token taken from `given`
 * (T,K) instead of the sort (each index in [0,E), else -1): the gates are O3
 * over the given experts' scores in the given slot order, and gap is still
 * that of the full sort. Used to evaluate a selection made elsewhere on
 * tokens whose k-th and (k+1)-th scores nearly tie. */
int orc_route_given(const void* x, const void* wr, int dt, const float* bias, int T, int H, int E, int K,
                    const int32_t* given, int32_t* topk_idx, double* topk_gate, double* logits,
                    double* gap);

/* O4-O5: counts[E], offsets[E+1] (exclusive scan), and the stable row map.
 *   perm_src[row] = t*K + k ; perm_dst[t*K + k] = row. */
int orc_permute(const int32_t* topk_idx, int T, int E, int K, int32_t* counts, int32_t* offsets,
                int32_t* perm_src, int32_t* perm_dst);

/* O6: xp[row] = x[perm_src[row] / K], byte copy of row_bytes per row. */
int orc_gather_rows(const void* x, int64_t row_bytes, const int32_t* perm_src, int A, int K, void* xp);

/* O7: grouped GEMM. Row r belongs to the expert ex with
 * offsets[ex] <= r < offsets[ex+1];
 *   out[r, n] = act( (sum_h a[r,h] * w[ex,h,n]) * a_scale * w_scale ).
 * a (A,Hin) in a_dt, w (e,Hin,N) row-major (N contiguous) in w_dt.
 * rows == NULL computes every row 0..offsets[e]-1 into out (A,N);
 * otherwise the nrows listed rows, in list order, into out (nrows,N).
 * nthreads > 1 splits the rows over threads (each output is computed
 * by one thread in the same order). */
int orc_gmm(const void* a, int a_dt, double a_scale, const void* w, int w_dt, double w_scale,
            const int32_t* offsets, int e, int Hin, int N, int act, const int32_t* rows, int nrows,
            double* out, int nthreads);

/* Grouped GEMM on MX block-scaled operands: every 32 consecutive reduction
 * elements of an activation row (scales a_scale, (A, Hin/32) bytes) and of a
 * weight column (w_scale, (e, Hin/32, N) bytes) share one E8M0 scale
 * 2^(s-127), s = 255 being NaN; out = act(sum over blocks of both scales times
 * the block's dot product). Quant mode 6 (mx) of
 * "aclnnQuantGroupedMatMulAlltoAllv"; block size and scale format are the
 * OCP MX reading. Hin must be a multiple of 32. */
double orc_e8m0(int s);
int orc_gmm_mx(const void* a, int a_dt, const uint8_t* a_scale, const void* w, int w_dt,
               const uint8_t* w_scale, const int32_t* offsets, int e, int Hin, int N, int act,
               const int32_t* rows, int nrows, double* out, int nthreads);

/* MX with E2M1 (OCP FP4) elements, packed two per byte along the reduction
 * index (even index in the low nibble): a (A, Hin/2) bytes, w (e, Hin/2, N)
 * bytes (byte (ex, k, n) holds rows 2k and 2k+1 of column n); scales as for
 * orc_gmm_mx. orc_e2m1: value of one 4-bit code (s ee m, bias 1, exponent 0
 * subnormal: m/2; largest 6). */
double orc_e2m1(int code);
int orc_gmm_mx4(const uint8_t* a, const uint8_t* a_scale, const uint8_t* w, const uint8_t* w_scale,
                const int32_t* offsets, int e, int Hin, int N, int act, const int32_t* rows, int nrows,
                double* out, int nthreads);

/* Per-token quantisation to E4M3 (quant modes 3 "pertoken" and 7 "pertoken
 * dynamic" of "aclnnQuantGroupedMatMulAlltoAllv", 量化模式 enumeration; the
 * formula there multiplies gmmX's scale back onto the product, so the codes
 * are the row divided by its scale). The page names the modes and gives no
 * formula; the plain reading taken here:
 *   amax     = max_h |x[t,h]|                          (exact)
 *   scale[r] = amax / 448 rounded to binary32          (448: E4M3's largest value)
 *   q[r,h]   = the E4M3 value nearest to the exact quotient x[t,h] / scale[r],
 *              ties to the even code
 * for output row r with source row t = src ? src[r] / div : r (x_rows rows,
 * H values each, in x_dt: binary32, bfloat16 or binary64). A source row
 * outside [0, x_rows), an all-zero row, or a row whose amax / 448 rounds to
 * zero in binary32 gives codes 0 and scale 0.
 * orc_e4m3_nearest_ratio: the code of the finite E4M3 value nearest to
 * num / den (den > 0 with at most 24 significant bits, e.g. a binary32
 * number), decided by exact comparisons; |num / den| >= 448 gives +-448, NaN
 * 0x7f. orc_e4m3_nearest(v) is the same with den = 1.
 * orc_div448_f32: amax / 448 rounded to the nearest binary32 number. */
uint8_t orc_e4m3_nearest_ratio(double num, double den);
uint8_t orc_e4m3_nearest(float v);
int orc_e4m3_nearest_array(const float* v, int64_t n, uint8_t* out);
float orc_div448_f32(double amax);
int orc_quant_rows(const void* x, int x_dt, int x_rows, int H, const int32_t* src, int div, int rows,
                   uint8_t* q, float* scale);

/* O7 with a per-row activation scale: as orc_gmm with a_scale replaced by
 * a_row_scale[r] for grouped row r (gmmXScale of shape (A,), per-token). */
int orc_gmm_row_scaled(const void* a, int a_dt, const double* a_row_scale, const void* w, int w_dt,
                       double w_scale, const int32_t* offsets, int e, int Hin, int N, int act,
                       const int32_t* rows, int nrows, double* out, int nthreads);

/* O8: combine. gate != NULL: y[t,n] = sum_{k ascending} gate[t,k] * yp[perm_dst[t*K+k], n]
 * (out is (T,N)). gate == NULL: Unpermute, out[t*K+k, n] = yp[perm_dst[t*K+k], n]
 * (out is (T*K,N)). */
int orc_combine(const double* yp, const int32_t* perm_dst, const double* gate, int T, int K, int N,
                double* out);

/* One expert on one token: out[H] = act(x . W1[ex]) . W2[ex], hidden in fp64.
 * x is H fp64 values; w1 (E,H,F), w2 (E,F,H) in dt. */
int orc_expert_ffn(const double* x, const void* w1, const void* w2, int dt, int ex, int H, int F,
                   int act, double* out);

/* O1-O8 on the whole batch: route, permute, gather, GEMM 1 (act), GEMM 2,
 * weighted combine. Outputs other than y are optional. */
int orc_layer(const void* x, const void* wr, const float* bias, const void* w1, const void* w2, int dt,
              int T, int H, int E, int K, int F, int act, double* y, int32_t* topk_idx,
              double* topk_gate, double* gap, int32_t* counts, int nthreads);

/* Per-token form on a list of tokens: route each listed token, run its K
 * experts with orc_expert_ffn, sum with the gates in slot order.
 * y is (ntok,H); topk_idx/topk_gate (ntok,K) and gap (ntok) optional. */
int orc_layer_tokens(const void* x, const void* wr, const float* bias, const void* w1, const void* w2,
                     int dt, int T, int H, int E, int K, int F, int act, const int32_t* tokens,
                     int ntok, double* y, int32_t* topk_idx, double* topk_gate, double* gap,
                     int nthreads);
/* The same with each listed token's experts given ((ntok,K), as for
 * orc_route_given); NULL given is orc_layer_tokens. */
int orc_layer_tokens_given(const void* x, const void* wr, const float* bias, const void* w1, const void* w2,
                           int dt, int T, int H, int E, int K, int F, int act, const int32_t* tokens,
                           int ntok, const int32_t* given, double* y, int32_t* topk_idx, double* topk_gate,
                           double* gap, int nthreads);

/* O9: dense masked sum, every expert on every token:
 * y[t] = sum_{e<E} m[t,e] * G[t,e] * E_e(x_t), with m the binary activation
 * mask and G the gates scattered to (T,E). Tiny inputs only. */
int orc_layer_dense(const void* x, const void* wr, const float* bias, const void* w1, const void* w2,
                    int dt, int T, int H, int E, int K, int F, int act, double* y);

#ifdef __cplusplus
}
#endif
#endif
