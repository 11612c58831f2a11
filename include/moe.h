/*
 * moe.h — C ABI of the single-GPU mixture-of-experts layer for MI355X (gfx950).
 *
 * The layer computes, per token x,  y = sum_{k<K} g_k(x) * E_{i_k}(x)
 * (the MoE combination of "稀疏矩阵乘法（SpMM）在大模型中的复兴：利用NVIDIA
 * Sparse Tensor Core加速MoE推理", section "MoE 模型与专家选择的挑战"), where
 * i_k are the K highest-scoring experts of a router and g the softmax over
 * those K scores only ("Advanced GPU Optimization: How to tech an LLM with
 * CUDA and ROCm? - Part 5", section 1.1 "The Router Kernel (Top-k Gating)").
 * It is split into the steps of that page's section 1.2 and of the routed-
 * expert formula of "aclnnQuantGroupedMatMulAlltoAllv" (section 计算公式):
 * route -> permute (dispatch) -> grouped GEMM -> combine / Unpermute.
 *
 * Conventions shared by every entry point
 *   - Pointers marked "device" are HIP device pointers; the caller owns every
 *     buffer. Tensors are dense, row-major, and each device pointer must be
 *     16-byte aligned (else MOE_ERR_MISALIGNED).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *     work is enqueued on it; no call synchronises the host, allocates or
 *     frees memory. Outputs are valid once the stream reaches that point.
 *   - Every argument is validated on the host before anything is enqueued;
 *     a call that returns an error has enqueued nothing and written nothing.
 *     MOE_ERR_DEVICE reports a failed launch (the state of the outputs is then
 *     undefined).
 *   - Results are deterministic: the same inputs give bit-identical outputs
 *     (the op is deterministic by default, as "aclnnQuantGroupedMatMulAlltoAllv"
 *     states in its constraints). No floating-point atomics are used.
 *   - Ranges follow the shape constraints of "aclnnQuantGroupedMatMulAlltoAllv":
 *     H, F, N in (0, 65536); K in [1, 8] (the page gives [2, 8]; K = 1 is
 *     accepted as the g = 1 special case) and K <= E; E <= 256 (its bound on
 *     experts times ranks); T*K < 52428800 (its bound on received rows). The
 *     page's 32-experts-per-card limit is not applied: one GPU here holds
 *     every expert.
 *   - Non-finite inputs give unspecified results.
 *
 * Element types: MOE_F32 = IEEE binary32, MOE_BF16 = bfloat16, MOE_FP8_E4M3 =
 * OCP 8-bit E4M3 ("fn": no infinities, max 448). Activations are rounded to
 * the output type once, round to nearest even.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_VERSION 11200 /* 1.12.0: moe_gmm_routed_shared, moe_gmm_mx_routed_shared */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL_POINTER = 1,        /* a required pointer is NULL */
  MOE_ERR_BAD_SHAPE = 2,           /* a size is out of range or inconsistent */
  MOE_ERR_BAD_DTYPE = 3,           /* an element-type code is unknown or not allowed here */
  MOE_ERR_UNSUPPORTED = 4,         /* a valid mode the library does not implement */
  MOE_ERR_WORKSPACE_TOO_SMALL = 5, /* ws_bytes below the *_workspace_size answer */
  MOE_ERR_MISALIGNED = 6,          /* a device pointer is not 16-byte aligned */
  MOE_ERR_DEVICE = 7,              /* the HIP runtime reported an error */
  MOE_ERR_SCRATCH_LIMIT = 8        /* moe_layer_noalloc: the call needs more than
                                      MOE_NOALLOC_SCRATCH_BYTES of scratch */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/* Quantisation modes, numbered as in "aclnnQuantGroupedMatMulAlltoAllv"
 * (parameter list): 0 none, 1 per-tensor, 2 per-channel, 3 per-token,
 * 4 per-group, 5 per-block, 6 mx, 7 dynamic per-token. moe_gmm and its
 * variants take modes 0 and 1, and mode 3 for the activations of an E4M3
 * product (per-row scales); mode 6 has entry points of its own
 * (moe_gmm_mx, moe_gmm_mxfp4); mode 7 is moe_quant_rows followed by mode 3.
 * Modes 2, 4, 5 and 7 passed to moe_gmm, and mode 3 for the weights or for a
 * product that is not E4M3, return MOE_ERR_UNSUPPORTED. */
typedef enum {
  MOE_QUANT_NONE = 0,
  MOE_QUANT_PER_TENSOR = 1,
  MOE_QUANT_PER_CHANNEL = 2,
  MOE_QUANT_PER_TOKEN = 3,
  MOE_QUANT_PER_GROUP = 4,
  MOE_QUANT_PER_BLOCK = 5,
  MOE_QUANT_MX = 6,
  MOE_QUANT_PER_TOKEN_DYNAMIC = 7
} moe_quant_mode;

typedef enum { MOE_ACT_NONE = 0, MOE_ACT_RELU = 1 } moe_act;

/* Message for a status code (static storage, never NULL). */
const char* moe_status_string(moe_status s);
/* MOE_VERSION of the built library. */
int moe_version(void);

/*
 * moe_route — router scores, top-k selection, softmax over the k kept scores
 * ("Part 5", section 1.1; the (N,K) top-K index matrix of the SpMM page,
 * section "专家选择的计算过程").
 *   x        device (T,H) in dt            token rows
 *   w_router device (H,E) in dt            router weights, E contiguous
 *   dt       MOE_F32 or MOE_BF16
 *   bias     device (E) fp32 or NULL       added to every score before
 *                                          selection and softmax
 *   topk_idx device (T,K) int32 out        experts by descending score; equal
 *                                          scores -> lower expert index first
 *   topk_gate device (T,K) fp32 out        g_k = exp(l_k - l_0) / sum_j exp(l_j - l_0)
 *   ws, ws_bytes device scratch of at least moe_route_workspace_size() bytes
 *                (may be NULL when that size is 0; with few tokens the router
 *                splits H over several blocks and keeps partial scores there)
 * Scores are accumulated in fp32. T = 0 is a no-op. Non-finite inputs are
 * outside the contract: a NaN score counts as -inf for selection, so the
 * indices always hold K distinct experts in [0, E); that token's gates are
 * then unspecified.
 */
moe_status moe_route_workspace_size(int T, int H, int E, int K, moe_dtype dt, size_t* bytes);
moe_status moe_route(const void* x, const void* w_router, moe_dtype dt, const float* bias, int T,
                     int H, int E, int K, int32_t* topk_idx, float* topk_gate, void* ws,
                     size_t ws_bytes, void* stream);

/*
 * moe_permute — dispatch: per-expert counts, their exclusive scan, and a
 * stable placement of the T*K (token, slot) pairs into per-expert contiguous
 * row blocks ("Part 5", section 1.2, token dispatch; the per-expert count
 * arrays of "aclnnQuantGroupedMatMulAlltoAllv"). With one GPU the dispatch
 * buffer is the permuted activation buffer. offsets + perm_src are the CSC
 * form of the (T,E) activation mask of the SpMM page (section "SpMM"/CSC).
 *   topk_idx device (T,K) int32            values must be in [0,E) (out-of-range
 *                                          values give unspecified placement but
 *                                          no out-of-bounds access)
 *   x        device (T,H) in dt or NULL    NULL: index work only
 *   counts   device (E) int32 out
 *   offsets  device (E+1) int32 out        offsets[0] = 0, offsets[E] = T*K
 *   perm_src device (T*K) int32 out        row -> t*K + k
 *   perm_dst device (T*K) int32 out        t*K + k -> row
 *   x_perm   device (T*K,H) in dt out      x_perm[perm_dst[t*K+k]] = x[t]; NULL iff x is
 *   ws, ws_bytes device scratch of at least moe_permute_workspace_size() bytes
 * Rows of one expert appear in ascending (t, k) order (stable, deterministic).
 */
moe_status moe_permute_workspace_size(int T, int E, int K, size_t* bytes);
moe_status moe_permute(const int32_t* topk_idx, const void* x, moe_dtype dt, int T, int H, int E,
                       int K, int32_t* counts, int32_t* offsets, int32_t* perm_src,
                       int32_t* perm_dst, void* x_perm, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_gmm — grouped GEMM over e experts whose rows are contiguous blocks:
 *   out[r, n] = act( (sum_h a[r,h] * w[ex,h,n]) * a_scale * w_scale )
 * for offsets[ex] <= r < offsets[ex+1]  (gmmY = (gmmX @ gmmWeight) * gmmXScale
 * * gmmWeightScale, "aclnnQuantGroupedMatMulAlltoAllv", section 计算公式; the
 * expert FFN of "Part 5", section 1.2, local expert execution; the shared-
 * expert MatMul of the same formula section is the case e = 1).
 *   a        device (A,Hin) in a_dt        rows grouped by expert
 *   w        device (e,Hin,N) in w_dt      N contiguous (shape of gmmWeight)
 *   a_q/w_q  MOE_QUANT_NONE (scale must be NULL) or MOE_QUANT_PER_TENSOR
 *            (scale = device pointer to one fp32); for E4M3 activations also
 *            a_q = MOE_QUANT_PER_TOKEN: a_scale = device fp32, one per row of
 *            a (16-byte aligned), multiplying that row's products (gmmXScale
 *            of shape (A,)); moe_quant_rows makes such rows. Other modes:
 *            UNSUPPORTED (MOE_QUANT_MX operands go through moe_gmm_mx;
 *            MOE_QUANT_PER_TOKEN_DYNAMIC is moe_quant_rows followed by
 *            MOE_QUANT_PER_TOKEN)
 *   offsets  device (e+1) int32, non-decreasing, offsets[0] = 0 and
 *            offsets[e] = A (not checked on the host: the values live on the
 *            device; offsets outside [0, A] are clamped to it)
 *   act      MOE_ACT_NONE or MOE_ACT_RELU
 *   out      device (A,N) in out_dt
 *   ws, ws_bytes device scratch of at least moe_gmm_workspace_size() bytes
 *            (may be NULL when that size is 0). When the output tiles leave
 *            a partial last round on the GPU, those tiles are split along
 *            the reduction and their fp32 partial sums meet here; the parts
 *            are added in a fixed order, so results do not depend on timing.
 *            It also holds the counters from which the bf16 kernel's
 *            persistent form (K <= 2048) hands out tiles. Its contents need
 *            no initialisation (the call clears what it uses, on the stream);
 *            calls that may run at the same time must not share it.
 * Supported types (a_dt, w_dt -> out_dt): F32,F32->F32; BF16,BF16->BF16;
 * FP8,FP8->BF16 (FP8 requires MOE_QUANT_PER_TENSOR or, for a, MOE_QUANT_PER_TOKEN
 * and MOE_QUANT_PER_TENSOR for w).
 * Accumulation is fp32; the scales multiply the fp32 sum; one rounding to
 * out_dt. Experts with no rows cost nothing and write nothing.
 */
moe_status moe_gmm_workspace_size(moe_dtype a_dt, int e, int A, int Hin, int N, size_t* bytes);
moe_status moe_gmm(const void* a, moe_dtype a_dt, moe_quant_mode a_q, const float* a_scale,
                   const void* w, moe_dtype w_dt, moe_quant_mode w_q, const float* w_scale,
                   const int32_t* offsets, int e, int A, int Hin, int N, moe_act act, void* out,
                   moe_dtype out_dt, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_gmm_gather — moe_gmm whose grouped row r is row row_src[r] / row_div of
 * a, so the dispatch copy (x_perm[perm_dst[t*K+k]] = x[t], "Part 5",
 * section 1.2 token dispatch) happens inside the GEMM's loads: with
 * row_src = perm_src of moe_permute and row_div = K, grouped row r is token
 * perm_src[r] / K, exactly the row moe_permute would have copied there.
 *   a        device (a_rows,Hin) in a_dt; a_rows * Hin * element size must be
 *            below 2^31 bytes (else MOE_ERR_UNSUPPORTED)
 *   row_src  device (A) int32; an entry whose quotient is outside
 *            [0, a_rows) (not checked on the host) reads as a zero row
 *   row_div  >= 1
 * Everything else (types, scales, offsets, act, out, workspace, errors) is
 * as for moe_gmm, with the same workspace size; results equal moe_gmm on the
 * gathered rows bit for bit.
 */
moe_status moe_gmm_gather(const void* a, int a_rows, const int32_t* row_src, int row_div, moe_dtype a_dt,
                          moe_quant_mode a_q, const float* a_scale, const void* w, moe_dtype w_dt,
                          moe_quant_mode w_q, const float* w_scale, const int32_t* offsets, int e, int A,
                          int Hin, int N, moe_act act, void* out, moe_dtype out_dt, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * moe_gmm_scatter — moe_gmm whose grouped row r is stored as row row_dst[r]
 * of out, times row_gate[row_dst[r]] when row_gate is not NULL:
 *   out[row_dst[r], n] = g * act( (sum_h a[r,h] * w[ex,h,n]) * a_scale * w_scale ),
 *   g = row_gate ? row_gate[row_dst[r]] : 1, fp32 product, one rounding.
 * With row_dst = perm_src of moe_permute (grouped row r's (token, slot)
 * index t*K+k), out is the GEMM's output already unpermuted into (t,k)
 * order: unpermuteOut = Unpermute(gmmY) ("aclnnQuantGroupedMatMulAlltoAllv",
 * section 计算公式) fused into the GEMM's stores. With row_gate = the (T,K)
 * top-k gates as well, out row t*K+k holds g[t,k] * E_k(x_t) and
 * moe_sum_slots completes y = sum_i g_i(x) E_i(x) (SpMM page, section
 * "MoE 模型与专家选择的挑战").
 *   row_dst  device (A) int32, required; each out row that should be written
 *            must be named by exactly one grouped row. Entries outside
 *            [0, A) (not checked on the host) are not stored.
 *   row_gate device fp32 indexed by the destination row (A entries), or NULL
 *   out      device (A,N) in out_dt; rows no entry names are left untouched
 * Everything else (types, scales, offsets, act, workspace, errors) is as for
 * moe_gmm, with the same workspace size; without a gate the stored rows equal
 * moe_gmm's rows bit for bit.
 */
moe_status moe_gmm_scatter(const void* a, moe_dtype a_dt, moe_quant_mode a_q, const float* a_scale,
                           const void* w, moe_dtype w_dt, moe_quant_mode w_q, const float* w_scale,
                           const int32_t* offsets, int e, int A, int Hin, int N, moe_act act,
                           const int32_t* row_dst, const float* row_gate, void* out, moe_dtype out_dt,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * moe_gmm_routed_shared — the routed experts' E4M3 grouped GEMM and the
 * shared expert's bf16 GEMM of one layer step in a single launch: the page's
 * two formulas, gmmY = (gmmX @ gmmWeight) * gmmXScale * gmmWeightScale and
 * mmY = (mmX @ mmWeight) * mmXScaleOptional * mmWeightScaleOptional
 * ("aclnnQuantGroupedMatMulAlltoAllv", section 计算公式), computed side by side
 * as its interface description (接口功能) has the routed GEMM run in parallel
 * with the shared expert's MatMul.
 *   routed:  a, a_q, a_scale, w, w_scale, offsets, e, A, Hin, N, act,
 *            row_dst, row_gate, out exactly as for moe_gmm_scatter with
 *            a_dt = w_dt = MOE_FP8_E4M3, w_q = MOE_QUANT_PER_TENSOR and
 *            out_dt = MOE_BF16, except that row_dst may be NULL (then grouped
 *            row r is stored as row r, as by moe_gmm)
 *   shared:  xs, ws_w, offsets_s, e_s, T, Hs, Ns, act_s, ys exactly as
 *            a, w, offsets, e, A, Hin, N, act, out of moe_gmm with all three
 *            types MOE_BF16 and no scales (mmX and mmWeight in bf16, the
 *            optional scales left out). The shared expert is e_s = 1,
 *            offsets_s = {0, T}: ys[t,n] = act_s( sum_h xs[t,h] * ws_w[h,n] ),
 *            xs (T,Hs) = mmX, ws_w (Hs,Ns) = mmWeight, ys (T,Ns) = mmY.
 * Either part may be empty (A = 0 or T = 0). One launch when both parts take
 * the tiled DMA kernels (E4M3: Hin and N multiples of 16; bf16: more than 48
 * rows per group on average, Hs % 8 == 0, Ns % 16 == 0; every expert's
 * weight matrix under 2 GiB); otherwise the two GEMMs are launched one after
 * the other on the stream. Either way out equals moe_gmm_scatter's (moe_gmm's)
 * result and ys equals moe_gmm's, bit for bit, whenever that moe_gmm call does
 * not split its last round of tiles along K: this call never splits, so it
 * takes no workspace. out and ys must not overlap each other or any input.
 * Errors: those of moe_gmm_scatter and moe_gmm for the two parts (no
 * workspace errors).
 */
moe_status moe_gmm_routed_shared(const void* a, moe_quant_mode a_q, const float* a_scale, const void* w,
                                 const float* w_scale, const int32_t* offsets, int e, int A, int Hin, int N,
                                 moe_act act, const int32_t* row_dst, const float* row_gate, void* out,
                                 const void* xs, const void* ws_w, const int32_t* offsets_s, int e_s, int T,
                                 int Hs, int Ns, moe_act act_s, void* ys, void* stream);

/*
 * moe_gmm_mx — grouped GEMM on MX block-scaled E4M3 operands (quant mode 6,
 * "mx", of "aclnnQuantGroupedMatMulAlltoAllv": the interface description
 * names per-tensor and mx as the supported quantisations). Every 32
 * consecutive reduction elements of an activation row and of a weight column
 * share one E8M0 scale byte s, value 2^(s-127) (255: NaN), the OCP MX
 * reading of the page's mx mode:
 *   out[r,n] = act( sum_b 2^(sa(r,b)-127) * 2^(sw(ex,b,n)-127)
 *                   * sum_{32b <= h < 32b+32} a[r,h] * w[ex,h,n] )
 * for offsets[ex] <= r < offsets[ex+1]; one rounding to bf16.
 *   a        device (A,Hin) E4M3 bytes, rows grouped by expert
 *   a_scale  device E8M0 bytes, slice-major: sa(r,b) is byte
 *            ((b/4)*A + r)*4 + b%4, i.e. (Hin/128, A, 4): for each 128-deep
 *            slice of the reduction, every row's 4 block scales, rows
 *            consecutive (the kernel then fetches contiguous bytes)
 *   w        device (e,Hin,N) E4M3 bytes, N contiguous
 *   w_scale  device E8M0 bytes (e, Hin/32, N64), N64 = N rounded up to a
 *            multiple of 64, columns interleaved within each group of 64:
 *            sw(ex,b,n) is byte (ex*(Hin/32) + b)*N64 + (n & ~63) + 4*(n%16)
 *            + (n%64)/16, so the scales of columns c, c+16, c+32, c+48 are
 *            adjacent (the padding bytes are not read)
 *   offsets, e, A, act   as for moe_gmm
 *   out      device (A,N) bf16
 * Hin must be a multiple of 128 and N of 16 (else MOE_ERR_UNSUPPORTED). No
 * workspace. Errors and validation as for moe_gmm.
 */
moe_status moe_gmm_mx(const void* a, const uint8_t* a_scale, const void* w, const uint8_t* w_scale,
                      const int32_t* offsets, int e, int A, int Hin, int N, moe_act act, void* out,
                      void* stream);

/*
 * moe_gmm_mxfp4 — moe_gmm_mx with E2M1 (OCP FP4: sign, 2 exponent bits with
 * bias 1, 1 mantissa bit; values 0, 0.5, 1, 1.5, 2, 3, 4, 6) elements, the
 * other element type of the page's mx mode ("aclnnQuantGroupedMatMulAlltoAllv",
 * quant-mode enumeration, mode 6; OCP MXFP4). Two elements per byte along the
 * reduction index, the even one in the low nibble:
 *   a       device (A, Hin/2) bytes: byte (r, k) holds a[r,2k] and a[r,2k+1]
 *   w       device (e, Hin/2, N) bytes: byte (ex, k, n) holds w[ex,2k,n] and
 *           w[ex,2k+1,n]
 *   a_scale device E8M0 bytes, slice-major with 256-deep slices: sa(r,b) is
 *           byte ((b/8)*A + r)*8 + b%8, i.e. (Hin/256, A, 8)
 *   w_scale device E8M0 bytes, the interleaved (e, Hin/32, N64) order of moe_gmm_mx
 *   out     device (A,N) bf16
 * Hin must be a multiple of 256 and N of 16 (else MOE_ERR_UNSUPPORTED).
 * Arithmetic, offsets, act and errors as moe_gmm_mx.
 */
moe_status moe_gmm_mxfp4(const void* a, const uint8_t* a_scale, const void* w, const uint8_t* w_scale,
                         const int32_t* offsets, int e, int A, int Hin, int N, moe_act act, void* out,
                         void* stream);

/*
 * moe_combine — back to token order.
 *   topk_gate != NULL: y[t,n] = sum_{k=0..K-1} gate[t,k] * y_perm[perm_dst[t*K+k], n],
 *     fp32 sum in ascending k, one rounding (y = sum g_i E_i(x), SpMM page);
 *     out is (T,N).
 *   topk_gate == NULL: Unpermute, out[t*K+k, n] = y_perm[perm_dst[t*K+k], n]
 *     (unpermuteOut = Unpermute(gmmY), "aclnnQuantGroupedMatMulAlltoAllv",
 *     section 计算公式); out is (T*K,N), a bit copy (in_dt must equal out_dt).
 *   y_perm   device (T*K,N) in in_dt; perm_dst device (T*K) int32 in [0,T*K)
 *   topk_gate device (T,K) fp32 or NULL
 * Types: F32->F32, BF16->BF16.
 */
moe_status moe_combine(const void* y_perm, moe_dtype in_dt, const int32_t* perm_dst,
                       const float* topk_gate, int T, int K, int N, void* out, moe_dtype out_dt,
                       void* stream);

/*
 * moe_gmm_mx_routed_shared — moe_gmm_mx (fp4 = 0) or moe_gmm_mxfp4 (fp4 = 1)
 * for the routed experts and the shared expert's bf16 GEMM in one launch, as
 * moe_gmm_routed_shared does for per-tensor E4M3 (the page's routed and
 * shared formulas, "aclnnQuantGroupedMatMulAlltoAllv" sections 计算公式 and
 * 接口功能, with its mx quant mode for the routed experts).
 *   routed:  a, a_scale, w, w_scale, offsets, e, A, Hin, N, act, out exactly
 *            as for moe_gmm_mx (fp4 = 0) or moe_gmm_mxfp4 (fp4 = 1)
 *   shared:  xs, ws_w, offsets_s, e_s, T, Hs, Ns, act_s, ys as for
 *            moe_gmm_routed_shared
 * One launch when the shared part takes the tiled DMA kernel (more than 48
 * rows per group on average, Hs % 8 == 0, Ns % 16 == 0) and A > 0; otherwise
 * two launches on the stream. out equals moe_gmm_mx's (moe_gmm_mxfp4's) and
 * ys moe_gmm's result bit for bit whenever that moe_gmm call does not split
 * along K. Errors: those of moe_gmm_mx / moe_gmm_mxfp4 and of moe_gmm for the
 * two parts; MOE_ERR_UNSUPPORTED for fp4 outside {0, 1}.
 */
moe_status moe_gmm_mx_routed_shared(const void* a, const uint8_t* a_scale, const void* w, const uint8_t* w_scale,
                                    const int32_t* offsets, int e, int A, int Hin, int N, moe_act act, int fp4,
                                    void* out, const void* xs, const void* ws_w, const int32_t* offsets_s,
                                    int e_s, int T, int Hs, int Ns, moe_act act_s, void* ys, void* stream);

/*
 * moe_sum_slots — y[t,n] = sum_{k=0..K-1} z[t*K+k, n], fp32 sum in ascending
 * k, one rounding: the K-row sum after moe_gmm_scatter has stored every
 * (token, slot) row already multiplied by its gate (y = sum_i g_i(x) E_i(x),
 * SpMM page, section "MoE 模型与专家选择的挑战").
 *   z device (T*K,N) in dt; out device (T,N) in dt; dt MOE_F32 or MOE_BF16.
 * Errors: as moe_combine.
 */
moe_status moe_sum_slots(const void* z, moe_dtype dt, int T, int K, int N, void* out, void* stream);

/*
 * moe_quant_rows — per-token dynamic quantisation to E4M3 (quant modes 3
 * "pertoken" and 7 "pertoken dynamic" of "aclnnQuantGroupedMatMulAlltoAllv",
 * 量化模式 enumeration; the page gives no formula, this is the plain
 * reading). Output row r quantises source row
 * t = row_src ? row_src[r] / row_div : r of x:
 *   scale[r] = max_h |x[t,h]| / 448, one binary32 division rounded to nearest
 *   q[r,h]   = the E4M3 value nearest to the exact quotient x[t,h] / scale[r],
 *              ties to the even code, saturating at +-448 (OCP E4M3, no
 *              infinities)
 * A zero row, a row whose max / 448 rounds to zero in binary32, or a source
 * row outside [0, x_rows) (not checked on the host), gives codes 0 and scale
 * 0. Non-finite inputs give unspecified codes. With row_src = perm_src of moe_permute and
 * row_div = K the dispatch copy and the quantisation are one pass (gmmX in
 * E4M3 with its per-row gmmXScale); with row_src = NULL the tokens are
 * quantised once and moe_gmm_gather reads them (and their scales) by index.
 *   x      device (x_rows,H) in x_dt (MOE_F32 or MOE_BF16), 16-byte aligned
 *   row_src device (rows) int32 or NULL (then rows <= x_rows); row_div >= 1
 *   q      device (rows,H) bytes, E4M3 codes; scale device (rows) fp32
 * Errors: BAD_DTYPE, BAD_SHAPE (H outside (0,65536), rows < 0, row_div < 1,
 * rows > x_rows without row_src), NULL_POINTER, MISALIGNED.
 */
moe_status moe_quant_rows(const void* x, moe_dtype x_dt, int x_rows, int H, const int32_t* row_src,
                          int row_div, int rows, uint8_t* q, float* scale, void* stream);

/*
 * moe_layer — the whole layer on one stream: route, permute, GEMM 1 with the
 * activation (hidden kept in dt), GEMM 2, weighted combine.
 *   x (T,H), w_router (H,E), bias (E) fp32 or NULL, w1 (E,H,F), w2 (E,F,H),
 *   y (T,H) out; all device, all in dt (MOE_F32 or MOE_BF16) except bias.
 *   topk_idx_out (T,K) int32, topk_gate_out (T,K) fp32, counts_out (E) int32:
 *   optional device outputs (NULL = not wanted).
 *   ws, ws_bytes: device scratch of at least moe_layer_workspace_size() bytes.
 */
moe_status moe_layer_workspace_size(int T, int H, int E, int K, int F, moe_dtype dt, size_t* bytes);
moe_status moe_layer(const void* x, const void* w_router, const float* bias, const void* w1,
                     const void* w2, moe_dtype dt, int T, int H, int E, int K, int F, moe_act act,
                     void* y, int32_t* topk_idx_out, float* topk_gate_out, int32_t* counts_out,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * moe_layer_noalloc — moe_layer for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments and results, bit for bit, without
 * the workspace. Its scratch memory is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES (32 MiB) inside the library, one copy per GPU,
 * held until the process ends; its address on a device is looked up on the
 * first call made with that device current. The call allocates nothing.
 *   A call whose moe_layer_workspace_size() exceeds MOE_NOALLOC_SCRATCH_BYTES
 *   returns MOE_ERR_SCRATCH_LIMIT and enqueues nothing (32 MiB holds, e.g.,
 *   every decode-shaped call up to T*K = 2048 rows at H = 4096, F = 1536).
 *   The stream must belong to the current device.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams, other host threads) race and must be serialised by the
 * caller; calls on one stream are ordered by it. Errors: as moe_layer, plus
 * MOE_ERR_SCRATCH_LIMIT, and MOE_ERR_DEVICE if the array's address cannot be
 * obtained.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status moe_layer_noalloc(const void* x, const void* w_router, const float* bias, const void* w1,
                             const void* w2, moe_dtype dt, int T, int H, int E, int K, int F, moe_act act,
                             void* y, int32_t* topk_idx_out, float* topk_gate_out, int32_t* counts_out,
                             void* stream);

/*
 * moe_layer_fp8 — the layer with E4M3 experts: route on the bf16 tokens,
 * permute, then each expert GEMM on E4M3 activations quantised per token on
 * the fly (quant mode 7, per-token dynamic, of "aclnnQuantGroupedMatMulAlltoAllv",
 * with per-tensor weight scales: gmmY = (gmmX @ gmmWeight) * gmmXScale *
 * gmmWeightScale, section 计算公式): the tokens are quantised once and GEMM 1
 * gathers them through the dispatch index; the bf16 hidden rows are
 * quantised per row before GEMM 2; the weighted combine as moe_layer.
 *   x (T,H) bf16, w_router (H,E) bf16, bias (E) fp32 or NULL
 *   w1 (E,H,F) and w2 (E,F,H) E4M3 bytes; w1_scale, w2_scale: one fp32 each
 *   (device); y (T,H) bf16; topk/counts outputs and errors as moe_layer
 *   ws, ws_bytes: device scratch of at least moe_layer_fp8_workspace_size().
 */
moe_status moe_layer_fp8_workspace_size(int T, int H, int E, int K, int F, size_t* bytes);
moe_status moe_layer_fp8(const void* x, const void* w_router, const float* bias, const uint8_t* w1,
                         const float* w1_scale, const uint8_t* w2, const float* w2_scale, int T, int H, int E,
                         int K, int F, moe_act act, void* y, int32_t* topk_idx_out, float* topk_gate_out,
                         int32_t* counts_out, void* ws, size_t ws_bytes, void* stream);

/* ---- diagnostics (not steps of the layer) --------------------------------
 *
 * moe_fetch_probe: measures how fast one compute unit reads from device
 * memory, the rate that bounds the grouped GEMM's tiles (each 256 x 256
 * ping-pong tile fetches 32 bytes per MFMA cycle of its CU at full MFMA
 * use). One block of 8 waves runs on every compute unit; each wave reads
 * kb_per_wave KB in 1 KB instructions, 8 in flight. Time the launch with
 * stream events for a rate per second: the per-block counts below come from
 * s_memtime, whose tick rate was seen to differ from the shader clock and
 * to vary between kernels, so they show the spread across CUs, not a rate.
 *   buf     device, bytes long, 16-byte aligned (its contents are not used)
 *   bytes   multiple of 1024, below 2^31; shared_window != 0: every block
 *           reads the first `bytes` bytes (>= 64 KB; a size that stays in
 *           L2, e.g. 2 MB, measures L2 -> CU); shared_window == 0: block b
 *           reads its own bytes / ncu slice (>= 1 KB each; measures HBM)
 *   mode    0: LDS DMA (buffer_load_dwordx4 ... lds, as the GEMM kernels
 *           fetch), 1: 16-byte vector loads into registers
 *   kb_per_wave  multiple of 8 in [8, 2^20]
 *   cycles  device, one uint64 per compute unit of the device
 *           (hipDeviceAttributeMultiprocessorCount): the s_memtime ticks
 *           block b spent reading 8 * kb_per_wave * 1024 bytes.
 * Errors: NULL_POINTER, MISALIGNED, UNSUPPORTED (mode), BAD_SHAPE; DEVICE.
 */
moe_status moe_fetch_probe(const void* buf, size_t bytes, int mode, int shared_window, int kb_per_wave,
                           uint64_t* cycles, void* stream);

/* moe_mfma_probe: the MFMA rate with no memory traffic, the achievable side of
 * the MFMA peak. One block of 8 waves runs on every compute unit; each wave
 * issues `iters` rounds of 8 independent MFMAs on register operands
 * (MOE_BF16: v_mfma_f32_16x16x32_bf16, 16384 flops each; MOE_FP8_E4M3:
 * v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales, 131072 flops each).
 *   iters   in [1, 2^24]
 *   sink    device, 512 floats per compute unit (results, kept so the work runs)
 *   cycles  device, one uint64 per compute unit: s_memtime ticks of block b
 * Flops per CU = 8 waves * 8 * iters * flops per MFMA; time the launch with
 * stream events for the rate.
 * Errors: NULL_POINTER, BAD_DTYPE, BAD_SHAPE; DEVICE.
 */
moe_status moe_mfma_probe(moe_dtype dt, int iters, float* sink, uint64_t* cycles, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
