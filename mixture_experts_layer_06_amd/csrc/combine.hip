// combine.hip — back to token order.
//  weighted: y[t] = sum_{k ascending} g[t,k] * y_perm[perm_dst[t*K+k]]
//            (y = sum_i g_i(x) E_i(x), SpMM page, section "MoE 模型与专家选择的挑战"),
//            fp32 sum, one rounding to the output type;
//  unweighted: out[t*K+k] = y_perm[perm_dst[t*K+k]]
//            (unpermuteOut = Unpermute(gmmY), "aclnnQuantGroupedMatMulAlltoAllv",
//            section 计算公式);
//  slot sum: y[t] = sum_{k ascending} z[t*K+k], the rows already in (t,k)
//            order and gated (by the GEMM's scattering epilogue).
// Both are pure bandwidth kernels: blocks over (output token, column
// stripe), 16-byte vector accesses when the row pitch allows, every input
// row read once (the weighted sum's loads and stores nontemporal). Few tokens (decode) get several column stripes per token,
// so that each thread issues the loads of all K rows of one vector at once.
#include "common.h"

namespace moe {
namespace {

template <bool BF16, int VE>  // VE = elements per vector access
__global__ __launch_bounds__(256) void combine_weighted_kernel(const void* __restrict__ yp_,
                                                               const int32_t* __restrict__ perm_dst,
                                                               const float* __restrict__ gate, int T,
                                                               int K, int N, void* __restrict__ out_) {
  typedef typename std::conditional<BF16, bf16_t, float>::type E;
  const E* yp = reinterpret_cast<const E*>(yp_);
  E* out = reinterpret_cast<E*>(out_);
  const int nv = N / VE;
  for (int t = blockIdx.x; t < T; t += gridDim.x) {
    int src[8];
    float g[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      // no permutation: rows t*K+k in place; no gate: weight 1
      src[k] = k < K ? (perm_dst != nullptr ? perm_dst[(int64_t)t * K + k] : t * K + k) : 0;
      g[k] = k < K ? (gate != nullptr ? gate[(int64_t)t * K + k] : 1.f) : 0.f;
    }
    if (VE * sizeof(E) == 16) {
      // 16-byte vectors: the loads of all K rows are in flight before the
      // first is used; rows are read once and outputs written once, so both
      // are nontemporal
      typedef unsigned int u4 __attribute__((ext_vector_type(4)));
      for (int j = blockIdx.y * blockDim.x + threadIdx.x; j < nv; j += gridDim.y * blockDim.x) {
        u4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k < K)
            v[k] = __builtin_nontemporal_load(reinterpret_cast<const u4*>(yp + (int64_t)src[k] * N + (int64_t)j * VE));
        float acc[VE];
#pragma unroll
        for (int q = 0; q < VE; ++q) acc[q] = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (k < K) {
            E e[VE];
            *reinterpret_cast<u4*>(e) = v[k];
#pragma unroll
            for (int q = 0; q < VE; ++q) {
              const float f = BF16 ? bf16_to_f32((bf16_t)e[q]) : (float)e[q];
              acc[q] = fmaf(g[k], f, acc[q]);
            }
          }
        }
        E o[VE];
#pragma unroll
        for (int q = 0; q < VE; ++q) {
          if (BF16) o[q] = (E)f32_to_bf16(acc[q]);
          else o[q] = (E)acc[q];
        }
        __builtin_nontemporal_store(*reinterpret_cast<u4*>(o),
                                    reinterpret_cast<u4*>(out + (int64_t)t * N + (int64_t)j * VE));
      }
      continue;
    }
    for (int j = blockIdx.y * blockDim.x + threadIdx.x; j < nv; j += gridDim.y * blockDim.x) {
      float acc[VE];
#pragma unroll
      for (int q = 0; q < VE; ++q) acc[q] = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (k < K) {
          const E* row = yp + (int64_t)src[k] * N + (int64_t)j * VE;
          E v[VE];
          if (VE * sizeof(E) == 16) {
            *reinterpret_cast<uint4*>(v) = *reinterpret_cast<const uint4*>(row);
          } else {
#pragma unroll
            for (int q = 0; q < VE; ++q) v[q] = row[q];
          }
#pragma unroll
          for (int q = 0; q < VE; ++q) {
            const float f = BF16 ? bf16_to_f32((bf16_t)v[q]) : (float)v[q];
            acc[q] = fmaf(g[k], f, acc[q]);
          }
        }
      }
      E o[VE];
#pragma unroll
      for (int q = 0; q < VE; ++q) {
        if (BF16) o[q] = (E)f32_to_bf16(acc[q]);
        else o[q] = (E)acc[q];
      }
      E* dst = out + (int64_t)t * N + (int64_t)j * VE;
      if (VE * sizeof(E) == 16) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<uint4*>(o);
      } else {
#pragma unroll
        for (int q = 0; q < VE; ++q) dst[q] = o[q];
      }
    }
  }
}

// Unpermute: one block per token copies its K rows. VB = bytes per access.
template <int VB>
__global__ __launch_bounds__(256) void unpermute_kernel(const unsigned char* __restrict__ yp,
                                                        const int32_t* __restrict__ perm_dst, int T,
                                                        int K, int64_t row_bytes,
                                                        unsigned char* __restrict__ out) {
  typedef typename std::conditional<VB == 16, uint4,
          typename std::conditional<VB == 8, uint2,
          typename std::conditional<VB == 4, uint32_t, uint16_t>::type>::type>::type V;
  const int64_t nv = row_bytes / VB;
  for (int t = blockIdx.x; t < T; t += gridDim.x) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k >= K) break;
      const int64_t i = (int64_t)t * K + k;
      const V* src = reinterpret_cast<const V*>(yp + (int64_t)perm_dst[i] * row_bytes);
      V* dst = reinterpret_cast<V*>(out + i * row_bytes);
      for (int64_t j = blockIdx.y * blockDim.x + threadIdx.x; j < nv; j += gridDim.y * blockDim.x)
        dst[j] = src[j];
    }
  }
}

}  // namespace

moe_status launch_combine(const void* y_perm, moe_dtype dt, const int32_t* perm_dst,
                          const float* gate, int T, int K, int N, void* out, hipStream_t s,
                          bool sum_slots) {
  if (T == 0) return MOE_OK;
  const bool bf = dt == MOE_BF16;
  if (sum_slots) {
    perm_dst = nullptr;
    gate = nullptr;
  }
  const bool weighted = gate != nullptr || sum_slots;
  // column stripes per token: one 256-vector stripe per block when tokens are few
  const int64_t vecs = weighted ? (bf ? N / 8 : N / 4) : (int64_t)N * (bf ? 2 : 4) / 16;
  int stripes = 1;
  if (T < 2048) {
    const int64_t st = (vecs + 255) / 256;
    stripes = st < 1 ? 1 : (st > 64 ? 64 : (int)st);
  }
  const dim3 grid(T < 65536 ? T : 65536, stripes);
  if (weighted) {
    if (bf) {
      if (N % 8 == 0)
        hipLaunchKernelGGL((combine_weighted_kernel<true, 8>), dim3(grid), dim3(256), 0, s, y_perm,
                           perm_dst, gate, T, K, N, out);
      else
        hipLaunchKernelGGL((combine_weighted_kernel<true, 1>), dim3(grid), dim3(256), 0, s, y_perm,
                           perm_dst, gate, T, K, N, out);
    } else {
      if (N % 4 == 0)
        hipLaunchKernelGGL((combine_weighted_kernel<false, 4>), dim3(grid), dim3(256), 0, s, y_perm,
                           perm_dst, gate, T, K, N, out);
      else
        hipLaunchKernelGGL((combine_weighted_kernel<false, 1>), dim3(grid), dim3(256), 0, s, y_perm,
                           perm_dst, gate, T, K, N, out);
    }
  } else {
    const int64_t rb = (int64_t)N * (bf ? 2 : 4);
    const unsigned char* src = (const unsigned char*)y_perm;
    unsigned char* dst = (unsigned char*)out;
    if (rb % 16 == 0)
      hipLaunchKernelGGL(unpermute_kernel<16>, dim3(grid), dim3(256), 0, s, src, perm_dst, T, K, rb, dst);
    else if (rb % 8 == 0)
      hipLaunchKernelGGL(unpermute_kernel<8>, dim3(grid), dim3(256), 0, s, src, perm_dst, T, K, rb, dst);
    else if (rb % 4 == 0)
      hipLaunchKernelGGL(unpermute_kernel<4>, dim3(grid), dim3(256), 0, s, src, perm_dst, T, K, rb, dst);
    else
      hipLaunchKernelGGL(unpermute_kernel<2>, dim3(grid), dim3(256), 0, s, src, perm_dst, T, K, rb, dst);
  }
  return launch_status();
}

}  // namespace moe
