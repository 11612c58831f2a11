// quant.hip — per-token dynamic quantisation to E4M3 (quant modes 3
// "pertoken" and 7 "pertoken dynamic" of "aclnnQuantGroupedMatMulAlltoAllv",
// 量化模式 enumeration; its formula multiplies gmmX's scale back onto the
// product). For every output row r, with source row t = src[r] / div (or r):
//   scale[r] = max_h |x[t,h]| / 448          (binary32 division)
//   q[r,h]   = nearest E4M3 value of x[t,h] / scale[r]   (binary32 division,
//              ties to the even code, saturating at +-448)
// An all-zero row, or a source row outside [0, x_rows), gives codes 0 and
// scale 0. With src = perm_src of the dispatch and div = K this is the
// permute and the quantisation in one pass (x_perm in E4M3 plus its
// per-row scales, the form gmmX and gmmXScale take on that page).
//
// HBM-bound: one wave per output row reads the row twice (the second pass
// hits L2), writes one byte per element and one scale.
#include "common.h"

namespace moe {
namespace {

// Code of the finite E4M3 value nearest to v, ties to the even code; |v| at
// or above 448 saturates, NaN gives 0x7f. Built from the format: subnormal
// steps of 2^-9 below 2^-6, else 3 mantissa bits per binade (exponent bias 7).
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 24) & 0x80u;
  const float a = __uint_as_float(b & 0x7fffffffu);
  if (!(a == a)) return 0x7fu;
  if (a >= 448.f) return sign | 0x7eu;
  if (a < 0.015625f) {                       // below 2^-6: multiples of 2^-9
    const float m = rintf(a * 512.f);        // exact scaling; rint ties to even
    return sign | (uint32_t)m;               // m == 8 is 2^-6, code 0x08
  }
  int e = (int)((b >> 23) & 0xffu) - 127;    // -6 .. 8
  uint32_t m = (uint32_t)rintf(__builtin_ldexpf(a, 3 - e));  // 8 .. 16
  if (m == 16u) {
    m = 8u;
    ++e;
  }
  return sign | ((uint32_t)(e + 7) << 3) | (m - 8u);  // a < 448 keeps it at or below 0x7e
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* x, int64_t i) {
  if (BF16) return bf16_to_f32(reinterpret_cast<const bf16_t*>(x)[i]);
  return reinterpret_cast<const float*>(x)[i];
}

// 8 consecutive elements starting at i (i a multiple of 8, 16-byte aligned rows)
template <bool BF16>
__device__ __forceinline__ void load8(const void* x, int64_t i, float v[8]) {
  if (BF16) {
    const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(x) + i);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + i);
    const float4 c = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
  }
}

// VEC: H % 8 == 0 and 16-byte aligned rows (8 elements per access).
template <bool BF16, bool VEC>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* __restrict__ x, int x_rows, int H,
                                                         const int32_t* __restrict__ src, int div, int rows,
                                                         uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  int t = r;
  if (src != nullptr) {
    const int v = src[r];
    t = v >= 0 ? v / div : -1;
  }
  uint8_t* qr = q + (int64_t)r * H;
  const bool valid = t >= 0 && t < x_rows;
  const int64_t base = (int64_t)(valid ? t : 0) * H;
  float amax = 0.f;
  if (valid) {
    if (VEC) {
      for (int h = lane * 8; h < H; h += 64 * 8) {
        float v[8];
        load8<BF16>(x, base + h, v);
#pragma unroll
        for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
      }
    } else {
      for (int h = lane; h < H; h += 64) amax = fmaxf(amax, fabsf(load_elem<BF16>(x, base + h)));
    }
    amax = wave_max(amax);
  }
  const float s = amax / 448.f;
  if (lane == 0) scale[r] = s;
  const bool zero = !(amax > 0.f);
  if (VEC) {
    for (int h = lane * 8; h < H; h += 64 * 8) {
      uint32_t lo = 0, hi = 0;
      if (!zero) {
        float v[8];
        load8<BF16>(x, base + h, v);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          lo |= e4m3_code(v[k] / s) << (8 * k);
          hi |= e4m3_code(v[k + 4] / s) << (8 * k);
        }
      }
      *reinterpret_cast<uint2*>(qr + h) = make_uint2(lo, hi);
    }
  } else {
    for (int h = lane; h < H; h += 64)
      qr[h] = zero ? 0 : (uint8_t)e4m3_code(load_elem<BF16>(x, base + h) / s);
  }
}

}  // namespace

moe_status launch_quant_rows(const void* x, moe_dtype dt, int x_rows, int H, const int32_t* src, int div,
                             int rows, uint8_t* q, float* scale, hipStream_t s) {
  if (rows == 0) return MOE_OK;
  const bool bf = dt == MOE_BF16;
  const bool vec = H % 8 == 0;  // rows then start 16-byte aligned (x 16-byte aligned)
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (bf) {
    if (vec)
      hipLaunchKernelGGL((quant_rows_kernel<true, true>), grid, dim3(256), 0, s, x, x_rows, H, src, div, rows, q,
                         scale);
    else
      hipLaunchKernelGGL((quant_rows_kernel<true, false>), grid, dim3(256), 0, s, x, x_rows, H, src, div, rows,
                         q, scale);
  } else {
    if (vec)
      hipLaunchKernelGGL((quant_rows_kernel<false, true>), grid, dim3(256), 0, s, x, x_rows, H, src, div, rows,
                         q, scale);
    else
      hipLaunchKernelGGL((quant_rows_kernel<false, false>), grid, dim3(256), 0, s, x, x_rows, H, src, div, rows,
                         q, scale);
  }
  return launch_status();
}

}  // namespace moe
