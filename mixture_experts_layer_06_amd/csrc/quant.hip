// quant.hip — per-token dynamic quantisation to E4M3 (quant modes 3
// "pertoken" and 7 "pertoken dynamic" of "aclnnQuantGroupedMatMulAlltoAllv",
// 量化模式 enumeration; its formula multiplies gmmX's scale back onto the
// product). For every output row r, with source row t = src[r] / div (or r):
//   scale[r] = max_h |x[t,h]| / 448          (binary32 division)
//   q[r,h]   = nearest E4M3 value of x[t,h] * (448 / max_h |x[t,h]|)
//              (binary32: one division per row, then products; ties to the
//              even code, saturating at +-448)
// An all-zero row, or a source row outside [0, x_rows), gives codes 0 and
// scale 0. With src = perm_src of the dispatch and div = K this is the
// permute and the quantisation in one pass (x_perm in E4M3 plus its
// per-row scales, the form gmmX and gmmXScale take on that page).
//
// HBM-bound: one wave per output row reads the row once (rows up to 14336
// bf16 or 4096 fp32 values stay in registers in their input encoding; longer
// ones are read again from L2), writes one byte per element and one scale.
#include "common.h"

namespace moe {
namespace {

// E4M3 codes of two binary32 values, written into byte pair HI of `old`:
// gfx950's conversion rounds to the nearest E4M3 value, ties to the even
// code (OCP E4M3, as the MFMAs read it). Inputs here are at most 448 in
// magnitude up to one rounding of x * (448 / amax), so they never overflow;
// non-finite inputs give unspecified codes.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
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

// 8 consecutive elements starting at i (i a multiple of 8, 16-byte aligned
// rows), as raw words: bf16 fills raw[0], fp32 raw[0] and raw[1].
template <bool BF16>
__device__ __forceinline__ void load8_raw(const void* x, int64_t i, uint4 raw[2]) {
  if (BF16) {
    raw[0] = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(x) + i);
  } else {
    raw[0] = *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(x) + i);
    raw[1] = *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(x) + i + 4);
  }
}

template <bool BF16>
__device__ __forceinline__ void unpack8(const uint4 raw[2], float v[8]) {
  if (BF16) {
    const uint32_t w[4] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  } else {
    const uint32_t w[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __uint_as_float(w[k]);
  }
}

template <bool BF16>
__device__ __forceinline__ void load8(const void* x, int64_t i, float v[8]) {
  uint4 raw[2];
  load8_raw<BF16>(x, i, raw);
  unpack8<BF16>(raw, v);
}

// Codes of 8 values, packed little-endian into two words.
__device__ __forceinline__ uint2 e4m3_pack8(const float v[8], float inv) {
  uint32_t lo = e4m3_pair<false>(v[0] * inv, v[1] * inv, 0u);
  lo = e4m3_pair<true>(v[2] * inv, v[3] * inv, lo);
  uint32_t hi = e4m3_pair<false>(v[4] * inv, v[5] * inv, 0u);
  hi = e4m3_pair<true>(v[6] * inv, v[7] * inv, hi);
  return make_uint2(lo, hi);
}

// Source row of output row r, or -1 (zero row).
__device__ __forceinline__ int quant_src_row(const int32_t* src, int div, int x_rows, int r) {
  int t = r;
  if (src != nullptr) {
    const int v = src[r];
    t = v >= 0 ? v / div : -1;
  }
  return t < x_rows ? t : -1;
}

// One wave per output row. VEC (H % 8 == 0, rows 16-byte aligned): 8
// elements per access; rows of at most kCh * 512 elements are held in
// registers (one HBM read, all loads in flight at once), longer rows are
// read twice (the second pass from L2). Otherwise one element per access.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* __restrict__ x, int x_rows, int H,
                                                         const int32_t* __restrict__ src, int div, int rows,
                                                         uint8_t* __restrict__ q, float* __restrict__ scale) {
  constexpr int kCh = BF16 ? 28 : 8;  // register-held chunks of 8 elements per lane
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int t = quant_src_row(src, div, x_rows, r);
  uint8_t* qr = q + (int64_t)r * H;
  const int64_t base = (int64_t)(t >= 0 ? t : 0) * H;
  if (VEC && H <= kCh * 512) {
    uint4 raw[kCh][BF16 ? 1 : 2];  // the row in its input encoding
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < kCh; ++c) {
      const int h = (c * 64 + lane) * 8;
      if (t >= 0 && h < H) {
        uint4 r2[2];
        load8_raw<BF16>(x, base + h, r2);
        raw[c][0] = r2[0];
        if (!BF16) raw[c][BF16 ? 0 : 1] = r2[1];
        float v[8];
        unpack8<BF16>(r2, v);
#pragma unroll
        for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
      }
    }
    amax = wave_max(amax);
    if (lane == 0) scale[r] = amax / 448.f;
    const float inv = 448.f / amax;
    const bool zero = !(amax > 0.f);
#pragma unroll
    for (int c = 0; c < kCh; ++c) {
      const int h = (c * 64 + lane) * 8;
      if (h < H) {
        uint2 o = make_uint2(0u, 0u);
        if (!zero) {
          uint4 r2[2];
          r2[0] = raw[c][0];
          if (!BF16) r2[1] = raw[c][BF16 ? 0 : 1];
          float v[8];
          unpack8<BF16>(r2, v);
          o = e4m3_pack8(v, inv);
        }
        *reinterpret_cast<uint2*>(qr + h) = o;
      }
    }
    return;
  }
  float amax = 0.f;
  if (t >= 0) {
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
  if (lane == 0) scale[r] = amax / 448.f;
  const float inv = 448.f / amax;
  const bool zero = !(amax > 0.f);
  if (VEC) {
    for (int h = lane * 8; h < H; h += 64 * 8) {
      uint2 o = make_uint2(0u, 0u);
      if (!zero) {
        float v[8];
        load8<BF16>(x, base + h, v);
        o = e4m3_pack8(v, inv);
      }
      *reinterpret_cast<uint2*>(qr + h) = o;
    }
  } else {
    for (int h = lane; h < H; h += 64)
      qr[h] = zero ? 0 : (uint8_t)(e4m3_pair<false>(load_elem<BF16>(x, base + h) * inv, 0.f, 0u) & 0xffu);
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
