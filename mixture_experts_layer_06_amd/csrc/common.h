// common.h — internal helpers of the gfx950 MoE library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "moe.h"

namespace moe {

typedef uint16_t bf16_t;  // bfloat16 bit pattern
typedef uint8_t fp8_t;    // OCP E4M3 byte

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;  // CDNA wavefront width

__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// binary32 -> bfloat16, round to nearest even, NaN stays NaN: gfx950's
// v_cvt_pk_bf16_f32, one instruction per pair (a bit-twiddled conversion
// with a NaN test compiles to per-value branches, which made the GEMM
// epilogues instruction-bound).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// v_perm_b32: result byte i = byte sel[i] of the 8-byte value {hi:lo}.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// bf16: rows r0..r7 of 4 columns (uint2 each) -> 4 columns of 8 rows (uint4 each).
__device__ __forceinline__ void transpose_8x4_bf16(const uint2 in[8], uint4 out[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    uint32_t d[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t a = (c >> 1) ? in[2 * p].y : in[2 * p].x;
      const uint32_t b = (c >> 1) ? in[2 * p + 1].y : in[2 * p + 1].x;
      d[p] = perm_b32(b, a, sel);
    }
    out[c] = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer, 32-bit data format; loads at offsets >= bytes return zero
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

constexpr uint32_t kOOB = 0x80000000u;  // offset bias that puts a load out of range

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int dtype_size(moe_dtype dt) { return dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 2 : 1; }

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline moe_status launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE;
}

// Launchers implemented by the kernel files. They assume validated arguments.
size_t route_ws_bytes(int T, int H, int E, moe_dtype dt);
moe_status launch_route(const void* x, const void* wr, moe_dtype dt, const float* bias, int T, int H,
                        int E, int K, int32_t* idx, float* gate, void* ws, hipStream_t s);
size_t permute_ws_bytes(int T, int E, int K);
// zero, nzero: ints that the index path's first kernel also sets to 0 (the
// grouped GEMMs' counters when a later launch on the stream needs them clear).
moe_status launch_permute(const int32_t* idx, const void* x, moe_dtype dt, int T, int H, int E, int K,
                          int32_t* counts, int32_t* offsets, int32_t* perm_src, int32_t* perm_dst,
                          void* x_perm, void* ws, hipStream_t s, int* zero = nullptr, int nzero = 0);
// Row maps of a grouped GEMM. Input: grouped row r reads row src[r] / div of
// an input with `rows` rows (src == nullptr: row r itself); row_scale, when
// set (E4M3 inputs), is a per-row activation scale indexed like the rows of
// the input. Output: grouped row r is stored as row dst[r] of out, multiplied
// by gate[dst[r]] when gate is set (dst == nullptr: row r, no gate);
// destinations outside [0, A) are not stored.
struct RowMap {
  const int32_t* src = nullptr;
  int div = 1;
  int rows = 0;
  const int32_t* dst = nullptr;
  const float* gate = nullptr;
  const float* row_scale = nullptr;
};
size_t gmm_ws_bytes(moe_dtype in_dt, int e, int A, int Hin, int N);
int gmm_counter_ints();  // counters of one bf16 ping-pong GEMM launch (split parts and queues)
int probe_device_cus();  // compute units of the current device (0 when the query fails)
moe_status launch_fetch_probe(const void* buf, size_t bytes, int mode, int shared_window, int kb_per_wave,
                              unsigned long long* cycles, int ncu, hipStream_t s);
moe_status launch_mfma_probe(int fp8, int iters, float* sink, unsigned long long* cycles, int ncu, hipStream_t s);
moe_status launch_gmm(const void* a, moe_dtype in_dt, const float* a_scale, const void* w,
                      const float* w_scale, const int32_t* offsets, int e, int A, int Hin, int N,
                      moe_act act, void* out, moe_dtype out_dt, void* ws, hipStream_t s,
                      RowMap gx = RowMap{}, int* cnt_zeroed = nullptr);
// cnt_zeroed: gmm_counter_ints() counters that an earlier launch on the
// stream has set to 0; the bf16 ping-pong GEMM then uses them in place of the
// counters in ws and launches no kernel to clear them.
// One grouped GEMM's operands (the arguments of launch_gmm).
struct GmmCall {
  const void* a;
  const float* a_scale;
  const void* w;
  const float* w_scale;
  const int32_t* offsets;
  int e, A, Hin, N;
  moe_act act;
  void* out;
  RowMap gx;
  const unsigned char* a_mx = nullptr;  // E8M0 block scales when mx != 0
  const unsigned char* w_mx = nullptr;
  int mx = 0;  // 0: E4M3 with per-tensor / per-row scales; 1: MX E4M3; 2: MX E2M1
};
// An E4M3 (or MX E4M3 / E2M1) grouped GEMM f and a bf16 grouped GEMM b
// (bf16 out for both) in one launch when both take the ping-pong kernels,
// else as two launches (launch_gmm_mx / launch_gmm, no workspace); either
// way each result equals its own launch with no workspace.
moe_status launch_gmm_pair(const GmmCall& f, const GmmCall& b, hipStream_t s);
// Grouped GEMM on MX (E8M0 block-scaled) operands: E4M3 (Hin % 128 == 0) or,
// fp4, E2M1 packed two per byte along K (Hin % 256 == 0); N % 16 == 0.
moe_status launch_gmm_mx(const void* a, const unsigned char* a_scale, const void* w,
                         const unsigned char* w_scale, const int32_t* offsets, int e, int A, int Hin, int N,
                         moe_act act, void* out, hipStream_t s, bool fp4 = false);
// sum_slots: y[t] = sum_k y_perm[t*K+k] (perm_dst and gate ignored).
// Per-token E4M3 quantisation of the rows src[r] / div (or r) of x.
moe_status launch_quant_rows(const void* x, moe_dtype dt, int x_rows, int H, const int32_t* src, int div,
                             int rows, uint8_t* q, float* scale, hipStream_t s);
moe_status launch_combine(const void* y_perm, moe_dtype dt, const int32_t* perm_dst,
                          const float* gate, int T, int K, int N, void* out, hipStream_t s,
                          bool sum_slots = false);

}  // namespace moe
