// probe.hip — read rate of one CU from device memory and the MFMA issue
// rate without memory traffic: diagnostics for the grouped GEMM's ceiling
// (not steps of the MoE layer).
//
// The ping-pong GEMM kernels fetch a 32 KB K slice per 1024 MFMA cycles per
// CU, so how fast one CU can pull bytes bounds their MFMA use.
// This kernel measures it: one block of 8 waves per CU (128 KB of dynamic
// LDS keeps a second block off the CU), each wave streaming `kb_per_wave`
// KB in 1 KB instructions with 8 of them in flight, either as LDS DMA
// (buffer_load_dwordx4 ... lds, what the GEMM kernels use) or as 16-byte
// vector loads into registers. Every block also counts s_memtime ticks
// across its reads (the spread across CUs; the rate comes from timing the
// launch, as these ticks do not keep the shader clock's pace). Shared window: every block reads the first `bytes`
// bytes (a size that stays in L2 measures the L2-to-CU path); private: block
// b reads its own 1/ncu of the buffer (the HBM path).
#include "common.h"

namespace moe {
namespace {

constexpr int kProbeWaves = 8;
constexpr int kProbeDepth = 8;
constexpr int kProbeLds = 128 * 1024;

// Byte offset of the 1 KB unit that wave w of block b reads at iteration i.
__device__ __forceinline__ uint32_t probe_unit(int b, int w, int i, uint32_t window, bool priv, int nb) {
  if (priv) {
    const uint32_t per = (window / (uint32_t)nb) & ~1023u;
    return (uint32_t)b * per + (uint32_t)(((uint64_t)(i * kProbeWaves + w) * 1024u) % per);
  }
  return (uint32_t)(((uint64_t)(i * kProbeWaves + w) * 1024u + (uint64_t)b * 37u * 1024u) % window);
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void probe_dma16(__amdgpu_buffer_rsrc_t srd, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(srd), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <bool DMA>
__global__ __launch_bounds__(kProbeWaves * kWave) void fetch_probe_kernel(const unsigned char* __restrict__ buf,
                                                                          uint32_t window, int priv, int iters,
                                                                          unsigned long long* __restrict__ cycles) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int w = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int b = blockIdx.x, nb = gridDim.x;
  __syncthreads();
  const unsigned long long t0 = clock64();
  if (DMA) {
    const __amdgpu_buffer_rsrc_t srd = make_rsrc(buf, window);
    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
    for (int i = 0; i < iters; ++i) {
      // ring of 16 KB-sized wave slots: (i % 16) * 8 KB + w KB
      probe_dma16(srd, probe_unit(b, w, i, window, priv, nb) + lane * 16, lds0 + ((i & 15) * kProbeWaves + w) * 1024);
      if (i >= kProbeDepth - 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kProbeDepth - 1) : "memory");
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    uint4 r[kProbeDepth];
    uint32_t acc = 0;
    const int rounds = iters / kProbeDepth;
#pragma unroll
    for (int j = 0; j < kProbeDepth; ++j)
      r[j] = *reinterpret_cast<const uint4*>(buf + probe_unit(b, w, j, window, priv, nb) + lane * 16);
    for (int q = 1; q < rounds; ++q) {
#pragma unroll
      for (int j = 0; j < kProbeDepth; ++j) {
        acc ^= r[j].x ^ r[j].y ^ r[j].z ^ r[j].w;
        r[j] = *reinterpret_cast<const uint4*>(buf + probe_unit(b, w, q * kProbeDepth + j, window, priv, nb) + lane * 16);
      }
    }
#pragma unroll
    for (int j = 0; j < kProbeDepth; ++j) acc ^= r[j].x ^ r[j].y ^ r[j].z ^ r[j].w;
    if (acc == 0x9e3779b9u) lds[threadIdx.x] = 1;  // keeps the loads
  }
  const unsigned long long t1 = clock64();
  __syncthreads();
  if (threadIdx.x == 0) cycles[b] = t1 - t0;
}

// MFMA issue rate with no memory traffic: 8 waves per CU, each running
// `iters` rounds of 8 independent MFMAs on register operands (bf16:
// v_mfma_f32_16x16x32_bf16; E4M3: v_mfma_scale_f32_32x32x64_f8f6f4 with unit
// scales), with s_memtime ticks per block. The accumulators are
// stored once so the work is kept.
template <bool FP8>
__global__ __launch_bounds__(kProbeWaves * kWave) void mfma_probe_kernel(int iters, float* __restrict__ sink,
                                                                         unsigned long long* __restrict__ cycles) {
  const int lane = threadIdx.x & (kWave - 1);
  __syncthreads();
  const unsigned long long t0 = clock64();
  float keep = 0.f;
  if (FP8) {
    i32x8_t a, b;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      a[q] = 0x38383838 ^ (lane << q);  // E4M3 bytes around 1.0
      b[q] = 0x30303030 ^ (q << 8);
    }
    f32x16_t acc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][r] = 0.f;
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int m = 0; m < 8; ++m)
        acc[m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[m], 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int m = 0; m < 8; ++m) keep += acc[m][lane & 15];
  } else {
    bf16x8_t a, b;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      a[q] = (__bf16)(1.0f + 0.001f * (float)(lane + q));
      b[q] = (__bf16)(0.5f - 0.001f * (float)q);
    }
    f32x4_t acc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[m], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < 8; ++m) keep += acc[m][lane & 3];
  }
  const unsigned long long t1 = clock64();
  sink[blockIdx.x * blockDim.x + threadIdx.x] = keep;
  __syncthreads();
  if (threadIdx.x == 0) cycles[blockIdx.x] = t1 - t0;
}

}  // namespace

moe_status launch_mfma_probe(int fp8, int iters, float* sink, unsigned long long* cycles, int ncu, hipStream_t s) {
  if (fp8)
    hipLaunchKernelGGL((mfma_probe_kernel<true>), dim3(ncu), dim3(kProbeWaves * kWave), 0, s, iters, sink, cycles);
  else
    hipLaunchKernelGGL((mfma_probe_kernel<false>), dim3(ncu), dim3(kProbeWaves * kWave), 0, s, iters, sink, cycles);
  return launch_status();
}

int probe_device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

// ncu: the device's compute units (one block each).
moe_status launch_fetch_probe(const void* buf, size_t bytes, int mode, int shared_window, int kb_per_wave,
                              unsigned long long* cycles, int ncu, hipStream_t s) {
  const int iters = kb_per_wave;
  if (mode == 0) {
    static bool attr = false;
    if (!attr) {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&fetch_probe_kernel<true>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kProbeLds);
      attr = true;
    }
    hipLaunchKernelGGL((fetch_probe_kernel<true>), dim3(ncu), dim3(kProbeWaves * kWave), kProbeLds, s,
                       (const unsigned char*)buf, (uint32_t)bytes, shared_window ? 0 : 1, iters, cycles);
  } else {
    static bool attr = false;
    if (!attr) {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&fetch_probe_kernel<false>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kProbeLds);
      attr = true;
    }
    hipLaunchKernelGGL((fetch_probe_kernel<false>), dim3(ncu), dim3(kProbeWaves * kWave), kProbeLds, s,
                       (const unsigned char*)buf, (uint32_t)bytes, shared_window ? 0 : 1, iters, cycles);
  }
  return launch_status();
}

}  // namespace moe
