// route.hip — router scores, top-k, softmax over the kept k scores.
//
// One score per (token, expert) from the token row and the router weights,
// the K best experts per token, then a softmax restricted to those K scores
// ("Advanced GPU Optimization: How to tech an LLM with CUDA and ROCm? -
// Part 5", section 1.1 "The Router Kernel (Top-k Gating)"; the (N,K) top-K
// index matrix of the SpMM page, section "专家选择的计算过程").
//
// gfx950 design. A block owns 16 tokens (one MFMA column tile). bf16: the
// router GEMM runs on v_mfma_f32_16x16x32_bf16 with the router weights as
// the 16-expert row operand and the token rows as the column operand; the
// four waves of the block split H into interleaved 32-wide chunks, each
// wave stages its chunk of W_r transposed (expert-major, h contiguous) in
// its own LDS slice, and the four partial score tiles are summed in a fixed
// order. fp32: plain FMA dot products (the fp32 layer is a small-shape
// correctness configuration). Top-k is K rounds of a wave-wide argmax
// butterfly on (score, expert) pairs: larger score wins, equal scores go to
// the lower expert index.
#include "common.h"

namespace moe {
namespace {

constexpr int kTok = 16;   // tokens per block
constexpr int kWaves = 4;  // waves per block
constexpr int kChunk = 32; // h per MFMA step
constexpr int kWsPitch = 80; // bytes per staged expert row: 64 data + 16 pad

__device__ __forceinline__ void wave_lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Argmax butterfly: (v,e) is better than (w,f) if v > w, or v == w and e < f.
__device__ __forceinline__ void wave_argmax(float& v, int& e) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float ov = __shfl_xor(v, off, kWave);
    int oe = __shfl_xor(e, off, kWave);
    bool take = (ov > v) || (ov == v && oe < e);
    v = take ? ov : v;
    e = take ? oe : e;
  }
}

// Top-k + sparse softmax for one token whose E scores sit in LDS row `lg`.
// Called by a whole wave; lane k < K writes slot k.
__device__ __forceinline__ void topk_softmax_token(const float* lg, int E, int K, int32_t* idx_out,
                                                   float* gate_out) {
  const int lane = threadIdx.x & (kWave - 1);
  float cand[4];
  bool taken[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = lane + kWave * i;
    cand[i] = e < E ? lg[e] : -INFINITY;
    taken[i] = e >= E;
  }
  float sel_v[8];
  int sel_e[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < K) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int e = lane + kWave * i;
        bool better = !taken[i] && ((cand[i] > bv) || (cand[i] == bv && e < be));
        bv = better ? cand[i] : bv;
        be = better ? e : be;
      }
      wave_argmax(bv, be);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + kWave * i == be) taken[i] = true;
      sel_v[k] = bv;
      sel_e[k] = be;
    } else {
      sel_v[k] = -INFINITY;
      sel_e[k] = 0;
    }
  }
  const float m = sel_v[0];
  float p[8];
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    p[k] = k < K ? expf(sel_v[k] - m) : 0.f;
    s += p[k];
  }
  const float inv = 1.0f / s;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < K && lane == k) {
      idx_out[k] = sel_e[k];
      gate_out[k] = p[k] * inv;
    }
  }
}

// 8 consecutive bf16 of a row, zero beyond `avail` elements (avail may be <= 0).
template <bool VEC>
__device__ __forceinline__ uint4 load_bf16x8(const bf16_t* p, int avail) {
  if (VEC) {
    if (avail >= 8) return *reinterpret_cast<const uint4*>(p);
    return make_uint4(0, 0, 0, 0);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = (2 * i < avail) ? p[2 * i] : 0u;
      uint32_t hi = (2 * i + 1 < avail) ? p[2 * i + 1] : 0u;
      w[i] = lo | (hi << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Transpose an 8x8 block of bf16: in[r] holds row r (8 columns); out[c] gets
// column c (8 rows).
__device__ __forceinline__ void transpose8x8_bf16(const uint4 in[8], uint4 out[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    uint32_t d[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&in[2 * p]);
      const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&in[2 * p + 1]);
      d[p] = perm_b32(r1[c >> 1], r0[c >> 1], sel);
    }
    out[c] = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

// ET = number of 16-expert tiles (E <= 16*ET). Dynamic LDS:
//   region A: max(staged W_r^T: kWaves * 16*ET * kWsPitch, scores: kTok * 16*ET * 4)
//   region B: partial scores kWaves * kTok * 16*ET * 4
template <int ET, bool VEC>
__global__ __launch_bounds__(256) void route_bf16_kernel(const bf16_t* __restrict__ x,
                                                         const bf16_t* __restrict__ wr,
                                                         const float* __restrict__ bias, int T,
                                                         int H, int E, int K,
                                                         int32_t* __restrict__ idx,
                                                         float* __restrict__ gate) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int EP = 16 * ET;
  constexpr int regionA = (kWaves * EP * kWsPitch > kTok * EP * 4) ? kWaves * EP * kWsPitch
                                                                    : kTok * EP * 4;
  unsigned char* ws_all = smem;
  float* part = reinterpret_cast<float*>(smem + regionA);  // [kWaves][kTok][EP]
  float* lg = reinterpret_cast<float*>(smem);             // [kTok][EP], after the GEMM

  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int t0 = blockIdx.x * kTok;
  unsigned char* ws = ws_all + w * EP * kWsPitch;

  f32x4_t acc[ET];
#pragma unroll
  for (int i = 0; i < ET; ++i) acc[i] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  const int tok = t0 + (lane & 15);
  const int kq = lane >> 4;  // which 8-wide h slice of the 32-wide chunk
  const int nch = cdiv(H, kChunk);
  for (int c = w; c < nch; c += kWaves) {
    const int h0 = c * kChunk;
    // Stage W_r[h0 : h0+32, 0:E] transposed into ws[e][h] (h contiguous).
    if (VEC) {
      // units of 8 h x 8 experts: 4 h-blocks x 2*ET expert-blocks
      for (int u = lane; u < 4 * 2 * ET; u += kWave) {
        const int hb = u & 3, eb = u >> 2;
        uint4 rows[8], cols[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int h = h0 + hb * 8 + r;
          const bool ok = h < H && eb * 8 < E;
          rows[r] = ok ? *reinterpret_cast<const uint4*>(wr + (int64_t)h * E + eb * 8)
                       : make_uint4(0, 0, 0, 0);
        }
        transpose8x8_bf16(rows, cols);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<uint4*>(ws + (eb * 8 + j) * kWsPitch + hb * 16) = cols[j];
      }
    } else {
      for (int p = lane; p < EP * kChunk; p += kWave) {
        const int e = p / kChunk, hh = p % kChunk;
        const int h = h0 + hh;
        bf16_t v = (h < H && e < E) ? wr[(int64_t)h * E + e] : (bf16_t)0;
        *reinterpret_cast<bf16_t*>(ws + e * kWsPitch + hh * 2) = v;
      }
    }
    wave_lds_fence();
    // Token fragment straight from global: lane -> token (lane&15), h slice kq.
    const int hs = h0 + kq * 8;
    uint4 xr = (tok < T) ? load_bf16x8<VEC>(x + (int64_t)tok * H + hs, H - hs) : make_uint4(0, 0, 0, 0);
    bf16x8_t xb = *reinterpret_cast<bf16x8_t*>(&xr);
#pragma unroll
    for (int et = 0; et < ET; ++et) {
      uint4 wv = *reinterpret_cast<const uint4*>(ws + (et * 16 + (lane & 15)) * kWsPitch + kq * 16);
      bf16x8_t wb = *reinterpret_cast<bf16x8_t*>(&wv);
      acc[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb, xb, acc[et], 0, 0, 0);
    }
    wave_lds_fence();
  }
  // acc[et][j]: expert et*16 + 4*(lane>>4) + j, token lane&15 (this wave's H share).
#pragma unroll
  for (int et = 0; et < ET; ++et)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      part[(w * kTok + (lane & 15)) * EP + et * 16 + 4 * (lane >> 4) + j] = acc[et][j];
  __syncthreads();
  for (int p = threadIdx.x; p < kTok * EP; p += blockDim.x) {
    const int tt = p / EP, e = p % EP;
    float s = part[(0 * kTok + tt) * EP + e];
#pragma unroll
    for (int q = 1; q < kWaves; ++q) s += part[(q * kTok + tt) * EP + e];
    if (bias && e < E) s += bias[e];
    lg[tt * EP + e] = s;
  }
  __syncthreads();
  for (int tt = w; tt < kTok; tt += kWaves) {
    const int t = t0 + tt;
    if (t < T) topk_softmax_token(lg + tt * EP, E, K, idx + (int64_t)t * K, gate + (int64_t)t * K);
  }
}

// fp32: one thread per (token, expert) pair, sequential fp32 FMA over h.
__global__ __launch_bounds__(256) void route_f32_kernel(const float* __restrict__ x,
                                                        const float* __restrict__ wr,
                                                        const float* __restrict__ bias, int T, int H,
                                                        int E, int K, int32_t* __restrict__ idx,
                                                        float* __restrict__ gate) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* lg = reinterpret_cast<float*>(smem);  // [kTok][E]
  const int t0 = blockIdx.x * kTok;
  for (int p = threadIdx.x; p < kTok * E; p += blockDim.x) {
    const int tt = p / E, e = p % E;
    const int t = t0 + tt;
    float s = 0.f;
    if (t < T) {
      const float* xr = x + (int64_t)t * H;
      for (int h = 0; h < H; ++h) s = fmaf(xr[h], wr[(int64_t)h * E + e], s);
    }
    if (bias) s += bias[e];
    lg[tt * E + e] = s;
  }
  __syncthreads();
  const int w = threadIdx.x / kWave;
  for (int tt = w; tt < kTok; tt += kWaves) {
    const int t = t0 + tt;
    if (t < T) topk_softmax_token(lg + tt * E, E, K, idx + (int64_t)t * K, gate + (int64_t)t * K);
  }
}

template <int ET, bool VEC>
void launch_bf16(const void* x, const void* wr, const float* bias, int T, int H, int E, int K,
                 int32_t* idx, float* gate, hipStream_t s) {
  constexpr int EP = 16 * ET;
  constexpr int regionA = (kWaves * EP * kWsPitch > kTok * EP * 4) ? kWaves * EP * kWsPitch
                                                                    : kTok * EP * 4;
  const size_t lds = regionA + (size_t)kWaves * kTok * EP * 4;
  static bool attr_done = false;
  if (!attr_done) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&route_bf16_kernel<ET, VEC>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr_done = true;
  }
  hipLaunchKernelGGL((route_bf16_kernel<ET, VEC>), dim3(cdiv(T, kTok)), dim3(256), lds, s,
                     (const bf16_t*)x, (const bf16_t*)wr, bias, T, H, E, K, idx, gate);
}

template <bool VEC>
void launch_bf16_e(const void* x, const void* wr, const float* bias, int T, int H, int E, int K,
                   int32_t* idx, float* gate, hipStream_t s) {
  if (E <= 16) launch_bf16<1, VEC>(x, wr, bias, T, H, E, K, idx, gate, s);
  else if (E <= 32) launch_bf16<2, VEC>(x, wr, bias, T, H, E, K, idx, gate, s);
  else if (E <= 64) launch_bf16<4, VEC>(x, wr, bias, T, H, E, K, idx, gate, s);
  else if (E <= 128) launch_bf16<8, VEC>(x, wr, bias, T, H, E, K, idx, gate, s);
  else launch_bf16<16, VEC>(x, wr, bias, T, H, E, K, idx, gate, s);
}

}  // namespace

moe_status launch_route(const void* x, const void* wr, moe_dtype dt, const float* bias, int T, int H,
                        int E, int K, int32_t* idx, float* gate, hipStream_t s) {
  if (T == 0) return MOE_OK;
  if (dt == MOE_BF16) {
    const bool vec = (H % 8 == 0) && (E % 8 == 0);
    if (vec) launch_bf16_e<true>(x, wr, bias, T, H, E, K, idx, gate, s);
    else launch_bf16_e<false>(x, wr, bias, T, H, E, K, idx, gate, s);
  } else {
    hipLaunchKernelGGL(route_f32_kernel, dim3(cdiv(T, kTok)), dim3(256), (size_t)kTok * E * 4, s,
                       (const float*)x, (const float*)wr, bias, T, H, E, K, idx, gate);
  }
  return launch_status();
}

}  // namespace moe
