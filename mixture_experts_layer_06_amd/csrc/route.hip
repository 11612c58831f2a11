// route.hip — router scores, top-k, softmax over the kept k scores.
//
// One score per (token, expert) from the token row and the router weights,
// the K best experts per token, then a softmax restricted to those K scores
// ("Advanced GPU Optimization: How to tech an LLM with CUDA and ROCm? -
// Part 5", section 1.1 "The Router Kernel (Top-k Gating)"; the (N,K) top-K
// index matrix of the SpMM page, section "专家选择的计算过程").
//
// gfx950 design. bf16: the router GEMM runs on v_mfma_f32_16x16x32_bf16
// with the router weights as the row operand (64 experts per group of four
// MFMAs) and the token rows as the column operand. Weights are loaded
// straight from global memory in MFMA layout: a lane reads 8 consecutive h
// of 4 adjacent experts (8 bytes per row) and transposes them in registers
// into four fragments, MFMA j's row i being expert 4i+j; token fragments
// are 16-byte loads. No LDS staging, so every wave keeps the loads of a
// whole 32-wide chunk in flight.
//
// A block owns 16 tokens and a range of H; its
// waves take interleaved 32-wide chunks of the range and their partial
// scores are summed in a fixed order in LDS. With few token tiles (decode)
// H is split over S blocks per tile so that W_r streams through many CUs:
// each block writes its fp32 partial scores to the workspace and a second
// kernel sums the S partials in split order before selection. fp32: plain
// FMA dot products (the fp32 layer is a small-shape correctness
// configuration). Top-k is K rounds of a wave-wide argmax butterfly on
// (score, expert) pairs: larger score wins, equal scores go to the lower
// expert index.
#include "common.h"


namespace moe {
namespace {

constexpr int kTok = 16;   // tokens per block
constexpr int kWaves = 4;  // waves per block
constexpr int kChunk = 32; // h per MFMA step

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
// Called by a whole wave; lane k < K writes slot k. A NaN score (from
// non-finite inputs) counts as -inf, so every round picks an unselected
// expert and the indices stay in [0, E); the gates of such a token are
// then unspecified.
__device__ __forceinline__ void topk_softmax_token(const float* lg, int E, int K, int32_t* idx_out,
                                                   float* gate_out) {
  const int lane = threadIdx.x & (kWave - 1);
  float cand[4];
  bool taken[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = lane + kWave * i;
    const float v = e < E ? lg[e] : -INFINITY;
    cand[i] = v == v ? v : -INFINITY;
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

// G = 64-expert groups (E <= 64*G).
// AL: H % 8 == 0, E % 4 == 0 and aligned rows, so a lane's 16-byte token
// loads and 8-byte weight loads never straddle a row end and can be buffer
// loads (out-of-range reads give 0). Grid: (token tiles, S). S == 1: the
// block selects; S > 1: it writes its partial scores to part[s][t][64*G].
// Dynamic LDS: partial scores [waves][16][64*G] fp32.
template <int G, bool AL>
__global__ __launch_bounds__(G <= 2 ? 1024 : 512) void route_bf16_kernel(const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ wr,
                                                          const float* __restrict__ bias, int T,
                                                          int H, int E, int K,
                                                          int32_t* __restrict__ idx,
                                                          float* __restrict__ gate,
                                                          float* __restrict__ part_out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int EP = 64 * G;
  float* part = reinterpret_cast<float*>(smem);
  const int nw = blockDim.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t0 = blockIdx.x * kTok;
  const int ntok = min(kTok, T - t0);
  const int ci = lane & 15, kq = lane >> 4;
  const int nch = cdiv(H, kChunk);
  const int S = gridDim.y;
  const int cps = cdiv(nch, S);  // chunks per split
  const int c_begin = blockIdx.y * cps, c_end = min(nch, c_begin + cps);

  const __amdgpu_buffer_rsrc_t xs = make_rsrc(x + (int64_t)t0 * H, (uint32_t)ntok * (uint32_t)H * 2u);
  const __amdgpu_buffer_rsrc_t ws = make_rsrc(wr, (uint32_t)H * (uint32_t)E * 2u);
  uint32_t wo[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int e0 = 64 * g + 4 * ci;
    wo[g] = (uint32_t)(kq * 8) * (uint32_t)E * 2u + (uint32_t)e0 * 2u + (e0 < E ? 0u : kOOB);
  }

  // Token fragment of chunk c: token ci, h = 32c + 8kq .. +7.
  auto load_x = [&](int c) -> uint4 {
    const int h = c * kChunk + 8 * kq;
    if (AL) return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                       xs, (uint32_t)ci * (uint32_t)H * 2u + (uint32_t)h * 2u + (h < H ? 0u : kOOB), 0, 0));
    uint32_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok0 = ci < ntok && h + 2 * i < H, ok1 = ci < ntok && h + 2 * i + 1 < H;
      const bf16_t* p = x + (int64_t)(t0 + ci) * H + h + 2 * i;
      v[i] = (ok0 ? (uint32_t)p[0] : 0u) | ((ok1 ? (uint32_t)p[1] : 0u) << 16);
    }
    return make_uint4(v[0], v[1], v[2], v[3]);
  };
  // Weight rows h = 32c + 8kq + r (r < 8) of experts 64g + 4ci .. +3.
  auto load_w = [&](int c, int g, uint2 raw[8]) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (AL) {
        raw[r] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                     ws, wo[g] + (uint32_t)(c * kChunk + r) * (uint32_t)E * 2u, 0, 0));
      } else {
        const int h = c * kChunk + 8 * kq + r, e0 = 64 * g + 4 * ci;
        uint32_t v[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const bool ok0 = h < H && e0 + 2 * i < E, ok1 = h < H && e0 + 2 * i + 1 < E;
          const bf16_t* p = wr + (int64_t)h * E + e0 + 2 * i;
          v[i] = (ok0 ? (uint32_t)p[0] : 0u) | ((ok1 ? (uint32_t)p[1] : 0u) << 16);
        }
        raw[r] = make_uint2(v[0], v[1]);
      }
    }
  };

  f32x4_t acc[G][4];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[g][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  for (int c = c_begin + w; c < c_end; c += nw) {
    uint2 raw[G][8];
    const uint4 xr = load_x(c);
#pragma unroll
    for (int g = 0; g < G; ++g) load_w(c, g, raw[g]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      uint4 wc[4];
      transpose_8x4_bf16(raw[g], wc);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[g][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, wc[j]), __builtin_bit_cast(bf16x8_t, xr), acc[g][j], 0, 0, 0);
    }
  }
  // acc[g][j][r]: token ci, expert 64g + 16kq + 4r + j (this wave's chunks).
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      *reinterpret_cast<f32x4_t*>(part + (w * kTok + ci) * EP + 64 * g + 16 * kq + 4 * r) =
          (f32x4_t){acc[g][0][r], acc[g][1][r], acc[g][2][r], acc[g][3][r]};
  __syncthreads();
  // Fixed-order sum over waves into the first wave's slice; with S > 1 it
  // goes to the workspace instead (bias is added once, after the splits).
  for (int p = threadIdx.x; p < ntok * EP; p += blockDim.x) {
    float sc = part[p];
    for (int q = 1; q < nw; ++q) sc += part[q * kTok * EP + p];
    if (S > 1) {
      part_out[((int64_t)blockIdx.y * T + t0) * EP + p] = sc;
    } else {
      const int e = p % EP;
      if (bias && e < E) sc += bias[e];
      part[p] = sc;
    }
  }
  if (S > 1) return;
  __syncthreads();
  for (int tt = w; tt < ntok; tt += nw)
    topk_softmax_token(part + tt * EP, E, K, idx + (int64_t)(t0 + tt) * K, gate + (int64_t)(t0 + tt) * K);
}

// Sum of the S partial score rows of 16 tokens (split order), bias, selection.
// Each thread sums whole (token, expert) columns; the loads of 8 splits are
// issued before they are added, in split order.
template <int G>
__global__ __launch_bounds__(1024) void route_finish_kernel(const float* __restrict__ part_in, int S,
                                                            const float* __restrict__ bias, int T,
                                                            int E, int K, int32_t* __restrict__ idx,
                                                            float* __restrict__ gate) {
  constexpr int EP = 64 * G;
  __shared__ float lg[kTok * EP];
  const int t0 = blockIdx.x * kTok;
  const int ntok = min(kTok, T - t0);
  const float* src = part_in + (int64_t)t0 * EP;
  const int64_t split = (int64_t)T * EP;
  // each thread owns PPT (token, expert) columns; the loads of 16 splits of
  // all of them are in flight before the adds, which go in split order
  constexpr int PPT = kTok * EP / 1024;
  static_assert(kTok * EP % 1024 == 0, "columns per thread");
  float sc[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) sc[i] = 0.f;
  for (int q0 = 0; q0 < S; q0 += 16) {
    float v[PPT][16];
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = threadIdx.x + 1024 * i;
#pragma unroll
      for (int u = 0; u < 16; ++u) v[i][u] = (q0 + u < S && p < ntok * EP) ? src[(q0 + u) * split + p] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < PPT; ++i)
#pragma unroll
      for (int u = 0; u < 16; ++u) sc[i] += v[i][u];
  }
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int p = threadIdx.x + 1024 * i;
    if (p >= ntok * EP) continue;
    const int e = p % EP;
    float x = sc[i];
    if (bias && e < E) x += bias[e];
    lg[p] = x;
  }
  __syncthreads();
  const int w = threadIdx.x / kWave;
  for (int tt = w; tt < ntok; tt += (int)(blockDim.x / kWave))
    topk_softmax_token(lg + tt * EP, E, K, idx + (int64_t)(t0 + tt) * K, gate + (int64_t)(t0 + tt) * K);
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

// Launch shape of the bf16 router for (T, H, E).
struct RoutePlan {
  int G, S, nw;
};

RoutePlan route_plan(int T, int H, int E) {
  RoutePlan p;
  p.G = E <= 64 ? 1 : (E <= 128 ? 2 : 4);
  const int tiles = cdiv(T, kTok);
  const int nch = cdiv(H, kChunk);
  // Fewer token tiles than CUs: split H (powers of two) until there are
  // about as many blocks as CUs, keeping at least 4 chunks per block.
  p.S = 1;
  if (tiles < 256)
    while (tiles * p.S < 256 && nch / (2 * p.S) >= 4) p.S *= 2;
  // waves: one chunk each up to the cap; LDS holds waves * 16 * 64*G floats (<= 128 KB)
  const int cap = p.G <= 2 ? 16 : 8;
  int nw = cdiv(nch, p.S);
  p.nw = nw < 1 ? 1 : (nw > cap ? cap : nw);
  return p;
}

template <int G, bool AL>
void launch_bf16(const RoutePlan& p, const void* x, const void* wr, const float* bias, int T, int H,
                 int E, int K, int32_t* idx, float* gate, float* part, hipStream_t s) {
  const size_t lds = (size_t)p.nw * kTok * 64 * G * 4;
  static bool attr_done = false;
  if (!attr_done) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&route_bf16_kernel<G, AL>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
    attr_done = true;
  }
  hipLaunchKernelGGL((route_bf16_kernel<G, AL>), dim3(cdiv(T, kTok), p.S), dim3(p.nw * kWave),
                     lds, s, (const bf16_t*)x, (const bf16_t*)wr, bias, T, H, E, K, idx, gate, part);
  if (p.S > 1)
    hipLaunchKernelGGL((route_finish_kernel<G>), dim3(cdiv(T, kTok)), dim3(1024), 0, s, part, p.S, bias,
                       T, E, K, idx, gate);
}

template <bool AL>
void launch_bf16_e(const RoutePlan& p, const void* x, const void* wr, const float* bias, int T, int H,
                   int E, int K, int32_t* idx, float* gate, float* part, hipStream_t s) {
  if (p.G == 1) launch_bf16<1, AL>(p, x, wr, bias, T, H, E, K, idx, gate, part, s);
  else if (p.G == 2) launch_bf16<2, AL>(p, x, wr, bias, T, H, E, K, idx, gate, part, s);
  else launch_bf16<4, AL>(p, x, wr, bias, T, H, E, K, idx, gate, part, s);
}

}  // namespace

size_t route_ws_bytes(int T, int H, int E, moe_dtype dt) {
  if (dt != MOE_BF16 || T == 0) return 0;
  const RoutePlan p = route_plan(T, H, E);
  return p.S > 1 ? (size_t)p.S * T * 64 * p.G * sizeof(float) : 0;
}

moe_status launch_route(const void* x, const void* wr, moe_dtype dt, const float* bias, int T, int H,
                        int E, int K, int32_t* idx, float* gate, void* ws, hipStream_t s) {
  if (T == 0) return MOE_OK;
  if (dt == MOE_BF16) {
    const RoutePlan p = route_plan(T, H, E);
    const bool al = (H % 8 == 0) && (E % 4 == 0) && aligned16(x) && ((uintptr_t)wr & 7u) == 0;
    float* part = reinterpret_cast<float*>(ws);
    if (al) launch_bf16_e<true>(p, x, wr, bias, T, H, E, K, idx, gate, part, s);
    else launch_bf16_e<false>(p, x, wr, bias, T, H, E, K, idx, gate, part, s);
  } else {
    hipLaunchKernelGGL(route_f32_kernel, dim3(cdiv(T, kTok)), dim3(256), (size_t)kTok * E * 4, s,
                       (const float*)x, (const float*)wr, bias, T, H, E, K, idx, gate);
  }
  return launch_status();
}

}  // namespace moe
