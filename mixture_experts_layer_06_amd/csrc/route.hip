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
// MFMAs) and the token rows as the column operand. A block owns 16, 32 or
// 64 tokens (more when there are many experts and many tokens, so that the
// weights are read once for more rows) and a range of H. It copies the
// router weights of its range into LDS with 16-byte loads, in slabs when
// they do not fit; its waves take interleaved 32-wide chunks of the range,
// keep the 16-byte token loads of several chunks in flight, read the
// weight rows of a chunk from LDS (8 consecutive h of 4 adjacent experts
// per lane) and transpose them in registers into four fragments, MFMA j's
// row i being expert 4i+j. The waves' partial scores are summed in a fixed
// order in LDS. Loading the weights per chunk from global memory instead
// made the address unit the bottleneck (8 weight loads per token load).
// With at most 16 experts and H not split, route_small_kernel instead gives
// each wave only the weight rows of its own chunks and one MFMA per chunk
// (experts as the 16 rows), with no block barrier before the multiply.
//
// With few token tiles (decode) H is split over S blocks per tile so that
// W_r streams through many CUs: each block writes its fp32 partial scores
// to the workspace and a second kernel sums the S partials in split order
// before selection, one wave per token. fp32: plain FMA dot products (the
// fp32 layer is a small-shape correctness configuration).
//
// Top-k is K rounds of a register-only argmax: the largest score among the
// experts not yet taken (DPP max across the lanes) and, among the experts
// holding it, the lowest index, so larger score wins and equal scores go to
// the lower expert index. With at most 64 experts a wave selects four
// tokens at once, one per 16-lane row.
#include "dispatch.h"


namespace moe {
namespace {

constexpr int kTok = 16;   // tokens per block
constexpr int kWaves = 4;  // waves per block
constexpr int kChunk = 32; // h per MFMA step

// Wave-wide max / min through DPP lane moves (quad permutes, row mirrors,
// then the row broadcasts of lanes 15 and 31), read from lane 63.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_mov(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, ROWS, 0xf, false);
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __int_as_float(dpp_mov<0xB1, 0xf>(__float_as_int(v))));   // quad_perm 1,0,3,2
  v = fmaxf(v, __int_as_float(dpp_mov<0x4E, 0xf>(__float_as_int(v))));   // quad_perm 2,3,0,1
  v = fmaxf(v, __int_as_float(dpp_mov<0x141, 0xf>(__float_as_int(v))));  // row_half_mirror
  v = fmaxf(v, __int_as_float(dpp_mov<0x140, 0xf>(__float_as_int(v))));  // row_mirror
  v = fmaxf(v, __int_as_float(dpp_mov<0x142, 0xa>(__float_as_int(v))));  // row_bcast:15
  v = fmaxf(v, __int_as_float(dpp_mov<0x143, 0xc>(__float_as_int(v))));  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ int wave_min(int v) {
  v = min(v, dpp_mov<0xB1, 0xf>(v));
  v = min(v, dpp_mov<0x4E, 0xf>(v));
  v = min(v, dpp_mov<0x141, 0xf>(v));
  v = min(v, dpp_mov<0x140, 0xf>(v));
  v = min(v, dpp_mov<0x142, 0xa>(v));
  v = min(v, dpp_mov<0x143, 0xc>(v));
  return __builtin_amdgcn_readlane(v, 63);
}

// Top-k + sparse softmax for one token whose E scores sit in LDS row `lg`,
// by a whole wave. Lane l holds experts l + 64i (i < G). K rounds: the
// largest score among the experts not yet taken (wave max), and among the
// experts holding it the lowest index, which goes to the next slot. A NaN
// score (from non-finite inputs) counts as -inf, so every slot names an
// unselected expert in [0, E); the gates of such a token are then
// unspecified. Gates: p_k = exp(v_k - v_0), summed in slot order, times the
// reciprocal of the sum.
__device__ __forceinline__ float nan_to_ninf(float v) { return v == v ? v : -INFINITY; }

template <int G>
__device__ __forceinline__ void topk_softmax_token(const float* lg, int E, int K, bool hb, const float (&bv)[G],
                                                   int32_t* idx_out, float* gate_out) {
  const int lane = threadIdx.x & (kWave - 1);
  float v[G];
  bool alive[G];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int e = lane + kWave * i;
    alive[i] = e < E;
    v[i] = alive[i] ? nan_to_ninf(hb ? lg[e] + bv[i] : lg[e]) : -INFINITY;
  }
  float sv[8];
  int se[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    sv[k] = -INFINITY;
    se[k] = 0;
    if (k < K) {
      // this lane's best live expert (its lowest index among equal scores)
      float best = -INFINITY;
      int bi = -1;
#pragma unroll
      for (int i = 0; i < G; ++i)
        if (alive[i] && (bi < 0 || v[i] > best)) {
          best = v[i];
          bi = i;
        }
      const float m = wave_max(best);
      const bool hit = bi >= 0 && best == m;
      int eb;
      if (G == 1) {
        eb = __ffsll((unsigned long long)__ballot(hit)) - 1;  // lane = expert
      } else {
        eb = wave_min(hit ? lane + kWave * bi : 0x7fffffff);
      }
      sv[k] = m;
      se[k] = eb;
#pragma unroll
      for (int i = 0; i < G; ++i)
        if (lane + kWave * i == eb) alive[i] = false;
    }
  }
  const float m = sv[0];
  float s = 0.f, mine = 0.f;
  int my_e = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < K) {
      const float p = expf(sv[k] - m);
      s += p;
      if (k == lane) {
        mine = p;
        my_e = se[k];
      }
    }
  }
  const float inv = 1.0f / s;
  if (lane < K) {
    idx_out[lane] = my_e;
    gate_out[lane] = mine * inv;
  }
}

// The same for four tokens at once, E <= 64: 16-lane row r of the wave
// takes token r (rows at lg + r * stride, present when r < nrow); lane j of
// a row holds experts j + 16i (i < 4). Row max / min through the in-row DPP
// moves only.
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, __int_as_float(dpp_mov<0xB1, 0xf>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_mov<0x4E, 0xf>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_mov<0x141, 0xf>(__float_as_int(v))));
  return fmaxf(v, __int_as_float(dpp_mov<0x140, 0xf>(__float_as_int(v))));
}
__device__ __forceinline__ int row_min(int v) {
  v = min(v, dpp_mov<0xB1, 0xf>(v));
  v = min(v, dpp_mov<0x4E, 0xf>(v));
  v = min(v, dpp_mov<0x141, 0xf>(v));
  return min(v, dpp_mov<0x140, 0xf>(v));
}

// v[i], alive[i]: this lane's scores (bias added, NaN as -inf) of experts
// j + 16i and whether they exist; live: row r names a token. hist (LDS, or
// nullptr): each selected expert's count is incremented.
__device__ __forceinline__ void topk_softmax_rows_core(float (&v)[4], bool (&alive)[4], bool live, int K,
                                                       int32_t* idx_out, float* gate_out, int* hist = nullptr) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane >> 4, j = lane & 15;
  float sv[8];
  int se[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    sv[k] = -INFINITY;
    se[k] = 0;
    if (k < K) {
      float best = -INFINITY;
      int bi = -1;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (alive[i] && (bi < 0 || v[i] > best)) {
          best = v[i];
          bi = i;
        }
      const float m = row_max(best);
      const int eb = row_min(bi >= 0 && best == m ? j + 16 * bi : 0x7fffffff);
      sv[k] = m;
      se[k] = eb;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (j + 16 * i == eb) alive[i] = false;
    }
  }
  const float m = sv[0];
  float s = 0.f, mine = 0.f;
  int my_e = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < K) {
      const float p = expf(sv[k] - m);
      s += p;
      if (k == j) {
        mine = p;
        my_e = se[k];
      }
    }
  }
  const float inv = 1.0f / s;
  if (live && j < K) {
    idx_out[r * K + j] = my_e;
    gate_out[r * K + j] = mine * inv;
    if (hist) atomicAdd(&hist[my_e], 1);
  }
}

__device__ __forceinline__ void topk_softmax_rows(const float* lg, int stride, int nrow, int E, int K, bool hb,
                                                  const float (&bv)[4], int32_t* idx_out, float* gate_out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane >> 4, j = lane & 15;
  const bool live = r < nrow;
  const float* row = lg + (live ? r : 0) * stride;
  float v[4];
  bool alive[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = j + 16 * i;
    alive[i] = e < E;
    v[i] = alive[i] ? nan_to_ninf(hb ? row[e] + bv[i] : row[e]) : -INFINITY;
  }
  topk_softmax_rows_core(v, alive, live, K, idx_out, gate_out);
}

// Fixed-order sum of the nw wave slices (stride `slice` floats) of element p.
__device__ __forceinline__ float sum_slices(const float* part, int p, int nw, int slice) {
  float v[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) v[q] = q < nw ? part[q * slice + p] : 0.f;
  float sc = v[0];
#pragma unroll
  for (int q = 1; q < 16; ++q)
    if (q < nw) sc += v[q];
  return sc;
}

// G = 64-expert groups (E <= 64*G); TF = 16-token fragments per block.
// AL: H % 8 == 0, E % 4 == 0 and aligned rows. Then the block copies the
// router weights of its H range into LDS in slabs of `slab_rows` rows (one
// slab when they fit), with 16-byte loads, and the multiply loop reads them
// from there: its only global loads are the token rows, 16 bytes per lane,
// D chunks of them in flight per wave. Otherwise (unaligned shapes) each
// wave loads its weight fragments with element loads, one chunk at a time.
// Out-of-range buffer loads give 0. Grid: (token tiles of 16*TF, S).
// S == 1: the block selects; S > 1 (TF == 1 only): it writes its partial
// scores to part[s][t][64*G].
// Dynamic LDS: the weight slab during the multiply loop, then the partial
// scores [waves][16*TF][64*G + 4] fp32.
template <int G, int TF, bool AL>
constexpr int route_depth() { return !AL ? 1 : (TF * G == 1 ? 5 : (TF == 4 ? 3 : 2)); }

template <int G, int TF, bool AL>
__global__ __launch_bounds__(G * TF <= 2 ? 1024 : 512) void route_bf16_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr, const float* __restrict__ bias, int T, int H,
    int E, int K, int slab_rows, int32_t* __restrict__ idx, float* __restrict__ gate,
    float* __restrict__ part_out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int EP = 64 * G;
  constexpr int EPS = EP + 4;    // LDS row stride of the partial scores (16 rows per store spread over the banks)
  constexpr int NT = kTok * TF;  // tokens per block
  static_assert(G * TF <= 4, "register budget");
  constexpr int D = route_depth<G, TF, AL>();
  float* part = reinterpret_cast<float*>(smem);
  const int nw = blockDim.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t0 = blockIdx.x * NT;
  const int ntok = min(NT, T - t0);
  const int ci = lane & 15, kq = lane >> 4;
  const int nch = cdiv(H, kChunk);
  const int S = gridDim.y;
  const int cps = cdiv(nch, S);  // chunks per split
  const int c_begin = blockIdx.y * cps, c_end = min(nch, c_begin + cps);

  const __amdgpu_buffer_rsrc_t xs = make_rsrc(x + (int64_t)t0 * H, (uint32_t)ntok * (uint32_t)H * 2u);
  const __amdgpu_buffer_rsrc_t ws = make_rsrc(wr, (uint32_t)H * (uint32_t)E * 2u);

  // Token fragment f of chunk c: token 16f + ci, h = 32c + 8kq .. +7; zeros
  // unless c < cend.
  auto load_x = [&](int c, int f, int cend) -> uint4 {
    const int h = c * kChunk + 8 * kq;
    const bool in = c < cend && h < H;
    if (AL) return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                       xs, ((uint32_t)(16 * f + ci) * (uint32_t)H * 2u + (uint32_t)h * 2u) | (in ? 0u : kOOB), 0, 0));
    uint32_t v[4];
    const int tt = 16 * f + ci;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok0 = in && tt < ntok && h + 2 * i < H, ok1 = in && tt < ntok && h + 2 * i + 1 < H;
      const bf16_t* p = x + (int64_t)(t0 + tt) * H + h + 2 * i;
      v[i] = (ok0 ? (uint32_t)p[0] : 0u) | ((ok1 ? (uint32_t)p[1] : 0u) << 16);
    }
    return make_uint4(v[0], v[1], v[2], v[3]);
  };
  // Weight rows h = 32c + 8kq + r (r < 8) of experts 64g + 4ci .. +3: from the
  // LDS slab holding rows [hs, he) (AL), else from global memory.
  auto load_w = [&](int c, int g, int hs, int he, uint2 raw[8]) {
    const int e0 = 64 * g + 4 * ci;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int h = c * kChunk + 8 * kq + r;
      if (AL) {
        raw[r] = (e0 < E && h < he)
                     ? *reinterpret_cast<const uint2*>(smem + ((size_t)(h - hs) * E + e0) * 2)
                     : make_uint2(0u, 0u);
      } else {
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

  f32x4_t acc[G][4][TF];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int f = 0; f < TF; ++f) acc[g][j][f] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  // Slabs of the H range (AL: slab_rows is a multiple of 32; otherwise one
  // slab). In each, this wave's chunks are cs + w, cs + w + nw, ...; the token
  // loads of D of them are in flight while the oldest is multiplied.
  const int h0 = c_begin * kChunk, h1 = min(H, c_end * kChunk);
  const int step = AL ? slab_rows : (h1 > h0 ? h1 - h0 : 1);
  for (int hs = h0; hs < h1; hs += step) {
    const int he = min(h1, hs + step);
    const int cs = hs / kChunk, ce = cdiv(he, kChunk);
    uint4 xr[D][TF];
    const int c0 = cs + w;
    const int nmine = c0 < ce ? cdiv(ce - c0, nw) : 0;
    auto issue = [&](int i, int slot) {
#pragma unroll
      for (int f = 0; f < TF; ++f) xr[slot][f] = load_x(c0 + i * nw, f, ce);
    };
    // the first token loads are in flight while the slab is copied
#pragma unroll
    for (int i = 0; i < D - 1; ++i) issue(i, i);
    if (AL) {
      // copy rows [hs, he) (contiguous in global memory) into the slab
      constexpr int U = 4;
      const int npiece = cdiv((he - hs) * E * 2, 16);
      const uint32_t gbase = (uint32_t)hs * (uint32_t)E * 2u;
      __syncthreads();  // every wave is done with the previous slab
      for (int p0 = 0; p0 < npiece; p0 += U * (int)blockDim.x) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int p = p0 + u * (int)blockDim.x + (int)threadIdx.x;
          v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                     ws, (gbase + (uint32_t)p * 16u) | (p < npiece ? 0u : kOOB), 0, 0));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int p = p0 + u * (int)blockDim.x + (int)threadIdx.x;
          if (p < npiece) *reinterpret_cast<uint4*>(smem + (size_t)p * 16) = v[u];
        }
      }
      __syncthreads();
    }
    for (int i0 = 0; i0 < nmine; i0 += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        issue(i0 + u + D - 1, (u + D - 1) % D);
        if (i0 + u < nmine) {
          const int c = c0 + (i0 + u) * nw;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            uint2 raw[8];
            load_w(c, g, hs, he, raw);
            uint4 wc[4];
            transpose_8x4_bf16(raw, wc);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int f = 0; f < TF; ++f)
                acc[g][j][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, wc[j]), __builtin_bit_cast(bf16x8_t, xr[u][f]), acc[g][j][f], 0,
                    0, 0);
          }
        }
      }
    }
  }
  if (AL) __syncthreads();  // the partial scores overwrite the slab
  // acc[g][j][f][r]: token 16f + ci, expert 64g + 16kq + 4r + j (this wave's chunks).
#pragma unroll
  for (int f = 0; f < TF; ++f)
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<f32x4_t*>(part + (w * NT + 16 * f + ci) * EPS + 64 * g + 16 * kq + 4 * r) =
            (f32x4_t){acc[g][0][f][r], acc[g][1][f][r], acc[g][2][f][r], acc[g][3][f][r]};
  __syncthreads();
  // Fixed-order sum over waves into the first wave's slice; with S > 1 it
  // goes to the workspace instead (the bias is added at the selection, or
  // after the splits).
  for (int p = threadIdx.x; p < ntok * EP; p += blockDim.x) {
    const int e = p % EP, pl = (p / EP) * EPS + e;
    float sc = sum_slices(part, pl, nw, NT * EPS);
    if (S > 1) part_out[((int64_t)blockIdx.y * T + t0) * EP + p] = sc;
    else part[pl] = sc;
  }
  if (S > 1) return;
  __syncthreads();
  // selection (the bias, if any, is added to the sums here)
  const bool hb = bias != nullptr;
  if (G == 1) {
    float bv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = (lane & 15) + 16 * i;
      bv[i] = (hb && e < E) ? bias[e] : 0.f;
    }
    for (int tt = 4 * w; tt < ntok; tt += 4 * nw)
      topk_softmax_rows(part + tt * EPS, EPS, min(4, ntok - tt), E, K, hb, bv, idx + (int64_t)(t0 + tt) * K,
                        gate + (int64_t)(t0 + tt) * K);
  } else {
    float bv[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int e = lane + kWave * i;
      bv[i] = (hb && e < E) ? bias[e] : 0.f;
    }
    for (int tt = w; tt < ntok; tt += nw)
      topk_softmax_token<G>(part + tt * EPS, E, K, hb, bv, idx + (int64_t)(t0 + tt) * K,
                            gate + (int64_t)(t0 + tt) * K);
  }
}

// Few experts (E <= 16, E % 4 == 0, H % 8 == 0, aligned rows), one block
// per 16 tokens and H not split. One MFMA per 32-wide chunk of H: the 16
// expert rows of W_r^T (rows past E zero) times the 16 token columns, so no
// expert row is padded to 64. Wave w owns chunks [w*cpw, (w+1)*cpw) and
// copies only the weight rows of those chunks (contiguous in W_r) into its
// own LDS slab, so no block barrier precedes the multiply: the weight loads
// and the token loads of a pass of up to small_pass<E_>() chunks are all issued
// at once, then the slab is written and read back in the row operand's
// layout (lane (i, kq): expert i, h = 32c + 8kq .. +7) by the same wave. The
// waves' partial scores (one 16 x 16 fragment each, written over the start
// of the wave's own slab) are summed in wave order by the selecting lanes
// themselves: 16-lane row r of wave w takes token 4w + r, lane j expert j.
// With blk_counts set the block also writes how many of its selections went
// to each expert (row blockIdx.x of E counts), the per-chunk counts of the
// dispatch.
// Chunks per pass: 16 (a wave's 16 token loads and its weight loads of a
// pass all in flight; 8 waves of 16 chunks measured 0.9 us faster than 16
// waves of 8 on the prefill shape), 8 with 16 experts, whose weight loads
// would not fit the register budget of 16 waves.
template <int E_>
constexpr int small_pass() { return E_ <= 12 ? 16 : 8; }

template <int E_>
constexpr int small_slab_bytes() { return small_pass<E_>() * kChunk * E_ * 2; }

// Waves per block: at most 16, and their slabs within 156 KB of LDS.
template <int E_>
constexpr int small_max_waves() { return (156 * 1024) / small_slab_bytes<E_>() < 16 ? (156 * 1024) / small_slab_bytes<E_>() : 16; }

template <int E_>
__global__ __launch_bounds__(1024) void route_small_kernel(const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ wr,
                                                          const float* __restrict__ bias, int T, int H, int K,
                                                          int32_t* __restrict__ idx, float* __restrict__ gate,
                                                          int32_t* __restrict__ blk_counts) {
  static_assert(E_ % 4 == 0 && E_ <= 16, "few experts");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int hist[16];  // the block's selections per expert (blk_counts != nullptr)
  if (threadIdx.x < 16) hist[threadIdx.x] = 0;
  constexpr int kSlab = small_slab_bytes<E_>();
  constexpr int kSmallPass = small_pass<E_>();
  constexpr int kPieces = kSmallPass * kChunk * E_ * 2 / 16;  // 16-byte pieces of a full pass
  constexpr int kPw = kPieces / kWave;                         // per lane
  static_assert(kPieces % kWave == 0 && kSlab >= kTok * 16 * 4, "slab holds a pass and a partial fragment");
  const int nw = blockDim.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t0 = blockIdx.x * kTok;
  const int ntok = min(kTok, T - t0);
  const int ci = lane & 15, kq = lane >> 4;
  const int nch = cdiv(H, kChunk);
  const int cpw = cdiv(nch, nw);
  const int c_begin = w * cpw, c_end = min(nch, c_begin + cpw);
  unsigned char* slab = smem + (size_t)w * kSlab;

  const bool hb = bias != nullptr;
  float bv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = ci + 16 * i;
    bv[i] = (hb && e < E_) ? bias[e] : 0.f;
  }

  const __amdgpu_buffer_rsrc_t xs = make_rsrc(x + (int64_t)t0 * H, (uint32_t)ntok * (uint32_t)H * 2u);
  const __amdgpu_buffer_rsrc_t ws = make_rsrc(wr, (uint32_t)H * (uint32_t)E_ * 2u);
  f32x4_t acc = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  for (int cp = c_begin; cp < c_end; cp += kSmallPass) {
    const int nc = min(kSmallPass, c_end - cp);
    // weight rows [32cp, 32(cp + nc)): pieces past the pass or past W_r read 0
    const int npiece = nc * kChunk * E_ * 2 / 16;
    const uint32_t wbase = (uint32_t)cp * kChunk * E_ * 2u;
    uint4 wv[kPw];
#pragma unroll
    for (int q = 0; q < kPw; ++q) {
      const int pc = lane + kWave * q;
      wv[q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                  ws, (wbase + (uint32_t)pc * 16u) | (pc < npiece ? 0u : kOOB), 0, 0));
    }
    // token ci, h = 32c + 8kq .. +7 (rows past the block's tokens read 0)
    uint4 xr[kSmallPass];
#pragma unroll
    for (int u = 0; u < kSmallPass; ++u) {
      const int h = (cp + u) * kChunk + 8 * kq;
      const bool in = u < nc && h < H;
      xr[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                  xs, ((uint32_t)ci * (uint32_t)H * 2u + (uint32_t)h * 2u) | (in ? 0u : kOOB), 0, 0));
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the pass is issued before the first wait
    // the whole slab is rewritten (zeros past the pass), so chunks past nc
    // multiply zeros by zeros and need no branch
#pragma unroll
    for (int q = 0; q < kPw; ++q)
      *reinterpret_cast<uint4*>(slab + (size_t)(lane + kWave * q) * 16) = wv[q];
    // the slab is this wave's alone: its LDS accesses complete in issue order
    const uint16_t* wl = reinterpret_cast<const uint16_t*>(slab);
    const int ce = ci < E_ ? ci : 0;
#pragma unroll
    for (int u = 0; u < kSmallPass; ++u) {
      uint32_t a[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = u * kChunk + 8 * kq + 2 * r;
        const uint32_t pr = (uint32_t)wl[row * E_ + ce] | ((uint32_t)wl[(row + 1) * E_ + ce] << 16);
        a[r] = ci < E_ ? pr : 0u;
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, make_uint4(a[0], a[1], a[2], a[3])),
                                                   __builtin_bit_cast(bf16x8_t, xr[u]), acc, 0, 0, 0);
    }
  }
  // acc[r]: token ci, expert 4kq + r; the fragment goes over the slab's start
  *reinterpret_cast<f32x4_t*>(slab + (size_t)(ci * 16 + 4 * kq) * 4) = acc;
  __syncthreads();
  // fixed-order sum over the waves by the selecting lanes: 16-lane row r of
  // wave w takes token tt + r, lane j expert j
  const int rr = lane >> 4;
  for (int tt = 4 * w; tt < ntok; tt += 4 * nw) {
    float sc = 0.f;
    for (int q = 0; q < nw; ++q)
      sc += reinterpret_cast<const float*>(smem + (size_t)q * kSlab)[(tt + rr) * 16 + ci];
    float v[4] = {ci < E_ ? nan_to_ninf(hb ? sc + bv[0] : sc) : -INFINITY, -INFINITY, -INFINITY, -INFINITY};
    bool alive[4] = {ci < E_, false, false, false};
    topk_softmax_rows_core(v, alive, rr < min(4, ntok - tt), K, idx + (int64_t)(t0 + tt) * K,
                           gate + (int64_t)(t0 + tt) * K, blk_counts ? hist : nullptr);
  }
  if (blk_counts) {
    __syncthreads();
    if (threadIdx.x < E_) blk_counts[(int64_t)blockIdx.x * E_ + threadIdx.x] = hist[threadIdx.x];
  }
}

// Sum of the S partial score rows of a token (split order), bias, selection:
// one wave per token, lane l owning experts l + 64i. The loads of 16 splits
// are in flight before they are added, in split order.
template <int G>
__global__ __launch_bounds__(256) void route_finish_kernel(const float* __restrict__ part_in, int S,
                                                           const float* __restrict__ bias, int T,
                                                           int E, int K, int32_t* __restrict__ idx,
                                                           float* __restrict__ gate) {
  constexpr int EP = 64 * G;
  __shared__ float lg[4][EP];
  const int w = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * 4 + w;
  const bool live = t < T;
  const float* src = part_in + (int64_t)(live ? t : 0) * EP;
  const int64_t split = (int64_t)T * EP;
  float sc[G];
#pragma unroll
  for (int i = 0; i < G; ++i) sc[i] = 0.f;
  for (int q0 = 0; q0 < S; q0 += 16) {
    float v[G][16];
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
      for (int u = 0; u < 16; ++u) v[i][u] = (live && q0 + u < S) ? src[(q0 + u) * split + lane + 64 * i] : 0.f;
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
      for (int u = 0; u < 16; ++u) sc[i] += v[i][u];
  }
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int e = lane + 64 * i;
    lg[w][e] = (bias && e < E) ? sc[i] + bias[e] : sc[i];
  }
  __syncthreads();
  const float nob[G] = {};
  if (live) topk_softmax_token<G>(lg[w], E, K, false, nob, idx + (int64_t)t * K, gate + (int64_t)t * K);
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
  const float nob[4] = {};
  for (int tt = w; tt < kTok; tt += kWaves) {
    const int t = t0 + tt;
    if (t < T) topk_softmax_token<4>(lg + tt * E, E, K, false, nob, idx + (int64_t)t * K, gate + (int64_t)t * K);
  }
}

// Launch shape of the bf16 router for (T, H, E).
struct RoutePlan {
  int G, TF, S, nw;
  size_t lds;     // dynamic LDS bytes
  int slab_rows;  // W_r rows per LDS slab (aligned path)
};

RoutePlan route_plan(int T, int H, int E) {
  RoutePlan p;
  p.G = E <= 64 ? 1 : (E <= 128 ? 2 : 4);
  const int tiles16 = cdiv(T, kTok);
  // With many experts the router weights (H x E) outweigh a 16-token block's
  // rows: blocks of 32 or 64 tokens read them once for more tokens, while
  // there are still at least as many blocks as CUs.
  p.TF = 1;
  if (E > 16) p.TF = tiles16 >= 4 * 256 ? 4 : (tiles16 >= 2 * 256 ? 2 : 1);
  if (p.TF * p.G > 4) p.TF = 4 / p.G;  // register budget
  const int tiles = cdiv(T, kTok * p.TF);
  const int nch = cdiv(H, kChunk);
  // Fewer token tiles than CUs: split H (powers of two) until there are
  // about as many blocks as CUs, keeping at least 4 chunks per block.
  p.S = 1;
  if (tiles < 256)
    while (tiles * p.S < 256 && nch / (2 * p.S) >= 4) p.S *= 2;
  // waves: one chunk each up to the cap; the partial scores take waves * 16TF * (64G + 4) floats (<= 139 KB)
  const int lds_cap = 32 / (p.TF * p.G);
  const int thr_cap = (p.G * p.TF <= 2 ? 1024 : 512) / kWave;
  const int cap = lds_cap < thr_cap ? lds_cap : thr_cap;
  int nw = cdiv(nch, p.S);
  p.nw = nw < 1 ? 1 : (nw > cap ? cap : nw);
  // LDS: the partial scores, or the weight slab if larger (<= 128 KB); a
  // slab holds whole 32-row chunks of W_r (E * 2 bytes per row)
  const size_t part_bytes = (size_t)p.nw * kTok * p.TF * (64 * p.G + 4) * 4;
  const size_t row_b = (size_t)E * 2;
  const int range_rows = cdiv(nch, p.S) * kChunk;
  size_t slab = (size_t)range_rows * row_b;
  if (slab > 128 * 1024) slab = 128 * 1024;
  p.lds = part_bytes > slab ? part_bytes : slab;
  p.slab_rows = (int)(p.lds / row_b) / kChunk * kChunk;
  return p;
}

template <int G, int TF, bool AL>
void launch_bf16(const RoutePlan& p, const void* x, const void* wr, const float* bias, int T, int H,
                 int E, int K, int32_t* idx, float* gate, float* part, hipStream_t s) {
  const size_t lds = AL ? p.lds : (size_t)p.nw * kTok * TF * (64 * G + 4) * 4;
  static bool attr_done = false;
  if (!attr_done) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&route_bf16_kernel<G, TF, AL>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr_done = true;
  }
  hipLaunchKernelGGL((route_bf16_kernel<G, TF, AL>), dim3(cdiv(T, kTok * TF), p.S), dim3(p.nw * kWave),
                     lds, s, (const bf16_t*)x, (const bf16_t*)wr, bias, T, H, E, K, p.slab_rows, idx, gate, part);
  if (p.S > 1)
    hipLaunchKernelGGL((route_finish_kernel<G>), dim3(cdiv(T, 4)), dim3(256), 0, s, part, p.S, bias, T, E, K,
                       idx, gate);
}

template <int G, bool AL>
void launch_bf16_tf(const RoutePlan& p, const void* x, const void* wr, const float* bias, int T, int H,
                    int E, int K, int32_t* idx, float* gate, float* part, hipStream_t s) {
  if constexpr (G == 4) {
    launch_bf16<G, 1, AL>(p, x, wr, bias, T, H, E, K, idx, gate, part, s);
  } else {
    if (p.TF == 1) launch_bf16<G, 1, AL>(p, x, wr, bias, T, H, E, K, idx, gate, part, s);
    else if (p.TF == 2) launch_bf16<G, 2, AL>(p, x, wr, bias, T, H, E, K, idx, gate, part, s);
    else launch_bf16<G, 4 / G, AL>(p, x, wr, bias, T, H, E, K, idx, gate, part, s);
  }
}

// Waves: up to one pass of chunks each, at most small_max_waves. LDS: one
// slab per wave.
template <int E_>
inline int small_waves(int H) {
  const int nw = cdiv(cdiv(H, kChunk), small_pass<E_>());
  return nw < 1 ? 1 : (nw > small_max_waves<E_>() ? small_max_waves<E_>() : nw);
}

template <int E_>
void launch_small(const void* x, const void* wr, const float* bias, int T, int H, int K, int32_t* idx,
                  float* gate, int32_t* blk_counts, hipStream_t s) {
  const int nw = small_waves<E_>(H);
  const size_t lds = (size_t)nw * small_slab_bytes<E_>();
  static bool attr_done = false;
  if (!attr_done) {
    // small_max_waves slabs at most; the kernel also has a small static array
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&route_small_kernel<E_>),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              small_max_waves<E_>() * small_slab_bytes<E_>());
    attr_done = true;
  }
  hipLaunchKernelGGL((route_small_kernel<E_>), dim3(cdiv(T, kTok)), dim3(nw * kWave), lds, s, (const bf16_t*)x,
                     (const bf16_t*)wr, bias, T, H, K, idx, gate, blk_counts);
}

template <bool AL>
void launch_bf16_e(const RoutePlan& p, const void* x, const void* wr, const float* bias, int T, int H,
                   int E, int K, int32_t* idx, float* gate, float* part, hipStream_t s) {
  if (p.G == 1) launch_bf16_tf<1, AL>(p, x, wr, bias, T, H, E, K, idx, gate, part, s);
  else if (p.G == 2) launch_bf16_tf<2, AL>(p, x, wr, bias, T, H, E, K, idx, gate, part, s);
  else launch_bf16_tf<4, AL>(p, x, wr, bias, T, H, E, K, idx, gate, part, s);
}

}  // namespace

size_t route_ws_bytes(int T, int H, int E, moe_dtype dt) {
  if (dt != MOE_BF16 || T == 0) return 0;
  const RoutePlan p = route_plan(T, H, E);
  return p.S > 1 ? (size_t)p.S * T * 64 * p.G * sizeof(float) : 0;
}

moe_status launch_route(const void* x, const void* wr, moe_dtype dt, const float* bias, int T, int H,
                        int E, int K, int32_t* idx, float* gate, void* ws, hipStream_t s) {
  return launch_route_counted(x, wr, dt, bias, T, H, E, K, idx, gate, ws, s, nullptr, nullptr);
}

moe_status launch_route_counted(const void* x, const void* wr, moe_dtype dt, const float* bias, int T, int H,
                                int E, int K, int32_t* idx, float* gate, void* ws, hipStream_t s,
                                int32_t* blk_counts, int* blk_tokens) {
  if (blk_tokens) *blk_tokens = 0;
  if (T == 0) return MOE_OK;
  if (dt == MOE_BF16) {
    const RoutePlan p = route_plan(T, H, E);
    const bool al = (H % 8 == 0) && (E % 4 == 0) && aligned16(x) && ((uintptr_t)wr & 7u) == 0;
    float* part = reinterpret_cast<float*>(ws);
    if (al && p.S == 1 && E <= 16) {
      if (!blk_tokens) blk_counts = nullptr;
      if (E == 4) launch_small<4>(x, wr, bias, T, H, K, idx, gate, blk_counts, s);
      else if (E == 8) launch_small<8>(x, wr, bias, T, H, K, idx, gate, blk_counts, s);
      else if (E == 12) launch_small<12>(x, wr, bias, T, H, K, idx, gate, blk_counts, s);
      else launch_small<16>(x, wr, bias, T, H, K, idx, gate, blk_counts, s);
      if (blk_counts) *blk_tokens = kTok;
    } else if (al) launch_bf16_e<true>(p, x, wr, bias, T, H, E, K, idx, gate, part, s);
    else launch_bf16_e<false>(p, x, wr, bias, T, H, E, K, idx, gate, part, s);
  } else {
    hipLaunchKernelGGL(route_f32_kernel, dim3(cdiv(T, kTok)), dim3(kWaves * kWave), (size_t)kTok * E * 4, s,
                       (const float*)x, (const float*)wr, bias, T, H, E, K, idx, gate);
  }
  return launch_status();
}

}  // namespace moe
