// permute.hip — dispatch of (token, slot) pairs into per-expert contiguous row
// blocks ("Advanced GPU Optimization ... Part 5", section 1.2, token dispatch;
// per-expert counts as in the count arrays of
// "aclnnQuantGroupedMatMulAlltoAllv"; offsets + perm_src are the CSC form of
// the (T,E) activation mask of the SpMM page).
//
// Placement is stable: inside one expert's block rows follow ascending
// flat index i = t*K + k. Ranks come from in-wave match masks (8 ballots on
// the expert id bits) plus ordered per-chunk prefix sums, never from the
// order in which atomics happen to land, so the result is deterministic.
//
// Index path, A = T*K pairs:
//   A <= kBlockA: one block of up to 16 waves, one launch. Wave w owns the
//   contiguous segment w of the pairs: it counts its segment per expert, a
//   prefix over (wave, expert) gives every wave its first row per expert,
//   and each wave ranks its own segment in order;
//   otherwise: the same three steps over chunks of kChunk pairs in three
//   launches (count per chunk -> one-block scan over (chunk, expert) ->
//   per-chunk rank and write).
// Data path: one block per token reads its row once (16-byte vectors when
// the row pitch allows) and writes it to its K destination rows.
#include "common.h"

namespace moe {
namespace {

constexpr int kChunk = 1024;   // pairs per chunk
constexpr int kBlockA = 16384;  // one-block path up to this many pairs
constexpr int kBlockWaves = 16;

__device__ __forceinline__ int clamp_e(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

// Lanes whose expert equals mine (among lanes with valid = true), via 8 ballots.
__device__ __forceinline__ uint64_t match_mask(int e, bool valid) {
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const uint64_t bal = __ballot(valid && ((e >> b) & 1));
    m &= ((e >> b) & 1) ? bal : ~bal;
  }
  return m;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Counts pairs [begin, end) per expert into hist[0:256] (LDS, zeroed here), by one wave.
__device__ __forceinline__ void count_range(const int32_t* __restrict__ idx, int begin, int end, int E,
                                            int* hist) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int e = lane; e < 256; e += kWave) hist[e] = 0;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  for (int base = begin; base < end; base += kWave) {
    const int i = base + lane;
    const bool valid = i < end;
    const int e = valid ? clamp_e(idx[i], E) : 0;
    const uint64_t m = match_mask(e, valid);
    // the highest lane of each group of equal experts adds the group's size
    if (valid && (m >> lane) == 1ull) hist[e] += __popcll(m);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

// Ranks pairs [begin, end) into rows, starting from run[e] (LDS), by one wave.
__device__ __forceinline__ void rank_range(const int32_t* __restrict__ idx, int begin, int end, int E,
                                           int* run, int32_t* __restrict__ perm_src,
                                           int32_t* __restrict__ perm_dst) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int base = begin; base < end; base += kWave) {
    const int i = base + lane;
    const bool valid = i < end;
    const int e = valid ? clamp_e(idx[i], E) : 0;
    const uint64_t m = match_mask(e, valid);
    const int rank = __popcll(m & lanemask_lt());
    int row = 0;
    if (valid) row = run[e] + rank;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // the highest lane of each group advances the running row
    if (valid && (m >> lane) == 1ull) run[e] += __popcll(m);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (valid) {
      perm_dst[i] = row;
      perm_src[row] = i;
    }
  }
}

// One block: whole index path for A <= kBlockA (see the file header).
__global__ __launch_bounds__(kBlockWaves * kWave) void permute_block_kernel(
    const int32_t* __restrict__ idx, int A, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src, int32_t* __restrict__ perm_dst) {
  __shared__ int hist[kBlockWaves][256];  // count, then first row, per (wave, expert)
  __shared__ int tot[256];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  const int seg = cdiv(A, nw);
  const int begin = min(A, w * seg), end = min(A, begin + seg);
  int* mine = hist[w];
  count_range(idx, begin, end, E, mine);
  __syncthreads();
  // thread e: prefix over waves (segment order), total per expert
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
    for (int q = 0; q < nw; ++q) {
      const int v = hist[q][e];
      hist[q][e] = run;
      run += v;
    }
    tot[e] = run;
  }
  __syncthreads();
  // exclusive scan over experts by wave 0 (4 consecutive experts per lane)
  if (w == 0) {
    int c[4], local = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane * 4 + j;
      c[j] = e < E ? tot[e] : 0;
      local += c[j];
    }
    int run = wave_incl_scan(local) - local;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane * 4 + j;
      if (e < E) {
        counts[e] = c[j];
        offsets[e] = run;
        tot[e] = run;
      }
      run += c[j];
    }
    if (lane == 0) offsets[E] = A;
  }
  __syncthreads();
  for (int e = lane; e < E; e += kWave) mine[e] += tot[e];
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  rank_range(idx, begin, end, E, mine, perm_src, perm_dst);
}

__global__ __launch_bounds__(256) void permute_count_kernel(const int32_t* __restrict__ idx, int A,
                                                            int E, int32_t* __restrict__ chunk_counts) {
  __shared__ int hist[256];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int begin = blockIdx.x * kChunk;
  const int end = min(A, begin + kChunk);
  for (int i = begin + threadIdx.x; i < end; i += blockDim.x) atomicAdd(&hist[clamp_e(idx[i], E)], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) chunk_counts[(int64_t)blockIdx.x * E + e] = hist[e];
}

// One block, thread e (E <= 256): total over chunks, exclusive scan over
// experts, then the running prefix over chunks. Each pass issues the loads
// of 16 chunks before adding them, in chunk order.
__global__ __launch_bounds__(256) void permute_scan_kernel(const int32_t* __restrict__ chunk_counts,
                                                           int nchunks, int E, int A,
                                                           int32_t* __restrict__ chunk_base,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets) {
  constexpr int U = 16;
  __shared__ int wsum[4];
  const int e = threadIdx.x;
  const int lane = e & (kWave - 1), w = e / kWave;
  int tot = 0;
  if (e < E) {
    for (int c0 = 0; c0 < nchunks; c0 += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = c0 + u < nchunks ? chunk_counts[(int64_t)(c0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u) tot += v[u];
    }
  }
  const int incl = wave_incl_scan(tot);
  if (lane == kWave - 1) wsum[w] = incl;
  __syncthreads();
  int excl = incl - tot;
  for (int q = 0; q < w; ++q) excl += wsum[q];
  if (e < E) {
    counts[e] = tot;
    offsets[e] = excl;
    int run = excl;
    for (int c0 = 0; c0 < nchunks; c0 += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = c0 + u < nchunks ? chunk_counts[(int64_t)(c0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (c0 + u < nchunks) chunk_base[(int64_t)(c0 + u) * E + e] = run;
        run += v[u];
      }
    }
  }
  if (e == 0) offsets[E] = A;
}

// Chunk c: four waves count and rank its four quarters; the quarters' first
// rows are the chunk's base plus the counts of the quarters before them.
__global__ __launch_bounds__(256) void permute_rank_kernel(const int32_t* __restrict__ idx, int A, int E,
                                                           const int32_t* __restrict__ chunk_base,
                                                           int32_t* __restrict__ perm_src,
                                                           int32_t* __restrict__ perm_dst) {
  constexpr int kQuarter = kChunk / 4;
  __shared__ int hist[4][256];
  const int w = threadIdx.x / kWave;
  const int begin = min(A, blockIdx.x * kChunk + w * kQuarter);
  const int end = min(A, begin + kQuarter);
  count_range(idx, begin, end, E, hist[w]);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = chunk_base[(int64_t)blockIdx.x * E + e];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int v = hist[q][e];
      hist[q][e] = run;
      run += v;
    }
  }
  __syncthreads();
  rank_range(idx, begin, end, E, hist[w], perm_src, perm_dst);
}

// Row scatter: x_perm[perm_dst[t*K+k]] = x[t]. VB = bytes per access.
template <int VB>
__global__ __launch_bounds__(256) void permute_rows_kernel(const unsigned char* __restrict__ x,
                                                           int64_t row_bytes, int T, int K,
                                                           const int32_t* __restrict__ perm_dst,
                                                           unsigned char* __restrict__ xp) {
  typedef typename std::conditional<VB == 16, uint4,
          typename std::conditional<VB == 8, uint2,
          typename std::conditional<VB == 4, uint32_t,
          typename std::conditional<VB == 2, uint16_t, uint8_t>::type>::type>::type>::type V;
  const int64_t nv = row_bytes / VB;
  for (int t = blockIdx.x; t < T; t += gridDim.x) {
    int dst[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) dst[k] = k < K ? perm_dst[(int64_t)t * K + k] : 0;
    const V* src = reinterpret_cast<const V*>(x + (int64_t)t * row_bytes);
    for (int64_t j = threadIdx.x; j < nv; j += blockDim.x) {
      const V v = src[j];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (k < K) reinterpret_cast<V*>(xp + (int64_t)dst[k] * row_bytes)[j] = v;
    }
  }
}

}  // namespace

size_t permute_ws_bytes(int T, int E, int K) {
  const int64_t A = (int64_t)T * K;
  if (A <= kBlockA) return 0;
  const int64_t nch = cdiv64(A, kChunk);
  return (size_t)(2 * nch * E * sizeof(int32_t));
}

moe_status launch_permute(const int32_t* idx, const void* x, moe_dtype dt, int T, int H, int E, int K,
                          int32_t* counts, int32_t* offsets, int32_t* perm_src, int32_t* perm_dst,
                          void* x_perm, void* ws, hipStream_t s) {
  const int A = T * K;
  if (A <= kBlockA) {
    // about 256 pairs per wave, at most kBlockWaves waves
    int nw = cdiv(A, 256);
    nw = nw < 1 ? 1 : (nw > kBlockWaves ? kBlockWaves : nw);
    hipLaunchKernelGGL(permute_block_kernel, dim3(1), dim3(nw * kWave), 0, s, idx, A, E, counts,
                       offsets, perm_src, perm_dst);
  } else {
    const int nch = cdiv(A, kChunk);
    int32_t* chunk_counts = reinterpret_cast<int32_t*>(ws);
    int32_t* chunk_base = chunk_counts + (int64_t)nch * E;
    hipLaunchKernelGGL(permute_count_kernel, dim3(nch), dim3(256), 0, s, idx, A, E, chunk_counts);
    hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(256), 0, s, chunk_counts, nch, E, A,
                       chunk_base, counts, offsets);
    hipLaunchKernelGGL(permute_rank_kernel, dim3(nch), dim3(256), 0, s, idx, A, E, chunk_base,
                       perm_src, perm_dst);
  }
  if (x && T > 0) {
    const int64_t rb = (int64_t)H * dtype_size(dt);
    const int grid = T < 65536 ? T : 65536;
    const unsigned char* xs = (const unsigned char*)x;
    unsigned char* xd = (unsigned char*)x_perm;
    if (rb % 16 == 0)
      hipLaunchKernelGGL(permute_rows_kernel<16>, dim3(grid), dim3(256), 0, s, xs, rb, T, K, perm_dst, xd);
    else if (rb % 8 == 0)
      hipLaunchKernelGGL(permute_rows_kernel<8>, dim3(grid), dim3(256), 0, s, xs, rb, T, K, perm_dst, xd);
    else if (rb % 4 == 0)
      hipLaunchKernelGGL(permute_rows_kernel<4>, dim3(grid), dim3(256), 0, s, xs, rb, T, K, perm_dst, xd);
    else if (rb % 2 == 0)
      hipLaunchKernelGGL(permute_rows_kernel<2>, dim3(grid), dim3(256), 0, s, xs, rb, T, K, perm_dst, xd);
    else
      hipLaunchKernelGGL(permute_rows_kernel<1>, dim3(grid), dim3(256), 0, s, xs, rb, T, K, perm_dst, xd);
  }
  return launch_status();
}

}  // namespace moe
