// gmm.hip — grouped GEMM over experts whose rows are contiguous blocks:
//   out[r, n] = act( (sum_h a[r,h] * w[ex,h,n]) * a_scale * w_scale ),
//   offsets[ex] <= r < offsets[ex+1]
// (gmmY = (gmmX @ gmmWeight) * gmmXScale * gmmWeightScale,
// "aclnnQuantGroupedMatMulAlltoAllv", section 计算公式; local expert
// execution, "Advanced GPU Optimization ... Part 5", section 1.2).
//
// Weights arrive as (e, Hin, N) with N contiguous, the shape the page gives
// for gmmWeight. MFMA wants both operands contiguous in the reduction
// dimension, so weight data is transposed on its way in: in registers with
// v_perm_b32, or (E4M3 ping-pong kernel) by the transposing LDS read.
//
// Kernels
//  * gmm_pp_kernel (bf16, many rows per expert, aligned): 256 x 256 output
//    tiles, 8 waves of 128 x 64, a 4-slot LDS ring of 32-deep K slices
//    filled by LDS DMA, the two row halves of the tile alternating multiply
//    and memory phases between barriers (ping-pong). Weights are read 8 rows
//    x 4 columns per lane and transposed with v_perm_b32, so MFMA j's row i
//    is output column 4i + j and each lane ends with 16 consecutive output
//    columns; the output tile is staged in LDS and stored as whole rows.
//    An expert's last row piece of at most 32 rows rides on the tile before
//    it, and a small last round of tiles is split 4 ways along K.
//  * gmm_pp8_kernel (E4M3, aligned): the same scheme on 16x16x128 f8f6f4
//    MFMAs with 256 x 128 tiles, 128-deep K slices and a 3-slot ring;
//    weight fragments come from ds_read_b64_tr_b8.
//  * gmm_tiled_kernel (bf16 / E4M3 shapes the DMA kernels do not take:
//    unaligned rows or columns): register-staged 256 x 256 tiles, 128-byte K
//    slices double-buffered in LDS, weights transposed on their way in.
//  * All tiled kernels: per expert ceil(rows/BM) x ceil(N/BN) tiles; the
//    block index is remapped so each of the 8 XCDs gets a contiguous run of
//    tiles, ordered in groups of 8 row tiles so concurrently running tiles
//    share weight and activation panels in that XCD's L2. The grid is an
//    upper bound sized on the host; the real tile count is computed on the
//    device from offsets, and surplus blocks exit at once.
//  * gmm_stream_kernel (bf16, few rows per expert: decode shapes): one wave
//    per (non-empty expert, 64 output columns), no LDS. Lane l loads rows
//    k0+8*(l/16)..+7 of columns n0+4*(l%16)..+3 (8-byte loads), transposes
//    them into 4 fragments and issues 4 MFMAs whose row i means column
//    n0 + 4i + j; every weight byte is read from HBM exactly once and the
//    lane's outputs come out as 16 consecutive columns.
//  * gmm_f32_kernel: fp32 FMA tiles (64 x 64, 4 x 4 per thread), sequential
//    fp32 accumulation over h.
#include <type_traits>

#include "common.h"

namespace moe {
namespace {

// Launch-shape constants (each the measured best of the alternatives named).
// Row tiles per group in the tile order of the bf16 and E4M3 ping-pong
// kernels: 8 for the 256 x 256 bf16 tiles; 4 for the 256 x 128 E4M3 tiles,
// where the ~32 tiles an XCD runs at once then span 4 row x 8 column tiles,
// the split that re-reads the fewest panel bytes.
constexpr int kPpGroup = 8;
constexpr int kPp8Group = 4;
// Pair launch: the E4M3 group's tiles are handed out first, the bf16 group's
// last (on the E4M3 workload with its bf16 shared expert: 0.3% faster than
// the other order, 3 of 3 pairs on one box).
constexpr bool kPairBf16First = false;
// Wave layout of the 256 x 256 register-staged tiled kernel (waves along
// rows x columns).
constexpr int kTiledWavesM = 2, kTiledWavesN = 4;


// ------------------------------------------------------------------ helpers

// Expert offsets (clamped to [0, A]) and the running count of row tiles per
// expert, in LDS: s_off[0..e], s_pre[0..e] (s_pre[q] = tiles before expert q).
// Row tiles of an expert with `rows` rows: ceil(rows / BM), except that a
// last piece of at most FOLD rows rides on the tile before it (that tile
// then has BM < rows <= BM + FOLD).
template <int BM, int FOLD>
__device__ __forceinline__ int row_tiles(int rows) {
  const int t = (rows + BM - 1) / BM;
  const int tail = rows - (t - 1) * BM;
  return (FOLD > 0 && t > 1 && tail <= FOLD) ? t - 1 : t;
}

template <int BM, int FOLD = 0>
__device__ __forceinline__ void load_tile_prefix(const int32_t* __restrict__ offsets, int e, int A,
                                                 int* s_off, int* s_pre) {
  for (int q = threadIdx.x; q <= e; q += blockDim.x) {
    int v = offsets[q];
    s_off[q] = v < 0 ? 0 : (v > A ? A : v);
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    // each lane covers 4 consecutive experts (e <= 256)
    int c[4], local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = lane * 4 + i;
      int rows = q < e ? s_off[q + 1] - s_off[q] : 0;
      rows = rows < 0 ? 0 : rows;
      c[i] = row_tiles<BM, FOLD>(rows);
      local += c[i];
    }
    const int incl = wave_incl_scan(local);
    int run = incl - local;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = lane * 4 + i;
      if (q < e) s_pre[q] = run;
      run += c[i];
    }
    if (lane == kWave - 1) s_pre[e] = incl;  // total row tiles
  }
  __syncthreads();
}

struct Tile {
  int ex, row0, rows, n0;
};

// Source row of grouped row r under a gather (gx.src != nullptr), or -1 when
// the entry's quotient falls outside [0, gx.rows).
__device__ __forceinline__ int gather_src(const RowMap& gx, int r) {
  const int v = gx.src[r];
  const int q = v >= 0 ? v / gx.div : -1;
  return q < gx.rows ? q : -1;
}

// Where grouped row m is stored (row m itself without an output map) and the
// factor it is multiplied by (its gate, else 1); row -1: not stored (a
// destination outside [0, A)).
struct OutRow {
  int64_t row;
  float gate;
};
__device__ __forceinline__ OutRow out_row_of(const RowMap& rm, int64_t m, int d, int A) {
  if (rm.dst == nullptr) return {m, 1.f};
  if (d < 0 || d >= A) return {-1, 0.f};
  return {d, rm.gate != nullptr ? rm.gate[d] : 1.f};
}
__device__ __forceinline__ OutRow out_row(const RowMap& rm, int64_t m, int A) {
  return out_row_of(rm, m, rm.dst != nullptr ? rm.dst[m] : 0, A);
}

// Per-row activation scale of grouped row m (1 without one); a gathered row
// whose index is out of range reads as a zero row, scale 0.
__device__ __forceinline__ float row_scale_of(const RowMap& rm, int m) {
  if (rm.row_scale == nullptr) return 1.f;
  if (rm.src == nullptr) return rm.row_scale[m];
  const int t = gather_src(rm, m);
  return t >= 0 ? rm.row_scale[t] : 0.f;
}

// Logical tile for this block, or false if the block has no work.
// XCD-aware: block p runs on XCD p % 8; XCD x takes logical tiles
// [x*per, (x+1)*per). Inside an expert, tiles go in groups of GM row tiles:
// group-major, then column tile, then row tile.
// Tile of logical index L (0 <= L < s_pre[e] * ntn). Inside an expert,
// tiles go in groups of GM row tiles: group-major, then column tile, then
// row tile.
template <int BM, int BN, int GM, int FOLD = 0>
__device__ __forceinline__ void tile_of(const int* s_off, const int* s_pre, int e, int ntn, int L, Tile& t) {
  const int g = L / ntn;  // global row-tile-major position among s_pre[e] row tiles
  // find expert ex with s_pre[ex] <= g < s_pre[ex+1] (binary search, s_pre non-decreasing)
  int lo = 0, hi = e - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pre[mid] <= g) lo = mid;
    else hi = mid - 1;
  }
  const int ex = lo;
  const int mt = s_pre[ex + 1] - s_pre[ex];
  const int q = L - s_pre[ex] * ntn;  // local index within the expert
  const int grp = q / (GM * ntn);
  const int within = q - grp * GM * ntn;
  const int gsz = min(GM, mt - grp * GM);
  const int nt = within / gsz;
  const int m = grp * GM + within % gsz;
  // every lane computed the same tile: say so, so that tile-derived bases and
  // buffer descriptors live in scalar registers
  t.ex = __builtin_amdgcn_readfirstlane(ex);
  t.row0 = __builtin_amdgcn_readfirstlane(s_off[ex] + m * BM);
  const int left = s_off[ex + 1] - (s_off[ex] + m * BM);  // the last tile takes a folded tail
  t.rows = __builtin_amdgcn_readfirstlane((FOLD > 0 && m == mt - 1) ? left : min(BM, left));
  t.n0 = __builtin_amdgcn_readfirstlane(nt * BN);
}

// Logical tile for this block, or false if the block has no work.
// XCD-aware: block p runs on XCD p % 8; XCD x takes logical tiles
// [x*per, (x+1)*per).
template <int BM, int BN, int GM, int FOLD = 0>
__device__ __forceinline__ bool pick_tile(const int* s_off, const int* s_pre, int e, int N, int p, Tile& t) {
  const int ntn = (N + BN - 1) / BN;
  const int total = s_pre[e] * ntn;
  if (total == 0) return false;
  const int per = (total + 7) / 8;
  const int slot = p >> 3;
  if (slot >= per) return false;
  const int L = (p & 7) * per + slot;
  if (L >= total) return false;
  tile_of<BM, BN, GM, FOLD>(s_off, s_pre, e, ntn, L, t);
  return true;
}

// Work of one block when the last, partial round of tiles may be split
// along K. With total tiles = rounds * ncu + rem and 0 < rem <= ncu/4, the
// first rounds * ncu blocks take whole tiles (XCD-aware as in pick_tile)
// and each of the rem remaining tiles is split over S = 4 blocks, part
// `part` of tile `rtile` (0 <= rtile < rem) taking K slices
// [part*nsteps/S, (part+1)*nsteps/S) (at least 4 each). Otherwise S = 1 and
// this is pick_tile. Measured on the prefill GEMMs: 4-way splits of a
// small remainder gain 12%; 2-way splits of a remainder near ncu/2 lose 2%.
// The host sizes the grid for the extra blocks (at most 3*ncu/4).
constexpr int kMaxSplit = 4;
struct Work {
  int S, part, rtile;
};
template <int BM, int BN, int GM, int FOLD = 0>
__device__ __forceinline__ bool pick_work(const int* s_off, const int* s_pre, int e, int N, int nsteps,
                                          int ncu, bool can_split, int p, Tile& t, Work& wk) {
  const int ntn = (N + BN - 1) / BN;
  const int total = s_pre[e] * ntn;
  wk.S = 1;
  wk.part = 0;
  wk.rtile = 0;
  if (total == 0) return false;
  const int rem = total % ncu;
  const int S = kMaxSplit;
  if (!can_split || rem == 0 || rem * S > ncu || nsteps < 4 * S) return pick_tile<BM, BN, GM, FOLD>(s_off, s_pre, e, N, p, t);
  const int full = total - rem;  // a multiple of ncu, hence of 8
  int L;
  if (p < full) {
    L = (p & 7) * (full >> 3) + (p >> 3);
  } else {
    const int u = p - full;
    if (u >= rem * S) return false;
    L = full + u / S;
    wk.S = S;
    wk.part = u % S;
    wk.rtile = u / S;
  }
  tile_of<BM, BN, GM, FOLD>(s_off, s_pre, e, ntn, L, t);
  return true;
}

// 16 bytes at p; bytes at or beyond `avail` read as zero. AL: p is 16-byte
// aligned and avail is a multiple of 16 (or <= 0).
template <bool AL, int ELEM>
__device__ __forceinline__ uint4 ld16(const unsigned char* p, int avail) {
  if (AL) return avail >= 16 ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
  uint32_t w[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t v = 0;
    if (ELEM == 2) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int b = d * 4 + h * 2;
        if (b < avail) v |= (uint32_t)(*reinterpret_cast<const uint16_t*>(p + b)) << (16 * h);
      }
    } else {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int b = d * 4 + h;
        if (b < avail) v |= (uint32_t)p[b] << (8 * h);
      }
    }
    w[d] = v;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <bool AL, int ELEM>
__device__ __forceinline__ uint2 ld8(const unsigned char* p, int avail) {
  if (AL) return avail >= 8 ? *reinterpret_cast<const uint2*>(p) : make_uint2(0, 0);
  uint32_t w[2];
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    uint32_t v = 0;
    if (ELEM == 2) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int b = d * 4 + h * 2;
        if (b < avail) v |= (uint32_t)(*reinterpret_cast<const uint16_t*>(p + b)) << (16 * h);
      }
    } else {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int b = d * 4 + h;
        if (b < avail) v |= (uint32_t)p[b] << (8 * h);
      }
    }
    w[d] = v;
  }
  return make_uint2(w[0], w[1]);
}

// E4M3: rows r0..r7 of 8 columns (uint2 each, one byte per column) ->
// 8 columns of 8 rows (uint2 each, one byte per row).
__device__ __forceinline__ void transpose_8x8_u8(const uint2 in[8], uint2 out[8]) {
#pragma unroll
  for (int c = 0; c < 8; c += 2) {
    // byte c and c+1 of each row; rows paired (0,1),(2,3),(4,5),(6,7)
    const int d = c >> 2;        // which dword of the row
    const int b = c & 3;         // byte within it (0 or 2)
    // pair[p] = {r2p[c], r2p+1[c], r2p[c+1], r2p+1[c+1]}
    const uint32_t sel_pair = (uint32_t)(b) | ((uint32_t)(4 + b) << 8) | ((uint32_t)(b + 1) << 16) |
                              ((uint32_t)(5 + b) << 24);
    uint32_t pr[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t lo = d ? in[2 * p].y : in[2 * p].x;
      const uint32_t hi = d ? in[2 * p + 1].y : in[2 * p + 1].x;
      pr[p] = perm_b32(hi, lo, sel_pair);
    }
    // column c: {r0,r1,r2,r3} = lo16(pr0) | lo16(pr1)<<16 ; {r4..r7} from pr2, pr3
    out[c].x = perm_b32(pr[1], pr[0], 0x05040100u);
    out[c].y = perm_b32(pr[3], pr[2], 0x05040100u);
    out[c + 1].x = perm_b32(pr[1], pr[0], 0x07060302u);
    out[c + 1].y = perm_b32(pr[3], pr[2], 0x07060302u);
  }
}

__device__ __forceinline__ float ld_scale(const float* p) { return p ? *p : 1.0f; }

// ------------------------------------------------------------------ tiled MFMA kernel

constexpr int kKB = 128;   // K-slice bytes per tile step (64 bf16 or 128 E4M3 values)
constexpr int kRowB = 128; // LDS bytes per tile row (one K slice, no padding)

// LDS byte offset of 16-byte chunk c (0..7) of tile row r. The chunk index is
// XORed with s(r) = (r ^ (r >> 3)) & 7: sixteen consecutive rows read at the
// same logical chunk land on sixteen distinct 16-byte bank groups, and so do
// the eight chunks of one row plus the eight of the next row.
__device__ __forceinline__ int lds_off(int r, int c) {
  return r * kRowB + ((c ^ ((r ^ (r >> 3)) & 7)) << 4);
}


template <int ELEM, int BM, int BN, int WM_, int WN_, bool AL, bool OUT_F32>
struct TiledCfg {
  static constexpr int kElem = ELEM;
  static constexpr int kBM = BM, kBN = BN;
  static constexpr int kWavesM = WM_, kWavesN = WN_;
  static constexpr int kNT = 64 * WM_ * WN_;
  static constexpr int kWM = BM / WM_;  // rows per wave
  static constexpr int kWN = BN / WN_;  // columns per wave
  static constexpr int kFI = kWM / 16, kFJ = kWN / 16;
  static constexpr int kKRows = kKB / ELEM;         // K rows of weights per step
  static constexpr int kKBlk = kKRows / 8;          // 8-row blocks
  static constexpr int kNQ = (BN * ELEM) / 8;       // 8-byte column groups per weight row
  static constexpr int kUnits = kKBlk * kNQ;        // weight load units per step
  static constexpr int kUPT = kUnits / kNT;         // units per thread
  static constexpr int kAChunks = BM * (kKB / 16);  // 16-byte activation chunks per step
  static constexpr int kAPT = kAChunks / kNT;
  static constexpr bool kAligned = AL;
  static constexpr bool kOutF32 = OUT_F32;
  static constexpr int kLdsA = BM * kRowB, kLdsB = BN * kRowB;
  static constexpr int kLds = 2 * (kLdsA + kLdsB);
  static_assert(kUnits % kNT == 0 && kAChunks % kNT == 0, "load split");
};

// AL (16-byte aligned rows, both matrices under 2 GiB per expert): buffer
// loads, the hardware returns zeros outside each tile's valid region.
// !AL: element-wise loads with explicit bounds (odd shapes only).
template <class C>
__global__ __launch_bounds__(C::kNT) void gmm_tiled_kernel(
    const unsigned char* __restrict__ a, const unsigned char* __restrict__ w,
    const float* __restrict__ a_scale, const float* __restrict__ w_scale,
    const int32_t* __restrict__ offsets, int e, int A, int Hin, int N, int relu,
    unsigned char* __restrict__ out, RowMap gx) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_off[257];
  __shared__ int s_pre[257];
  load_tile_prefix<C::kBM>(offsets, e, A, s_off, s_pre);
  Tile tile;
  if (!pick_tile<C::kBM, C::kBN, 8>(s_off, s_pre, e, N, blockIdx.x, tile)) return;

  constexpr int E_ = C::kElem;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::kWavesN, wn = wave % C::kWavesN;
  const int hin_b = Hin * E_;
  const int n_b = N * E_;
  const int n0b = tile.n0 * E_;
  // activation rows: relative to the tile's first row, or (gather) absolute rows of a
  const bool gat = gx.src != nullptr;
  const unsigned char* abase = gat ? a : a + (int64_t)tile.row0 * hin_b;
  const unsigned char* wbase = w + (int64_t)tile.ex * Hin * n_b;
  const int nsteps = (hin_b + kKB - 1) / kKB;

  // buffer: activations at smem + b*(A+B), weights right after them
  auto As = [&](int b) { return smem + b * (C::kLdsA + C::kLdsB); };
  auto Bs = [&](int b) { return smem + b * (C::kLdsA + C::kLdsB) + C::kLdsA; };

  // ---- per-thread load descriptors, fixed for the tile
  __amdgpu_buffer_rsrc_t arsrc, wrsrc;
  if (C::kAligned) {
    arsrc = make_rsrc(abase, (uint32_t)(gat ? gx.rows : tile.rows) * (uint32_t)hin_b);
    wrsrc = make_rsrc(wbase, (uint32_t)Hin * (uint32_t)n_b);
  }
  uint32_t aoff[C::kAPT];
  int alds[C::kAPT], akc[C::kAPT], asrc[C::kAPT];
#pragma unroll
  for (int i = 0; i < C::kAPT; ++i) {
    const int c = tid + i * C::kNT;
    const int row = c >> 3, kc = c & 7;
    // source row, -1 when there is none (past tile.rows or an out-of-range gather entry)
    asrc[i] = row >= tile.rows ? -1 : gat ? gather_src(gx, tile.row0 + row) : row;
    aoff[i] = (asrc[i] >= 0 ? (uint32_t)asrc[i] * (uint32_t)hin_b : kOOB) + kc * 16;
    akc[i] = kc * 16;
    alds[i] = lds_off(row, kc);
  }
  uint32_t woff[C::kUPT];
  int wkr[C::kUPT], wnq[C::kUPT], wkb[C::kUPT];
#pragma unroll
  for (int u = 0; u < C::kUPT; ++u) {
    const int unit = tid + u * C::kNT;
    const int kb = unit % C::kKBlk, nq = unit / C::kKBlk;
    const int nb = n0b + nq * 8;
    woff[u] = (uint32_t)(kb * 8) * (uint32_t)n_b + (uint32_t)nb + (nb < n_b ? 0u : kOOB);
    wkr[u] = kb * 8;
    wnq[u] = nq;
    wkb[u] = kb;
  }

  uint4 ra[C::kAPT];
  uint2 rb[C::kUPT][8];

  auto gload = [&](int step) {
    const int kb0 = step * kKB;
    const int k0 = step * C::kKRows;
    if (C::kAligned) {
#pragma unroll
      for (int i = 0; i < C::kAPT; ++i) {
        const uint32_t o = (aoff[i] + kb0) | (kb0 + akc[i] < hin_b ? 0u : kOOB);
        ra[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(arsrc, o, 0, 0));
      }
      const uint32_t kstep = (uint32_t)k0 * (uint32_t)n_b;
#pragma unroll
      for (int u = 0; u < C::kUPT; ++u)
#pragma unroll
        for (int r = 0; r < 8; ++r)
          rb[u][r] = __builtin_bit_cast(
              uint2, __builtin_amdgcn_raw_buffer_load_b64(wrsrc, woff[u] + kstep + r * n_b, 0, 0));
    } else {
#pragma unroll
      for (int i = 0; i < C::kAPT; ++i) {
        const int rem = hin_b - (kb0 + akc[i]);
        const int avail = asrc[i] >= 0 ? (rem < 16 ? rem : 16) : 0;
        ra[i] = ld16<false, E_>(abase + (int64_t)(asrc[i] >= 0 ? asrc[i] : 0) * hin_b + kb0 + akc[i], avail);
      }
#pragma unroll
      for (int u = 0; u < C::kUPT; ++u) {
        const int nb = n0b + wnq[u] * 8;
        const int remn = n_b - nb;
        const int avail_n = remn < 8 ? remn : 8;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int k = k0 + wkr[u] + r;
          rb[u][r] = ld8<false, E_>(wbase + (int64_t)k * n_b + nb, k < Hin ? avail_n : 0);
        }
      }
    }
  };
  auto lstore = [&](int buf) {
    unsigned char* Ab = As(buf);
    unsigned char* Bb = Bs(buf);
#pragma unroll
    for (int i = 0; i < C::kAPT; ++i) *reinterpret_cast<uint4*>(Ab + alds[i]) = ra[i];
#pragma unroll
    for (int u = 0; u < C::kUPT; ++u) {
      if (E_ == 2) {
        uint4 cols[4];
        transpose_8x4_bf16(rb[u], cols);
        // odd column groups write their four rows in the order 1,0,3,2 so that the
        // two groups sharing a 16-lane phase touch rows of opposite parity
        // (a bitwise select keeps the choice in registers; a ternary on array
        // elements gets turned into a dynamically indexed array in scratch)
        const int odd = wnq[u] & 1;
        const uint32_t msk = 0u - (uint32_t)odd;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 c0 = cols[j], c1 = cols[j ^ 1];
          uint4 v;
          v.x = c0.x ^ ((c0.x ^ c1.x) & msk);
          v.y = c0.y ^ ((c0.y ^ c1.y) & msk);
          v.z = c0.z ^ ((c0.z ^ c1.z) & msk);
          v.w = c0.w ^ ((c0.w ^ c1.w) & msk);
          *reinterpret_cast<uint4*>(Bb + lds_off(wnq[u] * 4 + (j ^ odd), wkb[u])) = v;
        }
      } else {
        uint2 cols[8];
        transpose_8x8_u8(rb[u], cols);
        // 8-byte half of 16-byte chunk (kb >> 1)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<uint2*>(Bb + lds_off(wnq[u] * 8 + j, wkb[u] >> 1) + (wkb[u] & 1) * 8) = cols[j];
      }
    }
  };

  f32x4_t acc[C::kFI][C::kFJ];
#pragma unroll
  for (int i = 0; i < C::kFI; ++i)
#pragma unroll
    for (int j = 0; j < C::kFJ; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  const bool wave_active = (wm * C::kWM < tile.rows) && (tile.n0 + wn * C::kWN < N);
  const int ci = lane & 15, kq = lane >> 4;

  gload(0);
  lstore(0);
  __syncthreads();
  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    if (step + 1 < nsteps) gload(step + 1);
    if (wave_active) {
      const unsigned char* Ab = As(buf);
      const unsigned char* Bb = Bs(buf);
      if (E_ == 2) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int c = kk * 4 + kq;
          bf16x8_t xa[C::kFI], wb[C::kFJ];
#pragma unroll
          for (int i = 0; i < C::kFI; ++i)
            xa[i] = *reinterpret_cast<const bf16x8_t*>(Ab + lds_off(wm * C::kWM + i * 16 + ci, c));
#pragma unroll
          for (int j = 0; j < C::kFJ; ++j)
            wb[j] = *reinterpret_cast<const bf16x8_t*>(Bb + lds_off(wn * C::kWN + j * 16 + ci, c));
#pragma unroll
          for (int i = 0; i < C::kFI; ++i)
#pragma unroll
            for (int j = 0; j < C::kFJ; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[j], xa[i], acc[i][j], 0, 0, 0);
        }
      } else {
        i32x8_t wb[C::kFJ];
#pragma unroll
        for (int j = 0; j < C::kFJ; ++j) {
          const int r = wn * C::kWN + j * 16 + ci;
          const uint4 lo = *reinterpret_cast<const uint4*>(Bb + lds_off(r, 2 * kq));
          const uint4 hi = *reinterpret_cast<const uint4*>(Bb + lds_off(r, 2 * kq + 1));
          wb[j] = (i32x8_t){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                            (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int i = 0; i < C::kFI; ++i) {
          const int r = wm * C::kWM + i * 16 + ci;
          const uint4 lo = *reinterpret_cast<const uint4*>(Ab + lds_off(r, 2 * kq));
          const uint4 hi = *reinterpret_cast<const uint4*>(Ab + lds_off(r, 2 * kq + 1));
          const i32x8_t xa = (i32x8_t){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
          for (int j = 0; j < C::kFJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wb[j], xa, acc[i][j], 0, 0, 0,
                                                                         0, 0, 0);
        }
      }
    }
    if (step + 1 < nsteps) lstore(buf ^ 1);
    __syncthreads();
  }

  if (!wave_active) return;
  const float sc = ld_scale(a_scale) * ld_scale(w_scale);
#pragma unroll
  for (int i = 0; i < C::kFI; ++i) {
    const int ml = wm * C::kWM + i * 16 + ci;
    if (ml >= tile.rows) continue;
    const OutRow orow = out_row(gx, tile.row0 + ml, A);
    if (orow.row < 0) continue;
    const int64_t m = orow.row;
    const float rsc = gx.row_scale != nullptr ? row_scale_of(gx, tile.row0 + ml) * sc : sc;
#pragma unroll
    for (int j = 0; j < C::kFJ; ++j) {
      const int n = tile.n0 + wn * C::kWN + j * 16 + 4 * kq;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = acc[i][j][r] * rsc;
        if (relu) v[r] = v[r] > 0.f ? v[r] : 0.f;
        v[r] *= orow.gate;
      }
      if (C::kOutF32) {
        float* o = reinterpret_cast<float*>(out) + m * N + n;
        if (C::kAligned && n + 3 < N) {
          *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) o[r] = v[r];
        }
      } else {
        bf16_t* o = reinterpret_cast<bf16_t*>(out) + m * N + n;
        if (C::kAligned && n + 3 < N) {
          *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) o[r] = f32_to_bf16(v[r]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ LDS DMA helpers
//
// gfx950 LDS DMA: buffer_load_dwordx4 ... lds moves 16 bytes per lane from
// global memory straight into LDS at M0 + 16*lane, with no staging
// registers; out-of-range buffer offsets write zeros. Every DMA instruction
// of the ping-pong kernels fills one contiguous KB of a ring slot; the
// swizzles live in which global bytes each lane fetches.

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDmaKB = 64;  // K bytes per stage: 32 bf16

__device__ __forceinline__ u32x4_t make_srd(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  u32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane((uint32_t)b);
  r.y = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) & 0xffffu;  // stride 0
  r.z = __builtin_amdgcn_readfirstlane(bytes);                          // loads past it read 0
  r.w = 0x00020000u;                                                    // 32-bit data format
  return r;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from buffer offset voff into LDS at lds_base + 16*lane
// (lds_base wave-uniform). The compiler does not see these loads, so the
// kernel waits for them itself with wait_vmcnt.
__device__ __forceinline__ void dma16(u32x4_t srd, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(srd), "s"(lds_base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// 4 bytes per lane from buffer offset voff into LDS at lds_base + 4*lane.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma4(u32x4_t srd, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(srd), "s"(lds_base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}


// ------------------------------------------------------------------ ping-pong bf16 kernel
//
// 256 x 256 output tile, 8 waves of 128 x 64. The K dimension is walked in
// 32-wide slices that stream through an S-slot LDS ring filled by
// buffer_load ... lds (each wave moves an equal share of every slice:
// activations 256 rows x 64 B, weights 32 rows x 512 B). Weights are read
// untransposed (8 rows x 4 columns per lane) and transposed in registers, so
// MFMA row i of fragment j is output column 4i+j and a lane ends with 16
// consecutive output columns.
//
// LDS layout. gfx950 serves a 16-byte-per-lane LDS read over 64 four-byte
// banks in four passes, each pass taking two groups of 8 lanes (lanes 0-7
// with 16-23, 8-15 with 24-31, and so on; measured: a pattern that is
// conflict-free under that pairing reads at the full 256 B/clk, the others
// at half). An activation fragment read has lane l on row l%16, 16-byte
// chunk l/16, so one pass covers rows r..r+7 and two adjacent chunks; with
// 64-byte rows, rows r and r+4 share banks. The chunk index is therefore
// XORed with (row/2)%4, which gives the four (row, chunk) pairs of each bank
// group distinct banks. Weight rows (512 B) keep their 128-byte segments
// XORed with (row/8)%4, so the 8-byte reads of the four 8-row groups of a
// slice fall in distinct banks.
//
// The two row halves of the tile (waves 0-3 and 4-7: one wave of each on
// every SIMD) run out of phase. Between two barriers one half multiplies a
// whole K slice while the other reads its next fragments from LDS and issues
// its share of the DMA; at the barrier they swap, so each SIMD's matrix pipe
// is fed by one wave while its partner works on memory.
//
// Barrier k = 0, 1, ...: the first half reads slice u between barriers 2u
// and 2u+1 and multiplies it between 2u+1 and 2u+2; the second half reads it
// between 2u+1 and 2u+2 and multiplies it between 2u+2 and 2u+3. While
// reading slice u each wave issues its share of slice u+S-1, which goes to
// the slot of slice u-1, read by both halves before barrier 2u. Slice t must
// have landed by barrier 2t: each wave waits for its share of t, leaving the
// shares of t+1 .. t+S-2 in flight. Barriers and the ring never depend on
// data, so a wave whose part of the tile is empty runs the same schedule
// without reads or multiplies.

template <int BM, int BN, int WM_, int WN_, int STAGES>
struct PpCfg {
  static constexpr int kStages = STAGES;
  static constexpr int kBM = BM, kBN = BN;
  static constexpr int kFold = 32;  // tail rows an expert's last tile may carry beyond BM
  static constexpr int kSegMask = (BN * 2) / 128 - 1;  // 128-byte segments per weight row - 1
  static constexpr int kWavesM = WM_, kWavesN = WN_;
  static constexpr int kNT = 64 * WM_ * WN_;
  static constexpr int kWM = BM / WM_, kWN = BN / WN_;
  static constexpr int kFI = kWM / 16;   // 16-row activation fragments per wave
  static constexpr int kFG = kWN / 64;   // 64-column weight groups per wave
  static constexpr int kLdsA = BM * kDmaKB;                 // activations per slot
  static constexpr int kLdsX = (BM + kFold) * kDmaKB;       // ... with the folded tail rows
  static constexpr int kLdsW = 32 * BN * 2;                 // weights per slot
  static constexpr int kStage = kLdsX + kLdsW;
  static constexpr int kRing = STAGES * kStage;
  static constexpr int kOutRow = BN * 2 + 16;                // bytes per row of the staged output tile
  static constexpr int kOut = (BM + kFold) * kOutRow;
  static constexpr int kLds = kRing > kOut ? kRing : kOut;  // 148.5 KB for 256 x 256
  static constexpr int kADma = kLdsA / 1024 / (kNT / 64);  // 1 KB DMA ops per wave per slot
  static constexpr int kWDma = kLdsW / 1024 / (kNT / 64);
  static constexpr int kPerStage = kADma + kWDma;          // vmcnt units per slot per lane
  static_assert(kLdsA % (1024 * (kNT / 64)) == 0 && kLdsW % (1024 * (kNT / 64)) == 0, "dma split");
  static_assert(kWN % 64 == 0, "weight groups");
  static_assert(WM_ == 2 && kFold == 16 * WM_, "two row halves, one tail fragment each");
  static_assert(STAGES >= 3 && (STAGES - 2) * (kPerStage + 1) <= 63, "ring depth");
  static_assert(kLds >= 2 * 257 * 4, "tile prefix lives in the ring");
};
// The bf16 configuration: 256 x 256 tiles, 2 x 4 waves, a 4-slot ring.
typedef PpCfg<256, 256, 2, 4, 4> PpBf16;

// The kernel's work for block p (smem: the dynamic LDS ring; s_last: an LDS
// flag of the block).
template <class C>
__device__ __forceinline__ bool pp_block(
    unsigned char* smem, int& s_last, int p, const unsigned char* __restrict__ a,
    const unsigned char* __restrict__ w, const float* __restrict__ a_scale, const float* __restrict__ w_scale,
    const int32_t* __restrict__ offsets, int e, int A, int Hin, int N, int relu,
    bf16_t* __restrict__ out, float* __restrict__ split_ws, int* __restrict__ split_cnt, int ncu,
    const RowMap& gx, const int* s_tab = nullptr) {
  // The tile prefix: in s_tab when the caller computed it (outside the
  // ring), else in the ring's first bytes before any DMA is issued.
  if (s_tab == nullptr) {
    int* s_off = reinterpret_cast<int*>(smem);
    int* s_pre = s_off + 257;
    load_tile_prefix<C::kBM, C::kFold>(offsets, e, A, s_off, s_pre);
  }
  const int* tab = s_tab != nullptr ? s_tab : reinterpret_cast<const int*>(smem);
  const int hin_b = Hin * 2;
  const int nsteps_all = (hin_b + kDmaKB - 1) / kDmaKB;
  Tile tile;
  Work wk;
  if (!pick_work<C::kBM, C::kBN, kPpGroup, C::kFold>(tab, tab + 257, e, N, nsteps_all, ncu, split_ws != nullptr, p,
                                                       tile, wk))
    return false;
  __syncthreads();  // every lane has its tile before the ring overwrites the prefix
  // K slices of this block: all of them, or part wk.part of wk.S
  const int ks0 = wk.part * nsteps_all / wk.S;
  const int ks1 = (wk.part + 1) * nsteps_all / wk.S;
  const int kext_b = (hin_b < ks1 * kDmaKB ? hin_b : ks1 * kDmaKB) - ks0 * kDmaKB;  // K bytes of the range
  // An expert's last tile may carry up to kFold tail rows beyond BM: then
  // each row half multiplies one more 16-row fragment (rows BM + 16*wm ..).
  const bool extra = tile.rows > C::kBM;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::kWavesN, wn = wave % C::kWavesN;
  const int n_b = N * 2;
  const int n0b = tile.n0 * 2;
  const int nsteps = ks1 - ks0;
  // descriptors start at the range's first K slice (rows past tile.rows and
  // K rows past Hin stay out of range)
  // activation rows: relative to the tile's first row, or (gather) absolute rows of a
  const bool gat = gx.src != nullptr;
  const u32x4_t asrd = make_srd(a + (gat ? 0 : (int64_t)tile.row0 * hin_b) + ks0 * kDmaKB,
                                (uint32_t)(gat ? gx.rows : tile.rows) * (uint32_t)hin_b -
                                    (uint32_t)(ks0 * kDmaKB));
  const u32x4_t wsrd = make_srd(w + (int64_t)tile.ex * Hin * n_b + (int64_t)ks0 * 32 * n_b,
                                (uint32_t)(Hin - ks0 * 32) * (uint32_t)n_b);
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  // ---- DMA: which global bytes this lane fetches for each KB of a slot it fills
  auto x_src = [&](int kb, uint32_t& voff, uint32_t& kc) {  // kb: byte within the slot's activations
    const int row = kb >> 6, pc = (kb >> 4) & 3;
    const int lc = pc ^ ((row >> 1) & 3);
    const int src = row >= tile.rows ? -1 : gat ? gather_src(gx, tile.row0 + row) : row;
    voff = (src >= 0 ? (uint32_t)src * (uint32_t)hin_b : kOOB) + lc * 16;
    kc = lc * 16;
  };
  uint32_t a_voff[C::kADma + 1];
  uint32_t a_kc[C::kADma + 1];
#pragma unroll
  for (int q = 0; q < C::kADma; ++q) x_src((wave * C::kADma + q) * 1024 + lane * 16, a_voff[q], a_kc[q]);
  // tail rows: waves 0 and 1 fetch rows BM..BM+15 and BM+16..BM+31 (one
  // more op per slice than the other waves, whose wait counts exclude it)
  const bool tail_dma = wave < C::kFold / 16;
  x_src(C::kLdsA + wave * 1024 + lane * 16, a_voff[C::kADma], a_kc[C::kADma]);
  uint32_t w_voff[C::kWDma];
#pragma unroll
  for (int q = 0; q < C::kWDma; ++q) {
    const int kb = (wave * C::kWDma + q) * 1024 + lane * 16;  // byte within the slot's weights
    const int k = kb / (C::kBN * 2), pb = kb % (C::kBN * 2);
    const int lseg = (pb >> 7) ^ ((k >> 3) & C::kSegMask);
    const int lb = (lseg << 7) + (pb & 127);
    w_voff[q] = (uint32_t)k * (uint32_t)n_b + (uint32_t)(n0b + lb) + (n0b + lb < n_b ? 0u : kOOB);
  }
  // Past-the-end slices are issued too (out-of-range loads write zeros), so
  // every wait count is fixed.
  // ex: the tile carries tail rows; td: this wave fetches some of them
  auto issue = [&](int step, auto ex, auto td) {
    const uint32_t base = lds0 + (step % C::kStages) * C::kStage;
    const int kb0 = step * kDmaKB;
#pragma unroll
    for (int q = 0; q < C::kADma; ++q)
      dma16(asrd, (a_voff[q] + kb0) | (kb0 + (int)a_kc[q] < kext_b ? 0u : kOOB),
            base + (wave * C::kADma + q) * 1024);
    if (decltype(ex)::value && decltype(td)::value)
      dma16(asrd, (a_voff[C::kADma] + kb0) | (kb0 + (int)a_kc[C::kADma] < kext_b ? 0u : kOOB),
            base + C::kLdsA + wave * 1024);
    const uint32_t kstep = step < nsteps ? (uint32_t)(step * 32) * (uint32_t)n_b : kOOB;
#pragma unroll
    for (int q = 0; q < C::kWDma; ++q)
      dma16(wsrd, w_voff[q] + kstep, base + C::kLdsX + (wave * C::kWDma + q) * 1024);
  };
  // The compiler may not move work across these barriers: the phases are the schedule.
  auto bar = [] {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  constexpr int S = C::kStages;

  const bool wave_active = (wm * C::kWM < tile.rows) && (tile.n0 + wn * C::kWN < N);
  const int ci = lane & 15, kq = lane >> 4;
  auto xoff_of = [&](int m) { return m * kDmaKB + ((kq ^ ((m >> 1) & 3)) << 4); };
  int xoff[C::kFI];
#pragma unroll
  for (int i = 0; i < C::kFI; ++i) xoff[i] = xoff_of(wm * C::kWM + i * 16 + ci);
  const int xoff_t = xoff_of(C::kBM + wm * 16 + ci);  // this half's tail fragment
  int woff[C::kFG];
#pragma unroll
  for (int g = 0; g < C::kFG; ++g) {
    const int cb = (wn * C::kWN + g * 64 + 4 * ci) * 2;  // byte of this lane's 4 columns
    woff[g] = C::kLdsX + (kq * 8) * (C::kBN * 2) + (((cb >> 7) ^ (kq & C::kSegMask)) << 7) + (cb & 127);
  }
  bf16x8_t xa[C::kFI], xt;
  uint4 wc[C::kFG][4];
  auto read_frags = [&](int slice, auto ex) {
    const unsigned char* st = smem + (slice % S) * C::kStage;
#pragma unroll
    for (int i = 0; i < C::kFI; ++i) xa[i] = *reinterpret_cast<const bf16x8_t*>(st + xoff[i]);
    if (decltype(ex)::value) xt = *reinterpret_cast<const bf16x8_t*>(st + xoff_t);
#pragma unroll
    for (int g = 0; g < C::kFG; ++g) {
      uint2 wraw[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) wraw[r] = *reinterpret_cast<const uint2*>(st + woff[g] + r * (C::kBN * 2));
      transpose_8x4_bf16(wraw, wc[g]);
    }
  };
  f32x4_t acc[C::kFI][C::kFG][4], acct[C::kFG][4];
#pragma unroll
  for (int g = 0; g < C::kFG; ++g)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int i = 0; i < C::kFI; ++i) acc[i][g][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      acct[g][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    }
  auto multiply = [&](auto ex) {
#pragma unroll
    for (int i = 0; i < C::kFI; ++i)
#pragma unroll
      for (int g = 0; g < C::kFG; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][g][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              *reinterpret_cast<bf16x8_t*>(&wc[g][j]), xa[i], acc[i][g][j], 0, 0, 0);
    if (decltype(ex)::value) {
#pragma unroll
      for (int g = 0; g < C::kFG; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acct[g][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              *reinterpret_cast<bf16x8_t*>(&wc[g][j]), xt, acct[g][j], 0, 0, 0);
    }
  };

  // The schedule; `ex` (compile time) adds the tail fragment and its DMA op.
  // Four straight-line loops (half x active), each with the same barriers and
  // DMA as its partner, so no loop carries a branch.
  auto run = [&](auto ex, auto td) {
    constexpr int kInFlight = (S - 2) * (C::kPerStage + (decltype(ex)::value && decltype(td)::value ? 1 : 0));
#pragma unroll
    for (int t = 0; t < S - 1; ++t) issue(t, ex, td);
    wait_vmcnt<kInFlight>();
    bar();  // barrier 0: slice 0 has landed
    if (wm == 0) {
      if (wave_active) {
        read_frags(0, ex);
        issue(S - 1, ex, td);
        bar();
        for (int s = 0; s < nsteps; ++s) {
          multiply(ex);
          wait_vmcnt<kInFlight>();
          bar();
          read_frags(s + 1, ex);
          issue(s + S, ex, td);
          bar();
        }
      } else {
        issue(S - 1, ex, td);
        bar();
        for (int s = 0; s < nsteps; ++s) {
          wait_vmcnt<kInFlight>();
          bar();
          issue(s + S, ex, td);
          bar();
        }
      }
      bar();  // matches the second half's last barrier
    } else {
      bar();
      issue(S - 1, ex, td);
      if (wave_active) {
        read_frags(0, ex);
        wait_vmcnt<kInFlight>();
        bar();
        for (int s = 0; s < nsteps; ++s) {
          multiply(ex);
          bar();
          read_frags(s + 1, ex);
          issue(s + S, ex, td);
          wait_vmcnt<kInFlight>();
          bar();
        }
      } else {
        wait_vmcnt<kInFlight>();
        bar();
        for (int s = 0; s < nsteps; ++s) {
          bar();
          issue(s + S, ex, td);
          wait_vmcnt<kInFlight>();
          bar();
        }
      }
    }
  };
  if (!extra) run(std::false_type{}, std::false_type{});
  else if (tail_dma) run(std::true_type{}, std::true_type{});
  else run(std::true_type{}, std::false_type{});
  wait_vmcnt<0>();  // no DMA may still be landing when the block's LDS is released

  const float sc = ld_scale(a_scale) * ld_scale(w_scale);
  // Fragment f of this wave: 0 .. kFI-1 are rows wm*kWM + 16f + ci, kFI is
  // the tail fragment (rows BM + 16*wm + ci).
  auto frag_row = [&](int f) { return f < C::kFI ? wm * C::kWM + f * 16 + ci : C::kBM + wm * 16 + ci; };
  auto frag_acc = [&](int f, int g, float* a16) {  // MFMA j, output row 4*kq + r -> column 4r + j
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) a16[4 * r + j] = f < C::kFI ? acc[f][g][j][r] : acct[g][j][r];
  };
  // M: 0-3 = compile-time ReLU (bit 0) and gate (bit 1) cases, 4 = both
  // decided at run time (the split-K path's one copy)
  auto store_out = [&](int f, int g, const float* acc16, auto M) {
    constexpr int kM = decltype(M)::value;
    const int ml = frag_row(f);
    const int nb = tile.n0 + wn * C::kWN + g * 64 + 16 * kq;
    if (ml >= tile.rows || nb >= N) return;  // N is a multiple of 16 here
    const OutRow orow = out_row(gx, tile.row0 + ml, A);
    if (orow.row < 0) return;
    float v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      float t = acc16[q] * sc;
      if (kM == 4) {
        t = ((relu && t < 0.f) ? 0.f : t) * orow.gate;
      } else {
        if (kM & 1) t = t < 0.f ? 0.f : t;
        if (kM & 2) t *= orow.gate;
      }
      v[q] = t;
    }
    bf16_t* o = out + orow.row * N + nb;
    reinterpret_cast<uint4*>(o)[0] = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    reinterpret_cast<uint4*>(o)[1] = make_uint4(pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]),
                                                pack_bf16x2(v[12], v[13]), pack_bf16x2(v[14], v[15]));
  };
  if (wk.S == 1) {
    // The output tile goes through LDS (rows of kOutRow bytes over the
    // ring, which every wave has finished with): each lane writes its 16
    // scaled, activated, gated bf16 columns per fragment, then 32 lanes per
    // tile row store whole 512-byte rows, so every global store covers full
    // cache lines instead of 64-byte pieces of 16 rows.
    __syncthreads();
    auto stage_all = [&](auto M) {
      constexpr int kM = decltype(M)::value;
#pragma unroll
      for (int f = 0; f < C::kFI + 1; ++f) {
        if (f == C::kFI && !extra) continue;  // compile-time f keeps the accumulators in registers
        const int ml = frag_row(f);
        if (ml >= tile.rows) continue;
        const OutRow orow = out_row(gx, tile.row0 + ml, A);
        if (orow.row < 0) continue;
        unsigned char* lrow = smem + ml * C::kOutRow;
#pragma unroll
        for (int g = 0; g < C::kFG; ++g) {
          float a16[16];
          frag_acc(f, g, a16);
          float v[16];
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            float t = a16[q] * sc;
            if (kM & 1) t = t < 0.f ? 0.f : t;
            if (kM & 2) t *= orow.gate;
            v[q] = t;
          }
          uint4* o = reinterpret_cast<uint4*>(lrow + (wn * C::kWN + g * 64 + 16 * kq) * 2);
          o[0] = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                            pack_bf16x2(v[6], v[7]));
          o[1] = make_uint4(pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]), pack_bf16x2(v[12], v[13]),
                            pack_bf16x2(v[14], v[15]));
        }
      }
    };
    if (wave_active) {
      const int m = (relu ? 1 : 0) | (gx.dst != nullptr && gx.gate != nullptr ? 2 : 0);
      if (m == 0) stage_all(std::integral_constant<int, 0>{});
      else if (m == 1) stage_all(std::integral_constant<int, 1>{});
      else if (m == 2) stage_all(std::integral_constant<int, 2>{});
      else stage_all(std::integral_constant<int, 3>{});
    }
    __syncthreads();
    // 16 bytes (8 columns) per lane; rows past the tile's rows, rows without
    // a destination and columns past N are skipped (N is a multiple of 16)
    constexpr int kLanesRow = C::kBN * 2 / 16;
    constexpr int kPasses = (C::kBM + C::kFold) * kLanesRow / C::kNT;
    static_assert((C::kBM + C::kFold) * kLanesRow % C::kNT == 0, "whole passes");
    const int nrows = tile.rows < C::kBM + C::kFold ? tile.rows : C::kBM + C::kFold;
#pragma unroll 1
    for (int ps = 0; ps < kPasses; ++ps) {
      const int idx = ps * C::kNT + tid;
      const int ml = idx / kLanesRow, c = (idx % kLanesRow) * 8;
      if (ml >= nrows || tile.n0 + c >= N) continue;
      const OutRow orow = out_row(gx, tile.row0 + ml, A);
      if (orow.row < 0) continue;
      *reinterpret_cast<uint4*>(out + orow.row * N + tile.n0 + c) =
          *reinterpret_cast<const uint4*>(smem + ml * C::kOutRow + c * 2);
    }
    return true;
  }
  // Split tile: every part stores its fp32 partial tile [BM + kFold][BN];
  // the last part to arrive sums the S partials in part order (its own from
  // registers), so the result does not depend on which part finished last.
  // Partials are written through to memory and read back past L1/L2
  // (system-scope cache policy): once a part's stores have completed it
  // counts itself with a device-scope atomic, and the part that brings the
  // count to S reads everything without the L2 writeback and invalidate a
  // device-scope fence would cost every tile running on its XCD.
  constexpr int kTileF = (C::kBM + C::kFold) * C::kBN;
  constexpr int kSysScope = 17;  // cache policy sc0 | sc1
  const __amdgpu_buffer_rsrc_t prsrc =
      make_rsrc(split_ws + (int64_t)wk.rtile * wk.S * kTileF, (uint32_t)(wk.S * kTileF * 4));
  auto part_off = [&](int q, int f, int g) {  // byte offset of a lane's 16 partial columns
    return (uint32_t)((q * kTileF + frag_row(f) * C::kBN + wn * C::kWN + g * 64 + 16 * kq) * 4);
  };
  if (wave_active) {
#pragma unroll
    for (int f = 0; f < C::kFI + 1; ++f) {
      if (f == C::kFI && !extra) continue;  // compile-time f keeps the accumulators in registers
#pragma unroll
      for (int g = 0; g < C::kFG; ++g) {
        float a16[16];
        frag_acc(f, g, a16);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const f32x4_t v = {a16[4 * r], a16[4 * r + 1], a16[4 * r + 2], a16[4 * r + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), prsrc,
                                                 part_off(wk.part, f, g) + r * 16, 0, kSysScope);
        }
      }
    }
  }
  wait_vmcnt<0>();  // this wave's partials have reached memory
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(split_cnt + wk.rtile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             wk.S - 1;
  __syncthreads();
  if (!s_last || !wave_active) return true;
#pragma unroll
  for (int f = 0; f < C::kFI + 1; ++f) {
    if (f == C::kFI && !extra) continue;  // compile-time f keeps the accumulators in registers
#pragma unroll
    for (int g = 0; g < C::kFG; ++g) {
      float own[16], a16[16];
      frag_acc(f, g, own);
      for (int q = 0; q < wk.S; ++q) {
        float p16[16];
        if (q == wk.part) {
#pragma unroll
          for (int c = 0; c < 16; ++c) p16[c] = own[c];
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const f32x4_t v = __builtin_bit_cast(
                f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(prsrc, part_off(q, f, g) + r * 16, 0, kSysScope));
#pragma unroll
            for (int j = 0; j < 4; ++j) p16[4 * r + j] = v[j];
          }
        }
#pragma unroll
        for (int c = 0; c < 16; ++c) a16[c] = q == 0 ? p16[c] : a16[c] + p16[c];
      }
      store_out(f, g, a16, std::integral_constant<int, 4>{});
    }
  }
  return true;
}

template <class C>
__global__ __launch_bounds__(C::kNT) __attribute__((amdgpu_waves_per_eu(2))) void gmm_pp_kernel(
    const unsigned char* __restrict__ a, const unsigned char* __restrict__ w,
    const float* __restrict__ a_scale, const float* __restrict__ w_scale,
    const int32_t* __restrict__ offsets, int e, int A, int Hin, int N, int relu,
    bf16_t* __restrict__ out, float* __restrict__ split_ws, int* __restrict__ split_cnt, int ncu,
    RowMap gx) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __shared__ int s_last;
  pp_block<C>(smem, s_last, blockIdx.x, a, w, a_scale, w_scale, offsets, e, A, Hin, N, relu, out, split_ws,
              split_cnt, ncu, gx);
}

// Persistent form: one block per CU runs pp_block's work items one after
// another, taking the next index of its XCD (blocks are placed on the 8
// XCDs round-robin, so block b is on XCD b % 8) from an atomic counter per
// XCD: item k of XCD x is pp_block's block x + 8k, so the tiles of an XCD
// still start in their XCD-aware order and its CUs keep sharing panels in
// L2. The tile prefix is computed once per block, into LDS past the ring.
// queue: 8 counters, zero at launch.
template <class C>
__global__ __launch_bounds__(C::kNT) __attribute__((amdgpu_waves_per_eu(2))) void gmm_ppd_kernel(
    const unsigned char* __restrict__ a, const unsigned char* __restrict__ w,
    const float* __restrict__ a_scale, const float* __restrict__ w_scale,
    const int32_t* __restrict__ offsets, int e, int A, int Hin, int N, int relu,
    bf16_t* __restrict__ out, float* __restrict__ split_ws, int* __restrict__ split_cnt, int ncu,
    RowMap gx, int* __restrict__ queue) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __shared__ int s_last, s_item;
  int* s_tab = reinterpret_cast<int*>(smem + C::kLds);
  load_tile_prefix<C::kBM, C::kFold>(offsets, e, A, s_tab, s_tab + 257);
  const int x = blockIdx.x & 7;
  for (;;) {
    if (threadIdx.x == 0) s_item = __hip_atomic_fetch_add(queue + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int k = __builtin_amdgcn_readfirstlane(s_item);
    if (!pp_block<C>(smem, s_last, x + 8 * k, a, w, a_scale, w_scale, offsets, e, A, Hin, N, relu, out, split_ws,
                     split_cnt, ncu, gx, s_tab))
      break;
  }
}

// ------------------------------------------------------------------ ping-pong E4M3 kernel
//
// The bf16 ping-pong design for E4M3 operands, on v_mfma_scale_f32_16x16x128
// _f8f6f4 (unit scales, both operands E4M3). One MFMA reduces 128 values, so
// a ring slot holds a 128-deep K slice: activations 256 rows x 128 B and
// weights 128 rows x 128 B (a 256 x 128 output tile; three 48 KB slots fit
// in LDS). 8 waves of 64 x 64: waves 0-3 hold rows 0-127, waves 4-7 rows
// 128-255, and the two halves alternate multiply and memory phases between
// barriers exactly as in gmm_pp_kernel (one phase = 16 MFMAs = 512 cycles).
//
// Weights go through gfx950's transposing LDS read (ds_read_b64_tr_b8). In
// each group of 16 lanes, lane s names 8 bytes; the 16 x 8-byte pieces are
// taken as 8 rows of 16 bytes (row b = the pieces of lanes 2b and 2b+1) and
// lane l receives column l: byte b of its result is byte l of row b
// (measured on the device). With lanes 2b, 2b+1 naming the two halves of
// K row k0 + b over 16 consecutive output columns, lane l gets column l's K
// values k0 .. k0+7, which is an MFMA fragment piece; four reads fill a
// 32-byte fragment. MFMA j's row i is then output column 16j + i, and a
// lane ends with 4 consecutive output columns per MFMA.
// LDS layout: activation row m holds its eight 16-byte chunks at positions
// c ^ ((m/2)%2 + 4*((m/4)%2)); weight K row k holds chunk c at position
// c ^ ((k/2)%4 + 4*((k/32)%2)), so the 16 rows that lanes 0-31 (or 32-63)
// of one transposing read touch fall in distinct banks.

// FP4 (MX only): E2M1 elements, two per byte along K, so a slot's 128 bytes
// per row hold 256 K values, two MFMA K steps of 128, and 8 scale blocks.
template <bool MX, bool FP4 = false>
struct Pp8Cfg {
  static_assert(MX || !FP4, "E2M1 operands come with MX block scales");
  static constexpr int kBM = 256, kBN = 128;
  static constexpr int kKB = 128;  // bytes per activation row (= weight K rows) per slot
  static constexpr int kStages = 3;
  static constexpr int kNT = 512;
  static constexpr int kLdsA = kBM * kKB;  // 32 KB
  static constexpr int kLdsW = kKB * kBN;  // 16 KB
  static constexpr int kBlk = FP4 ? 8 : 4;  // MX scale blocks per slot
  // MX: the slot's E8M0 scales, activations [kBlk/4][256 rows][4 blocks]
  // then weights [kBlk blocks][128 columns]
  static constexpr int kScA = kLdsA + kLdsW, kScW = kScA + kBM * kBlk;
  static constexpr int kStage = kLdsA + kLdsW + (MX ? kBM * kBlk + kBlk * kBN : 0);
  static constexpr int kDummy = kStages * kStage;  // 1 KB that soaks up the unused scale DMA (MX)
  static constexpr int kLds = kDummy + (MX ? 1024 : 0);
  static constexpr int kADma = kLdsA / 1024 / 8;  // 1 KB DMA ops per wave per slot
  static constexpr int kWDma = kLdsW / 1024 / 8;
  static constexpr int kSDma = MX ? kBlk / 4 : 0;  // 256-byte scale ops per wave per slot
  static constexpr int kPerStage = kADma + kWDma + kSDma;
  static_assert(kLds + 2 * 257 * 4 <= 160 * 1024 || kLds <= 160 * 1024, "LDS budget");
};

// Slot swizzles. The hardware's K order inside a 16x16x128 operand: lane
// group g (lanes 16g .. 16g+15) register bytes 0-15 are K 16g .. 16g+15 and
// bytes 16-31 are K 64+16g .. 64+16g+15 (measured with block scales: scale
// lane group b covers K 32b .. 32b+31). Fragments are read in that order so
// that K means the same thing in the data and in MX scale blocks: activation
// row m holds 16-byte chunk c at position c ^ (2*((m/2)%4)), weight K row k
// holds output-column chunk c at position c ^ ((k/2)%4 + 4*((k/16)%2)).
__device__ __forceinline__ int pp8_xswz(int m) { return 2 * ((m >> 1) & 3); }
// Tile row held by LDS activation row q: within each 64-row group, LDS row
// 16i + c (fragment i, lane c) holds tile row 4c + i, so the four rows a
// lane multiplies are adjacent (one 16-byte read then fetches their scales).
__device__ __forceinline__ int pp8_trow(int q) { return (q & ~63) | ((q & 15) << 2) | ((q >> 4) & 3); }
__device__ __forceinline__ int pp8_wswz(int k) { return ((k >> 1) & 3) | (((k >> 4) & 1) << 2); }

// The kernel's work for block p (smem: the dynamic LDS ring).
template <bool MX, bool FP4>
__device__ __forceinline__ void pp8_block(
    unsigned char* smem, int p, const unsigned char* __restrict__ a, const unsigned char* __restrict__ w,
    const float* __restrict__ a_scale, const float* __restrict__ w_scale,
    const unsigned char* __restrict__ a_mx, const unsigned char* __restrict__ w_mx,
    const int32_t* __restrict__ offsets, int e, int A, int Hin, int N, int relu,
    bf16_t* __restrict__ out, const RowMap& gx) {
  typedef Pp8Cfg<MX, FP4> C;
  // MX: LDS activation rows in the pp8_trow order, so that one 16-byte read
  // fetches the scales of a lane's four fragment rows
  constexpr bool kRowPerm = MX;
  {
    int* s_off = reinterpret_cast<int*>(smem);
    load_tile_prefix<C::kBM>(offsets, e, A, s_off, s_off + 257);
  }
  Tile tile;
  if (!pick_tile<C::kBM, C::kBN, kPp8Group>(reinterpret_cast<const int*>(smem),
                                     reinterpret_cast<const int*>(smem) + 257, e, N, p, tile))
    return;
  __syncthreads();  // every lane has its tile before the ring overwrites the prefix

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave >> 2, wm2 = (wave >> 1) & 1, wn = wave & 1;
  // bytes per activation row = weight K rows per expert (E2M1: two K values per byte)
  const int rowb = FP4 ? Hin / 2 : Hin;
  const int nsteps = (rowb + C::kKB - 1) / C::kKB;
  // activation rows: relative to the tile's first row, or (gather) absolute rows of a
  const bool gat = gx.src != nullptr;
  const u32x4_t asrd = make_srd(a + (gat ? 0 : (int64_t)tile.row0 * rowb),
                                (uint32_t)(gat ? gx.rows : tile.rows) * (uint32_t)rowb);
  const u32x4_t wsrd = make_srd(w + (int64_t)tile.ex * rowb * N, (uint32_t)rowb * (uint32_t)N);
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  // MX scales (whole slices): kBlk E8M0 blocks per row and slice. Activation
  // scales are stored slice-major, (Hin/32/kBlk, A, kBlk): a slice's scales
  // of consecutive rows are consecutive, so waves 0-3 (one row per lane, 4
  // blocks per op) each read 256 contiguous bytes; the next kBlk/2 waves
  // fetch the weight columns' (32 lanes per block, 2 blocks per op); every
  // other op is an out-of-range one into the dummy KB, so that every wave
  // counts kSDma ops per slice.
  const int nbk = Hin / 32;
  u32x4_t ssrd = {0u, 0u, 0u, 0u};
  uint32_t s_voff = kOOB, s_lds = lds0 + C::kDummy, s_step = 0;
  bool s_real = false;
  if (MX) {
    if (wave < 4) {
      const int m = 64 * wave + lane;
      ssrd = make_srd(a_mx, (uint32_t)A * (uint32_t)nbk);
      s_voff = m < tile.rows ? (uint32_t)(tile.row0 + m) * (uint32_t)C::kBlk : kOOB;
      s_lds = C::kScA + wave * 256;
      s_step = (uint32_t)A * (uint32_t)C::kBlk;
      s_real = true;
    } else if (wave < 4 + C::kBlk / 2) {
      // weight scales in interleaved column order, rows of N64 = N rounded
      // up to 64: position 4c + j of a 64-column group holds column 16j + c
      const int n64 = (N + 63) & ~63;
      const int bb = (64 * (wave - 4) + lane) / 32, col = tile.n0 + 4 * (lane % 32);
      ssrd = make_srd(w_mx + (int64_t)tile.ex * nbk * n64, (uint32_t)nbk * (uint32_t)n64);
      s_voff = (uint32_t)bb * (uint32_t)n64 + (uint32_t)col + (col < n64 ? 0u : kOOB);
      s_lds = C::kScW + (wave - 4) * 256;
      s_step = (uint32_t)C::kBlk * (uint32_t)n64;
      s_real = true;
    } else {
      ssrd = make_srd(a_mx, 4u);
    }
  }

  uint32_t a_voff[C::kADma];
  uint32_t a_kc[C::kADma];
#pragma unroll
  for (int q = 0; q < C::kADma; ++q) {
    const int kb = (wave * C::kADma + q) * 1024 + lane * 16;
    const int prow = kb >> 7, pc = (kb >> 4) & 7;
    const int lc = pc ^ pp8_xswz(prow);
    const int trow = kRowPerm ? pp8_trow(prow) : prow;
    const int src = trow >= tile.rows ? -1 : gat ? gather_src(gx, tile.row0 + trow) : trow;
    a_voff[q] = (src >= 0 ? (uint32_t)src * (uint32_t)rowb : kOOB) + lc * 16;
    a_kc[q] = lc * 16;
  }
  uint32_t w_voff[C::kWDma];
#pragma unroll
  for (int q = 0; q < C::kWDma; ++q) {
    const int kb = (wave * C::kWDma + q) * 1024 + lane * 16;
    const int k = kb >> 7, pc = (kb >> 4) & 7;  // LDS row (= K row) and chunk position
    const int nb = tile.n0 + (pc ^ pp8_wswz(k)) * 16;
    w_voff[q] = (uint32_t)k * (uint32_t)N + (uint32_t)nb + (nb < N ? 0u : kOOB);
  }
  // Past-the-end slices are issued too (out-of-range loads write zeros).
  auto issue = [&](int step) {
    const uint32_t base = lds0 + (step % C::kStages) * C::kStage;
    const int kb0 = step * C::kKB;
#pragma unroll
    for (int q = 0; q < C::kADma; ++q)
      dma16(asrd, (a_voff[q] + kb0) | (kb0 + (int)a_kc[q] < rowb ? 0u : kOOB),
            base + (wave * C::kADma + q) * 1024);
    const uint32_t kstep = step < nsteps ? (uint32_t)kb0 * (uint32_t)N : 0u;
    const uint32_t kend = step < nsteps ? 0u : kOOB;
#pragma unroll
    for (int q = 0; q < C::kWDma; ++q)
      dma16(wsrd, (w_voff[q] + kstep) | kend, base + C::kLdsA + (wave * C::kWDma + q) * 1024);
    if (MX) {
      const uint32_t soff = (s_voff + (step < nsteps ? (uint32_t)step * s_step : 0u)) | kend;
      dma4(ssrd, soff, s_real ? base + s_lds : lds0 + C::kDummy);
      if (FP4) {  // activation blocks 4..7 of the slice, or a filler op
        if (wave < 4)
          dma4(ssrd, soff + 4u, base + s_lds + C::kBM * 4);
        else
          dma4(ssrd, kOOB, lds0 + C::kDummy);
      }
    }
  };
  auto bar = [] {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  constexpr int S = C::kStages;
  constexpr int kInFlight = (S - 2) * C::kPerStage;

  const bool wave_active = (half * 128 + wm2 * 64 < tile.rows) && (tile.n0 + wn * 64 < N);
  const int ci = lane & 15, kq = lane >> 4;
  // tile row (within the wave's 64) of fragment i, lane ci
  auto frow = [&](int i) { return kRowPerm ? 4 * ci + i : 16 * i + ci; };
  // output map: this lane's destination rows, fetched now so that the
  // epilogue does not wait for them
  int dpre[4] = {0, 0, 0, 0};
  if (gx.dst != nullptr && wave_active) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ml = half * 128 + wm2 * 64 + frow(i);
      dpre[i] = ml < tile.rows ? gx.dst[tile.row0 + ml] : -1;
    }
  }
  // per-row activation scales (per-token quantised input), fetched now too
  float rpre[4] = {1.f, 1.f, 1.f, 1.f};
  if (gx.row_scale != nullptr && wave_active) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ml = half * 128 + wm2 * 64 + frow(i);
      rpre[i] = ml < tile.rows ? row_scale_of(gx, tile.row0 + ml) : 0.f;
    }
  }
  // activation fragment i: chunks kq (register bytes 0-15) and 4 + kq (16-31)
  int xoff[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = half * 128 + wm2 * 64 + i * 16 + ci;
      xoff[i][h] = m * C::kKB + (((4 * h + kq) ^ pp8_xswz(m)) << 4);
    }
  // transposing weight reads: read t (= 0..3, register bytes 8t .. 8t+7) takes
  // K rows 64*(t/2) + 16kq + 8*(t%2) + 0..7; this lane names row ... + ci/2,
  // half ci%2 of output-column chunk 4wn + j
  const int wk0 = 16 * kq + ci / 2;
  const int wsw = pp8_wswz(wk0);  // the same for every t
  const int wrow0 = C::kLdsA + wk0 * C::kBN + 8 * (ci & 1);
  int wch[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) wch[j] = ((4 * wn + j) ^ wsw) * 16;
  typedef int i32x2_t __attribute__((ext_vector_type(2)));
  i32x8_t xa[4], wf[4];
  int sxa[C::kBlk / 4][4], sxw[C::kBlk / 4][4];  // MX: this lane's E8M0 scales (block kq of each K step)
  auto read_frags = [&](int slice) {
    const unsigned char* st = smem + (slice % S) * C::kStage;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 lo = *reinterpret_cast<const uint4*>(st + xoff[i][0]);
      const uint4 hi = *reinterpret_cast<const uint4*>(st + xoff[i][1]);
      xa[i] = (i32x8_t){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2_t*)(st + wrow0 + wch[j] +
                                                          (64 * (t >> 1) + 8 * (t & 1)) * C::kBN));
        wf[j][2 * t] = v.x;
        wf[j][2 * t + 1] = v.y;
      }
    if (MX) {
#pragma unroll
      for (int u = 0; u < C::kBlk / 4; ++u) {
        {  // this lane's four rows are adjacent: one 16-byte read, then block kq of each
          const uint4 r4 = *reinterpret_cast<const uint4*>(st + C::kScA + u * C::kBM * 4 +
                                                           (half * 128 + wm2 * 64 + 4 * ci) * 4);
          sxa[u][0] = (int)(r4.x >> (8 * kq));
          sxa[u][1] = (int)(r4.y >> (8 * kq));
          sxa[u][2] = (int)(r4.z >> (8 * kq));
          sxa[u][3] = (int)(r4.w >> (8 * kq));
        }
        {  // columns 16j + ci (j = 0..3) of block kq: one 4-byte read of the interleaved row
          const uint32_t c4 = *reinterpret_cast<const uint32_t*>(st + C::kScW + (4 * u + kq) * C::kBN + wn * 64 + 4 * ci);
#pragma unroll
          for (int j = 0; j < 4; ++j) sxw[u][j] = (int)(c4 >> (8 * j));
        }
      }
    }
  };
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  auto multiply = [&]() {
    if (FP4) {
      // E2M1: each 32-byte fragment holds two K steps of 16 bytes per lane;
      // lane group g's 16 bytes are scale block g of the step (measured)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const i32x8_t wv = u ? __builtin_shufflevector(wf[j], wf[j], 4, 5, 6, 7, 4, 5, 6, 7) : wf[j];
            const i32x8_t xv = u ? __builtin_shufflevector(xa[i], xa[i], 4, 5, 6, 7, 4, 5, 6, 7) : xa[i];
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wv, xv, acc[i][j], 4, 4, 0,
                                                                         sxw[u % (C::kBlk / 4)][j], 0,
                                                                         sxa[u % (C::kBlk / 4)][i]);
          }
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = MX ? __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j], xa[i], acc[i][j], 0, 0, 0,
                                                                          sxw[0][j], 0, sxa[0][i])
                       : __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j], xa[i], acc[i][j], 0, 0, 0,
                                                                          0, 0, 0);
  };

#pragma unroll
  for (int t = 0; t < S - 1; ++t) issue(t);
  wait_vmcnt<kInFlight>();
  bar();  // barrier 0: slice 0 has landed
  if (half == 0) {
    if (wave_active) {
      read_frags(0);
      issue(S - 1);
      bar();
      for (int s = 0; s < nsteps; ++s) {
        multiply();
        wait_vmcnt<kInFlight>();
        bar();
        read_frags(s + 1);
        issue(s + S);
        bar();
      }
    } else {
      issue(S - 1);
      bar();
      for (int s = 0; s < nsteps; ++s) {
        wait_vmcnt<kInFlight>();
        bar();
        issue(s + S);
        bar();
      }
    }
    bar();  // matches the second half's last barrier
  } else {
    bar();
    issue(S - 1);
    if (wave_active) {
      read_frags(0);
      wait_vmcnt<kInFlight>();
      bar();
      for (int s = 0; s < nsteps; ++s) {
        multiply();
        bar();
        read_frags(s + 1);
        issue(s + S);
        wait_vmcnt<kInFlight>();
        bar();
      }
    } else {
      wait_vmcnt<kInFlight>();
      bar();
      for (int s = 0; s < nsteps; ++s) {
        bar();
        issue(s + S);
        wait_vmcnt<kInFlight>();
        bar();
      }
    }
  }
  wait_vmcnt<0>();  // no DMA may still be landing when the block's LDS is released
  if (!wave_active) return;

  const float sc = ld_scale(a_scale) * ld_scale(w_scale);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ml = half * 128 + wm2 * 64 + frow(i);
    if (ml >= tile.rows) continue;
    const OutRow orow = out_row_of(gx, tile.row0 + ml, dpre[i], A);
    if (orow.row < 0) continue;
    const int64_t m = orow.row;
    const float rsc = gx.row_scale != nullptr ? rpre[i] * sc : sc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // MFMA j, output row 4*kq + r  ->  column nb + r
      const int nb = tile.n0 + wn * 64 + 16 * j + 4 * kq;
      if (nb >= N) continue;  // N is a multiple of 16 here
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float t = acc[i][j][r] * rsc;
        v[r] = ((relu && t < 0.f) ? 0.f : t) * orow.gate;
      }
      *reinterpret_cast<uint2*>(out + m * N + nb) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
  }
}

template <bool MX, bool FP4 = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void gmm_pp8_kernel(
    const unsigned char* __restrict__ a, const unsigned char* __restrict__ w,
    const float* __restrict__ a_scale, const float* __restrict__ w_scale,
    const unsigned char* __restrict__ a_mx, const unsigned char* __restrict__ w_mx,
    const int32_t* __restrict__ offsets, int e, int A, int Hin, int N, int relu,
    bf16_t* __restrict__ out, RowMap gx) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  pp8_block<MX, FP4>(smem, blockIdx.x, a, w, a_scale, w_scale, a_mx, w_mx, offsets, e, A, Hin, N, relu, out, gx);
}

// ------------------------------------------------------------------ wide ping-pong E4M3 kernel
//
// E4M3 with per-tensor or per-row scales (no block scales) on 256 x 256
// tiles: the bf16 ping-pong kernel's ring geometry with E4M3 operands. A
// slot holds a 64-deep K slice, activations 256 rows x 64 B and weights 64
// K rows x 256 B (32 KB; four slots), so a slice brings 32 KB for 2048
// MFMA cycles per SIMD pair, the same bytes per MFMA cycle as the bf16
// kernel; the 256 x 128 E4M3 kernel needs half as many MFMA cycles per byte
// fetched. 8 waves of 128 x 64 on v_mfma_scale_f32_32x32x64_f8f6f4 (unit
// scales): waves 0-3 hold rows 0-127, waves 4-7 rows 128-255, the two
// halves alternating multiply and memory phases as in gmm_pp_kernel.
// MFMA operands: the weights are the row operand (row i = output column),
// the activations the column operand (column j = tile row). Lane l holds
// row / column l % 32 and K values 32 (l / 32) .. +31 in order: activation
// fragments are two 16-byte LDS reads, weight fragments four transposing
// reads (ds_read_b64_tr_b8, each 8 K rows of 16 columns per 16 lanes).
// Accumulator register r of lane l is output column 8 (r / 4) + 4 (l / 32)
// + r % 4 of the 32 x 32 block, tile row l % 32.
// LDS layout: activation row m keeps its four 16-byte chunks at positions
// c ^ ((m / 4) % 4), so 16 consecutive rows cover all banks; weight K row k
// keeps its sixteen 16-column chunks at c ^ (2 (k % 8)), so the 8 rows x 2
// chunks of a transposing read by 32 lanes fall in distinct banks.
// Epilogue: the accumulators (4 columns per lane and register group) go to
// an LDS copy of the bf16 output tile (rows padded to 528 bytes), which is
// then written out a whole 512-byte row per 32 lanes.
// An expert's last row piece of at most 32 rows rides on the tile before it
// (as in gmm_pp_kernel): then each row half multiplies one more 32 x 32
// block whose column j is tail row 16 * half + j % 16 (lanes j and j + 16
// read the same row; only the first is stored).
struct Pp8wCfg {
  static constexpr int kBM = 256, kBN = 256, kStages = 4, kNT = 512;
  static constexpr int kFold = 32;               // tail rows an expert's last tile may carry beyond BM
  static constexpr int kKB = 64;                 // K bytes (E4M3 values) per slot
  static constexpr int kLdsA = kBM * kKB;        // 16 KB
  static constexpr int kLdsX = (kBM + kFold) * kKB;  // ... with the folded tail rows
  static constexpr int kLdsW = kKB * kBN;        // 16 KB
  static constexpr int kStage = kLdsX + kLdsW;
  static constexpr int kRing = kStages * kStage;   // 136 KB
  static constexpr int kOutRow = kBN * 2 + 16;     // bytes per row of the staged output tile
  static constexpr int kOut = (kBM + kFold) * kOutRow;
  static constexpr int kLds = kRing > kOut ? kRing : kOut;  // 148.5 KB
  static constexpr int kADma = kLdsA / 1024 / 8;  // 1 KB DMA ops per wave per slot
  static constexpr int kWDma = kLdsW / 1024 / 8;
  static constexpr int kPerStage = kADma + kWDma;
  static_assert(kLds >= 2 * 257 * 4, "tile prefix lives in the ring");
  static_assert(kFold * kKB == 2 * 1024, "waves 0 and 1 fetch the tail rows");
};
__device__ __forceinline__ int pp8w_xpos(int m, int c) { return c ^ ((m >> 2) & 3); }
__device__ __forceinline__ int pp8w_wpos(int k, int c) { return c ^ (2 * (k & 7)); }

__device__ __forceinline__ void pp8w_block(unsigned char* smem, int p, const unsigned char* __restrict__ a,
                                           const unsigned char* __restrict__ w, const float* __restrict__ a_scale,
                                           const float* __restrict__ w_scale, const int32_t* __restrict__ offsets,
                                           int e, int A, int Hin, int N, int relu, bf16_t* __restrict__ out,
                                           const RowMap& gx) {
  typedef Pp8wCfg C;
  {
    int* s_off = reinterpret_cast<int*>(smem);
    load_tile_prefix<C::kBM, C::kFold>(offsets, e, A, s_off, s_off + 257);
  }
  Tile tile;
  if (!pick_tile<C::kBM, C::kBN, kPpGroup, C::kFold>(reinterpret_cast<const int*>(smem),
                                                     reinterpret_cast<const int*>(smem) + 257, e, N, p, tile))
    return;
  __syncthreads();  // every lane has its tile before the ring overwrites the prefix
  const bool extra = tile.rows > C::kBM;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int rowb = Hin;  // bytes per activation row = weight K rows
  const int nsteps = (rowb + C::kKB - 1) / C::kKB;
  const bool gat = gx.src != nullptr;
  const u32x4_t asrd = make_srd(a + (gat ? 0 : (int64_t)tile.row0 * rowb),
                                (uint32_t)(gat ? gx.rows : tile.rows) * (uint32_t)rowb);
  const u32x4_t wsrd = make_srd(w + (int64_t)tile.ex * rowb * N, (uint32_t)rowb * (uint32_t)N);
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  // ---- DMA: which global bytes this lane fetches for each KB of a slot it fills
  auto x_src = [&](int kb, uint32_t& voff, uint32_t& kc) {  // kb: byte within the slot's activations
    const int row = kb >> 6, lc = pp8w_xpos(row, (kb >> 4) & 3);
    const int src = row >= tile.rows ? -1 : gat ? gather_src(gx, tile.row0 + row) : row;
    voff = (src >= 0 ? (uint32_t)src * (uint32_t)rowb : kOOB) + lc * 16;
    kc = lc * 16;
  };
  uint32_t a_voff[C::kADma + 1], a_kc[C::kADma + 1];
#pragma unroll
  for (int q = 0; q < C::kADma; ++q) x_src((wave * C::kADma + q) * 1024 + lane * 16, a_voff[q], a_kc[q]);
  // tail rows: waves 0 and 1 fetch rows BM..BM+15 and BM+16..BM+31 (one
  // more op per slice than the other waves, whose wait counts exclude it)
  const bool tail_dma = wave < C::kFold * C::kKB / 1024;
  x_src(C::kLdsA + wave * 1024 + lane * 16, a_voff[C::kADma], a_kc[C::kADma]);
  uint32_t w_voff[C::kWDma];
#pragma unroll
  for (int q = 0; q < C::kWDma; ++q) {
    const int kb = (wave * C::kWDma + q) * 1024 + lane * 16;  // byte within the slot's weights
    const int k = kb >> 8, lc = pp8w_wpos(k, (kb >> 4) & 15);
    const int nb = tile.n0 + lc * 16;
    w_voff[q] = (uint32_t)k * (uint32_t)N + (uint32_t)nb + (nb < N ? 0u : kOOB);
  }
  // Past-the-end slices are issued too (out-of-range loads write zeros); K
  // rows past Hin lie past the weight descriptor's end.
  // ex: the tile carries tail rows; td: this wave fetches some of them
  auto issue = [&](int step, auto ex, auto td) {
    const uint32_t base = lds0 + (step % C::kStages) * C::kStage;
    const int kb0 = step * C::kKB;
#pragma unroll
    for (int q = 0; q < C::kADma; ++q)
      dma16(asrd, (a_voff[q] + kb0) | (kb0 + (int)a_kc[q] < rowb ? 0u : kOOB), base + (wave * C::kADma + q) * 1024);
    if (decltype(ex)::value && decltype(td)::value)
      dma16(asrd, (a_voff[C::kADma] + kb0) | (kb0 + (int)a_kc[C::kADma] < rowb ? 0u : kOOB),
            base + C::kLdsA + wave * 1024);
    const uint32_t kstep = step < nsteps ? (uint32_t)kb0 * (uint32_t)N : kOOB;
#pragma unroll
    for (int q = 0; q < C::kWDma; ++q)
      dma16(wsrd, w_voff[q] + kstep, base + C::kLdsX + (wave * C::kWDma + q) * 1024);
  };
  auto bar = [] {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  constexpr int S = C::kStages;

  const bool wave_active = (wm * 128 < tile.rows) && (tile.n0 + wn * 64 < N);
  const int l32 = lane & 31, g = lane >> 5;
  // output map and per-row scales of this lane's four tile rows, fetched now
  // tile row of block i's column l32 (block 4: this half's tail rows)
  auto blk_row = [&](int i) { return i < 4 ? wm * 128 + 32 * i + l32 : C::kBM + 16 * wm + (l32 & 15); };
  // activation fragment i: row blk_row(i), K chunks 2g and 2g+1; the chunk
  // positions depend on the row only through l32 % 16 / 4, the same for
  // every block, so blocks 1-3 are block 0 plus 32i rows
  int xoff0[2], xofft[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    xoff0[h] = blk_row(0) * C::kKB + (pp8w_xpos(blk_row(0), 2 * g + h) << 4);
    xofft[h] = blk_row(4) * C::kKB + (pp8w_xpos(blk_row(4), 2 * g + h) << 4);
  }
  // weight fragment j (columns wn*64 + 32j .. +31): in each 16-lane group,
  // lanes 2b, 2b+1 name the halves of K row 32g + 8t + b of the group's 16
  // columns (t = 0..3 for the four reads)
  const int s16 = lane & 15, grp = lane >> 4;
  const int wk0 = 32 * g + (s16 >> 1);  // K row of read t = 0 (k % 8 = s16 / 2 for every t)
  int woff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    woff[j] = C::kLdsX + wk0 * C::kBN + (pp8w_wpos(wk0, 4 * wn + 2 * j + (grp & 1)) << 4) + 8 * (s16 & 1);
  typedef int i32x2_t __attribute__((ext_vector_type(2)));
  i32x8_t xa[5], wf[2];
  auto read_frags = [&](int slice, auto ex) {
    const unsigned char* st = smem + (slice % S) * C::kStage;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      if (i == 4 && !decltype(ex)::value) continue;
      const int o0 = i < 4 ? xoff0[0] + i * 32 * C::kKB : xofft[0];
      const int o1 = i < 4 ? xoff0[1] + i * 32 * C::kKB : xofft[1];
      const uint4 lo = *reinterpret_cast<const uint4*>(st + o0);
      const uint4 hi = *reinterpret_cast<const uint4*>(st + o1);
      xa[i] = (i32x8_t){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2_t*)(st + woff[j] + t * 8 * C::kBN));
        wf[j][2 * t] = v.x;
        wf[j][2 * t + 1] = v.y;
      }
  };
  f32x16_t acc[5][2];
#pragma unroll
  for (int i = 0; i < 5; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  auto multiply = [&](auto ex) {
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      if (i == 4 && !decltype(ex)::value) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[j], xa[i], acc[i][j], 0, 0, 0, 0, 0, 0);
    }
  };

  // The schedule: gmm_pp_kernel's; `ex` (compile time) adds the tail block,
  // and `td` its DMA op in waves 0 and 1.
  auto run = [&](auto ex, auto td) {
    constexpr int kInFlight = (S - 2) * (C::kPerStage + (decltype(ex)::value && decltype(td)::value ? 1 : 0));
#pragma unroll
    for (int t = 0; t < S - 1; ++t) issue(t, ex, td);
    wait_vmcnt<kInFlight>();
    bar();  // barrier 0: slice 0 has landed
    if (wm == 0) {
      if (wave_active) {
        read_frags(0, ex);
        issue(S - 1, ex, td);
        bar();
        for (int s = 0; s < nsteps; ++s) {
          multiply(ex);
          wait_vmcnt<kInFlight>();
          bar();
          read_frags(s + 1, ex);
          issue(s + S, ex, td);
          bar();
        }
      } else {
        issue(S - 1, ex, td);
        bar();
        for (int s = 0; s < nsteps; ++s) {
          wait_vmcnt<kInFlight>();
          bar();
          issue(s + S, ex, td);
          bar();
        }
      }
      bar();  // matches the second half's last barrier
    } else {
      bar();
      issue(S - 1, ex, td);
      if (wave_active) {
        read_frags(0, ex);
        wait_vmcnt<kInFlight>();
        bar();
        for (int s = 0; s < nsteps; ++s) {
          multiply(ex);
          bar();
          read_frags(s + 1, ex);
          issue(s + S, ex, td);
          wait_vmcnt<kInFlight>();
          bar();
        }
      } else {
        wait_vmcnt<kInFlight>();
        bar();
        for (int s = 0; s < nsteps; ++s) {
          bar();
          issue(s + S, ex, td);
          wait_vmcnt<kInFlight>();
          bar();
        }
      }
    }
  };
  if (!extra) run(std::false_type{}, std::false_type{});
  else if (tail_dma) run(std::true_type{}, std::true_type{});
  else run(std::true_type{}, std::false_type{});
  // output map and per-row scales of this lane's rows, fetched while the
  // past-the-end DMA drains
  int dpre[5] = {0, 0, 0, 0, 0};
  float rpre[5] = {1.f, 1.f, 1.f, 1.f, 1.f};
  if (wave_active) {
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int ml = blk_row(i);
      if (gx.dst != nullptr) dpre[i] = ml < tile.rows ? gx.dst[tile.row0 + ml] : -1;
      if (gx.row_scale != nullptr) rpre[i] = ml < tile.rows ? row_scale_of(gx, tile.row0 + ml) : 0.f;
    }
  }
  wait_vmcnt<0>();  // no DMA may still be landing when the block's LDS is released
  __syncthreads();  // every wave is done with the ring

  // accumulators -> scaled, activated, gated bf16 in the LDS copy of the
  // output tile; ReLU and the gate are compile-time cases (one multiply per
  // value when neither applies: this loop's arithmetic is the epilogue's cost)
  auto stage = [&](auto relu_c, auto gate_c) {
    const float sc = ld_scale(a_scale) * ld_scale(w_scale);
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      if (i == 4 && (!extra || l32 >= 16)) continue;  // tail rows: lanes 0-15 of each half
      const int ml = blk_row(i);
      if (ml >= tile.rows) continue;
      const OutRow orow = out_row_of(gx, tile.row0 + ml, dpre[i], A);
      if (orow.row < 0) continue;
      const float rsc = gx.row_scale != nullptr ? rpre[i] * sc : sc;
      unsigned char* lrow = smem + ml * C::kOutRow;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // registers 4q .. 4q+3: columns 8q + 4g .. +3 of the 32-column block
          const int c = wn * 64 + 32 * j + 8 * q + 4 * g;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float t = acc[i][j][4 * q + r] * rsc;
            if (decltype(relu_c)::value) t = t < 0.f ? 0.f : t;
            if (decltype(gate_c)::value) t *= orow.gate;
            v[r] = t;
          }
          *reinterpret_cast<uint2*>(lrow + c * 2) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
    }
  };
  if (wave_active) {
    const bool gated = gx.dst != nullptr && gx.gate != nullptr;
    if (relu) {
      if (gated) stage(std::true_type{}, std::true_type{});
      else stage(std::true_type{}, std::false_type{});
    } else {
      if (gated) stage(std::false_type{}, std::true_type{});
      else stage(std::false_type{}, std::false_type{});
    }
  }
  __syncthreads();
  // 32 lanes per tile row, 16 bytes (8 columns) each; rows past the tile's
  // rows, rows without a destination and columns past N are skipped
  constexpr int kPasses = (C::kBM + C::kFold) * 32 / C::kNT;
#pragma unroll 4
  for (int ps = 0; ps < kPasses; ++ps) {
    const int idx = ps * C::kNT + tid;
    const int ml = idx >> 5, c = (idx & 31) * 8;
    if (ml >= tile.rows || tile.n0 + c >= N) continue;  // N is a multiple of 16 here
    const OutRow orow = out_row(gx, tile.row0 + ml, A);
    if (orow.row < 0) continue;
    *reinterpret_cast<uint4*>(out + orow.row * N + tile.n0 + c) =
        *reinterpret_cast<const uint4*>(smem + ml * C::kOutRow + c * 2);
  }
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void gmm_pp8w_kernel(
    const unsigned char* __restrict__ a, const unsigned char* __restrict__ w, const float* __restrict__ a_scale,
    const float* __restrict__ w_scale, const int32_t* __restrict__ offsets, int e, int A, int Hin, int N, int relu,
    bf16_t* __restrict__ out, RowMap gx) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  pp8w_block(smem, blockIdx.x, a, w, a_scale, w_scale, offsets, e, A, Hin, N, relu, out, gx);
}

// Two grouped GEMMs in one launch: a bf16 one on the ping-pong kernel's
// 256 x 256 tiles and an E4M3 one on the wide E4M3 kernel's 256 x 256 tiles
// (with MX block scales: the E4M3 kernel's 256 x 128 tiles), each block
// running exactly what its own kernel runs for that tile. The
// first nb0 blocks serve the group handed out first (kPairBf16First
// says which), the rest the other; nb0 is a multiple of 8, so both keep
// their XCD-aware tile order. The bf16 GEMM is never split along K here.
struct GroupArgs {
  const unsigned char* a;
  const unsigned char* w;
  const float* a_scale;
  const float* w_scale;
  const unsigned char* a_mx;  // E8M0 block scales (MX E4M3 / E2M1 groups)
  const unsigned char* w_mx;
  const int32_t* offsets;
  int e, A, Hin, N, relu;
  bf16_t* out;
  RowMap gx;
};

template <class C, bool MX, bool FP4>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void gmm_pair_kernel(GroupArgs b,
                                                                                               GroupArgs f,
                                                                                               int nb0) {
  static_assert(C::kNT == 512, "both halves run 8 waves");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __shared__ int s_last;
  const int p = blockIdx.x;
  const bool first = p < nb0;
  const int q = first ? p : p - nb0;
  if (first == kPairBf16First)
    pp_block<C>(smem, s_last, q, b.a, b.w, b.a_scale, b.w_scale, b.offsets, b.e, b.A, b.Hin, b.N, b.relu, b.out,
                nullptr, nullptr, 1, b.gx);  // no split workspace: ncu is not used
  else if constexpr (MX)
    pp8_block<MX, FP4>(smem, q, f.a, f.w, f.a_scale, f.w_scale, f.a_mx, f.w_mx, f.offsets, f.e,
                            f.A, f.Hin, f.N, f.relu, f.out, f.gx);
  else
    pp8w_block(smem, q, f.a, f.w, f.a_scale, f.w_scale, f.offsets, f.e, f.A, f.Hin, f.N, f.relu, f.out, f.gx);
}

// ------------------------------------------------------------------ streaming kernel (decode)

// XS: the block's 4 waves (one expert, 4 consecutive 64-column groups) share
// their activation rows through LDS, 32 KB chunks of 32/MB k-steps filled by
// LDS DMA and double-buffered, instead of each wave loading them itself.
template <int MB, bool AL, bool XS>
__global__ __launch_bounds__(256) void gmm_stream_kernel(
    const bf16_t* __restrict__ a, const bf16_t* __restrict__ w, const float* __restrict__ a_scale,
    const float* __restrict__ w_scale, const int32_t* __restrict__ offsets, int e, int A, int Hin,
    int N, int relu, bf16_t* __restrict__ out, RowMap gx) {
  // Tasks are (non-empty expert, 64 columns), numbered densely so that the
  // waves with work are spread evenly over the CUs: s_pre[q] counts the
  // non-empty experts before q (a "row tile" of 2^30 rows).
  __shared__ int s_off[257];
  __shared__ int s_pre[257];
  load_tile_prefix<0x40000000>(offsets, e, A, s_off, s_pre);
  const int lane = threadIdx.x & 63;
  const int ng = (N + 63) / 64;
  const int task = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int q = task / ng;
  if (q >= s_pre[e]) return;
  int lo = 0, hi = e - 1;  // largest expert with s_pre <= q: the q-th non-empty one
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pre[mid] <= q) lo = mid;
    else hi = mid - 1;
  }
  const int ex = lo;
  const int n0 = (task % ng) * 64;
  const int r0 = s_off[ex];
  const int cnt = s_off[ex + 1] - r0;
  const float sc = ld_scale(a_scale) * ld_scale(w_scale);
  const int kq = lane >> 4;  // k slice of the 32-wide step
  const int ci = lane & 15;  // fragment row/column index
  const int ncol = n0 + 4 * ci;
  const int avail_n = (int)min(N - ncol, 4) * 2;  // bytes of this lane's 4 columns
  const bf16_t* wex = w + (int64_t)ex * Hin * N;
  // AL: buffer loads (rows past Hin and columns past N read as zero); U
  // k-steps per register set, the next set's loads all issued before the
  // current set is multiplied.
  constexpr int U = MB == 1 ? 1 : 2;  // measured: deeper sets only pay with 32+ rows per wave
  const __amdgpu_buffer_rsrc_t wsrc = make_rsrc(wex, (uint32_t)Hin * (uint32_t)N * 2u);
  // activation rows: relative to the expert's first row, or (gather) absolute rows of a
  const bool gat = gx.src != nullptr;
  const __amdgpu_buffer_rsrc_t xsrc =
      make_rsrc(a + (gat ? 0 : (int64_t)r0 * Hin), (uint32_t)(gat ? gx.rows : cnt) * (uint32_t)Hin * 2u);
  // source row of the expert's row ml, -1 when there is none
  auto xrow = [&](int ml) { return ml >= cnt ? -1 : gat ? gather_src(gx, r0 + ml) : ml; };
  const uint32_t woff = (uint32_t)(kq * 8) * (uint32_t)N * 2u + (uint32_t)ncol * 2u + (ncol < N ? 0u : kOOB);
  struct Set {
    uint2 w[U][8];
    uint4 x[U][MB];
  };

  static_assert(!XS || (AL && MB >= 2), "shared activation chunks: aligned, 32+ rows per block");
  extern __shared__ __attribute__((aligned(1024))) unsigned char xs_lds[];
  const int wave = threadIdx.x >> 6;

  for (int mc = 0; mc < cnt; mc += 16 * MB) {
    f32x4_t acc[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[mb][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    if constexpr (XS) {
      // chunk ch holds k-steps ch*KC .. ch*KC+KC-1 of the block's 16*MB rows:
      // row r at r*RB, its 16-byte piece c at position c ^ ((2r) % 16), so
      // the 16 rows x 2 pieces one pass of a fragment read touches fall in
      // distinct banks
      constexpr int KC = 32 / MB;             // k-steps per chunk
      constexpr int RB = KC * 64;             // bytes of one row in a chunk
      constexpr int XB = 16 * MB * RB;        // 32 KB per buffer
      constexpr int OPS = XB / 1024 / 4;      // 1 KB pieces (16 bytes per lane) per wave per chunk
      constexpr int PPR = RB / 16;            // 16-byte pieces per row
      static_assert(XB == 32768 && 1024 % RB == 0, "chunk shape");
      // this lane's share of a chunk: piece `lane` of block rows wave*OPS + o
      uint32_t dsrc[OPS], dpc[OPS];
#pragma unroll
      for (int o = 0; o < OPS; ++o) {
        const int r = (wave * OPS + o) * (1024 / RB) + lane / PPR;  // block row
        const int c = (lane % PPR) ^ ((2 * r) & 15);                  // piece stored at position lane % PPR
        const int src = xrow(mc + r);
        dsrc[o] = (src >= 0 ? (uint32_t)src * (uint32_t)Hin * 2u : kOOB) + (uint32_t)c * 16u;
        dpc[o] = (uint32_t)c * 16u;
      }
      uint4 xst[OPS];
      auto load_x = [&](int ch) {  // global -> registers
        const uint32_t kb = (uint32_t)ch * RB;  // byte offset of the chunk within a row
#pragma unroll
        for (int o = 0; o < OPS; ++o)
          xst[o] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                       xsrc, (dsrc[o] + kb) | (kb + dpc[o] < (uint32_t)Hin * 2u ? 0u : kOOB), 0, 0));
      };
      auto store_x = [&](int ch) {  // registers -> LDS buffer ch % 2
        unsigned char* xb = xs_lds + (ch & 1) * XB;
#pragma unroll
        for (int o = 0; o < OPS; ++o) *reinterpret_cast<uint4*>(xb + (wave * OPS + o) * 1024 + lane * 16) = xst[o];
      };
      int xoff[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) xoff[mb] = (mb * 16 + ci) * RB;
      const int xsw = (2 * ci) & 15;  // swizzle of rows mb*16 + ci (the same for every mb)
      struct WSet {
        uint2 w[U][8];
      };
      auto load_w = [&](int k0, WSet& st) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int r = 0; r < 8; ++r)
            st.w[u][r] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                             wsrc, woff + (uint32_t)(k0 + 32 * u + r) * (uint32_t)N * 2u, 0, 0));
      };
      auto mul_w = [&](const WSet& st, int k0) {
        const int ch = k0 / (32 * KC);
        const unsigned char* xb = xs_lds + (ch & 1) * XB;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int step = (k0 / 32 + u) % KC;
          const int pos = ((4 * step + kq) ^ xsw) * 16;
          bf16x8_t xv[MB];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) xv[mb] = *reinterpret_cast<const bf16x8_t*>(xb + xoff[mb] + pos);
          uint4 cols[4];
          transpose_8x4_bf16(st.w[u], cols);
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cols[j]), xv[mb],
                                                                   acc[mb][j], 0, 0, 0);
        }
      };
      // Per chunk: the next chunk's activations go to registers before the
      // chunk's last weight sets are loaded and to the other LDS buffer after
      // its last multiply; the barrier then also tells every wave that the
      // buffer of the chunk before is free again.
      const int nch = (Hin + 32 * KC - 1) / (32 * KC);
      WSet sa, sb;
      load_x(0);
      load_w(0, sa);
      store_x(0);
      __syncthreads();
      for (int ch = 0; ch < nch; ++ch) {
        const int kc0 = ch * 32 * KC;
#pragma unroll 1
        for (int t = 0; t < KC / U; t += 2) {
          const int k0 = kc0 + t * 32 * U;
          if (t + 2 >= KC / U && ch + 1 < nch) load_x(ch + 1);
          load_w(k0 + 32 * U, sb);  // past Hin: zeros
          __builtin_amdgcn_sched_barrier(0);
          mul_w(sa, k0);
          load_w(k0 + 64 * U, sa);
          __builtin_amdgcn_sched_barrier(0);
          mul_w(sb, k0 + 32 * U);
        }
        if (ch + 1 < nch) store_x(ch + 1);
        __syncthreads();
      }
    } else if (AL) {
      uint32_t xoff[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int src = xrow(mc + mb * 16 + ci);
        xoff[mb] = (src >= 0 ? (uint32_t)src * (uint32_t)Hin * 2u : kOOB) + kq * 16;
      }
      auto load_set = [&](int k0, Set& st) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int k = k0 + 32 * u;
#pragma unroll
          for (int r = 0; r < 8; ++r)
            st.w[u][r] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                             wsrc, woff + (uint32_t)(k + r) * (uint32_t)N * 2u, 0, 0));
          const uint32_t kx = k + kq * 8 < Hin ? 0u : kOOB;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            st.x[u][mb] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(xsrc, (xoff[mb] + (uint32_t)k * 2u) | kx, 0, 0));
        }
      };
      auto mul_set = [&](const Set& st) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          uint4 cols[4];
          transpose_8x4_bf16(st.w[u], cols);
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8_t, cols[j]), __builtin_bit_cast(bf16x8_t, st.x[u][mb]),
                  acc[mb][j], 0, 0, 0);
        }
      };
      Set sa, sb;
      int k0 = 0;
      load_set(0, sa);
      while (k0 < Hin) {
        load_set(k0 + 32 * U, sb);  // past the end: zeros
        __builtin_amdgcn_sched_barrier(0);
        mul_set(sa);
        k0 += 32 * U;
        if (k0 >= Hin) break;
        load_set(k0 + 32 * U, sa);
        __builtin_amdgcn_sched_barrier(0);
        mul_set(sb);
        k0 += 32 * U;
      }
    } else {
      int xsr[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) xsr[mb] = xrow(mc + mb * 16 + ci);
      for (int k0 = 0; k0 < Hin; k0 += 32) {
        uint2 rows[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int k = k0 + kq * 8 + r;
          rows[r] = ld8<AL, 2>(reinterpret_cast<const unsigned char*>(wex + (int64_t)k * N + ncol),
                               k < Hin ? avail_n : 0);
        }
        bf16x8_t xa[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int kk = k0 + kq * 8;
          const int src = xsr[mb];
          const int avail = src >= 0 ? min(Hin - kk, 8) * 2 : 0;
          const int64_t arow = src < 0 ? 0 : gat ? src : (int64_t)r0 + src;
          uint4 v = ld16<AL, 2>(reinterpret_cast<const unsigned char*>(a + arow * Hin + kk), avail);
          xa[mb] = *reinterpret_cast<bf16x8_t*>(&v);
        }
        uint4 cols[4];
        transpose_8x4_bf16(rows, cols);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8_t wb = *reinterpret_cast<bf16x8_t*>(&cols[j]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb, xa[mb], acc[mb][j], 0, 0, 0);
        }
      }
    }
    // MFMA j, output row i = 4*kq + r  ->  column n0 + 4*i + j = n0 + 16*kq + 4r + j
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int ml = mc + mb * 16 + ci;
      if (ml >= cnt) continue;
      const OutRow orow = out_row(gx, r0 + ml, A);
      if (orow.row < 0) continue;
      float v[16];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float t = acc[mb][j][r] * sc;
          v[4 * r + j] = ((relu && t < 0.f) ? 0.f : t) * orow.gate;
        }
      const int nb = n0 + 16 * kq;
      bf16_t* o = out + orow.row * N + nb;
      if (AL && nb + 15 < N) {
        uint4 p0 = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                              pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
        uint4 p1 = make_uint4(pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]),
                              pack_bf16x2(v[12], v[13]), pack_bf16x2(v[14], v[15]));
        reinterpret_cast<uint4*>(o)[0] = p0;
        reinterpret_cast<uint4*>(o)[1] = p1;
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q)
          if (nb + q < N) o[q] = f32_to_bf16(v[q]);
      }
    }
  }
}

// ------------------------------------------------------------------ fp32 kernel

constexpr int kF32BM = 64, kF32BN = 64, kF32BK = 16;

__global__ __launch_bounds__(256) void gmm_f32_kernel(const float* __restrict__ a,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ a_scale,
                                                      const float* __restrict__ w_scale,
                                                      const int32_t* __restrict__ offsets, int e,
                                                      int A, int Hin, int N, int relu,
                                                      float* __restrict__ out, RowMap gx) {
  __shared__ int s_off[257];
  __shared__ int s_pre[257];
  __shared__ float As[kF32BK][kF32BM + 1];
  __shared__ float Bs[kF32BK][kF32BN + 1];
  load_tile_prefix<kF32BM>(offsets, e, A, s_off, s_pre);
  Tile tile;
  if (!pick_tile<kF32BM, kF32BN, 8>(s_off, s_pre, e, N, blockIdx.x, tile)) return;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  const float* wex = w + (int64_t)tile.ex * Hin * N;
  // rows this thread loads (p = tid + 256 q: row p / kF32BK), as rows of a; -1: none
  static_assert(kF32BM * kF32BK % 256 == 0, "load split");
  int arow[kF32BM * kF32BK / 256];
#pragma unroll
  for (int q = 0; q < kF32BM * kF32BK / 256; ++q) {
    const int r = (tid + 256 * q) / kF32BK;
    arow[q] = r >= tile.rows ? -1 : gx.src ? gather_src(gx, tile.row0 + r) : tile.row0 + r;
  }
  for (int k0 = 0; k0 < Hin; k0 += kF32BK) {
#pragma unroll
    for (int q = 0; q < kF32BM * kF32BK / 256; ++q) {
      const int p = tid + 256 * q;
      const int r = p / kF32BK, k = p % kF32BK;
      As[k][r] = (arow[q] >= 0 && k0 + k < Hin) ? a[(int64_t)arow[q] * Hin + k0 + k] : 0.f;
    }
    for (int p = tid; p < kF32BK * kF32BN; p += 256) {
      const int k = p / kF32BN, c = p % kF32BN;
      const int n = tile.n0 + c;
      Bs[k][c] = (k0 + k < Hin && n < N) ? wex[(int64_t)(k0 + k) * N + n] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kF32BK; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(As[k][ty * 4 + i], Bs[k][tx * 4 + j], acc[i][j]);
    __syncthreads();
  }
  const float sc = ld_scale(a_scale) * ld_scale(w_scale);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty * 4 + i;
    if (r >= tile.rows) continue;
    const OutRow orow = out_row(gx, tile.row0 + r, A);
    if (orow.row < 0) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = tile.n0 + tx * 4 + j;
      if (n >= N) continue;
      float v = acc[i][j] * sc;
      if (relu && v < 0.f) v = 0.f;
      out[orow.row * N + n] = v * orow.gate;
    }
  }
}

// ------------------------------------------------------------------ launch helpers

template <class C>
moe_status launch_tiled(const void* a, const float* as, const void* w, const float* ws,
                        const int32_t* offsets, int e, int A, int Hin, int N, int relu, void* out,
                        hipStream_t s, RowMap gx) {
  static bool attr_done = false;
  if (!attr_done) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gmm_tiled_kernel<C>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
    attr_done = true;
  }
  const int64_t mt_max = cdiv64(A, C::kBM) + (e < A ? e : A);
  const int64_t blocks = mt_max * cdiv64(N, C::kBN);
  const int64_t grid = cdiv64(blocks, 8) * 8;
  if (grid > 0x7fffffff) return MOE_ERR_BAD_SHAPE;
  hipLaunchKernelGGL(gmm_tiled_kernel<C>, dim3((unsigned)grid), dim3(C::kNT), C::kLds, s,
                     (const unsigned char*)a, (const unsigned char*)w, as, ws, offsets, e, A, Hin, N,
                     relu, (unsigned char*)out, gx);
  return launch_status();
}

// Split-K scratch of the bf16 ping-pong kernel: ncu fp32 partial tiles, then
// ncu arrival counters.
size_t split_ws_floats(int ncu) { return (size_t)ncu * (256 + 32) * 256; }  // tiles with folded tails

__global__ void split_reset_kernel(int* __restrict__ cnt, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) cnt[i] = 0;
}

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

constexpr int kPersistSlices = 64;
inline int hin_b_of(int Hin) { return Hin * 2; }  // bf16 bytes per activation row

template <class C>
moe_status launch_pp(const void* a, const float* as, const void* w, const float* ws,
                     const int32_t* offsets, int e, int A, int Hin, int N, int relu, void* out,
                     void* split, hipStream_t s, RowMap gx, int* cnt_zeroed) {
  static_assert(C::kBM == 256 && C::kBN == 256, "split scratch is sized for 256 x 256 tiles");
  static bool attr_done = false;
  if (!attr_done) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gmm_pp_kernel<C>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
    attr_done = true;
  }
  const int ncu = device_cus();
  float* sws = reinterpret_cast<float*>(split);
  int* cnt = sws ? reinterpret_cast<int*>(sws + split_ws_floats(ncu)) : nullptr;
  const bool zeroed = cnt && cnt_zeroed;  // counters cleared by an earlier launch
  if (zeroed) cnt = cnt_zeroed;
  const int64_t mt_max = cdiv64(A, C::kBM) + (e < A ? e : A);
  const int64_t blocks = mt_max * cdiv64(N, C::kBN) + (sws ? 3 * (int64_t)ncu / 4 : 0);
  const int64_t grid = cdiv64(blocks, 8) * 8;
  if (grid > 0x7fffffff) return MOE_ERR_BAD_SHAPE;
  // Short K (at most kPersistSlices slices per tile): the persistent kernel,
  // one block per CU, its 8 queue counters after the split counters (all
  // cleared here). Measured on skewed (64 and 44 slices) its GEMMs take 3%
  // less; on prefill GEMM 1 (128 slices) 0.5-1% more, GEMM 2 (448) no change.
  if (cnt && (hin_b_of(Hin) + kDmaKB - 1) / kDmaKB <= kPersistSlices) {
    constexpr int kTabLds = 2 * 257 * 4;
    static bool pattr_done = false;
    if (!pattr_done) {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gmm_ppd_kernel<C>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds + kTabLds);
      pattr_done = true;
    }
    if (!zeroed) hipLaunchKernelGGL(split_reset_kernel, dim3(1), dim3(256), 0, s, cnt, ncu + 8);
    const int64_t pgrid = grid < ncu ? grid : ncu;
    hipLaunchKernelGGL(gmm_ppd_kernel<C>, dim3((unsigned)pgrid), dim3(C::kNT), C::kLds + kTabLds, s,
                       (const unsigned char*)a, (const unsigned char*)w, as, ws, offsets, e, A, Hin, N, relu,
                       (bf16_t*)out, sws, cnt, ncu, gx, cnt + ncu);
    return launch_status();
  }
  if (cnt && !zeroed) hipLaunchKernelGGL(split_reset_kernel, dim3(1), dim3(256), 0, s, cnt, ncu);
  hipLaunchKernelGGL(gmm_pp_kernel<C>, dim3((unsigned)grid), dim3(C::kNT), C::kLds, s,
                     (const unsigned char*)a, (const unsigned char*)w, as, ws, offsets, e, A, Hin, N,
                     relu, (bf16_t*)out, sws, cnt, ncu, gx);
  return launch_status();
}

template <bool MX, bool FP4 = false>
moe_status launch_pp8(const void* a, const float* as, const void* w, const float* ws,
                      const unsigned char* a_mx, const unsigned char* w_mx, const int32_t* offsets, int e,
                      int A, int Hin, int N, int relu, void* out, hipStream_t s, RowMap gx) {
  typedef Pp8Cfg<MX, FP4> C;
  static bool attr_done = false;
  if (!attr_done) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gmm_pp8_kernel<MX, FP4>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
    attr_done = true;
  }
  const int64_t mt_max = cdiv64(A, C::kBM) + (e < A ? e : A);
  const int64_t blocks = mt_max * cdiv64(N, C::kBN);
  const int64_t grid = cdiv64(blocks, 8) * 8;
  if (grid > 0x7fffffff) return MOE_ERR_BAD_SHAPE;
  hipLaunchKernelGGL((gmm_pp8_kernel<MX, FP4>), dim3((unsigned)grid), dim3(C::kNT), C::kLds, s,
                     (const unsigned char*)a, (const unsigned char*)w, as, ws, a_mx, w_mx, offsets, e, A,
                     Hin, N, relu, (bf16_t*)out, gx);
  return launch_status();
}

moe_status launch_pp8w(const void* a, const float* as, const void* w, const float* ws, const int32_t* offsets,
                       int e, int A, int Hin, int N, int relu, void* out, hipStream_t s, RowMap gx) {
  typedef Pp8wCfg C;
  static bool attr_done = false;
  if (!attr_done) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gmm_pp8w_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
    attr_done = true;
  }
  const int64_t mt_max = cdiv64(A, C::kBM) + (e < A ? e : A);
  const int64_t blocks = mt_max * cdiv64(N, C::kBN);
  const int64_t grid = cdiv64(blocks, 8) * 8;
  if (grid > 0x7fffffff) return MOE_ERR_BAD_SHAPE;
  hipLaunchKernelGGL(gmm_pp8w_kernel, dim3((unsigned)grid), dim3(C::kNT), C::kLds, s, (const unsigned char*)a,
                     (const unsigned char*)w, as, ws, offsets, e, A, Hin, N, relu, (bf16_t*)out, gx);
  return launch_status();
}

template <int MB, bool AL>
moe_status launch_stream(const void* a, const float* as, const void* w, const float* ws,
                         const int32_t* offsets, int e, int A, int Hin, int N, int relu, void* out,
                         hipStream_t s, RowMap gx) {
  const int64_t tasks = (int64_t)e * cdiv(N, 64);
  const dim3 grid((unsigned)cdiv64(tasks, 4));
  if constexpr (AL && MB >= 2) {
    // a block's 4 waves share one expert's rows when the 64-column groups
    // come in fours (N a multiple of 256)
    if (N % 256 == 0) {
      constexpr int kXsLds = 2 * 32768;
      static bool attr_done = false;
      if (!attr_done) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gmm_stream_kernel<MB, AL, true>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kXsLds);
        attr_done = true;
      }
      hipLaunchKernelGGL((gmm_stream_kernel<MB, AL, true>), grid, dim3(256), kXsLds, s, (const bf16_t*)a,
                         (const bf16_t*)w, as, ws, offsets, e, A, Hin, N, relu, (bf16_t*)out, gx);
      return launch_status();
    }
  }
  hipLaunchKernelGGL((gmm_stream_kernel<MB, AL, false>), grid, dim3(256), 0, s, (const bf16_t*)a,
                     (const bf16_t*)w, as, ws, offsets, e, A, Hin, N, relu, (bf16_t*)out, gx);
  return launch_status();
}

template <int MB>
moe_status launch_stream_al(bool al, const void* a, const float* as, const void* w, const float* ws,
                            const int32_t* offsets, int e, int A, int Hin, int N, int relu, void* out,
                            hipStream_t s, RowMap gx) {
  return al ? launch_stream<MB, true>(a, as, w, ws, offsets, e, A, Hin, N, relu, out, s, gx)
            : launch_stream<MB, false>(a, as, w, ws, offsets, e, A, Hin, N, relu, out, s, gx);
}

}  // namespace

// Rows per expert at or below which the weight-streaming kernel is used.
constexpr int kStreamMaxAvgRows = 48;

// Kernel family moe_gmm uses for a shape.
enum class GmmPath { F32, STREAM, PP, PP8, TILED };
GmmPath gmm_path(moe_dtype in_dt, int e, int A, int Hin, int N) {
  if (in_dt == MOE_F32) return GmmPath::F32;
  const int elem = in_dt == MOE_BF16 ? 2 : 1;
  if (in_dt == MOE_BF16 && (int64_t)A <= (int64_t)kStreamMaxAvgRows * e) return GmmPath::STREAM;
  // buffer-load path: 16-byte aligned rows and each expert's weight matrix under 2 GiB
  const bool al = ((int64_t)Hin * elem % 16 == 0) && ((int64_t)N * elem % 16 == 0) &&
                  ((int64_t)Hin * N * elem < (1ll << 31));
  if (elem == 2 && al && N % 16 == 0) return GmmPath::PP;
  if (elem == 1 && al && N % 16 == 0) return GmmPath::PP8;
  return GmmPath::TILED;
}

size_t gmm_ws_bytes(moe_dtype in_dt, int e, int A, int Hin, int N) {
  if (A == 0 || gmm_path(in_dt, e, A, Hin, N) != GmmPath::PP) return 0;
  const int ncu = device_cus();
  return split_ws_floats(ncu) * sizeof(float) + (size_t)gmm_counter_ints() * sizeof(int);
}

int gmm_counter_ints() { return device_cus() + 8; }  // split counters, then the persistent kernel's queues

moe_status launch_gmm(const void* a, moe_dtype in_dt, const float* a_scale, const void* w,
                      const float* w_scale, const int32_t* offsets, int e, int A, int Hin, int N,
                      moe_act act, void* out, moe_dtype out_dt, void* ws, hipStream_t s, RowMap gx,
                      int* cnt_zeroed) {
  if (A == 0) return MOE_OK;
  const int relu = act == MOE_ACT_RELU;
  if (in_dt == MOE_F32) {
    const int64_t blocks = (cdiv64(A, kF32BM) + (e < A ? e : A)) * cdiv64(N, kF32BN);
    const int64_t grid = cdiv64(blocks, 8) * 8;
    hipLaunchKernelGGL(gmm_f32_kernel, dim3((unsigned)grid), dim3(256), 0, s, (const float*)a,
                       (const float*)w, a_scale, w_scale, offsets, e, A, Hin, N, relu, (float*)out, gx);
    return launch_status();
  }
  const int elem = in_dt == MOE_BF16 ? 2 : 1;
  if (in_dt == MOE_BF16 && (int64_t)A <= (int64_t)kStreamMaxAvgRows * e) {
    // aligned: buffer loads over each expert's weights and over the rows (both under 2 GiB)
    const int64_t a_rows = gx.src ? gx.rows : A;  // rows the activation loads address
    const bool al = (Hin % 8 == 0) && (N % 8 == 0) && ((int64_t)Hin * N * 2 < (1ll << 31)) &&
                    (a_rows * Hin * 2 < (1ll << 31));
    const int avg = cdiv(A, e);
    if (avg <= 8) return launch_stream_al<1>(al, a, a_scale, w, w_scale, offsets, e, A, Hin, N, relu, out, s, gx);
    if (avg <= 16) return launch_stream_al<2>(al, a, a_scale, w, w_scale, offsets, e, A, Hin, N, relu, out, s, gx);
    return launch_stream_al<4>(al, a, a_scale, w, w_scale, offsets, e, A, Hin, N, relu, out, s, gx);
  }
  // buffer-load path: 16-byte aligned rows and each expert's weight matrix under 2 GiB
  const bool al = ((int64_t)Hin * elem % 16 == 0) && ((int64_t)N * elem % 16 == 0) &&
                  ((int64_t)Hin * N * elem < (1ll << 31));
  constexpr int WM = kTiledWavesM, WN = kTiledWavesN;
  if (elem == 2 && al && N % 16 == 0)
    return launch_pp<PpBf16>(a, a_scale, w, w_scale, offsets, e, A, Hin, N, relu, out, ws, s, gx, cnt_zeroed);
  if (elem == 1 && al && N % 16 == 0)
    return launch_pp8w(a, a_scale, w, w_scale, offsets, e, A, Hin, N, relu, out, s, gx);
  if (elem == 2) {
    typedef TiledCfg<2, 256, 256, WM, WN, true, false> CA;
    typedef TiledCfg<2, 256, 256, WM, WN, false, false> CU;
    return al ? launch_tiled<CA>(a, a_scale, w, w_scale, offsets, e, A, Hin, N, relu, out, s, gx)
              : launch_tiled<CU>(a, a_scale, w, w_scale, offsets, e, A, Hin, N, relu, out, s, gx);
  }
  typedef TiledCfg<1, 256, 256, WM, WN, true, false> FA;
  typedef TiledCfg<1, 256, 256, WM, WN, false, false> FU;
  return al ? launch_tiled<FA>(a, a_scale, w, w_scale, offsets, e, A, Hin, N, relu, out, s, gx)
            : launch_tiled<FU>(a, a_scale, w, w_scale, offsets, e, A, Hin, N, relu, out, s, gx);
}

moe_status launch_gmm_mx(const void* a, const unsigned char* a_scale, const void* w,
                         const unsigned char* w_scale, const int32_t* offsets, int e, int A, int Hin, int N,
                         moe_act act, void* out, hipStream_t s, bool fp4) {
  if (A == 0) return MOE_OK;
  if (fp4)
    return launch_pp8<true, true>(a, nullptr, w, nullptr, a_scale, w_scale, offsets, e, A, Hin, N,
                                  act == MOE_ACT_RELU, out, s, RowMap{});
  return launch_pp8<true>(a, nullptr, w, nullptr, a_scale, w_scale, offsets, e, A, Hin, N,
                          act == MOE_ACT_RELU, out, s, RowMap{});
}


template <bool MX, bool FP4>
moe_status launch_pair(const GmmCall& f, const GmmCall& b, hipStream_t s) {
  typedef PpBf16 CP;
  typedef typename std::conditional<MX, Pp8Cfg<MX, FP4>, Pp8wCfg>::type C8;
  constexpr int kLds = CP::kLds > C8::kLds ? CP::kLds : C8::kLds;
  static bool attr_done = false;
  if (!attr_done) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gmm_pair_kernel<CP, MX, FP4>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    attr_done = true;
  }
  // grid upper bounds as in the two kernels' own launches (surplus blocks exit)
  const int64_t nb_b = cdiv64((cdiv64(b.A, CP::kBM) + (b.e < b.A ? b.e : b.A)) * cdiv64(b.N, CP::kBN), 8) * 8;
  const int64_t nb_f = cdiv64((cdiv64(f.A, C8::kBM) + (f.e < f.A ? f.e : f.A)) * cdiv64(f.N, C8::kBN), 8) * 8;
  if (nb_b + nb_f > 0x7fffffff) return MOE_ERR_BAD_SHAPE;
  const GroupArgs ga_b{(const unsigned char*)b.a, (const unsigned char*)b.w, b.a_scale, b.w_scale, nullptr,
                       nullptr, b.offsets, b.e, b.A, b.Hin, b.N, b.act == MOE_ACT_RELU, (bf16_t*)b.out, b.gx};
  const GroupArgs ga_f{(const unsigned char*)f.a, (const unsigned char*)f.w, f.a_scale, f.w_scale, f.a_mx,
                       f.w_mx, f.offsets, f.e, f.A, f.Hin, f.N, f.act == MOE_ACT_RELU, (bf16_t*)f.out, f.gx};
  hipLaunchKernelGGL((gmm_pair_kernel<CP, MX, FP4>), dim3((unsigned)(nb_b + nb_f)), dim3(512), kLds, s, ga_b,
                     ga_f, (int)(kPairBf16First ? nb_b : nb_f));
  return launch_status();
}

moe_status launch_gmm_pair(const GmmCall& f, const GmmCall& b, hipStream_t s) {
  const bool f_ok = f.mx != 0 || gmm_path(MOE_FP8_E4M3, f.e, f.A, f.Hin, f.N) == GmmPath::PP8;
  const bool fuse = f.A > 0 && b.A > 0 && f_ok && gmm_path(MOE_BF16, b.e, b.A, b.Hin, b.N) == GmmPath::PP;
  if (!fuse) {
    moe_status st = f.mx != 0 ? launch_gmm_mx(f.a, f.a_mx, f.w, f.w_mx, f.offsets, f.e, f.A, f.Hin, f.N, f.act,
                                              f.out, s, f.mx == 2)
                              : launch_gmm(f.a, MOE_FP8_E4M3, f.a_scale, f.w, f.w_scale, f.offsets, f.e, f.A,
                                           f.Hin, f.N, f.act, f.out, MOE_BF16, nullptr, s, f.gx);
    if (st != MOE_OK) return st;
    return launch_gmm(b.a, MOE_BF16, b.a_scale, b.w, b.w_scale, b.offsets, b.e, b.A, b.Hin, b.N, b.act, b.out,
                      MOE_BF16, nullptr, s, b.gx);
  }
  if (f.mx == 2) return launch_pair<true, true>(f, b, s);
  if (f.mx == 1) return launch_pair<true, false>(f, b, s);
  return launch_pair<false, false>(f, b, s);
}

}  // namespace moe
