// api.hip — the extern "C" entry points declared in include/moe.h.
//
// Every call validates all of its arguments on the host first and enqueues
// nothing when one is wrong (the two-stage "check, then execute" contract of
// "aclnnQuantGroupedMatMulAlltoAllv": the first stage checks parameters and
// sizes the workspace, the second runs on a stream). The shape limits are
// that page's constraints, adapted to one GPU that holds every expert.
#include <mutex>

#include "dispatch.h"

using namespace moe;

namespace {

constexpr int kMaxDim = 65536;        // H, F, N in (0, 65536)
constexpr int kMaxExperts = 256;      // experts x ranks <= 256
constexpr int kMaxK = 8;              // K in [2, 8] (K = 1 also accepted)
constexpr int64_t kMaxRows = 52428800;  // received rows in (0, 52428800)

bool dim_ok(int d) { return d > 0 && d < kMaxDim; }

moe_status check_route_shape(int T, int H, int E, int K) {
  if (T < 0 || !dim_ok(H)) return MOE_ERR_BAD_SHAPE;
  if (E < 1 || E > kMaxExperts) return MOE_ERR_BAD_SHAPE;
  if (K < 1 || K > kMaxK || K > E) return MOE_ERR_BAD_SHAPE;
  if ((int64_t)T * K >= kMaxRows) return MOE_ERR_BAD_SHAPE;
  return MOE_OK;
}

bool layer_dtype_ok(moe_dtype dt) { return dt == MOE_F32 || dt == MOE_BF16; }
bool any_dtype_ok(moe_dtype dt) { return dt == MOE_F32 || dt == MOE_BF16 || dt == MOE_FP8_E4M3; }

#define MOE_TRY(expr)                 \
  do {                                \
    moe_status _st = (expr);          \
    if (_st != MOE_OK) return _st;    \
  } while (0)

#define REQUIRE_PTR(p) \
  if (!(p)) return MOE_ERR_NULL_POINTER
#define REQUIRE_ALIGNED(p) \
  if ((p) && !aligned16(p)) return MOE_ERR_MISALIGNED

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

struct LayerWs {
  size_t idx, gate, counts, offsets, psrc, pdst, perm_ws, bcnt, gmm_ws, cnt, xp, hm, total;
  int ncnt;  // ints at cnt: each GEMM's counters, cleared by the permute launch
};

LayerWs layer_ws_layout(int T, int H, int E, int K, int F, moe_dtype dt) {
  const int64_t A = (int64_t)T * K;
  const size_t es = (size_t)dtype_size(dt);
  LayerWs L;
  size_t o = 0;
  L.idx = o; o += round256(A * 4);
  L.gate = o; o += round256(A * 4);
  L.counts = o; o += round256((size_t)E * 4);
  L.offsets = o; o += round256((size_t)(E + 1) * 4);
  L.psrc = o; o += round256(A * 4);
  L.pdst = o; o += round256(A * 4);
  L.perm_ws = o; o += round256(permute_ws_bytes(T, E, K));
  // the router's per-block expert counts (16-token blocks; few experts only)
  L.bcnt = o; o += round256(E <= 16 ? (size_t)((T + 15) / 16) * E * 4 : 0);
  {
    const size_t g1 = gmm_ws_bytes(dt, E, (int)A, H, F), g2 = gmm_ws_bytes(dt, E, (int)A, F, H);
    L.gmm_ws = o; o += round256(g1 > g2 ? g1 : g2);  // shared by the two GEMMs (same stream)
    // each GEMM's own counters, so both are cleared by the one permute launch
    L.ncnt = (g1 || g2) ? 2 * gmm_counter_ints() : 0;
    L.cnt = o; o += round256((size_t)L.ncnt * 4);
  }
  L.xp = o; o += round256((size_t)A * H * es);  // permuted rows; reused for GEMM 2 output
  // hidden activations; before GEMM 1 writes them the router's split-H partials live here
  const size_t hm = (size_t)A * F * es, rws = route_ws_bytes(T, H, E, dt);
  L.hm = o; o += round256(hm > rws ? hm : rws);
  L.total = o;
  return L;
}

// E4M3 layer: bf16 tokens and router, E4M3 experts with per-tensor scales,
// activations quantised per token on the way into each GEMM.
struct LayerFp8Ws {
  size_t idx, gate, counts, offsets, psrc, pdst, perm_ws, gmm_ws, xq, xs, hm, hq, hs, yp, total;
};

LayerFp8Ws layer_fp8_ws_layout(int T, int H, int E, int K, int F) {
  const int64_t A = (int64_t)T * K;
  // tokens are quantised once and gathered (rows of up to 2^31 bytes), else
  // quantised through the dispatch index into A rows
  const int64_t qrows = (int64_t)T * H < (1ll << 31) ? T : A;
  LayerFp8Ws L;
  size_t o = 0;
  L.idx = o; o += round256(A * 4);
  L.gate = o; o += round256(A * 4);
  L.counts = o; o += round256((size_t)E * 4);
  L.offsets = o; o += round256((size_t)(E + 1) * 4);
  L.psrc = o; o += round256(A * 4);
  L.pdst = o; o += round256(A * 4);
  L.perm_ws = o; o += round256(permute_ws_bytes(T, E, K));
  {
    const size_t g1 = gmm_ws_bytes(MOE_FP8_E4M3, E, (int)A, H, F), g2 = gmm_ws_bytes(MOE_FP8_E4M3, E, (int)A, F, H);
    L.gmm_ws = o; o += round256(g1 > g2 ? g1 : g2);
  }
  L.xq = o; o += round256((size_t)qrows * H);
  L.xs = o; o += round256((size_t)qrows * 4);
  const size_t hm = (size_t)A * F * 2, rws = route_ws_bytes(T, H, E, MOE_BF16);
  L.hm = o; o += round256(hm > rws ? hm : rws);
  L.hq = o; o += round256((size_t)A * F);
  L.hs = o; o += round256((size_t)A * 4);
  L.yp = o; o += round256((size_t)A * H * 2);
  L.total = o;
  return L;
}

// Host-side checks shared by moe_layer and moe_layer_noalloc (everything but
// the workspace).
moe_status layer_check(const void* x, const void* w_router, const float* bias, const void* w1, const void* w2,
                       moe_dtype dt, int T, int H, int E, int K, int F, moe_act act, const void* y,
                       const int32_t* topk_idx_out, const float* topk_gate_out, const int32_t* counts_out) {
  if (!layer_dtype_ok(dt)) return MOE_ERR_BAD_DTYPE;
  MOE_TRY(check_route_shape(T, H, E, K));
  if (!dim_ok(F)) return MOE_ERR_BAD_SHAPE;
  if (act != MOE_ACT_NONE && act != MOE_ACT_RELU) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(x);
  REQUIRE_PTR(w_router);
  REQUIRE_PTR(w1);
  REQUIRE_PTR(w2);
  REQUIRE_PTR(y);
  REQUIRE_ALIGNED(x);
  REQUIRE_ALIGNED(w_router);
  REQUIRE_ALIGNED(bias);
  REQUIRE_ALIGNED(w1);
  REQUIRE_ALIGNED(w2);
  REQUIRE_ALIGNED(y);
  REQUIRE_ALIGNED(topk_idx_out);
  REQUIRE_ALIGNED(topk_gate_out);
  REQUIRE_ALIGNED(counts_out);
  return MOE_OK;
}

// The layer's launches on a checked workspace `base` laid out as L.
moe_status layer_run(const void* x, const void* w_router, const float* bias, const void* w1, const void* w2,
                     moe_dtype dt, int T, int H, int E, int K, int F, moe_act act, void* y, int32_t* topk_idx_out,
                     float* topk_gate_out, int32_t* counts_out, unsigned char* base, const LayerWs& L,
                     hipStream_t s) {
  int32_t* idx = topk_idx_out ? topk_idx_out : (int32_t*)(base + L.idx);
  float* gate = topk_gate_out ? topk_gate_out : (float*)(base + L.gate);
  int32_t* counts = counts_out ? counts_out : (int32_t*)(base + L.counts);
  int32_t* offsets = (int32_t*)(base + L.offsets);
  int32_t* psrc = (int32_t*)(base + L.psrc);
  int32_t* pdst = (int32_t*)(base + L.pdst);
  void* xp = base + L.xp;
  void* hm = base + L.hm;
  const int A = T * K;
  // the router also writes its per-block expert counts where it can; the
  // dispatch then ranks from them in one launch
  int32_t* bcnt = E <= 16 ? (int32_t*)(base + L.bcnt) : nullptr;
  int btok = 0;
  MOE_TRY(launch_route_counted(x, w_router, dt, bias, T, H, E, K, idx, gate, hm, s, bcnt, &btok));
  void* gws = base + L.gmm_ws;  // sized for whichever GEMM needs more (possibly none)
  void* gws1 = gmm_ws_bytes(dt, E, A, H, F) ? gws : nullptr;
  // the GEMMs' counters, cleared by the permute launch (no clearing launch per GEMM)
  int* cnt1 = L.ncnt ? (int*)(base + L.cnt) : nullptr;
  int* cnt2 = L.ncnt ? cnt1 + L.ncnt / 2 : nullptr;
  if ((int64_t)T * H * dtype_size(dt) < (1ll << 31)) {
    // dispatch inside GEMM 1: its row r is token perm_src[r] / K. Above one
    // block's worth of pairs the index path takes two launches unless the
    // router's counts replace its counting launch.
    if (btok > 0 && A > kPermuteBlockPairs && permute_counted_fits(T, E, K, btok))
      MOE_TRY(launch_permute_counted(idx, T, E, K, bcnt, btok, counts, offsets, psrc, pdst, s, cnt1, L.ncnt));
    else
      MOE_TRY(launch_permute(idx, nullptr, dt, T, H, E, K, counts, offsets, psrc, pdst, nullptr,
                             base + L.perm_ws, s, cnt1, L.ncnt));
    MOE_TRY(launch_gmm(x, dt, nullptr, w1, nullptr, offsets, E, A, H, F, act, hm, dt, gws1, s,
                       RowMap{psrc, K, T}, cnt1));
  } else {
    MOE_TRY(launch_permute(idx, x, dt, T, H, E, K, counts, offsets, psrc, pdst, xp, base + L.perm_ws, s,
                           cnt1, L.ncnt));
    MOE_TRY(launch_gmm(xp, dt, nullptr, w1, nullptr, offsets, E, A, H, F, act, hm, dt, gws1, s, RowMap{},
                       cnt1));
  }
  void* gws2 = gmm_ws_bytes(dt, E, A, F, H) ? gws : nullptr;
  // GEMM 2 into the grouped rows, then the weighted combine (gates applied
  // once, in fp32, in the combine; storing gated rows from GEMM 2's epilogue
  // and summing K rows moves the same bytes and measured 1-5% slower)
  MOE_TRY(launch_gmm(hm, dt, nullptr, w2, nullptr, offsets, E, A, F, H, MOE_ACT_NONE, xp, dt, gws2, s, RowMap{},
                     cnt2));
  MOE_TRY(launch_combine(xp, dt, pdst, gate, T, K, H, y, s));
  return MOE_OK;
}


// Scratch memory of moe_layer_noalloc: moe_layer's workspace in a static
// device array, one copy per GPU, held until the process ends. Host code
// never uses the array's name as an address: the address on each device is
// looked up once (with that device current) and kept.
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
unsigned char* g_scratch[kMaxDevices] = {};

moe_status scratch_on_current_device(unsigned char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_DEVICE;
    g_scratch[dev] = static_cast<unsigned char*>(p);
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL_POINTER: return "a required pointer is NULL";
    case MOE_ERR_BAD_SHAPE: return "a size is out of range or inconsistent";
    case MOE_ERR_BAD_DTYPE: return "element type not allowed for this argument";
    case MOE_ERR_UNSUPPORTED: return "mode not implemented (quantisation mode or activation)";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than the size query returned";
    case MOE_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
    case MOE_ERR_SCRATCH_LIMIT:
      return "the call needs more scratch memory than the allocation-free entry point's static buffer holds";
    case MOE_ERR_DEVICE: return "HIP runtime error while enqueuing work";
  }
  return "unknown status";
}

int moe_version(void) { return MOE_VERSION; }

moe_status moe_route_workspace_size(int T, int H, int E, int K, moe_dtype dt, size_t* bytes) {
  REQUIRE_PTR(bytes);
  if (!layer_dtype_ok(dt)) return MOE_ERR_BAD_DTYPE;
  MOE_TRY(check_route_shape(T, H, E, K));
  *bytes = route_ws_bytes(T, H, E, dt);
  return MOE_OK;
}

moe_status moe_route(const void* x, const void* w_router, moe_dtype dt, const float* bias, int T,
                     int H, int E, int K, int32_t* topk_idx, float* topk_gate, void* ws,
                     size_t ws_bytes, void* stream) {
  if (!layer_dtype_ok(dt)) return MOE_ERR_BAD_DTYPE;
  MOE_TRY(check_route_shape(T, H, E, K));
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(x);
  REQUIRE_PTR(w_router);
  REQUIRE_PTR(topk_idx);
  REQUIRE_PTR(topk_gate);
  const size_t need = route_ws_bytes(T, H, E, dt);
  if (need > 0) {
    REQUIRE_PTR(ws);
    if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  }
  REQUIRE_ALIGNED(x);
  REQUIRE_ALIGNED(w_router);
  REQUIRE_ALIGNED(bias);
  REQUIRE_ALIGNED(topk_idx);
  REQUIRE_ALIGNED(topk_gate);
  REQUIRE_ALIGNED(ws);
  return launch_route(x, w_router, dt, bias, T, H, E, K, topk_idx, topk_gate, ws, (hipStream_t)stream);
}

moe_status moe_permute_workspace_size(int T, int E, int K, size_t* bytes) {
  REQUIRE_PTR(bytes);
  MOE_TRY(check_route_shape(T, 1, E, K));
  *bytes = permute_ws_bytes(T, E, K);
  return MOE_OK;
}

moe_status moe_permute(const int32_t* topk_idx, const void* x, moe_dtype dt, int T, int H, int E,
                       int K, int32_t* counts, int32_t* offsets, int32_t* perm_src,
                       int32_t* perm_dst, void* x_perm, void* ws, size_t ws_bytes, void* stream) {
  if (x && !any_dtype_ok(dt)) return MOE_ERR_BAD_DTYPE;
  MOE_TRY(check_route_shape(T, x ? H : 1, E, K));
  if ((x == nullptr) != (x_perm == nullptr)) return MOE_ERR_NULL_POINTER;
  REQUIRE_PTR(counts);
  REQUIRE_PTR(offsets);
  if (T > 0) {
    REQUIRE_PTR(topk_idx);
    REQUIRE_PTR(perm_src);
    REQUIRE_PTR(perm_dst);
  }
  const size_t need = permute_ws_bytes(T, E, K);
  if (need > 0) {
    REQUIRE_PTR(ws);
    if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  }
  REQUIRE_ALIGNED(topk_idx);
  REQUIRE_ALIGNED(x);
  REQUIRE_ALIGNED(counts);
  REQUIRE_ALIGNED(offsets);
  REQUIRE_ALIGNED(perm_src);
  REQUIRE_ALIGNED(perm_dst);
  REQUIRE_ALIGNED(x_perm);
  if (need > 0) REQUIRE_ALIGNED(ws);
  return launch_permute(topk_idx, x, dt, T, H, E, K, counts, offsets, perm_src, perm_dst, x_perm, ws,
                        (hipStream_t)stream);
}

moe_status moe_gmm_workspace_size(moe_dtype a_dt, int e, int A, int Hin, int N, size_t* bytes) {
  REQUIRE_PTR(bytes);
  if (!any_dtype_ok(a_dt)) return MOE_ERR_BAD_DTYPE;
  if (e < 1 || e > kMaxExperts) return MOE_ERR_BAD_SHAPE;
  if (A < 0 || (int64_t)A >= kMaxRows || !dim_ok(Hin) || !dim_ok(N)) return MOE_ERR_BAD_SHAPE;
  *bytes = gmm_ws_bytes(a_dt, e, A, Hin, N);
  return MOE_OK;
}

namespace {
// Shared argument checks of moe_gmm / moe_gmm_gather / moe_gmm_scatter; on
// MOE_OK, call holds launch_gmm's arguments and *ws_use the workspace to pass
// (no_split: no workspace is taken or required; the launch then never splits).
moe_status gmm_prepare(const void* a, moe_dtype a_dt, moe_quant_mode a_q, const float* a_scale,
                       const void* w, moe_dtype w_dt, moe_quant_mode w_q, const float* w_scale,
                       const int32_t* offsets, int e, int A, int Hin, int N, moe_act act, void* out,
                       moe_dtype out_dt, void* ws, size_t ws_bytes, const RowMap* gx, GmmCall& call,
                       void** ws_use, bool no_split = false) {
  if (!any_dtype_ok(a_dt) || !any_dtype_ok(w_dt) || !any_dtype_ok(out_dt)) return MOE_ERR_BAD_DTYPE;
  const bool pair_ok = (a_dt == MOE_F32 && w_dt == MOE_F32 && out_dt == MOE_F32) ||
                       (a_dt == MOE_BF16 && w_dt == MOE_BF16 && out_dt == MOE_BF16) ||
                       (a_dt == MOE_FP8_E4M3 && w_dt == MOE_FP8_E4M3 && out_dt == MOE_BF16);
  if (!pair_ok) return MOE_ERR_BAD_DTYPE;
  if ((int)a_q < 0 || (int)a_q > 7 || (int)w_q < 0 || (int)w_q > 7) return MOE_ERR_UNSUPPORTED;
  // per-token activation scales: E4M3 activations with a per-tensor weight scale
  const bool per_token = a_q == MOE_QUANT_PER_TOKEN;
  if (per_token && (a_dt != MOE_FP8_E4M3 || w_q != MOE_QUANT_PER_TENSOR)) return MOE_ERR_UNSUPPORTED;
  if ((a_q > MOE_QUANT_PER_TENSOR && !per_token) || w_q > MOE_QUANT_PER_TENSOR) return MOE_ERR_UNSUPPORTED;
  if (a_dt == MOE_FP8_E4M3 && ((a_q != MOE_QUANT_PER_TENSOR && !per_token) || w_q != MOE_QUANT_PER_TENSOR))
    return MOE_ERR_UNSUPPORTED;
  if (act != MOE_ACT_NONE && act != MOE_ACT_RELU) return MOE_ERR_UNSUPPORTED;
  if (e < 1 || e > kMaxExperts) return MOE_ERR_BAD_SHAPE;
  if (A < 0 || (int64_t)A >= kMaxRows || !dim_ok(Hin) || !dim_ok(N)) return MOE_ERR_BAD_SHAPE;
  if (gx && gx->src) {
    if (gx->div < 1 || gx->rows < 0 || (A > 0 && gx->rows < 1)) return MOE_ERR_BAD_SHAPE;
    // the gathered rows are addressed with 32-bit byte offsets
    if ((int64_t)gx->rows * Hin * dtype_size(a_dt) >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  }
  if (a_q == MOE_QUANT_PER_TENSOR || per_token) REQUIRE_PTR(a_scale);
  if (w_q == MOE_QUANT_PER_TENSOR) REQUIRE_PTR(w_scale);
  call = GmmCall{a, nullptr, w, nullptr, offsets, e, A, Hin, N, act, out, gx ? *gx : RowMap{}};
  *ws_use = nullptr;
  if (A == 0) return MOE_OK;
  REQUIRE_PTR(a);
  REQUIRE_PTR(w);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(out);
  if (gx) {
    if (gx->src == nullptr && gx->dst == nullptr) return MOE_ERR_NULL_POINTER;
    REQUIRE_ALIGNED(gx->src);
    REQUIRE_ALIGNED(gx->dst);
    REQUIRE_ALIGNED(gx->gate);
  }
  const size_t need = no_split ? 0 : gmm_ws_bytes(a_dt, e, A, Hin, N);
  if (need > 0) {
    REQUIRE_PTR(ws);
    if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  }
  REQUIRE_ALIGNED(a);
  REQUIRE_ALIGNED(w);
  REQUIRE_ALIGNED(offsets);
  REQUIRE_ALIGNED(out);
  REQUIRE_ALIGNED(ws);
  // per-tensor scales are 4-byte device scalars: natural alignment suffices
  call.a_scale = a_q == MOE_QUANT_PER_TENSOR ? a_scale : nullptr;
  call.w_scale = w_q == MOE_QUANT_PER_TENSOR ? w_scale : nullptr;
  if (per_token) {
    REQUIRE_ALIGNED(a_scale);
    call.gx.row_scale = a_scale;
  }
  *ws_use = need > 0 ? ws : nullptr;
  return MOE_OK;
}

// Checks and launch of moe_gmm / moe_gmm_gather / moe_gmm_scatter.
moe_status gmm_checked(const void* a, moe_dtype a_dt, moe_quant_mode a_q, const float* a_scale,
                       const void* w, moe_dtype w_dt, moe_quant_mode w_q, const float* w_scale,
                       const int32_t* offsets, int e, int A, int Hin, int N, moe_act act, void* out,
                       moe_dtype out_dt, void* ws, size_t ws_bytes, void* stream, const RowMap* gx) {
  GmmCall c;
  void* ws_use = nullptr;
  MOE_TRY(gmm_prepare(a, a_dt, a_q, a_scale, w, w_dt, w_q, w_scale, offsets, e, A, Hin, N, act, out, out_dt, ws,
                      ws_bytes, gx, c, &ws_use));
  if (A == 0) return MOE_OK;
  return launch_gmm(c.a, a_dt, c.a_scale, c.w, c.w_scale, c.offsets, c.e, c.A, c.Hin, c.N, c.act, c.out, out_dt,
                    ws_use, (hipStream_t)stream, c.gx);
}
}  // namespace

moe_status moe_gmm(const void* a, moe_dtype a_dt, moe_quant_mode a_q, const float* a_scale,
                   const void* w, moe_dtype w_dt, moe_quant_mode w_q, const float* w_scale,
                   const int32_t* offsets, int e, int A, int Hin, int N, moe_act act, void* out,
                   moe_dtype out_dt, void* ws, size_t ws_bytes, void* stream) {
  return gmm_checked(a, a_dt, a_q, a_scale, w, w_dt, w_q, w_scale, offsets, e, A, Hin, N, act, out,
                     out_dt, ws, ws_bytes, stream, nullptr);
}

moe_status moe_gmm_gather(const void* a, int a_rows, const int32_t* row_src, int row_div, moe_dtype a_dt,
                          moe_quant_mode a_q, const float* a_scale, const void* w, moe_dtype w_dt,
                          moe_quant_mode w_q, const float* w_scale, const int32_t* offsets, int e, int A,
                          int Hin, int N, moe_act act, void* out, moe_dtype out_dt, void* ws,
                          size_t ws_bytes, void* stream) {
  const RowMap gx{row_src, row_div, a_rows};
  return gmm_checked(a, a_dt, a_q, a_scale, w, w_dt, w_q, w_scale, offsets, e, A, Hin, N, act, out,
                     out_dt, ws, ws_bytes, stream, &gx);
}

moe_status moe_gmm_scatter(const void* a, moe_dtype a_dt, moe_quant_mode a_q, const float* a_scale,
                           const void* w, moe_dtype w_dt, moe_quant_mode w_q, const float* w_scale,
                           const int32_t* offsets, int e, int A, int Hin, int N, moe_act act,
                           const int32_t* row_dst, const float* row_gate, void* out, moe_dtype out_dt,
                           void* ws, size_t ws_bytes, void* stream) {
  RowMap gx;
  gx.dst = row_dst;
  gx.gate = row_gate;
  if (A > 0 && row_dst == nullptr) return MOE_ERR_NULL_POINTER;
  return gmm_checked(a, a_dt, a_q, a_scale, w, w_dt, w_q, w_scale, offsets, e, A, Hin, N, act, out,
                     out_dt, ws, ws_bytes, stream, &gx);
}

moe_status moe_gmm_routed_shared(const void* a, moe_quant_mode a_q, const float* a_scale, const void* w,
                                 const float* w_scale, const int32_t* offsets, int e, int A, int Hin, int N,
                                 moe_act act, const int32_t* row_dst, const float* row_gate, void* out,
                                 const void* xs, const void* ws_w, const int32_t* offsets_s, int e_s, int T,
                                 int Hs, int Ns, moe_act act_s, void* ys, void* stream) {
  RowMap gx;
  gx.dst = row_dst;
  gx.gate = row_gate;
  GmmCall f, b;
  void* ws_use = nullptr;
  MOE_TRY(gmm_prepare(a, MOE_FP8_E4M3, a_q, a_scale, w, MOE_FP8_E4M3, MOE_QUANT_PER_TENSOR, w_scale, offsets, e,
                      A, Hin, N, act, out, MOE_BF16, nullptr, 0, row_dst ? &gx : nullptr, f, &ws_use, true));
  MOE_TRY(gmm_prepare(xs, MOE_BF16, MOE_QUANT_NONE, nullptr, ws_w, MOE_BF16, MOE_QUANT_NONE, nullptr, offsets_s,
                      e_s, T, Hs, Ns, act_s, ys, MOE_BF16, nullptr, 0, nullptr, b, &ws_use, true));
  if (A == 0 && T == 0) return MOE_OK;
  return launch_gmm_pair(f, b, (hipStream_t)stream);
}

namespace {
// Argument checks of the MX grouped GEMMs (fp4: E2M1 operands packed two per
// byte along K, else E4M3).
moe_status mx_checked(const void* a, const uint8_t* a_scale, const void* w, const uint8_t* w_scale,
                      const int32_t* offsets, int e, int A, int Hin, int N, moe_act act, void* out, bool fp4) {
  if (act != MOE_ACT_NONE && act != MOE_ACT_RELU) return MOE_ERR_UNSUPPORTED;
  if (e < 1 || e > kMaxExperts) return MOE_ERR_BAD_SHAPE;
  if (A < 0 || (int64_t)A >= kMaxRows || !dim_ok(Hin) || !dim_ok(N)) return MOE_ERR_BAD_SHAPE;
  // whole K slices (128 bytes: 128 E4M3 or 256 E2M1 values) of whole scale
  // blocks, 16-byte column chunks, 32-bit offsets
  if (Hin % (fp4 ? 256 : 128) != 0 || N % 16 != 0) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)(fp4 ? Hin / 2 : Hin) * N >= (1ll << 31) ||
      (int64_t)(Hin / 32) * ((N + 63) & ~63) * e >= (1ll << 31) || (int64_t)(Hin / 32) * A >= (1ll << 31))
    return MOE_ERR_UNSUPPORTED;
  if (A == 0) return MOE_OK;
  REQUIRE_PTR(a);
  REQUIRE_PTR(a_scale);
  REQUIRE_PTR(w);
  REQUIRE_PTR(w_scale);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(out);
  REQUIRE_ALIGNED(a);
  REQUIRE_ALIGNED(a_scale);
  REQUIRE_ALIGNED(w);
  REQUIRE_ALIGNED(w_scale);
  REQUIRE_ALIGNED(offsets);
  REQUIRE_ALIGNED(out);
  return MOE_OK;
}
}  // namespace

moe_status moe_gmm_mx(const void* a, const uint8_t* a_scale, const void* w, const uint8_t* w_scale,
                      const int32_t* offsets, int e, int A, int Hin, int N, moe_act act, void* out,
                      void* stream) {
  MOE_TRY(mx_checked(a, a_scale, w, w_scale, offsets, e, A, Hin, N, act, out, false));
  if (A == 0) return MOE_OK;
  return launch_gmm_mx(a, a_scale, w, w_scale, offsets, e, A, Hin, N, act, out, (hipStream_t)stream);
}

moe_status moe_combine(const void* y_perm, moe_dtype in_dt, const int32_t* perm_dst,
                       const float* topk_gate, int T, int K, int N, void* out, moe_dtype out_dt,
                       void* stream) {
  if (!layer_dtype_ok(in_dt) || out_dt != in_dt) return MOE_ERR_BAD_DTYPE;
  if (T < 0 || K < 1 || K > kMaxK || !dim_ok(N) || (int64_t)T * K >= kMaxRows) return MOE_ERR_BAD_SHAPE;
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(y_perm);
  REQUIRE_PTR(perm_dst);
  REQUIRE_PTR(out);
  REQUIRE_ALIGNED(y_perm);
  REQUIRE_ALIGNED(perm_dst);
  REQUIRE_ALIGNED(topk_gate);
  REQUIRE_ALIGNED(out);
  return launch_combine(y_perm, in_dt, perm_dst, topk_gate, T, K, N, out, (hipStream_t)stream);
}

moe_status moe_quant_rows(const void* x, moe_dtype x_dt, int x_rows, int H, const int32_t* row_src,
                          int row_div, int rows, uint8_t* q, float* scale, void* stream) {
  if (x_dt != MOE_F32 && x_dt != MOE_BF16) return MOE_ERR_BAD_DTYPE;
  if (x_rows < 0 || rows < 0 || !dim_ok(H) || row_div < 1 || (int64_t)rows >= kMaxRows) return MOE_ERR_BAD_SHAPE;
  if (row_src == nullptr && rows > x_rows) return MOE_ERR_BAD_SHAPE;
  if (rows == 0) return MOE_OK;
  REQUIRE_PTR(x);
  REQUIRE_PTR(q);
  REQUIRE_PTR(scale);
  REQUIRE_ALIGNED(x);
  REQUIRE_ALIGNED(row_src);
  REQUIRE_ALIGNED(q);
  REQUIRE_ALIGNED(scale);
  return launch_quant_rows(x, x_dt, x_rows, H, row_src, row_div, rows, q, scale, (hipStream_t)stream);
}

moe_status moe_gmm_mxfp4(const void* a, const uint8_t* a_scale, const void* w, const uint8_t* w_scale,
                         const int32_t* offsets, int e, int A, int Hin, int N, moe_act act, void* out,
                         void* stream) {
  MOE_TRY(mx_checked(a, a_scale, w, w_scale, offsets, e, A, Hin, N, act, out, true));
  if (A == 0) return MOE_OK;
  return launch_gmm_mx(a, a_scale, w, w_scale, offsets, e, A, Hin, N, act, out, (hipStream_t)stream, true);
}

moe_status moe_gmm_mx_routed_shared(const void* a, const uint8_t* a_scale, const void* w, const uint8_t* w_scale,
                                    const int32_t* offsets, int e, int A, int Hin, int N, moe_act act, int fp4,
                                    void* out, const void* xs, const void* ws_w, const int32_t* offsets_s,
                                    int e_s, int T, int Hs, int Ns, moe_act act_s, void* ys, void* stream) {
  if (fp4 != 0 && fp4 != 1) return MOE_ERR_UNSUPPORTED;
  MOE_TRY(mx_checked(a, a_scale, w, w_scale, offsets, e, A, Hin, N, act, out, fp4 != 0));
  GmmCall f{a, nullptr, w, nullptr, offsets, e, A, Hin, N, act, out, RowMap{}, a_scale, w_scale, fp4 ? 2 : 1};
  GmmCall b;
  void* ws_use = nullptr;
  MOE_TRY(gmm_prepare(xs, MOE_BF16, MOE_QUANT_NONE, nullptr, ws_w, MOE_BF16, MOE_QUANT_NONE, nullptr, offsets_s,
                      e_s, T, Hs, Ns, act_s, ys, MOE_BF16, nullptr, 0, nullptr, b, &ws_use, true));
  if (A == 0 && T == 0) return MOE_OK;
  return launch_gmm_pair(f, b, (hipStream_t)stream);
}

moe_status moe_sum_slots(const void* z, moe_dtype dt, int T, int K, int N, void* out, void* stream) {
  if (!layer_dtype_ok(dt)) return MOE_ERR_BAD_DTYPE;
  if (T < 0 || K < 1 || K > kMaxK || !dim_ok(N) || (int64_t)T * K >= kMaxRows) return MOE_ERR_BAD_SHAPE;
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(z);
  REQUIRE_PTR(out);
  REQUIRE_ALIGNED(z);
  REQUIRE_ALIGNED(out);
  return launch_combine(z, dt, nullptr, nullptr, T, K, N, out, (hipStream_t)stream, true);
}

moe_status moe_fetch_probe(const void* buf, size_t bytes, int mode, int shared_window, int kb_per_wave,
                           uint64_t* cycles, void* stream) {
  REQUIRE_PTR(buf);
  REQUIRE_PTR(cycles);
  REQUIRE_ALIGNED(buf);
  if (mode != 0 && mode != 1) return MOE_ERR_UNSUPPORTED;
  if (bytes % 1024 != 0 || bytes > 0x7fffffffu) return MOE_ERR_BAD_SHAPE;
  if (kb_per_wave < 8 || kb_per_wave % 8 != 0 || kb_per_wave > (1 << 20)) return MOE_ERR_BAD_SHAPE;
  const int ncu = probe_device_cus();
  if (ncu <= 0) return MOE_ERR_DEVICE;
  if (bytes < (shared_window ? (size_t)65536 : (size_t)1024 * ncu)) return MOE_ERR_BAD_SHAPE;
  return launch_fetch_probe(buf, bytes, mode, shared_window, kb_per_wave, (unsigned long long*)cycles, ncu,
                            (hipStream_t)stream);
}

moe_status moe_mfma_probe(moe_dtype dt, int iters, float* sink, uint64_t* cycles, void* stream) {
  REQUIRE_PTR(sink);
  REQUIRE_PTR(cycles);
  if (dt != MOE_BF16 && dt != MOE_FP8_E4M3) return MOE_ERR_BAD_DTYPE;
  if (iters < 1 || iters > (1 << 24)) return MOE_ERR_BAD_SHAPE;
  const int ncu = probe_device_cus();
  if (ncu <= 0) return MOE_ERR_DEVICE;
  return launch_mfma_probe(dt == MOE_FP8_E4M3, iters, sink, (unsigned long long*)cycles, ncu, (hipStream_t)stream);
}

moe_status moe_layer_workspace_size(int T, int H, int E, int K, int F, moe_dtype dt, size_t* bytes) {
  REQUIRE_PTR(bytes);
  if (!layer_dtype_ok(dt)) return MOE_ERR_BAD_DTYPE;
  MOE_TRY(check_route_shape(T, H, E, K));
  if (!dim_ok(F)) return MOE_ERR_BAD_SHAPE;
  *bytes = layer_ws_layout(T, H, E, K, F, dt).total;
  return MOE_OK;
}

moe_status moe_layer(const void* x, const void* w_router, const float* bias, const void* w1,
                     const void* w2, moe_dtype dt, int T, int H, int E, int K, int F, moe_act act,
                     void* y, int32_t* topk_idx_out, float* topk_gate_out, int32_t* counts_out,
                     void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(layer_check(x, w_router, bias, w1, w2, dt, T, H, E, K, F, act, y, topk_idx_out, topk_gate_out,
                      counts_out));
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(ws);
  const LayerWs L = layer_ws_layout(T, H, E, K, F, dt);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  REQUIRE_ALIGNED(ws);
  return layer_run(x, w_router, bias, w1, w2, dt, T, H, E, K, F, act, y, topk_idx_out, topk_gate_out, counts_out,
                   (unsigned char*)ws, L, (hipStream_t)stream);
}

moe_status moe_layer_noalloc(const void* x, const void* w_router, const float* bias, const void* w1,
                             const void* w2, moe_dtype dt, int T, int H, int E, int K, int F, moe_act act,
                             void* y, int32_t* topk_idx_out, float* topk_gate_out, int32_t* counts_out,
                             void* stream) {
  MOE_TRY(layer_check(x, w_router, bias, w1, w2, dt, T, H, E, K, F, act, y, topk_idx_out, topk_gate_out,
                      counts_out));
  if (T == 0) return MOE_OK;
  const LayerWs L = layer_ws_layout(T, H, E, K, F, dt);
  if (L.total > kScratchBytes) return MOE_ERR_SCRATCH_LIMIT;
  unsigned char* base = nullptr;
  MOE_TRY(scratch_on_current_device(&base));
  return layer_run(x, w_router, bias, w1, w2, dt, T, H, E, K, F, act, y, topk_idx_out, topk_gate_out, counts_out,
                   base, L, (hipStream_t)stream);
}

moe_status moe_layer_fp8_workspace_size(int T, int H, int E, int K, int F, size_t* bytes) {
  REQUIRE_PTR(bytes);
  MOE_TRY(check_route_shape(T, H, E, K));
  if (!dim_ok(F)) return MOE_ERR_BAD_SHAPE;
  *bytes = layer_fp8_ws_layout(T, H, E, K, F).total;
  return MOE_OK;
}

moe_status moe_layer_fp8(const void* x, const void* w_router, const float* bias, const uint8_t* w1,
                         const float* w1_scale, const uint8_t* w2, const float* w2_scale, int T, int H, int E,
                         int K, int F, moe_act act, void* y, int32_t* topk_idx_out, float* topk_gate_out,
                         int32_t* counts_out, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_route_shape(T, H, E, K));
  if (!dim_ok(F)) return MOE_ERR_BAD_SHAPE;
  if (act != MOE_ACT_NONE && act != MOE_ACT_RELU) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  REQUIRE_PTR(x);
  REQUIRE_PTR(w_router);
  REQUIRE_PTR(w1);
  REQUIRE_PTR(w1_scale);
  REQUIRE_PTR(w2);
  REQUIRE_PTR(w2_scale);
  REQUIRE_PTR(y);
  REQUIRE_PTR(ws);
  const LayerFp8Ws L = layer_fp8_ws_layout(T, H, E, K, F);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  REQUIRE_ALIGNED(x);
  REQUIRE_ALIGNED(w_router);
  REQUIRE_ALIGNED(bias);
  REQUIRE_ALIGNED(w1);
  REQUIRE_ALIGNED(w2);
  REQUIRE_ALIGNED(y);
  REQUIRE_ALIGNED(topk_idx_out);
  REQUIRE_ALIGNED(topk_gate_out);
  REQUIRE_ALIGNED(counts_out);
  REQUIRE_ALIGNED(ws);

  hipStream_t s = (hipStream_t)stream;
  unsigned char* base = (unsigned char*)ws;
  int32_t* idx = topk_idx_out ? topk_idx_out : (int32_t*)(base + L.idx);
  float* gate = topk_gate_out ? topk_gate_out : (float*)(base + L.gate);
  int32_t* counts = counts_out ? counts_out : (int32_t*)(base + L.counts);
  int32_t* offsets = (int32_t*)(base + L.offsets);
  int32_t* psrc = (int32_t*)(base + L.psrc);
  int32_t* pdst = (int32_t*)(base + L.pdst);
  uint8_t* xq = base + L.xq;
  float* xs = (float*)(base + L.xs);
  void* hm = base + L.hm;
  uint8_t* hq = base + L.hq;
  float* hs = (float*)(base + L.hs);
  void* yp = base + L.yp;
  const int A = T * K;
  void* gws = base + L.gmm_ws;
  MOE_TRY(launch_route(x, w_router, MOE_BF16, bias, T, H, E, K, idx, gate, hm, s));
  MOE_TRY(launch_permute(idx, nullptr, MOE_BF16, T, H, E, K, counts, offsets, psrc, pdst, nullptr,
                         base + L.perm_ws, s));
  RowMap r1;
  r1.row_scale = xs;
  if ((int64_t)T * H < (1ll << 31)) {
    // tokens quantised once; GEMM 1 reads row r as token perm_src[r] / K with its scale
    MOE_TRY(launch_quant_rows(x, MOE_BF16, T, H, nullptr, 1, T, xq, xs, s));
    r1.src = psrc;
    r1.div = K;
    r1.rows = T;
  } else {
    // dispatch and quantisation in one pass into A rows
    MOE_TRY(launch_quant_rows(x, MOE_BF16, T, H, psrc, K, A, xq, xs, s));
  }
  MOE_TRY(launch_gmm(xq, MOE_FP8_E4M3, nullptr, w1, w1_scale, offsets, E, A, H, F, act, hm, MOE_BF16,
                     gmm_ws_bytes(MOE_FP8_E4M3, E, A, H, F) ? gws : nullptr, s, r1));
  MOE_TRY(launch_quant_rows(hm, MOE_BF16, A, F, nullptr, 1, A, hq, hs, s));
  RowMap r2;
  r2.row_scale = hs;
  MOE_TRY(launch_gmm(hq, MOE_FP8_E4M3, nullptr, w2, w2_scale, offsets, E, A, F, H, MOE_ACT_NONE, yp, MOE_BF16,
                     gmm_ws_bytes(MOE_FP8_E4M3, E, A, F, H) ? gws : nullptr, s, r2));
  MOE_TRY(launch_combine(yp, MOE_BF16, pdst, gate, T, K, H, y, s));
  return MOE_OK;
}

}  // extern "C"
