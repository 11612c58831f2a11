// dispatch.h — the router and the index path of moe_layer sharing the
// per-chunk expert counts: the router, which holds every selection, writes
// them, and the dispatch ranks from them in one launch instead of counting
// in a launch of its own.
#pragma once
#include "common.h"

namespace moe {

// launch_permute's index path is one block, one launch, up to this many pairs.
constexpr int kPermuteBlockPairs = 4096;

// launch_route, and where the router can (at most 16 experts, H not split)
// per-expert counts of the selections of each run of *blk_tokens consecutive
// tokens: row i of blk_counts (cdiv(T, 16) rows of E ints) covers tokens
// i * *blk_tokens ..; *blk_tokens is 0 when it wrote none.
moe_status launch_route_counted(const void* x, const void* wr, moe_dtype dt, const float* bias, int T, int H,
                                int E, int K, int32_t* idx, float* gate, void* ws, hipStream_t s,
                                int32_t* blk_counts, int* blk_tokens);

// The index path (counts, offsets, perm_src, perm_dst of launch_permute)
// from counts per run of tok_per_row tokens, in one launch; zero[0:nzero] is
// also set to 0. permute_counted_fits tells whether a shape fits it.
bool permute_counted_fits(int T, int E, int K, int tok_per_row);
moe_status launch_permute_counted(const int32_t* idx, int T, int E, int K, const int32_t* row_counts,
                                  int tok_per_row, int32_t* counts, int32_t* offsets, int32_t* perm_src,
                                  int32_t* perm_dst, hipStream_t s, int* zero, int nzero);

}  // namespace moe
