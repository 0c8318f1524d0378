// Count rows of the dispatch layout: the expert counts and the (token, rank) pair counts of
// consecutive slices of T tokens, which the layout scans down the slices to give every slot its
// row.
//
// Blog "Kernel fusion for expert parallelism", section "Fusing the layer into one kernel":
// stage "route" computes the routing metadata of a microbatch. Expert Coupling in MoE
// Pretraining section V-A: the deduplicating dispatcher counts a destination rank once per
// token. The rows are written by the layout's own count kernel or, when the route is given a
// layout workspace, by the route itself as it selects (moe_route's kernel or the gate kernel's
// fused epilogue), so the count kernel leaves the dispatch chain.
//
// T is fixed by E alone: the tokens one 256-lane route block covers (256 / lanes per token), at
// most 64 (one 64-bit mask per expert). Every route block, every 64-token gate tile and every
// 256-token layout block holds whole slices, so each writes its rows without atomics.
#pragma once

#include "moe_internal.h"

namespace moe {

// Lanes per token of the route for E experts (route_shape in route_token.h picks the same).
__host__ __device__ constexpr int route_seg(int E) {
  return E <= 1 ? 1 : E <= 2 ? 2 : E <= 4 ? 4 : E <= 8 ? 8 : 16;
}

// Tokens per count row.
__host__ __device__ constexpr int count_tokens(int E) {
  return 256 / route_seg(E) < 64 ? 256 / route_seg(E) : 64;
}

__host__ __device__ inline int count_nrows(int N, int E) {
  return (N + count_tokens(E) - 1) / count_tokens(E);
}

inline size_t count_align256(size_t b) { return (b + 255) & ~size_t(255); }

// The count rows inside a layout workspace, stored by column: [E][nrow] expert counts, then
// [W][nrow] pair counts (each array 256-byte aligned), so the layout's column scan, which turns
// each column into exclusive prefixes down the rows in place, reads contiguous words.
struct CountWs {
  int32_t* e;
  int32_t* p;
  int nrow;
};

inline size_t count_ws_bytes(int N, int E, int W) {
  const size_t nrow = static_cast<size_t>(count_nrows(N, E));
  return count_align256(nrow * E * 4) + count_align256(nrow * W * 4) + 256;
}

inline CountWs count_ws_carve(int N, int E, int W, void* ws) {
  (void)W;
  const size_t nrow = static_cast<size_t>(count_nrows(N, E));
  char* p = static_cast<char*>(ws);
  CountWs c;
  c.e = reinterpret_cast<int32_t*>(p);
  c.p = reinterpret_cast<int32_t*>(p + count_align256(nrow * E * 4));
  c.nrow = static_cast<int>(nrow);
  return c;
}

// Per-64-token bit masks a block fills while it routes: bit i of emask[g][e] is set when token
// 64 g + i of the block selects expert e, bit i of rmask[g][r] when it selects an expert on rank
// r (set once however many of its experts rank r holds: the dedup). OR is order-free, so the
// masks, and the counts below, do not depend on the order of the picks.
struct RouteCount {
  unsigned long long* emask;   // LDS [groups][E], or NULL: no counting
  unsigned long long* rmask;   // LDS [groups][W]
  const int32_t* placement;    // rank of each expert, or NULL (contiguous)
  int e_loc;                   // experts per rank
  int W;
};

__device__ __forceinline__ void count_pick(const RouteCount& rc, int E, int tl, int e) {
  const unsigned long long bit = 1ull << (tl & 63);
  atomicOr(&rc.emask[(tl >> 6) * E + e], bit);
  atomicOr(&rc.rmask[(tl >> 6) * rc.W + rank_of(rc.placement, e, rc.e_loc)], bit);
}

// Writes the count rows of the ntok tokens from t0 (t0 a multiple of T) from the block's masks.
// Rows past the last token (N) do not exist and are not written. All threads of the block call
// it after the barrier that follows the last mask update.
__device__ __forceinline__ void write_count_rows(const unsigned long long* emask,
                                                 const unsigned long long* rmask, int E, int W,
                                                 int T, int t0, int ntok, int N, CountWs cw) {
  const int rows = (ntok + T - 1) / T;
  const int row0 = t0 / T;
  const int cols = E + W;
  for (int i = threadIdx.x; i < rows * cols; i += blockDim.x) {
    const int q = i / cols, c = i - q * cols;
    if (t0 + q * T >= N) continue;
    const int g = (q * T) >> 6;
    const unsigned long long m = T == 64 ? ~0ull : ((1ull << T) - 1ull) << ((q * T) & 63);
    const int row = row0 + q;
    if (c < E) cw.e[static_cast<size_t>(c) * cw.nrow + row] = __popcll(emask[g * E + c] & m);
    else cw.p[static_cast<size_t>(c - E) * cw.nrow + row] = __popcll(rmask[g * W + (c - E)] & m);
  }
}

}  // namespace moe
