// Dispatch layout and permute.
//
// Blog "Kernel fusion for expert parallelism": section "All-to-All" (a selective send needs
// per-destination counts before the data moves) and section "Fusing the layer into one kernel"
// (Baseline "pack": a contiguous copy of each token per destination; stage "group": rows in
// expert-contiguous order for the grouped GEMM). Expert Coupling in MoE Pretraining section V-A
// and Appendix A-A2 (i): the deduplicating dispatcher sends one row per (token, rank).
//
// Rows are ordered by (rank, expert, token) and pair rows by (rank, token). The build is a
// deterministic counting sort with no global sort and no contended atomics:
//   1. count   (one block per 256 tokens, one wave per 64 tokens): each wave ORs a bit per
//              lane into an LDS mask per expert and per rank. OR is order-free, so a lane's
//              stable rank inside its wave is the popcount of the mask bits below it, and a
//              rank mask bit set by several slots of one token counts once: the dedup.
//              The counts of every slice of T tokens (count_rows.h) go to the workspace. The
//              route writes the same rows when it is given the workspace (counts_ready), and
//              this step is skipped.
//   2. columns (one block per expert / per rank column): exclusive scan of the count rows down
//              the slices, in place, plus the column totals; zeroes the send matrices.
//   3. scatter (same grid as 1): every block derives the group order (rank, expert) and the
//              exclusive scans of the expert and pair totals (block 0 also writes them to the
//              layout), rebuilds the masks and writes every slot's row and pair row, the
//              inverse maps, pair tokens, expand sources and the send matrices (LDS aggregated
//              integer atomics, exact and order-free).
//   4. permute (optional): copies each token row once from HBM into its destinations.
#include <algorithm>
#include <mutex>

#include "count_rows.h"
#include "moe_internal.h"

namespace moe {

constexpr int kLayoutTB = 256;  // tokens per block in count / scatter (4 waves)
constexpr int kSendLds = 2048;  // LDS ints per send matrix slice in scatter
constexpr size_t kScatterLdsMax = 60 * 1024;  // dynamic LDS of a scatter block at most

static inline int layout_nblk(int N) { return (N + kLayoutTB - 1) / kLayoutTB; }

constexpr int kIdsLds = 4096;  // LDS ints for a block's expert ids (k <= 16 with 256 tokens)

// LDS of the count and scatter blocks, sized from E, W and k at launch (dynamic shared memory):
// the per-wave expert and rank masks, the rank of every expert, the block's expert ids (when
// 256 k <= kIdsLds) and, in scatter, the send matrix slices of the owners the block spans and
// the per-wave first rows. Small layer shapes then need a few KB, so these blocks fit on a CU
// beside a grouped-GEMM workgroup (which leaves about 27 KB of the 160 KB free).
struct LayoutLds {
  unsigned long long* emask;  // [4][E]
  unsigned long long* rmask;  // [4][W]
  int* rank_e;                // [E]
  int* ids;                   // [256][k] or NULL
  int* sc;                    // [send_cap] (scatter)
  int* psc;                   // [send_cap] (scatter)
  int* base_e;                // [4][E] (scatter)
  int* base_p;                // [4][W] (scatter)
  int* g_of_e;                // [E] (scatter): group of each expert
  int* off_g;                 // [E] (scatter): first row of each group
  int* first_g;               // [W + 1] (scatter): first group of each rank
  int* pair_off;              // [W + 1] (scatter): first pair row of each rank
  int* tmp;                   // [17] (scatter): scan scratch and total
  unsigned long long* rbits;  // [W][ceil(E / 64)] (scatter): experts of each rank as bit sets
};

// send_cap: LDS ints per send matrix slice (0 in count); returns the bytes (lds == NULL) or
// carves lds.
__host__ __device__ inline size_t layout_lds(int E, int W, int k, int send_cap, bool scatter,
                                             unsigned char* lds, LayoutLds* out) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    unsigned char* p = lds ? lds + off : nullptr;
    off += (bytes + 15) & ~size_t(15);
    return p;
  };
  LayoutLds L{};
  L.emask = reinterpret_cast<unsigned long long*>(take(size_t(4) * E * 8));
  L.rmask = reinterpret_cast<unsigned long long*>(take(size_t(4) * W * 8));
  L.rank_e = reinterpret_cast<int*>(take(size_t(E) * 4));
  const bool stage_ids = k * kLayoutTB <= kIdsLds;
  int* ids = reinterpret_cast<int*>(take(stage_ids ? size_t(kLayoutTB) * k * 4 : 0));
  L.ids = stage_ids ? ids : nullptr;
  if (scatter) {
    L.sc = reinterpret_cast<int*>(take(size_t(send_cap) * 4));
    L.psc = reinterpret_cast<int*>(take(size_t(send_cap) * 4));
    L.base_e = reinterpret_cast<int*>(take(size_t(4) * E * 4));
    L.base_p = reinterpret_cast<int*>(take(size_t(4) * W * 4));
    L.g_of_e = reinterpret_cast<int*>(take(size_t(E) * 4));
    L.off_g = reinterpret_cast<int*>(take(size_t(E) * 4));
    L.first_g = reinterpret_cast<int*>(take(size_t(W + 1) * 4));
    L.pair_off = reinterpret_cast<int*>(take(size_t(W + 1) * 4));
    L.tmp = reinterpret_cast<int*>(take(17 * 4));
    L.rbits = reinterpret_cast<unsigned long long*>(take(size_t(W) * ((E + 63) / 64) * 8));
  }
  if (out) *out = L;
  return off;
}

// Owners (token slices of N / W) that one block of kLayoutTB tokens can span, bounded by W.
inline int layout_owner_span(int N, int W) {
  const int per_owner = N / W;
  return per_owner > 0 ? std::min(W, (kLayoutTB - 1) / per_owner + 2) : W;
}

// Block-local copies of what every slot of the block looks up: the rank of each expert and the
// block's expert ids (staged when they fit), so the per-slot loops touch LDS only.
struct BlockStage {
  int* rank_e;   // [E]
  int* ids;      // [tokens of the block][k], or NULL (then read from topk_idx)
};

// Stages the tables and fills the per-wave expert and rank masks of this block's tokens.
__device__ __forceinline__ void fill_masks(const int32_t* __restrict__ topk_idx,
                                           const int32_t* __restrict__ placement, int N, int E,
                                           int k, int W, const BlockStage& bs,
                                           unsigned long long* emask, unsigned long long* rmask) {
  const int e_loc = E / W;
  const int t0 = blockIdx.x * kLayoutTB;
  const int nt = min(kLayoutTB, N - t0);
  for (int i = threadIdx.x; i < 4 * E; i += blockDim.x) emask[i] = 0ull;
  for (int i = threadIdx.x; i < 4 * W; i += blockDim.x) rmask[i] = 0ull;
  for (int e = threadIdx.x; e < E; e += blockDim.x) bs.rank_e[e] = rank_of(placement, e, e_loc);
  if (bs.ids)
    for (int i = threadIdx.x; i < nt * k; i += blockDim.x)
      bs.ids[i] = topk_idx[static_cast<size_t>(t0) * k + i];
  __syncthreads();
  const int wave = threadIdx.x / kWave;
  const unsigned long long bit = 1ull << lane_id();
  if (static_cast<int>(threadIdx.x) < nt) {
    for (int j = 0; j < k; ++j) {
      const int e = bs.ids ? bs.ids[threadIdx.x * k + j]
                           : topk_idx[static_cast<size_t>(t0 + threadIdx.x) * k + j];
      atomicOr(&emask[wave * E + e], bit);
      atomicOr(&rmask[wave * W + bs.rank_e[e]], bit);
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void layout_count_kernel(const int32_t* __restrict__ topk_idx,
                                                           const int32_t* __restrict__ placement,
                                                           int N, int E, int k, int W, int T,
                                                           CountWs cw) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_dyn[];
  LayoutLds ll;
  layout_lds(E, W, k, 0, false, lds_dyn, &ll);
  unsigned long long* emask = ll.emask;
  unsigned long long* rmask = ll.rmask;
  const BlockStage bs{ll.rank_e, ll.ids};
  fill_masks(topk_idx, placement, N, E, k, W, bs, emask, rmask);
  // the per-wave masks are the 64-token groups write_count_rows reads
  const int t0 = blockIdx.x * kLayoutTB;
  write_count_rows(emask, rmask, E, W, T, t0, min(kLayoutTB, N - t0), N, cw);
}

// Wave-inclusive prefix sum of v over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// Sum of v over the 64 lanes (every lane gets it).
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// One block per column (E expert columns, then W rank columns): exclusive scan of the nrow count
// rows, in place, and the column total. The rows are split into 4 contiguous quarters, one per
// wave: each wave sums its quarter, then scans it from the sum of the quarters before it. Every
// pass issues kColBatch loads per lane (contiguous words of the column) before it uses them.
constexpr int kColBatch = 8;

__global__ __launch_bounds__(256) void layout_columns_kernel(int nrow, int E, int W, CountWs cw,
                                                             moe_layout L) {
  __shared__ int quarter_sum[4];
  // the send matrices start at zero for the scatter's atomic adds
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < W * W; i += gridDim.x * blockDim.x) {
    L.send_counts[i] = 0;
    L.pair_send_counts[i] = 0;
  }
  const int col = blockIdx.x;
  int32_t* base;
  int32_t* total;
  if (col < E) {
    base = cw.e + static_cast<size_t>(col) * nrow;
    total = L.expert_counts + col;
  } else {
    base = cw.p + static_cast<size_t>(col - E) * nrow;
    total = L.pair_counts + (col - E);
  }
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int per = (nrow + 3) / 4;
  const int r0 = min(nrow, wave * per), r1 = min(nrow, r0 + per);
  int sum = 0;
  for (int b0 = r0; b0 < r1; b0 += kWave * kColBatch) {
    int c[kColBatch];
#pragma unroll
    for (int u = 0; u < kColBatch; ++u) {
      const int r = b0 + u * kWave + lane;
      c[u] = r < r1 ? base[r] : 0;
    }
#pragma unroll
    for (int u = 0; u < kColBatch; ++u) sum += c[u];
  }
  sum = wave_sum(sum);
  if (lane == 0) quarter_sum[wave] = sum;
  __syncthreads();
  int carry = 0;
  for (int w2 = 0; w2 < wave; ++w2) carry += quarter_sum[w2];
  if (wave == 3 && lane == 0)
    *total = carry + sum;
  for (int b0 = r0; b0 < r1; b0 += kWave * kColBatch) {
    int c[kColBatch];
#pragma unroll
    for (int u = 0; u < kColBatch; ++u) {
      const int r = b0 + u * kWave + lane;
      c[u] = r < r1 ? base[r] : 0;
    }
#pragma unroll
    for (int u = 0; u < kColBatch; ++u) {
      const int r = b0 + u * kWave + lane;
      const int inc = wave_incl_scan(c[u]);
      if (r < r1) base[r] = carry + inc - c[u];
      carry += __shfl(inc, kWave - 1, kWave);
    }
  }
}

// Block-wide exclusive scan of one value per thread (blockDim.x a multiple of 64, <= 1024).
__device__ int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int inc = wave_incl_scan(v);
  if (lane == kWave - 1) tmp[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int nw = blockDim.x / kWave;
    const int wv = lane < nw ? tmp[lane] : 0;
    const int winc = wave_incl_scan(wv);
    if (lane < nw) tmp[lane] = winc - wv;
    if (lane == nw - 1) *total = winc;
  }
  __syncthreads();
  const int r = tmp[wave] + inc - v;
  __syncthreads();
  return r;
}

// Group order and offsets, computed by every scatter block from the column totals (a separate
// one-block launch would add a kernel boundary to the dispatch chain): group of expert e = its
// position in (rank, expert) order; exclusive scans of the expert totals in group order and of
// the pair totals. Block 0 also writes them to the layout. 256 threads, each holding
// kGroupsPer consecutive groups in the scan. tot_e[i] is the column total of expert
// tid + 256 i and tot_p that of rank tid (loaded by the caller at kernel start). The position
// of e among its rank's experts comes from a bit set per rank: the experts of lower ranks plus
// the bits below e in its own rank's set.
constexpr int kGroupsThreads = 256;
constexpr int kGroupsPer = (MOE_MAX_EXPERTS + kGroupsThreads - 1) / kGroupsThreads;
static_assert(MOE_MAX_RANKS < kGroupsThreads && MOE_MAX_RANKS <= kWave,
              "one thread per rank and one past the last, ranks scanned by one wave");

__device__ void block_groups(const int* rank_e, int E, int W, const moe_layout& L, bool write,
                             const LayoutLds& ll, const int (&tot_e)[kGroupsPer], int tot_p) {
  const int tid = threadIdx.x;
  const int nw = (E + 63) / 64;
  int* g_of_e = ll.g_of_e;
  int* off_g = ll.off_g;
  int* first_g = ll.first_g;
  unsigned long long* rbits = ll.rbits;
  for (int i = tid; i < W * nw; i += kGroupsThreads) rbits[i] = 0ull;
  __syncthreads();
  for (int e = tid; e < E; e += kGroupsThreads)
    atomicOr(&rbits[rank_e[e] * nw + (e >> 6)], 1ull << (e & 63));
  __syncthreads();
  // first group of each rank: exclusive scan of the ranks' expert counts (one wave)
  if (tid < kWave) {
    int c = 0;
    if (tid < W)
      for (int w = 0; w < nw; ++w) c += __popcll(rbits[tid * nw + w]);
    const int inc = wave_incl_scan(c);
    if (tid < W) first_g[tid] = inc - c;
    if (tid == 0) first_g[W] = E;
  }
  __syncthreads();
  for (int e = tid; e < E; e += kGroupsThreads) {
    const int r = rank_e[e];
    int g = first_g[r] + __popcll(rbits[r * nw + (e >> 6)] & ((1ull << (e & 63)) - 1ull));
    for (int w = 0; w < (e >> 6); ++w) g += __popcll(rbits[r * nw + w]);
    g_of_e[e] = g;
    if (write) L.group_expert[g] = e;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kGroupsPer; ++i) {
    const int e = tid + i * kGroupsThreads;
    if (e < E) off_g[g_of_e[e]] = tot_e[i];
  }
  __syncthreads();
  int loc[kGroupsPer];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kGroupsPer; ++i) {
    const int g = tid * kGroupsPer + i;
    loc[i] = g < E ? off_g[g] : 0;
    sum += loc[i];
  }
  int run = block_excl_scan(sum, ll.tmp, ll.tmp + 16);
  const int total = ll.tmp[16];
#pragma unroll
  for (int i = 0; i < kGroupsPer; ++i) {
    const int g = tid * kGroupsPer + i;
    if (g < E) off_g[g] = run;  // now group offsets
    run += loc[i];
  }
  __syncthreads();
  if (write) {
    for (int g = tid; g < E; g += kGroupsThreads) L.group_offsets[g] = off_g[g];
    for (int e = tid; e < E; e += kGroupsThreads) L.expert_offsets[e] = off_g[g_of_e[e]];
    if (tid == 0) L.group_offsets[E] = total;
    if (tid <= W) {
      const int g = first_g[tid];
      L.rank_offsets[tid] = g < E ? off_g[g] : total;
    }
    if (tid < W) {
      const int g0 = first_g[tid], g1 = first_g[tid + 1];
      const int lo = g0 < E ? off_g[g0] : total;
      const int hi = g1 < E ? off_g[g1] : total;
      L.rank_counts[tid] = hi - lo;
    }
  }
  // pair offsets: scan of the W pair totals
  const int pc = tid < W ? tot_p : 0;
  const int poff = block_excl_scan(pc, ll.tmp, ll.tmp + 16);
  if (tid < W) ll.pair_off[tid] = poff;
  if (tid == 0) ll.pair_off[W] = ll.tmp[16];
  if (write) {
    if (tid < W) L.pair_offsets[tid] = poff;
    if (tid == 0) L.pair_offsets[W] = ll.tmp[16];
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void layout_scatter_kernel(const int32_t* __restrict__ topk_idx,
                                                             const int32_t* __restrict__ placement,
                                                             int N, int E, int k, int W,
                                                             int send_cap, int T, CountWs cw,
                                                             moe_layout L) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_dyn[];
  LayoutLds ll;
  layout_lds(E, W, k, send_cap, true, lds_dyn, &ll);
  unsigned long long* emask = ll.emask;
  unsigned long long* rmask = ll.rmask;
  int* sc = ll.sc;
  int* psc = ll.psc;
  int* rank_e = ll.rank_e;
  int* base_e = ll.base_e;  // per wave: first row of expert e for that wave
  int* base_p = ll.base_p;  // per wave: first pair row of rank r
  const BlockStage bs{rank_e, ll.ids};
  // the column totals and this block's scanned count row (the prefix of its first token) do not
  // depend on the block's own work: their loads go out first, beside the expert ids
  const size_t b = static_cast<size_t>(blockIdx.x) * (kLayoutTB / T);
  int tot_e[kGroupsPer], pre_e[kGroupsPer];
#pragma unroll
  for (int i = 0; i < kGroupsPer; ++i) {
    const int e = threadIdx.x + i * kGroupsThreads;
    tot_e[i] = e < E ? L.expert_counts[e] : 0;
    pre_e[i] = e < E ? cw.e[static_cast<size_t>(e) * cw.nrow + b] : 0;
  }
  const int tot_p = static_cast<int>(threadIdx.x) < W ? L.pair_counts[threadIdx.x] : 0;
  const int pre_p =
      static_cast<int>(threadIdx.x) < W ? cw.p[static_cast<size_t>(threadIdx.x) * cw.nrow + b] : 0;
  fill_masks(topk_idx, placement, N, E, k, W, bs, emask, rmask);
  block_groups(rank_e, E, W, L, blockIdx.x == 0, ll, tot_e, tot_p);

  const int per_owner = N / W;
  const int t_first = blockIdx.x * kLayoutTB;
  const int t_last = min(N, t_first + kLayoutTB) - 1;
  const int s0 = t_first / per_owner;
  const int n_own = t_last / per_owner - s0 + 1;
  const bool lds_send = n_own * W <= send_cap;
  if (lds_send) {
    for (int i = threadIdx.x; i < n_own * W; i += blockDim.x) {
      sc[i] = 0;
      psc[i] = 0;
    }
  }
  // a slot's row = its expert's first row + this block's prefix (the scanned count row of its
  // first token) + the earlier waves' counts of the block + the lanes below it in its wave (same
  // for pair rows by rank)
#pragma unroll
  for (int i = 0; i < kGroupsPer; ++i) {
    const int e = threadIdx.x + i * kGroupsThreads;
    if (e >= E) continue;
    int v = ll.off_g[ll.g_of_e[e]] + pre_e[i];
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      base_e[w2 * E + e] = v;
      v += __popcll(emask[w2 * E + e]);
    }
  }
  if (static_cast<int>(threadIdx.x) < W) {
    const int r = threadIdx.x;
    int v = ll.pair_off[r] + pre_p;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      base_p[w2 * W + r] = v;
      v += __popcll(rmask[w2 * W + r]);
    }
  }
  __syncthreads();

  const int t = t_first + threadIdx.x;
  const int wave = threadIdx.x / kWave;
  const unsigned long long below = (1ull << lane_id()) - 1ull;
  if (t < N) {
    const int s = t / per_owner;
    unsigned long long seen = 0ull;   // ranks of this token's earlier slots (W <= 64)
    for (int j = 0; j < k; ++j) {
      const size_t slot = static_cast<size_t>(t) * k + j;
      const int e = bs.ids ? bs.ids[threadIdx.x * k + j] : topk_idx[slot];
      const int r = rank_e[e];
      const int row = base_e[wave * E + e] + __popcll(emask[wave * E + e] & below);
      const int prow = base_p[wave * W + r] + __popcll(rmask[wave * W + r] & below);
      L.row_of_slot[slot] = row;
      L.slot_of_row[row] = static_cast<int32_t>(slot);
      L.pair_of_slot[slot] = prow;
      L.expand_src[row] = prow;
      const bool first = !((seen >> r) & 1ull);
      seen |= 1ull << r;
      if (first) L.pair_token[prow] = t;
      if (lds_send) {
        atomicAdd(&sc[(s - s0) * W + r], 1);
        if (first) atomicAdd(&psc[(s - s0) * W + r], 1);
      } else {
        atomicAdd(&L.send_counts[s * W + r], 1);
        if (first) atomicAdd(&L.pair_send_counts[s * W + r], 1);
      }
    }
  }
  __syncthreads();
  if (lds_send) {
    for (int i = threadIdx.x; i < n_own * W; i += blockDim.x) {
      const int gi = (s0 + i / W) * W + i % W;
      if (sc[i]) atomicAdd(&L.send_counts[gi], sc[i]);
      if (psc[i]) atomicAdd(&L.pair_send_counts[gi], psc[i]);
    }
  }
}

// Permute: one block per source item; reads the token row once (16-byte vectors) and writes it
// to each of its destinations.
//   dst_rank < 0: item = token t; destinations = its k rows (dedup: its distinct pair rows).
//   dst_rank = r: item = the r-th rank's p-th pair row (grid is the bound N; items past the
//                 rank's pair count exit); destinations = the token's rows on rank r relative
//                 to the rank's first row (dedup: the pair row relative to the first pair row).
// The row's address needs only the token, so the first kPermVec vectors of each thread are
// loaded before the destination indices (one memory round trip instead of two before the
// stores).
constexpr int kPermVec = 4;

__global__ __launch_bounds__(256) void permute_kernel(const u32x4* __restrict__ x, int hv, int N,
                                                      int k, int E, int W,
                                                      const int32_t* __restrict__ topk_idx,
                                                      const int32_t* __restrict__ placement,
                                                      moe_layout L, int dedup, int dst_rank,
                                                      u32x4* __restrict__ rows) {
  __shared__ int dst[MOE_MAX_TOPK];
  const int e_loc = E / W;
  int t, p = 0;
  if (dst_rank < 0) {
    t = blockIdx.x;
  } else {
    p = blockIdx.x;
    if (p >= L.pair_counts[dst_rank]) return;
    t = L.pair_token[L.pair_offsets[dst_rank] + p];   // the same word for every thread
  }
  const u32x4* src = x + static_cast<size_t>(t) * hv;
  u32x4 v[kPermVec];
#pragma unroll
  for (int u = 0; u < kPermVec; ++u) {
    const int c = threadIdx.x + u * 256;
    if (c < hv) v[u] = src[c];
  }
  if (threadIdx.x < k) {
    const size_t slot = static_cast<size_t>(t) * k + threadIdx.x;
    int d = -1;
    if (dst_rank < 0) {
      if (!dedup) {
        d = L.row_of_slot[slot];
      } else {
        d = L.pair_of_slot[slot];
        for (int j2 = 0; j2 < static_cast<int>(threadIdx.x); ++j2)
          if (L.pair_of_slot[static_cast<size_t>(t) * k + j2] == d) d = -1;
      }
    } else if (!dedup) {
      if (rank_of(placement, topk_idx[slot], e_loc) == dst_rank)
        d = L.row_of_slot[slot] - L.rank_offsets[dst_rank];
    } else if (threadIdx.x == 0) {
      d = p;
    }
    dst[threadIdx.x] = d;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kPermVec; ++u) {
    const int c = threadIdx.x + u * 256;
    if (c < hv)
      for (int j = 0; j < k; ++j) {
        const int d = dst[j];
        if (d >= 0) rows[static_cast<size_t>(d) * hv + c] = v[u];
      }
  }
  for (int c = threadIdx.x + kPermVec * 256; c < hv; c += 256) {
    const u32x4 w = src[c];
    for (int j = 0; j < k; ++j) {
      const int d = dst[j];
      if (d >= 0) rows[static_cast<size_t>(d) * hv + c] = w;
    }
  }
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_layout_workspace_bytes(const moe_shape* s) {
  if (!moe_host::shape_ok(s)) return 0;
  return count_ws_bytes(s->N, s->E, s->W);
}

namespace {

// Arguments every dispatch entry point checks the same way (the workspace aside).
bool dispatch_args_ok(const moe_shape* s, const moe_layout* L, const void* x, int dtype,
                      int dst_rank, const void* rows_out) {
  return moe_host::shape_ok(s) && L && dst_rank >= -1 && dst_rank < s->W &&
         !(x && (!rows_out || s->H % 8 != 0 || (dtype != MOE_F32 && dtype != MOE_BF16)));
}

// The layout kernels (and the permute) with the per-block counts in `workspace`.
moe_status dispatch_layout_impl(const moe_shape* s, const int32_t* topk_idx,
                                const int32_t* expert_rank, const moe_layout* L, void* workspace,
                                const void* x, int dtype, int dedup, int dst_rank,
                                int counts_ready, void* rows_out, void* stream) {
  if (!topk_idx || !workspace || !L->expert_counts || !L->expert_offsets || !L->group_expert ||
      !L->group_offsets || !L->rank_counts || !L->rank_offsets || !L->send_counts ||
      !L->row_of_slot || !L->slot_of_row || !L->pair_counts || !L->pair_offsets ||
      !L->pair_token || !L->pair_of_slot || !L->pair_send_counts || !L->expand_src) {
    moe_host::set_error("moe_dispatch_layout: NULL pointer");
    return MOE_EINVAL;
  }
  hipStream_t st = moe_host::as_stream(stream);
  const int nblk = layout_nblk(s->N);
  const int T = count_tokens(s->E);
  const CountWs cw = count_ws_carve(s->N, s->E, s->W, workspace);
  const size_t count_lds = layout_lds(s->E, s->W, s->k, 0, false, nullptr, nullptr);
  const int span = layout_owner_span(s->N, s->W);
  int send_cap = span * s->W <= kSendLds ? span * s->W : 0;
  size_t scatter_lds = layout_lds(s->E, s->W, s->k, send_cap, true, nullptr, nullptr);
  if (scatter_lds > kScatterLdsMax) {  // largest shapes: send matrices by global atomics
    send_cap = 0;
    scatter_lds = layout_lds(s->E, s->W, s->k, 0, true, nullptr, nullptr);
  }
  if (!counts_ready)
    hipLaunchKernelGGL(layout_count_kernel, dim3(nblk), dim3(256), count_lds, st, topk_idx,
                       expert_rank, s->N, s->E, s->k, s->W, T, cw);
  hipLaunchKernelGGL(layout_columns_kernel, dim3(s->E + s->W), dim3(256), 0, st,
                     count_nrows(s->N, s->E), s->E, s->W, cw, *L);
  hipLaunchKernelGGL(layout_scatter_kernel, dim3(nblk), dim3(256), scatter_lds, st, topk_idx,
                     expert_rank, s->N, s->E, s->k, s->W, send_cap, T, cw, *L);
  if (x) {
    const int eb = dtype == MOE_F32 ? 4 : 2;
    const int hv = s->H * eb / 16;
    hipLaunchKernelGGL(permute_kernel, dim3(s->N), dim3(256), 0, st,
                       static_cast<const u32x4*>(x), hv, s->N, s->k, s->E, s->W, topk_idx,
                       expert_rank, *L, dedup, dst_rank, static_cast<u32x4*>(rows_out));
  }
  return moe_host::launch_status();
}

}  // namespace

extern "C" moe_status moe_dispatch_layout(const moe_shape* s, const int32_t* topk_idx,
                                          const int32_t* expert_rank, const moe_layout* L,
                                          void* workspace, const void* x, int dtype, int dedup,
                                          int dst_rank, int counts_ready, void* rows_out,
                                          void* stream) {
  if (!dispatch_args_ok(s, L, x, dtype, dst_rank, rows_out)) {
    moe_host::set_error("moe_dispatch_layout: invalid shape or arguments");
    return MOE_EINVAL;
  }
  if (s->N == 0) return MOE_OK;
  return dispatch_layout_impl(s, topk_idx, expert_rank, L, workspace, x, dtype, dedup, dst_rank,
                              counts_ready, rows_out, stream);
}

// ------------------------------------------------------------------------------------------
// The same call with the workspace in a fixed device array, for callers that cannot allocate.
// Each device holds its own copy of `scratch`; host code never passes the array's name to a
// kernel (on the host it only stands for the symbol): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and kept here.
// ------------------------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[MOE_LAYOUT_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[MOE_MAX_DEVICES];

static void* layout_scratch(int dev) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

extern "C" moe_status moe_dispatch_layout_noalloc(const moe_shape* s, const int32_t* topk_idx,
                                                  const int32_t* expert_rank,
                                                  const moe_layout* L, const void* x, int dtype,
                                                  int dedup, int dst_rank, void* rows_out,
                                                  void* stream) {
  if (!dispatch_args_ok(s, L, x, dtype, dst_rank, rows_out)) {
    moe_host::set_error("moe_dispatch_layout_noalloc: invalid shape or arguments");
    return MOE_EINVAL;
  }
  if (moe_layout_workspace_bytes(s) > MOE_LAYOUT_SCRATCH_BYTES) {
    moe_host::set_error("moe_dispatch_layout_noalloc: the layout needs more scratch than the "
                        "library's fixed array holds (ceil(N / 256) * (E + W) * 4 bytes must "
                        "stay within MOE_LAYOUT_SCRATCH_BYTES)");
    return MOE_EINVAL;
  }
  if (s->N == 0) return MOE_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MOE_MAX_DEVICES) {
    moe_host::set_error("moe_dispatch_layout_noalloc: no current device (or its ordinal is "
                        "beyond MOE_MAX_DEVICES)");
    return MOE_EHIP;
  }
  void* ws = layout_scratch(dev);
  if (!ws) {
    moe_host::set_error("moe_dispatch_layout_noalloc: hipGetSymbolAddress of the scratch array "
                        "failed");
    return MOE_EHIP;
  }
  return dispatch_layout_impl(s, topk_idx, expert_rank, L, ws, x, dtype, dedup, dst_rank,
                              /*counts_ready=*/0, rows_out, stream);
}
