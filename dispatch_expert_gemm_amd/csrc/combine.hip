// Combine: weighted gather-sum of expert output rows back into token order.
//
// FarSkip-Collective section 2.1 (the combine sums the routed experts' weighted outputs into the
// layer output, shared experts added); blog "Kernel fusion for expert parallelism", sections
// "All-to-All" (the owner of a token sums the rows returned to it) and "INC All-to-All-Combine"
// (the expert rank applies the routing weights before publishing its partial sums); Expert
// Coupling in MoE Pretraining section V-A (dedup combine: one weighted partial per (token, rank)).
//
// One block per output row. The block first lists the row's terms (source row, weight) in LDS,
// then each thread owns 16-byte column vectors and sums the terms in list order in fp32, so
// every source row is read with coalesced 16-byte loads and the output written once.
#include "moe_internal.h"

namespace moe {

enum CombineMode { kSlots = 0, kPairReduce = 1, kOwnerSum = 2 };

template <typename T>
struct Vec;  // one 16-byte vector of T as fp32 lanes
template <>
struct Vec<float> {
  static constexpr int n = 4;
  __device__ static void load(const void* p, float* f) {
    const f32x4 v = *static_cast<const f32x4*>(p);
    f[0] = v[0]; f[1] = v[1]; f[2] = v[2]; f[3] = v[3];
  }
  __device__ static void store(void* p, const float* f) {
    f32x4 v;
    v[0] = f[0]; v[1] = f[1]; v[2] = f[2]; v[3] = f[3];
    *static_cast<f32x4*>(p) = v;
  }
};
template <>
struct Vec<bf16_t> {
  static constexpr int n = 8;
  __device__ static void load(const void* p, float* f) {
    const u32x4 v = *static_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  __device__ static void store(void* p, const float* f) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = static_cast<uint32_t>(f32_to_bf16(f[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(f[2 * i + 1])) << 16);
    *static_cast<u32x4*>(p) = v;
  }
};

struct CombineArgs {
  const void* src;          // rows summed (y rows, or partials for kOwnerSum)
  const int32_t* topk_idx;
  const float* topk_w;
  const int32_t* placement;
  moe_layout L;
  const void* shared;       // [n_shared, N, H] or NULL
  int n_shared;
  void* out;
  int N, E, k, W, H;
  int row_begin;            // first output item (token, or pair row for kPairReduce)
  int src_is_pair;          // kPairReduce: every term reads src row p
  int pair_rank;            // kPairReduce: -1 = every pair row, r = rank r's pair rows only
};

template <typename T, int MODE>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  __shared__ int src_row[MOE_MAX_TOPK];
  __shared__ float src_w[MOE_MAX_TOPK];
  __shared__ int tok_s, rank_s;
  const int item = a.row_begin + blockIdx.x;
  const int k = a.k;
  const int e_loc = a.E / a.W;
  int t;
  int out_row = blockIdx.x;
  if (MODE == kPairReduce) {
    int p = item;
    if (a.pair_rank >= 0) {          // rank r's pair rows only: they start at pair_offsets[r]
      p = a.L.pair_offsets[a.pair_rank] + blockIdx.x;
      if (p >= a.L.pair_offsets[a.pair_rank + 1]) return;
    } else if (p >= a.L.pair_offsets[a.W]) {
      return;  // beyond D
    }
    out_row = p;
    if (threadIdx.x == 0) {
      tok_s = a.L.pair_token[p];
      int r = a.pair_rank;
      if (r < 0) {
        r = 0;
        while (r + 1 < a.W && a.L.pair_offsets[r + 1] <= p) ++r;
      }
      rank_s = r;
    }
    __syncthreads();
    t = tok_s;
  } else {
    t = item;
  }
  if (threadIdx.x < k) {
    const int j = threadIdx.x;
    const size_t slot = static_cast<size_t>(t) * k + j;
    int row = -1;
    float w = 0.f;
    if (MODE == kSlots) {
      row = a.L.row_of_slot[slot];
      w = a.topk_w[slot];
    } else if (MODE == kPairReduce) {
      if (rank_of(a.placement, a.topk_idx[slot], e_loc) == rank_s) {
        row = a.src_is_pair ? out_row : a.L.row_of_slot[slot];
        w = a.topk_w[slot];
      }
    } else {  // kOwnerSum: one term per distinct pair row, in first-slot order
      row = a.L.pair_of_slot[slot];
      for (int j2 = 0; j2 < j; ++j2)
        if (a.L.pair_of_slot[static_cast<size_t>(t) * k + j2] == row) row = -1;
      w = 1.f;
    }
    src_row[j] = row;
    src_w[j] = w;
  }
  __syncthreads();

  constexpr int VN = Vec<T>::n;
  const int hv = a.H / VN;
  const T* src = static_cast<const T*>(a.src);
  const T* shared = static_cast<const T*>(a.shared);
  T* out = static_cast<T*>(a.out) + static_cast<size_t>(out_row) * a.H;
  for (int c = threadIdx.x; c < hv; c += blockDim.x) {
    float acc[VN];
#pragma unroll
    for (int i = 0; i < VN; ++i) acc[i] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int row = src_row[j];
      if (row < 0) continue;
      float v[VN];
      Vec<T>::load(src + static_cast<size_t>(row) * a.H + c * VN, v);
      const float w = src_w[j];
      if (MODE == kOwnerSum) {
#pragma unroll
        for (int i = 0; i < VN; ++i) acc[i] += v[i];
      } else {
#pragma unroll
        for (int i = 0; i < VN; ++i) acc[i] += w * v[i];
      }
    }
    if (MODE != kPairReduce) {
      for (int s = 0; s < a.n_shared; ++s) {
        float v[VN];
        Vec<T>::load(shared + (static_cast<size_t>(s) * a.N + t) * a.H + c * VN, v);
#pragma unroll
        for (int i = 0; i < VN; ++i) acc[i] += v[i];
      }
    }
    Vec<T>::store(out + c * VN, acc);
  }
}

template <typename T>
static void launch_combine(const CombineArgs& a, int dedup, int dst_rank, int t_begin,
                           int t_end, void* partial, hipStream_t s) {
  if (!dedup) {
    CombineArgs b = a;
    b.row_begin = t_begin;
    hipLaunchKernelGGL((combine_kernel<T, kSlots>), dim3(t_end - t_begin), dim3(256), 0, s, b);
    return;
  }
  // expert-rank side: every pair row (grid is the bound N * min(k, W); items past D exit), or
  // rank dst_rank's pair rows only (at most N; blocks past the rank's last pair row exit)
  CombineArgs r = a;
  r.row_begin = 0;
  r.out = partial;
  r.pair_rank = dst_rank;
  const int bound = dst_rank >= 0 ? a.N : a.N * (a.k < a.W ? a.k : a.W);
  hipLaunchKernelGGL((combine_kernel<T, kPairReduce>), dim3(bound), dim3(256), 0, s, r);
  // owner side
  CombineArgs o = a;
  o.src = partial;
  o.row_begin = t_begin;
  hipLaunchKernelGGL((combine_kernel<T, kOwnerSum>), dim3(t_end - t_begin), dim3(256), 0, s, o);
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_combine(const moe_shape* s, const void* y, int y_is_pair_rows,
                                  const moe_layout* L, const int32_t* topk_idx,
                                  const float* topk_w, const int32_t* expert_rank, int dtype,
                                  int dedup, int dst_rank, int t_begin, int t_end,
                                  const void* shared,
                                  int n_shared, void* partial, void* out, void* stream) {
  if (!moe_host::shape_ok(s) || !L || (dtype != MOE_F32 && dtype != MOE_BF16) ||
      s->H % 8 != 0 || t_begin < 0 || t_end < t_begin || t_end > s->N || n_shared < 0 ||
      dst_rank < -1 || dst_rank >= s->W ||
      (n_shared > 0 && !shared)) {
    moe_host::set_error("moe_combine: invalid shape or arguments");
    return MOE_EINVAL;
  }
  if (t_end == t_begin || s->H == 0) return MOE_OK;
  if (!y || !topk_w || !out || !L->row_of_slot || (dedup && (!partial || !topk_idx ||
      !L->pair_offsets || !L->pair_token || !L->pair_of_slot))) {
    moe_host::set_error("moe_combine: NULL pointer");
    return MOE_EINVAL;
  }
  CombineArgs a;
  a.src = y;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.placement = expert_rank;
  a.L = *L;
  a.shared = n_shared > 0 ? shared : nullptr;
  a.n_shared = n_shared;
  a.out = out;
  a.N = s->N;
  a.E = s->E;
  a.k = s->k;
  a.W = s->W;
  a.H = s->H;
  a.row_begin = 0;
  a.src_is_pair = y_is_pair_rows;
  a.pair_rank = -1;
  hipStream_t st = moe_host::as_stream(stream);
  if (dtype == MOE_F32)
    launch_combine<float>(a, dedup, dst_rank, t_begin, t_end, partial, st);
  else
    launch_combine<bf16_t>(a, dedup, dst_rank, t_begin, t_end, partial, st);
  return moe_host::launch_status();
}
