// Token-shuffle planner: owner rank of every token of the coming MoE position.
//
// Expert Coupling in MoE Pretraining, section V-B ("Cross-Layer Correlation: Token Shuffling")
// and Appendix "Token shuffling", Algorithm 2. Offline, routing traces give, under the
// placement, the rank distribution of a token's position-m expert slots given the expert it
// used at m-1 (first-order table F) and the pair it used at m-2 and m-1 (second-order table S),
// with the pair's support n. At run time each token's distribution d_t mixes the two per pair
// with the back-off weight w = min(n / (n + beta), w_max); tokens are then assigned, most
// confident (largest minus second largest entry of d_t) first, to the best rank with capacity
// left under a cap of T / P per rank, and laid out owner-major.
//
// Kernels:
//   fit:     zero the counts, count with integer atomics (one thread per trace token), then
//            normalise each row with one fp32 division per entry;
//   predict: one wave per token, lane r for rank r (P <= 64); fp32 sums, wave reductions for the
//            normalisation and the two largest entries; the confidence becomes a 32-bit key
//            that orders tokens most confident first;
//   sort:    one workgroup, stable LSD radix sort of (key, token) by 4-bit digits (8 passes),
//            digit-major prefix counts in LDS;
//   assign:  one workgroup; three waves stage chunks of sorted tokens and their rows in LDS
//            while one wave walks the previous chunk 64 tokens at a time: every lane takes the
//            best rank with capacity left, lanes are committed in order up to the first one
//            whose rank the earlier lanes of the group have filled, and the rest choose again
//            (so the result is exactly the sequential greedy);
//   order:   the same sort, two passes, of the tokens by owner, then order and inverse.
#include "moe_internal.h"

namespace moe {

constexpr int kSortThreads = 1024;
constexpr int kSortDigits = 16;

__global__ void shuffle_zero_kernel(int32_t* a, long long n) {
  for (long long i = blockIdx.x * static_cast<long long>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<long long>(gridDim.x) * blockDim.x)
    a[i] = 0;
}

// One thread per trace token: F counts [E, P], S counts [E, E, P], supports n [E, E].
__global__ void shuffle_count_kernel(const int32_t* prev2, const int32_t* prev1,
                                     const int32_t* cur, int T, int k, int E, int P,
                                     const int32_t* placement, int32_t* f_cnt, int32_t* s_cnt,
                                     int32_t* n) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  int rk[MOE_MAX_TOPK];
  for (int j = 0; j < k; ++j) {
    const int x = cur[static_cast<size_t>(t) * k + j];
    const int r = (x >= 0 && x < E) ? placement[x] : -1;
    rk[j] = (r >= 0 && r < P) ? r : -1;
  }
  for (int b = 0; b < k; ++b) {
    const int e = prev1[static_cast<size_t>(t) * k + b];
    if (e < 0 || e >= E) continue;
    for (int j = 0; j < k; ++j)
      if (rk[j] >= 0) atomicAdd(&f_cnt[e * P + rk[j]], 1);
    for (int a = 0; a < k; ++a) {
      const int e2 = prev2[static_cast<size_t>(t) * k + a];
      if (e2 < 0 || e2 >= E) continue;
      const size_t pair = static_cast<size_t>(e2) * E + e;
      atomicAdd(&n[pair], 1);
      for (int j = 0; j < k; ++j)
        if (rk[j] >= 0) atomicAdd(&s_cnt[pair * P + rk[j]], 1);
    }
  }
}

// One thread per row: rows 0 .. E-1 of F, then the E*E rows of S.
__global__ void shuffle_normalize_kernel(const int32_t* f_cnt, const int32_t* s_cnt, int E, int P,
                                         float* F, float* S) {
  const long long row = blockIdx.x * static_cast<long long>(blockDim.x) + threadIdx.x;
  const long long rows = E + static_cast<long long>(E) * E;
  if (row >= rows) return;
  const bool first = row < E;
  const int32_t* c = first ? f_cnt + row * P : s_cnt + (row - E) * P;
  float* out = first ? F + row * P : S + (row - E) * P;
  long long tot = 0;
  for (int r = 0; r < P; ++r) tot += c[r];
  const float ft = static_cast<float>(tot);
  for (int r = 0; r < P; ++r)
    out[r] = tot > 0 ? static_cast<float>(c[r]) / ft
                     : (first ? 1.0f / static_cast<float>(P) : 0.0f);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// One wave per token, lane r < P for rank r.
__global__ __launch_bounds__(256) void shuffle_predict_kernel(
    const int32_t* prev2, const int32_t* prev1, int T, int k, int E, int P, const float* F,
    const float* S, const int32_t* n, float beta, float w_max, float* d, float* conf,
    uint32_t* keys, int32_t* vals) {
  const int t = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6);
  if (t >= T) return;
  const int l = threadIdx.x & 63;
  const bool on = l < P;
  float acc = 0.f;
  for (int b = 0; b < k; ++b) {
    const int e = prev1[static_cast<size_t>(t) * k + b];
    if (e < 0 || e >= E) continue;
    const float fr = on ? F[static_cast<size_t>(e) * P + l] : 0.f;
    for (int a = 0; a < k; ++a) {
      const int e2 = prev2[static_cast<size_t>(t) * k + a];
      if (e2 < 0 || e2 >= E) continue;
      const size_t pair = static_cast<size_t>(e2) * E + e;
      const float nn = static_cast<float>(n[pair]);
      const float w = nn > 0.f ? fminf(nn / (nn + beta), w_max) : 0.f;
      const float sr = on ? S[pair * P + l] : 0.f;
      acc += (1.f - w) * fr + w * sr;
    }
  }
  const float tot = wave_sum(on ? acc : 0.f);
  // a token with no valid expert index gets the uniform distribution
  const float v = on ? (tot > 0.f ? acc / tot : 1.f / static_cast<float>(P)) : -1.f;
  if (on) d[static_cast<size_t>(t) * P + l] = v;
  // confidence: largest minus second largest (the largest taken out once, at its lowest lane)
  const float top1 = wave_max(v);
  const unsigned long long at = __ballot(on && v == top1);
  const int first = __ffsll(static_cast<long long>(at)) - 1;
  const float top2 = P > 1 ? wave_max(l == first ? -1.f : v) : 0.f;
  if (l == 0) {
    const float c = top1 - top2;
    conf[t] = c;
    // non-negative floats order like their bit patterns: the complement sorts most confident
    // first
    keys[t] = ~__float_as_uint(c);
    vals[t] = t;
  }
}

// Stable ascending sort of (key, value) by one workgroup: `passes` passes of 4-bit digits from
// the lowest. Thread i owns elements [i c, (i + 1) c); per pass it counts its digits, the
// 16 x 1024 counts are scanned in digit-major order, and it scatters its elements in order.
// init_keys != NULL first loads keys = init_keys and vals = 0, 1, 2, ... The result ends in
// keys/vals (passes is even); tk/tv are the other buffers.
__global__ __launch_bounds__(kSortThreads) void shuffle_sort_kernel(uint32_t* keys, int32_t* vals,
                                                                    uint32_t* tk, int32_t* tv,
                                                                    int T, int passes,
                                                                    const int32_t* init_keys) {
  __shared__ int32_t hist[kSortDigits * kSortThreads];
  __shared__ int32_t wsum[kSortThreads / kWave];
  const int i = threadIdx.x;
  const int l = i & 63, wv = i >> 6;
  const int chunk = (T + kSortThreads - 1) / kSortThreads;
  const int lo = min(T, i * chunk), hi = min(T, lo + chunk);
  if (init_keys) {
    for (int j = lo; j < hi; ++j) {
      keys[j] = static_cast<uint32_t>(init_keys[j]);
      vals[j] = j;
    }
  }
  uint32_t* src_k = keys;
  int32_t* src_v = vals;
  uint32_t* dst_k = tk;
  int32_t* dst_v = tv;
  for (int pass = 0; pass < passes; ++pass) {
    const int sh = pass * 4;
    int cnt[kSortDigits];
#pragma unroll
    for (int dg = 0; dg < kSortDigits; ++dg) cnt[dg] = 0;
    for (int j = lo; j < hi; ++j) {
      const int dg = (src_k[j] >> sh) & 15;
#pragma unroll
      for (int q = 0; q < kSortDigits; ++q) cnt[q] += (q == dg);
    }
#pragma unroll
    for (int dg = 0; dg < kSortDigits; ++dg) hist[dg * kSortThreads + i] = cnt[dg];
    __syncthreads();
    // exclusive scan of hist[0 .. 16384): thread i scans entries [16 i, 16 i + 16)
    int local[kSortDigits];
    int s = 0;
#pragma unroll
    for (int q = 0; q < kSortDigits; ++q) {
      local[q] = s;
      s += hist[i * kSortDigits + q];
    }
    int inc = s;                                       // inclusive scan of s over threads
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int x = __shfl_up(inc, o, kWave);
      if (l >= o) inc += x;
    }
    if (l == kWave - 1) wsum[wv] = inc;
    __syncthreads();
    int before = 0;
    for (int w2 = 0; w2 < wv; ++w2) before += wsum[w2];
    const int base = before + inc - s;
#pragma unroll
    for (int q = 0; q < kSortDigits; ++q) hist[i * kSortDigits + q] = base + local[q];
    __syncthreads();
    int off[kSortDigits];
#pragma unroll
    for (int dg = 0; dg < kSortDigits; ++dg) off[dg] = hist[dg * kSortThreads + i];
    for (int j = lo; j < hi; ++j) {
      const uint32_t key = src_k[j];
      const int dg = (key >> sh) & 15;
      int pos = 0;
#pragma unroll
      for (int q = 0; q < kSortDigits; ++q)
        if (q == dg) pos = off[q]++;
      dst_k[pos] = key;
      dst_v[pos] = src_v[j];
    }
    __syncthreads();                                   // this pass's writes before next reads
    uint32_t* xk = src_k;
    int32_t* xv = src_v;
    src_k = dst_k;
    src_v = dst_v;
    dst_k = xk;
    dst_v = xv;
  }
}

constexpr int kAssignRows = 8192;                      // LDS floats per buffer of staged rows
constexpr int kAssignTokens = 1024;                    // tokens per chunk at most

// The capped greedy over the sorted tokens. Chunks of C tokens (C a multiple of 64) with their
// distribution rows are staged in LDS by waves 1-3 while wave 0 assigns the previous chunk, 64
// tokens at a time: every lane takes the best rank with capacity left, lanes are committed in
// order up to the first one whose rank the earlier lanes of the group have filled, and the rest
// choose again.
__global__ __launch_bounds__(256) void shuffle_assign_kernel(const int32_t* sorted, const float* d,
                                                             int T, int P, int32_t* owner) {
  __shared__ float rows[2][kAssignRows];
  __shared__ int32_t tok[2][kAssignTokens];
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int stride = P | 1;                            // odd: lanes reading entry r hit
                                                       // different banks
  int C = kAssignRows / stride;
  C = min(kAssignTokens, C) & ~(kWave - 1);            // P <= 64: at least 64
  const int chunks = (T + C - 1) / C;
  // stage chunk c into buffer b (threads first..first+nthr-1 of the workgroup take part)
  auto stage = [&](int c, int b, int first, int nthr) {
    const int j0 = c * C, n = min(C, T - j0);
    for (int j = tid - first; j < n; j += nthr) {
      const int t = sorted[j0 + j];
      tok[b][j] = t;
      for (int r = 0; r < P; ++r) rows[b][j * stride + r] = d[static_cast<size_t>(t) * P + r];
    }
  };
  stage(0, 0, 0, 256);
  __syncthreads();
  const unsigned long long lt = (1ull << l) - 1;       // lanes below this one
  int cap = l < P ? T / P : 0;                          // wave 0, lane r: capacity left on rank r
  for (int c = 0; c < chunks; ++c) {
    const int b = c & 1;
    if (w > 0) {
      if (c + 1 < chunks) stage(c + 1, b ^ 1, 64, 192);
    } else {
      const int j0 = c * C, n = min(C, T - j0);
      for (int g = 0; g < n; g += kWave) {
        const int t = g + l < n ? tok[b][g + l] : -1;
        const float* row = &rows[b][(g + l) * stride];
        bool pending = t >= 0;
        // every round commits at least the first pending lane (its rank is open, position 0);
        // the round limit and the open-rank test only guard against a malformed token list
        for (int round = 0; __ballot(pending) && round <= kWave + P; ++round) {
          const unsigned long long open = __ballot(cap > 0);
          int best = -1;
          float bv = 0.f;
          if (pending) {
            for (int r = 0; r < P; ++r) {
              if (!((open >> r) & 1)) continue;
              const float v = row[r];
              if (best < 0 || v > bv) {                // strict: the lower rank keeps ties
                best = r;
                bv = v;
              }
            }
          }
          if (!__ballot(pending && best >= 0)) break;
          // position of each pending lane among the pending lanes that chose the same rank
          int pos = 0, left = 0;
          for (int r = 0; r < P; ++r) {
            const unsigned long long m = __ballot(pending && best == r);
            const int cr = __shfl(cap, r, kWave);
            if (pending && best == r) {
              pos = __popcll(m & lt);
              left = cr;
            }
          }
          const unsigned long long over = __ballot(pending && pos >= left);
          const int f = over ? __ffsll(static_cast<long long>(over)) - 1 : kWave;
          const bool commit = pending && l < f;
          if (commit) owner[t] = best;
          for (int r = 0; r < P; ++r) {
            const int taken = __popcll(__ballot(commit && best == r));
            if (l == r) cap -= taken;
          }
          pending = pending && !commit;
        }
      }
    }
    __syncthreads();                                   // chunk c + 1 staged, chunk c done
  }
}

// order[i] = vals[i] (tokens sorted by owner, stably), inverse[order[i]] = i.
__global__ void shuffle_order_kernel(const int32_t* vals, int T, int32_t* order,
                                     int32_t* inverse) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T) return;
  const int t = vals[i];
  order[i] = t;
  if (t >= 0 && t < T) inverse[t] = i;
}

}  // namespace moe

using namespace moe;

static size_t align256(size_t b) { return (b + 255) / 256 * 256; }

extern "C" size_t moe_shuffle_fit_workspace_bytes(int E, int P) {
  if (E <= 0 || P <= 0) return 0;
  return align256(static_cast<size_t>(E) * P * 4) + align256(static_cast<size_t>(E) * E * P * 4);
}

extern "C" size_t moe_shuffle_plan_workspace_bytes(int T) {
  if (T <= 0) return 0;
  return 4 * align256(static_cast<size_t>(T) * 4);
}

static bool shuffle_shape_ok(int T, int k, int E, int P) {
  return T >= 0 && k >= 1 && k <= MOE_MAX_TOPK && P >= 1 && P <= 64 && E >= 1 && E <= 4096 &&
         static_cast<long long>(E) * E * P <= (1ll << 28);
}

extern "C" moe_status moe_shuffle_fit(const int32_t* prev2, const int32_t* prev1,
                                      const int32_t* cur, int T, int k, int E, int P,
                                      const int32_t* placement, void* workspace, float* F,
                                      float* S, int32_t* n, void* stream) {
  if (!shuffle_shape_ok(T, k, E, P) || T > (1 << 24)) {
    moe_host::set_error("moe_shuffle_fit: invalid shape (need 1 <= k <= MOE_MAX_TOPK, "
                        "1 <= P <= 64, 1 <= E <= 4096, E*E*P <= 2^28, 0 <= T <= 2^24)");
    return MOE_EINVAL;
  }
  if (!placement || !workspace || !F || !S || !n || (T > 0 && (!prev2 || !prev1 || !cur))) {
    moe_host::set_error("moe_shuffle_fit: NULL pointer");
    return MOE_EINVAL;
  }
  hipStream_t st = moe_host::as_stream(stream);
  int32_t* f_cnt = static_cast<int32_t*>(workspace);
  int32_t* s_cnt = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                              align256(static_cast<size_t>(E) * P * 4));
  const long long nf = static_cast<long long>(E) * P, ns = static_cast<long long>(E) * E * P,
                  nn = static_cast<long long>(E) * E;
  hipLaunchKernelGGL(shuffle_zero_kernel, dim3(256), dim3(256), 0, st, f_cnt, nf);
  hipLaunchKernelGGL(shuffle_zero_kernel, dim3(1024), dim3(256), 0, st, s_cnt, ns);
  hipLaunchKernelGGL(shuffle_zero_kernel, dim3(256), dim3(256), 0, st, n, nn);
  if (T > 0)
    hipLaunchKernelGGL(shuffle_count_kernel, dim3((T + 255) / 256), dim3(256), 0, st, prev2,
                       prev1, cur, T, k, E, P, placement, f_cnt, s_cnt, n);
  const long long rows = E + nn;
  hipLaunchKernelGGL(shuffle_normalize_kernel, dim3(static_cast<unsigned>((rows + 255) / 256)),
                     dim3(256), 0, st, f_cnt, s_cnt, E, P, F, S);
  return moe_host::launch_status();
}

extern "C" moe_status moe_shuffle_plan(const int32_t* prev2, const int32_t* prev1, int T, int k,
                                       int E, int P, const float* F, const float* S,
                                       const int32_t* n, float beta, float w_max,
                                       void* workspace, float* d, float* conf, int32_t* owner,
                                       int32_t* order, int32_t* inverse, void* stream) {
  if (!shuffle_shape_ok(T, k, E, P) || T > (1 << 20) || (P > 0 && T % P) || !(beta >= 0.f) ||
      !(w_max >= 0.f) || !(w_max <= 1.f)) {
    moe_host::set_error("moe_shuffle_plan: invalid shape (need T a multiple of P, T <= 2^20, "
                        "1 <= P <= 64, 1 <= k <= MOE_MAX_TOPK, beta >= 0, 0 <= w_max <= 1)");
    return MOE_EINVAL;
  }
  if (T == 0) return MOE_OK;
  if (!prev2 || !prev1 || !F || !S || !n || !workspace || !d || !conf || !owner || !order ||
      !inverse) {
    moe_host::set_error("moe_shuffle_plan: NULL pointer");
    return MOE_EINVAL;
  }
  hipStream_t st = moe_host::as_stream(stream);
  char* ws = static_cast<char*>(workspace);
  const size_t part = align256(static_cast<size_t>(T) * 4);
  uint32_t* keys = reinterpret_cast<uint32_t*>(ws);
  int32_t* vals = reinterpret_cast<int32_t*>(ws + part);
  uint32_t* tk = reinterpret_cast<uint32_t*>(ws + 2 * part);
  int32_t* tv = reinterpret_cast<int32_t*>(ws + 3 * part);
  hipLaunchKernelGGL(shuffle_predict_kernel, dim3((T + 3) / 4), dim3(256), 0, st, prev2, prev1,
                     T, k, E, P, F, S, n, beta, w_max, d, conf, keys, vals);
  // most confident first (8 passes over the 32-bit keys), the greedy, then the owner-major
  // order as a stable sort of the tokens by owner (2 passes cover owners below 256)
  hipLaunchKernelGGL(shuffle_sort_kernel, dim3(1), dim3(kSortThreads), 0, st, keys, vals, tk, tv,
                     T, 8, static_cast<const int32_t*>(nullptr));
  hipLaunchKernelGGL(shuffle_assign_kernel, dim3(1), dim3(256), 0, st, vals, d, T, P, owner);
  hipLaunchKernelGGL(shuffle_sort_kernel, dim3(1), dim3(kSortThreads), 0, st, keys, vals, tk, tv,
                     T, 2, static_cast<const int32_t*>(owner));
  hipLaunchKernelGGL(shuffle_order_kernel, dim3((T + 255) / 256), dim3(256), 0, st, vals, T,
                     order, inverse);
  return moe_host::launch_status();
}
