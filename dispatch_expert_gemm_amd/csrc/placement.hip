// Correlated expert placement (Expert Coupling in MoE Pretraining, section V-A "Correlated
// Placement" and Appendix A-D Algorithm 1): co-selection counts on the device, the balanced
// pairwise-swap partition on the host (a small E x E problem, run once per layer offline).
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "moe_internal.h"

namespace moe {

// One thread per (token, ordered slot pair): counts[e * E + e'] += 1 for e != e'. Integer atomics
// make the totals exact and independent of order.
__global__ __launch_bounds__(256) void zero_i32(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ __launch_bounds__(256) void coselect_kernel(const int32_t* __restrict__ topk_idx,
                                                       int N, int E, int k,
                                                       int32_t* __restrict__ counts) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= N) return;
  const int32_t* s = topk_idx + static_cast<size_t>(t) * k;
  for (int a = 0; a < k; ++a)
    for (int b = 0; b < k; ++b)
      if (a != b) atomicAdd(&counts[s[a] * E + s[b]], 1);
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_coselect_counts(const int32_t* topk_idx, int N, int E, int k,
                                          int32_t* counts, void* stream) {
  if (N < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > E || !counts || (N > 0 && !topk_idx)) {
    moe_host::set_error("moe_coselect_counts: invalid arguments");
    return MOE_EINVAL;
  }
  hipStream_t st = moe_host::as_stream(stream);
  hipLaunchKernelGGL(zero_i32, dim3((E * E + 255) / 256), dim3(256), 0, st, counts, E * E);
  if (N > 0)
    hipLaunchKernelGGL(coselect_kernel, dim3((N + 255) / 256), dim3(256), 0, st, topk_idx, N, E,
                       k, counts);
  return moe_host::launch_status();
}

extern "C" moe_status moe_placement_partition(const int64_t* counts, int E, int G, int i_max,
                                              int32_t* group, int* swaps) {
  if (!counts || !group || E < 1 || G < 1 || E % G) {
    moe_host::set_error("moe_placement_partition: invalid arguments");
    return MOE_EINVAL;
  }
  const int per = E / G;
  const long long limit = i_max > 0 ? i_max : static_cast<long long>(E) * E;
  std::vector<int> grp(E);
  for (int e = 0; e < E; ++e) grp[e] = e / per;
  // to_group[x * G + g]: weight from expert x to the experts of group g (W[x][x] = 0)
  std::vector<int64_t> to_group(static_cast<size_t>(E) * G, 0);
  for (int x = 0; x < E; ++x)
    for (int y = 0; y < E; ++y) to_group[static_cast<size_t>(x) * G + grp[y]] += counts[static_cast<size_t>(x) * E + y];
  int done = 0;
  for (long long it = 0; it < limit; ++it) {
    int64_t best = 0;
    int ba = -1, bb = -1;
    for (int a = 0; a < E; ++a) {
      const int ga = grp[a];
      const int64_t own_a = to_group[static_cast<size_t>(a) * G + ga];
      for (int b = a + 1; b < E; ++b) {
        const int gb = grp[b];
        if (ga == gb) continue;
        const int64_t gain = (to_group[static_cast<size_t>(a) * G + gb] - own_a) +
                             (to_group[static_cast<size_t>(b) * G + ga] -
                              to_group[static_cast<size_t>(b) * G + gb]) -
                             2 * counts[static_cast<size_t>(a) * E + b];
        if (gain > best) {  // strict: the first (smallest) (a, b) keeps equal gains
          best = gain;
          ba = a;
          bb = b;
        }
      }
    }
    if (ba < 0) break;
    const int ga = grp[ba], gb = grp[bb];
    for (int x = 0; x < E; ++x) {
      to_group[static_cast<size_t>(x) * G + ga] += counts[static_cast<size_t>(x) * E + bb] - counts[static_cast<size_t>(x) * E + ba];
      to_group[static_cast<size_t>(x) * G + gb] += counts[static_cast<size_t>(x) * E + ba] - counts[static_cast<size_t>(x) * E + bb];
    }
    grp[ba] = gb;
    grp[bb] = ga;
    ++done;
  }
  for (int e = 0; e < E; ++e) group[e] = grp[e];
  if (swaps) *swaps = done;
  return MOE_OK;
}
