// Route: top-k expert selection and gate weights, one token per segment of lanes (the
// selection itself is route_token, shared with the gate kernel's fused epilogue). The kernel
// reads N*E*4 bytes (+ the bias) and writes N*k*8 bytes. Given a layout workspace, each block
// also writes the count rows of its tokens (expert and pair counts per slice of T tokens), so
// moe_dispatch_layout can skip its own count kernel.
#include "route_token.h"

namespace moe {

// One token per segment of SEG lanes, B = 256 / SEG tokens per block (whole count rows).
template <int SEG, int PER, bool VEC>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int N, int E,
                                                    int k, int gate, int32_t* __restrict__ idx,
                                                    float* __restrict__ w,
                                                    const int32_t* __restrict__ placement, int W,
                                                    CountWs cw) {
  constexpr int B = 256 / SEG;
  constexpr int T = B < 64 ? B : 64;
  constexpr int G = (B + 63) / 64;   // 64-token mask groups per block
  extern __shared__ unsigned long long masks[];   // [G][E] then [G][W] when counting
  const bool count = cw.e != nullptr;
  const int sl = threadIdx.x & (SEG - 1);
  const int tl = threadIdx.x / SEG;
  const int t0 = blockIdx.x * B;
  const int t = t0 + tl;
  RouteCount rc{};
  if (count) {
    rc = RouteCount{masks, masks + G * E, placement, E / W, W};
    for (int i = threadIdx.x; i < G * (E + W); i += 256) masks[i] = 0ull;
    __syncthreads();
  }
  if (t < N)   // the whole segment of a token takes the same branch
    route_token<SEG, PER, VEC>(logits + static_cast<size_t>(t) * E, bias, E, k, gate, sl, t, idx,
                               w, rc, tl);
  if (count) {
    __syncthreads();
    write_count_rows(masks, masks + G * E, E, W, T, t0, min(B, N - t0), N, cw);
  }
}

template <int SEG, int PER, bool VEC>
static void launch_route(const float* logits, const float* bias, int N, int E, int k, int gate,
                         int32_t* idx, float* w, const int32_t* placement, int W, CountWs cw,
                         hipStream_t s) {
  constexpr int B = 256 / SEG;
  const int blocks = (N + B - 1) / B;
  const size_t lds = cw.e ? static_cast<size_t>((B + 63) / 64) * (E + W) * 8 : 0;
  hipLaunchKernelGGL((route_kernel<SEG, PER, VEC>), dim3(blocks), dim3(256), lds, s, logits, bias,
                     N, E, k, gate, idx, w, placement, W, cw);
}

}  // namespace moe

namespace moe_host {
// Checks of the optional count outputs shared by moe_route and moe_gate_route.
bool route_counts_ok(int N, int E, int W, const void* layout_ws) {
  return !layout_ws || (W >= 1 && W <= MOE_MAX_RANKS && E % W == 0 && N % W == 0);
}
}  // namespace moe_host

extern "C" moe_status moe_route(const float* logits, const float* bias, int N, int E, int k,
                                int gate, int32_t* topk_idx, float* topk_w,
                                const int32_t* expert_rank, int W, void* layout_workspace,
                                void* stream) {
  using namespace moe;
  if (N < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > E || k > MOE_MAX_TOPK ||
      (gate != MOE_GATE_SOFTMAX && gate != MOE_GATE_SIGMOID)) {
    moe_host::set_error("moe_route: invalid N, E, k or gate");
    return MOE_EINVAL;
  }
  if (!moe_host::route_counts_ok(N, E, W, layout_workspace)) {
    moe_host::set_error("moe_route: with a layout workspace W must be in 1..64 and divide E and N");
    return MOE_EINVAL;
  }
  if (N == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w) {
    moe_host::set_error("moe_route: NULL pointer");
    return MOE_EINVAL;
  }
  hipStream_t s = moe_host::as_stream(stream);
  const CountWs cw = layout_workspace ? count_ws_carve(N, E, W, layout_workspace) : CountWs{};
  bool same_rows = true;
  route_shape(E, [&](auto seg, auto per, auto vec) {
    constexpr int SEG = decltype(seg)::value;
    // the block's count rows are the layout's: 256 / SEG tokens per block, T = route_seg(E)'s
    same_rows = SEG == route_seg(E);
    if (same_rows)
      launch_route<SEG, decltype(per)::value, decltype(vec)::value>(
          logits, bias, N, E, k, gate, topk_idx, topk_w, expert_rank, W, cw, s);
  });
  if (!same_rows) {
    moe_host::set_error("moe_route: internal: route segment differs from route_seg(E)");
    return MOE_EINVAL;
  }
  return moe_host::launch_status();
}
