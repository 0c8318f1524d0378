// Route: top-k expert selection and gate weights, one token per segment of lanes (the
// selection itself is route_token, shared with the gate kernel's fused epilogue). The kernel
// reads N*E*4 bytes (+ the bias) and writes N*k*8 bytes.
#include "route_token.h"

namespace moe {

// One token per segment of SEG lanes, 256 / SEG tokens per block.
template <int SEG, int PER, bool VEC>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int N, int E,
                                                    int k, int gate, int32_t* __restrict__ idx,
                                                    float* __restrict__ w) {
  const int sl = threadIdx.x & (SEG - 1);
  const int t = blockIdx.x * (256 / SEG) + threadIdx.x / SEG;
  if (t >= N) return;  // the whole segment of a token leaves together
  route_token<SEG, PER, VEC>(logits + static_cast<size_t>(t) * E, bias, E, k, gate, sl, t, idx,
                             w);
}

template <int SEG, int PER, bool VEC>
static void launch_route(const float* logits, const float* bias, int N, int E, int k, int gate,
                         int32_t* idx, float* w, hipStream_t s) {
  const int tpb = 256 / SEG;
  const int blocks = (N + tpb - 1) / tpb;
  hipLaunchKernelGGL((route_kernel<SEG, PER, VEC>), dim3(blocks), dim3(256), 0, s, logits, bias,
                     N, E, k, gate, idx, w);
}

}  // namespace moe

extern "C" moe_status moe_route(const float* logits, const float* bias, int N, int E, int k,
                                int gate, int32_t* topk_idx, float* topk_w, void* stream) {
  using namespace moe;
  if (N < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > E || k > MOE_MAX_TOPK ||
      (gate != MOE_GATE_SOFTMAX && gate != MOE_GATE_SIGMOID)) {
    moe_host::set_error("moe_route: invalid N, E, k or gate");
    return MOE_EINVAL;
  }
  if (N == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w) {
    moe_host::set_error("moe_route: NULL pointer");
    return MOE_EINVAL;
  }
  hipStream_t s = moe_host::as_stream(stream);
  route_shape(E, [&](auto seg, auto per, auto vec) {
    launch_route<decltype(seg)::value, decltype(per)::value, decltype(vec)::value>(
        logits, bias, N, E, k, gate, topk_idx, topk_w, s);
  });
  return moe_host::launch_status();
}
