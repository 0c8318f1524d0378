// Route: top-k expert selection and gate weights, one token per lane segment.
//
// FarSkip-Collective section 2.1 (the gate is a linear layer followed by a sparse selection) and
// Expert Coupling in MoE Pretraining Appendix A-A1 Table II (softmax over all experts, then
// top-k). The k largest biased logits are found by k rounds of an (value, index) argmax over
// the token's segment of lanes; equal values resolve to the lower expert index. Lane j of the
// segment keeps the j-th pick, so the softmax over the selection is one segment reduction.
//
// Layout: SEG lanes (a power of two <= 64) per token, PER logits per lane, E <= SEG * PER.
// Logit e of the token sits in lane e % SEG, register e / SEG: a wave reads whole logit rows
// with unit-stride, coalesced loads. The kernel reads N*E*4 bytes and writes N*k*8 bytes.
#include <math.h>

#include "moe_internal.h"

namespace moe {

template <int SEG, int PER>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int N, int E,
                                                    int k, int gate, int32_t* __restrict__ idx,
                                                    float* __restrict__ w) {
  const int sl = threadIdx.x & (SEG - 1);
  const int t = blockIdx.x * (256 / SEG) + threadIdx.x / SEG;
  if (t >= N) return;  // the whole segment of a token leaves together

  const float* row = logits + static_cast<size_t>(t) * E;
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = sl + i * SEG;
    float x = -INFINITY;
    if (e < E) {
      x = row[e];
      if (bias) x = x + bias[e];
    }
    v[i] = x;
  }

  float top = 0.f, my_v = -INFINITY;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    // lane-local best; increasing e with a strict '>' keeps the lower index on ties
    float bv = v[0];
    int be = sl;
#pragma unroll
    for (int i = 1; i < PER; ++i) {
      if (v[i] > bv) {
        bv = v[i];
        be = sl + i * SEG;
      }
    }
    // padded entries (e >= E) never win: they are -inf with indices above every real expert
    if (be >= E) be = 0x7fffffff;
#pragma unroll
    for (int off = SEG / 2; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, SEG);
      const int oe = __shfl_xor(be, off, SEG);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if (j == 0) top = bv;
    if (sl == j) {
      my_v = bv;
      my_e = be;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (sl + i * SEG == be) v[i] = -INFINITY;
  }

  float wv;
  if (gate == MOE_GATE_SOFTMAX) {
    const float z = sl < k ? __expf(my_v - top) : 0.f;
    float s = z;
#pragma unroll
    for (int off = SEG / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, SEG);
    wv = z / s;
  } else {
    wv = 1.f / (1.f + __expf(-my_v));
  }
  if (sl < k) {
    idx[static_cast<size_t>(t) * k + sl] = my_e;
    w[static_cast<size_t>(t) * k + sl] = wv;
  }
}

template <int SEG, int PER>
static void launch_route(const float* logits, const float* bias, int N, int E, int k, int gate,
                         int32_t* idx, float* w, hipStream_t s) {
  const int tpb = 256 / SEG;
  const int blocks = (N + tpb - 1) / tpb;
  hipLaunchKernelGGL((route_kernel<SEG, PER>), dim3(blocks), dim3(256), 0, s, logits, bias, N,
                     E, k, gate, idx, w);
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
  if (E <= 1)        launch_route<1, 1>(logits, bias, N, E, k, gate, topk_idx, topk_w, s);
  else if (E <= 2)   launch_route<2, 1>(logits, bias, N, E, k, gate, topk_idx, topk_w, s);
  else if (E <= 4)   launch_route<4, 1>(logits, bias, N, E, k, gate, topk_idx, topk_w, s);
  else if (E <= 8)   launch_route<8, 1>(logits, bias, N, E, k, gate, topk_idx, topk_w, s);
  else if (E <= 16)  launch_route<16, 1>(logits, bias, N, E, k, gate, topk_idx, topk_w, s);
  else if (E <= 32)  launch_route<32, 1>(logits, bias, N, E, k, gate, topk_idx, topk_w, s);
  else if (E <= 64)  launch_route<64, 1>(logits, bias, N, E, k, gate, topk_idx, topk_w, s);
  else if (E <= 128) launch_route<64, 2>(logits, bias, N, E, k, gate, topk_idx, topk_w, s);
  else if (E <= 256) launch_route<64, 4>(logits, bias, N, E, k, gate, topk_idx, topk_w, s);
  else               launch_route<64, 8>(logits, bias, N, E, k, gate, topk_idx, topk_w, s);
  return moe_host::launch_status();
}
