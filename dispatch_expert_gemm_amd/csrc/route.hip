// Route: top-k expert selection and gate weights, one token per segment of lanes.
//
// FarSkip-Collective section 2.1 (the gate is a linear layer followed by a sparse selection) and
// Expert Coupling in MoE Pretraining Appendix A-A1 Table II (softmax over all experts, then
// top-k). The k largest biased logits are found by k rounds of an (value, index) argmax over
// the token's segment of lanes; equal values resolve to the lower expert index. Pick j is kept
// by lane j % SEG of the segment (slot j / SEG), so the softmax over the selection is one
// segment reduction.
//
// Layout: SEG lanes (1, 2, 4, 8 or 16) per token, PER logits per lane, E <= SEG * PER. Logit e
// of the token sits in lane e % SEG, register e / SEG, or, when E and PER are multiples of 4,
// in lane (e / 4) % SEG, register 4 (e / (4 SEG)) + e % 4, loaded 16 bytes at a time: a wave
// reads whole logit rows with coalesced loads. A segment never spans more than one 16-lane row, so its
// reductions are DPP lane moves inside the row (quad permutes, half-row and row mirrors) rather
// than LDS permutes. The kernel reads N*E*4 bytes and writes N*k*8 bytes.
#include <math.h>

#include <type_traits>

#include "moe_internal.h"

namespace moe {

// All-reduce of (value, index) over the SEG lanes of a segment: the larger value wins, equal
// values the lower index. Every lane of the segment ends with the result.
template <int SEG>
__device__ __forceinline__ void seg_argmax(float& v, int& e) {
  auto step = [&](auto ctrl) {
    constexpr int kCtrl = decltype(ctrl)::value;
    const float ov = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                                   __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF,
                                                   false));
    const int oe = __builtin_amdgcn_mov_dpp(e, kCtrl, 0xF, 0xF, false);
    if (ov > v || (ov == v && oe < e)) {
      v = ov;
      e = oe;
    }
  };
  if constexpr (SEG >= 2) step(std::integral_constant<int, 0xB1>{});   // quad lanes xor 1
  if constexpr (SEG >= 4) step(std::integral_constant<int, 0x4E>{});   // quad lanes xor 2
  if constexpr (SEG >= 8) step(std::integral_constant<int, 0x141>{});  // half-row mirror
  if constexpr (SEG >= 16) step(std::integral_constant<int, 0x140>{});  // row mirror
}

template <int SEG>
__device__ __forceinline__ float seg_sum(float s) {
  auto step = [&](auto ctrl) {
    constexpr int kCtrl = decltype(ctrl)::value;
    s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), kCtrl,
                                                             0xF, 0xF, false));
  };
  if constexpr (SEG >= 2) step(std::integral_constant<int, 0xB1>{});
  if constexpr (SEG >= 4) step(std::integral_constant<int, 0x4E>{});
  if constexpr (SEG >= 8) step(std::integral_constant<int, 0x141>{});
  if constexpr (SEG >= 16) step(std::integral_constant<int, 0x140>{});
  return s;
}

template <int SEG, int PER>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int N, int E,
                                                    int k, int gate, int32_t* __restrict__ idx,
                                                    float* __restrict__ w) {
  static_assert(SEG >= 1 && SEG <= 16 && (SEG & (SEG - 1)) == 0, "segments inside one row");
  // picks kept per lane, at most: k <= E <= SEG PER and k <= MOE_MAX_TOPK
  constexpr int KP = PER < (MOE_MAX_TOPK + SEG - 1) / SEG ? PER : (MOE_MAX_TOPK + SEG - 1) / SEG;
  const int sl = threadIdx.x & (SEG - 1);
  const int t = blockIdx.x * (256 / SEG) + threadIdx.x / SEG;
  if (t >= N) return;  // the whole segment of a token leaves together

  const float* row = logits + static_cast<size_t>(t) * E;
  // expert of register i: e = sl + i SEG, or with 16-byte loads (VEC: E a multiple of 4, PER a
  // multiple of 4) e = 4 (sl + SEG (i / 4)) + i % 4. Either way e grows with i for a lane.
  const bool vec = PER % 4 == 0 && E % 4 == 0;
  auto expert = [&](int i) { return vec ? 4 * (sl + SEG * (i / 4)) + (i & 3) : sl + i * SEG; };
  float v[PER];
  if (vec) {
#pragma unroll
    for (int i4 = 0; i4 < (PER >= 4 ? PER / 4 : 1); ++i4) {
      const int e = 4 * (sl + SEG * i4);
      float4 x = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      if (e < E) {
        x = *reinterpret_cast<const float4*>(row + e);
        if (bias) {
          x.x += bias[e];
          x.y += bias[e + 1];
          x.z += bias[e + 2];
          x.w += bias[e + 3];
        }
      }
      if (4 * i4 + 3 < PER) {
        v[4 * i4] = x.x;
        v[4 * i4 + 1] = x.y;
        v[4 * i4 + 2] = x.z;
        v[4 * i4 + 3] = x.w;
      }
    }
  } else {
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
  }

  float top = 0.f;
  float my_v[KP];
  int my_e[KP];
#pragma unroll
  for (int q = 0; q < KP; ++q) {
    my_v[q] = -INFINITY;
    my_e[q] = 0;
  }
  for (int j = 0; j < k; ++j) {
    // lane-local best; increasing e with a strict '>' keeps the lower index on ties
    float bv = v[0];
    int be = expert(0);
#pragma unroll
    for (int i = 1; i < PER; ++i) {
      if (v[i] > bv) {
        bv = v[i];
        be = expert(i);
      }
    }
    // padded entries (e >= E) never win: they are -inf with indices above every real expert
    if (be >= E) be = 0x7fffffff;
    seg_argmax<SEG>(bv, be);
    if (j == 0) top = bv;
    if (sl == j % SEG) {
#pragma unroll
      for (int q = 0; q < KP; ++q)
        if (q == j / SEG) {
          my_v[q] = bv;
          my_e[q] = be;
        }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (expert(i) == be) v[i] = -INFINITY;
  }

  // picks of this lane: j = sl + q SEG for j < k
  float z[KP];
  float part = 0.f;
#pragma unroll
  for (int q = 0; q < KP; ++q) {
    const bool mine = sl + q * SEG < k;
    z[q] = mine && gate == MOE_GATE_SOFTMAX ? __expf(my_v[q] - top) : 0.f;
    part += z[q];
  }
  const float sum = gate == MOE_GATE_SOFTMAX ? seg_sum<SEG>(part) : 1.f;
#pragma unroll
  for (int q = 0; q < KP; ++q) {
    const int j = sl + q * SEG;
    if (j < k) {
      const float wv = gate == MOE_GATE_SOFTMAX ? z[q] / sum : 1.f / (1.f + __expf(-my_v[q]));
      idx[static_cast<size_t>(t) * k + j] = my_e[q];
      w[static_cast<size_t>(t) * k + j] = wv;
    }
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
  else if (E <= 32)  launch_route<16, 2>(logits, bias, N, E, k, gate, topk_idx, topk_w, s);
  else if (E <= 64)  launch_route<16, 4>(logits, bias, N, E, k, gate, topk_idx, topk_w, s);
  else if (E <= 128) launch_route<16, 8>(logits, bias, N, E, k, gate, topk_idx, topk_w, s);
  else if (E <= 256) launch_route<16, 16>(logits, bias, N, E, k, gate, topk_idx, topk_w, s);
  else               launch_route<16, 32>(logits, bias, N, E, k, gate, topk_idx, topk_w, s);
  return moe_host::launch_status();
}
