// Top-k route of one token by a segment of SEG lanes: the body shared by moe_route's kernel and
// the gate kernel's fused epilogue, so both give bit-identical selections and weights on the
// same logits.
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
// reads whole logit rows with coalesced loads. A segment never spans more than one 16-lane row,
// so its reductions are DPP lane moves inside the row (quad permutes, half-row and row mirrors)
// rather than LDS permutes.
#pragma once

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

// Route token t from its E logits at `row` (global or LDS memory); sl is the lane's index in
// the token's segment. Every lane of the segment calls it together.
template <int SEG, int PER>
__device__ __forceinline__ void route_token(const float* row, const float* __restrict__ bias,
                                            int E, int k, int gate, int sl, size_t t,
                                            int32_t* __restrict__ idx, float* __restrict__ w) {
  static_assert(SEG >= 1 && SEG <= 16 && (SEG & (SEG - 1)) == 0, "segments inside one row");
  // picks kept per lane, at most: k <= E <= SEG PER and k <= MOE_MAX_TOPK
  constexpr int KP = PER < (MOE_MAX_TOPK + SEG - 1) / SEG ? PER : (MOE_MAX_TOPK + SEG - 1) / SEG;
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
      idx[t * k + j] = my_e[q];
      w[t * k + j] = wv;
    }
  }
}

// The route layout (SEG lanes, PER logits per lane) for E experts: f(SEG, PER) as integral
// constants. moe_route and the gate's fused epilogue use this one table.
template <typename F>
inline void route_shape(int E, F&& f) {
  using std::integral_constant;
  if (E <= 1)        f(integral_constant<int, 1>{}, integral_constant<int, 1>{});
  else if (E <= 2)   f(integral_constant<int, 2>{}, integral_constant<int, 1>{});
  else if (E <= 4)   f(integral_constant<int, 4>{}, integral_constant<int, 1>{});
  else if (E <= 8)   f(integral_constant<int, 8>{}, integral_constant<int, 1>{});
  else if (E <= 16)  f(integral_constant<int, 16>{}, integral_constant<int, 1>{});
  else if (E <= 32)  f(integral_constant<int, 16>{}, integral_constant<int, 2>{});
  else if (E <= 64)  f(integral_constant<int, 16>{}, integral_constant<int, 4>{});
  else if (E <= 128) f(integral_constant<int, 16>{}, integral_constant<int, 8>{});
  else if (E <= 256) f(integral_constant<int, 16>{}, integral_constant<int, 16>{});
  else               f(integral_constant<int, 16>{}, integral_constant<int, 32>{});
}

}  // namespace moe
