// Top-k route of one token by a segment of SEG lanes: the body shared by moe_route's kernel and
// the gate kernel's fused epilogue, so both give bit-identical selections and weights on the
// same logits.
//
// FarSkip-Collective section 2.1 (the gate is a linear layer followed by a sparse selection) and
// Expert Coupling in MoE Pretraining Appendix A-A1 Table II (softmax over all experts, then
// top-k). The k largest biased logits are found by k rounds over the token's segment of lanes
// (the segment's largest value, then the lowest expert holding it), on integer keys that order
// exactly as the floats do; equal values resolve to the lower expert index. Pick j is kept
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

#include "count_rows.h"
#include "moe_internal.h"

namespace moe {

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

// Order-preserving map of a float to a signed int: x < y exactly when key(x) < key(y), and
// -0 and +0 share the key of +0 (they compare equal as floats). NaN is outside the contract.
__device__ __forceinline__ int route_key(float x) {
  int b = __float_as_int(x);
  if (b == static_cast<int>(0x80000000u)) b = 0;
  return b >= 0 ? b : b ^ 0x7fffffff;
}
__device__ __forceinline__ float route_unkey(int k) {
  return __int_as_float(k >= 0 ? k : k ^ 0x7fffffff);
}
constexpr int kRouteNone = static_cast<int>(0x80000000u);   // below every key (-inf included)

// Segment all-reduces (every lane of the segment ends with the result).
template <int SEG, bool MAX>
__device__ __forceinline__ int seg_reduce(int v) {
  auto step = [&](auto ctrl) {
    constexpr int kCtrl = decltype(ctrl)::value;
    const int o = __builtin_amdgcn_mov_dpp(v, kCtrl, 0xF, 0xF, false);
    v = MAX ? max(v, o) : min(v, o);
  };
  if constexpr (SEG >= 2) step(std::integral_constant<int, 0xB1>{});   // quad lanes xor 1
  if constexpr (SEG >= 4) step(std::integral_constant<int, 0x4E>{});   // quad lanes xor 2
  if constexpr (SEG >= 8) step(std::integral_constant<int, 0x141>{});  // half-row mirror
  if constexpr (SEG >= 16) step(std::integral_constant<int, 0x140>{});  // row mirror
  return v;
}

// Register layout of a token's logits: register i of segment lane sl holds expert
// e0(sl) + off(i). VEC (E a multiple of 4, PER a multiple of 4; 16-byte loads):
// e = 4 (sl + SEG (i / 4)) + i % 4; otherwise e = sl + SEG i. Either way e grows with i.
template <int SEG, int PER, bool VEC>
struct RouteLayout {
  __device__ static int e0(int sl) { return VEC ? 4 * sl : sl; }
  __device__ static constexpr int off(int i) { return VEC ? 4 * SEG * (i / 4) + (i & 3) : SEG * i; }
};

// The token's biased logits, as keys, into the lane's PER registers (kRouteNone past E). Every
// load is issued unconditionally at a clamped, in-bounds address (entries past E are masked),
// so the loads of a lane go out back to back.
template <int SEG, int PER, bool VEC>
__device__ __forceinline__ void route_load(const float* row, const float* __restrict__ bias,
                                           int E, int sl, int (&key)[PER]) {
  using LY = RouteLayout<SEG, PER, VEC>;
  const int e0 = LY::e0(sl);
  float x[PER], b[PER];
  if constexpr (VEC) {
#pragma unroll
    for (int i4 = 0; i4 < PER / 4; ++i4) {
      const float4 q = *reinterpret_cast<const float4*>(row + min(e0 + LY::off(4 * i4), E - 4));
      x[4 * i4] = q.x;
      x[4 * i4 + 1] = q.y;
      x[4 * i4 + 2] = q.z;
      x[4 * i4 + 3] = q.w;
    }
    if (bias) {
#pragma unroll
      for (int i4 = 0; i4 < PER / 4; ++i4) {
        const float4 q =
            *reinterpret_cast<const float4*>(bias + min(e0 + LY::off(4 * i4), E - 4));
        b[4 * i4] = q.x;
        b[4 * i4 + 1] = q.y;
        b[4 * i4 + 2] = q.z;
        b[4 * i4 + 3] = q.w;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) x[i] = row[min(e0 + LY::off(i), E - 1)];
    if (bias) {
#pragma unroll
      for (int i = 0; i < PER; ++i) b[i] = bias[min(e0 + LY::off(i), E - 1)];
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i)
    key[i] = e0 + LY::off(i) < E ? route_key(bias ? x[i] + b[i] : x[i]) : kRouteNone;
}

// Top-k of one token whose biased logits the segment holds as keys (consumed). Each round: the
// largest key of the segment (a max tree over the lane's registers, then the segment's max),
// then the lowest expert holding exactly that key (a min tree, then the segment's min), which
// is removed. The same picks as an argmax over the logits with equal values resolved to the
// lower expert id; the pick's value is the logit itself (the key maps back exactly). With
// rc.emask set, each pick also sets token tl's bits in the block's count masks.
template <int SEG, int PER, bool VEC>
__device__ __forceinline__ void route_select(int (&key)[PER], int E, int k, int gate, int sl,
                                             size_t t, int32_t* __restrict__ idx,
                                             float* __restrict__ w, const RouteCount& rc,
                                             int tl) {
  static_assert(SEG >= 1 && SEG <= 16 && (SEG & (SEG - 1)) == 0, "segments inside one row");
  using LY = RouteLayout<SEG, PER, VEC>;
  const int e0 = LY::e0(sl);
  // picks kept per lane, at most: k <= E <= SEG PER and k <= MOE_MAX_TOPK
  constexpr int KP = PER < (MOE_MAX_TOPK + SEG - 1) / SEG ? PER : (MOE_MAX_TOPK + SEG - 1) / SEG;
  constexpr int kFar = 0x7fffffff;
  float top = 0.f;
  float my_v[KP];
  int my_e[KP];
#pragma unroll
  for (int q = 0; q < KP; ++q) {
    my_v[q] = -INFINITY;
    my_e[q] = 0;
  }
  for (int j = 0; j < k; ++j) {
    // the lane's largest key: a tree of 3-input maxima
    int m[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) m[i] = key[i];
#pragma unroll
    for (int lvl = 0, span = 1; lvl < 4; ++lvl, span *= 3)
#pragma unroll
      for (int i = 0; i < PER; i += 3) {
        const int a = i * span, b = a + span, c = b + span;
        if (c < PER) m[a] = max(max(m[a], m[b]), m[c]);
        else if (b < PER) m[a] = max(m[a], m[b]);
      }
    const int bk = seg_reduce<SEG, true>(m[0]);
    // the lowest register of this lane holding bk (offsets grow with the register), then the
    // lowest expert of the segment
#pragma unroll
    for (int i = 0; i < PER; ++i) m[i] = key[i] == bk ? LY::off(i) : kFar;
#pragma unroll
    for (int lvl = 0, span = 1; lvl < 4; ++lvl, span *= 3)
#pragma unroll
      for (int i = 0; i < PER; i += 3) {
        const int a = i * span, b = a + span, c = b + span;
        if (c < PER) m[a] = min(min(m[a], m[b]), m[c]);
        else if (b < PER) m[a] = min(m[a], m[b]);
      }
    const int be = seg_reduce<SEG, false>(m[0] == kFar ? kFar : e0 + m[0]);
    const float bv = route_unkey(bk);
    if (j == 0) top = bv;
    if (sl == j % SEG) {
#pragma unroll
      for (int q = 0; q < KP; ++q)
        if (q == j / SEG) {
          my_v[q] = bv;
          my_e[q] = be;
        }
    }
    const int d = be - e0;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (d == LY::off(i)) key[i] = kRouteNone;
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
      if (rc.emask) count_pick(rc, E, tl, my_e[q]);
    }
  }
}

// Route token t from its E logits at `row` (global or LDS memory); sl is the lane's index in
// the token's segment, tl the token's index in the block (its bit in the count masks). Every
// lane of the segment calls it together.
template <int SEG, int PER, bool VEC>
__device__ __forceinline__ void route_token(const float* row, const float* __restrict__ bias,
                                            int E, int k, int gate, int sl, size_t t,
                                            int32_t* __restrict__ idx, float* __restrict__ w,
                                            const RouteCount& rc, int tl) {
  int key[PER];
  route_load<SEG, PER, VEC>(row, bias, E, sl, key);
  route_select<SEG, PER, VEC>(key, E, k, gate, sl, t, idx, w, rc, tl);
}

// The route layout (SEG lanes, PER logits per lane, 16-byte loads or not) for E experts:
// f(SEG, PER, VEC) as integral constants. moe_route and the gate's fused epilogue use this one
// table; SEG is route_seg(E), which fixes the tokens per count row.
template <typename F>
__host__ __device__ inline void route_shape(int E, F&& f) {
  using std::integral_constant;
  auto g = [&](auto seg, auto per) __attribute__((always_inline)) {
    constexpr int PER = decltype(per)::value;
    if (PER % 4 == 0 && E % 4 == 0) f(seg, per, std::true_type{});
    else f(seg, per, std::false_type{});
  };
  if (E <= 1)        g(integral_constant<int, 1>{}, integral_constant<int, 1>{});
  else if (E <= 2)   g(integral_constant<int, 2>{}, integral_constant<int, 1>{});
  else if (E <= 4)   g(integral_constant<int, 4>{}, integral_constant<int, 1>{});
  else if (E <= 8)   g(integral_constant<int, 8>{}, integral_constant<int, 1>{});
  else if (E <= 16)  g(integral_constant<int, 16>{}, integral_constant<int, 1>{});
  else if (E <= 32)  g(integral_constant<int, 16>{}, integral_constant<int, 2>{});
  else if (E <= 64)  g(integral_constant<int, 16>{}, integral_constant<int, 4>{});
  else if (E <= 128) g(integral_constant<int, 16>{}, integral_constant<int, 8>{});
  else if (E <= 256) g(integral_constant<int, 16>{}, integral_constant<int, 16>{});
  else               g(integral_constant<int, 16>{}, integral_constant<int, 32>{});
}

}  // namespace moe
