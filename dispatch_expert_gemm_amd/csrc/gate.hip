// Gate: router logits l = x W_R^T on the matrix cores, then the top-k route.
//
// FarSkip-Collective section 2.1: the gate G(A) = s(A W_R^T) is a linear classification layer
// followed by the sparse selection s(). Expert Coupling in MoE Pretraining Appendix A-A1
// Table II: the router is an FP32 linear layer. The router weights stay fp32: each K step splits
// them into a bf16 high part and a bf16 remainder (w = hi + lo up to 2^-17 |w|), and the
// logits accumulate x hi + x lo with v_mfma_f32_32x32x16_bf16 in fp32. bf16 x is exact in that
// form; fp32 x is split the same way and x_lo hi is added (x_lo lo, below 2^-16 relative, is
// dropped).
//
// Tile: 64 tokens x all experts (E padded to a multiple of 32, at most 256) per workgroup of 4
// waves; wave w owns token block w % 2 and expert blocks w / 2, w / 2 + 2, ... K steps of 32 go
// through registers into a double-buffered LDS tile (64-byte rows, chunk c of row r at slot
// c ^ ((r / 4) % 4), conflict free for the fragment reads), one barrier per step.
#include "moe_internal.h"

namespace moe {

constexpr int kGT = 64;     // tokens per workgroup
constexpr int kGK = 32;     // K per step
constexpr int kGRow = 64;   // LDS bytes per row (32 bf16)

__device__ __forceinline__ int gate_swz(int r) { return (r >> 2) & 3; }

// Splits 8 floats into bf16 hi (round to nearest even) and the bf16 of the remainder.
__device__ __forceinline__ void split8(const f32x4& a, const f32x4& b, u32x4& hi, u32x4& lo) {
  float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  uint32_t h[4], o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const __bf16 h0 = static_cast<__bf16>(v[2 * i]), h1 = static_cast<__bf16>(v[2 * i + 1]);
    const __bf16 l0 = static_cast<__bf16>(v[2 * i] - static_cast<float>(h0));
    const __bf16 l1 = static_cast<__bf16>(v[2 * i + 1] - static_cast<float>(h1));
    const bf16x2 hh = {h0, h1}, ll = {l0, l1};
    h[i] = __builtin_bit_cast(uint32_t, hh);
    o[i] = __builtin_bit_cast(uint32_t, ll);
  }
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{o[0], o[1], o[2], o[3]};
}

// EB: expert blocks of 32 (E <= 32 EB); XF32: x is fp32 (else bf16).
template <int EB, bool XF32>
__global__ __launch_bounds__(256) void gate_kernel(const void* __restrict__ xv,
                                                   const float* __restrict__ w, int N, int H,
                                                   int E, float* __restrict__ logits) {
  constexpr int ER = EB * 32;                      // padded expert rows
  constexpr int WCH = ER * 4;                      // 16-byte chunks of a W step
  constexpr int WPT = (WCH + 255) / 256;           // W chunks per thread
  constexpr int NBW = EB >= 2 ? EB / 2 : 1;        // expert blocks per wave
  __shared__ __attribute__((aligned(16))) char xs_hi[2][kGT * kGRow];
  __shared__ __attribute__((aligned(16))) char xs_lo[XF32 ? 2 : 1][XF32 ? kGT * kGRow : 16];
  __shared__ __attribute__((aligned(16))) char ws_hi[2][ER * kGRow];
  __shared__ __attribute__((aligned(16))) char ws_lo[2][ER * kGRow];

  const int tid = threadIdx.x, l = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * kGT;
  const int KT = H / kGK;

  // staging registers of one K step
  u32x4 rwh[WPT], rwl[WPT], rxh, rxl;
  // x chunk of this thread: row tid / 4, chunk tid % 4
  const int xr = tid >> 2, xc = tid & 3;
  const bool x_ok = t0 + xr < N;
  auto load = [&](int kt) {
    const int k0 = kt * kGK;
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int c = tid + i * 256;
      if (c < WCH) {
        const int r = c >> 2, ch = c & 3;
        if (r < E) {
          const f32x4* src =
              reinterpret_cast<const f32x4*>(w + static_cast<size_t>(r) * H + k0 + ch * 8);
          split8(src[0], src[1], rwh[i], rwl[i]);
        } else {
          rwh[i] = rwl[i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
    if (!x_ok) {
      rxh = rxl = u32x4{0u, 0u, 0u, 0u};
    } else if (XF32) {
      const f32x4* src = reinterpret_cast<const f32x4*>(
          static_cast<const float*>(xv) + static_cast<size_t>(t0 + xr) * H + k0 + xc * 8);
      split8(src[0], src[1], rxh, rxl);
    } else {
      rxh = *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(xv) +
                                            static_cast<size_t>(t0 + xr) * H + k0 + xc * 8);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int c = tid + i * 256;
      if (c < WCH) {
        const int r = c >> 2, ch = c & 3;
        const int off = r * kGRow + ((ch ^ gate_swz(r)) << 4);
        *reinterpret_cast<u32x4*>(&ws_hi[buf][off]) = rwh[i];
        *reinterpret_cast<u32x4*>(&ws_lo[buf][off]) = rwl[i];
      }
    }
    const int off = xr * kGRow + ((xc ^ gate_swz(xr)) << 4);
    *reinterpret_cast<u32x4*>(&xs_hi[buf][off]) = rxh;
    if (XF32) *reinterpret_cast<u32x4*>(&xs_lo[buf][off]) = rxl;
  };

  const int tb = wv & 1;                  // token block of this wave
  const int eb0 = wv >> 1;                // first expert block; then +2, +4, ...
  const bool active = eb0 < EB;
  f32x16 acc[NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[i][q] = 0.f;

  const int frow = l & 31;
  const int fsw = gate_swz(frow);   // rows are 32-aligned: swz of the block row = swz(l % 32)
  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int slot = ((ks * 2 + (l >> 5)) ^ fsw) << 4;
      const int xo = (tb * 32 + frow) * kGRow + slot;
      const bf16x8 ah = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&xs_hi[buf][xo]));
      bf16x8 al;
      if (XF32) al = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&xs_lo[buf][xo]));
#pragma unroll
      for (int i = 0; i < NBW; ++i) {
        const int wo = ((eb0 + 2 * i) * 32 + frow) * kGRow + slot;
        const bf16x8 bh =
            __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&ws_hi[buf][wo]));
        const bf16x8 bl =
            __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&ws_lo[buf][wo]));
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc[i], 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc[i], 0, 0, 0);
        if (XF32) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc[i], 0, 0, 0);
      }
    }
  };

  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) load(kt + 1);
    if (active) compute(kt & 1);
    if (kt + 1 < KT) store((kt + 1) & 1);
    __syncthreads();
  }

  // lane l holds expert column l % 32 of its block and, for q = 0..15, token row
  // 8 (q / 4) + 4 (l / 32) + q % 4
  if (!active) return;
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int e = (eb0 + 2 * i) * 32 + (l & 31);
    if (e >= E) continue;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int t = t0 + tb * 32 + (q >> 2) * 8 + (l >> 5) * 4 + (q & 3);
      if (t < N) logits[static_cast<size_t>(t) * E + e] = acc[i][q];
    }
  }
}

template <int EB>
static void launch_gate(const void* x, bool xf32, const float* w, int N, int H, int E,
                        float* logits, hipStream_t s) {
  const dim3 grid((N + kGT - 1) / kGT), block(256);
  if (xf32)
    hipLaunchKernelGGL((gate_kernel<EB, true>), grid, block, 0, s, x, w, N, H, E, logits);
  else
    hipLaunchKernelGGL((gate_kernel<EB, false>), grid, block, 0, s, x, w, N, H, E, logits);
}

}  // namespace moe

extern "C" moe_status moe_gate_route(const void* x, int dtype, const float* w_router,
                                     const float* bias, int N, int H, int E, int k, int gate,
                                     float* logits, int32_t* topk_idx, float* topk_w,
                                     void* stream) {
  using namespace moe;
  if (N < 0 || H <= 0 || H % kGK != 0 || E < 1 || E > 256 || k < 1 || k > E ||
      k > MOE_MAX_TOPK || (dtype != MOE_F32 && dtype != MOE_BF16) ||
      (gate != MOE_GATE_SOFTMAX && gate != MOE_GATE_SIGMOID)) {
    moe_host::set_error("moe_gate_route: invalid shape (H a multiple of 32, E <= 256, k <= E), "
                        "dtype or gate");
    return MOE_EINVAL;
  }
  if (N == 0) return MOE_OK;
  if (!x || !w_router || !logits || !topk_idx || !topk_w) {
    moe_host::set_error("moe_gate_route: NULL pointer");
    return MOE_EINVAL;
  }
  hipStream_t s = moe_host::as_stream(stream);
  const bool xf32 = dtype == MOE_F32;
  if (E <= 32)       launch_gate<1>(x, xf32, w_router, N, H, E, logits, s);
  else if (E <= 64)  launch_gate<2>(x, xf32, w_router, N, H, E, logits, s);
  else if (E <= 128) launch_gate<4>(x, xf32, w_router, N, H, E, logits, s);
  else               launch_gate<8>(x, xf32, w_router, N, H, E, logits, s);
  const moe_status st = moe_host::launch_status();
  if (st != MOE_OK) return st;
  return moe_route(logits, bias, N, E, k, gate, topk_idx, topk_w, stream);
}
