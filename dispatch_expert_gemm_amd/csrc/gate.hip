// Gate: router logits l = x W_R^T on the matrix cores, then the top-k route.
//
// FarSkip-Collective section 2.1: the gate G(A) = s(A W_R^T) is a linear classification layer
// followed by the sparse selection s(). Expert Coupling in MoE Pretraining Appendix A-A1
// Table II: the router is an FP32 linear layer. The router weights stay fp32: a first pass splits
// them into a bf16 high part and a bf16 remainder (w = hi + lo up to 2^-17 |w|, stored
// interleaved per 32 K values: 64 bytes of hi then 64 of lo), and the logits accumulate
// x hi + x lo with v_mfma_f32_32x32x16_bf16 in fp32. bf16 x is exact in that form; fp32 x is
// split the same way when its fragments are read and x_lo hi is added (x_lo lo, below 2^-16
// relative, is dropped).
//
// Tile: 32 TB tokens x 32 EB experts per workgroup of 4 waves, or 8 where the copies split over
// eight (64 tokens x all experts, or 128 x 128 when many tokens meet many experts: the router
// weights are then read from L2 half as often); the (token block, expert block) pairs p = w,
// w + 4, ... go to wave w of each group of four, so a wave keeps one token block. K steps of 64
// (bf16 x, where the ring fits) or 32 go HBM -> LDS directly (global_load_lds_dwordx4) through a
// ring of 3-4 stages, so several steps of x and W_R are in flight while one is multiplied; the
// fp32 values are split into bf16 pairs when the fragments are read (fp32 x). Swizzled rows keep
// the fragment reads free of bank conflicts.
//
// Few experts (5-32): gate_small_kernel below, 32 tokens per workgroup with K steps of 64.
//
// When one workgroup holds all E logits of its tokens (64 tokens x up to 256 experts), the top-k
// route runs in the kernel's epilogue: the logits tile goes to LDS and each token's segment of
// lanes runs route_token on it, the same code as moe_route, so the selection equals moe_route on
// the written logits.
#include "route_token.h"

namespace moe {

constexpr int kGK = 32;     // K per step

// 16-byte chunk slot of row r: rows of 64 bytes use (r / 4) % 4, rows of 128 bytes (r / 2) % 8,
// rows of 256 bytes r % 16
template <int ROWB>
__device__ __forceinline__ int gate_swz(int r) {
  return ROWB == 64 ? ((r >> 2) & 3) : ROWB == 128 ? ((r >> 1) & 7) : (r & 15);
}

// s_waitcnt for a ring whose `young` newest steps (0-7) may still be in flight, P copies each
// (a kernel's ring depth keeps young * P within vmcnt's range of 63; larger cases are never
// reached and are clamped only so that every case encodes)
template <int P>
__device__ __forceinline__ void gate_wait(int young) {
  constexpr auto c = [](int n) { return n < 63 ? n : 63; };
  switch (young) {
    case 0: wait_vm_lgkm<0>(); break;
    case 1: wait_vm_lgkm<c(P)>(); break;
    case 2: wait_vm_lgkm<c(2 * P)>(); break;
    case 3: wait_vm_lgkm<c(3 * P)>(); break;
    case 4: wait_vm_lgkm<c(4 * P)>(); break;
    case 5: wait_vm_lgkm<c(5 * P)>(); break;
    case 6: wait_vm_lgkm<c(6 * P)>(); break;
    default: wait_vm_lgkm<c(7 * P)>(); break;
  }
}

// 8 floats -> bf16 high parts (round to nearest even) and bf16 of the remainders.
__device__ __forceinline__ void split8(const u32x4& a, const u32x4& b, bf16x8& hi, bf16x8& lo) {
  const float v[8] = {__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[2]),
                      __uint_as_float(a[3]), __uint_as_float(b[0]), __uint_as_float(b[1]),
                      __uint_as_float(b[2]), __uint_as_float(b[3])};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h = static_cast<__bf16>(v[i]);
    hi[i] = h;
    lo[i] = static_cast<__bf16>(v[i] - static_cast<float>(h));
  }
}

// W_R fp32 [E][H] -> split [E][H/32][hi 32 bf16, lo 32 bf16]: one thread per 8 values.
__global__ __launch_bounds__(256) void gate_split_kernel(const float* __restrict__ w, int E, int H,
                                                         u32x4* __restrict__ out) {
  const size_t c = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;   // 8-value chunk
  const size_t n = static_cast<size_t>(E) * (H / 8);
  if (c >= n) return;
  // chunk kc of row: 32-K block kc / 4, part kc % 4 of it
  const size_t row = c / (H / 8), kc = c % (H / 8);
  const u32x4* src = reinterpret_cast<const u32x4*>(w + row * H + kc * 8);
  bf16x8 hi, lo;
  split8(src[0], src[1], hi, lo);
  u32x4* dst = out + row * (H / 32) * 8 + (kc / 4) * 8 + (kc % 4);
  dst[0] = __builtin_bit_cast(u32x4, hi);
  dst[4] = __builtin_bit_cast(u32x4, lo);
}

// Waves of a gate_kernel workgroup: 8 when a step's x bytes and router bytes both split into
// 1 KB copies over eight waves, else 4. With 8, two groups of four waves take the two 16-wide
// halves of every K step into accumulators of their own (summed once at the end), so each SIMD
// runs two waves: a single wave per SIMD reads LDS at about a third of the rate two reach.
template <int EB, int TB, bool XF32>
constexpr int gate_waves() {
  return (TB * 32 * (XF32 ? 128 : 64)) % 8192 == 0 && (EB * 32 * 128) % 8192 == 0 ? 8 : 4;
}

// K per step of a gate_kernel tile: 64 for bf16 x when its ring of 64-wide steps (4 stages up
// to 32 KB, 3 above) fits in 144 KB of LDS, else 32. Measured after a 1 GiB read: 64 x 32 tiles
// on 4096 tokens x 2048 x 64 experts 24.8 -> 21.4 us, fused 64 x 64 on 16384 x 2048 x 48
// 30.9 -> 27.6 us, 128 x 128 on 16384 x 7168 x 256 147 -> 139 us; fp32 x keeps 32 (its 64-wide
// ring takes 128 KB for 64 x 64 tiles, one workgroup per CU: 32768 tokens 61 -> 68 us).
template <int EB, int TB, bool XF32>
constexpr int gate_gk() {
  constexpr int stage = TB * 32 * 64 * (XF32 ? 4 : 2) + EB * 32 * 64 * 4;
  return !XF32 && (stage > 32 * 1024 ? 3 : 4) * stage <= 144 * 1024 ? 64 : 32;
}

// EB: expert blocks of 32 per workgroup (expert tile blockIdx.y); TB: token blocks of 32 (1, 2
// or 4); XF32: x is fp32 (else bf16). ws: W_R split by gate_split_kernel. SEG > 0: the route
// with layout (SEG, PER) runs in the epilogue (one expert tile, E <= 32 EB). GK: K per step, 32
// or 64 (H a multiple of it): 64 halves the steps, and with them the per-step waits and
// barriers, for the large 128 x 128 tiles.
template <int EB, int TB, bool XF32, int SEG = 0, int PER = 0, bool VEC = false, int GK = kGK>
__global__ __launch_bounds__((gate_waves<EB, TB, XF32>() * 64)) void gate_kernel(
    const void* __restrict__ xv, const float* __restrict__ w, int N, int H, int E,
    float* __restrict__ logits, const float* __restrict__ bias, int k, int gate,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    const int32_t* __restrict__ placement, int W, CountWs cw) {
  static_assert(4 % TB == 0 && TB * EB >= 2, "every wave keeps one token block");
  constexpr int TM = TB * 32;                    // tokens per workgroup
  constexpr int ER = EB * 32;                    // expert rows per workgroup
  static_assert(GK == 32 || GK == 64, "K steps of 32 or 64");
  constexpr int XRB = GK * (XF32 ? 4 : 2);       // LDS bytes per x row per step
  constexpr int WRB = GK * 4;                    // LDS bytes per W_R row per step (hi, lo per 32)
  constexpr int XS = TM * XRB, WS = ER * WRB;    // stage bytes
  // ring depth: 4 stages up to 32 KB, 3 above (at most 144 KB of LDS)
  constexpr int S = XS + WS > 32 * 1024 ? 3 : 4;
  static_assert((S - 1) * ((XS + WS) / 1024 / gate_waves<EB, TB, XF32>()) <= 63, "vmcnt range");
  constexpr int NW = gate_waves<EB, TB, XF32>();
  constexpr int KG = NW / 4;                     // K groups: 2 take one half of each step
  constexpr int NT = NW * 64;
  constexpr int XD = XS / 1024 / NW, WD = WS / 1024 / NW;  // copies per wave per stage
  constexpr int kPer = XD + WD;
  constexpr int NBW = TB * EB >= 4 ? TB * EB / 4 : 1;  // 32 x 32 blocks per wave (fewer than
                                                         // 4 blocks: some waves only copy)
  // a wave's blocks: MT token blocks x ME expert blocks, 2 x 2 or 2 x 1 where the tile allows,
  // so that each fragment read from LDS feeds two MFMA pairs (1 x 4 reads one x fragment and
  // eight router fragments for four pairs, 2 x 2 two and four)
  // (bf16 x only: fp32 x is split into high and low parts per fragment, and the split's vector
  // work per MFMA would double)
  constexpr int MT = !XF32 && NBW >= 2 && TB >= 2 ? 2 : 1;
  constexpr int ME = NBW / MT;
  constexpr int TGN = TB / MT;                    // token groups of the tile
  static_assert(MT * ME == NBW && TB % MT == 0 && (NBW == 1 || TGN * (EB / ME) == 4),
                "the four waves of a K group cover the tile");
  __shared__ __attribute__((aligned(1024))) char xs[S * XS];
  __shared__ __attribute__((aligned(1024))) char ws[S * WS];

  const int l = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.x * TM;
  const int e0 = blockIdx.y * ER;
  const int KT = H / GK;
  const char* xb = uniform_ptr(static_cast<const char*>(xv) +
                               static_cast<size_t>(t0) * H * (XF32 ? 4 : 2));
  const char* wb = uniform_ptr(reinterpret_cast<const char*>(w));

  // copy offsets: instruction i of this wave fills rows (wave share) of 1 KB; lane l copies chunk
  // (l % CPR) ^ swz(row) of row q + l / CPR (rows past N or E repeat a valid row)
  uint32_t gx[XD], gw[WD];
#pragma unroll
  for (int i = 0; i < XD; ++i) {
    constexpr int cpr = XRB / 16;
    const int r = (wv * XD + i) * (1024 / XRB) + l / cpr;
    const int t = min(r, N - 1 - t0);
    gx[i] = static_cast<uint32_t>(t) * H * (XF32 ? 4 : 2) +
            (((l % cpr) ^ gate_swz<XRB>(r)) << 4);
  }
#pragma unroll
  for (int i = 0; i < WD; ++i) {
    constexpr int cpr = WRB / 16;
    const int r = (wv * WD + i) * (1024 / WRB) + l / cpr;
    const int e = min(e0 + r, E - 1);
    // split rows: 4H bytes
    gw[i] = static_cast<uint32_t>(e) * H * 4 + (((l % cpr) ^ gate_swz<WRB>(r)) << 4);
  }
  const uint32_t lx = lds_addr(xs) + wv * XD * 1024;
  const uint32_t lw = lds_addr(ws) + wv * WD * 1024;
  auto issue = [&](int kt) {
    const int slot = kt % S;
#pragma unroll
    for (int i = 0; i < XD; ++i)
      dma16(xb + kt * XRB, gx[i], lx + slot * XS + i * 1024);
#pragma unroll
    for (int i = 0; i < WD; ++i) dma16(wb + kt * WRB, gw[i], lw + slot * WS + i * 1024);
  };

  // wave wq of each K group: token blocks tg MT .. tg MT + MT - 1 and expert blocks
  // eg ME .. eg ME + ME - 1 (block i = a ME + b: token block tg MT + a, expert block eg ME + b)
  const int wq = wv & 3, kg = wv >> 2;
  const int tg = wq % TGN;
  const int eg = wq / TGN;
  const bool active = eg * ME < EB;
  f32x16 acc[NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[i][q] = 0.f;

  const int frow = l & 31;   // fragment rows are 32-aligned: swz of the row = swz(l % 32)
  // The fragments of one 16-wide K sub-step ks of the step in ring slot `slot`: this lane's 8 K
  // values start at kk. A split router row holds, per 32 K, 4 chunks of high parts then 4 of low
  // parts.
  struct Frags {
    bf16x8 ah[MT], al[MT], bh[ME], bl[ME];
  };
  auto read = [&](Frags& f, int slot, int ks) {
    const char* xsl = xs + slot * XS;
    const char* wsl = ws + slot * WS;
    const int kk = ks * 16 + (l >> 5) * 8;
#pragma unroll
    for (int a = 0; a < MT; ++a) {
      const int xr = (tg * MT + a) * 32 + frow;
      if (XF32) {
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(
            xsl + xr * XRB + (((kk / 4) ^ gate_swz<XRB>(frow)) << 4));
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(
            xsl + xr * XRB + (((kk / 4 + 1) ^ gate_swz<XRB>(frow)) << 4));
        split8(a0, a1, f.ah[a], f.al[a]);
      } else {
        f.ah[a] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
            xsl + xr * XRB + (((kk / 8) ^ gate_swz<XRB>(frow)) << 4)));
      }
    }
    const int ch = (kk / 32) * 8 + (kk % 32) / 8;
#pragma unroll
    for (int b = 0; b < ME; ++b) {
      const int wr = (eg * ME + b) * 32 + frow;
      f.bh[b] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
          wsl + wr * WRB + ((ch ^ gate_swz<WRB>(frow)) << 4)));
      f.bl[b] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
          wsl + wr * WRB + (((ch + 4) ^ gate_swz<WRB>(frow)) << 4)));
    }
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
      for (int b = 0; b < ME; ++b) {
        f32x16& c = acc[a * ME + b];
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.ah[a], f.bh[b], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.ah[a], f.bl[b], c, 0, 0, 0);
        if (XF32) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.al[a], f.bh[b], c, 0, 0, 0);
      }
  };
  // the step's GK / 16 sub-steps: all of them, or with two K groups each group its half
  constexpr int KSG = GK / 16 / KG;
  auto ks_of = [&](int j) { return KG == 2 ? kg * KSG + j : j; };

#pragma unroll
  for (int k0 = 0; k0 < S; ++k0)
    if (k0 < KT) issue(k0);
  if constexpr (!XF32 && KSG % 2 == 0) {
    // Sub-steps alternate between two fragment buffers; the wait and barrier for step kt + 1
    // sit inside step kt, before its last sub-step's MFMAs, and the first fragments of kt + 1
    // load while those multiply. At that barrier every wave has read all of step kt (its reads
    // are waited for with the copies), so step kt's slot takes step kt + S. The last step runs
    // apart, so that no code after the barrier is shared with a path whose reads are still in
    // flight (the compiler would then wait for the next step's reads before these MFMAs).
    // Scheduling barriers keep the reads of the next sub-step among the MFMAs of the current
    // one: one MFMA, one read, and so on (an MFMA first: a read ahead of it would make the wait
    // for the current fragments wait for that read too).
    auto overlap = [&]() {
      constexpr int NR = MT + 2 * ME, NM = 2 * MT * ME;
#pragma unroll
      for (int i = 0; i < (NR > NM ? NR : NM); ++i) {
        if (i < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    gate_wait<kPer>(min(S - 1, KT - 1));
    raw_barrier();
    Frags f0, f1;
    if (active) read(f0, 0, ks_of(0));
    for (int kt = 0; kt + 1 < KT; ++kt) {
#pragma unroll
      for (int j = 0; j < KSG; j += 2) {
        if (active) {
          read(f1, kt % S, ks_of(j + 1));
          mma(f0);
          overlap();
        }
        if (j + 2 < KSG) {
          if (active) read(f0, kt % S, ks_of(j + 2));
        } else {
          gate_wait<kPer>(min(S - 2, KT - 2 - kt));
          raw_barrier();
          if (kt + S < KT) issue(kt + S);
          if (active) read(f0, (kt + 1) % S, ks_of(0));
        }
        if (active) {
          mma(f1);
          overlap();
        }
      }
    }
    if (active) {
      const int slot = (KT - 1) % S;
#pragma unroll
      for (int j = 0; j < KSG; j += 2) {
        read(f1, slot, ks_of(j + 1));
        mma(f0);
        if (j + 2 < KSG) read(f0, slot, ks_of(j + 2));
        mma(f1);
      }
    }
  } else {
    for (int kt = 0; kt < KT; ++kt) {
      // step kt landed (its copies are the oldest in flight) and every wave is done with kt - 1
      const int young = kt == 0 ? min(S - 1, KT - 1) : min(S - 2, KT - 1 - kt);
      gate_wait<kPer>(young);
      raw_barrier();
      if (kt >= 1 && kt - 1 + S < KT) issue(kt - 1 + S);   // into the slot step kt - 1 freed
      if (active) {
#pragma unroll
        for (int j = 0; j < KSG; ++j) {
          Frags f;
          read(f, kt % S, ks_of(j));
          mma(f);
        }
      }
    }
  }

  // two K groups: the second group's partial tiles go through the (idle) weight ring to the
  // first, which adds them to its own
  if constexpr (KG == 2) {
    static_assert(4 * NBW * 16 * 64 * 4 <= S * WS, "the partial tiles fit the weight ring");
    float* red = reinterpret_cast<float*>(ws);
    __syncthreads();   // every wave has read its last fragments from the rings
    if (kg == 1 && active) {
#pragma unroll
      for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) red[((wq * NBW + i) * 16 + q) * 64 + l] = acc[i][q];
    }
    __syncthreads();
    if (kg == 0 && active) {
#pragma unroll
      for (int i = 0; i < NBW; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][q] += red[((wq * NBW + i) * 16 + q) * 64 + l];
    }
  }
  const bool holder = active && kg == 0;   // holds the tile's logits

  // lane l holds expert column l % 32 of its block and, for q = 0..15, token row
  // 8 (q / 4) + 4 (l / 32) + q % 4
  if (SEG == 0 && !holder) return;
  if (holder) {
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      const int e = e0 + (eg * ME + i % ME) * 32 + (l & 31);
      if (e >= E) continue;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int t = t0 + (tg * MT + i / ME) * 32 + (q >> 2) * 8 + (l >> 5) * 4 + (q & 3);
        if (t < N) logits[static_cast<size_t>(t) * E + e] = acc[i][q];
      }
    }
  }
  if constexpr (SEG > 0) {
    // fused route: the tile's logits [TM][E] into the (now idle) weight ring, then one segment
    // of SEG lanes per token
    static_assert(TM * ER * 4 <= S * WS, "the logits tile fits in the weight ring");
    // With a layout workspace, the tile's count masks (one 64-token group) go to the idle x
    // ring and the tile writes its count rows after the route.
    static_assert(TM == 64 && (ER + MOE_MAX_RANKS) * 8 <= S * XS, "count masks fit the x ring");
    float* tile = reinterpret_cast<float*>(ws);
    unsigned long long* masks = reinterpret_cast<unsigned long long*>(xs);
    const bool count = cw.e != nullptr;
    __syncthreads();   // every wave has read its last fragments (and partials) from the rings
    if (holder) {
#pragma unroll
      for (int i = 0; i < NBW; ++i) {
        const int e = (eg * ME + i % ME) * 32 + (l & 31);
        if (e >= E) continue;
#pragma unroll
        for (int q = 0; q < 16; ++q)
          tile[((tg * MT + i / ME) * 32 + (q >> 2) * 8 + (l >> 5) * 4 + (q & 3)) * E + e] =
              acc[i][q];
      }
    }
    RouteCount rc{};
    if (count) {
      rc = RouteCount{masks, masks + E, placement, E / W, W};
      for (int i = threadIdx.x; i < E + W; i += NT) masks[i] = 0ull;
    }
    __syncthreads();
    for (int tl = threadIdx.x / SEG; tl < TM; tl += NT / SEG) {
      if (t0 + tl >= N) break;   // whole segments stop together
      route_token<SEG, PER, VEC>(tile + tl * E, bias, E, k, gate, threadIdx.x & (SEG - 1), t0 + tl,
                                 topk_idx, topk_w, rc, tl);
    }
    if (count) {
      __syncthreads();
      write_count_rows(masks, masks + E, E, W, count_tokens(E), t0, min(TM, N - t0), N, cw);
    }
  }
}

// Launches gate_kernel with K steps of 64 where the ring fits (gate_gk) and H allows, else 32.
template <int EB, int TB, int SEG = 0, int PER = 0, bool VEC = false>
static void launch_gate(const void* x, bool xf32, const float* ws, int N, int H, int E,
                        float* logits, const float* bias, int k, int gate, int32_t* idx,
                        float* topw, const int32_t* placement, int W, CountWs cw, hipStream_t s) {
  const dim3 grid((N + 32 * TB - 1) / (32 * TB), (E + 32 * EB - 1) / (32 * EB));
  auto go = [&](auto xf, auto gk) {
    constexpr bool XF = decltype(xf)::value;
    constexpr int GK = decltype(gk)::value;
    hipLaunchKernelGGL((gate_kernel<EB, TB, XF, SEG, PER, VEC, GK>),
                       grid, dim3(gate_waves<EB, TB, XF>() * 64), 0, s, x, ws, N, H, E,
                       logits, bias, k, gate, idx, topw, placement, W, cw);
  };
  using std::integral_constant;
  const bool k64 = H % 64 == 0;
  if (xf32) {
    if (k64) go(std::true_type{}, integral_constant<int, gate_gk<EB, TB, true>()>{});
    else go(std::true_type{}, integral_constant<int, kGK>{});
  } else {
    if (k64) go(std::false_type{}, integral_constant<int, gate_gk<EB, TB, false>()>{});
    else go(std::false_type{}, integral_constant<int, kGK>{});
  }
}

// 64 tokens x all E experts per workgroup (E <= 32 EB) with the route in the epilogue, in the
// layout moe_route uses for E.
// Returns false (and launches nothing) when the segment shape route_shape picks for E has no
// fused instance for this EB; the caller then runs the unfused product and moe_route.
template <int EB>
static bool launch_gate_fused(const void* x, bool xf32, const float* ws, int N, int H, int E,
                              float* logits, const float* bias, int k, int gate, int32_t* idx,
                              float* topw, const int32_t* placement, int W, CountWs cw,
                              hipStream_t s) {
  bool launched = false;
  route_shape(E, [&](auto seg, auto per, auto vec) {
    constexpr int SEG = decltype(seg)::value, PER = decltype(per)::value;
    constexpr bool VEC = decltype(vec)::value;
    if constexpr (SEG * PER <= 32 * EB && (EB == 1 || SEG * PER == 32 * EB)) {
      if (SEG != route_seg(E)) return;   // count rows must be the layout's
      launch_gate<EB, 2, SEG, PER, VEC>(x, xf32, ws, N, H, E, logits, bias, k, gate, idx, topw,
                                        placement, W, cw, s);
      launched = true;
    }
  });
  return launched;
}

// ------------------------------------------------------------------------------------------
// Few experts (E <= 32): 32 tokens per workgroup, so token counts that give 64-token tiles
// fewer workgroups than the chip has CUs still spread over all of them. K steps are 64 wide,
// and only the router rows that exist are copied (E rounded up to 16 or 32), so that x and the
// router rows split evenly over the four waves' 1 KB copies. Each wave multiplies one 16-wide
// K sub-step of every step into accumulators of its own (the high and low router parts apart),
// and the four partial logits tiles are summed in a fixed order. The route and the count rows
// then run in the epilogue as in gate_kernel.
constexpr int kGK2 = 64;    // K per step

// 16-byte chunk slot of row r: 256-byte rows use r % 16, 128-byte rows (r / 2) % 8. A fragment
// read (lanes 16 i .. 16 i + 15 on rows 16 consecutive rows at one chunk) then hits 16
// different slots.
template <int ROWB>
__device__ __forceinline__ int gate_swz2(int r) {
  return ROWB == 256 ? (r & 15) : ((r >> 1) & 7);
}


// WR: router rows copied per step (16 or 32, >= E). The route layout (SEG, PER, VEC) is the one
// moe_route uses for E, and count_tokens(E) divides the 32-token tile.
template <int WR, bool XF32, int SEG, int PER, bool VEC>
__global__ __launch_bounds__(256) void gate_small_kernel(
    const void* __restrict__ xv, const float* __restrict__ w, int N, int H, int E,
    float* __restrict__ logits, const float* __restrict__ bias, int k, int gate,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    const int32_t* __restrict__ placement, int W, CountWs cw) {
  constexpr int TM = 32;                         // tokens per workgroup
  constexpr int XEB = XF32 ? 4 : 2;              // bytes per x value
  constexpr int XRB = kGK2 * XEB;                // LDS bytes per x row per step (128 or 256)
  constexpr int WRB = kGK2 * 4;                  // per router row per step: (hi 32, lo 32) x 2
  constexpr int XS = TM * XRB, WS = WR * WRB;
  constexpr int STAGE = XS + WS;
  constexpr int C = STAGE / 1024;                // 1 KB copies per step
  static_assert(C % 4 == 0, "the copies of a step split evenly over the four waves");
  constexpr int P = C / 4;                       // copies per wave per step
  constexpr int XC = XS / 1024;                  // copies 0 .. XC-1 are x, the rest router rows
  constexpr int S = 64 * 1024 / STAGE;           // ring depth: 64 KB of steps
  static_assert(S >= 2 && S <= 8 && (S - 1) * P <= 63, "ring depth and vmcnt range");
  static_assert(4 * TM * 32 * 4 + TM * 32 * 4 <= S * STAGE, "partials and tile fit the ring");
  __shared__ __attribute__((aligned(1024))) char ring[S * STAGE];
  __shared__ unsigned long long masks[32 + MOE_MAX_RANKS];

  const int l = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.x * TM;
  const int KT = H / kGK2;
  const bool count = cw.e != nullptr;
  if (count)
    for (int i = threadIdx.x; i < E + W; i += 256) masks[i] = 0ull;

  // copy j = wv * P + i fills LDS bytes j KB .. of a stage: x rows (XRB bytes each) first, then
  // router rows (256 bytes); lane l copies chunk (l % CPR) ^ swz(row) of row q + l / CPR. Rows
  // past N or E repeat a valid row.
  const char* xb = uniform_ptr(static_cast<const char*>(xv) +
                               static_cast<size_t>(t0) * H * XEB);
  const char* wb = uniform_ptr(reinterpret_cast<const char*>(w));
  uint32_t goff[P];
  const char* cbase[P];
  int cstep[P];                                  // global bytes per K step of the copy's row
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int j = wv * P + i;                    // wave-uniform: the base and step are scalar
    cbase[i] = j < XC ? xb : wb;
    cstep[i] = j < XC ? XRB : WRB;
    if (j < XC) {
      constexpr int cpr = XRB / 16;
      const int r = j * (1024 / XRB) + l / cpr;
      const int t = min(r, N - 1 - t0);
      goff[i] = static_cast<uint32_t>(t) * H * XEB + (((l % cpr) ^ gate_swz2<XRB>(r)) << 4);
    } else {
      const int r = (j - XC) * (1024 / WRB) + l / 16;
      const int e = min(r, E - 1);
      goff[i] = static_cast<uint32_t>(e) * H * 4 + (((l % 16) ^ gate_swz2<WRB>(r)) << 4);
    }
  }
  const uint32_t lds0 = lds_addr(ring) + wv * P * 1024;
  auto issue = [&](int kt) {
    const int slot = kt % S;
#pragma unroll
    for (int i = 0; i < P; ++i)
      dma16(cbase[i] + kt * cstep[i], goff[i], lds0 + slot * STAGE + i * 1024);
  };

  // fragment reads of wave wv: K values 16 wv + 8 (l / 32) .. + 7 of the step, for token row
  // l % 32 and router row l % 32 (rows past WR repeat: their logits columns are dropped)
  const int frow = l & 31;
  const int kk = wv * 16 + (l >> 5) * 8;
  const int wrow = frow < WR ? frow : frow - WR;
  int xo0, xo1 = 0;
  if (XF32) {
    xo0 = frow * XRB + (((kk / 4) ^ gate_swz2<XRB>(frow)) << 4);
    xo1 = frow * XRB + (((kk / 4 + 1) ^ gate_swz2<XRB>(frow)) << 4);
  } else {
    xo0 = frow * XRB + (((kk / 8) ^ gate_swz2<XRB>(frow)) << 4);
  }
  const int chi = (kk / 32) * 8 + (kk % 32) / 8;   // split row: per 32 K, 4 chunks hi, 4 lo
  const int who = XS + wrow * WRB + ((chi ^ gate_swz2<WRB>(wrow)) << 4);
  const int wlo = XS + wrow * WRB + (((chi + 4) ^ gate_swz2<WRB>(wrow)) << 4);

  f32x16 ah_bh, ah_bl, al_bh;
#pragma unroll
  for (int q = 0; q < 16; ++q) ah_bh[q] = ah_bl[q] = al_bh[q] = 0.f;
  auto compute = [&](int slot) {
    const char* st = ring + slot * STAGE;
    bf16x8 ah, al;
    if (XF32) {
      split8(*reinterpret_cast<const u32x4*>(st + xo0), *reinterpret_cast<const u32x4*>(st + xo1),
             ah, al);
    } else {
      ah = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + xo0));
    }
    const bf16x8 bh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + who));
    const bf16x8 bl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + wlo));
    ah_bh = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, ah_bh, 0, 0, 0);
    ah_bl = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, ah_bl, 0, 0, 0);
    if (XF32) al_bh = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, al_bh, 0, 0, 0);
  };

#pragma unroll
  for (int k0 = 0; k0 < S; ++k0)
    if (k0 < KT) issue(k0);
  for (int kt = 0; kt < KT; ++kt) {
    // step kt landed (its copies are the oldest in flight) and every wave is done with kt - 1
    gate_wait<P>(kt == 0 ? min(S - 1, KT - 1) : min(S - 2, KT - 1 - kt));
    raw_barrier();
    if (kt >= 1 && kt - 1 + S < KT) issue(kt - 1 + S);   // into the slot step kt - 1 freed
    compute(kt % S);
  }

  // partial tiles [4][32 tokens][32 columns] in the ring, then the sum [32][E] after them. Lane
  // l holds column l % 32 and, for q = 0..15, token row 8 (q / 4) + 4 (l / 32) + q % 4.
  __syncthreads();   // every wave has read its last fragments
  float* part = reinterpret_cast<float*>(ring);
  float* tile = part + 4 * TM * 32;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int m = (q >> 2) * 8 + (l >> 5) * 4 + (q & 3);
    float v = ah_bh[q] + ah_bl[q];
    if (XF32) v += al_bh[q];
    part[(wv * TM + m) * 32 + (l & 31)] = v;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < TM * 32; i += 256) {
    const int m = i >> 5, e = i & 31;
    if (e >= E) continue;
    const float v = ((part[i] + part[TM * 32 + i]) + part[2 * TM * 32 + i]) + part[3 * TM * 32 + i];
    tile[m * E + e] = v;
    if (t0 + m < N) logits[static_cast<size_t>(t0 + m) * E + e] = v;
  }
  __syncthreads();
  const RouteCount rc = count ? RouteCount{masks, masks + E, placement, E / W, W} : RouteCount{};
  for (int tl = threadIdx.x / SEG; tl < TM; tl += 256 / SEG) {
    if (t0 + tl >= N) break;   // whole segments stop together
    route_token<SEG, PER, VEC>(tile + tl * E, bias, E, k, gate, threadIdx.x & (SEG - 1), t0 + tl,
                               topk_idx, topk_w, rc, tl);
  }
  if (count) {
    __syncthreads();
    write_count_rows(masks, masks + E, E, W, count_tokens(E), t0, min(TM, N - t0), N, cw);
  }
}

// The few-expert gate with the route fused, when it applies: E <= 32, H a multiple of 64, a
// count row of at most 32 tokens (E >= 5), and either E <= 16 (then it never copies more bytes
// per token than the 64-token tiles) or at most 512 token tiles of 32. Returns false otherwise.
static bool launch_gate_small(const void* x, bool xf32, const float* ws, int N, int H, int E,
                              float* logits, const float* bias, int k, int gate, int32_t* idx,
                              float* topw, const int32_t* placement, int W, CountWs cw,
                              hipStream_t s) {
  if (E > 32 || H % kGK2 != 0 || count_tokens(E) > 32 || (E > 16 && N > 16 * 1024)) return false;
  bool launched = false;
  route_shape(E, [&](auto seg, auto per, auto vec) {
    constexpr int SEG = decltype(seg)::value, PER = decltype(per)::value;
    constexpr bool VEC = decltype(vec)::value;
    if constexpr (SEG * PER <= 32 && SEG >= 8) {
      if (SEG != route_seg(E)) return;
      const dim3 grid((N + 31) / 32), block(256);
      auto go = [&](auto wr) {
        constexpr int WR = decltype(wr)::value;
        if (xf32)
          hipLaunchKernelGGL((gate_small_kernel<WR, true, SEG, PER, VEC>), grid, block, 0, s, x, ws,
                             N, H, E, logits, bias, k, gate, idx, topw, placement, W, cw);
        else
          hipLaunchKernelGGL((gate_small_kernel<WR, false, SEG, PER, VEC>), grid, block, 0, s, x,
                             ws, N, H, E, logits, bias, k, gate, idx, topw, placement, W, cw);
      };
      if (E <= 16) go(std::integral_constant<int, 16>{});
      else go(std::integral_constant<int, 32>{});
      launched = true;
    }
  });
  return launched;
}

}  // namespace moe

extern "C" size_t moe_gate_workspace_bytes(int E, int H) {
  return E > 0 && H > 0 ? static_cast<size_t>(E) * H * 4 : 0;
}

namespace moe {
static void launch_split(const float* w_router, int E, int H, void* workspace, hipStream_t s) {
  const size_t chunks = static_cast<size_t>(E) * (H / 8);
  hipLaunchKernelGGL(gate_split_kernel, dim3(static_cast<unsigned>((chunks + 255) / 256)),
                     dim3(256), 0, s, w_router, E, H, static_cast<u32x4*>(workspace));
}
}  // namespace moe

extern "C" moe_status moe_gate_prepare(const float* w_router, int E, int H, void* workspace,
                                       void* stream) {
  using namespace moe;
  if (H <= 0 || H % kGK != 0 || E < 1 || E > 256) {
    moe_host::set_error("moe_gate_prepare: invalid shape (H a multiple of 32, E <= 256)");
    return MOE_EINVAL;
  }
  if (!w_router || !workspace) {
    moe_host::set_error("moe_gate_prepare: NULL pointer");
    return MOE_EINVAL;
  }
  launch_split(w_router, E, H, workspace, moe_host::as_stream(stream));
  return moe_host::launch_status();
}

extern "C" moe_status moe_gate_route(const void* x, int dtype, const float* w_router,
                                     const float* bias, int N, int H, int E, int k, int gate,
                                     void* workspace, float* logits, int32_t* topk_idx,
                                     float* topk_w, const int32_t* expert_rank, int W,
                                     void* layout_workspace, void* stream) {
  using namespace moe;
  if (N < 0 || H <= 0 || H % kGK != 0 || E < 1 || E > 256 || k < 1 || k > E ||
      k > MOE_MAX_TOPK || (dtype != MOE_F32 && dtype != MOE_BF16) ||
      (gate != MOE_GATE_SOFTMAX && gate != MOE_GATE_SIGMOID)) {
    moe_host::set_error("moe_gate_route: invalid shape (H a multiple of 32, E <= 256, k <= E), "
                        "dtype or gate");
    return MOE_EINVAL;
  }
  // the copies address rows of W_R and of a token tile with 32-bit byte offsets
  if (static_cast<long long>(E > 128 ? E : 128) * H * 4 >= (1ll << 32)) {
    moe_host::set_error("moe_gate_route: max(E, 128) * H * 4 bytes reach 4 GiB");
    return MOE_EINVAL;
  }
  if (!moe_host::route_counts_ok(N, E, W, layout_workspace)) {
    moe_host::set_error("moe_gate_route: with a layout workspace W must be in 1..64 and divide "
                        "E and N");
    return MOE_EINVAL;
  }
  if (N == 0) return MOE_OK;
  if (!x || !workspace || !logits || !topk_idx || !topk_w) {
    moe_host::set_error("moe_gate_route: NULL pointer");
    return MOE_EINVAL;
  }
  const CountWs cw = layout_workspace ? count_ws_carve(N, E, W, layout_workspace) : CountWs{};
  hipStream_t s = moe_host::as_stream(stream);
  if (w_router) launch_split(w_router, E, H, workspace, s);   // else prepared by moe_gate_prepare
  const float* ws = static_cast<const float*>(workspace);
  const bool xf32 = dtype == MOE_F32;
  // many tokens and many experts: 128 x 128 tiles (the router weights are read by half as many
  // token tiles, x by two expert tiles); 33-64 experts on fewer than 16384 tokens: 64 tokens x
  // 32 experts (twice the workgroups of 64 x 64: 26-28 against 33 us for the fused 64 x 64 on
  // 4096 tokens); both then run moe_route on the logits. Otherwise all experts per workgroup
  // with the route fused into the epilogue: 32 tokens for 5-32 experts (gate_small_kernel: on
  // the Llama-4-Scout-shaped layer's 8192 tokens x 16 experts, twice the workgroups of 64-token
  // tiles and half the router-row copies), else 64.
  const bool tiles128 = E > 128 && N >= 16 * 1024;
  if (tiles128 || (E > 32 && E <= 64 && N < 16 * 1024)) {
    if (tiles128)
      launch_gate<4, 4>(x, xf32, ws, N, H, E, logits, nullptr, 0, 0, nullptr, nullptr, nullptr, 0,
                        CountWs{}, s);
    else
      launch_gate<1, 2>(x, xf32, ws, N, H, E, logits, nullptr, 0, 0, nullptr, nullptr, nullptr, 0,
                        CountWs{}, s);
    const moe_status st = moe_host::launch_status();
    if (st != MOE_OK) return st;
    return moe_route(logits, bias, N, E, k, gate, topk_idx, topk_w, expert_rank, W,
                     layout_workspace, stream);
  }
  if (launch_gate_small(x, xf32, ws, N, H, E, logits, bias, k, gate, topk_idx, topk_w,
                        expert_rank, W, cw, s))
    return moe_host::launch_status();
  auto fused = [&](auto eb) {
    return launch_gate_fused<decltype(eb)::value>(x, xf32, ws, N, H, E, logits, bias, k, gate,
                                                  topk_idx, topk_w, expert_rank, W, cw, s);
  };
  bool done;
  if (E <= 32)       done = fused(std::integral_constant<int, 1>{});
  else if (E <= 64)  done = fused(std::integral_constant<int, 2>{});
  else if (E <= 128) done = fused(std::integral_constant<int, 4>{});
  else               done = fused(std::integral_constant<int, 8>{});
  if (!done) {   // no fused instance for this shape: the product, then the route kernel
    launch_gate<1, 2>(x, xf32, ws, N, H, E, logits, nullptr, 0, 0, nullptr, nullptr, nullptr, 0,
                      CountWs{}, s);
    const moe_status st = moe_host::launch_status();
    if (st != MOE_OK) return st;
    return moe_route(logits, bias, N, E, k, gate, topk_idx, topk_w, expert_rank, W,
                     layout_workspace, stream);
  }
  return moe_host::launch_status();
}
