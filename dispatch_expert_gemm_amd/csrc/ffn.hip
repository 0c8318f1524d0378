// Grouped SwiGLU expert FFN: per group g, h = silu(A W_g^T) * (A W_u^T), y = h W_d^T.
//
// Blog "Kernel fusion for expert parallelism", section "Fusing the layer into one kernel": stage
// MatMul (gate and up projection), stage SwiGLU, stage MatMul (down projection); the two grouped
// matrix multiplications dominate the layer. FarSkip-Collective section 2.1: shared experts run on
// every token in addition to the routed ones; here they are extra groups of the same launches.
//
// Two launches per call, each a grouped GEMM C = A B^T over all groups with both operands
// K-contiguous ("NT"):
//   GEMM1 (NB = 2): B = [gate rows; up rows] of w_gate_up, epilogue h = silu(gate) * up;
//   GEMM2 (NB = 1): A = h, B = w_down.
// The tile list lives on the device: the row counts per group come from group_offsets, so no
// host synchronisation is needed. A persistent grid walks the tiles; tiles are ordered
// group-major, then output column panel, then row tile, and each of the 8 XCDs takes one
// contiguous eighth of that order, so the row tiles that share a weight panel run together on one
// XCD and reuse it from that XCD's L2.
//
// bf16 path: 128 x 128 tiles per B matrix, K step 64, 4 waves (2 x 2) each owning 64 x 64 per B
// matrix as 4 x 4 MFMA 16x16x32 bf16 blocks with fp32 accumulators. Global loads of the next K
// step are issued into registers before the MFMAs of the current one (LDS single buffer, rows
// padded by 8 bf16 so the 16-byte fragment reads of 16 consecutive rows hit distinct banks).
// f32 path: a plain LDS-tiled FMA kernel (64 x 64 tiles) for fp32 problems.
#include "moe_internal.h"

namespace moe {

constexpr int kMaxGroups = MOE_MAX_EXPERTS + 16;

struct GemmArgs {
  const void* a;              // routed A rows (relative to offs[0], or gathered)
  const int32_t* gather;      // absolute-row indexed source row, or NULL
  const int32_t* gather_base; // device int subtracted from gather values, or NULL
  const int32_t* offs;        // [G+1]
  int G;
  const void* w;              // [G][NB*Nn][K]
  void* c;                    // [rows][Nn] relative rows
  int S, M_sh;
  const void* a_sh;
  long long a_sh_stride;      // elements between the shared groups' A blocks (0: all read one)
  const void* w_sh;           // [S][NB*Nn][K]
  void* c_sh;                 // [S][M_sh][Nn]
  int Nn, K;
};

// Exclusive prefix of row tiles per group into mt_pre[0..G+S]; wave 0 computes, all wait.
template <int BM>
__device__ void build_tile_prefix(const GemmArgs& p, int* mt_pre) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int ng = p.G + p.S;
    int running = 0;
    for (int base = 0; base < ng; base += kWave) {
      const int g = base + lane;
      int rows = 0;
      if (g < p.G) rows = p.offs[g + 1] - p.offs[g];
      else if (g < ng) rows = p.M_sh;
      const int mt = (rows + BM - 1) / BM;
      int inc = mt;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(inc, off, kWave);
        if (lane >= off) inc += o;
      }
      if (g < ng) mt_pre[g] = running + inc - mt;
      running += __shfl(inc, kWave - 1, kWave);
    }
    if (lane == 0) mt_pre[ng] = running;
  }
  __syncthreads();
}

// Logical tile L -> (group, row tile, column tile).
__device__ __forceinline__ void decode_tile(const int* mt_pre, int ng, int NT, int L, int& g,
                                            int& mt, int& nt) {
  int lo = 0, hi = ng - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mt_pre[mid] * NT <= L) lo = mid;
    else hi = mid - 1;
  }
  g = lo;
  const int mtg = mt_pre[g + 1] - mt_pre[g];
  const int q = L - mt_pre[g] * NT;
  nt = q / mtg;
  mt = q - nt * mtg;
}

// Logical tile for this block's it-th step; -1 when done. Block b runs on XCD b % 8 and walks
// that XCD's contiguous eighth of the tile order.
__device__ __forceinline__ int next_tile(int T, int it) {
  const int xcd = blockIdx.x & 7;
  const int per = (T + 7) >> 3;
  const int local = (blockIdx.x >> 3) + it * (gridDim.x >> 3);
  if (local >= per) return -1;
  const int L = xcd * per + local;
  return L < T ? L : -1;
}

struct TileGeom {
  int rows;          // rows of the group
  int abs0;          // absolute row of the group's first row (routed)
  int rel0;          // relative row of the group's first row (routed)
  bool shared;
  const char* a;     // A base (shared: this group's block)
  const char* w;     // B base of this group
  char* c;           // C base of this group's first row
};

template <typename T, int NB>
__device__ __forceinline__ TileGeom tile_geom(const GemmArgs& p, int g) {
  TileGeom t;
  const size_t wsz = static_cast<size_t>(NB) * p.Nn * p.K * sizeof(T);
  if (g < p.G) {
    const int o0 = p.offs[0];
    t.abs0 = p.offs[g];
    t.rows = p.offs[g + 1] - t.abs0;
    t.rel0 = t.abs0 - o0;
    t.shared = false;
    t.a = static_cast<const char*>(p.a);
    t.w = static_cast<const char*>(p.w) + g * wsz;
    t.c = static_cast<char*>(p.c) + static_cast<size_t>(t.rel0) * p.Nn * sizeof(T);
  } else {
    const int s = g - p.G;
    t.abs0 = t.rel0 = 0;
    t.rows = p.M_sh;
    t.shared = true;
    t.a = static_cast<const char*>(p.a_sh) + s * p.a_sh_stride * static_cast<long long>(sizeof(T));
    t.w = static_cast<const char*>(p.w_sh) + s * wsz;
    t.c = static_cast<char*>(p.c_sh) + static_cast<size_t>(s) * p.M_sh * p.Nn * sizeof(T);
  }
  return t;
}

// Source row of the tile's m-th row (relative to TileGeom.a), or -1 beyond the group.
__device__ __forceinline__ long long a_row(const GemmArgs& p, const TileGeom& t, int m,
                                           int gbase) {
  if (m >= t.rows) return -1;
  if (t.shared) return m;
  if (p.gather) return static_cast<long long>(p.gather[t.abs0 + m]) - gbase;
  return t.rel0 + m;
}

__device__ __forceinline__ float silu(float g) { return g / (1.f + __expf(-g)); }

// ------------------------------------------------------------------------------------------
// bf16 MFMA path
// ------------------------------------------------------------------------------------------
constexpr int kBM = 128, kBN = 128, kBK = 64, kLDK = kBK + 8;

__device__ __forceinline__ bf16x8 lds_frag(const bf16_t* s) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(s);
  return __builtin_bit_cast(bf16x8, v);
}

template <int NB>
__global__ __launch_bounds__(256) void ffn_gemm_bf16(GemmArgs p) {
  __shared__ int mt_pre[kMaxGroups + 1];
  __shared__ __attribute__((aligned(16))) bf16_t As[kBM * kLDK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[NB * kBN * kLDK];

  build_tile_prefix<kBM>(p, mt_pre);
  const int ng = p.G + p.S;
  const int NT = p.Nn / kBN;
  const int T = mt_pre[ng] * NT;
  const int gbase = (p.gather && p.gather_base) ? *p.gather_base : 0;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ld_row = tid >> 3, ld_chunk = (tid & 7) * 8;  // 8 threads x 16 B per 128 B row
  const int KT = p.K / kBK;

  for (int it = 0;; ++it) {
    const int L = next_tile(T, it);
    if (L < 0) break;
    int g, mt, nt;
    decode_tile(mt_pre, ng, NT, L, g, mt, nt);
    const TileGeom tg = tile_geom<bf16_t, NB>(p, g);
    const int m0 = mt * kBM, n0 = nt * kBN;

    const bf16_t* ap[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long long r = a_row(p, tg, m0 + ld_row + 32 * i, gbase);
      ap[i] = r < 0 ? nullptr
                    : reinterpret_cast<const bf16_t*>(tg.a) + r * p.K + ld_chunk;
    }
    const bf16_t* bp[4 * NB];
#pragma unroll
    for (int i = 0; i < 4 * NB; ++i) {
      const int rb = ld_row + 32 * i;  // 0 .. NB*128-1
      const int nb = rb / kBN;
      const int wr = nb * p.Nn + n0 + (rb - nb * kBN);
      bp[i] = reinterpret_cast<const bf16_t*>(tg.w) + static_cast<size_t>(wr) * p.K + ld_chunk;
    }

    f32x4 acc[NB][4][4];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[b][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 ra[4], rb[4 * NB];
    auto gload = [&](int kt) {
      const int ko = kt * kBK;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ra[i] = ap[i] ? *reinterpret_cast<const u32x4*>(ap[i] + ko) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 4 * NB; ++i) rb[i] = *reinterpret_cast<const u32x4*>(bp[i] + ko);
    };
    auto lstore = [&]() {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4*>(&As[(ld_row + 32 * i) * kLDK + ld_chunk]) = ra[i];
#pragma unroll
      for (int i = 0; i < 4 * NB; ++i)
        *reinterpret_cast<u32x4*>(&Bs[(ld_row + 32 * i) * kLDK + ld_chunk]) = rb[i];
    };

    gload(0);
    __syncthreads();  // previous tile's readers are done with the LDS
    lstore();
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
      for (int kk = 0; kk < kBK / 32; ++kk) {
        const int col = kk * 32 + (lane >> 4) * 8;
        bf16x8 af[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          af[i] = lds_frag(&As[(wm * 64 + i * 16 + (lane & 15)) * kLDK + col]);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bf16x8 bf =
                lds_frag(&Bs[(b * kBN + wn * 64 + j * 16 + (lane & 15)) * kLDK + col]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[b][i][j] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf, acc[b][i][j], 0, 0, 0);
          }
        }
      }
      __syncthreads();
      if (kt + 1 < KT) {
        lstore();
        __syncthreads();
      }
    }

    // epilogue: lane holds column lane % 16 and rows 4 * (lane / 16) + r of each 16 x 16 block
    bf16_t* C = reinterpret_cast<bf16_t*>(tg.c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
        if (m >= tg.rows) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn * 64 + j * 16 + (lane & 15);
          float v;
          if (NB == 2) v = silu(acc[0][i][j][r]) * acc[NB - 1][i][j][r];
          else v = acc[0][i][j][r];
          C[static_cast<size_t>(m) * p.Nn + n] = f32_to_bf16(v);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// f32 path
// ------------------------------------------------------------------------------------------
constexpr int kFM = 64, kFN = 64, kFK = 16;

template <int NB>
__global__ __launch_bounds__(256) void ffn_gemm_f32(GemmArgs p) {
  __shared__ int mt_pre[kMaxGroups + 1];
  __shared__ float As[kFK][kFM + 4];
  __shared__ float Bs[NB][kFK][kFN + 4];
  build_tile_prefix<kFM>(p, mt_pre);
  const int ng = p.G + p.S;
  const int NT = p.Nn / kFN;
  const int T = mt_pre[ng] * NT;
  const int gbase = (p.gather && p.gather_base) ? *p.gather_base : 0;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  // loads: 64 rows x 16 k = 1024 floats = 256 threads x 4 (one float4 per thread per matrix)
  const int lr = tid >> 2, lk = (tid & 3) * 4;

  for (int it = 0;; ++it) {
    const int L = next_tile(T, it);
    if (L < 0) break;
    int g, mt, nt;
    decode_tile(mt_pre, ng, NT, L, g, mt, nt);
    const TileGeom tg = tile_geom<float, NB>(p, g);
    const int m0 = mt * kFM, n0 = nt * kFN;
    const long long ar = a_row(p, tg, m0 + lr, gbase);
    const float* ap = ar < 0 ? nullptr : reinterpret_cast<const float*>(tg.a) + ar * p.K + lk;
    const float* bp[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
      bp[b] = reinterpret_cast<const float*>(tg.w) +
              static_cast<size_t>(b * p.Nn + n0 + lr) * p.K + lk;
    float acc[NB][4][4] = {};
    for (int k0 = 0; k0 < p.K; k0 += kFK) {
      const f32x4 av = ap ? *reinterpret_cast<const f32x4*>(ap + k0) : f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 bv[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) bv[b] = *reinterpret_cast<const f32x4*>(bp[b] + k0);
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        As[lk + q][lr] = av[q];
#pragma unroll
        for (int b = 0; b < NB; ++b) Bs[b][lk + q][lr] = bv[b][q];
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < kFK; ++kk) {
        float a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float bb = Bs[b][kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[b][i][j] += a[i] * bb;
          }
      }
    }
    float* C = reinterpret_cast<float*>(tg.c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + ty * 4 + i;
      if (m >= tg.rows) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + tx * 4 + j;
        C[static_cast<size_t>(m) * p.Nn + n] =
            NB == 2 ? silu(acc[0][i][j]) * acc[NB - 1][i][j] : acc[0][i][j];
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------------
struct DevInfo {
  int cus = 0;
};
static DevInfo g_dev[64];

static int device_cus() {
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= 64) return 256;
  if (!g_dev[d].cus) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess ||
        n <= 0)
      n = 256;
    g_dev[d].cus = n;
  }
  return g_dev[d].cus;
}

// Blocks per CU that fit, cached per kernel (the occupancy query is not free).
static int blocks_per_cu(const void* kernel) {
  static const void* keys[16];
  static int vals[16];
  static int n = 0;
  for (int i = 0; i < n; ++i)
    if (keys[i] == kernel) return vals[i];
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  if (n < 16) {
    keys[n] = kernel;
    vals[n] = per_cu;
    ++n;
  }
  return per_cu;
}

template <typename K>
static int persistent_grid(K kernel, long long tiles_ub) {
  const int per_cu = blocks_per_cu(reinterpret_cast<const void*>(kernel));
  long long g = static_cast<long long>(device_cus()) * per_cu;
  if (tiles_ub < g) g = tiles_ub;
  g = (g + 7) / 8 * 8;
  if (g < 8) g = 8;
  return static_cast<int>(g);
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_expert_ffn(const void* rows, const int32_t* group_offsets, int G,
                                     const int32_t* row_gather, const int32_t* gather_base,
                                     int max_rows, const void* w_gate_up, const void* w_down,
                                     int H, int I, int dtype, void* h, void* y, int n_shared,
                                     const void* shared_x, int M_sh,
                                     const void* shared_w_gate_up, const void* shared_w_down,
                                     void* shared_h, void* shared_y, int phases,
                                     void* stream) {
  const bool bf = dtype == MOE_BF16;
  const int tile_n = bf ? kBN : kFN;
  const int tile_k = bf ? kBK : kFK;
  if ((dtype != MOE_F32 && !bf) || G < 0 || G > MOE_MAX_EXPERTS || n_shared < 0 ||
      n_shared > 16 || max_rows < 0 || H <= 0 || I <= 0 || H % tile_n || I % tile_n ||
      H % tile_k || I % tile_k || (n_shared > 0 && M_sh < 0) || G + n_shared == 0 ||
      phases < MOE_FFN_GATE_UP || phases > MOE_FFN_ALL) {
    moe_host::set_error("moe_expert_ffn: invalid shape (bf16 needs H, I multiples of 128; f32 "
                        "multiples of 64)");
    return MOE_EINVAL;
  }
  if ((G > 0 && (!rows || !group_offsets || !w_gate_up || !w_down || !h || !y)) ||
      (n_shared > 0 && (!shared_x || !shared_w_gate_up || !shared_w_down || !shared_h ||
                        !shared_y))) {
    moe_host::set_error("moe_expert_ffn: NULL pointer");
    return MOE_EINVAL;
  }
  const int S = n_shared > 0 ? n_shared : 0;
  const int bm = bf ? kBM : kFM;
  const long long mt_ub = (static_cast<long long>(max_rows) + bm - 1) / bm + G +
                          static_cast<long long>(S) * ((M_sh + bm - 1) / bm);
  hipStream_t st = moe_host::as_stream(stream);

  GemmArgs g1{};
  g1.a = rows;
  g1.gather = row_gather;
  g1.gather_base = gather_base;
  g1.offs = group_offsets;
  g1.G = G;
  g1.w = w_gate_up;
  g1.c = h;
  g1.S = S;
  g1.M_sh = M_sh;
  g1.a_sh = shared_x;
  g1.a_sh_stride = 0;
  g1.w_sh = shared_w_gate_up;
  g1.c_sh = shared_h;
  g1.Nn = I;
  g1.K = H;

  GemmArgs g2 = g1;
  g2.a = h;
  g2.gather = nullptr;
  g2.gather_base = nullptr;
  g2.w = w_down;
  g2.c = y;
  g2.a_sh = shared_h;
  g2.a_sh_stride = static_cast<long long>(M_sh) * I;
  g2.w_sh = shared_w_down;
  g2.c_sh = shared_y;
  g2.Nn = H;
  g2.K = I;

  const bool p1 = phases & MOE_FFN_GATE_UP, p2 = phases & MOE_FFN_DOWN;
  if (bf) {
    const long long t1 = mt_ub * (I / kBN), t2 = mt_ub * (H / kBN);
    if (p1)
      hipLaunchKernelGGL(ffn_gemm_bf16<2>, dim3(persistent_grid(ffn_gemm_bf16<2>, t1)),
                         dim3(256), 0, st, g1);
    if (p2)
      hipLaunchKernelGGL(ffn_gemm_bf16<1>, dim3(persistent_grid(ffn_gemm_bf16<1>, t2)),
                         dim3(256), 0, st, g2);
  } else {
    const long long t1 = mt_ub * (I / kFN), t2 = mt_ub * (H / kFN);
    if (p1)
      hipLaunchKernelGGL(ffn_gemm_f32<2>, dim3(persistent_grid(ffn_gemm_f32<2>, t1)), dim3(256),
                         0, st, g1);
    if (p2)
      hipLaunchKernelGGL(ffn_gemm_f32<1>, dim3(persistent_grid(ffn_gemm_f32<1>, t2)), dim3(256),
                         0, st, g2);
  }
  return moe_host::launch_status();
}
