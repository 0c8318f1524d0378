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
// host synchronisation is needed. A persistent grid walks the tiles; tiles are ordered by group,
// then by bands of 8 row tiles, column panel and row tile inside a band, and the order is dealt
// to the 8 XCDs in chunks of 32 tiles, round robin, so the workgroups of one XCD that run
// together share a few row panels and weight panels in that XCD's L2. The tiles left over for a
// last, partial step of the grid run as two half tiles each when that keeps them within it.
//
// bf16 path: MFMA 16x16x32 bf16 with fp32 accumulators (the chip is power-limited under this
// load, and the 16x16x32 form costs less energy per flop than 32x32x16: same structure, higher
// sustained clock, 7% faster on the Llama-4-Scout shape). A tile is BM rows (128, or 256 when the
// groups average 256 rows or more) by 256 weight rows (GEMM1: 128 gate and the 128 matching up
// rows; GEMM2: 256 output columns). Operands go HBM -> LDS by direct copies into a ring of K
// steps, so later steps load while one is multiplied; one barrier per K step. One wave per SIMD
// issues all the copies while its partner wave only multiplies.
// f32 path: a plain LDS-tiled FMA kernel (64 x 64 tiles) for fp32 problems.
#include <atomic>
#include <mutex>

#include "moe_internal.h"

namespace moe {

constexpr int kMaxGroups = MOE_MAX_EXPERTS + 16;
constexpr int kGemmBK = 64;           // K step of the 128-row bf16 tiles
constexpr int kGemmStages = 3;        // LDS ring depth of the 128-row tiles
constexpr int kGemmWaveRows = 32;     // rows per wave of the 128-row tiles (8 waves)
struct GemmArgs {
  const void* a;              // routed A rows (relative to offs[0], or gathered)
  const int32_t* gather;      // absolute-row indexed source row, or NULL
  const int32_t* gather_base; // device int subtracted from gather values, or NULL
  const int32_t* offs;        // [G+1]
  int G;
  const void* w;              // [G][NB*Nn][K]
  void* c;                    // [rows][Nn]: relative rows, or absolute rows when c_abs
  int c_abs;                  // 1: C row index = absolute row (a group_offsets value)
  int S, M_sh;
  const void* a_sh;
  long long a_sh_stride;      // elements between the shared groups' A blocks (0: all read one)
  const void* w_sh;           // [S][NB*Nn][K]
  void* c_sh;                 // [S][M_sh][Nn]
  int Nn, K;
  int w_packed;               // 1: weights in the packed tile order (moe_pack_weights)
};

// Packed weights (bf16): for each group, weight panel p and K step kt, the 32 KB image of the
// tile's B operand in LDS, i.e. 32 chunks q of 1 KB, lane l of chunk q holding the 8 K values
// kt * 64 + 8 ((l % 8) ^ ((r / 2) % 8)) .. + 7 of tile B-row r = 8 q + l / 8. A panel is 256
// B-rows: NB = 2, gate rows 128 p .. + 127 then the matching up rows Nn + 128 p ..; NB = 1,
// rows 256 p .. + 255. Panel p of K step kt starts at byte (p * KT + kt) * 32768 of the group.
constexpr int kPackedStep = 32768;
__device__ __forceinline__ int packed_panel_rows(int NB) { return NB == 2 ? 128 : 256; }

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

// Logical tile L -> (group, row tile, column tile). Inside a group the row tiles are cut into
// bands of kBand; a band's tiles run column-panel-major (all its row tiles of one column panel,
// then the next panel), bands one after the other. The workgroups of one XCD that run at the
// same time then share a few A row panels and a few weight panels in that XCD's L2, instead of
// each reading its own A panel from beyond the L2 (as a plain column-major walk of a tall group
// would have them do).
constexpr int kGemmBigBK = 64;        // K step of the 256-row tiles
constexpr int kGemmBigStages = 2;     // LDS ring depth of the 256-row tiles
constexpr int kGemmBigMW = 64;        // rows per wave of the 256-row tiles (8 waves)
constexpr int kGemmBigRows = 256;     // 256-row tiles from this many rows per group
// Waves that issue the HBM -> LDS copies: one per SIMD (waves 0-3); while the copy issue of one
// wave waits on the address unit, its SIMD partner keeps the matrix core busy.
constexpr int kGemmCopyWaves = 4;
constexpr int kBand = 8;
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
  const int b = q / (kBand * NT);                  // band
  const int hb = min(kBand, mtg - b * kBand);      // row tiles in this band
  const int r = q - b * kBand * NT;
  nt = r / hb;
  mt = b * kBand + (r - nt * hb);
}

// Logical tile for this block's it-th step; -1 when done. Block b runs on XCD b % 8. The tile
// order is dealt to the XCDs in chunks of c consecutive tiles, round robin, c = the XCD's block
// count capped at kXcdChunk: the workgroups of an XCD run one chunk together (a block of row
// tiles and column panels that share operands in that XCD's L2), and every XCD gets a share of
// every part of the order, so groups whose weights stream from HBM and groups that hit in L2
// spread over all XCDs (a contiguous eighth per XCD left the XCDs with the streaming groups last
// to finish: Llama-4-Scout gate/up 2714 -> 2461 us with chunks of 32). A small grid takes chunks
// of its own block count per XCD, so a launch of a few dozen tiles spreads over all eight XCDs
// in one round. Each XCD walks its chunks in increasing order, so the first tile past the end
// ends its blocks. The grid is a multiple of 8.
constexpr int kXcdChunk = 32;
__device__ __forceinline__ int next_tile(int T, int it) {
  const int xcd = blockIdx.x & 7;
  const int per_xcd = gridDim.x >> 3;
  const int c = per_xcd < kXcdChunk ? per_xcd : kXcdChunk;
  const int local = (blockIdx.x >> 3) + it * per_xcd;
  const int L = ((local / c) * 8 + xcd) * c + local % c;
  return L < T ? L : -1;
}

// With half tiles: step it covers tiles it * G .. it * G + G - 1 of the order (G = gridDim.x),
// so the last step holds the r = T mod G tiles left over, and without more the blocks that get
// none wait a whole tile for the others (the Llama-4-Scout-shaped gate/up launch has 4672
// tiles: 18 full steps on 256 blocks and 64 tiles in a 19th). When r <= G / 2, each of those
// tiles runs as its two halves (rows 0-127 and 128-255, as a group's last half tile does) on two
// blocks of one XCD, so the last step takes about half a tile (when r is at most 8 times the
// pairs of blocks per XCD). sub: -1 the whole tile, 0 or 1 a half.
__device__ __forceinline__ int next_tile_split(int T, int it, int& sub) {
  sub = -1;
  const int G = gridDim.x;
  const int full = T / G, r = T - full * G;
  // (a step is a contiguous run of the order only while an XCD's chunk is its block count)
  if (it == full && r > 0 && r <= 8 * ((G >> 3) >> 1) && (G >> 3) <= kXcdChunk) {
    const int s = blockIdx.x >> 3;             // block s of XCD blockIdx.x % 8
    const int u = (blockIdx.x & 7) + 8 * (s >> 1);
    if (u >= r) return -1;
    sub = s & 1;
    return full * G + u;
  }
  return next_tile(T, it);
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
    t.c = static_cast<char*>(p.c) +
          static_cast<size_t>(p.c_abs ? t.abs0 : t.rel0) * p.Nn * sizeof(T);
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
// Same with the hardware reciprocal (1 ulp) in place of the IEEE division, for bf16 outputs.
__device__ __forceinline__ float silu_fast(float g) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g));
}

// ------------------------------------------------------------------------------------------
// bf16 MFMA path
// ------------------------------------------------------------------------------------------
// Tile: BM rows x 64 NBLK B rows; BM / MW x 2 waves, each owning MW rows and 32 NBLK B rows.
// Operands go HBM -> LDS directly (global_load_lds_dwordx4: lane l of a wave writes 16 bytes at
// LDS base + 16 l) through an S-stage ring, S - 1 steps of copies in flight while one step is
// multiplied. A ring stage holds (BM + 64 NBLK) rows of 2 BK bytes: 128-row tiles (BK = 64,
// S = 3) take 144 KB, 256-row tiles (BK = 64, S = 2) 128 KB, so one workgroup runs per CU.
//
// LDS rows hold one operand row's BK values (2 BK bytes, CPR = 2 BK / 16 chunks of 16 bytes);
// chunk c of row r sits at slot c ^ swz(r), with swz(r) = (r / 2) % 8 for 128-byte rows and
// (r / 4) % 4 for 64-byte rows. A fragment read has lane l read row 16 b + l % 16 at chunk
// c + l / 16, so each quarter wave reads 16 consecutive rows at one chunk: with (r / 2) % 8 the
// 16 rows' (r % 2, slot) pairs are distinct, i.e. the quarter wave's 256 bytes cover the 64
// banks once (free of LDS bank conflicts; checked with the SQ_LDS_BANK_CONFLICT counter).


template <int NB, int NBLK, int BK, int BM, int MW = 64>
struct Bf16Tile {
  static constexpr int kBM = BM;                        // rows per tile (128 or 256)
  static constexpr int kMW = MW;                        // rows per wave (32 or 64)
  static constexpr int kMB = MW / 16;                   // 16-row MFMA blocks of A per wave
  static constexpr int kNB = 2 * NBLK;                  // 16-row MFMA blocks of B per wave
  static constexpr int kWaves = (BM / MW) * 2;          // compute waves: BM / MW x 2
  static constexpr int kRowB = BK * 2;                  // LDS bytes per operand row
  static constexpr int kCpr = kRowB / 16;               // 16-byte chunks per row
  static constexpr int kRowsPerKB = 1024 / kRowB;       // rows one DMA instruction fills
  static constexpr int kBRows = 64 * NBLK;              // B rows per tile (2 waves x NBLK x 32)
  static constexpr int kStageA = BM * kRowB;
  static constexpr int kStageB = kBRows * kRowB;
  // waves that issue the copies: one per SIMD (waves 0-3) or all
  static constexpr int kIssuers = kGemmCopyWaves;
  static_assert(kWaves >= kIssuers, "one copy wave per SIMD");
  static constexpr int kDmaA = kStageA / 1024 / kIssuers;  // copies per issuing wave per stage
  static constexpr int kDmaB = kStageB / 1024 / kIssuers;
  static constexpr int kCols = NB == 2 ? kBRows / 2 : kBRows;  // output columns per tile
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kStages = BM == 256 ? kGemmBigStages : kGemmStages;  // LDS ring depth
  // 256-row tiles with one copy wave per SIMD run a group's last tile of <= 128 rows as a half
  // tile: the copy waves only copy (A rows 0-127 and B), their partners do the whole tile
  static constexpr bool kHalfTiles = BM == 256 && MW == 64 && kIssuers == 4;
  __device__ static constexpr int swz(int r) { return kCpr == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
};

// Geometry of one tile as both kinds of wave need it. half: a 256-row tile with at most 128
// rows inside its group (the last tile of a group), worked as a 128-row tile (see below).
struct TilePos {
  TileGeom tg;
  int m0, n0;
  bool half;
};

template <typename TT, int NB>
__device__ __forceinline__ bool tile_at(const GemmArgs& p, const int* mt_pre, int ng, int NT,
                                        int T, int it, TilePos& tp) {
  int sub = -1;
  const int L = TT::kHalfTiles ? next_tile_split(T, it, sub) : next_tile(T, it);
  if (L < 0) return false;
  int g, mt, nt;
  decode_tile(mt_pre, ng, NT, L, g, mt, nt);
  // the decode reads LDS, so the compiler cannot tell these are the same in every lane
  g = __builtin_amdgcn_readfirstlane(g);
  mt = __builtin_amdgcn_readfirstlane(mt);
  nt = __builtin_amdgcn_readfirstlane(nt);
  tp.tg = tile_geom<bf16_t, NB>(p, g);
  tp.m0 = mt * TT::kBM;
  tp.n0 = nt * TT::kCols;
  if (sub >= 0) {          // half of a tile of the last step (a half tile has no second half)
    if (sub == 1 && tp.tg.rows - tp.m0 <= TT::kBM / 2) return false;
    tp.m0 += sub * (TT::kBM / 2);
    tp.half = true;
    return true;
  }
  tp.half = TT::kHalfTiles && tp.tg.rows - tp.m0 <= TT::kBM / 2;
  return true;
}

// Weight (B) row wr of the tile's b-th B row.
template <typename TT, int NB>
__device__ __forceinline__ int b_weight_row(const GemmArgs& p, int n0, int rb) {
  if (NB == 2) return rb < TT::kBRows / 2 ? n0 + rb : p.Nn + n0 + rb - TT::kBRows / 2;
  return n0 + rb;
}

// Epilogue of a bf16 tile: the MFMAs take the weight fragment as their first operand, so in
// block acc[i][j] lane l holds tile row 16 i + l % 16 and the four adjacent output columns
// 16 j + 4 (l / 16) .. + 3, written as one 8-byte store. NB = 2: blocks j and j + NBX / 2 are
// the gate and up values of the same columns, h = silu(g) u.
template <int NB, int MB, int NBX, int MW>
__device__ __forceinline__ void store_tile(const f32x4 (&acc)[MB][NBX], const TileGeom& tg,
                                           int m0, int n0, int Nn, int wm, int wn, int l) {
  bf16_t* C = reinterpret_cast<bf16_t*>(tg.c);
  constexpr int JO = NB == 2 ? NBX / 2 : NBX;          // output column blocks per wave
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int m = m0 + wm * MW + i * 16 + (l & 15);
    if (m >= tg.rows) continue;
    bf16_t* crow = C + static_cast<size_t>(m) * Nn + n0 + wn * JO * 16 + (l >> 4) * 4;
#pragma unroll
    for (int j = 0; j < JO; ++j) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = NB == 2 ? silu_fast(acc[i][j][e]) * acc[i][j + JO][e] : acc[i][j][e];
      const bf16x2 lo = {static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1])};
      const bf16x2 hi = {static_cast<__bf16>(v[2]), static_cast<__bf16>(v[3])};
      *reinterpret_cast<u32x2*>(crow + j * 16) =
          u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
    }
  }
}

// Tile: BM rows x (64 NBLK) B rows; wave (wm, wn) owns rows wm*MW .. + MW - 1 (MW / 16 blocks of
// 16 rows) and 2 NBLK 16-row blocks of B rows (NB = 2: NBLK gate blocks and the matching up
// blocks), accumulated with v_mfma_f32_16x16x32_bf16. Operand fragment of a 16 x 32 block: lane l
// holds row l % 16 and the 8 K values starting at 8 (l / 16).

template <int NB, int NBLK, int BK, int BM, int MW>
__global__ __launch_bounds__((Bf16Tile<NB, NBLK, BK, BM, MW>::kThreads)) void ffn_gemm_bf16(
    GemmArgs p) {
  using TT = Bf16Tile<NB, NBLK, BK, BM, MW>;
  constexpr int MB = TT::kMB;
  constexpr int NBX = TT::kNB;
  constexpr int RB = TT::kRowB;
  constexpr int KS = BK / 32;                            // MFMA K steps per stage
  __shared__ int mt_pre[kMaxGroups + 1];
  constexpr int S = TT::kStages;
  __shared__ __attribute__((aligned(1024))) char ringA[S * TT::kStageA];
  __shared__ __attribute__((aligned(1024))) char ringB[S * TT::kStageB];

  build_tile_prefix<BM>(p, mt_pre);
  const int ng = p.G + p.S;
  const int NT = p.Nn / TT::kCols;
  const int T = mt_pre[ng] * NT;
  const int gbase = (p.gather && p.gather_base) ? *p.gather_base : 0;

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int KT = p.K / BK;

  const int wm = w >> 1, wn = w & 1;
  const size_t krow = static_cast<size_t>(p.K) * 2;     // bytes per operand row in HBM
  // DMA: lane l fills LDS slot l % CPR of row (rows per KB) q + l / CPR, so it copies chunk
  // (l % CPR) ^ swz(row) of that operand row
  const int dma_row = l / TT::kCpr;
  // fragment reads: row = 16-aligned base + l % 16, chunk = 4 s + l / 16 at slot chunk ^ swz
  const int fswz = TT::swz(l & 15);
  int b_row_off[NBX];
#pragma unroll
  for (int j = 0; j < NBX; ++j) {
    int rb;
    if (NB == 2)
      rb = (j < NBX / 2 ? 0 : TT::kBRows / 2) + wn * (NBX / 2) * 16 + (j % (NBX / 2)) * 16;
    else
      rb = wn * NBX * 16 + j * 16;
    b_row_off[j] = (rb + (l & 15)) * RB;
  }

  // per-lane byte offsets of a tile's copies from its (wave-uniform) operand bases; operands
  // stay below 4 GB (checked by the host)
  const char* abase;
  const char* bbase;
  uint32_t ga[TT::kDmaA], gb[TT::kDmaB];
  const bool issuer = w < TT::kIssuers;
  // A copies of a half tile: kDmaA / 2 per issuing wave, rows 0-127
  int dma_a0 = w * TT::kDmaA;                           // this wave's first A copy block
  bool half = false;
  auto setup = [&](const TilePos& t) {
    abase = uniform_ptr(t.tg.a);
    bbase = uniform_ptr(t.tg.w);
    half = t.half;
    dma_a0 = w * (half ? TT::kDmaA / 2 : TT::kDmaA);
    if (!issuer) return;
#pragma unroll
    for (int i = 0; i < TT::kDmaA; ++i) {
      if (half && i >= TT::kDmaA / 2) break;
      const int r = (dma_a0 + i) * TT::kRowsPerKB + dma_row;
      int m = t.m0 + r;
      if (m >= t.tg.rows) m = t.tg.rows - 1;        // rows past the group: any valid row
      ga[i] = static_cast<uint32_t>(a_row(p, t.tg, m, gbase) * static_cast<long long>(krow)) +
              ((l % TT::kCpr) ^ TT::swz(r)) * 16;
    }
    if (p.w_packed) {   // the tile's B image of K step kt is 32 KB at bbase + kt * 32 KB
      static_assert(TT::kStageB == kPackedStep || NB == 1, "packed panels are 256 B-rows");
      bbase = uniform_ptr(t.tg.w + static_cast<size_t>(t.n0 / TT::kCols) * KT * kPackedStep);
#pragma unroll
      for (int i = 0; i < TT::kDmaB; ++i) gb[i] = (w * TT::kDmaB + i) * 1024 + 16 * l;
      return;
    }
#pragma unroll
    for (int i = 0; i < TT::kDmaB; ++i) {
      const int rb = (w * TT::kDmaB + i) * TT::kRowsPerKB + dma_row;
      gb[i] = static_cast<uint32_t>(b_weight_row<TT, NB>(p, t.n0, rb)) *
                  static_cast<uint32_t>(krow) + ((l % TT::kCpr) ^ TT::swz(rb)) * 16;
    }
  };
  // this wave's LDS destinations inside a ring slot (wave-uniform byte addresses)
  const uint32_t ldsA = lds_addr(ringA);
  const uint32_t ldsB = lds_addr(ringB) + w * TT::kDmaB * 1024;
  auto issue = [&](int kt) {
    if (!issuer) return;
    const char* ak = abase + kt * RB;
    const char* bk = bbase + kt * (p.w_packed ? kPackedStep : RB);
    const int slot = kt % S;
#pragma unroll
    for (int i = 0; i < TT::kDmaA; ++i) {
      if (half && i >= TT::kDmaA / 2) break;
      dma16(ak, ga[i], ldsA + slot * TT::kStageA + (dma_a0 + i) * 1024);
    }
#pragma unroll
    for (int i = 0; i < TT::kDmaB; ++i) dma16(bk, gb[i], ldsB + slot * TT::kStageB + i * 1024);
  };
  // the ring holds S steps: a tile's steps 0 .. S-1 go out first; at the barrier inside step kt
  // (all waves have read step kt into registers) its slot takes step kt + S
  auto prologue = [&]() {
#pragma unroll
    for (int k0 = 0; k0 < S; ++k0)
      if (k0 < KT) issue(k0);
  };

  TilePos tp;
  if (!tile_at<TT, NB>(p, mt_pre, ng, NT, T, 0, tp)) return;
  setup(tp);
  prologue();
  for (int it = 0;; ++it) {
    // half tile: waves 4-7 (the partners of the copy waves) compute rows 0-127 as a 2 x 2
    // arrangement of the usual 64 x 128 wave tiles; waves 0-3 only copy
    const bool computes = !half || w >= 4;
    const int wmt = half ? (wm & 1) : wm;
    int a_row_off[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) a_row_off[i] = (wmt * MW + i * 16 + (l & 15)) * RB;
    f32x4 acc[MB][NBX];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NBX; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][j][q] = 0.f;

    constexpr int kPer = TT::kDmaA + TT::kDmaB;        // copies per stage per lane
    constexpr int kPerHalf = TT::kDmaA / 2 + TT::kDmaB;  // the same in a half tile
    // Fragment of A block i / B block j of K sub-step ks (32 deep) of step kt: lane l reads row
    // 16 i + l % 16 (16 j + l % 16) at chunk 4 ks + l / 16, slot chunk ^ swz.
    auto frag_a = [&](int i, int kt, int ks) {
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
          ringA + (kt % S) * TT::kStageA + a_row_off[i] + ((ks * 4 + (l >> 4)) ^ fswz) * 16));
    };
    auto frag_b = [&](int j, int kt, int ks) {
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
          ringB + (kt % S) * TT::kStageB + b_row_off[j] + ((ks * 4 + (l >> 4)) ^ fswz) * 16));
    };
    // wait until this lane's copies of a K step are done while `young` later steps' copies may
    // still be in flight, and its LDS reads have returned; then publish to all waves: after the
    // barrier every wave's reads of older steps are complete. Copies complete in issue order
    // among themselves; epilogue stores of the previous tile may also be counted, which only
    // makes the wait longer.
    auto arrive = [&](int young) {
      // a wave that issues no copies has none to wait for (its own epilogue stores need not
      // drain); the barrier orders it after the issuing waves' waits
      if (!issuer) wait_lgkm0();
      else if (young >= 3 && half) wait_vm_lgkm<3 * kPerHalf>();
      else if (young >= 3) wait_vm_lgkm<3 * kPer>();
      else if (young == 2 && half) wait_vm_lgkm<2 * kPerHalf>();
      else if (young == 2) wait_vm_lgkm<2 * kPer>();
      else if (young == 1 && half) wait_vm_lgkm<kPerHalf>();
      else if (young == 1) wait_vm_lgkm<kPer>();
      else wait_vm_lgkm<0>();
      raw_barrier();
    };

    arrive(min(S - 1, KT - 1));
    if (!computes) {
      // copy wave of a half tile: the same barriers and copies as the loop below
      for (int kt = 0; kt + 1 < KT; ++kt) {
        arrive(min(S - 2, KT - 2 - kt));
        if (kt + S < KT) issue(kt + S);
      }
    }
    // The current sub-step's fragments: A blocks fa (the next sub-step's are read into na at its
    // start) and B blocks fb, each re-read for the next sub-step right after its last MFMA, so
    // only A is held twice. The barrier of K step kt + 1 sits inside step kt, before its last
    // sub-step, so the next step's first fragments load while the last sub-step multiplies.
    // After a tile's last sub-step the reads fetch a valid ring slot whose values go unused
    // (they keep the reads and MFMAs in one scheduling region). The compiler places the reads
    // among the MFMAs itself: it issues them in a cluster and waits for each fragment just before
    // its first MFMA, which measured about 1% faster than a fixed interleave of one read per
    // group of MFMAs.
    bf16x8 fa[MB], fb[NBX];
    if (computes) {
#pragma unroll
      for (int i = 0; i < MB; ++i) fa[i] = frag_a(i, 0, 0);
#pragma unroll
      for (int j = 0; j < NBX; ++j) fb[j] = frag_b(j, 0, 0);
    }
    for (int kt = 0; computes && kt < KT; ++kt) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bool last = ks + 1 == KS;
        const int nkt = last ? kt + 1 : kt, nks = last ? 0 : ks + 1;   // the next sub-step
        if (last && nkt < KT) {
          arrive(min(S - 2, KT - 2 - kt));   // step kt+1 landed; every wave is done with step kt
          if (kt + S < KT) issue(kt + S);
        }
        bf16x8 na[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) na[i] = frag_a(i, nkt, nks);
#pragma unroll
        for (int j = 0; j < NBX; ++j) {
#pragma unroll
          for (int i = 0; i < MB; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
          fb[j] = frag_b(j, nkt, nks);
        }
#pragma unroll
        for (int i = 0; i < MB; ++i) fa[i] = na[i];
      }
    }

    // every wave is done reading the ring: the next tile's first steps go out now and land
    // while this tile's epilogue runs
    const TileGeom tg = tp.tg;
    const int m0 = tp.m0, n0 = tp.n0;
    const bool more = tile_at<TT, NB>(p, mt_pre, ng, NT, T, it + 1, tp);
    wait_lgkm0();
    raw_barrier();
    if (more) {
      setup(tp);
      prologue();
    }

    if (computes) store_tile<NB, MB, NBX, MW>(acc, tg, m0, n0, p.Nn, wmt, wn, l);
    if (!more) break;
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
// Per-device compute unit counts and per-(device, kernel) occupancy, queried once and cached;
// the caches are shared by all host threads and guarded by one mutex.
static std::mutex g_cache_mu;
static int g_cus[64];

static int device_cus() {
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= 64) return 256;
  std::lock_guard<std::mutex> lock(g_cache_mu);
  if (!g_cus[d]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess ||
        n <= 0)
      n = 256;
    g_cus[d] = n;
  }
  return g_cus[d];
}

// Blocks per CU that fit (the occupancy query is not free).
static int blocks_per_cu(const void* kernel, int threads) {
  struct Entry {
    int dev;
    const void* kernel;
    int per_cu;
  };
  static Entry cache[64];
  static int n = 0;
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess) d = -1;
  std::lock_guard<std::mutex> lock(g_cache_mu);
  for (int i = 0; i < n; ++i)
    if (cache[i].dev == d && cache[i].kernel == kernel) return cache[i].per_cu;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  if (n < 64) cache[n++] = Entry{d, kernel, per_cu};
  return per_cu;
}

// Compute units the persistent GEMM grids may use (0: all), set by moe_set_gemm_max_cus.
static std::atomic<int> g_gemm_max_cus{0};

template <typename K>
static int persistent_grid(K kernel, int threads, long long tiles_ub) {
  const int per_cu = blocks_per_cu(reinterpret_cast<const void*>(kernel), threads);
  int cus = device_cus();
  const int cap = g_gemm_max_cus.load(std::memory_order_relaxed);
  if (cap > 0 && cap < cus) cus = cap / 8 * 8 < 8 ? 8 : cap / 8 * 8;
  long long g = static_cast<long long>(cus) * per_cu;
  if (tiles_ub < g) g = tiles_ub;
  g = (g + 7) / 8 * 8;
  if (g < 8) g = 8;
  return static_cast<int>(g);
}

template <int BM, int BK, int MW>
static void launch_bf16(const GemmArgs& g1, const GemmArgs& g2, int G, int S, int M_sh,
                        int max_rows, int H, int I, bool p1, bool p2, hipStream_t st) {
  const long long mt_ub = (static_cast<long long>(max_rows) + BM - 1) / BM + G +
                          static_cast<long long>(S) * ((M_sh + BM - 1) / BM);
  using T1 = Bf16Tile<2, 4, BK, BM, MW>;
  if (p1)
    hipLaunchKernelGGL((ffn_gemm_bf16<2, 4, BK, BM, MW>),
                       dim3(persistent_grid(ffn_gemm_bf16<2, 4, BK, BM, MW>, T1::kThreads,
                                            mt_ub * (I / T1::kCols))),
                       dim3(T1::kThreads), 0, st, g1);
  if (!p2) return;
  if (H % 256 == 0) {
    using T2 = Bf16Tile<1, 4, BK, BM, MW>;
    hipLaunchKernelGGL((ffn_gemm_bf16<1, 4, BK, BM, MW>),
                       dim3(persistent_grid(ffn_gemm_bf16<1, 4, BK, BM, MW>, T2::kThreads,
                                            mt_ub * (H / T2::kCols))),
                       dim3(T2::kThreads), 0, st, g2);
  } else {
    using T2 = Bf16Tile<1, 2, BK, BM, MW>;
    hipLaunchKernelGGL((ffn_gemm_bf16<1, 2, BK, BM, MW>),
                       dim3(persistent_grid(ffn_gemm_bf16<1, 2, BK, BM, MW>, T2::kThreads,
                                            mt_ub * (H / T2::kCols))),
                       dim3(T2::kThreads), 0, st, g2);
  }
}

}  // namespace moe

namespace moe {

__global__ __launch_bounds__(256) void pack_weights_kernel(const u32x4* __restrict__ w, int NB,
                                                           int Nn, int K, long long items,
                                                           u32x4* __restrict__ out) {
  const int KT = K / 64;
  const int prow = NB == 2 ? 128 : 256;
  const int panels = Nn / prow;
  const long long R = static_cast<long long>(NB) * Nn;
  for (long long idx = blockIdx.x * 256ll + threadIdx.x; idx < items;
       idx += static_cast<long long>(gridDim.x) * 256) {
    const int l = static_cast<int>(idx & 63);
    const int q = static_cast<int>((idx >> 6) & 31);
    long long rest = idx >> 11;
    const int kt = static_cast<int>(rest % KT);
    rest /= KT;
    const int pnl = static_cast<int>(rest % panels);
    const long long g = rest / panels;
    const int r = 8 * q + (l >> 3);                     // tile B-row
    const int row = NB == 2 ? (r < 128 ? 128 * pnl + r : Nn + 128 * pnl + r - 128)
                            : 256 * pnl + r;
    const int chunk = (l & 7) ^ ((r >> 1) & 7);
    out[idx] = w[((g * R + row) * K + kt * 64 + chunk * 8) / 8];
  }
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_set_gemm_max_cus(int n) {
  if (n < 0) {
    moe_host::set_error("moe_set_gemm_max_cus: n must be >= 0 (0 = every compute unit)");
    return MOE_EINVAL;
  }
  g_gemm_max_cus.store(n, std::memory_order_relaxed);
  return MOE_OK;
}

extern "C" moe_status moe_pack_weights(const void* w, int G, int NB, int Nn, int K, void* out,
                                       void* stream) {
  if (G < 0 || (NB != 1 && NB != 2) || Nn <= 0 || K <= 0 || K % 64 ||
      Nn % (NB == 2 ? 128 : 256)) {
    moe_host::set_error("moe_pack_weights: invalid shape (K % 64, and Nn % 128 for gate/up or "
                        "Nn % 256 for down)");
    return MOE_EINVAL;
  }
  if (G == 0) return MOE_OK;
  if (!w || !out || w == out) {
    moe_host::set_error("moe_pack_weights: NULL or in-place pointer");
    return MOE_EINVAL;
  }
  const long long items = static_cast<long long>(G) * NB * Nn * K / 8;
  long long blocks = (items + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(pack_weights_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     moe_host::as_stream(stream), static_cast<const u32x4*>(w), NB, Nn, K, items,
                     static_cast<u32x4*>(out));
  return moe_host::launch_status();
}

extern "C" moe_status moe_expert_ffn(const void* rows, const int32_t* group_offsets, int G,
                                     const int32_t* row_gather, const int32_t* gather_base,
                                     int max_rows, const void* w_gate_up, const void* w_down,
                                     int H, int I, int dtype, void* h, void* y,
                                     int y_absolute, int n_shared,
                                     const void* shared_x, int M_sh,
                                     const void* shared_w_gate_up, const void* shared_w_down,
                                     void* shared_h, void* shared_y, int phases,
                                     int weights_packed, void* stream) {
  const bool bf = dtype == MOE_BF16;
  const int tile_n = bf ? 128 : kFN;
  const int tile_k = bf ? 64 : kFK;
  if ((dtype != MOE_F32 && !bf) || G < 0 || G > MOE_MAX_EXPERTS || n_shared < 0 ||
      n_shared > 16 || max_rows < 0 || H <= 0 || I <= 0 || H % tile_n || I % tile_n ||
      H % tile_k || I % tile_k || (n_shared > 0 && M_sh < 0) || G + n_shared == 0 ||
      phases < MOE_FFN_GATE_UP || phases > MOE_FFN_ALL) {
    moe_host::set_error("moe_expert_ffn: invalid shape (bf16 needs H, I multiples of 128; f32 "
                        "multiples of 64)");
    return MOE_EINVAL;
  }
  if (weights_packed && (!bf || I % 128 || H % 256)) {
    moe_host::set_error("moe_expert_ffn: packed weights need bf16, I % 128 == 0 and "
                        "H % 256 == 0");
    return MOE_EINVAL;
  }
  if ((G > 0 && (!rows || !group_offsets || !w_gate_up || !w_down || !h || !y)) ||
      (n_shared > 0 && (!shared_x || !shared_w_gate_up || !shared_w_down || !shared_h ||
                        !shared_y))) {
    moe_host::set_error("moe_expert_ffn: NULL pointer");
    return MOE_EINVAL;
  }
  // the bf16 kernels address each operand block with 32-bit byte offsets
  const long long kmax = H > I ? H : I;
  if (bf && ((static_cast<long long>(max_rows) + 1) * kmax * 2 > 0xFFFFFFFFll ||
             (static_cast<long long>(M_sh) + 1) * kmax * 2 > 0xFFFFFFFFll ||
             2ll * I * H * 2 > 0xFFFFFFFFll)) {
    moe_host::set_error("moe_expert_ffn: a bf16 operand block reaches 4 GiB (rows x max(H, I) "
                        "or one expert's weights)");
    return MOE_EINVAL;
  }
  const int S = n_shared > 0 ? n_shared : 0;
  const int bm = kFM;
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
  g1.w_packed = weights_packed ? 1 : 0;

  GemmArgs g2 = g1;
  g2.a = h;
  g2.gather = nullptr;
  g2.gather_base = nullptr;
  g2.w = w_down;
  g2.c = y;
  g2.c_abs = y_absolute ? 1 : 0;
  g2.a_sh = shared_h;
  g2.a_sh_stride = static_cast<long long>(M_sh) * I;
  g2.w_sh = shared_w_down;
  g2.c_sh = shared_y;
  g2.Nn = H;
  g2.K = I;

  const bool p1 = phases & MOE_FFN_GATE_UP, p2 = phases & MOE_FFN_DOWN;
  if (bf) {
    // 256-row tiles (8 waves, 33% fewer operand bytes per flop) when groups are large enough
    // on average that padding the last row tile costs little; 128-row tiles otherwise
    const long long rows_total = static_cast<long long>(max_rows) + static_cast<long long>(S) * M_sh;
    const bool big = rows_total >= static_cast<long long>(kGemmBigRows) * (G + S);
    if (big)
      launch_bf16<256, kGemmBigBK, kGemmBigMW>(g1, g2, G, S, M_sh, max_rows, H, I, p1, p2, st);
    else
      launch_bf16<128, kGemmBK, kGemmWaveRows>(g1, g2, G, S, M_sh, max_rows, H, I,
                                                               p1, p2, st);
  } else {
    const long long t1 = mt_ub * (I / kFN), t2 = mt_ub * (H / kFN);
    if (p1)
      hipLaunchKernelGGL(ffn_gemm_f32<2>, dim3(persistent_grid(ffn_gemm_f32<2>, 256, t1)), dim3(256),
                         0, st, g1);
    if (p2)
      hipLaunchKernelGGL(ffn_gemm_f32<1>, dim3(persistent_grid(ffn_gemm_f32<1>, 256, t2)), dim3(256),
                         0, st, g2);
  }
  return moe_host::launch_status();
}
