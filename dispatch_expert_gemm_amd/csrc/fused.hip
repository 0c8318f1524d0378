// The whole layer in one persistent launch, for small batches (decode: N <= 1024 tokens,
// N k <= 4096 slots).
//
// Blog "Kernel fusion for expert parallelism", section "Fusing the layer into one kernel": one
// kernel runs the stages route, group, MatMul (gate, up), SwiGLU, MatMul (down) and reduce, so
// that no stage pays a launch or a round trip through the host; its "Results" section finds the
// gain largest for small batches, where those fixed costs are a large share of the layer.
// FarSkip-Collective section 2.1: out[t] = sum_j w[t, j] FFN_e(x_t) + sum_s FFN_s(x_t).
//
// One workgroup per compute unit (all of them resident, which the stage waits rely on), 256
// threads. Stages, separated by device-wide barriers:
//   R   route: tokens dealt to the workgroups; route_token, the code moe_route runs, so the
//       selection is bit-identical to moe_route's. When N times the lanes per token is at most
//       1024 (four passes of a workgroup), every workgroup routes every token into its own LDS
//       instead, and barrier 1 is not needed.
//   --- barrier 1
//   L   layout, in every workgroup's LDS (no barrier needed after it): per-expert counts and
//       offsets, and each routed row's token in (expert, token) order, by the per-wave bit mask
//       counting of the dispatch layout (deterministic).
//   G1  gate/up + SwiGLU items (group, up to 64 rows, 128 columns of h): the rows' x are gathered
//       straight from x into the LDS operand tile (the "group" stage and the permute become the
//       operand gather); h goes to the workspace.
//   --- barrier 2
//   G2  down items (group, up to 64 rows, 128 columns of y), A = h.
//   --- barrier 3
//   C   combine: out[t] = sum_j w[t, j] y[row(t, j)] + sum_s y_s[t], fp32 in slot order.
// The barriers are counters in device memory: a workgroup publishes its writes (a device-scope
// release), counts itself in its group (per XCD) and spins (with a sleep) until every group has
// arrived. A spin gives up after kFusedSpinLimit rounds, sets the error flag and the workgroup
// leaves, so the kernel always exits. The last workgroup to leave returns the counters to zero
// for the next launch.
//
// GEMM items: 4 waves, wave w owns 32 output columns; up to 2 row tiles of 32 rows, accumulated
// with v_mfma_f32_32x32x16_bf16 (bf16) or v_mfma_f32_32x32x2_f32 (fp32) in fp32. Each weight row is
// used by one wave only, so its fragments are loaded from global memory straight into registers
// (64 contiguous bytes per lane per K step, a ring of kFusedDepth K steps in flight); the A rows,
// shared by the 4 waves, go through LDS (two buffers, one K step ahead). The number of row tiles
// is a template parameter chosen per item (1 or 2), so a decode-sized group carries only the
// accumulators it needs; larger groups take several 64-row items. Within a K step of 128 bytes per row, lane half kh of a wave
// multiplies the K values of bytes 64 kh .. 64 kh + 63 of the row (A and B the same), so each lane
// loads one contiguous 64-byte piece of its weight row.
#include <mutex>

#include "route_token.h"

namespace moe {

constexpr int kFusedThreads = 256;
constexpr int kFusedRows = 64;            // rows per GEMM item (at most 2 row tiles of 32)
constexpr int kFusedCols = 128;           // output columns per GEMM item (32 per wave)
constexpr int kFusedMaxSlots = 4096;      // N k: the layout lives in LDS
constexpr int kFusedMaxTokens = 1024;
constexpr unsigned kFusedSpinLimit = 1u << 24;   // x s_sleep 2 (~128 cycles): about 1 s

struct FusedArgs {
  const void* x;        // [N][H]
  const float* logits;  // [N][E]
  const float* bias;    // [E] or NULL
  int N, H, E, k, gate, I, S;
  int packed;           // expert weights in the packed layout (moe_pack_weights, bf16)
  int local_route;      // every workgroup routes every token into its LDS (no first barrier)
  const void* wgu;      // [E][2I][H]
  const void* wd;       // [E][H][I]
  const void* swgu;     // [S][2I][H]
  const void* swd;      // [S][H][I]
  int32_t* topk_idx;    // [N][k] out
  float* topk_w;        // [N][k] out
  void* h;              // [N k + S N][I]
  void* y;              // [N k + S N][H]
  void* out;            // [N][H]
  unsigned* sync;       // the sync words (sync_* below), the workspace's first 4 KB
};

// LDS of one workgroup, carved from dynamic shared memory.
struct FusedLds {
  int* cnt;                    // [E] rows of expert e
  int* off;                    // [E + 1] first row of expert e
  int* run;                    // [E] rows placed so far
  int* item0;                  // [E + S + 1] first GEMM item of each group (then the total)
  unsigned long long* mask;    // [4][E] per-wave expert masks
  int* row_tok;                // [N k] token of routed row r
  int* slot_row;               // [N k] row of slot t k + j
  int* tidx;                   // [N k] the selection, when every workgroup routes (else NULL)
  float* tw;                   // [N k] its weights
  char* atile;                 // [2][64 rows][128 bytes] operand tile
  int* flag;                   // [1]
};

__host__ __device__ inline size_t fused_lds(int N, int E, int k, int S, bool local, char* base,
                                            FusedLds* o) {
  size_t off = 0;
  auto take = [&](size_t bytes, size_t align) {
    off = (off + align - 1) / align * align;
    char* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  };
  FusedLds L;
  L.atile = take(2 * kFusedRows * 128, 1024);
  L.mask = reinterpret_cast<unsigned long long*>(take(size_t(4) * E * 8, 16));
  L.cnt = reinterpret_cast<int*>(take(size_t(E) * 4, 16));
  L.off = reinterpret_cast<int*>(take(size_t(E + 1) * 4, 16));
  L.run = reinterpret_cast<int*>(take(size_t(E) * 4, 16));
  L.item0 = reinterpret_cast<int*>(take(size_t(E + S + 1) * 4, 16));
  L.row_tok = reinterpret_cast<int*>(take(size_t(N) * k * 4, 16));
  L.slot_row = reinterpret_cast<int*>(take(size_t(N) * k * 4, 16));
  L.tidx = local ? reinterpret_cast<int*>(take(size_t(N) * k * 4, 16)) : nullptr;
  L.tw = local ? reinterpret_cast<float*>(take(size_t(N) * k * 4, 16)) : nullptr;
  L.flag = reinterpret_cast<int*>(take(16, 16));
  if (o) *o = L;
  return off;
}

// Sync words of the workspace (unsigned, each in its own 128-byte line): the arrival counters of
// the 8 workgroup groups g = blockIdx % 8 (one per XCD), the count of groups arrived, the release
// word of each group, the workgroups done, and the error flag.
constexpr int kSyncLine = 32;   // words per 128-byte line
__device__ __forceinline__ unsigned* sync_group(unsigned* s, int g) { return s + kSyncLine * g; }
__device__ __forceinline__ unsigned* sync_all(unsigned* s) { return s + kSyncLine * 8; }
__device__ __forceinline__ unsigned* sync_release(unsigned* s, int g) {
  return s + kSyncLine * (9 + g);
}
__device__ __forceinline__ unsigned* sync_done(unsigned* s) { return s + kSyncLine * 17; }
__device__ __forceinline__ unsigned* sync_error(unsigned* s) { return s + kSyncLine * 18; }
constexpr int kSyncBytes = 4 * kSyncLine * 19;

// Device-wide barrier number nth (1, 2, 3) of this launch; false when the wait gave up. Arrivals
// are counted per group of workgroups (the 256 workgroups' atomics on one word would serialize):
// the last of a group counts the group in sync_all, the workgroup that completes sync_all
// releases every group, and each workgroup polls its own group's release word.
__device__ __forceinline__ bool fused_barrier(unsigned* sync, unsigned nth, int* flag) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const int g = blockIdx.x & 7;
    const unsigned groups = gridDim.x < 8 ? gridDim.x : 8;   // groups with a workgroup
    const unsigned in_group = (gridDim.x - g + 7) / 8;
    __threadfence();   // release: this workgroup's global writes, before it is counted
    if (atomicAdd(sync_group(sync, g), 1u) + 1 == nth * in_group)
      if (atomicAdd(sync_all(sync), 1u) + 1 == nth * groups)
        for (unsigned g2 = 0; g2 < groups; ++g2) atomicExch(sync_release(sync, g2), nth);
    int ok = 1;
    unsigned spins = 0;
    // relaxed polls (an acquire per poll would invalidate this XCD's L2 each time), one acquire
    // once the group is released
    while (__hip_atomic_load(sync_release(sync, g), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
           nth) {
      if (__hip_atomic_load(sync_error(sync), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
          ++spins > kFusedSpinLimit) {
        atomicOr(sync_error(sync), 1u);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    __threadfence();   // acquire: the other workgroups' writes
    *flag = ok;
  }
  __syncthreads();
  return *flag != 0;
}

// Wave-inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int fused_wave_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

// Exclusive scan of n values (wave 0), out[n] = total. in and out may alias.
__device__ __forceinline__ void fused_scan(const int* in, int* out, int n) {
  if (threadIdx.x < kWave) {
    int carry = 0;
    for (int b = 0; b < n; b += kWave) {
      const int i = b + lane_id();
      const int v = i < n ? in[i] : 0;
      const int inc = fused_wave_scan(v);
      if (i < n) out[i] = carry + inc - v;
      carry += __shfl(inc, kWave - 1, kWave);
    }
    if (threadIdx.x == 0) out[n] = carry;
  }
}

// Stage L: counts, offsets and the routed rows in (expert, token) order.
__device__ __forceinline__ void fused_layout(const FusedArgs& a, const FusedLds& L,
                                             const int32_t* idx) {
  const int E = a.E, k = a.k, N = a.N;
  const int tid = threadIdx.x, wave = tid / kWave;
  for (int e = tid; e < E; e += kFusedThreads) {
    L.cnt[e] = 0;
    L.run[e] = 0;
  }
  __syncthreads();
  for (int i = tid; i < N * k; i += kFusedThreads) atomicAdd(&L.cnt[idx[i]], 1);
  __syncthreads();
  fused_scan(L.cnt, L.off, E);
  __syncthreads();
  const unsigned long long below = (1ull << lane_id()) - 1ull;
  for (int c0 = 0; c0 < N; c0 += kFusedThreads) {
    for (int i = tid; i < 4 * E; i += kFusedThreads) L.mask[i] = 0ull;
    __syncthreads();
    const int t = c0 + tid;
    if (t < N)
      for (int j = 0; j < k; ++j)
        atomicOr(&L.mask[wave * E + idx[t * k + j]], 1ull << lane_id());
    __syncthreads();
    if (t < N)
      for (int j = 0; j < k; ++j) {
        const int e = idx[t * k + j];
        int pos = L.off[e] + L.run[e] + __popcll(L.mask[wave * E + e] & below);
        for (int w2 = 0; w2 < wave; ++w2) pos += __popcll(L.mask[w2 * E + e]);
        L.row_tok[pos] = t;
        L.slot_row[t * k + j] = pos;
      }
    __syncthreads();
    for (int e = tid; e < E; e += kFusedThreads)
      L.run[e] += __popcll(L.mask[e]) + __popcll(L.mask[E + e]) + __popcll(L.mask[2 * E + e]) +
                  __popcll(L.mask[3 * E + e]);
    __syncthreads();
  }
}

// Items of a GEMM stage: group g (routed experts, then shared experts) has ceil(rows / 64) row
// chunks times `panels` column panels. item0[g] = first item of group g.
__device__ __forceinline__ void fused_items(const FusedArgs& a, const FusedLds& L, int panels) {
  const int ng = a.E + a.S;
  for (int g = threadIdx.x; g < ng; g += kFusedThreads) {
    const int rows = g < a.E ? L.cnt[g] : a.N;
    L.item0[g] = (rows + kFusedRows - 1) / kFusedRows * panels;
  }
  __syncthreads();
  fused_scan(L.item0, L.item0, ng);
  __syncthreads();
}

__device__ __forceinline__ int fused_group_of(const FusedLds& L, int ng, int item) {
  int lo = 0, hi = ng - 1;   // last g with item0[g] <= item
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (L.item0[mid] <= item) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

template <typename T>
struct FusedType;
template <>
struct FusedType<bf16_t> {
  static constexpr int kStep = 64;   // K values per 128-byte row piece
};
template <>
struct FusedType<float> {
  static constexpr int kStep = 32;
};

// Multiplies one 128-byte K piece: acc[n][rt] += A[rows of tile rt] x B_n (this lane's 64-byte
// half of its weight row n, b[n]), A read once per 16-byte chunk from the LDS tile `at` (128-byte
// rows, chunk c of row r at slot c ^ ((r / 2) % 8)) and used for every B.
template <typename T, int NB, int RT>
__device__ __forceinline__ void fused_mma(const char* at, const u32x4 (&b)[NB][4],
                                          f32x16 (&acc)[NB][4]) {
  const int l = lane_id();
  const int kh = l >> 5;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = 4 * kh + j;
    u32x4 av[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int r = rt * 32 + (l & 31);
      av[rt] = *reinterpret_cast<const u32x4*>(at + r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
    }
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        if constexpr (sizeof(T) == 2) {
          acc[n][rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[rt]),
                                                               __builtin_bit_cast(bf16x8, b[n][j]),
                                                               acc[n][rt], 0, 0, 0);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[n][rt] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                __uint_as_float(av[rt][q]), __uint_as_float(b[n][j][q]), acc[n][rt], 0, 0, 0);
        }
      }
  }
}

// Where each lane finds its weight fragments: the 64 bytes (lane half kh of the 128-byte K piece)
// of its weight row n (0: gate or down, 1: up) for K step kt. Plain weights: row-major rows of K
// values. Packed weights (moe_pack_weights, bf16): each K step of a 256-row panel is one 32 KB
// block holding row r's 128 bytes at r * 128, chunk c at slot c ^ ((r / 2) % 8), so the waves of a
// workgroup read whole contiguous blocks.
struct FusedB {
  const char* base;     // plain: this lane's row n = 0; packed: the panel's first K-step block
  long long up_bytes;   // plain: from row n = 0 to row n = 1
  int r0;               // packed: this lane's panel row for n = 0 (n = 1: r0 + 128)
  int packed;
};

__device__ __forceinline__ const u32x4* fused_b_ptr(const FusedB& b, int n, int kt, int kh,
                                                    int j) {
  if (!b.packed)
    return reinterpret_cast<const u32x4*>(b.base + n * b.up_bytes + kt * 128 + 64 * kh + 16 * j);
  const int r = b.r0 + 128 * n;
  return reinterpret_cast<const u32x4*>(b.base + static_cast<long long>(kt) * 32768 + r * 128 +
                                        (((4 * kh + j) ^ ((r >> 1) & 7)) << 4));
}

// One GEMM item: rows (at most 32 RT) x 128 output columns, K = K. Row i of the item reads its A
// row at a_row(i) (element offset); the weight fragments come from `wb`. Both operands run
// kFusedDepth K steps ahead in registers (rings), and the A tile of the next K step goes to LDS
// (two buffers) while the current one is multiplied. Output through store(rt, acc, column).
constexpr int kFusedDepth = 3;

template <typename T, int NB, int RT, typename ARow, typename Store>
__device__ __forceinline__ void fused_gemm_item(const T* A, ARow a_row, int rows, const FusedB& wb,
                                                int K, const FusedLds& L, Store store) {
  constexpr int KS = FusedType<T>::kStep;
  constexpr int D = kFusedDepth;
  constexpr int AU = RT;   // A copy instructions per thread: 32 RT rows of 8 chunks
  const int tid = threadIdx.x, l = lane_id(), w = tid / kWave;
  const int kh = l >> 5;
  const int KT = K / KS;
  // A copy: thread tid moves chunk tid % 8 of rows tid / 8 + 32 u, u < RT
  const int ck = tid & 7;
  long long arow[AU];
#pragma unroll
  for (int u = 0; u < AU; ++u) {
    const int r = (tid >> 3) + 32 * u;
    arow[u] = r < rows ? a_row(r) : -1;
  }
  f32x16 acc[NB][4];
#pragma unroll
  for (int n = 0; n < NB; ++n)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[n][rt][q] = 0.f;

  u32x4 aq[D][AU], bq[D][NB][4];
  auto load_a = [&](int kt, u32x4 (&dst)[AU]) {
    const int kc = kt < KT ? kt : KT - 1;   // past the end: a repeated, unused in-bounds load
#pragma unroll
    for (int u = 0; u < AU; ++u)
      dst[u] = arow[u] >= 0
                   ? *reinterpret_cast<const u32x4*>(A + arow[u] + kc * KS + ck * (16 / sizeof(T)))
                   : u32x4{0u, 0u, 0u, 0u};
  };
  auto store_a = [&](int buf, const u32x4 (&src)[AU]) {
    char* at = L.atile + buf * kFusedRows * 128;
#pragma unroll
    for (int u = 0; u < AU; ++u) {
      const int r = (tid >> 3) + 32 * u;
      *reinterpret_cast<u32x4*>(at + r * 128 + ((ck ^ ((r >> 1) & 7)) << 4)) = src[u];
    }
  };
  auto load_b = [&](int kt, u32x4 (&dst)[NB][4]) {
    const int kc = kt < KT ? kt : KT - 1;
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[n][j] = *fused_b_ptr(wb, n, kc, kh, j);
  };

#pragma unroll
  for (int d = 0; d < D; ++d) {
    load_a(d, aq[d]);
    load_b(d, bq[d]);
  }
  store_a(0, aq[0]);
  load_a(D, aq[0]);
  __syncthreads();
  // K steps in groups of D, so that each ring slot is a fixed register set. At step kt: A of
  // step kt + 1 (loaded D - 1 steps ago) goes to LDS and its slot takes step kt + 1 + D; the B
  // slot of step kt takes step kt + D.
  for (int k0 = 0; k0 < KT; k0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int kt = k0 + d;
      if (kt < KT) {
        const char* at = L.atile + (kt & 1) * kFusedRows * 128;
        fused_mma<T, NB, RT>(at, bq[d], acc);
        load_b(kt + D, bq[d]);
        if (kt + 1 < KT) {
          const int dn = d + 1 < D ? d + 1 : 0;
          store_a((kt + 1) & 1, aq[dn]);
          load_a(kt + 1 + D, aq[dn]);
        }
        __syncthreads();
      }
    }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) store(rt, acc, 32 * w + (l & 31));
}

template <typename T>
__device__ __forceinline__ void fused_put(T* p, float v);
template <>
__device__ __forceinline__ void fused_put<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void fused_put<bf16_t>(bf16_t* p, float v) { *p = f32_to_bf16(v); }

// silu(g) = g / (1 + e^-g); for bf16 outputs with the hardware reciprocal (1 ulp), whose error
// is far below the output's rounding.
template <typename T>
__device__ __forceinline__ float fused_silu(float g) {
  if constexpr (sizeof(T) == 2) return g * __builtin_amdgcn_rcpf(1.f + __expf(-g));
  else return g / (1.f + __expf(-g));
}

// Stages G1 and G2. G1 (NB = 2): h = silu(A Wg^T) * (A Wu^T) for 128 columns of h per item; G2
// (NB = 1): y = h Wd^T for 128 columns of y per item.
template <typename T, int NB>
__device__ __forceinline__ void fused_ffn_stage(const FusedArgs& a, const FusedLds& L) {
  const int N = a.N, H = a.H, I = a.I, E = a.E, k = a.k;
  const int ng = E + a.S;
  const int Nout = NB == 2 ? I : H;   // output columns
  const int K = NB == 2 ? H : I;
  const int panels = Nout / kFusedCols;
  fused_items(a, L, panels);
  const int total = L.item0[ng];
  const T* x = static_cast<const T*>(a.x);
  T* h = static_cast<T*>(a.h);
  T* y = static_cast<T*>(a.y);
  const long long nk = static_cast<long long>(N) * k;
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int g = fused_group_of(L, ng, item);
    const int rel = item - L.item0[g];
    const int chunk = rel / panels, panel = rel % panels;
    const bool routed = g < E;
    const int rows_g = routed ? L.cnt[g] : N;
    const int r0 = chunk * kFusedRows;
    const int rows = min(kFusedRows, rows_g - r0);
    // row i of the item: its output row in h / y, and its A row
    const long long first = routed ? static_cast<long long>(L.off[g]) + r0
                                   : nk + static_cast<long long>(g - E) * N + r0;
    const T* W;
    if (NB == 2)
      W = static_cast<const T*>(routed ? a.wgu : a.swgu) +
          static_cast<long long>(routed ? g : g - E) * 2 * I * H;
    else
      W = static_cast<const T*>(routed ? a.wd : a.swd) +
          static_cast<long long>(routed ? g : g - E) * H * I;
    const int c0 = panel * kFusedCols;
    // this lane's weight rows: output columns c0 + 32 w + lane % 32 (gate/up: the gate row, and
    // the up row I further on)
    const int wl = 32 * (static_cast<int>(threadIdx.x) / kWave) + (lane_id() & 31);
    FusedB wb;
    wb.packed = a.packed;
    if (!a.packed) {
      wb.base = reinterpret_cast<const char*>(W + static_cast<long long>(c0 + wl) * K);
      wb.up_bytes = static_cast<long long>(I) * H * sizeof(T);
      wb.r0 = 0;
    } else {
      // packed panels: 128 gate + 128 up rows (gate/up), 256 rows (down), K / 64 blocks each
      const int prow = NB == 2 ? 128 : 256;
      wb.base = reinterpret_cast<const char*>(W) +
                static_cast<long long>(c0 / prow) * (K / 64) * 32768;
      wb.up_bytes = 0;
      wb.r0 = c0 % prow + wl;
    }
    if constexpr (NB == 2) {
      const int* row_tok = L.row_tok + L.off[g] + r0;
      auto a_row = [=](int i) -> long long {
        const int t = routed ? row_tok[i] : r0 + i;
        return static_cast<long long>(t) * H;
      };
      T* hb = h + first * I + c0;
      auto store = [=](int rt, const f32x16 (&acc)[2][4], int col) {
        const int l = lane_id();
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int i = rt * 32 + (q >> 2) * 8 + (l >> 5) * 4 + (q & 3);
          if (i < rows) fused_put<T>(hb + i * I + col, fused_silu<T>(acc[0][rt][q]) * acc[1][rt][q]);
        }
      };
      if (rows <= 32) fused_gemm_item<T, 2, 1>(x, a_row, rows, wb, H, L, store);
      else fused_gemm_item<T, 2, 2>(x, a_row, rows, wb, H, L, store);
    } else {
      auto a_row = [=](int i) -> long long { return (first + i) * I; };
      T* yb = y + first * H + c0;
      auto store = [=](int rt, const f32x16 (&acc)[1][4], int col) {
        const int l = lane_id();
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int i = rt * 32 + (q >> 2) * 8 + (l >> 5) * 4 + (q & 3);
          if (i < rows) fused_put<T>(yb + i * H + col, acc[0][rt][q]);
        }
      };
      if (rows <= 32) fused_gemm_item<T, 1, 1>(h, a_row, rows, wb, I, L, store);
      else fused_gemm_item<T, 1, 2>(h, a_row, rows, wb, I, L, store);
    }
  }
}

// Stage C: one token per item, fp32 sum over the slots in order, then the shared experts.
template <typename T>
__device__ __forceinline__ void fused_combine(const FusedArgs& a, const FusedLds& L,
                                              const float* wts) {
  const int N = a.N, H = a.H, k = a.k;
  const T* y = static_cast<const T*>(a.y);
  T* out = static_cast<T*>(a.out);
  const long long nk = static_cast<long long>(N) * k;
  for (int t = blockIdx.x; t < N; t += gridDim.x) {
    for (int c = threadIdx.x; c < H; c += kFusedThreads) {
      float s = 0.f;
      for (int j = 0; j < k; ++j)
        s += wts[t * k + j] * load_f32<T>(y + static_cast<long long>(L.slot_row[t * k + j]) * H + c);
      for (int sh = 0; sh < a.S; ++sh)
        s += load_f32<T>(y + (nk + static_cast<long long>(sh) * N + t) * H + c);
      fused_put<T>(out + static_cast<long long>(t) * H + c, s);
    }
  }
}

// Stage R with the route layout (lanes per token, logits per lane) that moe_route uses for E.
// local: every workgroup routes every token into its LDS (idx, w); otherwise the tokens are dealt
// to the workgroups and the selection goes to the global outputs.
template <int SEG, int PER, bool VEC>
__device__ __forceinline__ void fused_route(const FusedArgs& a, bool local, int32_t* idx,
                                            float* w) {
  constexpr int TPB = kFusedThreads / SEG;
  const int b0 = local ? 0 : blockIdx.x, bs = local ? 1 : gridDim.x;
  for (int b = b0; b * TPB < a.N; b += bs) {
    const int t = b * TPB + static_cast<int>(threadIdx.x) / SEG;
    if (t < a.N)
      route_token<SEG, PER, VEC>(a.logits + static_cast<size_t>(t) * a.E, a.bias, a.E, a.k,
                                 a.gate, threadIdx.x & (SEG - 1), t, idx, w, RouteCount{}, 0);
  }
}

template <typename T>
__global__ __launch_bounds__(kFusedThreads, 1) void fused_layer_kernel(FusedArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char fused_lds_buf[];
  const bool local = a.local_route != 0;
  FusedLds L;
  fused_lds(a.N, a.E, a.k, a.S, local, fused_lds_buf, &L);
  const unsigned P = gridDim.x;
  static_assert(kSyncBytes <= 4096, "sync words fit the workspace's first 4 KB");
  int32_t* idx = local ? L.tidx : a.topk_idx;
  float* wts = local ? L.tw : a.topk_w;
  route_shape(a.E, [&](auto seg, auto per, auto vec) __attribute__((always_inline)) {
    fused_route<decltype(seg)::value, decltype(per)::value, decltype(vec)::value>(a, local, idx,
                                                                                    wts);
  });
  unsigned nth = 0;
  bool ok = true;
  if (local) {
    // every workgroup holds every token's selection; workgroup 0 also writes the outputs
    __syncthreads();
    if (blockIdx.x == 0)
      for (int i = threadIdx.x; i < a.N * a.k; i += kFusedThreads) {
        a.topk_idx[i] = idx[i];
        a.topk_w[i] = wts[i];
      }
  } else {
    ok = fused_barrier(a.sync, ++nth, L.flag);
  }
  if (ok) {
    fused_layout(a, L, idx);
    fused_ffn_stage<T, 2>(a, L);
    ok = fused_barrier(a.sync, ++nth, L.flag);
  }
  if (ok) {
    fused_ffn_stage<T, 1>(a, L);
    ok = fused_barrier(a.sync, ++nth, L.flag);
  }
  if (ok) fused_combine<T>(a, L, wts);
  // the last workgroup out returns the counters to zero
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    if (atomicAdd(sync_done(a.sync), 1u) == P - 1) {
      for (int g = 0; g < 8; ++g) {
        atomicExch(sync_group(a.sync, g), 0u);
        atomicExch(sync_release(a.sync, g), 0u);
      }
      atomicExch(sync_all(a.sync), 0u);
      atomicExch(sync_done(a.sync), 0u);
    }
  }
}

static std::mutex g_fused_mu;
static int g_fused_cus[64];

static int fused_cus() {
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= 64) return 0;
  std::lock_guard<std::mutex> lock(g_fused_mu);
  if (!g_fused_cus[d]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess) return 0;
    g_fused_cus[d] = n;
  }
  return g_fused_cus[d];
}

template <typename T>
static moe_status launch_fused(const FusedArgs& a, size_t lds, hipStream_t s) {
  auto kern = fused_layer_kernel<T>;
  const int cus = fused_cus();
  int per_cu = 0;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(lds)) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kFusedThreads, lds) !=
          hipSuccess ||
      per_cu < 1 || cus < 1) {
    moe_host::set_error("moe_layer_fused: the kernel does not fit one workgroup per CU");
    return MOE_EINVAL;
  }
  // one workgroup per CU: every workgroup is resident, so the stage waits can complete
  hipLaunchKernelGGL(kern, dim3(cus), dim3(kFusedThreads), lds, s, a);
  return moe_host::launch_status();
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_layer_fused_workspace_bytes(int N, int H, int k, int I, int n_shared,
                                                  int dtype) {
  if (N <= 0 || H <= 0 || k <= 0 || I <= 0 || n_shared < 0 ||
      (dtype != MOE_F32 && dtype != MOE_BF16))
    return 0;
  const size_t eb = dtype == MOE_F32 ? 4 : 2;
  const size_t rows = static_cast<size_t>(N) * k + static_cast<size_t>(n_shared) * N;
  auto a256 = [](size_t b) { return (b + 255) & ~size_t(255); };
  return 4096 + a256(rows * I * eb) + a256(rows * H * eb);
}

extern "C" moe_status moe_layer_fused(const void* x, int dtype, const float* logits,
                                      const float* bias, int N, int H, int E, int k, int gate,
                                      int I, const void* w_gate_up, const void* w_down,
                                      int n_shared, const void* shared_w_gate_up,
                                      const void* shared_w_down, int weights_packed,
                                      int32_t* topk_idx, float* topk_w, void* workspace,
                                      void* out, void* stream) {
  const bool bf = dtype == MOE_BF16;
  if ((dtype != MOE_F32 && !bf) || N < 0 || N > kFusedMaxTokens || E < 1 ||
      E > MOE_MAX_EXPERTS || k < 1 || k > E || k > MOE_MAX_TOPK ||
      static_cast<long long>(N) * k > kFusedMaxSlots || H <= 0 || H % kFusedCols ||
      I <= 0 || I % kFusedCols || n_shared < 0 || n_shared > 16 ||
      (gate != MOE_GATE_SOFTMAX && gate != MOE_GATE_SIGMOID)) {
    moe_host::set_error("moe_layer_fused: invalid shape (N <= 1024, N k <= 4096, H and I "
                        "multiples of 128, E <= 512, k <= min(E, 64), at most 16 shared)");
    return MOE_EINVAL;
  }
  if (weights_packed && (!bf || H % 256)) {
    moe_host::set_error("moe_layer_fused: packed weights need bf16 and H a multiple of 256");
    return MOE_EINVAL;
  }
  const size_t rows = static_cast<size_t>(N) * k + static_cast<size_t>(n_shared) * N;
  if (rows * (H > I ? H : I) >= (size_t(1) << 31)) {
    moe_host::set_error("moe_layer_fused: workspace rows exceed 2^31 elements");
    return MOE_EINVAL;
  }
  if (N == 0) return MOE_OK;
  if (!x || !logits || !w_gate_up || !w_down || !topk_idx || !topk_w || !workspace || !out ||
      (n_shared > 0 && (!shared_w_gate_up || !shared_w_down))) {
    moe_host::set_error("moe_layer_fused: NULL pointer");
    return MOE_EINVAL;
  }
  const size_t eb = bf ? 2 : 4;
  auto a256 = [](size_t b) { return (b + 255) & ~size_t(255); };
  char* ws = static_cast<char*>(workspace);
  FusedArgs a;
  a.x = x;
  a.logits = logits;
  a.bias = bias;
  a.N = N;
  a.H = H;
  a.E = E;
  a.k = k;
  a.gate = gate;
  a.I = I;
  a.S = n_shared;
  a.packed = weights_packed ? 1 : 0;
  a.wgu = w_gate_up;
  a.wd = w_down;
  a.swgu = shared_w_gate_up;
  a.swd = shared_w_down;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.sync = reinterpret_cast<unsigned*>(ws);
  a.h = ws + 4096;
  a.y = ws + 4096 + a256(rows * I * eb);
  a.out = out;
  // every workgroup routes every token itself when that takes at most 4 passes of its 256 lanes
  // (cheaper than a device-wide barrier)
  a.local_route = static_cast<long long>(N) * route_seg(E) <= 4 * kFusedThreads ? 1 : 0;
  const size_t lds = fused_lds(N, E, k, n_shared, a.local_route != 0, nullptr, nullptr);
  hipStream_t s = moe_host::as_stream(stream);
  return bf ? launch_fused<bf16_t>(a, lds, s) : launch_fused<float>(a, lds, s);
}
