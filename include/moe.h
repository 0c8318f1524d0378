/*
 * moe.h: C ABI of libmoe.so, the hot path of one expert-parallel Mixture-of-Experts layer on one
 * MI355X (gfx950): route -> dispatch layout and permute -> grouped SwiGLU expert GEMM -> combine.
 *
 * Problem (blog "Kernel fusion for expert parallelism", section "Expert parallelism: dispatch and
 * combine"): N tokens of width H, E experts, each token picks its top-k experts; W expert-parallel
 * ranks hold E / W experts each. The W ranks are simulated as W contiguous partitions of one HBM
 * buffer, so one GPU runs one rank's share (or every rank's share) of dispatch and combine at
 * real shape.
 *
 * Conventions shared by every entry point
 *  - All array arguments are DEVICE pointers (hipMalloc'ed or torch CUDA memory) unless marked
 *    "host". The caller owns and allocates every buffer; the library never allocates, frees,
 *    synchronises the device or reads device data on the host.
 *  - Every call only enqueues kernels on `stream` (a hipStream_t; NULL = the null stream) and
 *    returns at once. Data-dependent sizes (rows per expert, dedup row count) stay on the device.
 *  - Arguments are checked on the host before any launch: a bad size, null pointer or
 *    unsupported shape returns MOE_EINVAL and launches nothing. A launch failure returns
 *    MOE_EHIP. Device-side contents (expert ids out of range, non-finite logits, a placement
 *    that is not a map into [0, W)) are preconditions and are not checked: results are
 *    undefined.
 *  - Results are deterministic: identical inputs give bit-identical outputs (no float atomics).
 *  - slot = t * k + j names the j-th selected expert of token t.
 *  - Element types: MOE_F32 (float) or MOE_BF16 (bfloat16, stored as 16-bit words). Routing
 *    weights are always float. Integers are int32.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_OK = 0, MOE_EINVAL = 1, MOE_EHIP = 2 } moe_status;
typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;
typedef enum { MOE_GATE_SOFTMAX = 0, MOE_GATE_SIGMOID = 1 } moe_gate;
typedef enum { MOE_FFN_GATE_UP = 1, MOE_FFN_DOWN = 2, MOE_FFN_ALL = 3 } moe_ffn_phase;

/* Limits of this library (checked on the host). */
#define MOE_MAX_EXPERTS 512
#define MOE_MAX_RANKS 64
#define MOE_MAX_TOPK 64

/* Static description of one layer problem (host struct, passed by pointer). */
typedef struct moe_shape {
  int N; /* tokens (multiple of W: each rank owns a contiguous slice of N / W tokens) */
  int E; /* routed experts, 1..MOE_MAX_EXPERTS, multiple of W */
  int k; /* experts per token, 1..min(E, MOE_MAX_TOPK) */
  int W; /* simulated expert-parallel ranks, 1..MOE_MAX_RANKS */
  int H; /* hidden width (multiple of 8) */
} moe_shape;

/*
 * Layout arrays, all caller-allocated int32 device arrays (moe_layout_carve places them inside
 * one buffer of moe_layout_bytes bytes). Rows are the (token, expert) assignments ordered by
 * (rank of the expert, expert, token): rank r's rows are one contiguous partition, expert-major
 * inside, tokens ascending inside an expert. Groups are the experts in the same (rank, expert)
 * order. Pair rows (deduplicated dispatch) are the unique (token, rank) pairs ordered by
 * (rank, token).
 */
typedef struct moe_layout {
  int32_t* expert_counts;    /* [E]     rows of expert e */
  int32_t* expert_offsets;   /* [E]     first row of expert e */
  int32_t* group_expert;     /* [E]     expert at group position g */
  int32_t* group_offsets;    /* [E+1]   first row of group g; [E] = N*k */
  int32_t* rank_counts;      /* [W]     rows on rank r */
  int32_t* rank_offsets;     /* [W+1]   first row of rank r */
  int32_t* send_counts;      /* [W*W]   [s*W+r]: rows from owner s to rank r */
  int32_t* row_of_slot;      /* [N*k] */
  int32_t* slot_of_row;      /* [N*k] */
  int32_t* pair_counts;      /* [W]     pair rows on rank r */
  int32_t* pair_offsets;     /* [W+1]   first pair row of rank r; [W] = D, the dedup row count */
  int32_t* pair_token;       /* [N*min(k,W)] token of pair row p (first D entries valid) */
  int32_t* pair_of_slot;     /* [N*k]   pair row carrying slot s */
  int32_t* pair_send_counts; /* [W*W]   pair rows from owner s to rank r */
  int32_t* expand_src;       /* [N*k]   pair row that expert-major row i expands from */
} moe_layout;

/* Bytes of one buffer holding every moe_layout array (256-byte aligned sub-arrays). */
size_t moe_layout_bytes(const moe_shape* shape);
/* Fill *L with pointers into `base` (a device buffer of moe_layout_bytes bytes). Host only. */
moe_status moe_layout_carve(const moe_shape* shape, void* base, moe_layout* L);
/*
 * Device workspace that moe_dispatch_layout needs (caller-allocated, any contents): the count
 * rows, i.e. the expert counts and (token, rank) pair counts of every slice of T consecutive
 * tokens (T = 64 for E <= 4, 32 for E 5..8, 16 above), about ceil(N / T) * (E + W) * 4 bytes.
 */
size_t moe_layout_workspace_bytes(const moe_shape* shape);

/*
 * moe_route: top-k expert selection and gate weights, and optionally the dispatch layout's
 * count rows.
 * FarSkip-Collective (arXiv 2511.11505) section 2.1: the gate is a linear layer followed by a
 * sparse selection; Expert Coupling in MoE Pretraining (arXiv 2610.09372) Appendix A-A1 Table II:
 * softmax over all experts, then top-k. Blog "Kernel fusion for expert parallelism", section
 * "Fusing the layer into one kernel": stage "route" computes the routing metadata.
 *   logits   [N, E] float, row-major: the router's linear output.
 *   bias     [E] float or NULL: added to every row of logits (one fp32 add); the biased logit
 *            drives both the selection and the weight.
 *   gate     MOE_GATE_SOFTMAX: weights = softmax over the k selected logits (sum to 1);
 *            MOE_GATE_SIGMOID: weight = 1 / (1 + exp(-l)), not renormalised.
 *   topk_idx [N, k] int32 out: the k largest biased logits in descending order, equal logits
 *            listed lower expert index first.
 *   topk_w   [N, k] float out.
 *   layout_workspace NULL, or the workspace of a following moe_dispatch_layout call for the
 *            shape (N, E, k, W) (moe_layout_workspace_bytes bytes): the route then also writes
 *            the count rows of that workspace, and that call may pass counts_ready = 1 to skip
 *            its own count step. expert_rank ([E] int32 or NULL, contiguous) and W must be the
 *            ones that call uses; both are ignored when layout_workspace is NULL.
 * Errors: MOE_EINVAL if N < 0, E < 1, E > MOE_MAX_EXPERTS, k < 1, k > min(E, MOE_MAX_TOPK), a
 * required pointer is NULL, gate is unknown, or (with layout_workspace) W is outside
 * 1..MOE_MAX_RANKS or does not divide E and N. N = 0 launches nothing.
 */
moe_status moe_route(const float* logits, const float* bias, int N, int E, int k, int gate,
                     int32_t* topk_idx, float* topk_w, const int32_t* expert_rank, int W,
                     void* layout_workspace, void* stream);

/*
 * moe_gate_route: the router's linear layer on the device, then moe_route.
 * FarSkip-Collective (arXiv 2511.11505) section 2.1: G(A) = s(A W_R^T); Expert Coupling in MoE
 * Pretraining (arXiv 2610.09372) Appendix A-A1 Table II: the gate is an FP32 linear layer.
 *   x        [N, H] of dtype (MOE_BF16 or MOE_F32), row-major, 16-byte aligned.
 *   w_router [E, H] float, row-major: W_R, kept fp32 (the call first splits it into a bf16 high
 *            part and a bf16 remainder in `workspace`; the logits accumulate in fp32 on the
 *            matrix cores), or NULL: `workspace` already holds that split, written by
 *            moe_gate_prepare for the same E and H (the split is skipped).
 *   workspace moe_gate_workspace_bytes(E, H) bytes of device memory (16-byte aligned).
 *   bias     [E] float or NULL: as for moe_route, which adds it when it runs on `logits`;
 *            `logits` itself holds x W_R^T without the bias.
 *   logits   [N, E] float out (caller-allocated): x W_R^T.
 *   k, gate, topk_idx, topk_w, expert_rank, W, layout_workspace: as for moe_route. The
 *            selection (and the count rows) runs in the product's epilogue when one workgroup
 *            holds all E logits of its tokens (E <= 32, 33-64 with N >= 16384, 65-128, or
 *            129-256 with N < 16384), else as moe_route on `logits` after the product; it runs
 *            the same code as moe_route, so the result equals moe_route on the written `logits`
 *            either way.
 * Errors: MOE_EINVAL if N < 0, H is not a positive multiple of 32, E < 1 or E > 256, k < 1 or
 * k > min(E, MOE_MAX_TOPK), dtype or gate is unknown, a required pointer is NULL, or W is
 * invalid as for moe_route. N = 0 launches nothing.
 */
moe_status moe_gate_route(const void* x, int dtype, const float* w_router, const float* bias,
                          int N, int H, int E, int k, int gate, void* workspace, float* logits,
                          int32_t* topk_idx, float* topk_w, const int32_t* expert_rank, int W,
                          void* layout_workspace, void* stream);

/* moe_gate_workspace_bytes: scratch moe_gate_route needs (E * H * 4), 0 for E or H <= 0. */
size_t moe_gate_workspace_bytes(int E, int H);

/*
 * moe_gate_prepare: the split of the router weights that moe_gate_route multiplies with, done
 * once (router weights change only between training steps): writes the bf16 high part and bf16
 * remainder of w_router ([E, H] float) into workspace (moe_gate_workspace_bytes(E, H) bytes).
 * moe_gate_route with w_router = NULL then uses it. Errors: MOE_EINVAL if H is not a positive
 * multiple of 32, E < 1 or E > 256, or a pointer is NULL.
 */
moe_status moe_gate_prepare(const float* w_router, int E, int H, void* workspace, void* stream);

/*
 * moe_dispatch_layout: builds the dispatch layout and (optionally) permutes the token rows into
 * the W rank partitions.
 * Blog "Kernel fusion for expert parallelism": section "All-to-All" (a selective send needs the
 * per-destination counts), section "Fusing the layer into one kernel" (Baseline "pack": a copy of
 * each token laid out contiguously per destination; stage "group": rows in expert-contiguous
 * order). Expert Coupling in MoE Pretraining section V-A and Appendix A-A2 (i): the
 * deduplicating dispatcher sends one row per unique (token, destination rank).
 *   topk_idx    [N, k] int32 (moe_route output).
 *   expert_rank [E] int32 or NULL: placement, rank of each expert (NULL = contiguous, expert e
 *               on rank e / (E / W), Expert Coupling section I). Each rank must hold E / W
 *               experts for the group order to match the weights the caller stacks per rank.
 *   L           the layout arrays to fill (all of them are always written).
 *   workspace   moe_layout_workspace_bytes(shape) bytes of device scratch.
 *   counts_ready 1: `workspace` already holds the count rows for these topk_idx, expert_rank
 *               and W, written by moe_route or moe_gate_route (given this workspace) on the same
 *               stream, so the count step is skipped; 0: the call counts.
 *   x           [N, H] of dtype, or NULL for the layout alone.
 *   dedup       0: rows_out gets one row per (token, expert) in row order;
 *               1: rows_out gets one row per (token, rank) pair in pair order.
 *   dst_rank    -1: rows_out holds every rank's partition (N*k rows, or D pair rows);
 *               r >= 0: rows_out holds rank r's partition only, starting at its first row.
 *   rows_out    [capacity, H] of dtype; capacity N*k (dedup: N*min(k,W)) for dst_rank -1, or
 *               N*min(k, E/W) (dedup: N) for one rank.
 * Errors: MOE_EINVAL for an invalid shape, NULL required pointers, dst_rank out of [-1, W),
 * or x given without rows_out.
 */
moe_status moe_dispatch_layout(const moe_shape* shape, const int32_t* topk_idx,
                               const int32_t* expert_rank, const moe_layout* L, void* workspace,
                               const void* x, int dtype, int dedup, int dst_rank,
                               int counts_ready, void* rows_out, void* stream);

/*
 * moe_dispatch_layout_noalloc: moe_dispatch_layout without the workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Arguments, results and errors are those of
 * moe_dispatch_layout with counts_ready = 0 (the call always counts); the workspace is a fixed
 * device array inside the library of MOE_LAYOUT_SCRATCH_BYTES bytes per device, which each
 * device holds from its first call until the process ends. The call allocates nothing and calls
 * no allocating routine.
 * Limits: moe_layout_workspace_bytes(shape) must not exceed MOE_LAYOUT_SCRATCH_BYTES (about
 * ceil(N / 16) * (E + W) * 4 bytes for E > 8: N = 116480 tokens at E = 512, W = 64, N = 254192
 * at E = 256, W = 8), else MOE_EINVAL; the current device's ordinal must be below
 * MOE_MAX_DEVICES, else MOE_EHIP.
 * Every call on one device shares that device's array, which keeps the last call's contents
 * (the layout kernels overwrite every entry they later read, so nothing needs clearing): calls
 * on one device that may overlap (different streams with no ordering between them) race and
 * give undefined results; order them, or use moe_dispatch_layout with one workspace per stream.
 */
#define MOE_LAYOUT_SCRATCH_BYTES (16u << 20)
#define MOE_MAX_DEVICES 64
moe_status moe_dispatch_layout_noalloc(const moe_shape* shape, const int32_t* topk_idx,
                                       const int32_t* expert_rank, const moe_layout* L,
                                       const void* x, int dtype, int dedup, int dst_rank,
                                       void* rows_out, void* stream);

/*
 * moe_expert_ffn: grouped SwiGLU expert FFN, y = W_d (silu(W_g a) * (W_u a)) for every row a of
 * every group, plus optional shared experts over a dense block of rows.
 * Blog "Kernel fusion for expert parallelism", section "Fusing the layer into one kernel"
 * (stages MatMul gate and up, SwiGLU, MatMul down); FarSkip-Collective section 2.1 (shared
 * experts run on every token in addition to the routed ones).
 *   rows          routed input rows of dtype, [*, H].
 *   group_offsets [G+1] int32: group g covers rows group_offsets[g] .. group_offsets[g+1]-1,
 *                 indexed RELATIVE to group_offsets[0] (pass layout.group_offsets + r*(E/W)
 *                 with G = E/W for rank r's partition, or layout.group_offsets with G = E).
 *   row_gather    NULL, or int32 indexed by ABSOLUTE row (a group_offsets value): the row at
 *                 absolute index a reads rows[row_gather[a] - base] instead of
 *                 rows[a - group_offsets[0]], where base = *gather_base (device int) or 0 when
 *                 gather_base is NULL. This is the dedup expand of the receiving rank: pass
 *                 layout.expand_src with rows = pair rows; for one rank's pair partition pass
 *                 gather_base = layout.pair_offsets + r.
 *   max_rows      host upper bound on group_offsets[G] - group_offsets[0] (sizes the grid).
 *   w_gate_up     [G, 2I, H] of dtype: rows 0..I-1 gate, I..2I-1 up (K = H contiguous).
 *   w_down        [G, H, I] of dtype (K = I contiguous).
 *   h             [max_rows, I] of dtype: intermediate workspace (silu(gate) * up), written.
 *   y             of dtype out: [max_rows, H] indexed by relative rows like `rows`, or, when
 *                 y_absolute is 1, indexed by ABSOLUTE row (row a at y + a * H, so one rank's
 *                 outputs land in place inside an [N*k, H] array of every rank's rows without
 *                 the host reading where the rank's partition starts).
 *   n_shared      shared experts (0 = none); then shared_x [M_sh, H], shared_w_gate_up
 *                 [S, 2I, H], shared_w_down [S, H, I], shared_h [S, M_sh, I] workspace and
 *                 shared_y [S, M_sh, H] out, all of dtype.
 *   phases        MOE_FFN_ALL (both GEMMs), or MOE_FFN_GATE_UP (h only) / MOE_FFN_DOWN (y from
 *                 an h written earlier) for callers that place or time the two launches apart.
 *   weights_packed 0: w_gate_up, w_down and the shared weights are in the plain layout above;
 *                 1: all four were converted by moe_pack_weights (w_gate_up and
 *                 shared_w_gate_up with NB = 2, Nn = I, K = H; w_down and shared_w_down with
 *                 NB = 1, Nn = H, K = I). Needs bf16, I % 128 == 0 and H % 256 == 0.
 * Shapes: bf16 needs H % 128 == 0 and I % 128 == 0; f32 needs H % 64 == 0 and I % 64 == 0.
 * bf16 addresses each operand block with 32-bit byte offsets: (max_rows + 1) * max(H, I) * 2,
 * (M_sh + 1) * max(H, I) * 2 and one expert's gate/up weights (4 * I * H bytes) must stay below
 * 4 GiB, and with row_gather every gathered source index times 2 H as well.
 * At most 16 shared experts; G <= MOE_MAX_EXPERTS.
 * Errors: MOE_EINVAL for bad shapes, operand blocks of 4 GiB or more, or NULL required pointers.
 */
moe_status moe_expert_ffn(const void* rows, const int32_t* group_offsets, int G,
                          const int32_t* row_gather, const int32_t* gather_base, int max_rows,
                          const void* w_gate_up,
                          const void* w_down, int H, int I, int dtype, void* h, void* y,
                          int y_absolute, int n_shared, const void* shared_x, int M_sh,
                          const void* shared_w_gate_up, const void* shared_w_down,
                          void* shared_h, void* shared_y, int phases, int weights_packed,
                          void* stream);

/*
 * moe_set_gemm_max_cus: caps the persistent grid of moe_expert_ffn's GEMM launches at n compute
 * units' worth of workgroups (rounded down to a multiple of 8, one per XCD, and at least 8);
 * n = 0 restores the default, every compute unit of the device. For callers that run the
 * grouped GEMM beside other kernels and leave compute units to them (blog "Kernel fusion for
 * expert parallelism", section "Pipelining and three-way overlap": the exchange runs beside the
 * expert matrix multiplications). A process-wide setting, read at each launch (atomic: safe to
 * change from any host thread; launches already enqueued keep their grid). Every output element
 * is computed by one tile with the same K order whatever the grid, so results are bit-identical
 * for every setting; only the time changes.
 * Errors: MOE_EINVAL for n < 0.
 */
moe_status moe_set_gemm_max_cus(int n);

/*
 * moe_pack_weights: converts bf16 expert weights from the plain K-contiguous layout
 * [G][NB * Nn][K] into the packed layout moe_expert_ffn reads with weights_packed = 1: a pure
 * permutation of the same G * NB * Nn * K values (same byte size), done once when the weights
 * are loaded. The grouped GEMM reads each K step of a 256-row weight panel as one contiguous
 * 32 KB block instead of 128 bytes from each of 256 rows, which keeps the weight stream from HBM
 * in whole DRAM pages (blog "Kernel fusion for expert parallelism", section "Fusing the layer
 * into one kernel": the expert weights are the bytes the grouped matrix multiplications stream).
 * Layout: for group g, panel p and K step kt (KT = K / 64), 32 KB at byte
 * ((g * panels + p) * KT + kt) * 32768 hold 32 chunks q of 1 KB; the 16 bytes at 16 l of chunk q
 * are the 8 values W[row][kt * 64 + 8 c .. + 7] of panel row r = 8 q + l / 8, with
 * c = (l % 8) XOR ((r / 2) % 8). Panel rows: NB = 2 (gate/up, panels = Nn / 128): r < 128 is gate
 * row 128 p + r, r >= 128 up row Nn + 128 p + r - 128; NB = 1 (down, panels = Nn / 256): row
 * 256 p + r.
 *   w   [G, NB * Nn, K] bf16 (device), not modified; out: the same number of bytes, not
 *       overlapping w.
 * Errors: MOE_EINVAL if NB is not 1 or 2, K % 64 != 0, Nn % 128 (NB = 2) or Nn % 256 (NB = 1)
 * is not 0, or a pointer is NULL or out == w. G = 0 launches nothing.
 */
moe_status moe_pack_weights(const void* w, int G, int NB, int Nn, int K, void* out,
                            void* stream);

/*
 * moe_layer_fused: the whole layer for a small batch (decode) in one persistent launch: route,
 * layout, gate/up GEMM with SwiGLU, down GEMM and combine, every rank's share, flat combine.
 * Blog "Kernel fusion for expert parallelism", section "Fusing the layer into one kernel" (one
 * kernel runs route, group, MatMul, SwiGLU, MatMul and reduce) and "Results" (the gain is largest
 * for small batches); FarSkip-Collective section 2.1:
 *   out[t] = sum_j topk_w[t,j] FFN_{topk_idx[t,j]}(x_t) + sum_s FFN_s(x_t).
 *   x, logits, bias, k, gate: as for moe_route (routing from the router logits); topk_idx and
 *               topk_w are written (bit-identical to moe_route's).
 *   w_gate_up [E, 2I, H], w_down [E, H, I], shared_w_gate_up [S, 2I, H], shared_w_down [S, H, I]
 *               of dtype: plain K-contiguous, or (weights_packed = 1, bf16, H % 256 == 0) all
 *               four converted by moe_pack_weights.
 *   workspace   moe_layer_fused_workspace_bytes(...) bytes: its first 4096 bytes are the launch's
 *               device-wide counters and must be zero before the first call (each call returns
 *               them to zero), then h and the expert outputs.
 *   out         [N, H] of dtype.
 * The launch runs one workgroup per compute unit and separates its stages with device-wide
 * barriers; it needs every workgroup resident, so it must not overlap other work on the device
 * that holds compute units, nor another call on the same workspace. A barrier wait gives up after
 * about one second: the workgroups then leave, the kernel ends, the outputs are undefined and the
 * 32-bit word at byte 2304 of the workspace is nonzero (write 0 to it before the next call).
 * Results are deterministic (no float atomics); they equal the separate entry points' up to the
 * order of the fp32 accumulation inside the GEMMs.
 * Errors: MOE_EINVAL for dtype other than MOE_F32 / MOE_BF16, N > 1024, N * k > 4096, H or I not a
 * multiple of 128, E > MOE_MAX_EXPERTS, k > min(E, MOE_MAX_TOPK), more than 16 shared experts, an
 * unknown gate, packed weights without bf16 and H % 256 == 0, a NULL required pointer, or a
 * device whose compute units cannot hold the kernel. N = 0 launches nothing.
 */
moe_status moe_layer_fused(const void* x, int dtype, const float* logits, const float* bias,
                           int N, int H, int E, int k, int gate, int I, const void* w_gate_up,
                           const void* w_down, int n_shared, const void* shared_w_gate_up,
                           const void* shared_w_down, int weights_packed, int32_t* topk_idx,
                           float* topk_w, void* workspace, void* out, void* stream);

/* Workspace of moe_layer_fused: 4096 + (N k + S N) (I + H) elements of dtype (256-aligned parts);
 * 0 for invalid arguments. */
size_t moe_layer_fused_workspace_bytes(int N, int H, int k, int I, int n_shared, int dtype);

/*
 * moe_combine: weighted top-k combine for the owned tokens t_begin .. t_end-1.
 * FarSkip-Collective section 2.1 (the combine sums the routed experts' weighted outputs back into
 * the layer output; shared experts are added); blog "Kernel fusion for expert parallelism",
 * sections "All-to-All" (the owner sums the returned rows) and "INC All-to-All-Combine" (the
 * expert rank applies the routing weights before publishing its partial results); Expert
 * Coupling section V-A (dedup combine: one weighted partial per (token, rank)).
 *   dedup 0: out[t - t_begin] = sum_j topk_w[t,j] * y[row_of_slot[t*k+j]] (+ shared), slot
 *            order, fp32 accumulation. y holds every rank's rows in row order (absolute rows).
 *   dedup 1: two stages. Expert-rank side: for every pair row p = (t, r),
 *            partial[p] = sum over slots j of t whose expert is on rank r of
 *            topk_w[t,j] * y[row_of_slot[t*k+j]], in slot order (when y_is_pair_rows, every
 *            term reads y[p] instead: identity experts applied to the pair rows). Owner side:
 *            out[t - t_begin] = sum of the token's partials, ranks taken in the order of
 *            their first slot (+ shared).
 *   dst_rank  dedup only: -1 = the expert-rank side runs for every pair row; r >= 0 = only
 *            for rank r's pair rows (one rank's share: the partials of the other ranks' pair
 *            rows are what those ranks would send, and must already be in `partial`).
 *            Ignored when dedup is 0.
 *   topk_idx, topk_w, expert_rank (NULL = contiguous): as given to the layout.
 *   shared    NULL or [n_shared, N, H] of dtype: shared-expert outputs added to every token.
 *   partial   dedup only: [N*min(k,W), H] of dtype workspace.
 *   out       [t_end - t_begin, H] of dtype.
 * Errors: MOE_EINVAL for bad shapes, 0 <= t_begin <= t_end <= N violated, dst_rank outside
 * [-1, W), NULL required pointers.
 */
moe_status moe_combine(const moe_shape* shape, const void* y, int y_is_pair_rows,
                       const moe_layout* L, const int32_t* topk_idx, const float* topk_w,
                       const int32_t* expert_rank, int dtype, int dedup, int dst_rank,
                       int t_begin, int t_end, const void* shared, int n_shared, void* partial,
                       void* out, void* stream);

/*
 * moe_coselect_counts: co-selection counts for correlated placement (Expert Coupling section
 * V-A "Correlated Placement", Appendix A-D Algorithm 1 first step): counts[e*E+e'] = tokens
 * selecting both e and e' (e != e'), int32, symmetric, zero diagonal. counts [E*E] is
 * overwritten.
 */
moe_status moe_coselect_counts(const int32_t* topk_idx, int N, int E, int k, int32_t* counts,
                               void* stream);

/*
 * moe_placement_partition: HOST function. Balanced partition of E experts into G groups of
 * E / G that raises the total co-selection weight inside groups (Expert Coupling Appendix A-D
 * Algorithm 1, procedure Partition): start from contiguous groups; repeat at most i_max times
 * (i_max <= 0 means E*E): take the single swap of two experts in different groups with the
 * largest gain D_a + D_b - 2 W[a,b] (D_x = weight from x to the other group minus weight to
 * its own group), the lexicographically smallest (a, b) among equal gains; stop when the best
 * gain is not positive.
 *   counts [E*E] host int64 (symmetric, zero diagonal); group [E] host int32 out.
 * Returns MOE_EINVAL if E % G != 0 or pointers are NULL. *swaps (host, may be NULL) receives the
 * number of swaps made.
 */
moe_status moe_placement_partition(const int64_t* counts, int E, int G, int i_max,
                                   int32_t* group, int* swaps);

/*
 * moe_shuffle_fit: offline tables of the token-shuffle planner from one routing trace (Expert
 * Coupling section V-B "Cross-Layer Correlation: Token Shuffling", Appendix "Token shuffling"
 * Algorithm 2, offline step). For trace token t with top-k sets prev2[t] (position m-2),
 * prev1[t] (m-1) and cur[t] (m), every e in prev1[t] adds, for each slot x of cur[t], one count
 * to F[e, placement[x]]; every pair (e' in prev2[t], e in prev1[t]) adds one to n[e', e] and one
 * per slot to S[e', e, placement[x]]. Each row of F and S is then divided by its total in fp32
 * (one division per entry); a row of F with no counts is 1/P, a row of S with none is 0.
 *   prev2, prev1, cur [T, k] int32 device; placement [E] int32 device (rank of each expert).
 *   workspace: moe_shuffle_fit_workspace_bytes(E, P) bytes of device scratch.
 *   F [E, P], S [E, E, P] float and n [E, E] int32: device outputs, overwritten.
 * Indices outside [0, E) and ranks outside [0, P) add nothing. Deterministic (integer counts).
 * Errors: MOE_EINVAL if k < 1 or k > MOE_MAX_TOPK, P < 1 or P > 64, E < 1 or E > 4096,
 * E*E*P > 2^28, T < 0 or T > 2^24, or a required pointer is NULL.
 */
moe_status moe_shuffle_fit(const int32_t* prev2, const int32_t* prev1, const int32_t* cur,
                           int T, int k, int E, int P, const int32_t* placement, void* workspace,
                           float* F, float* S, int32_t* n, void* stream);
/* moe_shuffle_fit_workspace_bytes: scratch moe_shuffle_fit needs (its int32 counts). */
size_t moe_shuffle_fit_workspace_bytes(int E, int P);

/*
 * moe_shuffle_plan: owner rank of each of T tokens for the coming MoE position, and the
 * owner-major token order (Expert Coupling Appendix "Token shuffling" Algorithm 2).
 *   d[t, r] = normalised sum over e in prev1[t], e' in prev2[t] of
 *             (1 - w) F[e, r] + w S[e', e, r],  w = min(n[e', e] / (n[e', e] + beta), w_max)
 *             (w = 0 when n[e', e] = 0), in fp32;
 *   conf[t] = largest minus second largest entry of d[t] (1 when P = 1);
 *   owner:    tokens in decreasing conf (equal conf: lower token first) each take the rank of
 *             largest d[t, r] (equal d: lower rank) among ranks still below T / P tokens;
 *   order[i]: the token at new position i, tokens grouped by owner and in token order inside
 *             a rank (rank r holds positions r T/P .. (r+1) T/P - 1); inverse[t]: position of t.
 *   prev2, prev1 [T, k] int32; F, S, n as written by moe_shuffle_fit; all device.
 *   workspace: moe_shuffle_plan_workspace_bytes(T) bytes of device scratch.
 *   d [T, P], conf [T] float, owner, order, inverse [T] int32: device outputs.
 * Indices outside [0, E) add nothing (a token with none gets d = 1/P). T = 0 launches nothing.
 * The sort and the assignment each run on one workgroup, so the plan takes O(T) time on one CU;
 * it is meant for a side stream (the pages overlap it with attention).
 * Errors: MOE_EINVAL if T is not a multiple of P, T > 2^20, P outside [1, 64], k outside
 * [1, MOE_MAX_TOPK], E outside [1, 4096] or E*E*P > 2^28, beta < 0, w_max outside [0, 1], or a
 * required pointer is NULL.
 */
moe_status moe_shuffle_plan(const int32_t* prev2, const int32_t* prev1, int T, int k, int E,
                            int P, const float* F, const float* S, const int32_t* n, float beta,
                            float w_max, void* workspace, float* d, float* conf, int32_t* owner,
                            int32_t* order, int32_t* inverse, void* stream);
/* moe_shuffle_plan_workspace_bytes: scratch moe_shuffle_plan needs (sort keys and values). */
size_t moe_shuffle_plan_workspace_bytes(int T);

/*
 * moe_device_info: HOST function. The current device's compute units, LDS bytes per compute
 * unit, peak shader clock and memory clock (kHz), as the HIP runtime reports them. Any output
 * pointer may be NULL. Errors: MOE_EHIP if there is no device or an attribute query fails.
 */
moe_status moe_device_info(int* cus, int* lds_bytes_per_cu, int* clock_khz, int* mem_clock_khz);

/* Static description of a status code. */
const char* moe_status_string(moe_status s);
/* Last HIP error text seen by the library on this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
