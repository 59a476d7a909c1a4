/*
 * mk.h -- C ABI of libmk: persistent, role-specialised fused GEMM kernels for
 * AMD Instinct MI355X (gfx950).
 *
 * The operations are the data-parallel hot path of the fused
 * communication+GEMM kernels described on the mKernel pages:
 *   [P1] "Conozca mKernel, una biblioteca de núcleo fusionado con múltiples GPU
 *        y múltiples nodos para comunicación impulsada por GPU" (7minutos.es),
 *        section "Los cinco núcleos fusionados" and explainer slide
 *        "04 / 07 — Granos";
 *   [P3] the Arabic translation (k7ail.com), table "الحبات الخمس المنصهرة".
 * Per [P1] section "¿Qué hace mKernel?", each operation is ONE persistent
 * kernel whose workgroups assign themselves roles (compute, copy, reduce) and
 * the number of workgroups per role can be tuned per shape.
 *
 * This library runs one GPU's share of each operation.  The peers' data (A
 * shards, partial sums, token rows) are resident device buffers; copy-role
 * workgroups move them under an arrival schedule while compute-role
 * workgroups run the GEMM tile by tile as their operands land.
 *
 * Conventions for every entry point
 *   - Matrices are dense row-major.  Pointers marked "device" must be device
 *     memory of the current HIP device, 16-byte aligned; row lengths in
 *     elements must be multiples of 8 (16 bytes of bf16).
 *   - Pointer arrays (a_shards, partials, out_owner, W) and mk_arrival /
 *     mk_launch are HOST memory, read during the call only.
 *   - The caller owns every buffer.  The library allocates no device memory.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = default).
 *     Argument and schedule errors are returned synchronously, before any
 *     HIP call, and nothing is launched.  A watchdog expiry inside a kernel
 *     (a wait that exceeded launch->spin_limit_us) is sticky in the
 *     workspace and is reported by mk_poll_status() after the stream syncs.
 *   - One call may be in flight per workspace.  A workspace must be zero
 *     filled before its first use (mk_workspace_init does that); every
 *     kernel leaves it ready for the next call.
 *   - Return value: MK_OK (0) or a negative mk_status; mk_last_error() gives
 *     a thread-local description.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mk_dtype { MK_BF16 = 0, MK_F32 = 1 } mk_dtype;

typedef enum mk_status {
  MK_OK = 0,
  MK_ERR_INVALID = -1,      /* bad pointer, shape, dtype or option */
  MK_ERR_UNSUPPORTED = -2,  /* valid request outside this library's limits */
  MK_ERR_WORKSPACE = -3,    /* workspace missing or too small */
  MK_ERR_HIP = -4,          /* a HIP runtime call failed */
  MK_ERR_TIMEOUT = -5,      /* a kernel wait exceeded its watchdog */
  MK_ERR_SCHEDULE = -6      /* arrival schedule is not a permutation / bad delays */
} mk_status;

/* Limits of this library. */
#define MK_MAX_RANKS 64     /* R: shards, partial-sum contributors, owners */
#define MK_MAX_UNITS 256    /* delivery units in one schedule */
#define MK_MAX_EXPERTS 1024 /* E */
#define MK_MAX_TOPK 16      /* k */
#define MK_MAX_LOCAL 64     /* L: local experts */
#define MK_MAX_COLS (1 << 22) /* N (AG, GEMM+RS) and F (MoE): a 256-row output
                                 tile must span less than 4 GiB */

/*
 * Arrival schedule (host memory).  Unit c becomes available to copy no
 * earlier than `delay_ns[c]` nanoseconds after the kernel's first copy
 * workgroup starts; units are handed to copy workgroups in `order`.
 *   order     [n_units] permutation of 0..n_units-1 (issue order)
 *   delay_ns  [n_units] or NULL (= all zero); each <= 1e9
 *   n_units   number of delivery units (<= MK_MAX_UNITS)
 *   unit_rows AG: gathered rows per unit; MoE: tokens per source block;
 *             GEMM+RS/AR: partial-sum rows per unit (one row block of one peer)
 *   withhold  -1, or one unit id that is never delivered: waits on it expire
 *             after spin_limit_us and the call reports MK_ERR_TIMEOUT.  Used
 *             to test failure handling; every kernel still exits.
 * The schedule decides WHEN operands land, never the result.
 */
typedef struct mk_arrival {
  const int32_t* order;
  const uint32_t* delay_ns;
  int32_t n_units;
  int32_t unit_rows;
  int32_t withhold;
} mk_arrival;

/* Launch options.  A zero-filled struct (or NULL) selects per-shape defaults. */
typedef struct mk_launch {
  int32_t mode;           /* 0 fused persistent kernel; 1 unfused baseline:
                             the same steps as separate kernels in stream order;
                             for measurement, one phase of the baseline alone:
                             AG 2 = the copy kernel, 3 = the GEMM kernel (reads
                             a_gathered as it is); GEMM+RS/AR (no arrival) 2 =
                             the reduce kernel (on what is staged), 3 = the GEMM
                             kernel; MoE 2 = routing and the permute kernel,
                             3 = routing and the grouped GEMM kernel (reads Xs
                             and perm as they are) */
  int32_t grid;           /* persistent workgroups; 0 = CUs x occupancy */
  int32_t n_copy;         /* copy-role workgroups (AG, MoE, GEMM+RS/AR with an
                             arrival schedule); 0 = default (AG: three quarters
                             of the grid copy first, a quarter starts on tiles;
                             others: every workgroup copies first, then computes) */
  int32_t n_reduce;       /* GEMM+RS: reduce-role workgroups; 0 = default;
                             -1 = each compute workgroup reduces its own tiles */
  int32_t tile;           /* tile configuration id (name: mk_tile_name); 0 = per-shape default.
                             1 256x256, 2 128x128, 3 256x128, 4 128x256: register-staged
                             (any K multiple of 8; 1 not for GEMM+RS/AR);
                             5 256x256, 6 128x128, 7 256x128, 8 128x256: direct-to-LDS,
                             4-slice ring (K % 128 == 0);
                             9 128x128 direct-to-LDS with an 8-slice ring (AG only,
                             K % 256 == 0; the AG default when M <= 128);
                             10 256x256 direct-to-LDS with 8 waves (AG only, K % 128 == 0);
                             11 128x128 producer/consumer: B streamed by 4 producer waves
                             into a 16-slice ring, A read from a packed copy in the
                             workspace that the copy workgroups write (AG only, M <= 128,
                             K % 128 == 0, not mk_ag_gemm_noalloc).
                             Defaults: AG 11 for a single 128-row tile row with N >= 256
                             (9 without a workspace, 8 if K % 256 != 0 as well); with M and
                             N >= 256 and K % 128 == 0 whichever of 10 (with its column plan),
                             8 and 7 an estimate of the schedule on the CU count finishes
                             first (10 on ties: always where 256x256 tiles give every CU at
                             least one); else a register-staged tile; GEMM+RS/AR with
                             K % 128 == 0 whichever of 5 and 8 the same estimate favours
                             among those whose height divides the owner blocks (5 on ties),
                             else 2; MoE 5 when F >= 256 and H % 128 == 0, 2 when F < 256,
                             else 1.
                             An id an operation does not build returns MK_ERR_UNSUPPORTED
                             (MK_ERR_INVALID if out of range). */
  uint32_t spin_limit_us; /* watchdog for every wait; 0 = 2,000,000 us */
  int32_t* tile_log;      /* device int32 or NULL: per-tile record, see each op */
  int32_t copy_kib;       /* AG, GEMM+RS/AR: bytes per copy work item in KiB (one release each);
                             0 = 1024 (AG: at most the bytes of A / CUs, at least one row,
                             so every workgroup starts with about one item);
                             rounded to whole rows inside one unit and shard */
  int32_t copy_policy;    /* AG copy stores: 0 = default (2), 1 = write-back
                             through the XCD L2, 2 = write-through (sc1): the
                             release after each item then has little to write back */
  int32_t* copy_log;      /* AG, MoE, GEMM+RS/AR: device int32 or NULL: per copy work item
                             (in queue order), 8 int32, see each op; times are
                             the low 32 bits of the device wall clock
                             (mk_wall_clock_khz) */
  int32_t queue_mode;     /* AG: 0 = default: one tile queue in landing order
                             (with the 8-wave 256x256 tile, 256-wide column
                             tiles and then, where that shortens the schedule
                             on the grid, 192-wide ones: M = 8192, N = 3584 on
                             256 workgroups gives 8 of each per tile row);
                             1 = 8 per-XCD queues (the tiles that share an A
                             row block run on one XCD and share its L2; a
                             drained queue's workgroups help the others);
                             2 = one queue, 256-wide column tiles only.
                             MoE (fused): 0 = one queue of M-tiles, expert by
                             expert, each expert's M-tiles in readiness order (the
                             latest arrival position among the source blocks their
                             rows come from); 1 = the same order in 8
                             per-XCD queues keyed by tile column (when the tile
                             columns split evenly over them: the tiles on one XCD
                             share the same column blocks of the expert weights);
                             2 = one queue in expert order; 3 = expert order with
                             every tile held until all copy items have landed;
                             4 = as 3 in per-XCD queues; 5 = expert order in
                             per-XCD queues.
                             GEMM+RS/AR: 0 = one queue, tile row after tile row
                             (in landing order with an arrival schedule);
                             1 = 8 per-XCD queues where the tile columns split
                             evenly over them: queue x holds columns x, x + 8,
                             ... of band after band of tile rows (about one
                             tile per workgroup of an XCD per band), so the
                             tiles on one XCD share few operand blocks in its
                             L2; else as 0.  Any other value: MK_ERR_INVALID. */
} mk_launch;

/* ---------------------------------------------------------------------------
 * AllGather -> GEMM  ([P1] "Los cinco núcleos fusionados", row AllGather + GEMM)
 *
 * Each of R ranks holds a shard A_r [m_shard x K] (bf16).  The gathered
 * A = [A_0; A_1; ...; A_{R-1}] (rank order, M = R*m_shard rows) is assembled
 * in `a_gathered` [M x K] by copy workgroups, unit by unit (unit_rows rows
 * each) under `arrival`; compute workgroups produce C = A @ B, B [K x N]
 * bf16, C [M x N] of `c_dtype` (fp32 accumulation, one final rounding to
 * nearest-even for bf16), starting each output tile as soon as the units
 * covering its rows have landed.
 *   arrival NULL = one unit per shard, issued in rank order, no delay.
 *   tile_log (optional): per tile in queue order, 8 int32 {tile_row,
 *   tile_col, first unit, last unit, workgroup, t_take, t_ready, t_done}:
 *   when the tile was taken from the queue, when its units had landed, and
 *   when its stores were issued (low 32 bits of the device wall clock).
 *   With 192-wide column tiles (queue_mode 0) tile_col counts the 256-wide
 *   ones first.  The number of tiles depends on the tile and the plan; at
 *   most ceil(M/128) * ceil(N/128) records are written.
 *   copy_log (optional): per copy work item (in queue order), 8 int32
 *   {unit, part, workgroup, t_start, t_end, 0, 0, 0}.
 * ------------------------------------------------------------------------- */
/* Workspace bytes: a 256-byte header, 256 arrival counters and, for a single
 * 128-row tile row (R*m_shard <= 128) with K % 128 == 0, room for the packed
 * copy of A (128 x K bf16) that tile 11 reads. */
size_t mk_ag_gemm_workspace(int R, int64_t m_shard, int64_t K, int64_t N, int32_t unit_rows);
int mk_ag_gemm(const void* const* a_shards, int R, int64_t m_shard, int64_t K,
               const void* B, int64_t N, void* C, int c_dtype, void* a_gathered,
               const mk_arrival* arrival, const mk_launch* launch,
               void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * AllGather -> GEMM without a workspace argument.
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation, arguments and results as mk_ag_gemm, but the workspace is a
 * fixed 4 KiB device array inside the library (one per GPU, held until the
 * process ends); the call allocates nothing.  On its first call on a device
 * the library looks up that array's address (hipGetSymbolAddress, with the
 * device current); every call clears it with a fill kernel on `stream` before
 * the operation's kernels (no memset node).
 *   All calls on one GPU share the array: calls that overlap on one GPU (on
 *   different streams without ordering between them, or from several host
 *   threads) race and give undefined results.  Order them.
 *   The array holds the header and the arrival counters (1280 bytes; the
 *   packed copy of A that tile 11 reads is not kept, so that tile is not
 *   used here: MK_ERR_UNSUPPORTED if launch->tile asks for it); it must fit in 4 KiB, else
 *   MK_ERR_UNSUPPORTED.  arrival->withhold must be -1 (MK_ERR_INVALID
 *   otherwise): with no workspace there is no status for mk_poll_status, so
 *   a watchdog expiry is not reported (the kernels still exit).
 * ------------------------------------------------------------------------- */
int mk_ag_gemm_noalloc(const void* const* a_shards, int R, int64_t m_shard, int64_t K,
                       const void* B, int64_t N, void* C, int c_dtype, void* a_gathered,
                       const mk_arrival* arrival, const mk_launch* launch, void* stream);

/* ---------------------------------------------------------------------------
 * GEMM -> ReduceScatter  ([P1] "Los cinco núcleos fusionados", row
 * GEMM + ReduceScatter)
 *
 * This GPU's contribution is A @ B (A [M x K], B [K x N] bf16, fp32
 * accumulate).  The other R-1 contributions are fp32 partial sums
 * partials[p] [M x N] (resident device buffers standing for the peers).  The
 * reduced S = A@B + P_1 + ... + P_{R-1} (summed in fp32 in exactly that
 * order) is scattered by row block: out_owner[r] [(M/R) x N] of `out_dtype`
 * receives rows [r*M/R, (r+1)*M/R).  Each output tile is reduced and written
 * to its owner as soon as its GEMM tile is done and the partial sums of its
 * rows have arrived.
 *   arrival  NULL: every partial sum is there from the start (read in place).
 *            Otherwise the partial sums arrive in units u = (p-1)*(M/unit_rows)
 *            + b, rows [b*unit_rows, (b+1)*unit_rows) of partials[p-1] (peer
 *            p = 1..R-1), n_units = (R-1)*M/unit_rows (unit_rows must divide
 *            M), released by copy workgroups in arrival->order no earlier than
 *            delay_ns[u] after the first copy workgroup starts; a tile's
 *            reduction waits for the units under its rows.  Needs R >= 2.
 *   p_landing  NULL, or (arrival given) a host array of R-1 device pointers,
 *            each [M x N] fp32, caller-owned and overwritten: the copy
 *            workgroups move each unit's rows from partials[p-1] into
 *            p_landing[p-1] (items of launch->copy_kib KiB, default 1 MiB) and
 *            the reduction reads the landing buffers.  NULL with an arrival:
 *            a unit is only released at its time and read in place.
 *   launch->n_copy: copy workgroups (default: every workgroup copies first,
 *            then computes); copy_log as for mk_ag_gemm, {unit, part,
 *            workgroup, t_start, t_end, 0, 0, 0}, t_end taken once the item's
 *            stores are complete and before its release.
 *   The schedule decides when tiles are reduced, never the result: the sum
 *   order is fixed, so every schedule, role split and landing choice gives
 *   the same bits.
 *   M must be divisible by R; M/R must be a multiple of the tile height.
 *   tile_log (optional): per output tile id (tile_row*tiles_n + tile_col),
 *   8 int32 {owner, production rank, reducing workgroup, first row block of
 *   its rows (-1 without arrival), t_take (the reduction starts waiting for
 *   its partial sums), t_ready (they have landed), t_done (stores issued),
 *   0} (low 32 bits of the device wall clock).
 *   Errors: MK_ERR_SCHEDULE for a bad schedule (not a permutation, unit_rows
 *   not dividing M, delays over 1 s, R < 2); MK_ERR_INVALID for landing
 *   buffers without a schedule; MK_ERR_UNSUPPORTED for more than
 *   MK_MAX_UNITS units or (with a schedule) more than MK_MAX_UNITS tile rows.
 * ------------------------------------------------------------------------- */
size_t mk_gemm_rs_workspace(int64_t M, int64_t K, int64_t N, int R, int out_dtype);
int mk_gemm_rs(const void* A, const void* B, int64_t M, int64_t K, int64_t N,
               const float* const* partials, int R, void* const* out_owner, int out_dtype,
               const mk_arrival* arrival, float* const* p_landing,
               const mk_launch* launch, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * GEMM -> AllReduce  ([P1] "Los cinco núcleos fusionados", row
 * GEMM + AllReduce)
 *
 * The same contributions and the same fp32 sum S = A@B + P_1 + ... + P_{R-1}
 * (in exactly that order) as mk_gemm_rs, delivered whole to every rank:
 * out_rank[r] [M x N] of `out_dtype` receives all of S for r = 0..R-1 (the
 * reduce-scatter followed by the all-gather of the owner blocks; on one GPU
 * the R outputs stand for the R ranks' buffers).  Each output tile is reduced
 * and written to every rank as soon as its GEMM tile is done and its partial
 * sums have arrived.  M need not be divisible by R.  Arrival schedule,
 * landing buffers, workspace, launch options and errors as for mk_gemm_rs;
 * tile_log records owner 0 for every tile.
 * ------------------------------------------------------------------------- */
size_t mk_gemm_ar_workspace(int64_t M, int64_t K, int64_t N, int R, int out_dtype);
int mk_gemm_ar(const void* A, const void* B, int64_t M, int64_t K, int64_t N,
               const float* const* partials, int R, void* const* out_rank, int out_dtype,
               const mk_arrival* arrival, float* const* p_landing,
               const mk_launch* launch, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * MoE dispatch -> grouped GEMM  ([P1] "Los cinco núcleos fusionados", row
 * Envío MoE + GEMM)
 *
 * Routing: topk_idx[t, :] = the k experts with the largest logits[t, :]
 * (fp32, finite), descending; equal values (+0 == -0) go to the lower id.
 * Dispatch: counts[e] = tokens choosing e; offsets = exclusive prefix sum
 * (E+1 entries); perm[p] = t*k + j for the p-th (token, slot) pair in
 * (expert, token) ascending order.  n_local_rows[0] = offsets[expert_begin+L]
 * - offsets[expert_begin].
 * Landing: Xs is the receive buffer [T x H] bf16: row t of Xs is X[t] for
 * every token t with at least one local expert (received once, however many
 * local experts it picked); the other rows are not written.  Copy workgroups
 * write the rows as the tokens' source blocks land (blocks of
 * arrival->unit_rows tokens, issued in arrival->order).  Grouped GEMM: for
 * local expert e, Y row q (q = p - offsets[expert_begin] for the pair at
 * position p) = Xs[perm[p] / k] @ W[e] (W[e] [H x F] bf16), each M-tile
 * starting once all of its rows have landed.
 *   Xs has room for T rows [x H] bf16 (T * H * 2 < 2^31 bytes), Y for
 *   T*min(k, L) rows [x F].
 *   tile_log (optional): per output tile q = m_tile*ceil(F/BN) + tile_col
 *   (BN the tile width of the chosen tile), 8 int32 {local expert, first row
 *   (expert-relative), rows, landed count seen, workgroup, t_take, t_ready,
 *   t_done} (times as in the AG tile log).
 *   copy_log (optional): per copy work item (source block x part of 4 or
 *   fewer tokens, in queue order), 8 int32 {block, part, workgroup, t_start,
 *   t_end, local pairs, t_indexed, t_copied}: t_indexed when the item's
 *   pairs were placed, t_copied when its stores were issued.
 * ------------------------------------------------------------------------- */
size_t mk_moe_dispatch_gemm_workspace(int64_t T, int64_t H, int E, int k, int L, int64_t F);
int mk_moe_dispatch_gemm(const void* X, const float* logits, int64_t T, int64_t H, int E, int k,
                         const void* const* W, int expert_begin, int L, int64_t F,
                         int32_t* topk_idx, int32_t* counts, int32_t* offsets, int32_t* perm,
                         int32_t* n_local_rows, void* Xs, void* Y, int y_dtype,
                         const mk_arrival* arrival, const mk_launch* launch,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * MoE gate GEMM  (the step before [P1] "Los cinco núcleos fusionados", row
 * Envío MoE + GEMM: routing ranks one logit per token and expert; the pages
 * start from those logits)
 *
 * logits [T x E] fp32 = X [T x H] bf16 @ W_gate [H x E] bf16 (column e is
 * expert e's gate vector), fp32 accumulation of the exact bf16 products, no
 * bias.  The output feeds mk_moe_dispatch_gemm's `logits`.  When the output
 * has fewer 128 x 128 tiles than the device has CUs, the contraction is cut
 * into up to 8 parts whose fp32 sums are parked in the workspace and added in
 * part order by the part that finishes last (the result does not depend on
 * timing).  Workspace: mk_moe_gate_workspace(T, H, E) bytes, zero-filled
 * before first use (mk_workspace_init); every call leaves it ready for the
 * next.  Limits: H and E multiples of 8, E <= MK_MAX_EXPERTS.
 * ------------------------------------------------------------------------- */
size_t mk_moe_gate_workspace(int64_t T, int64_t H, int E);
int mk_moe_gate(const void* X, const void* W_gate, int64_t T, int64_t H, int E, float* logits,
                void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * MoE combine  (the step after [P1] "Los cinco núcleos fusionados", row
 * Envío MoE + GEMM, which the pages do not describe)
 *
 * For every token t of this rank: out[t] = sum_j g[t, j] * Y_row(t, j), j in
 * slot order, fp32 arithmetic, one final rounding to out_dtype, where
 *   g[t, :] = softmax over logits[t, topk_idx[t, 0..k-1]] (fp32 [T x E]),
 *   Y_row(t, j) = the expert output of pair (t, j) at its dispatch position
 *   pos (perm[pos] = t*k + j): row pos - offsets[expert_begin] of y_local
 *   when offsets[expert_begin] <= pos < offsets[expert_begin + L] (the
 *   local grouped-GEMM output, bf16
 *   [y_local_rows x F]), otherwise row pos of y_peer (the outputs the other
 *   ranks return, bf16 [T*k x F]; rows of local positions are not read).
 * topk_idx, offsets and perm are mk_moe_dispatch_gemm's outputs (device).
 * out [T x F] of out_dtype.  A position outside a buffer reads zero.
 * Workspace: mk_moe_combine_workspace(T, k) bytes (the inverse permutation;
 * no zero fill needed).  Limits: F % 8 == 0, T*k*F*2 and y_local_rows*F*2
 * below 2^32 bytes.
 * ------------------------------------------------------------------------- */
size_t mk_moe_combine_workspace(int64_t T, int k);
int mk_moe_combine(const float* logits, int64_t T, int E, int k, const int32_t* topk_idx,
                   const int32_t* offsets, const int32_t* perm, int expert_begin, int L,
                   const void* y_local, int64_t y_local_rows, const void* y_peer, int64_t F,
                   void* out, int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Ring attention  ([P1] "Los cinco núcleos fusionados", row Ring Attention)
 *
 * R ranks each hold S consecutive tokens of a sequence: rank r's keys and
 * values k_shards[r], v_shards[r], each [H][S][D] bf16 (H heads, D = 128).
 * This GPU is rank 0 with queries Q [H][S][D] bf16.  Its output is full
 * (non-causal) attention of its queries over all R*S keys:
 *   O[h, i] = sum_j softmax_j(Q[h, i] . K[h, j] / sqrt(D)) V[h, j]
 * written to O [H][S][D] of `o_dtype` (fp32 arithmetic, one final rounding).
 * The shards arrive round a ring: step s = 1..R-1 delivers rank (R-s) mod R's
 * shard.  Copy workgroups move unit u = (s-1)*H + h (head h's keys and
 * values of step s) from the owner's buffers into the receive buffers
 * k_recv, v_recv [(R-1)][H][S][D] bf16 (caller-owned, overwritten), in
 * arrival->order; the attention workgroups consume the own shard first and
 * then step after step, each head's step s as soon as its unit has landed
 * (online softmax in ring order).
 *   arrival NULL = units in index order (step by step), no delay; otherwise
 *   n_units = (R-1)*H and unit_rows = 1.  R = 1 takes no arrival and no
 *   receive buffers (NULL allowed).
 *   launch: mode 0 fused, 1 unfused (all copies, then attention); grid,
 *   n_copy (default: every workgroup copies first), spin_limit_us,
 *   tile_log, copy_log.  Other fields are ignored.
 *   tile_log (optional): per compute item q (head_order[q / ceil(S/128)],
 *   query block q % ceil(S/128)) 8 int32 {head, query block, R, 0,
 *   workgroup, t_take, t_ready (last unit acquired), t_done}.
 *   copy_log (optional): per copy item w = 2*position + part (0 keys, 1
 *   values), 8 int32 {unit, part, workgroup, t_start, t_end, 0, 0, 0}.
 *   Limits: D = 128, H <= 256, S <= 2^20, H*S <= 2^26, (R-1)*H <= MK_MAX_UNITS.
 * ------------------------------------------------------------------------- */
size_t mk_ring_attn_workspace(int H, int64_t S, int R);
int mk_ring_attn(const void* Q, const void* const* k_shards, const void* const* v_shards, int R, int H,
                 int64_t S, int D, void* O, int o_dtype, void* k_recv, void* v_recv,
                 const mk_arrival* arrival, const mk_launch* launch, void* workspace,
                 size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Measurement (the rates the operations are compared with; not part of the
 * hot path)
 *
 * mk_peak_mfma: an MFMA-only loop on every CU (two 256-thread workgroups per
 * CU, each wave `iters` rounds of 16 bf16 32x32x16 MFMA updates on 8
 * independent accumulators, the operands rotating through 8 random register
 * fragments so that they switch as in a GEMM on real data).  *flops = floating-point operations of the launch (time
 * it with events on `stream`); *waves = waves launched.  The workspace
 * (mk_peak_workspace() bytes, device) receives at byte offset 256 one pair
 * of uint64 per wave: {core clock ticks, wall clock ticks} of its loop, from
 * which the average engine clock under a full MFMA load follows.
 * mk_peak_hbm: mode 0 reads `bytes` of src (16-byte loads, every CU), mode 1
 * copies them to dst; *bytes_moved = bytes read plus written (the region is
 * rounded down to whole 64 KiB per workgroup).  Limits: iters in [1, 2^24];
 * each workgroup's region below 2 GiB.
 * ------------------------------------------------------------------------- */
size_t mk_peak_workspace(void);
int mk_peak_mfma(int iters, void* workspace, size_t workspace_bytes, double* flops, int* waves, void* stream);
int mk_peak_hbm(const void* src, void* dst, size_t bytes, int mode, void* workspace, size_t workspace_bytes,
                double* bytes_moved, void* stream);

/* ---------------------------------------------------------------------------
 * Cross-XCD message-passing litmus test (diagnostic)
 *
 * Runs the publication protocol every fused kernel relies on between pairs
 * of workgroups on different XCDs: in each of `rounds` rounds the producer
 * of a pair overwrites `words` uint32 of payload with the round number
 * (plain stores), publishes them (every wave waits for its stores, barrier,
 * one agent-scope release, relaxed flag store), and the consumer waits for
 * the flag with relaxed loads, takes one agent-scope acquire, reads the
 * payload and counts the words that do not hold the round number, then
 * acknowledges.  fenced = 0 leaves out the release and the acquire (the
 * count may then be non-zero: stale data, no fault).
 *   result: device uint32[4], 16-byte aligned, written by the call: {stale
 *   words seen, pairs whose two workgroups ran on different XCDs, mask of the
 *   producers' XCDs, mask of the consumers' XCDs}.
 *   workspace: mk_litmus_workspace(pairs, words) bytes, cleared by the call
 *   (fill kernel on `stream`).  Every wait is bounded by spin_limit_us (0 =
 *   2 s); an expiry is reported by mk_poll_status.
 *   Limits: pairs in [1, 64] and 2 * pairs <= CUs; words, rounds in [1, 2^20].
 * ------------------------------------------------------------------------- */
size_t mk_litmus_workspace(int pairs, int words);
int mk_litmus_mp(int pairs, int words, int rounds, int fenced, uint32_t* result, void* workspace,
                 size_t workspace_bytes, uint32_t spin_limit_us, void* stream);

/* ---------------------------------------------------------------------------
 * Per-shape defaults  ([P1] "¿Qué hace mKernel?": how many workgroups each
 * role gets, and the tile, are chosen per shape)
 *
 * mk_plan fills *out with the launch options an operation uses for a shape
 * when the caller leaves them 0 -- the same functions the entry points call
 * for those fields -- so a caller can read, log, adjust and pass them back
 * as the launch.  Fields set: tile (the tile id), n_copy (0: the default
 * split, which depends on the grid: AG three quarters of it copy first,
 * other operations every workgroup), n_reduce (0: each compute workgroup
 * reduces the tiles it produced), copy_kib (AG: the copy item size in KiB, rounded
 * up; the entry point then rounds items to whole rows; RS/AR: 1024),
 * queue_mode (0); every other field is zero.
 *   op MK_OP_AG_GEMM: M = R * m_shard, N, K as in mk_ag_gemm (R >= 1); the
 *     tile assumes a caller workspace (mk_ag_gemm_noalloc keeps tile 9 where
 *     this gives 11); the item size uses the current device's CU count, or
 *     256 CUs when no device is present.
 *   op MK_OP_GEMM_RS / MK_OP_GEMM_AR: M, N, K and R as in mk_gemm_rs.
 *   op MK_OP_MOE: N = F, K = H (M and R unused: routing decides the rows).
 * Returns MK_OK, or MK_ERR_INVALID (unknown op, NULL out, non-positive
 * dimension).  No GPU work.
 * ------------------------------------------------------------------------- */
enum { MK_OP_AG_GEMM = 0, MK_OP_GEMM_RS = 1, MK_OP_GEMM_AR = 2, MK_OP_MOE = 3 };
int mk_plan(int op, int64_t M, int64_t N, int64_t K, int R, mk_launch* out);

/* mk_ag_column_plan: the column tiles mk_ag_gemm uses with the 8-wave 256x256
 * tile (tile 10) and queue_mode 0 on `grid` workgroups for M rows and N
 * columns: *tn_wide tiles 256 wide, then *tn_narrow tiles 192 wide, per tile
 * row (the last tile may be ragged).  A mix is chosen when a greedy schedule
 * of the one tile queue (wide tiles first, a narrow tile costing 0.8 of a
 * wide one) finishes at least 3 % earlier than 256-wide tiles alone; with more
 * than 8 tiles per workgroup the plan keeps 256-wide tiles.  grid is the
 * workgroup count of the launch (the CU count at one workgroup per CU).
 * Returns MK_OK, or MK_ERR_INVALID (NULL outputs, non-positive M, N or grid).
 * No GPU work. */
int mk_ag_column_plan(int64_t M, int64_t N, int grid, int* tn_wide, int* tn_narrow);

/* ---------------------------------------------------------------------------
 * Support
 * ------------------------------------------------------------------------- */
/* Zero-fill a workspace with a fill kernel (no memset node), asynchronously. */
int mk_workspace_init(void* workspace, size_t workspace_bytes, void* stream);
/* Synchronise `stream`; return MK_ERR_TIMEOUT (and clear it) if any kernel of a
 * previous call on this workspace hit its watchdog, else MK_OK. */
int mk_poll_status(void* workspace, void* stream);
const char* mk_status_string(int status);

/* Rate of the device wall clock that stamps the logs, in kHz (100000 on
 * gfx950), for the current HIP device; negative mk_status on failure. */
int mk_wall_clock_khz(void);
const char* mk_last_error(void);
/* Name of tile configuration `id` (NULL if out of range); id 0 is "auto". */
const char* mk_tile_name(int id);
int mk_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
