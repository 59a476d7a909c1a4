// MoE dispatch -> grouped GEMM.
//
// [P1] "Los cinco núcleos fusionados", row Envío MoE + GEMM: tokens are routed
// to the ranks of their experts (all-to-all) and the per-expert grouped GEMM
// runs in the same kernel on the tokens as they land, with no staging round
// trip.  Here each token with at least one local expert lands once, in row
// t of the receive buffer Xs (a rank receives a token once, however many of
// its experts the token picked), and the grouped GEMM gathers each expert's
// rows from Xs through the dispatch permutation, tile by tile as they arrive.
//
// Kernels, in stream order:
//   route_kernel   one wave per token: top-k of the fp32 logits by k rounds of
//                  a wave-wide arg-max (ties to the lower expert id); then, per
//                  block of 64 tokens, each expert's count and each pair's rank
//                  among the block's pairs for that expert (token order).
//   scan_kernel    one workgroup: per expert, exclusive prefix of the block
//                  counts (token order), totals, the exclusive expert prefix
//                  (offsets) and the grouped-GEMM M-tile table of the local
//                  experts.  Everything is integer and deterministic.
//   moe_kernel     persistent.  copy role: source blocks in arrival order; for
//                  each (token, slot) write perm; copy each token with a local
//                  expert into its row of Xs, then count each of its local
//                  pairs into its M-tile's arrival counter (release).  compute
//                  role: grouped-GEMM tiles, each started once its M-tile's
//                  counter equals the tile's row count (acquire), its A rows
//                  read from Xs at the tokens that perm names.
#include <string.h>

#include <algorithm>
#include <type_traits>

#include "mk_device.h"
#include "mk_gemm_dma.h"
#include "mk_host.h"
#include "mk_tiles.h"

using namespace mk;

namespace {

constexpr int RB = 64;          // tokens per routing block
constexpr int ROUTE_NT = 1024;  // 16 waves, 4 tokens each

struct MoeWs {                  // device workspace layout (offsets in bytes)
  size_t block_cnt, rank, tile_base, tile_cnt, mt_order, kp_cnt, kp_slots, total;
};

// M-tiles ranked by readiness in one workgroup (a rank count over all pairs)
// up to this many; beyond it the queue keeps expert order.
constexpr int ORDER_CAP = 2048;

// K parts of a tail tile.  More parts shorten the parts but lengthen the
// finishing part's read-back of the parked sums (one workgroup reads
// parts x BM x BN x 4 bytes); at 256x256, 4 and 8 parts come out even, and 8
// would double the registers the read-back needs.
constexpr int KP_MAX = 4;

// The split tail (see moe_compute_role) holds at most one tile per four
// workgroups of the full grid, cut into parts that together number at most
// the full grid; occupancy x BM x BN <= 256 x 256 for every tile here, so the
// parked parts fit in n_cu x 256 KiB and the counters in n_cu words.
inline MoeWs moe_ws_layout(int64_t T, int E, int k, int L, int n_cu) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  MoeWs w;
  const int64_t nrb = (T + RB - 1) / RB;
  const int64_t rows = T * std::min(k, L);
  const int64_t max_tiles = rows / 128 + L + 1;
  w.block_cnt = sizeof(WsHeader);
  w.rank = up(w.block_cnt + (size_t)nrb * E * 4);
  w.tile_base = up(w.rank + (size_t)T * k * 4);
  w.tile_cnt = up(w.tile_base + (size_t)(L + 1) * 4 + 4);
  w.mt_order = up(w.tile_cnt + (size_t)max_tiles * 4);
  w.kp_cnt = up(w.mt_order + (size_t)max_tiles * 4);
  w.kp_slots = up(w.kp_cnt + (size_t)n_cu * 4);
  w.total = w.kp_slots + (size_t)n_cu * 256 * 256 * 4;
  return w;
}

// ------------------------------------------------------------------ routing
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// PL = logits per lane (E <= 64*PL), a compile-time bound so the per-round
// scan of a lane's logits has no dead slots.
template <int PL>
__global__ __launch_bounds__(ROUTE_NT) void route_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int32_t* __restrict__ topk, int32_t* __restrict__ block_cnt,
                                                         int32_t* __restrict__ rank) {
  __shared__ int16_t s_top[RB * MK_MAX_TOPK];
  __shared__ unsigned long long s_mask[MK_MAX_EXPERTS];   // bit tl set: token tl of the block chose e
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t_blk = blockIdx.x * RB;
  const int nt = min(RB, T - t_blk);
  for (int e = threadIdx.x; e < E; e += ROUTE_NT) s_mask[e] = 0ull;
  __syncthreads();
  // A wave routes its PER_WAVE tokens together: their arg-max rounds are
  // independent, so the shuffle chains of the tokens overlap.
  constexpr int PER_WAVE = RB / (ROUTE_NT / 64);
  const int tl0 = w * PER_WAVE;
  float v[PER_WAVE][PL];
  uint32_t taken[PER_WAVE];
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int t = t_blk + tl0 + i;
    taken[i] = 0;
#pragma unroll
    for (int s = 0; s < PL; ++s) {
      const int e = lane + 64 * s;
      const float x = (t < T && e < E) ? logits[(int64_t)t * E + e] : -__builtin_inff();
      v[i][s] = x == x ? x : -__builtin_inff();   // NaN ranks below every number
    }
  }
  for (int j = 0; j < k; ++j) {
    float bv[PER_WAVE];
    int bi[PER_WAVE];
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      bv[i] = -__builtin_inff();
      bi[i] = 0x7fffffff;
#pragma unroll
      for (int s = 0; s < PL; ++s) {
        const int e = lane + 64 * s;
        if (e < E && !((taken[i] >> s) & 1u) && better(v[i][s], e, bv[i], bi[i])) {
          bv[i] = v[i][s];
          bi[i] = e;
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) {
        const float ov = __shfl_xor(bv[i], off, 64);
        const int oi = __shfl_xor(bi[i], off, 64);
        if (better(ov, oi, bv[i], bi[i])) {
          bv[i] = ov;
          bi[i] = oi;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int tl = tl0 + i, t = t_blk + tl;
      if ((bi[i] & 63) == lane) taken[i] |= 1u << (bi[i] >> 6);
      if (lane == 0 && t < T) {
        topk[(int64_t)t * k + j] = bi[i];
        s_top[tl * MK_MAX_TOPK + j] = (int16_t)bi[i];
        atomicOr(&s_mask[bi[i]], 1ull << tl);
      }
    }
  }
  __syncthreads();
  // Per expert: count within this routing block, and the rank of each pair
  // (the number of earlier tokens of the block that chose the same expert; a
  // token's k experts are distinct, so this is its position in token order).
  for (int q = threadIdx.x; q < nt * k; q += ROUTE_NT) {
    const int tl = q / k, j = q - (q / k) * k;
    const int e = s_top[tl * MK_MAX_TOPK + j];
    rank[(int64_t)(t_blk + tl) * k + j] = __popcll(s_mask[e] & ((1ull << tl) - 1ull));
  }
  for (int e = threadIdx.x; e < E; e += ROUTE_NT) block_cnt[(int64_t)blockIdx.x * E + e] = __popcll(s_mask[e]);
}

// Arrival positions of the source blocks, for the readiness order.
struct ScanOrder {
  int T, block_tokens, n_blocks;
  uint16_t pos[MK_MAX_UNITS];     // pos[b] = issue position of source block b
};

// One workgroup of 1024 threads.  After the counts, offsets and M-tile table,
// the M-tiles are ranked expert by expert, and within an expert by readiness:
// the latest issue position among the source blocks their rows come from (an
// M-tile's rows are tokens in ascending order, so they span the routing blocks
// between those of its first and last row), ties in M-tile order.
// mt_order[i] = the i-th M-tile to queue.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ block_cnt, int nrb, int E,
                                                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ n_local, int eb, int L, int BM,
                                                    int32_t* __restrict__ tile_base, int32_t* __restrict__ mt_order,
                                                    const ScanOrder so) {
  __shared__ int32_t s[1024];
  __shared__ int32_t s_tb[MK_MAX_LOCAL + 1];
  __shared__ int32_t s_key[ORDER_CAP];
  const int e = threadIdx.x;
  int tot = 0;
  if (e < E) {
    // 16 independent loads per round trip, then the running sum over them
    for (int b0 = 0; b0 < nrb; b0 += 16) {
      int c[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) c[u] = b0 + u < nrb ? block_cnt[(int64_t)(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (b0 + u < nrb) {
          block_cnt[(int64_t)(b0 + u) * E + e] = tot;   // becomes the block offset within expert e
          tot += c[u];
        }
    }
    counts[e] = tot;
  }
  s[e] = e < E ? tot : 0;
  __syncthreads();
  // Inclusive Hillis-Steele scan over experts.
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = e >= off ? s[e - off] : 0;
    __syncthreads();
    s[e] += add;
    __syncthreads();
  }
  if (e < E) offsets[e + 1] = s[e];
  if (e == 0) offsets[0] = 0;
  __syncthreads();
  if (e == 0) {
    const int base = eb > 0 ? s[eb - 1] : 0;
    n_local[0] = s[eb + L - 1] - base;
    int acc = 0;
    for (int l = 0; l < L; ++l) {
      tile_base[l] = acc;
      s_tb[l] = acc;
      const int c = s[eb + l] - (eb + l > 0 ? s[eb + l - 1] : 0);
      acc += (c + BM - 1) / BM;
    }
    tile_base[L] = acc;
    s_tb[L] = acc;
  }
  __syncthreads();
  const int n_mt = s_tb[L];
  if (n_mt > ORDER_CAP) {
    for (int mt = e; mt < n_mt; mt += 1024) mt_order[mt] = mt;
    return;
  }
  // routing block holding row r of expert x: the last block whose offset
  // within x is <= r (empty blocks share their successor's offset)
  auto row_block = [&](int x, int r) {
    int lo = 0, hi = nrb - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (block_cnt[(int64_t)mid * E + x] <= r) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  for (int mt = e; mt < n_mt; mt += 1024) {
    int l = 0;
    while (l + 1 < L && s_tb[l + 1] <= mt) ++l;
    const int x = eb + l;
    const int cnt = s[x] - (x > 0 ? s[x - 1] : 0);
    const int r0 = (mt - s_tb[l]) * BM, r1 = min(r0 + BM, cnt) - 1;
    const int t_first = row_block(x, r0) * RB, t_last = min(so.T, (row_block(x, r1) + 1) * RB) - 1;
    int key = 0;
    for (int b = t_first / so.block_tokens; b <= t_last / so.block_tokens && b < so.n_blocks; ++b)
      key = max(key, (int)so.pos[b]);
    // expert first: the experts in flight at once stay few, so their weights
    // stay in the last-level cache (all of them do not); readiness within an
    // expert
    s_key[mt] = l * MK_MAX_UNITS + key;
  }
  __syncthreads();
  for (int mt = e; mt < n_mt; mt += 1024) {
    const int key = s_key[mt];
    int rk = 0;
    for (int i = 0; i < n_mt; ++i) rk += (s_key[i] < key) || (s_key[i] == key && i < mt);
    mt_order[rk] = mt;
  }
}

// ------------------------------------------------------ dispatch + grouped GEMM
enum { MODE_FUSED = 0, MODE_COPY = 1, MODE_GEMM = 2 };

struct MoeParams {
  const uint16_t* X;
  const uint16_t* W[MK_MAX_LOCAL];
  uint16_t* Xs;
  void* Y;
  const int32_t* topk;
  const int32_t* block_off;     // [nrb x E]
  const int32_t* rank;          // [T x k]
  const int32_t* counts;
  const int32_t* offsets;
  int32_t* perm;
  const int32_t* tile_base;     // [L+1]
  const int32_t* mt_order;      // [tiles] M-tiles in readiness order (fused queue)
  uint32_t* tile_cnt;           // [tiles] rows landed per M-tile
  WsHeader* hdr;
  int32_t* tile_log;
  int32_t* copy_log;
  uint64_t spin_limit;
  int T, H, E, k, L, F, eb, y_bf16;
  int n_blocks, block_tokens, part_tokens, parts;
  int mode, n_copy, tiles_n, withhold;
  int full_grid;                // CUs x occupancy of this kernel (the split plan's grid)
  int xcd_queues;               // whole tiles from per-XCD queues keyed by tile column
  int ready_order;              // fused queue in readiness order (else expert order)
  int hold;                     // fused: no tile before every copy item has landed
  int kp_len;                   // K-part counters in the workspace
  uint32_t* kp_cnt;             // [kp_len] parts of a split tail tile finished
  float* kp_slots;              // parked K parts
  uint16_t order[MK_MAX_UNITS];
  uint32_t delay_ticks[MK_MAX_UNITS];
};

// Tokens per copy item (at most): an item's fixed costs (index loads, a
// release, its counts) against how evenly the items spread over the copy
// workgroups; at the MoE shape 4 measured best (fused 0.767 ms, against 0.776
// with 8, 0.787 with 2 and 0.848 with 1; 16, one item per workgroup, 0.837).
constexpr int PART_TOKENS = 4;
constexpr int COPY_BATCH = PART_TOKENS < 8 ? PART_TOKENS : 8;   // token rows loaded before their stores
constexpr int SC1 = 16;                      // cache-policy bits: write through the L2

// Copy role.  An item is (source block, part of at most PART_TOKENS tokens).
// Its pairs' positions are computed first (perm for every pair; for a local
// expert its M-tile), grouped by token; then each token row with at least
// one local pair is loaded and stored once, into its own row of Xs (a token
// that picks several local experts is received once; the grouped GEMM reads
// the row for each of them).
__device__ __forceinline__ void moe_copy_role(const MoeParams& p, WsHeader* h, uint32_t* sb, int BM) {
  __shared__ int32_t s_tile[PART_TOKENS][MK_MAX_TOPK];
  __shared__ int32_t s_cnt[PART_TOKENS];
  const int tid = threadIdx.x, nt = blockDim.x;
  uint64_t t0 = 0;
  if (tid == 0) {
    const uint64_t now = now_ticks();
    const uint64_t old = atomicCAS((unsigned long long*)&h->t0, 0ull, (unsigned long long)now);
    t0 = old ? old : now;
  }
  const uint32_t n_work = (uint32_t)p.n_blocks * p.parts;
  const int cpr = p.H / 8;                        // 16-byte chunks per row
  const uint32_t row_bytes = (uint32_t)p.H * 2u;
  // One uniform exit at the top, next item taken at the bottom: every barrier
  // stays in wave-uniform control flow.
  uint32_t w = wg_bcast(tid == 0 ? add_relaxed(&h->copy_next, 1u) : 0u, sb);
  while (w < n_work) {
    const int j = w / p.parts, part = w % p.parts;
    const int blk = p.order[j];
    if (blk != p.withhold) {                       // a withheld block never lands (failure tests)
      uint32_t t_start = 0;
      if (tid == 0) {
        wait_until(t0 + p.delay_ticks[blk], p.spin_limit);
        t_start = (uint32_t)now_ticks();
      }
      if (tid < PART_TOKENS) s_cnt[tid] = 0;
      __syncthreads();
      const int t0k = blk * p.block_tokens + part * p.part_tokens;
      const int ntok = min(p.part_tokens, p.T - t0k);
      const int npair = ntok * p.k;
      // Positions of this part's pairs; perm for all of them, landing rows for local ones.
      if (tid < npair) {
        const int tl = tid / p.k, jj = tid % p.k, t = t0k + tl;
        const int e = p.topk[(int64_t)t * p.k + jj];
        const int pos = p.offsets[e] + p.block_off[(int64_t)(t / RB) * p.E + e] + p.rank[(int64_t)t * p.k + jj];
        p.perm[pos] = t * p.k + jj;
        const int l = e - p.eb;
        if (l >= 0 && l < p.L) {
          const int slot = atomicAdd(&s_cnt[tl], 1);
          s_tile[tl][slot] = p.tile_base[l] + (pos - p.offsets[e]) / BM;
        }
      }
      __syncthreads();
      const uint32_t t_indexed = (uint32_t)now_ticks();
      // Every token's row, COPY_BATCH rows at a time: all loads first (one
      // round trip per batch), then the stores into their rows of Xs.
      // Descriptors are bounded to one row: chunks past the row end load zero
      // and their stores are dropped, so there is no per-element guard.  A
      // token with no local pair moves nothing (its count is uniform: read
      // from LDS by every lane).  Stores write through the L2 (sc1): the
      // release below then has little to write back.
      int n = 0;                                   // local pairs of the item
#pragma unroll
      for (int tl = 0; tl < PART_TOKENS; ++tl) n += tl < ntok ? uni(s_cnt[tl]) : 0;
      for (int b0 = 0; b0 < PART_TOKENS; b0 += COPY_BATCH) {
        for (int c0 = 0; c0 < cpr; c0 += 4 * nt) {
          u32x4 v[COPY_BATCH][4];
#pragma unroll
          for (int i = 0; i < COPY_BATCH; ++i) {
            const int tl = b0 + i;
            const int cnt = uni(s_cnt[tl]);
            if (tl < ntok && cnt > 0) {
              const __amdgpu_buffer_rsrc_t src = make_rsrc(uni(p.X + (int64_t)(t0k + tl) * p.H), row_bytes);
#pragma unroll
              for (int cc = 0; cc < 4; ++cc) v[i][cc] = bload(src, (uint32_t)(c0 + cc * nt + tid) * 16u, 0);
            }
          }
#pragma unroll
          for (int i = 0; i < COPY_BATCH; ++i) {
            const int tl = b0 + i;
            if (tl < ntok && uni(s_cnt[tl]) > 0) {
              const __amdgpu_buffer_rsrc_t dst = make_rsrc(uni(p.Xs + (int64_t)(t0k + tl) * p.H), row_bytes);
#pragma unroll
              for (int cc = 0; cc < 4; ++cc) bstore<SC1>(dst, (uint32_t)(c0 + cc * nt + tid) * 16u, 0, v[i][cc]);
            }
          }
        }
      }
      const uint32_t t_copied = (uint32_t)now_ticks();
      // Release only (no acquire: a copier reads nothing that others publish,
      // and an L2 invalidate would drop the lines of GEMM tiles on this XCD).
      wg_release();
      // stores complete, not yet counted: a tile that sees the counts reads a later clock
      const uint32_t t_end = (uint32_t)now_ticks();
      if (tid < PART_TOKENS * MK_MAX_TOPK) {
        const int tl = tid / MK_MAX_TOPK, d = tid % MK_MAX_TOPK;
        if (tl < ntok && d < s_cnt[tl]) add_relaxed(&p.tile_cnt[s_tile[tl][d]], 1u);
      }
      if (tid == 0) add_relaxed(&h->aux[0], 1u);        // items landed in total
      if (p.copy_log && tid == 0) {
        int32_t* L = p.copy_log + 8 * (int64_t)w;
        L[0] = blk; L[1] = part; L[2] = (int32_t)blockIdx.x; L[3] = (int32_t)t_start;
        L[4] = (int32_t)t_end; L[5] = n; L[6] = (int32_t)t_indexed; L[7] = (int32_t)t_copied;
      }
      __syncthreads();
    }
    w = wg_bcast(tid == 0 ? add_relaxed(&h->copy_next, 1u) : 0u, sb);
  }
}

// Split tail: when the tiles leave a last round that fills at most a quarter
// of the full grid, those tail tiles are cut along K into `split` parts
// (a power of two up to KP_MAX that keeps the parts within the grid and divides
// H into 128-deep units) so the otherwise idle workgroups share them; each
// part parks its sums and the last part of a tile adds them in part order
// (see park_acc / store_parked_sum).  The plan depends only on the routed
// tile count and the device's full grid, so every launch option gives the
// same bits.
struct MoeSplit { uint32_t n_whole, n_items; int split; };
__device__ __forceinline__ MoeSplit moe_split_plan(uint32_t n_tiles, int full, int H) {
  MoeSplit sp{n_tiles, n_tiles, 1};
  const uint32_t tail = n_tiles % (uint32_t)full;
  if (n_tiles > (uint32_t)full && tail > 0 && tail * 4 <= (uint32_t)full && H % 128 == 0)
    for (int s2 = 2; s2 <= KP_MAX; s2 *= 2)
      if (tail * s2 <= (uint32_t)full && (H / 128) % s2 == 0) sp.split = s2;
  if (sp.split > 1) {
    sp.n_whole = n_tiles - tail;
    sp.n_items = sp.n_whole + tail * sp.split;
  }
  return sp;
}

// Half-height engine for the last M-tile of an expert that holds at most 128
// rows: a 256x256 tile would spend half its MFMAs on padding rows (at the MoE
// shape about a tenth of the M-tiles are such tails).  The 128x256 tile runs
// the same MFMA sequence per output element, so the bits do not change; it
// uses the same stage buffers (smaller stages).
template <class G> struct HalfTile { using type = void; };
template <bool I, int S> struct HalfTile<TileGemmD<256, 256, I, S, 4, 2, 256, true>> {
  using type = TileGemmD<128, 256, I, S, 4, 2, 256, true>;
};

template <class G, class SM>
__device__ __forceinline__ void moe_compute_role(const MoeParams& p, WsHeader* h, SM sm, uint32_t* sb) {
  using G2 = typename HalfTile<G>::type;
  const int tid = threadIdx.x;
  const int n_mt = (int)uni((uint32_t)p.tile_base[p.L]);
  const uint32_t n_tiles = (uint32_t)n_mt * p.tiles_n;
  const int base_local = p.offsets[p.eb];
  const uint32_t all_items = (uint32_t)p.n_blocks * p.parts;   // never reached with a withheld block
  const MoeSplit sp = moe_split_plan(n_tiles, p.full_grid, p.H);
  // Once every copy item has landed and this workgroup has taken an acquire
  // after seeing that, its later tiles need neither a wait nor an acquire
  // (each acquire invalidates the XCD's L2 under the other tiles there).
  bool all_landed = p.mode != MODE_FUSED;
  // Per-XCD queues (when the tile columns split evenly over the XCDs): queue
  // x holds the whole tiles of columns x, x + XQ, ... in queue order, so the
  // tiles on one XCD share the same column blocks of the expert weights in
  // its L2 whichever workgroups take them; a drained queue's workgroups help
  // the others, then all take the split tail items from the common counter.
  const bool xq_on = p.xcd_queues && p.tiles_n % XQ == 0;
  const int xc = p.tiles_n / XQ;                               // columns per queue and tile row
  const uint32_t whole_rows = sp.n_whole / (uint32_t)p.tiles_n, whole_rem = sp.n_whole % (uint32_t)p.tiles_n;
  auto qlen = [&](int x) -> uint32_t {
    uint32_t n = whole_rows * (uint32_t)xc;
    for (int i = 0; i < xc; ++i) n += (uint32_t)(x + XQ * i) < whole_rem ? 1u : 0u;
    return n;
  };
  XcdQueues xq(&h->aux[XQ_AUX]);
  auto next_item = [&]() -> uint32_t {
    uint32_t it = 0;
    if (tid == 0) {
      int x;
      uint32_t j;
      if (!xq_on) it = add_relaxed(&h->tile_next, 1u);
      else if (xq.take(qlen, x, j)) it = (j / xc) * (uint32_t)p.tiles_n + (uint32_t)(x + XQ * (int)(j % xc));
      else it = sp.n_whole + add_relaxed(&h->tile_next, 1u);
    }
    return wg_bcast(it, sb);
  };
  if (p.hold && !all_landed) {
    uint32_t ok = 1;
    if (tid == 0) {
      ok = wait_geq_sparse(&h->aux[0], all_items, h, p.spin_limit);
      if (ok) fence_acquire();
    }
    all_landed = wg_bcast(ok, sb) != 0u;            // on a watchdog expiry the per-tile waits give up too
  }
  G g;
  int l = 0;
  for (;;) {
    const uint32_t it = next_item();
    if (it >= sp.n_items) break;
    // work item -> tile q and K part kp (kp < 0: the whole tile)
    uint32_t q = it;
    int kp = -1;
    if (it >= sp.n_whole) {
      q = sp.n_whole + (it - sp.n_whole) / sp.split;
      kp = (int)((it - sp.n_whole) % sp.split);
    }
    const uint32_t t_take = (uint32_t)now_ticks();
    // queue slot -> M-tile: readiness order in the fused kernel, expert order
    // in the baseline's GEMM kernel
    const int slot = (int)(q / p.tiles_n), tn = (int)(q % p.tiles_n);
    const int mt = p.mode == MODE_FUSED && p.ready_order ? uni(p.mt_order[slot]) : slot;
    while (l + 1 < p.L && p.tile_base[l + 1] <= mt) ++l;
    while (l > 0 && p.tile_base[l] > mt) --l;
    const int e = p.eb + l;
    const int r0 = (mt - p.tile_base[l]) * G::BM;              // expert-relative first row
    const int rows = min(G::BM, p.counts[e] - r0);
    if (!all_landed) {
      uint32_t ok = 1, all = 0;
      if (tid == 0) {
        ok = wait_geq_relaxed(&p.tile_cnt[mt], (uint32_t)rows, h, p.spin_limit);
        if (ok) {
          all = ld_relaxed(&h->aux[0]) >= all_items;
          fence_acquire();
        }
      }
      const uint32_t v = wg_bcast(ok | (all << 1), sb);
      all_landed = (v >> 1) & 1u;
      if (!(v & 1u)) continue;
    }
    const uint32_t t_ready = (uint32_t)now_ticks();
    const int q0 = p.offsets[e] - base_local + r0;              // first Y row (local pair) of the tile
    const int n0 = tn * G::BN;
    const int kpart = p.H / sp.split, k0 = kp < 0 ? 0 : kp * kpart;
    const int64_t esz = p.y_bf16 ? 2 : 4;
    char* const Yt = (char*)p.Y + ((int64_t)q0 * p.F + n0) * esz;
    // A rows: the received token of each of the tile's pairs (pair id / k)
    const int32_t* const ix = p.perm + p.offsets[e] + r0;
    uint32_t done = 1;
    bool half = false;
    if constexpr (!std::is_void<G2>::value) {
      if (kp < 0 && rows <= G2::BM) {             // a whole tail tile of at most 128 rows
        G2 g2;
        g2.bind_rows(p.Xs, p.H, p.T, ix, p.k, rows, 0, p.W[l] + n0, p.F, p.F - n0, p.W[l] + (int64_t)p.H * p.F, p.H);
        g2.run(sm);
        store_tile<G2, 16>(g2, Yt, p.F, rows, p.F - n0, p.y_bf16);
        half = true;
      }
    }
    if (!half) {
      g.bind_rows(p.Xs, p.H, p.T, ix, p.k, rows, k0, p.W[l] + (int64_t)k0 * p.F + n0, p.F, p.F - n0,
                  p.W[l] + (int64_t)p.H * p.F, kp < 0 ? p.H : kpart);
      g.run(sm);
      if (kp < 0) {
        store_tile<G, 16>(g, Yt, p.F, rows, p.F - n0, p.y_bf16);   // through the L2: little for a release to write back
      } else {
        const uint32_t tq = q - sp.n_whole;                        // tail tile index
        float* slots = p.kp_slots + (int64_t)tq * sp.split * (G::BM * G::BN);
        park_acc(g, slots + (int64_t)kp * (G::BM * G::BN));
        wg_release();
        done = wg_bcast(tid == 0 ? (uint32_t)(add_relaxed(&p.kp_cnt[tq], 1u) == (uint32_t)(sp.split - 1)) : 0u, sb);
        if (done) {
          if (sp.split == 2) store_parked_sum<G, 2>(slots, Yt, p.F, rows, p.F - n0, p.y_bf16);
          else store_parked_sum<G, 4>(slots, Yt, p.F, rows, p.F - n0, p.y_bf16);
        }
      }
    }
    if (done && p.tile_log && tid == 0) {
      int32_t* L = p.tile_log + 8 * ((int64_t)mt * p.tiles_n + tn);
      L[0] = l; L[1] = r0; L[2] = rows;
      L[3] = p.mode == MODE_FUSED ? (int32_t)ld_relaxed(&p.tile_cnt[mt]) : rows;
      L[4] = (int32_t)blockIdx.x; L[5] = (int32_t)t_take; L[6] = (int32_t)t_ready;
      L[7] = (int32_t)(uint32_t)now_ticks();
    }
  }
}

__device__ __forceinline__ void moe_finish(const MoeParams& p, WsHeader* h, uint32_t* sb) {
  __syncthreads();
  uint32_t last = 0;
  if (threadIdx.x == 0) {
    fence_release();
    last = add_relaxed(&h->done, 1u) == gridDim.x - 1;
    if (last) fence_acquire();
  }
  last = wg_bcast(last, sb);
  if (!last) return;
  const int n_mt = p.tile_base[p.L];
  for (int i = threadIdx.x; i < n_mt; i += blockDim.x) st_relaxed(&p.tile_cnt[i], 0u);
  for (int i = threadIdx.x; i < p.kp_len; i += blockDim.x) st_relaxed(&p.kp_cnt[i], 0u);
  if (threadIdx.x == 0) {
    st_relaxed(&h->ticket, 0u);
    st_relaxed(&h->tile_next, 0u);
    st_relaxed(&h->copy_next, 0u);
    st_relaxed(&h->aux[0], 0u);
    for (int i = 0; i < XQ; ++i) st_relaxed(&h->aux[XQ_AUX + i], 0u);
    st_relaxed(&h->abort, 0u);
    __hip_atomic_store(&h->t0, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    st_relaxed(&h->done, 0u);
  }
}

template <class G, class SM>
__device__ __forceinline__ void moe_body(const MoeParams& p, SM sm, uint32_t* sb) {
  WsHeader* h = p.hdr;
  const uint32_t ticket = wg_bcast(threadIdx.x == 0 ? add_relaxed(&h->ticket, 1u) : 0u, sb);
  if (p.mode == MODE_COPY || (p.mode == MODE_FUSED && ticket < (uint32_t)p.n_copy)) moe_copy_role(p, h, sb, G::BM);
  if (p.mode != MODE_COPY) moe_compute_role<G>(p, h, sm, sb);
  moe_finish(p, h, sb);
}

template <class G>
__global__ __launch_bounds__(G::NT) void moe_kernel(const MoeParams p) {
  static_assert(G::NT >= PART_TOKENS * MK_MAX_TOPK, "one thread per pair of a copy item");
  __shared__ uint32_t sb[2];
  if constexpr (G::STAGES == 4) {
    __shared__ u32x4 a0[G::SA_U4], a1[G::SA_U4], a2[G::SA_U4], a3[G::SA_U4];
    __shared__ u32x4 b0[G::SB_U4], b1[G::SB_U4], b2[G::SB_U4], b3[G::SB_U4];
    moe_body<G>(p, Smem4{{a0, a1, a2, a3}, {b0, b1, b2, b3}}, sb);
  } else {
    __shared__ u32x4 lds[G::LDS_U4];
    moe_body<G>(p, Smem1{lds}, sb);
  }
}

template <class G>
int run_moe(MoeParams& p, const mk_launch& o, const mkh::DevInfo* d, hipStream_t st, int32_t* counts,
            int32_t* offsets, int32_t* n_local, int32_t* block_cnt, int nrb, const ScanOrder& so) {
  hipError_t e;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, block_cnt, nrb, p.E, counts, offsets, n_local,
                     p.eb, p.L, G::BM, const_cast<int32_t*>(p.tile_base), const_cast<int32_t*>(p.mt_order), so);
  if ((e = hipGetLastError()) != hipSuccess) return mkh::hip_fail(e, "scan kernel launch");
  p.tiles_n = (p.F + G::BN - 1) / G::BN;
  int occ = 0;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, moe_kernel<G>, G::NT, 0)) != hipSuccess)
    return mkh::hip_fail(e, "occupancy query");
  if (occ < 1) return mkh::fail(MK_ERR_UNSUPPORTED, "kernel does not fit on a CU");
  const int full = d->n_cu * occ;
  const int grid = o.grid > 0 ? std::min(o.grid, full) : full;
  const int n_work = p.n_blocks * p.parts;
  p.full_grid = full;
  if ((int64_t)full * G::BM * G::BN > (int64_t)d->n_cu * 256 * 256)
    return mkh::fail(MK_ERR_UNSUPPORTED, "tile slots exceed the workspace plan");
  if (o.mode >= 1) {   // unfused baseline: permute kernel, then grouped GEMM kernel
    // (measurement: mode 2 = routing and the permute kernel alone, 3 = routing
    // and the grouped GEMM kernel alone on the landing buffer as it is)
    if (o.mode != 3) {
      p.mode = MODE_COPY;
      p.n_copy = grid;
      hipLaunchKernelGGL(moe_kernel<G>, dim3(grid), dim3(G::NT), 0, st, p);
      if ((e = hipGetLastError()) != hipSuccess) return mkh::hip_fail(e, "permute kernel launch");
    }
    if (o.mode != 2) {
      p.mode = MODE_GEMM;
      p.n_copy = 0;
      hipLaunchKernelGGL(moe_kernel<G>, dim3(grid), dim3(G::NT), 0, st, p);
      if ((e = hipGetLastError()) != hipSuccess) return mkh::hip_fail(e, "grouped gemm kernel launch");
    }
    return MK_OK;
  }
  p.mode = MODE_FUSED;
  // Default: every workgroup starts as a copier (the landing copies are short
  // and bandwidth-bound; measured faster than a quarter of the grid copying).
  int n_copy = o.n_copy > 0 ? o.n_copy : grid;
  p.n_copy = std::min(std::min(n_copy, grid), n_work);
  hipLaunchKernelGGL(moe_kernel<G>, dim3(grid), dim3(G::NT), 0, st, p);
  if ((e = hipGetLastError()) != hipSuccess) return mkh::hip_fail(e, "fused kernel launch");
  return MK_OK;
}

}  // namespace

// Per-shape default tile (mk_plan reports it): 256x256, direct-to-LDS when
// H % 128 == 0; 128x128 when F < 256.  Only the 256x256 tile switches to the
// direct-to-LDS engine by default: at 128 rows the register-staged engine
// measured faster.
namespace mkp {
int moe_default_tile(int64_t H, int64_t F) {
  if (F < 256) return TILE_128x128;
  return TileGemmD<256, 256>::supports_k((int)H) ? TILE_256x256_DMA : TILE_256x256;
}
}  // namespace mkp

extern "C" size_t mk_moe_dispatch_gemm_workspace(int64_t T, int64_t H, int E, int k, int L, int64_t F) {
  (void)H; (void)F;
  if (T <= 0 || E <= 0 || k <= 0 || L <= 0) return sizeof(WsHeader);
  const mkh::DevInfo* d = mkh::dev_info();
  return moe_ws_layout(T, E, k, L, d ? d->n_cu : 256).total;
}

extern "C" int mk_moe_dispatch_gemm(const void* X, const float* logits, int64_t T, int64_t H, int E, int k,
                                    const void* const* W, int expert_begin, int L, int64_t F,
                                    int32_t* topk_idx, int32_t* counts, int32_t* offsets, int32_t* perm,
                                    int32_t* n_local_rows, void* Xs, void* Y, int y_dtype,
                                    const mk_arrival* arrival, const mk_launch* launch,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  using mkh::fail;
  if (!X || !logits || !W || !topk_idx || !counts || !offsets || !perm || !n_local_rows || !Xs || !Y)
    return fail(MK_ERR_INVALID, "NULL pointer argument");
  if (T < 1 || H < 8 || F < 8) return fail(MK_ERR_INVALID, "empty or too small shape");
  if (H % 8 || F % 8) return fail(MK_ERR_UNSUPPORTED, "H and F must be multiples of 8");
  if (E < 1 || E > MK_MAX_EXPERTS) return fail(MK_ERR_UNSUPPORTED, "E=%d outside [1,%d]", E, MK_MAX_EXPERTS);
  if (k < 1 || k > MK_MAX_TOPK || k > E) return fail(MK_ERR_INVALID, "k=%d outside [1,min(E,%d)]", k, MK_MAX_TOPK);
  if (L < 1 || L > MK_MAX_LOCAL) return fail(MK_ERR_UNSUPPORTED, "L=%d outside [1,%d]", L, MK_MAX_LOCAL);
  if (expert_begin < 0 || expert_begin + L > E) return fail(MK_ERR_INVALID, "local experts outside [0,E)");
  if (y_dtype != MK_BF16 && y_dtype != MK_F32) return fail(MK_ERR_INVALID, "y_dtype %d", y_dtype);
  const int64_t cap = T * std::min(k, L);
  // (Xs is read through 32-bit buffer offsets: T * H * 2 bytes at most 2^31)
  if (T * k > (1 << 30) || T * H * 2 >= (1ll << 31) || cap * F * 4 >= (1ll << 40) || H * F * 2 >= (1ll << 31) ||
      F > MK_MAX_COLS)
    return fail(MK_ERR_UNSUPPORTED, "dimension too large");
  for (int l = 0; l < L; ++l)
    if (!W[l] || !mkh::aligned16(W[l])) return fail(MK_ERR_INVALID, "W[%d] NULL or misaligned", l);
  if (!mkh::aligned16(X) || !mkh::aligned16(Xs) || !mkh::aligned16(Y))
    return fail(MK_ERR_INVALID, "X, Xs and Y must be 16-byte aligned");
  mkh::Schedule s;
  int rc = mkh::make_schedule(arrival, T, 1, &s);
  if (rc) return rc;
  if (!workspace) return fail(MK_ERR_WORKSPACE, "workspace is NULL");
  const size_t need0 = moe_ws_layout(T, E, k, L, 0).total;   // before the split-tail slots
  if (workspace_bytes < need0) return fail(MK_ERR_WORKSPACE, "workspace %zu bytes < %zu", workspace_bytes, need0);
  const mk_launch o = mkh::launch_opts(launch);
  if (o.mode < 0 || o.mode > 3) return fail(MK_ERR_INVALID, "mode %d", o.mode);
  if (o.grid < 0 || o.n_copy < 0) return fail(MK_ERR_INVALID, "negative grid or n_copy");
  if (o.queue_mode < 0 || o.queue_mode > 5) return fail(MK_ERR_INVALID, "queue_mode %d", o.queue_mode);
  const mkh::DevInfo* d = mkh::dev_info();
  if (!d) return MK_ERR_HIP;
  const MoeWs lay = moe_ws_layout(T, E, k, L, d->n_cu);
  if (workspace_bytes < lay.total) return fail(MK_ERR_WORKSPACE, "workspace %zu bytes < %zu", workspace_bytes, lay.total);
  const hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  int32_t* block_cnt = (int32_t*)(ws + lay.block_cnt);
  int32_t* rank = (int32_t*)(ws + lay.rank);
  const int nrb = (int)((T + RB - 1) / RB);

  if (E <= 256)
    hipLaunchKernelGGL(route_kernel<4>, dim3(nrb), dim3(ROUTE_NT), 0, st, logits, (int)T, E, k, topk_idx, block_cnt, rank);
  else if (E <= 512)
    hipLaunchKernelGGL(route_kernel<8>, dim3(nrb), dim3(ROUTE_NT), 0, st, logits, (int)T, E, k, topk_idx, block_cnt, rank);
  else
    hipLaunchKernelGGL(route_kernel<16>, dim3(nrb), dim3(ROUTE_NT), 0, st, logits, (int)T, E, k, topk_idx, block_cnt, rank);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return mkh::hip_fail(e, "route kernel launch");

  MoeParams p;
  memset(&p, 0, sizeof p);
  p.X = (const uint16_t*)X;
  for (int l = 0; l < L; ++l) p.W[l] = (const uint16_t*)W[l];
  p.Xs = (uint16_t*)Xs;
  p.Y = Y;
  p.topk = topk_idx;
  p.block_off = block_cnt;
  p.rank = rank;
  p.counts = counts;
  p.offsets = offsets;
  p.perm = perm;
  p.tile_base = (const int32_t*)(ws + lay.tile_base);
  p.tile_cnt = (uint32_t*)(ws + lay.tile_cnt);
  p.mt_order = (const int32_t*)(ws + lay.mt_order);
  p.kp_cnt = (uint32_t*)(ws + lay.kp_cnt);
  p.kp_slots = (float*)(ws + lay.kp_slots);
  p.kp_len = d->n_cu;
  p.hdr = (WsHeader*)workspace;
  p.tile_log = o.tile_log;
  p.copy_log = o.copy_log;
  p.spin_limit = mkh::spin_ticks(o, d);
  // queue_mode: 0 readiness order, 1 per-XCD queues (readiness order within
  // each), 2 expert order, 3 expert order with every tile held until all copy
  // items have landed (the baseline's phases inside one kernel), 4 as 3 with
  // per-XCD queues, 5 expert order in per-XCD queues
  p.xcd_queues = o.queue_mode == 1 || o.queue_mode >= 4;
  p.ready_order = o.queue_mode <= 1;
  p.hold = o.queue_mode == 3 || o.queue_mode == 4;
  p.T = (int)T; p.H = (int)H; p.E = E; p.k = k; p.L = L; p.F = (int)F; p.eb = expert_begin;
  p.y_bf16 = y_dtype == MK_BF16;
  p.n_blocks = s.n_units;
  p.block_tokens = s.unit_rows;
  p.part_tokens = std::min(PART_TOKENS, s.unit_rows);
  while (s.unit_rows % p.part_tokens) --p.part_tokens;
  p.parts = s.unit_rows / p.part_tokens;
  p.withhold = s.withhold;
  for (int j = 0; j < s.n_units; ++j) {
    p.order[j] = (uint16_t)s.order[j];
    p.delay_ticks[j] = (uint32_t)mkh::ns_to_ticks(s.delay_ns[j], d->wall_khz);
  }
  ScanOrder so;
  memset(&so, 0, sizeof so);
  so.T = (int)T;
  so.block_tokens = s.unit_rows;
  so.n_blocks = s.n_units;
  for (int b = 0; b < s.n_units; ++b) so.pos[b] = (uint16_t)s.pos[b];
  const int tile = o.tile ? o.tile : mkp::moe_default_tile(H, F);
  if (mk_is_dma_tile(tile) && !TileGemmD<256, 256>::supports_k((int)H))
    return fail(MK_ERR_UNSUPPORTED, "tile %d needs H %% 128 == 0", tile);
  if (tile == TILE_128x128_DMA8 || tile == TILE_256x256_DMA_W8 || tile == TILE_128x128_PC)
    return fail(MK_ERR_UNSUPPORTED, "tile %d is built for AllGather+GEMM only", tile);
  switch (tile) {
    case TILE_256x256: return run_moe<TileGemm<256, 256, 2, 2, true>>(p, o, d, st, counts, offsets, n_local_rows, block_cnt, nrb, so);
    case TILE_128x128: return run_moe<TileGemm<128, 128, 2, 2, true>>(p, o, d, st, counts, offsets, n_local_rows, block_cnt, nrb, so);
    case TILE_256x128: return run_moe<TileGemm<256, 128, 2, 2, true>>(p, o, d, st, counts, offsets, n_local_rows, block_cnt, nrb, so);
    case TILE_128x256: return run_moe<TileGemm<128, 256, 2, 2, true>>(p, o, d, st, counts, offsets, n_local_rows, block_cnt, nrb, so);
    case TILE_256x256_DMA: return run_moe<TileGemmD<256, 256, true, 4, 4, 2, 256, true>>(p, o, d, st, counts, offsets, n_local_rows, block_cnt, nrb, so);
    case TILE_128x128_DMA: return run_moe<TileGemmD<128, 128, true, 4, 4, 2, 128, true>>(p, o, d, st, counts, offsets, n_local_rows, block_cnt, nrb, so);
    case TILE_256x128_DMA: return run_moe<TileGemmD<256, 128, true, 4, 4, 2, 128, true>>(p, o, d, st, counts, offsets, n_local_rows, block_cnt, nrb, so);
    case TILE_128x256_DMA: return run_moe<TileGemmD<128, 256, true, 4, 4, 2, 256, true>>(p, o, d, st, counts, offsets, n_local_rows, block_cnt, nrb, so);
    default: return fail(MK_ERR_INVALID, "tile id %d", tile);
  }
}
