// AllGather -> GEMM as one persistent kernel.
//
// [P1] "Los cinco núcleos fusionados", row AllGather + GEMM: every rank holds a
// shard of A; while the shards are gathered, the local GEMM starts on the
// tiles whose rows have already arrived.  [P1] "¿Qué hace mKernel?": the
// kernel is persistent and its workgroups pick their roles themselves.
//
// Roles (by start-order ticket):
//   copy    tickets [0, n_copy): take (unit, part) work items in arrival order,
//           wait for the unit's release time, copy its rows from the owning
//           shard into the gathered buffer, publish with an agent-scope
//           release on the unit's arrival counter.  When the copy queue is
//           empty a copy workgroup becomes a compute workgroup.
//   compute take output tiles from a queue ordered by when their rows land,
//           acquire the arrival counters of the units under the tile, run the
//           MFMA K loop and store the tile.
// With the producer/consumer tile (a single 128-row tile row) the copy
// workgroups also write each part into a packed copy of A in MFMA operand
// order (in the workspace), which that tile reads instead of the gathered
// rows; it is published by the same release.
// Producers always hold earlier tickets than the consumers that wait on
// them, so the spin waits cannot deadlock even if the grid is not fully
// co-resident.  Every wait is bounded by a watchdog.
#include <string.h>

#include <algorithm>
#include <mutex>

#include "mk_device.h"
#include "mk_gemm_dma.h"
#include "mk_gemm_pc.h"
#include "mk_host.h"
#include "mk_tiles.h"

using namespace mk;

namespace {

enum { MODE_FUSED = 0, MODE_COPY = 1, MODE_GEMM = 2, MODE_PACK = 3 };

template <class G> struct PackedA { static constexpr bool value = false; };
template <int S, int P> struct PackedA<TileGemmPC<S, P>> { static constexpr bool value = true; };

// Narrow companion of the 8-wave 256x256 tile: 256 rows by 192 columns,
// the same LDS stages and DMA pattern (B loaded 256 wide, the columns past
// 192 not fetched), 4x2 waves of 64x96.  Tiles of the two widths can share
// one queue (every column block comes out bit for bit the same).
template <class G> struct NarrowTile { static constexpr bool ok = false; static constexpr int cn = G::BN; using type = G; };
template <bool I, int S> struct NarrowTile<TileGemmD<256, 256, I, S, 8>> {
  static constexpr bool ok = true;
  static constexpr int cn = 192;
  using type = TileGemmD<256, 256, I, S, 8, 4, cn>;
};

// Copy of one part (a contiguous block of n16 16-byte chunks: whole rows of
// kc chunks, the first being row row0 of the gathered A) that also writes
// every chunk into the packed copy of A: row r, chunk c at block r / 128,
// offset TileGemmPC::packed_offset(r % 128, c).  Chunks past the part are
// loaded as zeros and stored nowhere (their packed offset is made out of
// range).  store_ag false: the packed copy only (A already gathered).
template <int POLICY>
__device__ __forceinline__ void copy_pack_block(__amdgpu_buffer_rsrc_t src, __amdgpu_buffer_rsrc_t dst,
                                                __amdgpu_buffer_rsrc_t packed, int row0, int kc, int n16, int tid,
                                                int nt, bool store_ag) {
  const uint32_t block_bytes = (uint32_t)TileGemmPC<>::BM * (uint32_t)kc * 16u;
  for (int base = 0; base < n16; base += nt * COPY_UNROLL) {
    u32x4 v[COPY_UNROLL];
#pragma unroll
    for (int u = 0; u < COPY_UNROLL; ++u) v[u] = bload(src, (uint32_t)(base + u * nt + tid) * 16u, 0);
#pragma unroll
    for (int u = 0; u < COPY_UNROLL; ++u) {
      const int e = base + u * nt + tid;
      if (store_ag) bstore<POLICY>(dst, (uint32_t)e * 16u, 0, v[u]);
      const int r = row0 + e / kc, c = e % kc;
      const uint32_t off = e < n16 ? (uint32_t)(r >> 7) * block_bytes + TileGemmPC<>::packed_offset(r & 127, c) : OOB;
      bstore<POLICY>(packed, off, 0, v[u]);
    }
  }
}

struct AgParams {
  const uint16_t* shard[MK_MAX_RANKS];
  const uint16_t* B;
  void* C;
  uint16_t* Ag;
  uint16_t* Ap;         // packed copy of A for the producer/consumer tile, else NULL
  uint32_t ap_bytes;
  WsHeader* hdr;
  uint32_t* unit_cnt;   // [n_units] parts landed
  int32_t* tile_log;
  int32_t* copy_log;
  uint64_t spin_limit;
  int R, m_shard, M, K, N, c_bf16;
  int n_units, unit_rows, parts, part_rows;
  uint32_t part_bytes;
  int copy_wt;          // copy stores written through the L2
  int c_wt;             // output tiles written through the L2
  int mode, n_copy, tiles_m, tiles_n, n_tiles, withhold;
  // Column tiles: tn_wide of G::BN columns, then (NarrowTile) tn_narrow of
  // 192 columns; the queue holds all wide tiles (tile rows in landing order,
  // tn_wide per row: n_wide in all), then all narrow ones in the same order.
  int tn_wide, tn_narrow, n_wide;
  int xcd_queues;       // tiles from per-XCD queues (else one queue in landing order)
  uint16_t order[MK_MAX_UNITS];
  uint16_t rb_order[MK_MAX_UNITS];   // tile rows in landing order
  uint32_t delay_ticks[MK_MAX_UNITS];
};

// Role loops take their next work index at the bottom of the body and test it
// at the top (no `continue`), so every barrier stays in wave-uniform control
// flow.  Log timestamps are the low 32 bits of the 100 MHz wall clock.
__device__ __forceinline__ void ag_copy_role(const AgParams& p, WsHeader* h, uint32_t* sb) {
  const int tid = threadIdx.x, nt = blockDim.x;
  uint64_t t0 = 0;
  if (tid == 0) {
    const uint64_t now = now_ticks();
    const uint64_t old = atomicCAS((unsigned long long*)&h->t0, 0ull, (unsigned long long)now);
    t0 = old ? old : now;
  }
  const uint32_t n_work = (uint32_t)p.n_units * p.parts;
  const int n16 = p.part_rows * (p.K / 8);       // 16-byte chunks per part
  // MODE_PACK: only the packed copy, from the gathered rows, with no delays
  const bool pack_only = p.mode == MODE_PACK;
  const __amdgpu_buffer_rsrc_t packed = make_rsrc(uni(p.Ap), p.Ap ? p.ap_bytes : 0u);
  uint32_t w = wg_bcast(tid == 0 ? add_relaxed(&h->copy_next, 1u) : 0u, sb);
  while (w < n_work) {
    const int j = w / p.parts, part = w % p.parts;
    const int c = p.order[j];
    if (c != p.withhold || pack_only) {            // a withheld unit never lands (failure tests)
      uint32_t t_start = 0;
      if (tid == 0) {
        if (!pack_only) wait_until(t0 + p.delay_ticks[c], p.spin_limit);
        t_start = (uint32_t)now_ticks();
      }
      __syncthreads();
      // A part lies inside one shard, so it is one contiguous block on both sides.
      const int row0 = c * p.unit_rows + part * p.part_rows;
      // Buffer accesses bounded to the part: past its end loads return zero
      // and stores are dropped, so the loop needs no per-element guard (a
      // guarded store would be its own branch, and the compiler would wait for
      // every earlier memory operation before each one).
      const __amdgpu_buffer_rsrc_t dst = make_rsrc(uni(p.Ag + (int64_t)row0 * p.K), p.part_bytes);
      const __amdgpu_buffer_rsrc_t src =
          pack_only ? dst
                    : make_rsrc(uni(p.shard[row0 / p.m_shard] + (int64_t)(row0 % p.m_shard) * p.K), p.part_bytes);
      if (p.Ap) {
        if (p.copy_wt) copy_pack_block<16>(src, dst, packed, row0, p.K / 8, n16, tid, nt, !pack_only);
        else copy_pack_block<0>(src, dst, packed, row0, p.K / 8, n16, tid, nt, !pack_only);
      } else if (p.copy_wt) {
        copy_block<16>(src, dst, n16, tid, nt);
      } else {
        copy_block<0>(src, dst, n16, tid, nt);
      }
      // Release only: the copier never reads what others publish, so the
      // acquire half of a full fence (an L2 invalidate that would also drop
      // the lines of the GEMM tiles running on this XCD) is not needed.
      wg_release();
      if (tid == 0) {
        // t_end is stamped once every thread's stores are complete and before
        // the counters are raised, so a consumer that sees them reads a later clock
        const uint32_t t_end = (uint32_t)now_ticks();
        add_relaxed(&p.unit_cnt[c], 1u);
        add_relaxed(&h->aux[0], 1u);                 // parts landed in total
        if (p.copy_log && !pack_only) {
          int32_t* L = p.copy_log + 8 * (int64_t)w;
          L[0] = c; L[1] = part; L[2] = (int32_t)blockIdx.x;
          L[3] = (int32_t)t_start; L[4] = (int32_t)t_end;
        }
      }
    }
    w = wg_bcast(tid == 0 ? add_relaxed(&h->copy_next, 1u) : 0u, sb);
  }
}

template <class G, class SM>
__device__ __forceinline__ void ag_compute_role(const AgParams& p, WsHeader* h, SM sm, uint32_t* sb) {
  using GN = typename NarrowTile<G>::type;
  const int tid = threadIdx.x;
  const uint32_t all_parts = (uint32_t)p.n_units * p.parts;
  bool all_landed = (p.mode == MODE_GEMM);
  // Tile q < n_wide covers tile row rb_order[q / tn_wide] (tile rows in
  // landing order) and column tile q % tn_wide (G::BN wide); a later q the
  // narrow tiles after them, in the same row order.  Per-XCD queues (no
  // narrow tiles): queue x holds the tile rows at landing positions x, x +
  // XQ, x + 2*XQ, ..., each with all its columns, so the tiles that share an
  // A row block run on one XCD.
  XcdQueues xq(&h->aux[XQ_AUX]);
  const int tm_n = p.tiles_m, tn_n = p.tiles_n;
  auto qlen = [tm_n, tn_n](int x) -> uint32_t { return x < tm_n ? (uint32_t)((tm_n - 1 - x) / XQ + 1) * tn_n : 0u; };
  auto next_tile = [&]() -> uint32_t {
    uint32_t q = (uint32_t)p.n_tiles;
    if (tid == 0) {
      if (!p.xcd_queues) {
        q = add_relaxed(&h->tile_next, 1u);
      } else {
        int x;
        uint32_t j;
        if (xq.take(qlen, x, j)) q = (uint32_t)(x + XQ * (int)(j / tn_n)) * tn_n + j % tn_n;
      }
    }
    return wg_bcast(q, sb);
  };
  uint32_t q = next_tile();
  while (q < (uint32_t)p.n_tiles) {
    const bool narrow = NarrowTile<G>::ok && q >= (uint32_t)p.n_wide;
    const int qq = narrow ? (int)q - p.n_wide : (int)q, per_row = narrow ? p.tn_narrow : p.tn_wide;
    const int tm = p.rb_order[qq / per_row], tn = (narrow ? p.tn_wide : 0) + qq % per_row;
    const int m0 = tm * G::BM, n0 = narrow ? p.tn_wide * G::BN + (qq % per_row) * NarrowTile<G>::cn : tn * G::BN;
    const int u0 = m0 / p.unit_rows, u1 = (min(p.M, m0 + G::BM) - 1) / p.unit_rows;
    const uint32_t t_take = (uint32_t)now_ticks();
    uint32_t ok = 1;
    if (!all_landed) {
      uint32_t all = 0;
      if (tid == 0) {
        for (int u = u0; u <= u1 && ok; ++u) ok = wait_geq_relaxed(&p.unit_cnt[u], p.parts, h, p.spin_limit);
        // Once every part has landed (and the acquire below has been taken
        // after that), no later tile of this workgroup needs to wait.
        if (ok) {
          all = ld_relaxed(&h->aux[0]) >= all_parts;
          fence_acquire();                       // one acquire for all the tile's units
        }
      }
      const uint32_t v = wg_bcast(ok | (all << 1), sb);
      ok = v & 1u;
      all_landed = (v >> 1) & 1u;
    }
    if (ok) {                                      // else the watchdog expired: skip the tile
      const uint32_t t_ready = (uint32_t)now_ticks();
      const uint16_t* A = PackedA<G>::value ? p.Ap + (int64_t)tm * G::BM * p.K : p.Ag + (int64_t)m0 * p.K;
      const int64_t esz = p.c_bf16 ? 2 : 4;
      char* const C = (char*)p.C + ((int64_t)m0 * p.N + n0) * esz;
      if (!narrow) {
        G g;
        g.bind(A, p.K, p.M - m0, p.B + n0, p.N, p.N - n0, p.B + (int64_t)p.K * p.N, p.K);
        g.run(sm);
        // written through the L2: a copy workgroup's release on this XCD then
        // has no output lines to write back
        if (p.c_wt) store_tile<G, 16>(g, C, p.N, p.M - m0, p.N - n0, p.c_bf16);
        else store_tile(g, C, p.N, p.M - m0, p.N - n0, p.c_bf16);
      } else if constexpr (NarrowTile<G>::ok) {
        const int cols = min(NarrowTile<G>::cn, p.N - n0);   // the DMA fetches no column past these
        GN g;
        g.bind(A, p.K, p.M - m0, p.B + n0, p.N, cols, p.B + (int64_t)p.K * p.N, p.K);
        g.run(sm);
        if (p.c_wt) store_tile<GN, 16>(g, C, p.N, p.M - m0, cols, p.c_bf16);
        else store_tile(g, C, p.N, p.M - m0, cols, p.c_bf16);
      }
      if (p.tile_log && tid == 0) {
        int32_t* L = p.tile_log + 8 * (int64_t)q;
        L[0] = tm; L[1] = tn; L[2] = u0; L[3] = u1; L[4] = (int32_t)blockIdx.x;
        L[5] = (int32_t)t_take; L[6] = (int32_t)t_ready; L[7] = (int32_t)(uint32_t)now_ticks();
      }
    }
    q = next_tile();
  }
}

// Last workgroup out restores the workspace for the next call.
__device__ __forceinline__ void ag_finish(const AgParams& p, WsHeader* h, uint32_t* sb) {
  __syncthreads();
  uint32_t last = 0;
  if (threadIdx.x == 0) {
    fence_release();
    last = add_relaxed(&h->done, 1u) == gridDim.x - 1;
    if (last) fence_acquire();
  }
  last = wg_bcast(last, sb);
  if (!last) return;
  for (int i = threadIdx.x; i < p.n_units; i += blockDim.x) st_relaxed(&p.unit_cnt[i], 0u);
  if (threadIdx.x == 0) {
    st_relaxed(&h->ticket, 0u);
    st_relaxed(&h->tile_next, 0u);
    st_relaxed(&h->copy_next, 0u);
    st_relaxed(&h->abort, 0u);
    st_relaxed(&h->aux[0], 0u);
    for (int i = 0; i < XQ; ++i) st_relaxed(&h->aux[XQ_AUX + i], 0u);
    __hip_atomic_store(&h->t0, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    st_relaxed(&h->done, 0u);
  }
}

template <class G, class SM>
__device__ __forceinline__ void ag_body(const AgParams& p, SM sm, uint32_t* sb) {
  WsHeader* h = p.hdr;
  const uint32_t ticket = wg_bcast(threadIdx.x == 0 ? add_relaxed(&h->ticket, 1u) : 0u, sb);
  if (p.mode == MODE_COPY || p.mode == MODE_PACK || (p.mode == MODE_FUSED && ticket < (uint32_t)p.n_copy))
    ag_copy_role(p, h, sb);
  if (p.mode == MODE_FUSED || p.mode == MODE_GEMM) ag_compute_role<G>(p, h, sm, sb);
  ag_finish(p, h, sb);
}

template <class G>
__global__ __launch_bounds__(G::NT) void ag_kernel(const AgParams p) {
  __shared__ uint32_t sb[2];
  if constexpr (G::STAGES == 4) {
    __shared__ u32x4 a0[G::SA_U4], a1[G::SA_U4], a2[G::SA_U4], a3[G::SA_U4];
    __shared__ u32x4 b0[G::SB_U4], b1[G::SB_U4], b2[G::SB_U4], b3[G::SB_U4];
    ag_body<G>(p, Smem4{{a0, a1, a2, a3}, {b0, b1, b2, b3}}, sb);
  } else {
    __shared__ u32x4 lds[G::LDS_U4];
    ag_body<G>(p, Smem1{lds}, sb);
  }
}

}  // namespace

// Workspace: header | per-unit arrival counters | (when A is a single
// 128-row tile row with K % 128 == 0) the packed copy of A for the
// producer/consumer tile, 128 x K bf16.
struct AgWs { size_t pack, total; };
static bool ag_packs(int64_t M, int64_t K) { return M >= 1 && M <= TileGemmPC<>::BM && K >= 8 && TileGemmPC<>::supports_k((int)K); }
static AgWs ag_ws_layout(int64_t K, bool pack) {
  AgWs w;
  const size_t base = sizeof(WsHeader) + MK_MAX_UNITS * sizeof(uint32_t);
  w.pack = (base + 255) & ~(size_t)255;
  w.total = pack ? w.pack + (size_t)TileGemmPC<>::BM * (size_t)K * 2 : base;
  return w;
}

// ------------------------------------------------------------ per-shape defaults
// (mk_plan reports these; the entry point applies them to zero launch fields)
namespace mkp {

// Copy item size: the bytes of A over the CUs (at most 1 MiB, at least one
// row), so every workgroup starts with about one item: a single item's copy
// is bound by load and store latency (at M = 128, K = 8192 eight 256 KiB
// items took 40 us to land, 128 one-row items 12 us), and at M = 8192,
// K = 8192 items of 512 KiB measured 1-2 % faster than 1 MiB.
int64_t ag_default_item_bytes(int64_t M, int64_t K, int n_cu) {
  const int64_t row_bytes = K * 2;
  return std::min<int64_t>(1 << 20, std::max<int64_t>(row_bytes, M * row_bytes / std::max(n_cu, 1)));
}

bool ag_default_pack(int64_t M, int64_t K) { return ag_packs(M, K); }

// Finishing time of a greedy schedule on `grid` workgroups: W tiles of cost
// 1 first, then Nn of cost r, each taken by the first free workgroup.  After
// the wide tiles, grid - W % grid workgroups are free at k = W / grid and the
// others at k + 1; the narrow tiles take the earliest start times k + i r
// and k + 1 + i r.
static double ag_makespan(int64_t W, int64_t Nn, int grid, double r) {
  const int64_t k = W / grid, B = W % grid, A = grid - B;
  const double wide_end = (double)k + (B > 0 ? 1.0 : 0.0);
  if (Nn == 0) return wide_end;
  int64_t ia = 0, ib = 0, left = Nn;
  double last = 0.0;
  while (left > 0) {
    const double ta = (double)k + (double)ia * r, tb = B > 0 ? (double)(k + 1) + (double)ib * r : 1e300;
    if (ta <= tb) { last = ta; left -= A; ++ia; }
    else { last = tb; left -= B; ++ib; }
  }
  return std::max(wide_end, last + r);
}

// Column tiles of the 8-wave 256x256 tile: tn_wide tiles 256 wide, then
// tn_narrow 192 wide.  The whole width in 256-wide tiles leaves the last
// round part empty when the tile count is not a multiple of the grid; at
// M = 8192, N = 3584 on 256 workgroups 448 tiles take two rounds, while 8
// wide and 8 narrow tiles per tile row give every workgroup one of each.  A
// narrow tile does 3/4 of the work; AG_NARROW_COST is its measured time
// relative to a wide one.  A mix is taken when the greedy schedule finishes
// at least 3 % earlier; with more than 8 tiles per workgroup the last round
// matters little and the plan is not searched.
constexpr double AG_NARROW_COST = 0.8;
void ag_column_plan(int tiles_m, int64_t N, int grid, int* tn_wide, int* tn_narrow) {
  const int a0 = (int)((N + 255) / 256);
  *tn_wide = a0;
  *tn_narrow = 0;
  if (grid < 1 || (int64_t)tiles_m * a0 > 8ll * grid) return;
  double best = ag_makespan((int64_t)tiles_m * a0, 0, grid, AG_NARROW_COST);
  for (int a = a0 - 1; a >= 0 && a >= a0 - 64; --a) {
    const int b = (int)((N - 256ll * a + 191) / 192);
    const double m = ag_makespan((int64_t)tiles_m * a, (int64_t)tiles_m * b, grid, AG_NARROW_COST);
    if (m < 0.97 * best) {
      best = m;
      *tn_wide = a;
      *tn_narrow = b;
    }
  }
}

// Copy workgroups: three quarters of the grid start as copiers (while copy
// work remains, then compute) and a quarter starts on the tiles whose rows
// land first.  At M = 8192, K = 8192, N = 3584 (512 KiB items) this measured
// 0.460 against 0.472 ms with every workgroup copying first, and 0.467 with
// 160 or 224 copiers of 256 (settled, interleaved, on two boxes).  Far fewer
// copiers are slower: one workgroup's copy rate is bound by load latency, so
// a few copiers cannot keep ahead of the tiles.
int ag_default_n_copy(int grid) { return grid > 1 ? grid - grid / 4 : 1; }

// Tile choice.  A single 128-row tile row (a skinny A, the GEMM streams B)
// takes a 128x128 tile at one workgroup per CU: every CU with a tile streams
// its own B column stripe, with no MFMA work spent on empty rows.  The
// producer/consumer tile (A from its packed copy) is the default there: at
// M = 128, K = 8192, N = 28672 its GEMM kernel took 0.128 ms against
// 0.152 ms for the direct-to-LDS tile with the 8-slice ring (which loads A
// through the same DMA stream as B), 0.177 ms for the 128x256 tile (112
// CUs with a tile) and 0.160 ms for the half-empty 256x128 tile.  Without
// a workspace for the packed copy the 8-slice ring is used, and where K is
// not a multiple of 256 the 128x256 direct-to-LDS tile.
//
// With M and N of at least 256 and K % 128 == 0 the direct-to-LDS tiles
// compete on an estimate of when the last tile ends on the grid (one
// workgroup per CU), in units of one 256x256 tile: the 8-wave 256x256 tile
// with its column plan (a 192-wide tile 0.8, see ag_column_plan), or the
// 4-wave 128x256 and 256x128 tiles at 0.55 each (half the work; measured
// 0.54 of the 8-wave tile at M = 4096, N = 3584, K = 8192, where 448 of them
// took 0.266 ms against 0.247 ms for 224 tiles of 256x256).  The 8-wave tile
// wins ties.  At M = 8192, N = 3584 (448 tiles of 256x256) it is the 8-wave
// tile; below one round of 256x256 tiles the half tiles spread the work over
// more CUs: at K = 8192, N = 3584 the fused call took 0.129 ms (128x256)
// against 0.149 ms (8-wave, 192-wide tiles) and 0.216 ms (the register-staged
// 128x128 tile chosen before) at M = 1024, and 0.152 against 0.170 and 0.230
// ms at M = 2048.  Otherwise the register-staged tiles by size.
constexpr double AG_HALF_COST = 0.55;
int ag_default_tile(int64_t M, int64_t N, int64_t K, bool pack, int n_cu) {
  if (M <= 128 && N >= 256) {
    if (pack) return TILE_128x128_PC;
    if (TileGemmD<128, 128, true, 8>::supports_k((int)K)) return TILE_128x128_DMA8;
    if (TileGemmD<128, 256>::supports_k((int)K)) return TILE_128x256_DMA;
  }
  if (M >= 256 && N >= 256 && TileGemmD<256, 256>::supports_k((int)K)) {
    const int grid = std::max(n_cu, 1);
    const int tm = (int)((M + 255) / 256);
    int a = 0, b = 0;
    ag_column_plan(tm, N, grid, &a, &b);
    const double w8 = ag_makespan((int64_t)tm * a, (int64_t)tm * b, grid, AG_NARROW_COST);
    auto rounds = [grid](int64_t tiles) { return (double)((tiles + grid - 1) / grid); };
    const double t8 = AG_HALF_COST * rounds(((M + 127) / 128) * ((N + 255) / 256));
    const double t7 = AG_HALF_COST * rounds(((M + 255) / 256) * ((N + 127) / 128));
    if (w8 <= t8 && w8 <= t7) return TILE_256x256_DMA_W8;
    return t8 <= t7 ? TILE_128x256_DMA : TILE_256x128_DMA;
  }
  return mk_default_tile(M, N, K);
}

}  // namespace mkp

extern "C" int mk_ag_column_plan(int64_t M, int64_t N, int grid, int* tn_wide, int* tn_narrow) {
  if (!tn_wide || !tn_narrow) return mkh::fail(MK_ERR_INVALID, "tn_wide and tn_narrow must be non-NULL");
  if (M < 1 || N < 1 || grid < 1) return mkh::fail(MK_ERR_INVALID, "non-positive M, N or grid");
  if (M > (1 << 30) || N > MK_MAX_COLS) return mkh::fail(MK_ERR_INVALID, "dimension too large");
  mkp::ag_column_plan((int)((M + 255) / 256), N, grid, tn_wide, tn_narrow);
  return MK_OK;
}


extern "C" size_t mk_ag_gemm_workspace(int R, int64_t m_shard, int64_t K, int64_t N, int32_t unit_rows) {
  (void)N; (void)unit_rows;
  return ag_ws_layout(K, ag_packs((int64_t)R * m_shard, K)).total;
}

// ------------------------------------------------- entry point without allocation
// mk_ag_gemm_noalloc keeps its workspace (header and per-unit arrival
// counters) in this file-scope device array instead of a caller buffer.  Each
// GPU holds its own copy until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol):
// its device address is looked up once per device with hipGetSymbolAddress,
// with that device current, and only that address is used.
constexpr size_t AG_SCRATCH_BYTES = 4096;
static __device__ __align__(256) uint32_t scratch[AG_SCRATCH_BYTES / 4];

// Device address of `scratch` on device `dev` (looked up on first use).
static int scratch_address(int dev, void** out) {
  static std::mutex mu;
  static void* addr[64];
  if (dev < 0 || dev >= 64) return mkh::fail(MK_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return mkh::hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return mkh::fail(MK_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return MK_OK;
}

// clear_bytes > 0: zero that many workspace bytes (fill kernel) on the
// stream before the first launch.
template <class G>
static int run_ag(AgParams& p, const mk_launch& o, const mkh::Schedule& s, const mkh::DevInfo* d,
                  hipStream_t st, size_t clear_bytes) {
  p.tiles_m = (p.M + G::BM - 1) / G::BM;
  if (p.tiles_m > MK_MAX_UNITS) return mkh::fail(MK_ERR_UNSUPPORTED, "M too large: %d tile rows", p.tiles_m);
  // Tile rows ordered by the issue position of the last unit under them.
  std::vector<int> rb(p.tiles_m), key(p.tiles_m);
  for (int t = 0; t < p.tiles_m; ++t) {
    const int u0 = t * G::BM / p.unit_rows, u1 = (std::min(p.M, (t + 1) * G::BM) - 1) / p.unit_rows;
    int k = 0;
    for (int u = u0; u <= u1; ++u) k = std::max(k, s.pos[u]);
    rb[t] = t;
    key[t] = k;
  }
  std::stable_sort(rb.begin(), rb.end(), [&](int a, int b) { return key[a] < key[b]; });
  for (int t = 0; t < p.tiles_m; ++t) p.rb_order[t] = (uint16_t)rb[t];

  int occ = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, ag_kernel<G>, G::NT, 0);
  if (e != hipSuccess) return mkh::hip_fail(e, "occupancy query");
  if (occ < 1) return mkh::fail(MK_ERR_UNSUPPORTED, "kernel does not fit on a CU");
  const int full = d->n_cu * occ;
  const int grid = o.grid > 0 ? std::min(o.grid, full) : full;
  const uint32_t n_work = (uint32_t)p.n_units * p.parts;
  // Column tiles: all G::BN wide, or (one queue, queue_mode 0) a mix with
  // 192-wide tiles where that shortens the schedule on this grid.
  int tn_wide = (p.N + G::BN - 1) / G::BN, tn_narrow = 0;
  if constexpr (NarrowTile<G>::ok)
    if (o.queue_mode == 0) mkp::ag_column_plan(p.tiles_m, p.N, grid, &tn_wide, &tn_narrow);
  p.tn_wide = tn_wide;
  p.tn_narrow = tn_narrow;
  p.tiles_n = tn_wide + tn_narrow;
  p.n_tiles = p.tiles_m * p.tiles_n;
  p.n_wide = p.tiles_m * tn_wide;
  if (clear_bytes) {
    const int rc = mkh::zero_fill(p.hdr, clear_bytes, st);
    if (rc) return rc;
  }

  if (o.mode >= 1) {   // unfused baseline: copy kernel, then GEMM kernel (modes 2/3: one of them)
    if (o.mode != 3) {
      p.mode = MODE_COPY;
      p.n_copy = grid;
      hipLaunchKernelGGL(ag_kernel<G>, dim3(grid), dim3(G::NT), 0, st, p);
      if ((e = hipGetLastError()) != hipSuccess) return mkh::hip_fail(e, "copy kernel launch");
    } else if (p.Ap) {   // the GEMM alone reads the packed copy: pack a_gathered as it is first
      p.mode = MODE_PACK;
      p.n_copy = grid;
      hipLaunchKernelGGL(ag_kernel<G>, dim3(grid), dim3(G::NT), 0, st, p);
      if ((e = hipGetLastError()) != hipSuccess) return mkh::hip_fail(e, "pack kernel launch");
    }
    if (o.mode != 2) {
      p.mode = MODE_GEMM;
      p.n_copy = 0;
      hipLaunchKernelGGL(ag_kernel<G>, dim3(grid), dim3(G::NT), 0, st, p);
      if ((e = hipGetLastError()) != hipSuccess) return mkh::hip_fail(e, "gemm kernel launch");
    }
    return MK_OK;
  }
  p.mode = MODE_FUSED;
  int n_copy = o.n_copy > 0 ? o.n_copy : mkp::ag_default_n_copy(grid);
  n_copy = std::min<int>(n_copy, (int)std::min<uint32_t>(n_work, (uint32_t)grid));
  p.n_copy = n_copy;
  hipLaunchKernelGGL(ag_kernel<G>, dim3(grid), dim3(G::NT), 0, st, p);
  if ((e = hipGetLastError()) != hipSuccess) return mkh::hip_fail(e, "fused kernel launch");
  return MK_OK;
}

// mk_ag_gemm, and (no_alloc) mk_ag_gemm_noalloc, whose workspace is the
// device's `scratch` array, cleared on the stream before the kernel.
static int ag_gemm(const void* const* a_shards, int R, int64_t m_shard, int64_t K, const void* B, int64_t N,
                   void* C, int c_dtype, void* a_gathered, const mk_arrival* arrival, const mk_launch* launch,
                   void* workspace, size_t workspace_bytes, void* stream, bool no_alloc) {
  using mkh::fail;
  if (!a_shards) return fail(MK_ERR_INVALID, "a_shards is NULL");
  if (R < 1 || R > MK_MAX_RANKS) return fail(MK_ERR_UNSUPPORTED, "R=%d outside [1,%d]", R, MK_MAX_RANKS);
  if (m_shard < 1 || K < 8 || N < 8) return fail(MK_ERR_INVALID, "empty or too small shape");
  if (K % 8 || N % 8) return fail(MK_ERR_UNSUPPORTED, "K (%lld) and N (%lld) must be multiples of 8",
                                  (long long)K, (long long)N);
  const int64_t M = (int64_t)R * m_shard;
  if (M > (1 << 30) || K > (1 << 20) || N > MK_MAX_COLS || K * N * 2 >= (1ll << 31))
    return fail(MK_ERR_UNSUPPORTED, "dimension too large");
  if (!B || !C || !a_gathered) return fail(MK_ERR_INVALID, "B, C and a_gathered must be non-NULL");
  if (c_dtype != MK_BF16 && c_dtype != MK_F32) return fail(MK_ERR_INVALID, "c_dtype %d", c_dtype);
  for (int r = 0; r < R; ++r)
    if (!a_shards[r] || !mkh::aligned16(a_shards[r])) return fail(MK_ERR_INVALID, "shard %d NULL or misaligned", r);
  if (!mkh::aligned16(B) || !mkh::aligned16(C) || !mkh::aligned16(a_gathered))
    return fail(MK_ERR_INVALID, "B, C and a_gathered must be 16-byte aligned");
  mkh::Schedule s;
  int rc = mkh::make_schedule(arrival, M, R, &s);
  if (rc) return rc;
  // Without a workspace argument there is no room for the packed copy of A,
  // so the producer/consumer tile is not used.
  const bool pack = !no_alloc && ag_packs(M, K);
  const AgWs lay = ag_ws_layout(K, pack);
  const size_t ws_need = lay.total;
  if (no_alloc) {
    if (s.withhold != -1)
      return fail(MK_ERR_INVALID, "withhold is not available without a workspace (no status to poll)");
    if (ws_need > AG_SCRATCH_BYTES)
      return fail(MK_ERR_UNSUPPORTED, "needs %zu bytes of scratch, the built-in array holds %zu", ws_need,
                  AG_SCRATCH_BYTES);
  } else {
    if (!workspace) return fail(MK_ERR_WORKSPACE, "workspace is NULL");
    if (workspace_bytes < ws_need)
      return fail(MK_ERR_WORKSPACE, "workspace %zu bytes < %zu", workspace_bytes, ws_need);
  }
  const mk_launch o = mkh::launch_opts(launch);
  if (o.mode < 0 || o.mode > 3) return fail(MK_ERR_INVALID, "mode %d", o.mode);
  if (o.grid < 0 || o.n_copy < 0 || o.copy_kib < 0) return fail(MK_ERR_INVALID, "negative grid, n_copy or copy_kib");
  if (o.copy_policy < 0 || o.copy_policy > 3) return fail(MK_ERR_INVALID, "copy_policy %d", o.copy_policy);
  if (o.queue_mode < 0 || o.queue_mode > 2) return fail(MK_ERR_INVALID, "queue_mode %d", o.queue_mode);
  const mkh::DevInfo* d = mkh::dev_info();
  if (!d) return MK_ERR_HIP;
  if (no_alloc) {
    rc = scratch_address(d->device, &workspace);
    if (rc) return rc;
  }

  AgParams p;
  memset(&p, 0, sizeof p);
  for (int r = 0; r < R; ++r) p.shard[r] = (const uint16_t*)a_shards[r];
  p.B = (const uint16_t*)B;
  p.C = C;
  p.Ag = (uint16_t*)a_gathered;
  p.hdr = (WsHeader*)workspace;
  p.unit_cnt = (uint32_t*)((char*)workspace + sizeof(WsHeader));
  p.tile_log = o.tile_log;
  p.copy_log = o.copy_log;
  p.copy_wt = o.copy_policy != 1;              // default: written through
  p.c_wt = o.copy_policy != 3;                 // default: output tiles written through too
  p.xcd_queues = o.queue_mode == 1;            // default: one queue in landing order
  p.spin_limit = mkh::spin_ticks(o, d);
  p.R = R; p.m_shard = (int)m_shard; p.M = (int)M; p.K = (int)K; p.N = (int)N;
  p.c_bf16 = c_dtype == MK_BF16;
  p.n_units = s.n_units;
  p.unit_rows = s.unit_rows;
  p.withhold = s.withhold;
  // Copy work items ("parts") of about copy_kib KiB: each is published with
  // one release, which writes back the XCD's L2, so fewer larger items cost
  // fewer write-backs.  A part never crosses a unit or shard boundary (one
  // contiguous copy).
  const int64_t row_bytes = K * 2;
  int g = s.unit_rows, b = (int)m_shard;
  while (b) { const int t = g % b; g = b; b = t; }   // gcd(unit_rows, m_shard)
  const int64_t item_bytes = o.copy_kib > 0 ? (int64_t)o.copy_kib << 10 : mkp::ag_default_item_bytes(M, K, d->n_cu);
  int part_rows = (int)std::max<int64_t>(1, std::min<int64_t>(g, item_bytes / row_bytes));
  // whole rows that divide the unit and the shard; at most 1 GiB per part so
  // 32-bit buffer offsets cover it
  while (part_rows > 1 && (g % part_rows || (int64_t)part_rows * row_bytes > (1ll << 30))) --part_rows;
  p.part_rows = part_rows;
  p.part_bytes = (uint32_t)(part_rows * row_bytes);
  p.parts = s.unit_rows / part_rows;
  for (int j = 0; j < s.n_units; ++j) {
    p.order[j] = (uint16_t)s.order[j];
    p.delay_ticks[j] = (uint32_t)mkh::ns_to_ticks(s.delay_ns[j], d->wall_khz);
  }
  const hipStream_t st = (hipStream_t)stream;
  const size_t clear = no_alloc ? ws_need : 0;
  const int tile = o.tile ? o.tile : mkp::ag_default_tile(M, N, K, pack, d->n_cu);
  if (mk_is_dma_tile(tile) && !TileGemmD<256, 256>::supports_k((int)K))
    return fail(MK_ERR_UNSUPPORTED, "tile %d needs K %% 128 == 0", tile);
  if (tile == TILE_128x128_DMA8 && !TileGemmD<128, 128, true, 8>::supports_k((int)K))
    return fail(MK_ERR_UNSUPPORTED, "tile %d needs K %% 256 == 0", tile);
  if (tile == TILE_256x256_DMA_W8 && !TileGemmD<256, 256, true, 4, 8>::supports_k((int)K))
    return fail(MK_ERR_UNSUPPORTED, "tile %d needs K %% 128 == 0", tile);
  if (tile == TILE_128x128_PC && !pack)
    return fail(MK_ERR_UNSUPPORTED, "tile %d needs M <= 128, K %% 128 == 0 and a workspace (packed copy of A)", tile);
  if (tile == TILE_128x128_PC) {
    p.Ap = (uint16_t*)((char*)workspace + lay.pack);
    p.ap_bytes = (uint32_t)(lay.total - lay.pack);
  }
  switch (tile) {
    case TILE_256x256: return run_ag<TileGemm<256, 256, 2, 2>>(p, o, s, d, st, clear);
    case TILE_128x128: return run_ag<TileGemm<128, 128, 2, 2>>(p, o, s, d, st, clear);
    case TILE_256x128: return run_ag<TileGemm<256, 128, 2, 2>>(p, o, s, d, st, clear);
    case TILE_128x256: return run_ag<TileGemm<128, 256, 2, 2>>(p, o, s, d, st, clear);
    case TILE_256x256_DMA: return run_ag<TileGemmD<256, 256>>(p, o, s, d, st, clear);
    case TILE_128x128_DMA: return run_ag<TileGemmD<128, 128>>(p, o, s, d, st, clear);
    case TILE_256x128_DMA: return run_ag<TileGemmD<256, 128>>(p, o, s, d, st, clear);
    case TILE_128x256_DMA: return run_ag<TileGemmD<128, 256>>(p, o, s, d, st, clear);
    case TILE_128x128_DMA8: return run_ag<TileGemmD<128, 128, true, 8>>(p, o, s, d, st, clear);
    case TILE_256x256_DMA_W8: return run_ag<TileGemmD<256, 256, true, 4, 8>>(p, o, s, d, st, clear);
    case TILE_128x128_PC: return run_ag<TileGemmPC<>>(p, o, s, d, st, clear);
    default: return fail(MK_ERR_INVALID, "tile id %d", tile);
  }
}

extern "C" int mk_ag_gemm(const void* const* a_shards, int R, int64_t m_shard, int64_t K,
                          const void* B, int64_t N, void* C, int c_dtype, void* a_gathered,
                          const mk_arrival* arrival, const mk_launch* launch,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return ag_gemm(a_shards, R, m_shard, K, B, N, C, c_dtype, a_gathered, arrival, launch, workspace,
                 workspace_bytes, stream, false);
}

extern "C" int mk_ag_gemm_noalloc(const void* const* a_shards, int R, int64_t m_shard, int64_t K,
                                  const void* B, int64_t N, void* C, int c_dtype, void* a_gathered,
                                  const mk_arrival* arrival, const mk_launch* launch, void* stream) {
  return ag_gemm(a_shards, R, m_shard, K, B, N, C, c_dtype, a_gathered, arrival, launch, nullptr, 0, stream,
                 true);
}
