// GEMM -> ReduceScatter as one persistent kernel.
//
// [P1] "Los cinco núcleos fusionados", row GEMM + ReduceScatter: C = A @ B is
// reduced across ranks and scattered, each output tile being reduced and sent
// to the rank that owns it as soon as it is produced.  On one GPU the other
// ranks' contributions are resident fp32 partial sums, and the owners are the
// R row blocks of the output.
//
// The other ranks' partial sums may also arrive over time: with an arrival
// schedule, units (peer, row block) are released in a given order and at
// given times by copy workgroups, which move each unit's rows from the
// resident partial sum into a landing buffer when the caller passes one (or
// only publish it, the partial then being read in place); the reduction of a
// tile waits for the units under its rows.  Without a schedule every partial
// sum is resident from the start.
//
// Roles:
//   copy     tickets [0, n_copy) (arrival schedule only): take (unit, part)
//            items in arrival order, wait for the unit's release time, copy,
//            publish with an agent-scope release on the unit's counter; then
//            continue as a compute (or reduce) workgroup.
//   compute  tickets [0, n_compute): GEMM tiles from a queue (tile rows in the
//            order their partial sums land).  With reduce
//            workgroups present, a finished fp32 tile is staged, published
//            (release) and its id appended to a produced-tile FIFO; a compute
//            workgroup whose queue is empty turns into a reduce workgroup.
//            Without them (n_reduce <= 0) the compute workgroup reduces the
//            tile itself, straight from its accumulator registers: it loads
//            the partial sums for the elements it holds, adds them and
//            stores the owner's rows (no fp32 staging).
//   reduce   tickets [n_compute, grid): pop produced tiles in production order,
//            acquire, sum local + P_1 + ... + P_{R-1} in that fixed fp32 order
//            (so every role split and schedule gives identical bits) and
//            store the result in the owner's block.
#include <string.h>

#include <algorithm>

#include "mk_device.h"
#include "mk_gemm_dma.h"
#include "mk_host.h"
#include "mk_tiles.h"

using namespace mk;

namespace {

enum { MODE_EPI = 0, MODE_ROLES = 1, MODE_GEMM = 2, MODE_REDUCE = 3, MODE_COPY = 4 };

struct RsParams {
  const uint16_t* A;
  const uint16_t* B;
  const float* P[MK_MAX_RANKS];   // R-1 partial sums as the reduction reads them (landing buffers if given)
  const float* Psrc[MK_MAX_RANKS];// the resident partial sums the copy role moves into P (copy_data)
  void* out[MK_MAX_RANKS];        // R owner blocks
  float* stage;                   // fp32 staging [M x N], or NULL to stage in out (fp32)
  WsHeader* hdr;
  uint32_t* fifo;                 // [n_tiles] produced tile id + 1
  uint32_t* unit_cnt;             // [n_units] parts landed per unit; NULL: every partial resident
  int32_t* tile_log;
  int32_t* copy_log;
  uint64_t spin_limit;
  int M, K, N, R, out_bf16, mb;   // mb = rows per owner
  int n_dst;                      // outputs per row block: 1 (reduce-scatter) or R (all-reduce)
  int mode, n_compute, tiles_m, tiles_n, n_tiles;
  // per-XCD band queues (tiles_n % XQ == 0): queue x holds the columns
  // x, x + XQ, x + 2 XQ, ... of band after band of band_rows tile rows,
  // row-major within a band
  int xcd_queues, band_rows;
  // arrival schedule of the partial sums: unit u = q * n_blocks + b is row
  // block b (unit_rows rows) of partial q (0-based peer), copied in `parts`
  // items of part_rows rows
  int n_units, unit_rows, n_blocks, parts, part_rows, n_copy, withhold, copy_data;
  uint32_t part_bytes;
  uint16_t order[MK_MAX_UNITS];
  uint16_t rb_order[MK_MAX_UNITS];   // tile rows in landing order (arrival schedule only)
  uint32_t delay_ticks[MK_MAX_UNITS];
};
static_assert(sizeof(RsParams) <= 4096, "kernel argument size");

// Tile row of queue position q (tiles are queued row by row).
__device__ __forceinline__ int queued_tile_row(const RsParams& p, int q) {
  return p.unit_cnt ? (int)p.rb_order[q / p.tiles_n] : q / p.tiles_n;
}

__device__ __forceinline__ float* stage_ptr(const RsParams& p, int gr, int gc) {
  if (p.stage) return p.stage + (int64_t)gr * p.N + gc;
  const int o = gr / p.mb;
  return (float*)p.out[o] + (int64_t)(gr - o * p.mb) * p.N + gc;
}

// Reduce one staged tile: out = stage + P_1 + ... + P_{R-1}, 4 columns per
// access, in that fixed order.  Each thread takes UNROLL 4-column runs; for
// each group of up to PG partial sums every load is issued before the first
// add (PG x UNROLL 16-byte loads in flight per thread), so the kernel streams
// instead of waiting one load latency per partial.  All accesses go through
// buffer descriptors bounded to the tile's rows; a run past N gets the
// out-of-range offset (loads return zero, stores are dropped).
template <int BM, int BN>
__device__ __forceinline__ void reduce_tile(const RsParams& p, int t) {
  const int tm = t / p.tiles_n, tn = t % p.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  constexpr int V = BN / 4;                  // 4-column runs per tile row
  constexpr int UNROLL = 4, PG = 8;
  const int nt = blockDim.x;
  const int rows = min(BM, p.M - m0);
  const int o = m0 / p.mb;                   // a tile never straddles two owners
  const uint32_t rb4 = (uint32_t)p.N * 4u;
  const uint32_t esz = p.out_bf16 ? 2u : 4u, rbo = (uint32_t)p.N * esz;
  const uint32_t in_bytes = uni((uint32_t)rows * rb4), out_bytes = uni((uint32_t)rows * rbo);
  const __amdgpu_buffer_rsrc_t ds = make_rsrc(uni(stage_ptr(p, m0, 0)), in_bytes);
  const int64_t dofs = (int64_t)(m0 - o * p.mb) * p.N * esz;
  const int nq = p.R - 1;
  for (int base = 0; base < BM * V; base += nt * UNROLL) {
    uint32_t vin[UNROLL], vout[UNROLL];
    f32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int idx = base + u * nt + threadIdx.x;
      const int r = idx / V, c = n0 + (idx % V) * 4;
      const bool ok = idx < BM * V && r < rows && c < p.N;
      vin[u] = ok ? (uint32_t)r * rb4 + (uint32_t)c * 4u : OOB;
      vout[u] = ok ? (uint32_t)r * rbo + (uint32_t)c * esz : OOB;
      v[u] = __builtin_bit_cast(f32x4, bload(ds, vin[u], 0));
    }
    for (int q0 = 0; q0 < nq; q0 += PG) {
      f32x4 w[PG][UNROLL];
#pragma unroll
      for (int g = 0; g < PG; ++g) {
        const int q = q0 + g < nq ? q0 + g : nq - 1;
        const __amdgpu_buffer_rsrc_t dp = make_rsrc(uni(p.P[q] + (int64_t)m0 * p.N), in_bytes);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) w[g][u] = __builtin_bit_cast(f32x4, bload(dp, vin[u], 0));
      }
#pragma unroll
      for (int g = 0; g < PG; ++g)
        if (q0 + g < nq) {
#pragma unroll
          for (int u = 0; u < UNROLL; ++u) v[u] += w[g][u];
        }
    }
    for (int d = 0; d < p.n_dst; ++d) {
      const __amdgpu_buffer_rsrc_t dout = make_rsrc(uni((const char*)p.out[o + d] + dofs), out_bytes);
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        if (p.out_bf16) {
          u32x2 b;
          b[0] = (uint32_t)f2bf(v[u][0]) | ((uint32_t)f2bf(v[u][1]) << 16);
          b[1] = (uint32_t)f2bf(v[u][2]) | ((uint32_t)f2bf(v[u][3]) << 16);
          __builtin_amdgcn_raw_buffer_store_b64(b, dout, vout[u], 0, 0);
        } else {
          bstore_alu16(dout, vout[u], 0, v[u]);
        }
      }
    }
  }
}

// out = acc + P_1 + ... + P_{R-1} for the elements this thread holds, in that
// order (the same fp32 order as reduce_tile, so every mode gives the same
// bits).  In a 32x32 accumulator block each quad of lanes holds 4 columns x
// 16 rows; a quad transpose (DPP) turns every 4x4 piece into one 4-column row
// run per lane, so the partial sums are read and the outputs written with
// 16-byte accesses.  All accesses go through buffer descriptors bounded to
// the tile's rows, and a column past N gets an out-of-range offset: such a
// load returns zero and such a store is dropped, so no memory operation sits
// behind a branch (a guarded store would wait for every earlier access).
template <class G>
__device__ __forceinline__ void reduce_from_acc(const G& g, const RsParams& p, int m0, int n0) {
  const int lane = threadIdx.x & 63, w = uni((int)(threadIdx.x >> 6));
  const int wm = w % G::WM, wn = w / G::WM;
  const int o = m0 / p.mb;                       // a tile never straddles two owners
  const int nq = p.R - 1;
  const int rows = min(G::BM, p.M - m0);
  const uint32_t esz = p.out_bf16 ? 2u : 4u;
  const uint32_t rb4 = (uint32_t)p.N * 4u, rbo = (uint32_t)p.N * esz;   // row bytes in / out
  const uint32_t in_bytes = uni((uint32_t)rows * rb4);
  const int64_t dofs = ((int64_t)(m0 - o * p.mb) * p.N) * esz;   // tile origin in its row block
  const uint32_t dbytes = uni((uint32_t)rows * rbo);
  // Per-lane part of every offset (the lane's row in a 4-row group and its
  // 4-column run); the block and group parts are scalar offsets.
  const int lrow = (lane >> 5) * 4 + (lane & 3), lcol = (lane & 31) & ~3;
  const uint32_t lin = (uint32_t)lrow * rb4 + (uint32_t)lcol * 4u;
  const uint32_t lout = (uint32_t)lrow * rbo + (uint32_t)lcol * esz;
#pragma unroll
  for (int i = 0; i < G::FM; ++i) {
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
      // keep the blocks in order: otherwise the scheduler hoists every
      // block's transpose ahead of the loads and runs out of registers
      __builtin_amdgcn_sched_barrier(0);
      const int cb = n0 + wn * G::TN + j * 32;                 // first column of the block
      const bool colok = cb + lcol < p.N;
      const uint32_t vin = colok ? lin : OOB, vout = colok ? lout : OOB;
      const int rb = wm * G::TM + i * 32;                      // first row of the block in the tile
      f32x4 v[4];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
        v[gq] = quad_transpose(f32x4{g.acc[i][j][4 * gq], g.acc[i][j][4 * gq + 1], g.acc[i][j][4 * gq + 2],
                                     g.acc[i][j][4 * gq + 3]});
      for (int q0 = 0; q0 < nq; q0 += 4) {
        f32x4 t[4][4];
#pragma unroll
        for (int dq = 0; dq < 4; ++dq) {
          const int q = q0 + dq < nq ? q0 + dq : nq - 1;
          const __amdgpu_buffer_rsrc_t dp = make_rsrc(uni(p.P[q] + (int64_t)m0 * p.N), in_bytes);
#pragma unroll
          for (int gq = 0; gq < 4; ++gq)
            t[dq][gq] = __builtin_bit_cast(f32x4, bload(dp, vin, uni((uint32_t)(rb + 8 * gq) * rb4 + (uint32_t)cb * 4u)));
        }
#pragma unroll
        for (int dq = 0; dq < 4; ++dq)
          if (q0 + dq < nq) {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) v[gq] += t[dq][gq];
          }
      }
      for (int d = 0; d < p.n_dst; ++d) {
        const __amdgpu_buffer_rsrc_t dout = make_rsrc(uni((const char*)p.out[o + d] + dofs), dbytes);
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const uint32_t so = uni((uint32_t)(rb + 8 * gq) * rbo + (uint32_t)cb * esz);
          if (p.out_bf16) {
            u32x2 b;
            b[0] = (uint32_t)f2bf(v[gq][0]) | ((uint32_t)f2bf(v[gq][1]) << 16);
            b[1] = (uint32_t)f2bf(v[gq][2]) | ((uint32_t)f2bf(v[gq][3]) << 16);
            __builtin_amdgcn_raw_buffer_store_b64(b, dout, vout, so, 0);
          } else {
            bstore_alu16(dout, vout, so, v[gq]);
          }
        }
      }
    }
  }
}

// The same reduction for the direct-to-LDS engine, with the partial sums
// brought in by LDS DMA instead of register loads: after the K loop the
// engine's four stages (128 KiB) are free, so each wave owns 32 KiB = 32
// slots of 1 KiB.  The wave walks its 32x32 blocks in pieces of one row
// group (four rows): one DMA per partial -- lane L's 16 bytes land at slot +
// 16 L, exactly the 4-column run it holds after the quad transpose -- into
// one of four sets of 7 slots, so three pieces (21 KiB) are in flight while
// a piece is added in the fixed order and stored.  Every piece issues all
// seven partials' DMAs (a partial past R - 1 has an empty descriptor: it
// reads nothing and writes zero, and is not added), so the wait counts are
// constants: before piece n is read the wave waits until at most the DMAs
// issued after piece n's are outstanding; loads complete in order, so piece
// n has landed.  Columns past N get an out-of-range offset (the DMA writes
// zero).  Used with the 256x256 tile (16 KiB per stage and operand, so a[w]
// and b[w] hold 32 slots) when R - 1 <= 7.
template <class G>
__device__ __forceinline__ void reduce_from_acc_lds(const G& g, const RsParams& p, int m0, int n0, Smem4 sm) {
  static_assert(G::SA_U4 * 16 >= 16384 && G::SB_U4 * 16 >= 16384, "32 slots of 1 KiB per wave");
  constexpr int NP = 7;                          // partials per piece (R - 1 <= 7)
  constexpr int NSET = 4;                        // slot sets of NP slots
  constexpr int LA = NSET - 1;                   // pieces in flight while one is added
  constexpr int NPC = 4 * G::FM * G::FN;         // pieces per wave
  const int lane = threadIdx.x & 63, w = uni((int)(threadIdx.x >> 6));
  const int wm = w % G::WM, wn = w / G::WM;
  const int o = m0 / p.mb;
  const int nq = p.R - 1;
  const int rows = min(G::BM, p.M - m0);
  const uint32_t esz = p.out_bf16 ? 2u : 4u;
  const uint32_t rb4 = (uint32_t)p.N * 4u, rbo = (uint32_t)p.N * esz;
  const uint32_t in_bytes = uni((uint32_t)rows * rb4);
  const int64_t dofs = ((int64_t)(m0 - o * p.mb) * p.N) * esz;   // tile origin in its row block
  const uint32_t dbytes = uni((uint32_t)rows * rbo);
  const int lrow = (lane >> 5) * 4 + (lane & 3), lcol = (lane & 31) & ~3;
  const uint32_t lin = (uint32_t)lrow * rb4 + (uint32_t)lcol * 4u;
  const uint32_t lout = (uint32_t)lrow * rbo + (uint32_t)lcol * esz;
  // this wave's 32 slots: 16 in stage a[w], 16 in stage b[w]
  const uint32_t la = uni(lds_addr(w == 0 ? sm.a[0] : w == 1 ? sm.a[1] : w == 2 ? sm.a[2] : sm.a[3]));
  const uint32_t lb = uni(lds_addr(w == 0 ? sm.b[0] : w == 1 ? sm.b[1] : w == 2 ? sm.b[2] : sm.b[3]));
  const char* pa = (const char*)(w == 0 ? sm.a[0] : w == 1 ? sm.a[1] : w == 2 ? sm.a[2] : sm.a[3]);
  const char* pb = (const char*)(w == 0 ? sm.b[0] : w == 1 ? sm.b[1] : w == 2 ? sm.b[2] : sm.b[3]);
  u32x4 dp[NP];
#pragma unroll
  for (int q = 0; q < NP; ++q) dp[q] = buf_desc(p.P[q < nq ? q : 0] + (int64_t)m0 * p.N, q < nq ? in_bytes : 0u);
  // piece pn: block pn / 4 = (i, j), row group pn % 4, slot set pn % NSET
  auto issue_piece = [&](int pn) {
    const int blk = pn >> 2, i = blk / G::FN, j = blk % G::FN, gq = pn & 3;
    const int cb = n0 + wn * G::TN + j * 32;
    const uint32_t vin = cb + lcol < p.N ? lin : OOB;
    const int rb = wm * G::TM + i * 32;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int sl = (pn % NSET) * NP + q;
      dma16(dp[q], uni(sl < 16 ? la + sl * 1024 : lb + (sl - 16) * 1024), vin,
            uni((uint32_t)(rb + 8 * gq) * rb4 + (uint32_t)cb * 4u));
    }
  };
#pragma unroll
  for (int pn = 0; pn < LA; ++pn) issue_piece(pn);
#pragma unroll
  for (int i = 0; i < G::FM; ++i) {
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int pn = 4 * (i * G::FN + j) + gq;
        // keep the pieces in order: otherwise the scheduler hoists later
        // pieces' transposes and address arithmetic and runs out of registers
        __builtin_amdgcn_sched_barrier(0);
        if (pn + LA < NPC) {
          issue_piece(pn + LA);
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NP * LA) : "memory");   // piece pn has landed
        } else if (pn + 2 < NPC) {
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NP * 2) : "memory");
        } else if (pn + 1 < NPC) {
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NP) : "memory");
        } else {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        const int cb = n0 + wn * G::TN + j * 32;
        const uint32_t vout = cb + lcol < p.N ? lout : OOB;
        const int rb = wm * G::TM + i * 32;
        f32x4 v = quad_transpose(f32x4{g.acc[i][j][4 * gq], g.acc[i][j][4 * gq + 1], g.acc[i][j][4 * gq + 2],
                                       g.acc[i][j][4 * gq + 3]});
#pragma unroll
        for (int q = 0; q < NP; ++q)
          if (q < nq) {
            const int sl = (pn % NSET) * NP + q;
            v += *(const f32x4*)((sl < 16 ? pa + sl * 1024 : pb + (sl - 16) * 1024) + 16 * lane);
          }
        const uint32_t so = uni((uint32_t)(rb + 8 * gq) * rbo + (uint32_t)cb * esz);
        for (int d = 0; d < p.n_dst; ++d) {
          const __amdgpu_buffer_rsrc_t dout = make_rsrc(uni((const char*)p.out[o + d] + dofs), dbytes);
          if (p.out_bf16) {
            u32x2 b;
            b[0] = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
            b[1] = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
            __builtin_amdgcn_raw_buffer_store_b64(b, dout, vout, so, 0);
          } else {
            bstore_alu16(dout, vout, so, v);
          }
        }
      }
    }
  }
}

// The role loops take their next work index at the bottom of the body and
// test it at the top, with no `continue`: one uniform exit and one latch, so
// the compiler keeps every barrier in wave-uniform control flow.

// Copy role: (unit, part) items in arrival order.  Log stamps are the low 32
// bits of the 100 MHz wall clock; t_end is taken once the item's stores are
// complete and before its release.
__device__ __forceinline__ void rs_copy_role(const RsParams& p, WsHeader* h, uint32_t* sb) {
  const int tid = threadIdx.x, nt = blockDim.x;
  uint64_t t0 = 0;
  if (tid == 0) {
    const uint64_t now = now_ticks();
    const uint64_t old = atomicCAS((unsigned long long*)&h->t0, 0ull, (unsigned long long)now);
    t0 = old ? old : now;
  }
  const uint32_t n_work = (uint32_t)p.n_units * p.parts;
  const int n16 = p.part_rows * (p.N / 4);       // 16-byte chunks of fp32 per part
  uint32_t w = wg_bcast(tid == 0 ? add_relaxed(&h->copy_next, 1u) : 0u, sb);
  while (w < n_work) {
    const int j = w / p.parts, part = w % p.parts;
    const int u = p.order[j];
    if (u != p.withhold) {                         // a withheld unit never lands (failure tests)
      uint32_t t_start = 0;
      if (tid == 0) {
        wait_until(t0 + p.delay_ticks[u], p.spin_limit);
        t_start = (uint32_t)now_ticks();
      }
      __syncthreads();
      if (p.copy_data) {
        // rows of one row block of one partial: one contiguous block on both sides
        const int q = u / p.n_blocks, b = u % p.n_blocks;
        const int64_t ofs = ((int64_t)b * p.unit_rows + (int64_t)part * p.part_rows) * p.N;
        const __amdgpu_buffer_rsrc_t src = make_rsrc(uni(p.Psrc[q] + ofs), p.part_bytes);
        const __amdgpu_buffer_rsrc_t dst = make_rsrc(uni(p.P[q] + ofs), p.part_bytes);
        copy_block<16>(src, dst, n16, tid, nt);    // written through the L2
      }
      wg_release();                                // release only: the copier reads nothing others publish
      if (tid == 0) {
        const uint32_t t_end = (uint32_t)now_ticks();
        add_relaxed(&p.unit_cnt[u], 1u);
        add_relaxed(&h->aux[0], 1u);               // parts landed in total
        if (p.copy_log) {
          int32_t* L = p.copy_log + 8 * (int64_t)w;
          L[0] = u; L[1] = part; L[2] = (int32_t)blockIdx.x;
          L[3] = (int32_t)t_start; L[4] = (int32_t)t_end; L[5] = 0; L[6] = 0; L[7] = 0;
        }
      }
    }
    w = wg_bcast(tid == 0 ? add_relaxed(&h->copy_next, 1u) : 0u, sb);
  }
}

// Before a tile with BM rows starting at m0 is reduced: thread 0 waits until
// every peer's units under those rows have landed, then takes one acquire for
// all of them.  Returns (broadcast to the workgroup) bit 0 = ok (0: the
// watchdog expired, the tile is dropped) and bit 1 = every part of every unit
// had landed (later tiles of this workgroup need not wait).
template <int BM>
__device__ __forceinline__ uint32_t wait_partials(const RsParams& p, WsHeader* h, int m0, uint32_t* sb) {
  uint32_t ok = 1, all = 0;
  if (threadIdx.x == 0) {
    const int b0 = m0 / p.unit_rows, b1 = (min(p.M, m0 + BM) - 1) / p.unit_rows;
    for (int q = 0; q + 1 < p.R && ok; ++q)
      for (int b = b0; b <= b1 && ok; ++b)
        ok = wait_geq_relaxed(&p.unit_cnt[q * p.n_blocks + b], (uint32_t)p.parts, h, p.spin_limit);
    if (ok) {
      all = ld_relaxed(&h->aux[0]) >= (uint32_t)p.n_units * p.parts;
      fence_acquire();
    }
  }
  return wg_bcast(ok | (all << 1), sb);
}

// Tile log record of tile t: {owner, production rank, reducing workgroup,
// first row block (-1: partials resident), t_take (reduction about to wait
// for its partial sums), t_ready (they had landed), t_done (stores issued),
// 0}.
__device__ __forceinline__ void log_reduction(const RsParams& p, int t, int m0, uint32_t t_take, uint32_t t_ready) {
  int32_t* L = p.tile_log + 8 * (int64_t)t;
  L[2] = (int32_t)blockIdx.x;
  L[3] = p.unit_cnt ? m0 / p.unit_rows : -1;
  L[4] = (int32_t)t_take; L[5] = (int32_t)t_ready; L[6] = (int32_t)(uint32_t)now_ticks(); L[7] = 0;
}

template <class G, class SM>
__device__ __forceinline__ void rs_compute_role(const RsParams& p, WsHeader* h, SM sm, uint32_t* sb) {
  const int tid = threadIdx.x;
  G g;
  // Phase offset (fused epilogue): every workgroup alternates an MFMA-bound K
  // loop with an HBM-bound reduction, so if all start together all reduce
  // together.  Odd workgroups therefore start their first tile only when
  // the first even one is three quarters through its first K loop (aux[1];
  // measured best among fixed offsets of 0 to 1.3 K loops); from then on the
  // two halves of the grid are out of phase.  Even workgroups wait on
  // nothing, so the wait always ends.
  const bool offset = p.mode == MODE_EPI && p.n_tiles > (int)gridDim.x / 2;
  if (offset && (blockIdx.x & 1)) {
    if (tid == 0) wait_geq_relaxed(&h->aux[1], 1u, h, p.spin_limit);
    __syncthreads();
  }
  bool first = true;
  // partial sums all landed (or resident): no more waits before reductions
  bool all_landed = p.unit_cnt == nullptr;
  // Queue position of the next tile.  With per-XCD band queues (opt-in) the
  // 32 or so tiles that run at once on one XCD lie in one band of band_rows
  // tile rows and tiles_n / XQ columns, so they share few A row blocks and B
  // column blocks in that XCD's L2, and every XCD works on the same band at
  // the same time.  A drained queue's workgroups help the others.  (This
  // speeds up the K loops but slows the partial-sum reads, which then come
  // from a few columns of each row per XCD.)
  const int cw = p.tiles_n / XQ;
  XcdQueues xq(&h->aux[XQ_AUX]);
  auto take_tile = [&]() -> uint32_t {
    if (!p.xcd_queues) return add_relaxed(&h->tile_next, 1u);
    int x;
    uint32_t j;
    if (!xq.take([&](int) { return (uint32_t)(p.tiles_m * cw); }, x, j)) return (uint32_t)p.n_tiles;
    const uint32_t per_band = (uint32_t)(p.band_rows * cw), b = j / per_band, w = j % per_band;
    const uint32_t c = (uint32_t)x + XQ * (w % (uint32_t)cw);
    return (b * (uint32_t)p.band_rows + w / (uint32_t)cw) * (uint32_t)p.tiles_n + c;
  };
  uint32_t q = wg_bcast(tid == 0 ? take_tile() : 0u, sb);
  while (q < (uint32_t)p.n_tiles) {
    const int tm = queued_tile_row(p, (int)q), tn = (int)q % p.tiles_n;
    const int t = tm * p.tiles_n + tn;             // tile id (row-major)
    const int m0 = tm * G::BM, n0 = tn * G::BN;
    g.bind(p.A + (int64_t)m0 * p.K, p.K, p.M - m0, p.B + n0, p.N, p.N - n0, p.B + (int64_t)p.K * p.N, p.K);
    uint32_t* mark = offset && first && !(blockIdx.x & 1) ? &h->aux[1] : nullptr;
    if constexpr (G::STAGES == 4) {
      g.run(sm, mark);                             // raised three quarters into the K loop
    } else {
      g.run(sm);
      if (mark && tid == 0) st_relaxed(mark, 1u);
    }
    first = false;
    if (p.mode == MODE_EPI) {
      const uint32_t t_take = (uint32_t)now_ticks();
      uint32_t ready = 1;
      if (!all_landed) {
        const uint32_t v = wait_partials<G::BM>(p, h, m0, sb);
        ready = v & 1u;
        all_landed = (v >> 1) & 1u;
      }
      const uint32_t t_ready = (uint32_t)now_ticks();
      if (ready) {                                 // else the watchdog expired: the tile is dropped
        // the LDS path needs 32 KiB of stage buffers per wave: 256x256 tile only
        if constexpr (G::STAGES == 4 && G::BM == 256 && G::BN == 256) {
          if (p.R <= 8) {
            reduce_from_acc_lds(g, p, m0, n0, sm);
            __syncthreads();                       // LDS back to the K loop of the next tile
          } else {
            reduce_from_acc(g, p, m0, n0);
          }
        } else {
          reduce_from_acc(g, p, m0, n0);
        }
        if (p.tile_log && tid == 0) {
          p.tile_log[8 * t] = m0 / p.mb;
          p.tile_log[8 * t + 1] = t;
          log_reduction(p, t, m0, t_take, t_ready);
        }
      }
    } else {
      // Stage the fp32 tile (in the owner block for fp32 output, else in the
      // workspace staging area) for the reduce role or the reduce kernel.
      float* __restrict__ S = p.stage ? p.stage + (int64_t)m0 * p.N
                                      : (float*)p.out[m0 / p.mb] + (int64_t)(m0 % p.mb) * p.N;
      store_tile(g, S + n0, p.N, p.M - m0, p.N - n0, false);
      if (p.mode == MODE_ROLES) wg_release();      // the staged tile, before its FIFO entry
    }
    uint32_t next = 0;
    if (tid == 0) {
      if (p.mode == MODE_ROLES) {
        const uint32_t slot = add_relaxed(&h->prod_next, 1u);
        if (p.tile_log) {                          // before the release: the reducer may log next
          p.tile_log[8 * t] = m0 / p.mb;
          p.tile_log[8 * t + 1] = (int32_t)slot;
        }
        st_relaxed(&p.fifo[slot], (uint32_t)t + 1u);   // after wg_release: the tile is visible
      }
      next = take_tile();
    }
    q = wg_bcast(next, sb);
  }
}

template <class G>
__device__ __forceinline__ void rs_reduce_role(const RsParams& p, WsHeader* h, uint32_t* sb) {
  const int tid = threadIdx.x;
  // the unfused reduce kernel runs after the copy kernel: everything has landed
  bool all_landed = p.unit_cnt == nullptr || p.mode == MODE_REDUCE;
  uint32_t i = wg_bcast(tid == 0 ? add_relaxed(&h->red_next, 1u) : 0u, sb);
  while (i < (uint32_t)p.n_tiles) {
    uint32_t t = i;
    if (p.mode == MODE_ROLES) {
      uint32_t v = 0;
      if (tid == 0) v = wait_geq(&p.fifo[i], 1u, h, p.spin_limit) ? ld_relaxed(&p.fifo[i]) : 0u;
      v = wg_bcast(v, sb);
      t = v - 1u;                                // v == 0: watchdog expired, nothing to reduce
    }
    if (t < (uint32_t)p.n_tiles) {
      const int m0 = (int)(t / p.tiles_n) * G::BM;
      const uint32_t t_take = (uint32_t)now_ticks();
      uint32_t ready = 1;
      if (!all_landed) {
        const uint32_t v = wait_partials<G::BM>(p, h, m0, sb);
        ready = v & 1u;
        all_landed = (v >> 1) & 1u;
      }
      const uint32_t t_ready = (uint32_t)now_ticks();
      if (ready) {
        reduce_tile<G::BM, G::BN>(p, (int)t);
        if (p.tile_log && tid == 0) {
          if (p.mode == MODE_REDUCE) {
            p.tile_log[8 * t] = m0 / p.mb;
            p.tile_log[8 * t + 1] = (int32_t)t;
          }
          log_reduction(p, (int)t, m0, t_take, t_ready);
        }
      }
    }
    const uint32_t next = tid == 0 ? add_relaxed(&h->red_next, 1u) : 0u;
    i = wg_bcast(next, sb);
  }
}

__device__ __forceinline__ void rs_finish(const RsParams& p, WsHeader* h, uint32_t* sb) {
  __syncthreads();
  uint32_t last = 0;
  if (threadIdx.x == 0) {
    fence_release();
    last = add_relaxed(&h->done, 1u) == gridDim.x - 1;
    if (last) fence_acquire();
  }
  last = wg_bcast(last, sb);
  if (!last) return;
  if (p.mode == MODE_ROLES)
    for (int i = threadIdx.x; i < p.n_tiles; i += blockDim.x) st_relaxed(&p.fifo[i], 0u);
  if (p.unit_cnt && (p.mode == MODE_COPY || p.mode == MODE_EPI || p.mode == MODE_ROLES))
    for (int i = threadIdx.x; i < p.n_units; i += blockDim.x) st_relaxed(&p.unit_cnt[i], 0u);
  if (threadIdx.x == 0) {
    st_relaxed(&h->ticket, 0u);
    st_relaxed(&h->tile_next, 0u);
    st_relaxed(&h->red_next, 0u);
    st_relaxed(&h->prod_next, 0u);
    st_relaxed(&h->copy_next, 0u);
    st_relaxed(&h->aux[0], 0u);
    st_relaxed(&h->aux[1], 0u);
    for (int i = 0; i < XQ; ++i) st_relaxed(&h->aux[XQ_AUX + i], 0u);
    st_relaxed(&h->abort, 0u);
    __hip_atomic_store(&h->t0, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    st_relaxed(&h->done, 0u);
  }
}

template <class G, class SM>
__device__ __forceinline__ void rs_body(const RsParams& p, SM sm, uint32_t* sb) {
  WsHeader* h = p.hdr;
  const uint32_t ticket = wg_bcast(threadIdx.x == 0 ? add_relaxed(&h->ticket, 1u) : 0u, sb);
  // copy workgroups hold the earliest tickets, so every wait for a unit is a
  // wait for a workgroup that is already running
  const bool copier = p.mode == MODE_COPY ||
                      (p.unit_cnt && (p.mode == MODE_EPI || p.mode == MODE_ROLES) && ticket < (uint32_t)p.n_copy);
  if (copier) rs_copy_role(p, h, sb);
  if (p.mode != MODE_COPY) {
    const bool reducer = p.mode == MODE_REDUCE || (p.mode == MODE_ROLES && ticket >= (uint32_t)p.n_compute);
    if (!reducer) rs_compute_role<G>(p, h, sm, sb);
    if (p.mode == MODE_ROLES || p.mode == MODE_REDUCE) rs_reduce_role<G>(p, h, sb);
  }
  rs_finish(p, h, sb);
}

template <class G>
__global__ __launch_bounds__(G::NT) void rs_kernel(const RsParams p) {
  __shared__ uint32_t sb[2];
  if constexpr (G::STAGES == 4) {
    __shared__ u32x4 a0[G::SA_U4], a1[G::SA_U4], a2[G::SA_U4], a3[G::SA_U4];
    __shared__ u32x4 b0[G::SB_U4], b1[G::SB_U4], b2[G::SB_U4], b3[G::SB_U4];
    rs_body<G>(p, Smem4{{a0, a1, a2, a3}, {b0, b1, b2, b3}}, sb);
  } else {
    __shared__ u32x4 lds[G::LDS_U4];
    rs_body<G>(p, Smem1{lds}, sb);
  }
}

// Default: the direct-to-LDS 256x256 tile when K is a multiple of 128 and
// the owner blocks hold whole tile rows, else 128x128.
inline int tile_bm(int t) {
  return (t == TILE_256x256 || t == TILE_256x128 || t == TILE_256x256_DMA || t == TILE_256x128_DMA) ? 256 : 128;
}

}  // namespace

// Per-shape default tile (mk_plan reports it).  With K % 128 == 0 the
// direct-to-LDS tiles whose height divides the owner row blocks (mb rows;
// 256 for the all-reduce, where a ragged last tile row is masked) compete on
// an estimate of when the last tile ends on the CU count, in units of one
// 256x256 tile: rounds of 256x256 tiles at 1, or rounds of 128x256 tiles at
// 0.6 (measured 0.57 at M = N = 8192, K = 3584); the 256x256 tile wins ties.  Below one round of 256x256 tiles the
// 128x256 tile spreads the work over more CUs: at K = 4096 GEMM+RS over 8
// owners took 0.149 against 0.169 ms at M = 2048, N = 4096 (0.238 against
// 0.285 ms as GEMM+AR), and 0.203 against 0.220 ms at M = 4096, N = 2048,
// K = 8192, R = 4; from one round up the 256x256 tile was as fast or faster
// (0.736 against 0.842 ms at M = N = 8192, K = 3584).  Without a direct-to-LDS
// fit, the register-staged 128x128 tile.
namespace mkp {
int rs_default_tile(int64_t M, int64_t N, int64_t K, int mb, int n_cu) {
  if (!TileGemmD<256, 256>::supports_k((int)K)) return TILE_128x128;
  const int64_t grid = std::max(n_cu, 1);
  const int64_t t5 = ((M + 255) / 256) * ((N + 255) / 256), t8 = ((M + 127) / 128) * ((N + 255) / 256);
  const double c5 = (double)((t5 + grid - 1) / grid), c8 = 0.6 * (double)((t8 + grid - 1) / grid);
  if (mb % 256 == 0 && c5 <= c8) return TILE_256x256_DMA;
  if (mb % 128 == 0) return TILE_128x256_DMA;
  return TILE_128x128;
}
}  // namespace mkp

// Workspace: header, per-unit arrival counters, produced-tile FIFO, then
// (bf16 output) the fp32 staging area of the reduce role.
constexpr size_t RS_UNIT_BYTES = MK_MAX_UNITS * sizeof(uint32_t);

extern "C" size_t mk_gemm_rs_workspace(int64_t M, int64_t K, int64_t N, int R, int out_dtype) {
  (void)K; (void)R;
  if (M <= 0 || N <= 0) return sizeof(WsHeader) + RS_UNIT_BYTES;
  const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
  size_t bytes = sizeof(WsHeader) + RS_UNIT_BYTES + (size_t)tiles * 4;
  bytes = (bytes + 255) & ~(size_t)255;
  if (out_dtype == MK_BF16) bytes += (size_t)M * N * 4;   // fp32 staging for the reduce role
  return bytes;
}

template <class G>
static int run_rs(RsParams& p, const mk_launch& o, const mkh::Schedule* s, const mkh::DevInfo* d, hipStream_t st,
                  bool can_stage) {
  p.tiles_m = (p.M + G::BM - 1) / G::BM;
  p.tiles_n = (p.N + G::BN - 1) / G::BN;
  p.n_tiles = p.tiles_m * p.tiles_n;
  if (s) {
    // Tile rows ordered by the issue position of the last unit (over every
    // peer) under them, so the GEMM tiles whose partial sums land first are
    // produced first.
    if (p.tiles_m > MK_MAX_UNITS)
      return mkh::fail(MK_ERR_UNSUPPORTED, "%d tile rows: at most %d with an arrival schedule", p.tiles_m,
                       MK_MAX_UNITS);
    std::vector<int> rb(p.tiles_m), key(p.tiles_m);
    for (int t = 0; t < p.tiles_m; ++t) {
      const int b0 = t * G::BM / p.unit_rows, b1 = (std::min(p.M, (t + 1) * G::BM) - 1) / p.unit_rows;
      int k = 0;
      for (int q = 0; q + 1 < p.R; ++q)
        for (int b = b0; b <= b1; ++b) k = std::max(k, s->pos[q * p.n_blocks + b]);
      rb[t] = t;
      key[t] = k;
    }
    std::stable_sort(rb.begin(), rb.end(), [&](int a, int b) { return key[a] < key[b]; });
    for (int t = 0; t < p.tiles_m; ++t) p.rb_order[t] = (uint16_t)rb[t];
  }
  int occ = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, rs_kernel<G>, G::NT, 0);
  if (e != hipSuccess) return mkh::hip_fail(e, "occupancy query");
  if (occ < 1) return mkh::fail(MK_ERR_UNSUPPORTED, "kernel does not fit on a CU");
  const int full = d->n_cu * occ;
  const int grid = o.grid > 0 ? std::min(o.grid, full) : full;
  if (!can_stage) return mkh::fail(MK_ERR_WORKSPACE, "bf16 output needs the fp32 staging workspace");
  // Per-XCD band queues where the tile columns split evenly over the XCDs; a
  // band holds about as many tiles per XCD as the XCD has workgroups.
  p.xcd_queues = o.queue_mode == 1 && p.tiles_n % XQ == 0;
  p.band_rows = p.xcd_queues ? std::max(1, grid / (XQ * (p.tiles_n / XQ))) : 1;
  // Copy workgroups (arrival schedule): every workgroup copies first by
  // default, then computes; n_copy selects fewer.
  const uint32_t n_work = (uint32_t)p.n_units * p.parts;
  p.n_copy = s ? (int)std::min<int64_t>(o.n_copy > 0 ? o.n_copy : grid, std::min<int64_t>(grid, n_work)) : 0;
  if (o.mode >= 1) {   // unfused baseline: copies, GEMM to fp32 staging, then a reduce-scatter kernel
    // (measurement: mode 2 = the reduce kernel alone on what is staged, 3 = the GEMM kernel alone)
    if (s && o.mode == 1) {
      p.mode = MODE_COPY;
      hipLaunchKernelGGL(rs_kernel<G>, dim3(grid), dim3(G::NT), 0, st, p);
      if ((e = hipGetLastError()) != hipSuccess) return mkh::hip_fail(e, "copy kernel launch");
    }
    if (o.mode != 2) {
      p.mode = MODE_GEMM;
      hipLaunchKernelGGL(rs_kernel<G>, dim3(grid), dim3(G::NT), 0, st, p);
      if ((e = hipGetLastError()) != hipSuccess) return mkh::hip_fail(e, "gemm kernel launch");
    }
    if (o.mode != 3) {
      p.mode = MODE_REDUCE;
      hipLaunchKernelGGL(rs_kernel<G>, dim3(grid), dim3(G::NT), 0, st, p);
      if ((e = hipGetLastError()) != hipSuccess) return mkh::hip_fail(e, "reduce kernel launch");
    }
    return MK_OK;
  }
  const int n_reduce = o.n_reduce;   // 0 = default (epilogue reduction), -1 = epilogue
  if (n_reduce > 0) {
    if (n_reduce >= grid) return mkh::fail(MK_ERR_INVALID, "n_reduce %d leaves no compute workgroup", n_reduce);
    p.mode = MODE_ROLES;
    p.n_compute = grid - n_reduce;
  } else {
    p.mode = MODE_EPI;
    p.n_compute = grid;
  }
  hipLaunchKernelGGL(rs_kernel<G>, dim3(grid), dim3(G::NT), 0, st, p);
  if ((e = hipGetLastError()) != hipSuccess) return mkh::hip_fail(e, "fused kernel launch");
  return MK_OK;
}

// GEMM + reduce-scatter (all_reduce false: row block r of the reduced sum
// goes to outs[r]) or GEMM + all-reduce (true: the whole reduced sum goes to
// every outs[r]); one kernel for both, the all-reduce writing each reduced
// tile R times.
static int gemm_reduce(const void* A, const void* B, int64_t M, int64_t K, int64_t N, const float* const* partials,
                       int R, void* const* outs, int out_dtype, const mk_arrival* arrival,
                       float* const* p_landing, const mk_launch* launch, void* workspace, size_t workspace_bytes,
                       void* stream, bool all_reduce) {
  using mkh::fail;
  if (!A || !B || !outs) return fail(MK_ERR_INVALID, "A, B and the outputs must be non-NULL");
  if (R < 1 || R > MK_MAX_RANKS) return fail(MK_ERR_UNSUPPORTED, "R=%d outside [1,%d]", R, MK_MAX_RANKS);
  if (M < 1 || K < 8 || N < 8) return fail(MK_ERR_INVALID, "empty or too small shape");
  if (K % 8 || N % 8) return fail(MK_ERR_UNSUPPORTED, "K and N must be multiples of 8");
  if (!all_reduce && M % R) return fail(MK_ERR_INVALID, "M (%lld) not divisible by R (%d)", (long long)M, R);
  if (M > (1 << 30) || K > (1 << 20) || N > MK_MAX_COLS || K * N * 2 >= (1ll << 31) || M * N * 4 >= (1ll << 40))
    return fail(MK_ERR_UNSUPPORTED, "dimension too large");
  if (R > 1 && !partials) return fail(MK_ERR_INVALID, "partials is NULL");
  if (out_dtype != MK_BF16 && out_dtype != MK_F32) return fail(MK_ERR_INVALID, "out_dtype %d", out_dtype);
  for (int r = 0; r + 1 < R; ++r)
    if (!partials[r] || !mkh::aligned16(partials[r])) return fail(MK_ERR_INVALID, "partial %d NULL or misaligned", r);
  for (int r = 0; r < R; ++r)
    if (!outs[r] || !mkh::aligned16(outs[r])) return fail(MK_ERR_INVALID, "output %d NULL or misaligned", r);
  if (!mkh::aligned16(A) || !mkh::aligned16(B)) return fail(MK_ERR_INVALID, "A and B must be 16-byte aligned");
  // Arrival schedule of the partial sums: (R-1) * (M / unit_rows) units.
  mkh::Schedule sched;
  const mkh::Schedule* s = nullptr;
  if (arrival) {
    if (R < 2) return fail(MK_ERR_SCHEDULE, "an arrival schedule needs partial sums (R >= 2)");
    if (arrival->unit_rows <= 0 || M % arrival->unit_rows)
      return fail(MK_ERR_SCHEDULE, "unit_rows (%d) must divide M (%lld)", arrival->unit_rows, (long long)M);
    const int rc = mkh::make_schedule(arrival, (int64_t)(R - 1) * M, 1, &sched);
    if (rc) return rc;
    s = &sched;
  }
  if (p_landing) {
    if (!s) return fail(MK_ERR_INVALID, "landing buffers need an arrival schedule");
    for (int r = 0; r + 1 < R; ++r)
      if (!p_landing[r] || !mkh::aligned16(p_landing[r]))
        return fail(MK_ERR_INVALID, "landing buffer %d NULL or misaligned", r);
  }
  const int mb = all_reduce ? (int)M : (int)(M / R);   // rows per output block
  const mk_launch o = mkh::launch_opts(launch);
  if (o.mode < 0 || o.mode > 3) return fail(MK_ERR_INVALID, "mode %d", o.mode);
  if (o.mode >= 2 && arrival) return fail(MK_ERR_INVALID, "modes 2 and 3 (one phase alone) take no arrival schedule");
  if (o.grid < 0 || o.n_reduce < -1 || o.n_copy < 0 || o.copy_kib < 0)
    return fail(MK_ERR_INVALID, "bad grid, n_reduce, n_copy or copy_kib");
  if (o.queue_mode < 0 || o.queue_mode > 1) return fail(MK_ERR_INVALID, "queue_mode %d", o.queue_mode);
  // Default: by shape and the CU count (mkp::rs_default_tile; 256 CUs when
  // no device answers, which then fails below).
  int tile = o.tile;
  if (!tile) {
    const mkh::DevInfo* dd = mkh::dev_info();
    tile = mkp::rs_default_tile(M, N, K, all_reduce ? 256 : mb, dd ? dd->n_cu : 256);
  }
  if (tile <= 0 || tile >= TILE_COUNT) return fail(MK_ERR_INVALID, "tile id %d", tile);
  // The register-staged 256x256 tile is not built for this operation: with
  // the partial sums added from its accumulators its K loop spills.
  if (tile == TILE_256x256)
    return fail(MK_ERR_UNSUPPORTED, "tile %d is not available for GEMM+RS/AR (use tile %d)", tile, TILE_256x256_DMA);
  if (tile == TILE_128x128_DMA8 || tile == TILE_256x256_DMA_W8 || tile == TILE_128x128_PC)
    return fail(MK_ERR_UNSUPPORTED, "tile %d is built for AllGather+GEMM only", tile);
  if (mk_is_dma_tile(tile) && !TileGemmD<256, 256>::supports_k((int)K))
    return fail(MK_ERR_UNSUPPORTED, "tile %d needs K %% 128 == 0", tile);
  if (!all_reduce && mb % tile_bm(tile))
    return fail(MK_ERR_UNSUPPORTED, "rows per owner (%d) must be a multiple of the tile height %d", mb, tile_bm(tile));
  if (!workspace) return fail(MK_ERR_WORKSPACE, "workspace is NULL");
  const size_t need_min = mk_gemm_rs_workspace(M, K, N, R, MK_F32);
  if (workspace_bytes < need_min) return fail(MK_ERR_WORKSPACE, "workspace %zu bytes < %zu", workspace_bytes, need_min);
  const size_t need_stage = need_min + (size_t)M * N * 4;
  const bool have_stage = workspace_bytes >= need_stage;
  const mkh::DevInfo* d = mkh::dev_info();
  if (!d) return MK_ERR_HIP;

  RsParams p;
  memset(&p, 0, sizeof p);
  p.A = (const uint16_t*)A;
  p.B = (const uint16_t*)B;
  for (int r = 0; r + 1 < R; ++r) {
    p.Psrc[r] = partials[r];
    p.P[r] = p_landing ? p_landing[r] : partials[r];
  }
  for (int r = 0; r < R; ++r) p.out[r] = outs[r];
  p.hdr = (WsHeader*)workspace;
  p.fifo = (uint32_t*)((char*)workspace + sizeof(WsHeader) + RS_UNIT_BYTES);
  // fp32 output can be staged in place in the output blocks (all-reduce: in
  // output 0, which the reduction then rewrites in place).
  p.stage = out_dtype == MK_F32 ? nullptr : (have_stage ? (float*)((char*)workspace + need_min) : nullptr);
  const bool can_stage = out_dtype == MK_F32 || have_stage;
  p.tile_log = o.tile_log;
  p.copy_log = o.copy_log;
  p.spin_limit = mkh::spin_ticks(o, d);
  p.M = (int)M; p.K = (int)K; p.N = (int)N; p.R = R; p.mb = mb;
  p.n_dst = all_reduce ? R : 1;
  p.out_bf16 = out_dtype == MK_BF16;
  p.withhold = -1;
  if (s) {
    p.unit_cnt = (uint32_t*)((char*)workspace + sizeof(WsHeader));
    p.n_units = s->n_units;
    p.unit_rows = s->unit_rows;
    p.n_blocks = (int)(M / s->unit_rows);
    p.withhold = s->withhold;
    p.copy_data = p_landing != nullptr;
    // Copy items ("parts") of about copy_kib KiB in whole rows that divide the
    // unit (1 MiB by default; one release each).  Without landing buffers
    // nothing is moved and a unit is one item.
    const int64_t row_bytes = N * 4;
    const int64_t item_bytes = (int64_t)(o.copy_kib > 0 ? o.copy_kib : 1024) << 10;
    int part_rows = p.copy_data ? (int)std::max<int64_t>(1, std::min<int64_t>(s->unit_rows, item_bytes / row_bytes))
                                : s->unit_rows;
    while (part_rows > 1 && (s->unit_rows % part_rows || (int64_t)part_rows * row_bytes > (1ll << 30))) --part_rows;
    p.part_rows = part_rows;
    p.part_bytes = (uint32_t)std::min<int64_t>((int64_t)part_rows * row_bytes, 1ll << 30);
    p.parts = s->unit_rows / part_rows;
    for (int j = 0; j < s->n_units; ++j) {
      p.order[j] = (uint16_t)s->order[j];
      p.delay_ticks[j] = (uint32_t)mkh::ns_to_ticks(s->delay_ns[j], d->wall_khz);
    }
  }
  const hipStream_t st = (hipStream_t)stream;
  switch (tile) {
    case TILE_128x128: return run_rs<TileGemm<128, 128, 2, 2>>(p, o, s, d, st, can_stage);
    case TILE_256x128: return run_rs<TileGemm<256, 128, 2, 2>>(p, o, s, d, st, can_stage);
    case TILE_128x256: return run_rs<TileGemm<128, 256, 2, 2>>(p, o, s, d, st, can_stage);
    case TILE_256x256_DMA: return run_rs<TileGemmD<256, 256, false>>(p, o, s, d, st, can_stage);
    case TILE_128x128_DMA: return run_rs<TileGemmD<128, 128, false>>(p, o, s, d, st, can_stage);
    case TILE_256x128_DMA: return run_rs<TileGemmD<256, 128, false>>(p, o, s, d, st, can_stage);
    case TILE_128x256_DMA: return run_rs<TileGemmD<128, 256, false>>(p, o, s, d, st, can_stage);
  }
  return fail(MK_ERR_INVALID, "tile id %d", tile);
}

extern "C" int mk_gemm_rs(const void* A, const void* B, int64_t M, int64_t K, int64_t N,
                          const float* const* partials, int R, void* const* out_owner, int out_dtype,
                          const mk_arrival* arrival, float* const* p_landing, const mk_launch* launch,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_reduce(A, B, M, K, N, partials, R, out_owner, out_dtype, arrival, p_landing, launch, workspace,
                     workspace_bytes, stream, false);
}

extern "C" size_t mk_gemm_ar_workspace(int64_t M, int64_t K, int64_t N, int R, int out_dtype) {
  return mk_gemm_rs_workspace(M, K, N, R, out_dtype);
}

extern "C" int mk_gemm_ar(const void* A, const void* B, int64_t M, int64_t K, int64_t N,
                          const float* const* partials, int R, void* const* out_rank, int out_dtype,
                          const mk_arrival* arrival, float* const* p_landing, const mk_launch* launch,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_reduce(A, B, M, K, N, partials, R, out_rank, out_dtype, arrival, p_landing, launch, workspace,
                     workspace_bytes, stream, true);
}
