// Direct-to-LDS variant of the block tile GEMM (gfx950).
//
// Operands go HBM -> LDS with buffer_load_dwordx4 ... lds (no VGPR staging)
// through a 4-stage ring of 32-deep K slices.  A is stored [row][k] and read
// with ds_read_b128; B stays row-major [k][n] in LDS and each MFMA B fragment
// is assembled by two ds_read_b64_tr_b16 (the gfx950 LDS transpose read:
// within each group of 16 lanes, lane i receives element i%4 of the 64-bit
// rows addressed by lanes 4r + (i%16)/4, r = 0..3; pointing lane L at row
// k0 + (L%16)/4, column nb + 4(L%4) therefore hands lane i the four k-values
// of column nb + i%16).
//
// gfx950 LDS has 64 four-byte banks (256 bytes per clock).  Both layouts are
// XOR-swizzled in 16-byte units so that every fragment read is free of bank
// conflicts at that width: A (64-byte rows) swaps chunk c of row r with
// c ^ ((r >> 2) & 3), so 16 consecutive rows cover all 64 banks; B (512-byte
// rows) swaps chunk c of k-row r with c ^ ((r & 3) << 2), so the four k-rows a
// transpose read touches fall on four different 64-byte bank groups.  The
// swizzle is applied on the global side of each copy, because every DMA
// instruction fills 1 KiB of LDS linearly.
//
// Schedule, per K slice kt (stage kt%4), with no branch in the loop:
//   wait for this wave's DMA of slice kt+1 and for its own fragment reads of
//        slice kt, barrier   (slice kt+1 visible to all waves; no wave reads
//        stage kt%4 any more)
//   the MFMAs of slice kt (fragments read one slice earlier) in chunks, each
//        followed by its share of the fragment reads of slice kt+1 and of the
//        DMA of slice kt+4 into stage kt%4
// so three slices are in flight while a slice is multiplied, and the DMA
// issue overlaps the matrix pipeline (issued all at once after the barrier
// it held back each slice's first MFMA: 11% of the GEMM time).  The DMA is
// issued through inline asm so the compiler does not add its own
// (conservative) waits on it; the explicit waits and the barrier are one asm
// statement with a memory clobber, so no LDS access moves across them.
#pragma once

#include "mk_device.h"

namespace mk {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Buffer descriptor as four scalars: base, stride 0, num_records = bytes,
// raw 32-bit data format.
__device__ __forceinline__ u32x4 buf_desc(const void* p, uint32_t bytes) {
  const uint64_t b = (uint64_t)p;
  u32x4 d;
  d[0] = uni((uint32_t)b);
  d[1] = uni((uint32_t)(b >> 32)) & 0xffffu;
  d[2] = uni(bytes);
  d[3] = 0x00020000u;
  return d;
}

// One 16-byte-per-lane DMA: lane i's 16 bytes land at LDS byte lds + 16*i.
// M0 is saved and restored around it.  A scalar write of M0 followed by an
// LDS DMA needs one wait state on gfx9-family parts (the DMA could otherwise
// take the previous M0 as its LDS address); inline asm is outside the
// compiler's hazard recognizer, so the s_nop is written here.
__device__ __forceinline__ void dma16(u32x4 desc, uint32_t lds, uint32_t voff, uint32_t soff) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds), "v"(voff), "s"(desc), "s"(soff)
      : "memory");
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding and all its LDS reads have returned, then barrier.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Tiles of 128 or 256 rows by 128 or 256 columns, 4 waves (2x2, each wave a
// (BM/2)x(BN/2) block of 32x32 MFMA tiles) or 8 waves (2x4, two per SIMD,
// each wave (BM/2)x(BN/4)), with a ring of STAGES K slices (4 by default; a
// deeper ring keeps more operand bytes in flight per CU, which pays where
// the GEMM streams B and the tile is small).  Per 32-deep K slice the
// workgroup's DMA moves BM/16 KiB of A (16 rows per instruction) and BN/16
// KiB of B (1024 / (2*BN) k-rows per instruction); block blk is moved by
// wave blk % WAVES.
//
// A narrow tile computes only the first CN < BN columns of the BN loaded
// (CN a multiple of 32 * WN; the caller binds at most CN columns, so the DMA
// of the columns past them reads nothing and writes zeros), with WM wave
// rows: 256x192 with 8 waves as 4x2, each wave 64x96.  Every 32x32 output
// block is formed by the same MFMA sequence as in the full-width tile, so
// the two give identical bits.
//
// INTERLEAVE pins one LDS read after each MFMA inside a chunk.  It helps
// when registers are to spare; a kernel that keeps more state live across
// the K loop (GEMM+RS) turns it off to keep the loop free of spills.
//
// GA (gathered A): tile row r is A row idx[r] / div for an index array idx
// given at bind time (the MoE grouped GEMM reads each expert's rows from the
// received tokens through the dispatch permutation); each A DMA instruction
// then has its own per-lane row offset, and only the K slice goes into the
// scalar offset.
template <int BM_ = 256, int BN_ = 256, bool INTERLEAVE = true, int STAGES_ = 4, int WAVES_ = 4, int WM_ = 2,
          int CN_ = BN_, bool GA = false>
struct TileGemmD {
  static constexpr int BM = BM_, BN = BN_, WAVES = WAVES_, WM = WM_, WN = WAVES_ / WM_, BK = 32, STAGES = STAGES_;
  static constexpr int CN = CN_;                                       // columns computed
  static constexpr int NT = 64 * WAVES;
  static constexpr int TM = BM / WM, TN = CN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2;   // per stage
  static constexpr int A_INS = A_BYTES / 1024 / WAVES, B_INS = B_BYTES / 1024 / WAVES;  // DMA per wave per slice
  static constexpr int D = A_INS + B_INS;                              // vm operations per slice
  static constexpr int B_ROWS = 1024 / (2 * BN);                       // k-rows per B instruction
  static constexpr int SA_U4 = A_BYTES / 16, SB_U4 = B_BYTES / 16;
  static constexpr int LDS_U4 = STAGES * (SA_U4 + SB_U4);
  static constexpr int READS = 2 * (FM + 2 * FN), MFMAS = 2 * FM * FN;  // per slice and wave
  static_assert((BM == 128 || BM == 256) && (BN == 128 || BN == 256), "tile shape");
  static_assert(WAVES % WM == 0 && TM % 32 == 0 && TN % 32 == 0 && CN <= BN, "wave grid of 32x32 blocks");
  static_assert(STAGES == 4 || STAGES == 8, "ring depth");
  static_assert(WAVES == 4 || WAVES == 8, "waves per workgroup");
  static_assert(A_INS >= 1 && B_INS >= 1 && (WAVES * B_ROWS) % 4 == 0, "DMA blocks per wave; B swizzle phase");
  static_assert((STAGES - 1) * D < 64, "vmcnt holds at most 63 outstanding operations");

  f32x16 acc[FM][FN];
  u32x4 dA, dB;
  uint32_t ldaB, ldbB, voA, voB;
  uint32_t voG[GA ? A_INS : 1];   // gathered A: per-instruction row offsets
  int nk;

  static __host__ __device__ constexpr bool supports_k(int K) { return K % (STAGES * BK) == 0; }

  __device__ __forceinline__ void bind(const uint16_t* A, int64_t lda, int mrows, const uint16_t* B,
                                       int64_t ldb, int ncols, const uint16_t* B_end, int K) {
    const int lane = threadIdx.x & 63;
    ldaB = uni((uint32_t)(lda * 2));
    ldbB = uni((uint32_t)(ldb * 2));
    const int rows = mrows < BM ? mrows : BM;
    dA = buf_desc(A, uni((uint32_t)(rows > 0 ? rows : 0) * ldaB));
    dB = buf_desc(B, uni((uint32_t)((B_end - B) * 2)));
    nk = uni(K) / BK;
    // A: LDS unit p = blk*64 + lane holds tile row p/4 = blk*16 + lane/4 and
    // physical chunk p%4, which is logical k-chunk (p%4) ^ ((row>>2)&3).
    voA = (uint32_t)(lane >> 2) * ldaB + (uint32_t)((lane & 3) ^ ((lane >> 4) & 3)) * 16u;
    // B: an instruction covers B_ROWS k-rows of BN/8 chunks; physical chunk
    // = logical ^ ((k-row & 3) << 2).  Block blk = i*WAVES + w starts at k-row
    // blk*B_ROWS, so k-row & 3 = (w*B_ROWS + lane / (BN/8)) & 3.
    const int w = threadIdx.x >> 6;
    const int rin = lane / (BN / 8);
    const int brow = (w * B_ROWS + rin) & 3;
    const int lchunk = (lane % (BN / 8)) ^ (brow << 2);
    voB = (lchunk * 8 < ncols) ? (uint32_t)rin * ldbB + (uint32_t)lchunk * 16u : OOB;
  }

  // Gathered A (GA): tile row r (r < mrows) is row idx[r] / div of A, which
  // has a_rows rows of lda elements, starting at column k0; rows past mrows
  // or whose index falls outside [0, a_rows) read as zero.  a_rows * lda * 2
  // must stay below 2^31 bytes, the out-of-range offset OOB.
  __device__ __forceinline__ void bind_rows(const uint16_t* A, int64_t lda, int a_rows, const int32_t* idx,
                                            int div, int mrows, int k0, const uint16_t* B, int64_t ldb, int ncols,
                                            const uint16_t* B_end, int K) {
    static_assert(GA, "gathered-A engine");
    bind(A, lda, 0, B, ldb, ncols, B_end, K);
    dA = buf_desc(A, uni((uint32_t)a_rows * ldaB));
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int rows = mrows < BM ? mrows : BM;
    const uint32_t chunk = (uint32_t)((lane & 3) ^ ((lane >> 4) & 3)) * 16u + (uint32_t)k0 * 2u;
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
      const int r = (i * WAVES + w) * 16 + (lane >> 2);
      const int t = r < rows ? idx[r] / div : -1;
      voG[i] = (uint32_t)t < (uint32_t)a_rows ? (uint32_t)t * ldaB + chunk : OOB;
    }
  }
  __device__ __forceinline__ uint32_t a_voff(int i) const {
    if constexpr (GA) return voG[i];
    else return voA;
  }
  __device__ __forceinline__ uint32_t a_soff(int blk, int kt) const {
    if constexpr (GA) return (uint32_t)(kt * BK * 2);
    else return (uint32_t)(blk * 16) * ldaB + (uint32_t)(kt * BK * 2);
  }

  // DMA of K slice kt into stage buffers (sa, sb): each wave fills A_INS KiB
  // of A (16-row blocks) and B_INS KiB of B (B_ROWS-row blocks).
  __device__ __forceinline__ void issue(u32x4* sa, u32x4* sb, int kt) {
    const int w = uni((int)(threadIdx.x >> 6));   // wave index: the same in every lane
    const uint32_t la = uni(lds_addr(sa)), lb = uni(lds_addr(sb));
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
      const int blk = i * WAVES + w;
      dma16(dA, uni(la + blk * 1024), a_voff(i), uni(a_soff(blk, kt)));
    }
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
      const int blk = i * WAVES + w;
      dma16(dB, uni(lb + blk * 1024), voB, uni((uint32_t)(kt * BK + blk * B_ROWS) * ldbB));
    }
  }

  __device__ __forceinline__ void zero_acc() {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }

  // Per-lane fragment byte offsets inside a stage.
  struct FragOfs { int a[2]; int b[FN]; };
  __device__ __forceinline__ FragOfs frag_offsets() const {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w % WM, wn = w / WM;
    const int hi = lane >> 5, g = lane >> 4, Lg = lane & 15;
    FragOfs f;
    const int arow = wm * TM + (lane & 31);
    const int as = ((lane & 31) >> 2) & 3;
    f.a[0] = arow * 64 + ((0 + hi) ^ as) * 16;
    f.a[1] = arow * 64 + ((2 + hi) ^ as) * 16;
    const int brow = (g >> 1) * 8 + (Lg >> 2);
    const int u = 2 * (g & 1) + ((Lg & 3) >> 1);
    // fragment j covers logical chunks 4c + (0..3), c = (wn*TN + 32j) / 32;
    // its k-rows have (row & 3) == Lg >> 2, so the group c is XORed with it
#pragma unroll
    for (int j = 0; j < FN; ++j)
      f.b[j] = brow * (BN * 2) + (4 * ((wn * FN + j) ^ (Lg >> 2)) + u) * 16 + (Lg & 1) * 8;
    return f;
  }

  // B fragments are kept as their two transposed-read halves and joined at
  // the MFMA (the join is register naming only).
  struct Frags { bf16x8 a[2][FM]; i16x4 bl[2][FN]; i16x4 bu[2][FN]; };

  static constexpr int CH = 2 * FM;                 // chunks per slice: (substep, A fragment)
  static constexpr int RPC = READS / CH;            // fragment reads per chunk
  static_assert(READS % CH == 0, "reads per chunk");

  // Fragment read r (0..READS-1) of a slice: per 16-deep substep, the FM A
  // fragments (one ds_read_b128 each), then the two halves of each of the FN
  // B fragments (one ds_read_b64_tr_b16 each).
  __device__ __forceinline__ void read_one(const u32x4* sa, const u32x4* sb, const FragOfs& fo, int r,
                                           Frags& f) const {
    const char* pa = (const char*)sa;
    const char* pb = (const char*)sb;
    const int ks = r / (READS / 2), rr = r % (READS / 2);
    if (rr < FM) {
      f.a[ks][rr] = __builtin_bit_cast(bf16x8, *(const u32x4*)(pa + fo.a[ks] + rr * 32 * 64));
    } else {
      const int j = (rr - FM) / 2, up = (rr - FM) % 2;
      const int base = fo.b[j] + ks * 16 * (BN * 2) + up * 4 * (BN * 2);
      const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pb + base));
      if (up) f.bu[ks][j] = v;
      else f.bl[ks][j] = v;
    }
  }

  // DMA instruction d (0..D-1) of slice kt into stage (sa, sb): A blocks
  // first, then B.  Past the last slice the offset is out of range, so the
  // instruction reads nothing and every slice keeps the same wait counts.
  __device__ __forceinline__ void issue_one(u32x4* sa, u32x4* sb, int kt, int d, bool more) {
    const int w = uni((int)(threadIdx.x >> 6));   // wave index: the same in every lane
    if (d < A_INS) {
      const int blk = d * WAVES + w;
      dma16(dA, uni(lds_addr(sa) + blk * 1024), more ? a_voff(d) : OOB, uni(a_soff(blk, kt)));
    } else {
      const int blk = (d - A_INS) * WAVES + w;
      dma16(dB, uni(lds_addr(sb) + blk * 1024), more ? voB : OOB, uni((uint32_t)(kt * BK + blk * B_ROWS) * ldbB));
    }
  }

  // One K slice: cur holds the fragments of slice kt, nxt receives those of
  // slice kt+1 (na/nb); slice kt+STAGES is loaded into stage kt%STAGES
  // (fa/fb).  The slice runs in CH chunks, chunk c = (substep c / FM, A
  // fragment c % FM):
  // its FN MFMAs, RPC of the next slice's fragment reads and its share of
  // the DMA.  Each DMA is an inline-asm statement the compiler schedules
  // around, so it ends a chunk; spread this way the DMA issue overlaps the
  // matrix pipeline instead of holding back the slice's first MFMA.
  __device__ __forceinline__ void step(int kt, const FragOfs& fo, const u32x4* na, const u32x4* nb,
                                       u32x4* fa, u32x4* fb, Frags& cur, Frags& nxt) {
    wait_barrier<(STAGES - 2) * D>();       // slice kt+1 landed (kt+2 .. kt+STAGES-1 may be in flight)
    const bool more = kt + STAGES < nk;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ks = c / FM, i = c % FM;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const bf16x8 bop =
            __builtin_bit_cast(bf16x8, __builtin_shufflevector(cur.bl[ks][j], cur.bu[ks][j], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[ks][i], bop, acc[i][j], 0, 0, 0);
      }
      // on the last slice these read a stage nobody uses
#pragma unroll
      for (int r = 0; r < RPC; ++r) read_one(na, nb, fo, c * RPC + r, nxt);
      // Interleave: one LDS read after each MFMA of the chunk.
      if constexpr (INTERLEAVE) {
        constexpr int PAIRS = FN < RPC ? FN : RPC;
#pragma unroll
        for (int q = 0; q < PAIRS; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        }
        if constexpr (FN > PAIRS) __builtin_amdgcn_sched_group_barrier(0x008, FN - PAIRS, 0);
        if constexpr (RPC > PAIRS) __builtin_amdgcn_sched_group_barrier(0x100, RPC - PAIRS, 0);
      }
#pragma unroll
      for (int d = c * D / CH; d < (c + 1) * D / CH; ++d) issue_one(fa, fb, kt + STAGES, d, more);
    }
  }

  // Full K loop.  With the default ring the four stages are distinct LDS
  // objects; a deeper ring lives in one array, stage s at a fixed offset.  If
  // `mark` is given, thread 0 sets *mark once three quarters of the K slices
  // are done (a workgroup that wants to start later than this one can wait
  // for it).
  __device__ __forceinline__ void run(Smem4 m, uint32_t* mark = nullptr) {
    static_assert(STAGES == 4, "four stage objects");
    run_ring(m.a, m.b, mark);
  }
  __device__ __forceinline__ void run(Smem1 m, uint32_t* mark = nullptr) {
    u32x4* a[STAGES];
    u32x4* b[STAGES];
#pragma unroll
    for (int s = 0; s < STAGES; ++s) {
      a[s] = m.lds + s * (SA_U4 + SB_U4);
      b[s] = a[s] + SA_U4;
    }
    run_ring(a, b, mark);
  }

  __device__ __forceinline__ void run_ring(u32x4* const* a, u32x4* const* b, uint32_t* mark) {
    const FragOfs fo = frag_offsets();
    zero_acc();
    if (nk == 0) return;
    // nk is a multiple of STAGES (supports_k), so every stage starts loaded
#pragma unroll
    for (int s = 0; s < STAGES; ++s) issue(a[s], b[s], s);
    wait_barrier<(STAGES - 1) * D>();
    Frags r0, r1;
#pragma unroll
    for (int r = 0; r < READS; ++r) read_one(a[0], b[0], fo, r, r0);
    const int mark_kt = (nk * 3 / 4) & ~(STAGES - 1);
    for (int kt = 0; kt < nk; kt += STAGES) {
      if (mark && kt == mark_kt && threadIdx.x == 0) st_relaxed(mark, 1u);
#pragma unroll
      for (int s = 0; s < STAGES; s += 2) {
        step(kt + s, fo, a[(s + 1) % STAGES], b[(s + 1) % STAGES], a[s], b[s], r0, r1);
        step(kt + s + 1, fo, a[(s + 2) % STAGES], b[(s + 2) % STAGES], a[s + 1], b[s + 1], r1, r0);
      }
    }
    // the out-of-range DMAs issued past the last slice must not land in LDS
    // after the caller has started reusing it
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();                        // LDS free for the next tile
  }

  template <class Fn>
  __device__ __forceinline__ void for_each(Fn&& f) const {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w % WM, wn = w / WM;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * TM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const int col = wn * TN + j * 32 + (lane & 31);
          f(row, col, acc[i][j][r]);
        }
  }
};

}  // namespace mk
