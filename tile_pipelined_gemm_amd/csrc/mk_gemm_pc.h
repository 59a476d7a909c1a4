// Producer/consumer block tile for bandwidth-bound GEMMs whose A is small
// (a skinny A: a single 128-row tile row, every tile of which reads all of
// A while it streams its own column stripe of B).  128 x 128 output tile,
// 8 waves:
//
//  * waves 0-3 compute (by default 4 x 1, each a 32 x 128 block of 32x32
//    MFMA tiles, so every A fragment is loaded once per workgroup; 2 x 2
//    waves load each one twice and measured 2 % slower at M = 128,
//    K = 8192, N = 28672).  They load their A fragments straight from global
//    memory into registers (A is L2-resident: all tiles share it), PA slices
//    ahead, and read their B fragments from LDS with the transposing
//    ds_read_b64_tr_b16;
//  * waves 4-7 produce: they only move B from HBM into a ring of STAGES
//    32-deep K slices in LDS (buffer_load_dwordx4 ... lds, 8 KiB per slice),
//    so the whole LDS holds B in flight.
//
// A is read from a packed copy in MFMA operand order, written once per call
// by whoever gathers A (packed_offset): per 32-deep slice, per 32-row group
// and per 16-deep half of the slice, one 1 KiB block in which lane l holds
// the 16 bytes that the 32x32x16 MFMA takes from it (row l % 32, k-chunk
// l / 32).  Each A load is then one contiguous 1 KiB (8 whole cache lines);
// loading the fragments from row-major A touches 32 lines per instruction,
// 32 bytes of each, and at the skinny shape those scattered requests slowed
// the B stream by half.
//
// Vector-memory waits complete in issue order, so a wave that waited for its
// A loads would also wait for every DMA it had issued before them: with the
// DMA in separate waves, the compute waves' A waits never drain the B ring,
// and the producers keep STAGES - 1 slices of B in flight.
//
// Schedule, per slice kt (one barrier per slice for all 8 waves; the barriers
// are raw s_barrier after explicit waits, so neither side drains the vector
// loads it keeps in flight):
//   producers: wait until slice kt+1 has landed, barrier, DMA slice
//              kt+STAGES into stage kt % STAGES (freed: the consumers read its
//              fragments during slice kt-1 and waited for them before the
//              barrier);
//   consumers: wait for their fragment reads of slice kt, barrier, load the A
//              fragments of slice kt+PA, then the MFMAs of slice kt with the B
//              fragments of slice kt+1 read in between.
// DMAs and A loads past the last slice take the out-of-range offset (nothing
// is read; a DMA then writes zeros), so every slice has the same wait counts.
// B stays row-major [k][n] in LDS, XOR-swizzled in 16-byte units (chunk c of
// k-row r at c ^ ((r & 3) << 2)) so the transposing reads are free of bank
// conflicts, as in the direct-to-LDS engine.  Each output element sees the
// same MFMA sequence as in the other engines, so the results are the same bits.
#pragma once

#include "mk_gemm_dma.h"

namespace mk {

template <int STAGES_ = 16, int PA_ = 4, int CWM_ = 4>
struct TileGemmPC {
  static constexpr int BM = 128, BN = 128, BK = 32, STAGES = STAGES_, PA = PA_;
  static constexpr int WM = CWM_, WN = 4 / CWM_, CW = 4, PW = 4, WAVES = CW + PW;
  static constexpr int NT = 64 * WAVES;
  static constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  static_assert(WM * WN == CW && FM >= 1 && FN >= 1, "compute wave grid");
  static constexpr bool PACKED_A = true;                      // A from a packed copy (packed_offset)
  static constexpr int B_BYTES = BK * BN * 2;                 // 8 KiB per stage
  static constexpr int B_INS = B_BYTES / 1024 / PW;           // DMA per producer wave per slice
  static constexpr int B_ROWS = 1024 / (2 * BN);              // k-rows per DMA instruction
  static constexpr int SB_U4 = B_BYTES / 16, SA_U4 = 0;
  static constexpr int LDS_U4 = STAGES * SB_U4;
  static_assert(B_INS >= 1 && B_ROWS == 4, "B DMA blocks");
  static_assert((STAGES - 1) * B_INS < 64, "vmcnt holds at most 63 outstanding operations");
  static_assert(PA % 2 == 0 && STAGES % PA == 0, "register ring of A and double-buffered B fragments");

  f32x16 acc[FM][FN];
  __amdgpu_buffer_rsrc_t rA;
  u32x4 dB;
  uint32_t wmA, ldbB, voA, voB;   // wmA: the wave's first 32-row group
  int nk;

  static __host__ __device__ constexpr bool supports_k(int K) { return K % (PA * BK) == 0; }

  // Byte offset, inside the packed copy of one 128-row block of A, of the 16
  // bytes at row rr (0..127) and 16-byte chunk c (elements 8c .. 8c+7) of
  // that row: slice c / 4, 32-row group rr / 32, half (c / 2) % 2 of the
  // slice, lane rr % 32 + 32 (c % 2).  A block holds 128 * K bf16.
  static __host__ __device__ __forceinline__ uint32_t packed_offset(int rr, int c) {
    return ((((uint32_t)(c >> 2) * 4u + (uint32_t)(rr >> 5)) * 2u + (uint32_t)((c >> 1) & 1)) * 64u +
            (uint32_t)((rr & 31) + 32 * (c & 1))) * 16u;
  }

  __device__ __forceinline__ int wave() const { return uni((int)(threadIdx.x >> 6)); }

  // The consumers' barrier: waits for their own LDS reads only, so the A
  // loads they keep in flight (vector memory) are not drained at every slice
  // (a plain __syncthreads would wait for them).
  static __device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }

  // A: the packed copy of the tile's 128-row block (its rows past the
  // matrix's last row hold whatever was there; they only reach output rows
  // that are not stored).  lda and mrows are not used.
  __device__ __forceinline__ void bind(const uint16_t* A, int64_t lda, int mrows, const uint16_t* B, int64_t ldb,
                                       int ncols, const uint16_t* B_end, int K) {
    (void)lda; (void)mrows;
    const int lane = threadIdx.x & 63, w = wave();
    ldbB = uni((uint32_t)(ldb * 2));
    nk = uni(K) / BK;
    rA = make_rsrc(uni(A), uni((uint32_t)nk * (BM * BK * 2)));
    const int wm = (w % CW) % WM;
    wmA = uni((uint32_t)(wm * FM));                // first of the wave's FM 32-row groups
    voA = (uint32_t)lane * 16u;
    // B: DMA instruction blk of a slice covers k-rows 4 blk .. 4 blk + 3;
    // lane L lands at 16 L, k-row L / 16, physical chunk L % 16 = logical
    // chunk (L % 16) ^ ((k-row & 3) << 2)
    dB = buf_desc(B, uni((uint32_t)((B_end - B) * 2)));
    const int rin = lane / (BN / 8);
    const int lchunk = (lane % (BN / 8)) ^ ((rin & 3) << 2);
    voB = (lchunk * 8 < ncols) ? (uint32_t)rin * ldbB + (uint32_t)lchunk * 16u : OOB;
  }

  __device__ __forceinline__ void zero_acc() {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }

  // ---------------------------------------------------------- producer side
  // DMA of slice kt into stage `st`: producer p moves blocks p, p + PW, ...
  __device__ __forceinline__ void produce(const u32x4* lds, int st, int kt, int p) {
    const uint32_t base = uni(lds_addr(lds + st * SB_U4));
    const bool more = kt < nk;
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
      const int blk = i * PW + p;
      dma16(dB, uni(base + blk * 1024), more ? voB : OOB, uni((uint32_t)(kt * BK + blk * B_ROWS) * ldbB));
    }
  }

  // ---------------------------------------------------------- consumer side
  struct AFrag { u32x4 v[2][FM]; };                  // [substep][fragment] of one slice
  struct BFrag { i16x4 bl[2][FN], bu[2][FN]; };

  __device__ __forceinline__ void load_a(int kt, AFrag& a) const {
    const bool more = kt < nk;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a.v[ks][i] = bload(rA, more ? voA : OOB, uni((((uint32_t)kt * 4u + wmA + (uint32_t)i) * 2u + (uint32_t)ks) * 1024u));
  }

  // byte offset of B fragment j's first transposing read in a stage
  __device__ __forceinline__ int frag_b(int j) const {
    const int lane = threadIdx.x & 63, w = wave() % CW;
    const int wn = w / WM;
    const int g = lane >> 4, Lg = lane & 15;
    const int brow = (g >> 1) * 8 + (Lg >> 2);
    const int u = 2 * (g & 1) + ((Lg & 3) >> 1);
    return brow * (BN * 2) + (4 * ((wn * FN + j) ^ (Lg >> 2)) + u) * 16 + (Lg & 1) * 8;
  }

  __device__ __forceinline__ void read_b(const u32x4* lds, int st, const int (&fb)[FN], BFrag& b) const {
    const char* pb = (const char*)(lds + st * SB_U4);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int base = fb[j] + ks * 16 * (BN * 2);
        b.bl[ks][j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pb + base));
        b.bu[ks][j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pb + base + 4 * (BN * 2)));
      }
  }

  __device__ __forceinline__ void mma(const AFrag& a, const BFrag& b) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const bf16x8 bop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(b.bl[ks][j], b.bu[ks][j], 0, 1, 2,
                                                                                3, 4, 5, 6, 7));
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v[ks][i]), bop,
                                                              acc[i][j], 0, 0, 0);
        }
  }

  // Full K loop.  Every wave runs the same number of barriers (one before the
  // loop, one per slice, one at the end).
  __device__ __forceinline__ void run(Smem1 m) {
    const u32x4* lds = m.lds;
    zero_acc();
    if (nk == 0) return;
    const int w = wave();
    if (w >= CW) {                                   // producer
      const int p = w - CW;
#pragma unroll 1
      for (int s = 0; s < STAGES; ++s) produce(lds, s, s, p);
      wait_barrier<(STAGES - 1) * B_INS>();        // slice 0 landed
#pragma unroll 1
      for (int kt = 0; kt < nk; ++kt) {
        wait_barrier<(STAGES - 2) * B_INS>();      // slice kt+1 landed
        produce(lds, kt % STAGES, kt + STAGES, p);
      }
      wait_barrier<0>();                           // the zero-filling DMAs past the end, before LDS is reused
    } else {                                         // consumer
      int fb[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[j] = frag_b(j);
      AFrag a[PA];
#pragma unroll
      for (int s = 0; s < PA; ++s) load_a(s, a[s]);
      lds_barrier();                                 // slice 0 landed
      BFrag b0, b1;
      read_b(lds, 0, fb, b0);
#pragma unroll 1
      for (int kt = 0; kt < nk; kt += PA) {
#pragma unroll
        for (int s = 0; s < PA; s += 2) {
          step(lds, kt + s, fb, a[s], b0, b1);
          step(lds, kt + s + 1, fb, a[s + 1], b1, b0);
        }
      }
      lds_barrier();
    }
  }

  // Consumer slice kt: fragments of kt in a / cur; reads slice kt+1 into nxt
  // and reloads a with slice kt+PA.
  __device__ __forceinline__ void step(const u32x4* lds, int kt, const int (&fb)[FN], AFrag& a, BFrag& cur,
                                       BFrag& nxt) {
    lds_barrier();                                       // this wave's reads of slice kt returned; slice kt+1
                                                         // landed; stage kt % STAGES free
    read_b(lds, (kt + 1) % STAGES, fb, nxt);
    mma(a, cur);
    load_a(kt + PA, a);
  }
};

}  // namespace mk
