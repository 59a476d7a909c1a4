// Device building blocks shared by the persistent fused kernels (gfx950).
//
//  * WsHeader / flag helpers: role tickets, work queues and per-unit arrival
//    counters live in the caller's workspace; producers publish with an
//    agent-scope release, consumers spin with relaxed loads and then take an
//    agent-scope acquire fence (gfx950 has one L2 per XCD, so cross-XCD
//    visibility needs exactly these fences).
//  * TileGemm: a bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulate) block
//    tile with a double-buffered, XOR-swizzled LDS stage per operand.  B is
//    row-major [K x N]; each 8x8 bf16 block of B is transposed in registers on
//    its way into LDS so that both MFMA operands are read as contiguous
//    16-byte k-runs (ds_read_b128).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Status codes stored in the workspace (positive; the host negates them).
enum : uint32_t { ST_OK = 0, ST_TIMEOUT = 5 };

// Fixed header at the start of every workspace (256 bytes).
struct WsHeader {
  uint32_t ticket;     // role tickets, handed out in workgroup start order
  uint32_t tile_next;  // compute tile queue head
  uint32_t copy_next;  // copy work queue head
  uint32_t done;       // workgroups that have finished
  uint32_t status;     // sticky ST_* code, cleared by the host
  uint32_t abort;      // set on watchdog expiry so every other wait gives up
  uint32_t red_next;   // reduce queue head
  uint32_t prod_next;  // produced-tile FIFO tail
  uint64_t t0;         // wall-clock ticks when the first copy workgroup started
  uint32_t aux[54];
};
static_assert(sizeof(WsHeader) == 256, "header size");

// ---------------------------------------------------------------- atomics
__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_release(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_relaxed(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_release(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ void fence_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }

// Publication of a workgroup's stores at agent scope with ONE release: every
// wave waits for its own stores to complete, the barrier orders them before
// thread 0, thread 0 takes the agent-scope release (on gfx950 it writes back
// the XCD's dirty L2 lines, so one per item instead of one per wave), and
// after the second barrier any thread may publish with relaxed atomics.
// Called by every thread of the workgroup.
__device__ __forceinline__ void wg_release() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) fence_release();
  __syncthreads();
}

// Constant-rate (100 MHz on MI300-class parts) wall clock shared by all CUs.
__device__ __forceinline__ uint64_t now_ticks() { return wall_clock64(); }

// Thread-0 helper: spin until *p >= target, with relaxed loads only (the
// caller takes one acquire fence after all its waits).  Polls back off to
// about 1 us apart: hundreds of workgroups polling a few flag lines every
// few cycles would take memory bandwidth from the copies they wait for.
// Returns false if the watchdog expired (status and abort are then set) or
// another wait already aborted.
__device__ inline bool wait_geq_relaxed(const uint32_t* p, uint32_t target, WsHeader* h,
                                        uint64_t limit_ticks) {
  if (ld_relaxed(p) >= target) return true;
  const uint64_t t_begin = now_ticks();
  for (uint32_t it = 0; ld_relaxed(p) < target; ++it) {
    if ((it & 15u) == 15u && ld_relaxed(&h->abort)) return false;
    if (now_ticks() - t_begin > limit_ticks) {
      st_relaxed(&h->status, ST_TIMEOUT);
      st_relaxed(&h->abort, 1u);
      return false;
    }
    if (it < 8) __builtin_amdgcn_s_sleep(4);
    else __builtin_amdgcn_s_sleep(32);
  }
  return true;
}

// As wait_geq_relaxed, for a wait that the whole grid may share (every
// workgroup polling one counter): polls about every 4 us, so hundreds of
// waiters do not load one memory channel that the work they wait for uses.
__device__ inline bool wait_geq_sparse(const uint32_t* p, uint32_t target, WsHeader* h, uint64_t limit_ticks) {
  if (ld_relaxed(p) >= target) return true;
  const uint64_t t_begin = now_ticks();
  for (uint32_t it = 0; ld_relaxed(p) < target; ++it) {
    if ((it & 3u) == 3u && ld_relaxed(&h->abort)) return false;
    if (now_ticks() - t_begin > limit_ticks) {
      st_relaxed(&h->status, ST_TIMEOUT);
      st_relaxed(&h->abort, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(127);
  }
  return true;
}

// As wait_geq_relaxed, then an agent-scope acquire.
__device__ inline bool wait_geq(const uint32_t* p, uint32_t target, WsHeader* h, uint64_t limit_ticks) {
  const bool ok = wait_geq_relaxed(p, target, h, limit_ticks);
  if (ok) fence_acquire();
  return ok;
}

// Thread-0 helper: wait until the wall clock reaches `deadline`, but never
// longer than `limit_ticks` (a corrupt deadline cannot stall the kernel).
__device__ inline void wait_until(uint64_t deadline, uint64_t limit_ticks) {
  const uint64_t t_begin = now_ticks();
  for (uint64_t t = t_begin; t < deadline && t - t_begin < limit_ticks; t = now_ticks())
    __builtin_amdgcn_s_sleep(8);
}

// Value of thread 0 broadcast to the workgroup (uses one LDS word).  The
// result is made wave-uniform (readfirstlane), so everything derived from it
// -- tile coordinates, buffer descriptors, loop exits -- lives in scalar
// registers and branches are uniform.
__device__ __forceinline__ uint32_t wg_bcast(uint32_t v, uint32_t* slot) {
  if (threadIdx.x == 0) *slot = v;
  __syncthreads();
  const uint32_t r = (uint32_t)__builtin_amdgcn_readfirstlane((int)*slot);
  __syncthreads();
  return r;
}

// Per-XCD work queues.  MI355X has 8 XCDs of 32 CUs, each with its own L2:
// tiles that share an operand block reuse it from L2 only when they run on
// the same XCD, so work is split into XQ queues, one per XCD, and a
// workgroup drains its own XCD's queue before it helps with the others.
constexpr int XQ = 8;
constexpr int XQ_AUX = 16;   // WsHeader::aux[XQ_AUX .. XQ_AUX + XQ) are the queue heads

// The XCD this wave runs on (hardware register XCC_ID, bits 3:0).
__device__ __forceinline__ int xcd_id() {
  return __builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11)) & (XQ - 1);
}

// Thread-0 state of one workgroup walking the queues: its home queue first,
// then the others in order; a drained queue is never visited again, so every
// workgroup stops after at most XQ failed takes.
struct XcdQueues {
  uint32_t* head;
  int home, visited;
  __device__ explicit XcdQueues(uint32_t* heads) : head(heads), home(xcd_id()), visited(0) {}
  // Next item: true with its queue x and index j, or false once every queue
  // is drained.  len(x) is the length of queue x.
  template <class Len>
  __device__ bool take(Len len, int& x, uint32_t& j) {
    while (visited < XQ) {
      x = (home + visited) & (XQ - 1);
      j = __hip_atomic_fetch_add(&head[x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (j < len(x)) return true;
      ++visited;
    }
    return false;
  }
};

// Transpose the 4x4 blocks held by each quad of lanes: on entry lane j of a
// quad holds v[k] = element (row k, column j) of the block, on exit (row j,
// column k).  Two butterfly stages over DPP quad permutations (lane ^ 1, then
// lane ^ 2); in each, the lane with the bit clear sends element k|m and keeps
// element k, its partner sends k and keeps k|m.
__device__ __forceinline__ float dpp_xor1(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_xor2(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));
}
__device__ __forceinline__ f32x4 quad_transpose(f32x4 v) {
  const bool b0 = threadIdx.x & 1, b1 = threadIdx.x & 2;
#pragma unroll
  for (int k = 0; k < 4; k += 2) {                    // stage 1: pairs (k, k+1) across lane ^ 1
    const float r = dpp_xor1(b0 ? v[k] : v[k + 1]);
    if (b0) v[k] = r;
    else v[k + 1] = r;
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {                       // stage 2: pairs (k, k+2) across lane ^ 2
    const float r = dpp_xor2(b1 ? v[k] : v[k + 2]);
    if (b1) v[k] = r;
    else v[k + 2] = r;
  }
  return v;
}

// fp32 -> bf16 bits, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f2bf(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

// --------------------------------------------------------------- LDS layout
// An operand stage holds ROWS rows of 64 bf16 = 8 chunks of 16 bytes.  Chunk c
// of row n sits at 16-byte unit 9*n + n/8 + c: the one-chunk pad per row makes
// eight consecutive rows read at the same chunk hit distinct bank groups
// (MFMA fragment reads), and the extra unit every 8 rows does the same for
// rows 8 apart (the transposed B writes).  Every offset is affine in the loop
// indices, so the compiler folds them into instruction immediates.
__host__ __device__ constexpr uint32_t lds_units(uint32_t rows) { return rows * 9 + rows / 8; }
__device__ __forceinline__ uint32_t lofs(uint32_t n, uint32_t c) { return n * 9 + (n >> 3) + c; }

// Raw buffer resource over [p, p + bytes); loads at or past `bytes` return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// POLICY is the instruction's cache-policy field: 0 default, 16 = sc1 (a
// device-coherent load: it sees what other XCDs wrote through their L2).
template <int POLICY = 0>
__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, POLICY);
}
// A store past the descriptor's range is dropped by the hardware.  POLICY is
// the instruction's cache-policy field: 0 default (write-back L2), 16 = sc1
// (written through the L2 at device scope).
template <int POLICY = 0>
__device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, POLICY);
}
constexpr uint32_t OOB = 0x80000000u;   // a voffset that is always past the end

// Store 16 bytes of values just computed by vector ALU instructions, as two
// 8-byte stores.  A 16-byte buffer store can read its data registers late
// enough that the next ALU instruction has already overwritten them: seen on
// gfx950 with two waves per SIMD, where the first dword of some lanes' stores
// took the following value.  The compiler inserts no wait there, and stores
// of at most 8 bytes are outside that hazard.  Copies (data straight from
// loads, not rewritten by ALU instructions) keep 16-byte stores.
template <int POLICY = 0>
__device__ __forceinline__ void bstore_alu16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, f32x4 v) {
  const u32x4 u = __builtin_bit_cast(u32x4, v);
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{u[0], u[1]}, r, voff, soff, POLICY);
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{u[2], u[3]}, r, voff, soff + 8u, POLICY);
}

// Copy n16 16-byte chunks from src to dst (buffer resources bounded to the
// block: past the end loads return zero and stores are dropped, so the loop
// has no per-element guard -- a guarded store would be its own branch, and
// the compiler would wait for every earlier memory operation before each
// one).  Each thread keeps COPY_UNROLL loads in flight (64 KiB per 256-thread
// workgroup).  POLICY is the stores' cache-policy field (16 = written through
// the L2).
constexpr int COPY_UNROLL = 16;
template <int POLICY>
__device__ __forceinline__ void copy_block(__amdgpu_buffer_rsrc_t src, __amdgpu_buffer_rsrc_t dst, int n16, int tid,
                                           int nt) {
  for (int base = 0; base < n16; base += nt * COPY_UNROLL) {
    u32x4 v[COPY_UNROLL];
#pragma unroll
    for (int u = 0; u < COPY_UNROLL; ++u) v[u] = bload(src, (uint32_t)(base + u * nt + tid) * 16u, 0);
#pragma unroll
    for (int u = 0; u < COPY_UNROLL; ++u) bstore<POLICY>(dst, (uint32_t)(base + u * nt + tid) * 16u, 0, v[u]);
  }
}

// Values the caller knows to be the same in every lane, moved to scalar
// registers (buffer descriptors must live there).  The builtin works on int:
// each 32-bit half is taken back as uint32_t before widening, so a low half
// with bit 31 set is not sign-extended into the high half of a pointer.
__device__ __forceinline__ uint32_t uni(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
template <class T>
__device__ __forceinline__ const T* uni(const T* p) {
  const uint64_t v = (uint64_t)p;
  const uint64_t lo = uni((uint32_t)v);
  const uint64_t hi = uni((uint32_t)(v >> 32));
  return (const T*)(lo | (hi << 32));
}

// ------------------------------------------------------------ block tile GEMM
// BM x BN output tile per workgroup, WM x WN waves, each wave owning a
// (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA blocks; K advances 64 at a
// time.  Rows past `mrows`, columns past `ncols` and k past K read as zero,
// so ragged edges need no special path (K and N are multiples of 8).
// LDS handed to a tile engine: one array (register-staged engine) or four
// stages of A and B as separate objects (direct-to-LDS engine).
struct Smem1 { u32x4* lds; };
struct Smem4 { u32x4* a[4]; u32x4* b[4]; };

// GA (gathered A): tile row r is A row idx[r] / div for an index array idx
// given at bind time (bind_rows); each A load then has its own row offset.
template <int BM_, int BN_, int WM_, int WN_, bool GA = false>
struct TileGemm {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = 64, STAGES = 2;
  static __host__ __device__ constexpr bool supports_k(int) { return true; }
  static constexpr int NT = 64 * WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int A_CH = BM * 8;        // 16-byte chunks per A stage
  static constexpr int A_PT = (A_CH + NT - 1) / NT;
  static constexpr int B_NB = BN / 8;        // 8-column groups
  static constexpr int B_BL = 8 * B_NB;      // 8x8 blocks per B stage
  static constexpr int B_PT = (B_BL + NT - 1) / NT;
  static constexpr int SA = lds_units(BM), SB = lds_units(BN);   // 16-byte units per stage
  static constexpr int LDS_U4 = 2 * (SA + SB);
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 blocks");
  static_assert(NT % 64 == 0 && NT % B_NB == 0, "thread/operand mapping");

  u32x4 ra[A_PT];
  u32x4 rb[B_PT][8];
  f32x16 acc[FM][FN];
  __amdgpu_buffer_rsrc_t rsA, rsB;
  uint32_t voA, voB, ldaB, ldbB;   // per-thread byte offsets; row pitches in bytes
  uint32_t voG[GA ? A_PT : 1];     // gathered A: per-load row offsets
  int K, ncols;

  __device__ __forceinline__ void zero_acc() {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }

  // Bind the operands of one output tile: A at its first row (mrows valid
  // rows), B at its first column (ncols valid columns), B_end = one past the
  // last element of B.
  __device__ __forceinline__ void bind(const uint16_t* A, int64_t lda, int mrows,
                                       const uint16_t* B, int64_t ldb, int ncols_, const uint16_t* B_end,
                                       int K_) {
    // Every argument is uniform across the workgroup.
    const int tid = threadIdx.x;
    K = uni(K_);
    ncols = uni(ncols_);
    ldaB = uni((uint32_t)(lda * 2));
    ldbB = uni((uint32_t)(ldb * 2));
    const int rows = mrows < BM ? mrows : BM;
    rsA = make_rsrc(uni(A), uni((uint32_t)(rows > 0 ? rows : 0) * ldaB));
    rsB = make_rsrc(uni(B), uni((uint32_t)((B_end - B) * 2)));
    voA = (uint32_t)(tid >> 3) * ldaB + (uint32_t)(tid & 7) * 16u;
    const int kb = tid / B_NB, nb = tid % B_NB;
    voB = (nb * 8 < ncols) ? (uint32_t)(kb * 8) * ldbB + (uint32_t)nb * 16u : OOB;
  }

  // Gathered A (GA): tile row r (r < mrows) is row idx[r] / div of A, which
  // has a_rows rows of lda elements, starting at column k0; rows past mrows
  // or whose index falls outside [0, a_rows) read as zero.  a_rows * lda * 2
  // must stay below 2^31 bytes, the out-of-range offset OOB.
  __device__ __forceinline__ void bind_rows(const uint16_t* A, int64_t lda, int a_rows, const int32_t* idx,
                                            int div, int mrows, int k0, const uint16_t* B, int64_t ldb,
                                            int ncols_, const uint16_t* B_end, int K_) {
    static_assert(GA, "gathered-A engine");
    bind(A, lda, 0, B, ldb, ncols_, B_end, K_);
    rsA = make_rsrc(uni(A), uni((uint32_t)a_rows * ldaB));
    const int tid = threadIdx.x;
    const int rows = mrows < BM ? mrows : BM;
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
      const int r = (tid >> 3) + i * (NT / 8);
      const int t = r < rows ? idx[r] / div : -1;
      voG[i] = (uint32_t)t < (uint32_t)a_rows ? (uint32_t)t * ldaB + (uint32_t)(tid & 7) * 16u + (uint32_t)k0 * 2u
                                              : OOB;
    }
  }

  // Global -> registers for the K-step starting at k0.
  __device__ __forceinline__ void load(int k0) {
    const int tid = threadIdx.x;
    const bool kin = k0 + (tid & 7) * 8 < K;
#pragma unroll
    for (int i = 0; i < A_PT; ++i)
      if (A_CH % NT == 0 || tid + i * NT < A_CH) {
        if constexpr (GA) ra[i] = bload(rsA, kin ? voG[i] : OOB, (uint32_t)k0 * 2u);
        else ra[i] = bload(rsA, kin ? voA : OOB, (uint32_t)(i * (NT / 8)) * ldaB + (uint32_t)k0 * 2u);
      }
#pragma unroll
    for (int i = 0; i < B_PT; ++i)
      if (B_BL % NT == 0 || tid + i * NT < B_BL) {
#pragma unroll
        for (int rr = 0; rr < 8; ++rr)
          rb[i][rr] = bload(rsB, voB, (uint32_t)(k0 + i * (NT / B_NB) * 8 + rr) * ldbB);
      }
  }

  // Registers -> LDS stage; B blocks are transposed to [n][k].
  __device__ __forceinline__ void store(u32x4* __restrict__ lds, int stage) {
    const int tid = threadIdx.x;
    u32x4* sa = lds + stage * (SA + SB);
    u32x4* sb = sa + SA;
    const uint32_t ra0 = lofs(tid >> 3, tid & 7);
#pragma unroll
    for (int i = 0; i < A_PT; ++i)
      if (A_CH % NT == 0 || tid + i * NT < A_CH) sa[ra0 + i * lds_units(NT / 8)] = ra[i];
    const uint32_t kb0 = tid / B_NB, nb = tid % B_NB;
#pragma unroll
    for (int i = 0; i < B_PT; ++i)
      if (B_BL % NT == 0 || tid + i * NT < B_BL) {
        const uint32_t base = nb * 73 + kb0 + i * (NT / B_NB);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          u32x4 col;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const uint32_t lo = rb[i][2 * m][j >> 1], hi = rb[i][2 * m + 1][j >> 1];
            col[m] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
          }
          sb[base + j * 9] = col;
        }
      }
  }

  // Operand fragments of k-substep ks (16 deep) from one LDS stage.
  __device__ __forceinline__ void frags(const u32x4* __restrict__ sa, const u32x4* __restrict__ sb,
                                        int ks, bf16x8 (&af)[FM], bf16x8 (&bfr)[FN]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w % WM, wn = w / WM;
    const uint32_t ba = lofs(wm * TM + (lane & 31), lane >> 5) + ks * 2;
    const uint32_t bb = lofs(wn * TN + (lane & 31), lane >> 5) + ks * 2;
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i] = __builtin_bit_cast(bf16x8, sa[ba + i * lds_units(32)]);
#pragma unroll
    for (int j = 0; j < FN; ++j) bfr[j] = __builtin_bit_cast(bf16x8, sb[bb + j * lds_units(32)]);
  }

  // 64-deep MFMA update from one LDS stage; the fragments of substep ks+1 are
  // read while the MFMAs of substep ks run.
  __device__ __forceinline__ void mma(const u32x4* __restrict__ lds, int stage) {
    const u32x4* sa = lds + stage * (SA + SB);
    const u32x4* sb = sa + SA;
    bf16x8 af[2][FM], bfr[2][FN];
    frags(sa, sb, 0, af[0], bfr[0]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int cur = ks & 1;
      if (ks < 3) frags(sa, sb, ks + 1, af[cur ^ 1], bfr[cur ^ 1]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j], acc[i][j], 0, 0, 0);
    }
  }

  // Full K loop for the bound tile.  Ends with a barrier so LDS may be reused.
  __device__ __forceinline__ void run(Smem1 m) {
    u32x4* __restrict__ lds = m.lds;
    zero_acc();
    const int nk = (K + BK - 1) / BK;
    load(0);
    store(lds, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const bool more = kt + 1 < nk;
      if (more) load((kt + 1) * BK);
      mma(lds, kt & 1);
      if (more) store(lds, (kt + 1) & 1);
      __syncthreads();
    }
  }

  // Visit every accumulator element: f(row_in_tile, col_in_tile, value).
  // MFMA 32x32 output layout: lane l, register r holds
  //   row = 8*(r/4) + 4*(l/32) + r%4,  col = l%32  (within its 32x32 block).
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

// Store an accumulator tile (either engine: acc[FM][FN], waves WM x WN) to a
// row-major C at the tile's origin: ld elements per row, the first `rows` x
// `cols` valid, fp32 or bf16 (round to nearest even).  Each lane's 4x4 blocks
// are transposed across its quad of lanes so a lane holds 4 consecutive
// columns of one row, then stored as one 16-byte (fp32) or 8-byte (bf16)
// access through a descriptor bounded to the valid rows; a 4-column run past
// `cols` gets the out-of-range offset.  No store is guarded, so none waits
// for the ones before it.  cols is a multiple of 4 and rows*ld*esize < 2^32.
// POLICY is the stores' cache-policy field: 16 (sc1) writes the tile through
// the XCD's L2, so it leaves no dirty lines there for a later release fence
// (a copy workgroup's publication) to write back.
template <class G, int POLICY = 0>
__device__ __forceinline__ void store_tile(const G& g, void* C, int64_t ld, int rows, int cols, bool bf16) {
  const int lane = threadIdx.x & 63, w = uni((int)(threadIdx.x >> 6));
  if (w >= G::WM * G::WN) return;                   // waves that hold no accumulators (producers)
  const int wm = w % G::WM, wn = w / G::WM;
  const uint32_t esz = bf16 ? 2u : 4u;
  const uint32_t rbo = uni((uint32_t)ld * esz);
  rows = rows < G::BM ? rows : G::BM;
  const __amdgpu_buffer_rsrc_t d = make_rsrc(uni(C), uni((uint32_t)(rows > 0 ? rows : 0) * rbo));
  const int lrow = (lane >> 5) * 4 + (lane & 3), lcol = (lane & 31) & ~3;
  const uint32_t lout = (uint32_t)lrow * rbo + (uint32_t)lcol * esz;
#pragma unroll
  for (int i = 0; i < G::FM; ++i) {
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
      const int cb = wn * G::TN + j * 32;                  // first column of the block
      const uint32_t vo = cb + lcol < cols ? lout : OOB;
      const int rb = wm * G::TM + i * 32;                  // first row of the block
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const f32x4 v = quad_transpose(f32x4{g.acc[i][j][4 * gq], g.acc[i][j][4 * gq + 1], g.acc[i][j][4 * gq + 2],
                                             g.acc[i][j][4 * gq + 3]});
        const uint32_t so = uni((uint32_t)(rb + 8 * gq) * rbo + (uint32_t)cb * esz);
        if (bf16) {
          u32x2 b;
          b[0] = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
          b[1] = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
          __builtin_amdgcn_raw_buffer_store_b64(b, d, vo, so, POLICY);
        } else {
          bstore_alu16<POLICY>(d, vo, so, v);
        }
      }
    }
  }
}

// K parts of one tile (a tile split along K): each part parks its fp32
// accumulators in its slot, in register order (chunk c of 4 floats of thread
// t at byte 16*(c*NT + t)), written through the L2; the part that finishes
// last reads every slot back with device-coherent loads and sums them in part
// order, so the bits do not depend on which part finished last.
template <class G>
__device__ __forceinline__ void park_acc(const G& g, float* slot) {
  constexpr int NCH = G::FM * G::FN * 4;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(uni(slot), (uint32_t)(NCH * G::NT * 16));
  const uint32_t vo = threadIdx.x * 16u;
#pragma unroll
  for (int i = 0; i < G::FM; ++i)
#pragma unroll
    for (int j = 0; j < G::FN; ++j)
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const int c = (i * G::FN + j) * 4 + c4;
        const f32x16& a = g.acc[i][j];
        bstore_alu16(rs, vo, (uint32_t)(c * G::NT * 16),
                     f32x4{a[4 * c4], a[4 * c4 + 1], a[4 * c4 + 2], a[4 * c4 + 3]});
      }
}

// The finishing part's output: for each 4x4 piece, the PARTS slots' values
// are summed in part order, then transposed and stored like store_tile (the
// accumulators themselves are left alone).
template <class G, int PARTS>
__device__ __forceinline__ void store_parked_sum(const float* slots, void* C, int64_t ld, int rows, int cols,
                                                 bool bf16) {
  constexpr int NCH = G::FM * G::FN * 4;
  const int lane = threadIdx.x & 63, w = uni((int)(threadIdx.x >> 6));
  const int wm = w % G::WM, wn = w / G::WM;
  const uint32_t vin = threadIdx.x * 16u;
  const uint32_t esz = bf16 ? 2u : 4u;
  const uint32_t rbo = uni((uint32_t)ld * esz);
  rows = rows < G::BM ? rows : G::BM;
  const __amdgpu_buffer_rsrc_t d = make_rsrc(uni(C), uni((uint32_t)(rows > 0 ? rows : 0) * rbo));
  const int lrow = (lane >> 5) * 4 + (lane & 3), lcol = (lane & 31) & ~3;
  const uint32_t lout = (uint32_t)lrow * rbo + (uint32_t)lcol * esz;
#pragma unroll
  for (int i = 0; i < G::FM; ++i) {
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
      u32x4 t[PARTS][4];
#pragma unroll
      for (int k = 0; k < PARTS; ++k) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(uni(slots + (int64_t)k * (G::BM * G::BN)), (uint32_t)(NCH * G::NT * 16));
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) t[k][gq] = bload<16>(rs, vin, (uint32_t)(((i * G::FN + j) * 4 + gq) * G::NT * 16));
      }
      const int cb = wn * G::TN + j * 32, rb = wm * G::TM + i * 32;
      const uint32_t vo = cb + lcol < cols ? lout : OOB;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        f32x4 v = __builtin_bit_cast(f32x4, t[0][gq]);
#pragma unroll
        for (int k = 1; k < PARTS; ++k) v += __builtin_bit_cast(f32x4, t[k][gq]);
        v = quad_transpose(v);
        const uint32_t so = uni((uint32_t)(rb + 8 * gq) * rbo + (uint32_t)cb * esz);
        if (bf16) {
          u32x2 b;
          b[0] = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
          b[1] = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
          __builtin_amdgcn_raw_buffer_store_b64(b, d, vo, so, 0);
        } else {
          bstore_alu16(d, vo, so, v);
        }
      }
    }
  }
}

}  // namespace mk
