// Measurement kernels: the rates the fused kernels are compared with, taken
// on the device itself (not part of any operation).
//
//  * mfma_peak_kernel: every wave of a full grid (two 256-thread workgroups
//    per CU, so two waves per SIMD) runs a loop of independent bf16
//    v_mfma_f32_32x32x16_bf16 updates on register operands that change from
//    one MFMA to the next (random bits, as in a GEMM on real data): no memory
//    traffic, no LDS, only the matrix pipeline.  Each wave records how many
//    shader-clock and wall-clock ticks its loop took, so the average engine
//    clock under a full MFMA load follows.
//  * hbm_read_kernel / hbm_copy_kernel: each workgroup streams one contiguous
//    region with 16-byte buffer loads (16 in flight per thread), the copy
//    writing it back elsewhere; the read folds what it loads into a value
//    stored only if it equals a constant no input produces here, so the loads
//    stay and nothing is written.
#include "mk_device.h"
#include "mk_host.h"

using namespace mk;

namespace {

constexpr int PEAK_WG_PER_CU = 2;
constexpr int PEAK_NT = 256;
constexpr int PEAK_CHAINS = 8;       // independent accumulators per wave

// Operand bits from a 32-bit integer hash (lowbias32, Chris Wellons' published
// constants): bf16 values with a random sign and mantissa and exponents
// spread over [2^-4, 2^4), so every MFMA multiplies fresh, fully switching
// operands as a GEMM on real data does (constant operands draw less power and
// run at a higher clock).
__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352du;
  x ^= x >> 15; x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}
__device__ __forceinline__ bf16x8 random_frag(uint32_t seed) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t h = hash32(seed * 8u + (uint32_t)i);
    const uint16_t bits = (uint16_t)((h & 0x807fu) | ((123u + ((h >> 8) & 7u)) << 7));
    v[i] = __builtin_bit_cast(__bf16, bits);
  }
  return v;
}

constexpr int PEAK_FRAGS = 8;        // distinct A and B fragments per lane, rotated through

__global__ __launch_bounds__(PEAK_NT) void mfma_peak_kernel(int iters, uint64_t* clocks, float* sink) {
  const uint32_t gid = blockIdx.x * PEAK_NT + threadIdx.x;
  const int lane = threadIdx.x & 63;
  bf16x8 a[PEAK_FRAGS], b[PEAK_FRAGS];
#pragma unroll
  for (int f = 0; f < PEAK_FRAGS; ++f) {
    a[f] = random_frag(gid * 2u * PEAK_FRAGS + 2u * f);
    b[f] = random_frag(gid * 2u * PEAK_FRAGS + 2u * f + 1u);
  }
  f32x16 acc[PEAK_CHAINS];
#pragma unroll
  for (int j = 0; j < PEAK_CHAINS; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  const uint64_t c0 = clock64(), w0 = wall_clock64();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < PEAK_CHAINS; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j % PEAK_FRAGS], b[(j * 3 + 1) % PEAK_FRAGS], acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < PEAK_CHAINS; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j + 4) % PEAK_FRAGS], b[(j * 5 + 2) % PEAK_FRAGS], acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < PEAK_CHAINS; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  const uint64_t c1 = clock64(), w1 = wall_clock64();
  const int wave = (blockIdx.x * PEAK_NT + threadIdx.x) >> 6;
  if (lane == 0) {
    clocks[2 * wave] = c1 - c0;
    clocks[2 * wave + 1] = w1 - w0;
  }
  if (s == 1234567.f) sink[0] = s;   // keeps the loop; never true for these operands
}

constexpr int STREAM_UNROLL = 16;

__global__ __launch_bounds__(PEAK_NT) void hbm_read_kernel(const uint8_t* src, uint64_t bytes_per_wg, float* sink) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(uni(src + blockIdx.x * bytes_per_wg), (uint32_t)bytes_per_wg);
  const uint32_t n16 = (uint32_t)(bytes_per_wg / 16);
  u32x4 x = {0u, 0u, 0u, 0u};
  for (uint32_t base = 0; base < n16; base += PEAK_NT * STREAM_UNROLL) {
    u32x4 v[STREAM_UNROLL];
#pragma unroll
    for (int u = 0; u < STREAM_UNROLL; ++u) v[u] = bload(r, (base + u * PEAK_NT + threadIdx.x) * 16u, 0);
#pragma unroll
    for (int u = 0; u < STREAM_UNROLL; ++u) x ^= v[u];
  }
  if ((x[0] ^ x[1] ^ x[2] ^ x[3]) == 0x9e3779b9u) sink[0] = 1.f;
}

__global__ __launch_bounds__(PEAK_NT) void hbm_copy_kernel(const uint8_t* src, uint8_t* dst, uint64_t bytes_per_wg) {
  const __amdgpu_buffer_rsrc_t s = make_rsrc(uni(src + blockIdx.x * bytes_per_wg), (uint32_t)bytes_per_wg);
  const __amdgpu_buffer_rsrc_t d = make_rsrc(uni(dst + blockIdx.x * bytes_per_wg), (uint32_t)bytes_per_wg);
  copy_block<0>(s, d, (int)(bytes_per_wg / 16), threadIdx.x, PEAK_NT);
}

}  // namespace

extern "C" size_t mk_peak_workspace(void) {
  const mkh::DevInfo* d = mkh::dev_info();
  const int waves = (d ? d->n_cu : 256) * PEAK_WG_PER_CU * (PEAK_NT / 64);
  return 256 + (size_t)waves * 16;
}

extern "C" int mk_peak_mfma(int iters, void* workspace, size_t workspace_bytes, double* flops, int* waves,
                            void* stream) {
  using mkh::fail;
  if (iters < 1 || iters > (1 << 24)) return fail(MK_ERR_INVALID, "iters %d outside [1, 2^24]", iters);
  if (!workspace || !mkh::aligned16(workspace)) return fail(MK_ERR_WORKSPACE, "workspace NULL or misaligned");
  if (!flops || !waves) return fail(MK_ERR_INVALID, "flops and waves must be non-NULL");
  const mkh::DevInfo* d = mkh::dev_info();
  if (!d) return MK_ERR_HIP;
  const int grid = d->n_cu * PEAK_WG_PER_CU;
  const int nw = grid * (PEAK_NT / 64);
  if (workspace_bytes < 256 + (size_t)nw * 16) return fail(MK_ERR_WORKSPACE, "workspace %zu bytes too small", workspace_bytes);
  float* sink = (float*)workspace;
  uint64_t* clocks = (uint64_t*)((char*)workspace + 256);
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(grid), dim3(PEAK_NT), 0, (hipStream_t)stream, iters, clocks, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return mkh::hip_fail(e, "mfma peak kernel launch");
  *flops = (double)nw * iters * 2 * PEAK_CHAINS * (2.0 * 32 * 32 * 16);
  *waves = nw;
  return MK_OK;
}

extern "C" int mk_peak_hbm(const void* src, void* dst, size_t bytes, int mode, void* workspace, size_t workspace_bytes,
                           double* bytes_moved, void* stream) {
  using mkh::fail;
  if (!src || !mkh::aligned16(src) || (mode == 1 && (!dst || !mkh::aligned16(dst))))
    return fail(MK_ERR_INVALID, "src/dst NULL or misaligned");
  if (mode != 0 && mode != 1) return fail(MK_ERR_INVALID, "mode %d", mode);
  if (!bytes_moved) return fail(MK_ERR_INVALID, "bytes_moved must be non-NULL");
  if (!workspace || workspace_bytes < 256) return fail(MK_ERR_WORKSPACE, "workspace NULL or too small");
  const mkh::DevInfo* d = mkh::dev_info();
  if (!d) return MK_ERR_HIP;
  const int grid = d->n_cu * PEAK_WG_PER_CU;
  const uint64_t per = (uint64_t)(bytes / grid) & ~(uint64_t)((PEAK_NT * STREAM_UNROLL * 16) - 1);
  if (per == 0 || per >= (1ull << 31)) return fail(MK_ERR_INVALID, "bytes %zu: each of %d workgroups needs a region of 64 KiB to 2 GiB", bytes, grid);
  if (mode == 0)
    hipLaunchKernelGGL(hbm_read_kernel, dim3(grid), dim3(PEAK_NT), 0, (hipStream_t)stream, (const uint8_t*)src, per,
                       (float*)workspace);
  else
    hipLaunchKernelGGL(hbm_copy_kernel, dim3(grid), dim3(PEAK_NT), 0, (hipStream_t)stream, (const uint8_t*)src,
                       (uint8_t*)dst, per);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return mkh::hip_fail(e, "stream kernel launch");
  *bytes_moved = (double)per * grid * (mode == 1 ? 2.0 : 1.0);
  return MK_OK;
}
