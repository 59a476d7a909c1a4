// MoE combine: the step after the grouped GEMM.
//
// [P1] "Los cinco núcleos fusionados", row "Envío MoE + GEMM" sends each
// token to the ranks of its experts; the way back is not described there.
// Here each token's k expert outputs -- local rows of the grouped-GEMM
// output, or rows the other ranks returned (resident buffers, one row per
// dispatch position) -- are weighted by a softmax over the token's k
// selected logits and summed in slot order:
//   out[t] = sum_j g[t, j] * Y_row(t, j),  g[t, :] = softmax(l[t, e_0..e_{k-1}])
// The step is HBM-bound (k rows of F read per token, one written), so it is
// two plain kernels: the inverse of the dispatch permutation (pair ->
// position), then one workgroup per token, each thread summing 8 columns of
// the token's k rows in fp32.
#include <string.h>

#include "mk_device.h"
#include "mk_host.h"

using namespace mk;

namespace {

constexpr int CT = 256;

__global__ void inv_perm_kernel(const int32_t* __restrict__ perm, int n, int32_t* __restrict__ pos) {
  for (int p = blockIdx.x * blockDim.x + threadIdx.x; p < n; p += gridDim.x * blockDim.x) {
    const int pair = perm[p];
    if ((unsigned)pair < (unsigned)n) pos[pair] = p;     // perm is a permutation of [0, n)
  }
}

__device__ __forceinline__ float bf_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// One workgroup per token; thread c sums columns 8c .. 8c+7 (and every CT-th
// group after them).  Rows are read through descriptors bounded to their
// buffers: a position outside them reads zero.
__global__ __launch_bounds__(CT) void combine_kernel(const float* __restrict__ logits, int E, int k,
                                                     const int32_t* __restrict__ topk, const int32_t* __restrict__ offsets,
                                                     int eb, int L, const int32_t* __restrict__ pos,
                                                     const uint16_t* Yl, uint32_t yl_rows, const uint16_t* Yp,
                                                     uint32_t yp_rows, int F, void* out, int o_bf16) {
  const int t = blockIdx.x, tid = threadIdx.x;
  const int lo = offsets[eb], hi = offsets[eb + L];
  // gate weights (every thread computes the token's k of them)
  float w[MK_MAX_TOPK];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < MK_MAX_TOPK; ++j) {
    w[j] = -INFINITY;
    if (j < k) {
      int e = topk[(int64_t)t * k + j];
      e = (unsigned)e < (unsigned)E ? e : 0;
      w[j] = logits[(int64_t)t * E + e];
      mx = fmaxf(mx, w[j]);
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < MK_MAX_TOPK; ++j) {
    w[j] = j < k ? __builtin_amdgcn_exp2f((w[j] - mx) * 1.44269504088896340736f) : 0.f;
    sum += w[j];
  }
  const float inv = 1.f / sum;
#pragma unroll
  for (int j = 0; j < MK_MAX_TOPK; ++j) w[j] *= inv;
  // the k source rows of this token
  const uint32_t row_bytes = (uint32_t)F * 2u;
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(Yl, yl_rows * row_bytes);
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(Yp, yp_rows * row_bytes);
  int p[MK_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MK_MAX_TOPK; ++j) p[j] = j < k ? pos[(int64_t)t * k + j] : 0;
  const int esz = o_bf16 ? 2 : 4;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc((char*)out + (int64_t)t * F * esz, (uint32_t)F * esz);
  for (int c = tid; c < F / 8; c += CT) {
    u32x4 v[MK_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MK_MAX_TOPK; ++j)
      if (j < k) {
        const bool local = p[j] >= lo && p[j] < hi;
        const uint32_t off = (uint32_t)c * 16u;
        v[j] = local ? bload(rl, (uint32_t)(p[j] - lo) * row_bytes + off, 0)
                     : bload(rp, (uint32_t)p[j] * row_bytes + off, 0);
      }
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < MK_MAX_TOPK; ++j)
      if (j < k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = __builtin_fmaf(w[j], bf_lo(v[j][i]), acc[2 * i]);
          acc[2 * i + 1] = __builtin_fmaf(w[j], bf_hi(v[j][i]), acc[2 * i + 1]);
        }
      }
    if (o_bf16) {
      const u32x2 a{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
      const u32x2 b{pack_bf16(acc[4], acc[5]), pack_bf16(acc[6], acc[7])};
      __builtin_amdgcn_raw_buffer_store_b64(a, ro, (uint32_t)c * 16u, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b64(b, ro, (uint32_t)c * 16u + 8u, 0, 0);
    } else {
      bstore_alu16(ro, (uint32_t)c * 32u, 0, f32x4{acc[0], acc[1], acc[2], acc[3]});
      bstore_alu16(ro, (uint32_t)c * 32u + 16u, 0, f32x4{acc[4], acc[5], acc[6], acc[7]});
    }
  }
}

}  // namespace

extern "C" size_t mk_moe_combine_workspace(int64_t T, int k) {
  if (T <= 0 || k <= 0) return 256;
  return ((size_t)T * (size_t)k * 4 + 255) & ~(size_t)255;
}

extern "C" int mk_moe_combine(const float* logits, int64_t T, int E, int k, const int32_t* topk_idx,
                              const int32_t* offsets, const int32_t* perm, int expert_begin, int L,
                              const void* y_local, int64_t y_local_rows, const void* y_peer, int64_t F,
                              void* out, int out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  using mkh::fail;
  if (!logits || !topk_idx || !offsets || !perm || !y_local || !y_peer || !out)
    return fail(MK_ERR_INVALID, "NULL input or output pointer");
  if (T < 1 || E < 1 || F < 8) return fail(MK_ERR_INVALID, "empty shape (T=%lld, E=%d, F=%lld)", (long long)T, E,
                                           (long long)F);
  if (E > MK_MAX_EXPERTS) return fail(MK_ERR_UNSUPPORTED, "E=%d outside [1,%d]", E, MK_MAX_EXPERTS);
  if (k < 1 || k > MK_MAX_TOPK || k > E) return fail(MK_ERR_INVALID, "k=%d outside [1,min(E,%d)]", k, MK_MAX_TOPK);
  if (L < 1 || expert_begin < 0 || expert_begin + L > E)
    return fail(MK_ERR_INVALID, "local experts [%d, %d) outside [0, %d)", expert_begin, expert_begin + L, E);
  if (F % 8) return fail(MK_ERR_UNSUPPORTED, "F=%lld must be a multiple of 8", (long long)F);
  if (y_local_rows < 0 || T > (1 << 24) || F > MK_MAX_COLS || T * k * F * 2 >= (1ll << 32) ||
      y_local_rows * F * 2 >= (1ll << 32))
    return fail(MK_ERR_UNSUPPORTED, "buffers too large");
  if (out_dtype != MK_BF16 && out_dtype != MK_F32) return fail(MK_ERR_INVALID, "out_dtype %d", out_dtype);
  if (!mkh::aligned16(y_local) || !mkh::aligned16(y_peer) || !mkh::aligned16(out))
    return fail(MK_ERR_INVALID, "y_local, y_peer and out must be 16-byte aligned");
  if (!workspace) return fail(MK_ERR_WORKSPACE, "workspace is NULL");
  if (workspace_bytes < mk_moe_combine_workspace(T, k))
    return fail(MK_ERR_WORKSPACE, "workspace %zu bytes < %zu", workspace_bytes, mk_moe_combine_workspace(T, k));
  hipStream_t st = (hipStream_t)stream;
  const int n = (int)(T * k);
  int32_t* pos = (int32_t*)workspace;
  hipLaunchKernelGGL(inv_perm_kernel, dim3((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024), dim3(256), 0, st, perm, n,
                     pos);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return mkh::hip_fail(e, "inverse permutation launch");
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)T), dim3(CT), 0, st, logits, E, k, topk_idx, offsets, expert_begin,
                     L, pos, (const uint16_t*)y_local, (uint32_t)y_local_rows, (const uint16_t*)y_peer, (uint32_t)n,
                     (int)F, out, out_dtype == MK_BF16 ? 1 : 0);
  if ((e = hipGetLastError()) != hipSuccess) return mkh::hip_fail(e, "combine launch");
  return MK_OK;
}
