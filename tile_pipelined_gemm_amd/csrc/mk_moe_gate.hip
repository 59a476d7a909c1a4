// MoE gate GEMM: logits = X @ W_gate (bf16 in, fp32 accumulate, fp32 out).
//
// The step before [P1] "Los cinco núcleos fusionados", row Envío MoE + GEMM:
// routing ranks one logit per (token, expert), and the gate produces them as a
// linear map of each token's hidden state.  At the MoE shape (T = 4096 tokens,
// H = 7168, E = 256 experts) the output is only 32 x 2 tiles of 128 x 128, so
// the 7168-deep contraction is cut into kp parts to give every CU work: each
// part parks its fp32 sums in the workspace, and the part that finishes last
// adds the kp parks in part order and stores the tile (the order is fixed, so
// the bits do not depend on which part finishes last).  No part waits for
// another, so the grid need not be co-resident.
#include <string.h>

#include <algorithm>

#include "mk_device.h"
#include "mk_gemm_dma.h"
#include "mk_host.h"

using namespace mk;

namespace {

struct GateParams {
  const uint16_t* X;
  const uint16_t* W;
  float* out;
  float* slots;       // [n_tiles][kp][BM*BN] parked parts
  uint32_t* cnt;      // [n_tiles] parts finished (restored to 0 by the last)
  int T, H, E, tiles_n, n_tiles, kp;
};

template <class G, int KP>
__device__ __forceinline__ void gate_finish(const GateParams& p, const G& g, int t, int part, int m0, int n0,
                                            uint32_t* sb) {
  float* const C = p.out + (int64_t)m0 * p.E + n0;
  if constexpr (KP == 1) {
    store_tile(g, C, p.E, p.T - m0, p.E - n0, false);
  } else {
    float* slots = p.slots + (int64_t)t * KP * (G::BM * G::BN);
    park_acc(g, slots + (int64_t)part * (G::BM * G::BN));
    wg_release();                                   // the part's parked sums, before it is counted
    uint32_t last = 0;
    if (threadIdx.x == 0) {
      last = add_relaxed(&p.cnt[t], 1u) == (uint32_t)(KP - 1);
      if (last) fence_acquire();                    // the other parts' parks
    }
    last = wg_bcast(last, sb);
    if (last) {
      store_parked_sum<G, KP>(slots, C, p.E, p.T - m0, p.E - n0, false);
      if (threadIdx.x == 0) st_relaxed(&p.cnt[t], 0u);   // every part has counted: ready for the next call
    }
  }
}

template <class G, int KP, class SM>
__device__ __forceinline__ void gate_body(const GateParams& p, SM sm, uint32_t* sb) {
  // Workgroups are dispatched to the 8 XCDs in turn (i to XCD i mod 8): with
  // the tile row fastest-varying, both column tiles and every part of a tile
  // row run on one XCD, so its rows of X are fetched into one L2 and shared.
  // (Only the speed depends on this; any mapping gives the same bits.)
  const int item = blockIdx.x;
  const int tiles_m = p.n_tiles / p.tiles_n;
  const int tm = item % tiles_m, tn = (item / tiles_m) % p.tiles_n, part = item / p.n_tiles;
  const int t = tm * p.tiles_n + tn;
  const int m0 = tm * G::BM, n0 = tn * G::BN;
  const int kpart = p.H / KP, k0 = part * kpart;
  G g;
  g.bind(p.X + (int64_t)m0 * p.H + k0, p.H, p.T - m0, p.W + (int64_t)k0 * p.E + n0, p.E, p.E - n0,
         p.W + (int64_t)p.H * p.E, kpart);
  g.run(sm);
  gate_finish<G, KP>(p, g, t, part, m0, n0, sb);
}

template <class G, int KP>
__global__ __launch_bounds__(G::NT) void gate_kernel(const GateParams p) {
  __shared__ uint32_t sb[2];
  if constexpr (G::STAGES == 4) {
    __shared__ u32x4 a0[G::SA_U4], a1[G::SA_U4], a2[G::SA_U4], a3[G::SA_U4];
    __shared__ u32x4 b0[G::SB_U4], b1[G::SB_U4], b2[G::SB_U4], b3[G::SB_U4];
    gate_body<G, KP>(p, Smem4{{a0, a1, a2, a3}, {b0, b1, b2, b3}}, sb);
  } else {
    __shared__ u32x4 lds[G::LDS_U4];
    gate_body<G, KP>(p, Smem1{lds}, sb);
  }
}

constexpr int GBM = 128, GBN = 128, KP_MAX = 8;
using GateD = TileGemmD<128, 128>;            // direct-to-LDS engine (K part % 128 == 0)
using GateR = TileGemm<128, 128, 2, 2>;       // register-staged engine (any K multiple of 8)

// Parts per tile: the smallest power of two (<= KP_MAX) that gives every CU
// an item, dividing H into 128-deep units; 1 where H is not a multiple of 128.
inline int gate_parts(int64_t T, int64_t H, int E, int n_cu) {
  if (H % 128) return 1;
  const int64_t tiles = ((T + GBM - 1) / GBM) * ((E + GBN - 1) / GBN);
  int kp = 1;
  while (kp < KP_MAX && tiles * kp < n_cu && (H / 128) % (2 * kp) == 0) kp *= 2;
  return kp;
}

struct GateWs { size_t cnt, slots, total; };
inline GateWs gate_ws_layout(int64_t T, int64_t H, int E, int n_cu) {
  GateWs w;
  const int64_t tiles = ((T + GBM - 1) / GBM) * ((E + GBN - 1) / GBN);
  const int kp = gate_parts(T, H, E, n_cu);
  w.cnt = 0;
  w.slots = ((size_t)tiles * 4 + 255) & ~(size_t)255;
  w.total = w.slots + (kp > 1 ? (size_t)tiles * kp * GBM * GBN * 4 : 0);
  return w;
}

template <class G, int KP>
int launch_gate(const GateParams& p, hipStream_t st) {
  hipLaunchKernelGGL((gate_kernel<G, KP>), dim3(p.n_tiles * KP), dim3(G::NT), 0, st, p);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MK_OK : mkh::hip_fail(e, "gate kernel launch");
}

}  // namespace

extern "C" size_t mk_moe_gate_workspace(int64_t T, int64_t H, int E) {
  if (T <= 0 || H <= 0 || E <= 0) return 256;
  const mkh::DevInfo* d = mkh::dev_info();
  return gate_ws_layout(T, H, E, d ? d->n_cu : 256).total;
}

extern "C" int mk_moe_gate(const void* X, const void* W_gate, int64_t T, int64_t H, int E, float* logits,
                           void* workspace, size_t workspace_bytes, void* stream) {
  using mkh::fail;
  if (!X || !W_gate || !logits) return fail(MK_ERR_INVALID, "X, W_gate and logits must be non-NULL");
  if (T < 1 || H < 8 || E < 8) return fail(MK_ERR_INVALID, "empty or too small shape");
  if (H % 8 || E % 8) return fail(MK_ERR_UNSUPPORTED, "H and E must be multiples of 8");
  if (E > MK_MAX_EXPERTS || T > (1 << 30) || H * E * 2 >= (1ll << 31) || (int64_t)GBM * H * 2 >= (1ll << 31) ||
      (int64_t)GBM * E * 4 >= (1ll << 31))
    return fail(MK_ERR_UNSUPPORTED, "dimension too large");
  if (!mkh::aligned16(X) || !mkh::aligned16(W_gate) || !mkh::aligned16(logits))
    return fail(MK_ERR_INVALID, "X, W_gate and logits must be 16-byte aligned");
  if (!workspace || !mkh::aligned16(workspace)) return fail(MK_ERR_WORKSPACE, "workspace NULL or misaligned");
  const mkh::DevInfo* d = mkh::dev_info();
  if (!d) return MK_ERR_HIP;
  const GateWs lay = gate_ws_layout(T, H, E, d->n_cu);
  if (workspace_bytes < lay.total) return fail(MK_ERR_WORKSPACE, "workspace %zu bytes < %zu", workspace_bytes, lay.total);
  GateParams p;
  memset(&p, 0, sizeof p);
  p.X = (const uint16_t*)X;
  p.W = (const uint16_t*)W_gate;
  p.out = logits;
  p.cnt = (uint32_t*)((char*)workspace + lay.cnt);
  p.slots = (float*)((char*)workspace + lay.slots);
  p.T = (int)T; p.H = (int)H; p.E = E;
  p.tiles_n = (E + GBN - 1) / GBN;
  p.n_tiles = (int)((T + GBM - 1) / GBM) * p.tiles_n;
  p.kp = gate_parts(T, H, E, d->n_cu);
  const hipStream_t st = (hipStream_t)stream;
  if (H % 128) return launch_gate<GateR, 1>(p, st);
  switch (p.kp) {
    case 1: return launch_gate<GateD, 1>(p, st);
    case 2: return launch_gate<GateD, 2>(p, st);
    case 4: return launch_gate<GateD, 4>(p, st);
    default: return launch_gate<GateD, 8>(p, st);
  }
}
