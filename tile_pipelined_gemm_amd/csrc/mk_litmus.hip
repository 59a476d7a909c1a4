// Message-passing litmus test of the cross-XCD publication protocol that the
// fused kernels use (a diagnostic, not part of any operation).
//
// MI355X has 8 XCDs with one L2 each; a workgroup on one XCD sees another
// XCD's stores only if the writer's release has written its L2 lines back
// and the reader's acquire has dropped stale lines from its own L2.  The
// kernels publish a work item as: every wave waits for its stores, barrier,
// one agent-scope release, relaxed atomic on a counter (wg_release); and
// consume it as: relaxed polls, one agent-scope acquire, then plain loads.
// This test runs exactly that pattern between pairs of workgroups: producer
// 2i and consumer 2i + 1 (adjacent workgroups are dispatched to different
// XCDs).  In round r the producer overwrites its pair's payload with r
// (plain write-back stores, so the data sits in its XCD's L2 until the
// release writes it back) and publishes flag = r; the consumer waits for the
// flag, acquires, reads the whole payload and counts words that are not r,
// then acknowledges r so the producer may write round r + 1.  With the
// fences the count must be zero.  `fenced` = 0 drops the consumer's acquire
// and the producer's release (keeping the waits for stores), so a run can
// show what the fences guard against; that mode reads stale data at worst.
//
// Every wait is bounded by the watchdog (spin_limit); a timed-out pair
// stops, sets the workspace status and abort flag, and the others stop at
// their next wait, so the grid always drains.  The grid is small (pairs <=
// 64 workgroup pairs) so producers and consumers are co-resident.
#include <string.h>

#include "mk_device.h"
#include "mk_host.h"

using namespace mk;

namespace {

constexpr int LIT_NT = 256;
constexpr int LIT_MAX_PAIRS = 64;

struct LitParams {
  WsHeader* hdr;
  uint32_t* flag;      // [pairs] round published by the producer
  uint32_t* ack;       // [pairs] round consumed by the consumer
  uint32_t* xcd;       // [2 pairs] XCD id + 1 of each workgroup
  uint32_t* payload;   // [pairs][words]
  uint32_t* result;    // {stale words, pairs on different XCDs, producer XCD mask, consumer XCD mask}
  uint64_t spin_limit;
  int words, rounds, fenced;
};

__global__ __launch_bounds__(LIT_NT) void litmus_kernel(const LitParams p) {
  __shared__ uint32_t sb[2];
  WsHeader* h = p.hdr;
  const int pair = blockIdx.x >> 1;
  const bool producer = (blockIdx.x & 1) == 0;
  const int tid = threadIdx.x;
  uint32_t* const data = p.payload + (int64_t)pair * p.words;
  // where each side runs: the consumer compares the two XCD ids
  if (tid == 0) {
    const uint32_t x = (uint32_t)xcd_id();
    atomicOr(&p.result[producer ? 2 : 3], 1u << x);
    st_relaxed(&p.xcd[blockIdx.x], x + 1u);
  }
  uint32_t stale = 0;
  for (int r = 1; r <= p.rounds; ++r) {
    uint32_t ok = 1;
    if (producer) {
      // wait until the consumer has read round r - 1
      if (tid == 0) ok = wait_geq_relaxed(&p.ack[pair], (uint32_t)(r - 1), h, p.spin_limit);
      if (!wg_bcast(ok, sb)) break;
      for (int i = tid; i < p.words; i += LIT_NT) data[i] = (uint32_t)r;
      if (p.fenced) {
        wg_release();
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
      }
      if (tid == 0) st_relaxed(&p.flag[pair], (uint32_t)r);
    } else {
      if (tid == 0) {
        ok = wait_geq_relaxed(&p.flag[pair], (uint32_t)r, h, p.spin_limit);
        if (ok && p.fenced) fence_acquire();
      }
      if (!wg_bcast(ok, sb)) break;
      for (int i = tid; i < p.words; i += LIT_NT) stale += data[i] != (uint32_t)r;
      // the loads above have returned before the acknowledgement
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (tid == 0) st_relaxed(&p.ack[pair], (uint32_t)r);
    }
  }
  if (!producer) {
    if (stale) atomicAdd(&p.result[0], stale);
    if (tid == 0) {
      const uint32_t a = ld_relaxed(&p.xcd[2 * pair]), b = ld_relaxed(&p.xcd[2 * pair + 1]);
      if (a && b && a != b) atomicAdd(&p.result[1], 1u);
    }
  }
}

struct LitWs { size_t flag, ack, xcd, payload, total; };
LitWs lit_layout(int pairs, int words) {
  LitWs w;
  w.flag = sizeof(WsHeader);
  w.ack = w.flag + (size_t)pairs * 4;
  w.xcd = w.ack + (size_t)pairs * 4;
  w.payload = (w.xcd + (size_t)pairs * 8 + 255) & ~(size_t)255;
  w.total = w.payload + (size_t)pairs * words * 4;
  return w;
}

}  // namespace

extern "C" size_t mk_litmus_workspace(int pairs, int words) {
  if (pairs < 1 || words < 1) return sizeof(WsHeader);
  return lit_layout(pairs, words).total;
}

extern "C" int mk_litmus_mp(int pairs, int words, int rounds, int fenced, uint32_t* result, void* workspace,
                            size_t workspace_bytes, uint32_t spin_limit_us, void* stream) {
  using mkh::fail;
  if (pairs < 1 || pairs > LIT_MAX_PAIRS) return fail(MK_ERR_INVALID, "pairs %d outside [1, %d]", pairs, LIT_MAX_PAIRS);
  if (words < 1 || words > (1 << 20)) return fail(MK_ERR_INVALID, "words %d outside [1, 2^20]", words);
  if (rounds < 1 || rounds > (1 << 20)) return fail(MK_ERR_INVALID, "rounds %d outside [1, 2^20]", rounds);
  if (fenced != 0 && fenced != 1) return fail(MK_ERR_INVALID, "fenced %d", fenced);
  if (!result || !mkh::aligned16(result)) return fail(MK_ERR_INVALID, "result NULL or misaligned");
  if (!workspace || !mkh::aligned16(workspace)) return fail(MK_ERR_WORKSPACE, "workspace NULL or misaligned");
  const LitWs lay = lit_layout(pairs, words);
  if (workspace_bytes < lay.total) return fail(MK_ERR_WORKSPACE, "workspace %zu bytes < %zu", workspace_bytes, lay.total);
  const mkh::DevInfo* d = mkh::dev_info();
  if (!d) return MK_ERR_HIP;
  if (2 * pairs > d->n_cu) return fail(MK_ERR_UNSUPPORTED, "%d workgroups need as many CUs", 2 * pairs);
  LitParams p;
  memset(&p, 0, sizeof p);
  p.hdr = (WsHeader*)workspace;
  p.flag = (uint32_t*)((char*)workspace + lay.flag);
  p.ack = (uint32_t*)((char*)workspace + lay.ack);
  p.xcd = (uint32_t*)((char*)workspace + lay.xcd);
  p.payload = (uint32_t*)((char*)workspace + lay.payload);
  p.result = result;
  mk_launch o;
  memset(&o, 0, sizeof o);
  o.spin_limit_us = spin_limit_us;
  p.spin_limit = mkh::spin_ticks(o, d);
  p.words = words;
  p.rounds = rounds;
  p.fenced = fenced;
  const hipStream_t st = (hipStream_t)stream;
  // the workspace and the result start from zero on every call
  int rc = mkh::zero_fill(workspace, lay.total, st);
  if (rc) return rc;
  rc = mkh::zero_fill(result, 16, st);
  if (rc) return rc;
  hipLaunchKernelGGL(litmus_kernel, dim3(2 * pairs), dim3(LIT_NT), 0, st, p);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MK_OK : mkh::hip_fail(e, "litmus kernel launch");
}
