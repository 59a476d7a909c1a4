// Host-side helpers and the support entry points of libmk.
#include "mk_host.h"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "mk_device.h"

namespace mkh {

static thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

const DevInfo* dev_info() {
  static DevInfo cache[64];
  static bool have[64];
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    hip_fail(e, "hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= 64) {
    fail(MK_ERR_UNSUPPORTED, "device index %d out of range", dev);
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(mu);
  if (!have[dev]) {
    DevInfo d{dev, 0, 0};
    if ((e = hipDeviceGetAttribute(&d.n_cu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess ||
        (e = hipDeviceGetAttribute(&d.wall_khz, hipDeviceAttributeWallClockRate, dev)) != hipSuccess) {
      hip_fail(e, "hipDeviceGetAttribute");
      return nullptr;
    }
    if (d.wall_khz <= 0) d.wall_khz = 100000;
    cache[dev] = d;
    have[dev] = true;
  }
  return &cache[dev];
}

int make_schedule(const mk_arrival* a, int64_t total_rows, int default_units, Schedule* s) {
  if (!a) {
    s->n_units = default_units;
    s->unit_rows = (int)(total_rows / default_units);
    s->withhold = -1;
    s->order.resize(default_units);
    for (int i = 0; i < default_units; ++i) s->order[i] = i;
    s->delay_ns.assign(default_units, 0u);
  } else {
    if (a->n_units <= 0 || a->unit_rows <= 0)
      return fail(MK_ERR_SCHEDULE, "n_units (%d) and unit_rows (%d) must be positive", a->n_units, a->unit_rows);
    if (a->n_units > MK_MAX_UNITS)
      return fail(MK_ERR_UNSUPPORTED, "n_units %d exceeds %d", a->n_units, MK_MAX_UNITS);
    if ((int64_t)a->n_units * a->unit_rows != total_rows)
      return fail(MK_ERR_SCHEDULE, "n_units*unit_rows = %lld does not cover %lld rows",
                  (long long)a->n_units * a->unit_rows, (long long)total_rows);
    if (!a->order) return fail(MK_ERR_SCHEDULE, "schedule order is NULL");
    s->n_units = a->n_units;
    s->unit_rows = a->unit_rows;
    s->withhold = a->withhold;
    if (s->withhold < -1 || s->withhold >= s->n_units)
      return fail(MK_ERR_SCHEDULE, "withhold %d out of range", s->withhold);
    s->order.assign(a->order, a->order + a->n_units);
    s->delay_ns.assign(a->n_units, 0u);
    if (a->delay_ns) s->delay_ns.assign(a->delay_ns, a->delay_ns + a->n_units);
    for (uint32_t d : s->delay_ns)
      if (d > 1000000000u) return fail(MK_ERR_SCHEDULE, "delay %u ns exceeds 1 s", d);
  }
  s->pos.assign(s->n_units, -1);
  for (int j = 0; j < s->n_units; ++j) {
    const int c = s->order[j];
    if (c < 0 || c >= s->n_units || s->pos[c] != -1)
      return fail(MK_ERR_SCHEDULE, "order is not a permutation (entry %d = %d)", j, c);
    s->pos[c] = j;
  }
  return MK_OK;
}

mk_launch launch_opts(const mk_launch* l) {
  mk_launch o;
  memset(&o, 0, sizeof o);
  if (l) o = *l;
  return o;
}

uint64_t spin_ticks(const mk_launch& l, const DevInfo* d) {
  const uint64_t us = l.spin_limit_us ? l.spin_limit_us : 2000000u;
  return ns_to_ticks(us * 1000ull, d->wall_khz);
}

namespace {
__global__ void fill_zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}
}  // namespace

int zero_fill(void* p, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 4;
  const int blocks = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, st, (uint32_t*)p, n);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MK_OK : hip_fail(e, "fill kernel launch");
}

}  // namespace mkh

// ---------------------------------------------------------------- support ABI
extern "C" int mk_workspace_init(void* ws, size_t bytes, void* stream) {
  if (!ws) return mkh::fail(MK_ERR_WORKSPACE, "workspace is NULL");
  if (bytes < sizeof(mk::WsHeader) || (bytes & 3u))
    return mkh::fail(MK_ERR_WORKSPACE, "workspace size %zu too small or not a multiple of 4", bytes);
  if (!mkh::aligned16(ws)) return mkh::fail(MK_ERR_INVALID, "workspace not 16-byte aligned");
  return mkh::zero_fill(ws, bytes, (hipStream_t)stream);
}

extern "C" int mk_poll_status(void* ws, void* stream) {
  if (!ws) return mkh::fail(MK_ERR_WORKSPACE, "workspace is NULL");
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return mkh::hip_fail(e, "hipStreamSynchronize");
  uint32_t st = 0;
  mk::WsHeader* h = (mk::WsHeader*)ws;
  e = hipMemcpy(&st, &h->status, sizeof st, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return mkh::hip_fail(e, "read status");
  if (st == mk::ST_OK) return MK_OK;
  const uint32_t zero = 0;
  e = hipMemcpy(&h->status, &zero, sizeof zero, hipMemcpyHostToDevice);
  if (e != hipSuccess) return mkh::hip_fail(e, "clear status");
  if (st == mk::ST_TIMEOUT) return mkh::fail(MK_ERR_TIMEOUT, "a kernel wait exceeded its watchdog");
  return mkh::fail(MK_ERR_HIP, "unknown device status %u", st);
}

extern "C" const char* mk_status_string(int s) {
  switch (s) {
    case MK_OK: return "ok";
    case MK_ERR_INVALID: return "invalid argument";
    case MK_ERR_UNSUPPORTED: return "unsupported";
    case MK_ERR_WORKSPACE: return "workspace missing or too small";
    case MK_ERR_HIP: return "HIP runtime error";
    case MK_ERR_TIMEOUT: return "watchdog timeout";
    case MK_ERR_SCHEDULE: return "invalid arrival schedule";
    default: return "unknown status";
  }
}

extern "C" const char* mk_last_error(void) { return mkh::g_err.c_str(); }

extern "C" int mk_version(void) { return 1; }

extern "C" int mk_wall_clock_khz(void) {
  const mkh::DevInfo* d = mkh::dev_info();
  return d ? d->wall_khz : MK_ERR_HIP;
}

#include "mk_tiles.h"

extern "C" int mk_plan(int op, int64_t M, int64_t N, int64_t K, int R, mk_launch* out) {
  using mkh::fail;
  if (!out) return fail(MK_ERR_INVALID, "out is NULL");
  const bool shaped = op == MK_OP_MOE ? (N > 0 && K > 0) : (M > 0 && N > 0 && K > 0 && R >= 1);
  if (!shaped) return fail(MK_ERR_INVALID, "non-positive dimension");
  mk_launch o;
  memset(&o, 0, sizeof o);
  // the CU count of the current device, or 256 when none answers
  int dev = 0, n_cu = 256;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
    n_cu = prop.multiProcessorCount;
  else
    (void)hipGetLastError();
  switch (op) {
    case MK_OP_AG_GEMM: {
      o.tile = mkp::ag_default_tile(M, N, K, mkp::ag_default_pack(M, K), n_cu);
      o.copy_kib = (int32_t)((mkp::ag_default_item_bytes(M, K, n_cu) + 1023) >> 10);
      break;
    }
    case MK_OP_GEMM_RS:
    case MK_OP_GEMM_AR:
      o.tile = mkp::rs_default_tile(M, N, K, op == MK_OP_GEMM_AR ? 256 : (int)(M / R), n_cu);
      o.copy_kib = 1024;
      break;
    case MK_OP_MOE:
      o.tile = mkp::moe_default_tile(K, N);
      break;
    default:
      return fail(MK_ERR_INVALID, "op %d", op);
  }
  *out = o;
  return MK_OK;
}

extern "C" const char* mk_tile_name(int id) {
  static const char* names[TILE_COUNT] = {"auto",       "256x256",    "128x128",    "256x128",   "128x256",
                                               "256x256dma", "128x128dma", "256x128dma", "128x256dma",
                                               "128x128dma8", "256x256dma_w8", "128x128pc"};
  return (id >= 0 && id < TILE_COUNT) ? names[id] : nullptr;
}
