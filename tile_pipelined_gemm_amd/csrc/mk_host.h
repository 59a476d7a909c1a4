// Host-side helpers shared by the C-ABI entry points: error reporting,
// cached device properties, schedule validation and option defaults.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "../../include/mk.h"

namespace mkh {

// Record a thread-local message and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int hip_fail(hipError_t e, const char* what);

struct DevInfo {
  int device;
  int n_cu;
  int wall_khz;  // wall_clock64() rate
};
// Properties of the current device (cached per device).  NULL on failure
// (mk_last_error set).
const DevInfo* dev_info();

inline uint64_t ns_to_ticks(uint64_t ns, int khz) { return ns * (uint64_t)khz / 1000000ull; }

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Validated copy of an arrival schedule.
struct Schedule {
  int n_units = 0, unit_rows = 0, withhold = -1;
  std::vector<int32_t> order;     // issue order
  std::vector<int32_t> pos;       // pos[unit] = position in order
  std::vector<uint32_t> delay_ns;
};
// Validate `a` (or build the default: n_units units of unit_rows, identity
// order, zero delay) against `total_rows`.  Returns MK_OK or an error code.
int make_schedule(const mk_arrival* a, int64_t total_rows, int default_units, Schedule* out);

// Zero `bytes` (a multiple of 4) at device address p with a fill kernel on
// stream st (never a memset node).  MK_OK or MK_ERR_HIP.
int zero_fill(void* p, size_t bytes, hipStream_t st);

// Resolved launch options (0 fields replaced by defaults by each op).
mk_launch launch_opts(const mk_launch* l);
uint64_t spin_ticks(const mk_launch& l, const DevInfo* d);

}  // namespace mkh

// Per-shape defaults of each operation (defined beside its kernels; mk_plan
// reports them, the entry points apply them).
namespace mkp {
int ag_default_tile(int64_t M, int64_t N, int64_t K, bool pack, int n_cu);
int64_t ag_default_item_bytes(int64_t M, int64_t K, int n_cu);
bool ag_default_pack(int64_t M, int64_t K);
int ag_default_n_copy(int grid);
void ag_column_plan(int tiles_m, int64_t N, int grid, int* tn_wide, int* tn_narrow);
int rs_default_tile(int64_t M, int64_t N, int64_t K, int mb, int n_cu);
int moe_default_tile(int64_t H, int64_t F);
}  // namespace mkp
