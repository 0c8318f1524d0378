// Host-side parts of the C ABI: status strings, error text, layout buffer sizing and carving.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

#include "moe_internal.h"

namespace {
thread_local char g_err[256] = "";
size_t align256(size_t b) { return (b + 255) & ~size_t(255); }
}  // namespace

namespace moe_host {
void set_error(const char* msg) {
  strncpy(g_err, msg, sizeof(g_err) - 1);
  g_err[sizeof(g_err) - 1] = 0;
}
moe_status launch_status() {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return MOE_OK;
  snprintf(g_err, sizeof(g_err), "HIP launch error: %s", hipGetErrorString(e));
  return MOE_EHIP;
}
}  // namespace moe_host

extern "C" const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EHIP: return "MOE_EHIP: HIP launch failure";
  }
  return "unknown moe_status";
}

extern "C" const char* moe_last_error(void) { return g_err; }

extern "C" moe_status moe_device_info(int* cus, int* lds_bytes_per_cu, int* clock_khz,
                                      int* mem_clock_khz) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    moe_host::set_error("moe_device_info: no current HIP device");
    return MOE_EHIP;
  }
  const struct {
    int* out;
    hipDeviceAttribute_t attr;
  } q[] = {{cus, hipDeviceAttributeMultiprocessorCount},
           {lds_bytes_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor},
           {clock_khz, hipDeviceAttributeClockRate},
           {mem_clock_khz, hipDeviceAttributeMemoryClockRate}};
  for (const auto& e : q) {
    if (!e.out) continue;
    if (hipDeviceGetAttribute(e.out, e.attr, dev) != hipSuccess) {
      moe_host::set_error("moe_device_info: hipDeviceGetAttribute failed");
      return MOE_EHIP;
    }
  }
  return MOE_OK;
}

// Element counts of the layout arrays, in struct order.
static void layout_counts(const moe_shape* s, size_t* n) {
  const size_t N = s->N, E = s->E, k = s->k, W = s->W;
  const size_t kw = k < W ? k : W;
  const size_t c[15] = {E, E, E, E + 1, W, W + 1, W * W, N * k, N * k, W, W + 1, N * kw,
                        N * k, W * W, N * k};
  memcpy(n, c, sizeof(c));
}

extern "C" size_t moe_layout_bytes(const moe_shape* s) {
  if (!moe_host::shape_ok(s)) return 0;
  size_t n[15], b = 0;
  layout_counts(s, n);
  for (int i = 0; i < 15; ++i) b += align256(n[i] * 4);
  return b;
}

extern "C" moe_status moe_layout_carve(const moe_shape* s, void* base, moe_layout* L) {
  if (!moe_host::shape_ok(s) || !base || !L) {
    moe_host::set_error("moe_layout_carve: invalid shape or NULL pointer");
    return MOE_EINVAL;
  }
  size_t n[15];
  layout_counts(s, n);
  int32_t** f[15] = {&L->expert_counts, &L->expert_offsets, &L->group_expert,
                     &L->group_offsets, &L->rank_counts,    &L->rank_offsets,
                     &L->send_counts,   &L->row_of_slot,    &L->slot_of_row,
                     &L->pair_counts,   &L->pair_offsets,   &L->pair_token,
                     &L->pair_of_slot,  &L->pair_send_counts, &L->expand_src};
  char* p = static_cast<char*>(base);
  for (int i = 0; i < 15; ++i) {
    *f[i] = reinterpret_cast<int32_t*>(p);
    p += align256(n[i] * 4);
  }
  return MOE_OK;
}
