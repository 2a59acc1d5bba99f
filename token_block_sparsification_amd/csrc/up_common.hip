// Error reporting, device checks and host helpers of the C ABI.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "up_internal.h"

namespace up {

static thread_local char g_err[512] = "";

up_status set_error(up_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_err[0] = '\0'; }

// Per-device result of the architecture check: 0 unknown, 1 ok, 2 wrong arch.
static int g_dev_ok[64];
static std::mutex g_dev_mu;

up_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(UP_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return set_error(UP_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return set_error(UP_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    g_dev_ok[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
  }
  if (g_dev_ok[dev] != 1)
    return set_error(UP_ERR_UNSUPPORTED, "device %d is not gfx950 (MI355X)", dev);
  return UP_OK;
}

up_status check_cu_seqlens(int num_seqs, const int32_t* cu_h, int64_t* T, int* max_len) {
  if (num_seqs < 0) return set_error(UP_ERR_INVALID, "num_seqs < 0");
  if (cu_h == nullptr) return set_error(UP_ERR_INVALID, "cu_seqlens_h is NULL");
  if (cu_h[0] != 0) return set_error(UP_ERR_INVALID, "cu_seqlens_h[0] != 0");
  int mx = 0;
  for (int r = 0; r < num_seqs; ++r) {
    if (cu_h[r + 1] < cu_h[r])
      return set_error(UP_ERR_INVALID, "cu_seqlens_h decreases at %d", r);
    int L = cu_h[r + 1] - cu_h[r];
    if (L > mx) mx = L;
  }
  *T = cu_h[num_seqs];
  *max_len = mx;
  return UP_OK;
}

up_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(UP_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return UP_OK;
}

}  // namespace up

extern "C" {

int up_abi_version(void) { return UP_ABI_VERSION; }

const char* up_last_error(void) { return up::g_err; }

const char* up_status_string(int status) {
  switch (status) {
    case UP_OK: return "UP_OK";
    case UP_ERR_INVALID: return "UP_ERR_INVALID";
    case UP_ERR_UNSUPPORTED: return "UP_ERR_UNSUPPORTED";
    case UP_ERR_WORKSPACE: return "UP_ERR_WORKSPACE";
    case UP_ERR_CAPACITY: return "UP_ERR_CAPACITY";
    case UP_ERR_HIP: return "UP_ERR_HIP";
    default: return "UP_STATUS_UNKNOWN";
  }
}

up_status up_make_cu_blocks(int num_seqs, const int32_t* cu_seqlens_h, int block,
                            int32_t* cu_blocks_h, int64_t* num_blocks) {
  up::clear_error();
  if (block < 1) return up::set_error(UP_ERR_INVALID, "block < 1");
  if (cu_blocks_h == nullptr) return up::set_error(UP_ERR_INVALID, "cu_blocks_h is NULL");
  int64_t T;
  int mx;
  up_status st = up::check_cu_seqlens(num_seqs, cu_seqlens_h, &T, &mx);
  if (st != UP_OK) return st;
  int64_t acc = 0;
  cu_blocks_h[0] = 0;
  for (int r = 0; r < num_seqs; ++r) {
    int L = cu_seqlens_h[r + 1] - cu_seqlens_h[r];
    acc += (L + block - 1) / block;
    cu_blocks_h[r + 1] = (int32_t)acc;
  }
  if (num_blocks) *num_blocks = acc;
  return UP_OK;
}

}  // extern "C"
