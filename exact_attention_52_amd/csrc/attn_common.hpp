// attn_common.hpp -- host-side argument checks shared by the C-ABI sources
// of libattn.so (attn_api.hip) and libattn_unfused.so (attn_unfused.hip):
// error reporting, size limits, buffer overlap and the gfx950 device check.
// Each library includes this from exactly one translation unit, so each has
// its own thread-local error text and device cache.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "attn.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return ATTN_OK;
}

int check_sizes(int64_t B, int64_t H, int64_t S, int64_t D, int dtype) {
  if (B < 0 || H < 0 || S < 0)
    return fail(ATTN_ERR_BAD_SHAPE, "B, H and S must be >= 0 (got B=%lld H=%lld S=%lld)",
                (long long)B, (long long)H, (long long)S);
  if (D != 64 && D != 128 && D != 256)
    return fail(ATTN_ERR_UNSUPPORTED_HEAD_DIM, "head_dim %lld not supported; must be one of 64, 128, 256",
                (long long)D);
  if (dtype != ATTN_F16 && dtype != ATTN_BF16)
    return fail(ATTN_ERR_UNSUPPORTED_DTYPE, "dtype %d not supported; must be ATTN_F16 (0) or ATTN_BF16 (1)",
                dtype);
  // Per-head offsets are 32-bit byte offsets (buffer loads); keep one head's
  // S*D elements, plus a tile of padding, far inside that range.
  const int64_t lim = (int64_t)1 << 30;
  if (S > lim / D)
    return fail(ATTN_ERR_BAD_SHAPE, "S=%lld too large for head_dim %lld", (long long)S, (long long)D);
  if (B > 0 && H > 0 && S > 0) {
    const int64_t bh_lim = ((int64_t)1 << 62) / (S * D);
    if (H > bh_lim / (B > 0 ? B : 1) || B * H > bh_lim)
      return fail(ATTN_ERR_BAD_SHAPE, "B*H*S*D overflows");
  }
  return ATTN_OK;
}

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

// gfx950 check, cached per device.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];  // 0 unknown, 1 yes, 2 no

int check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0)
    return fail(ATTN_ERR_UNSUPPORTED_DEVICE, "no current HIP device (%s)", hipGetErrorString(e));
  int state = dev < kMaxDevices ? g_arch_ok[dev].load(std::memory_order_relaxed) : 0;
  if (state == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(ATTN_ERR_UNSUPPORTED_DEVICE, "hipGetDeviceProperties failed (%s)", hipGetErrorString(e));
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    if (dev < kMaxDevices) g_arch_ok[dev].store(state, std::memory_order_relaxed);
    if (state == 2)
      return fail(ATTN_ERR_UNSUPPORTED_DEVICE, "device %d is %s; this library is built for gfx950 only", dev,
                  prop.gcnArchName);
  }
  if (state == 2) return fail(ATTN_ERR_UNSUPPORTED_DEVICE, "device %d is not gfx950", dev);
  return ATTN_OK;
}

}  // namespace
