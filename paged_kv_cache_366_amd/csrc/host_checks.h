// Host-side argument checks shared by the device entry points.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdlib>
#include <cstring>
#include <vector>

#include "status.h"

namespace pkv {

inline int dtype_bytes(pkv_dtype d) {
  switch (d) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
    case PKV_I8: return 1;
    case PKV_I4: return 1;   // raw byte; two elements share it (see row_bytes)
    default: return 0;
  }
}

// Bytes of one row of `n` elements (4-bit storage: n / 2, n even).
inline int64_t row_bytes(pkv_dtype d, int64_t n) {
  return d == PKV_I4 ? n / 2 : n * dtype_bytes(d);
}

// Storage with per-(block, kv head) scales beside the codes.
inline bool has_scales(pkv_dtype d) { return d == PKV_I8 || d == PKV_I4; }

inline const char* dtype_name(pkv_dtype d) {
  switch (d) {
    case PKV_F32: return "f32";
    case PKV_F16: return "f16";
    case PKV_BF16: return "bf16";
    case PKV_I8: return "i8";
    case PKV_I4: return "i4";
    default: return "?";
  }
}

// PKV_VALIDATE=1 turns on device-array checks (copies to host, synchronises).
inline bool deep_validation() {
  const char* v = std::getenv("PKV_VALIDATE");
  return v && v[0] && std::strcmp(v, "0") != 0;
}

// Copies `n` int32 values from device memory to a host vector.
inline pkv_status fetch_i32(const int32_t* dev, size_t n, void* stream, std::vector<int32_t>& out) {
  out.resize(n);
  if (n == 0) return PKV_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(out.data(), dev, n * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess)
    return fail(PKV_ERR_DEVICE, "copying indices for validation failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace pkv
