// Error plumbing shared by the host sources of libpkv.
#pragma once

#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/pkv.h"

namespace pkv {

// Records a thread-local message and returns `code`.
pkv_status fail(pkv_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pkv_status ok();

}  // namespace pkv

// Runs a body that may throw; converts escapes into PKV_ERR_INTERNAL so no
// exception crosses the C boundary.
#define PKV_GUARD(...)                                                         \
  try {                                                                        \
    __VA_ARGS__                                                                \
  } catch (const std::bad_alloc&) {                                            \
    return pkv::fail(PKV_ERR_INTERNAL, "host allocation failed");              \
  } catch (const std::exception& e) {                                          \
    return pkv::fail(PKV_ERR_INTERNAL, "internal error: %s", e.what());        \
  } catch (...) {                                                              \
    return pkv::fail(PKV_ERR_INTERNAL, "internal error");                      \
  }
