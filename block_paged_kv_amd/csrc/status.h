// Thread-local status reporting shared by every C entry point of libpagedkv.
#pragma once

#include <cstdarg>
#include <cstdint>
#include <exception>
#include <new>

#include "pagedkv.h"

namespace pagedkv {

// Record a formatted message for paged_last_error() and return `code`.
int32_t fail(int32_t code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the message and return PAGED_OK.
int32_t ok();

}  // namespace pagedkv

// Run the lambda given as the macro argument (returning int32_t) with C++ exceptions turned into codes.
#define PAGEDKV_GUARD(...)                                                        \
  try {                                                                           \
    return (__VA_ARGS__)();                                                         \
  } catch (const std::bad_alloc&) {                                               \
    return ::pagedkv::fail(PAGED_ERR_NO_BLOCKS, "host allocation failed");        \
  } catch (const std::exception& e) {                                             \
    return ::pagedkv::fail(PAGED_ERR_STATE, "internal error: %s", e.what());      \
  } catch (...) {                                                                 \
    return ::pagedkv::fail(PAGED_ERR_STATE, "internal error");                    \
  }
