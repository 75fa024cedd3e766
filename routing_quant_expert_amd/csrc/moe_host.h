// Host-side helpers of the entry points (no device code).
#pragma once

#include <new>

#include "moe_internal.h"

namespace moe {

// Runs a host-side entry-point body that allocates host memory, turning a C++
// exception into an error code (nothing may unwind through the C ABI).
template <class F>
int guarded(F&& body) {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    return fail(MOE_EUNSUPPORTED, "host memory exhausted%s%lld");
  } catch (...) {
    return fail(MOE_EINVAL, "unexpected host-side error%s%lld");
  }
}

}  // namespace moe
