// The library's static device scratch for callers that cannot allocate (moe_permute_noalloc).
#pragma once

#include <stddef.h>

namespace moe {

// Size of the scratch: 4 MiB per device.
constexpr size_t kNoallocScratchBytes = size_t(4) << 20;

// Device address of that scratch on the current device (looked up once per device), or
// NULL when the lookup fails.
void* permute_noalloc_scratch();

}  // namespace moe
