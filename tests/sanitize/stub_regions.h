// Regions of fake device addresses a sanitizer-build call may touch.
#pragma once

#include <cstddef>
#include <cstdint>

namespace stub {

struct Region {
  const char* name;
  uintptr_t base;
  size_t bytes;
};

constexpr int kMaxRegions = 32;
// Fake address of the no-alloc scratch array.
constexpr uintptr_t kScratchBase = (uintptr_t)0x7e0000000000ull;

extern long g_launches;
void clear();
void add(const char* name, const void* base, size_t bytes);

}  // namespace stub
