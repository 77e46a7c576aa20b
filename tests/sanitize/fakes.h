// Bookkeeping of the host-only launch stand-ins (host_fakes.cpp).
#pragma once
#include <cstdint>

namespace fake {
void reset();                                  // forget ranges, zero the counters
void add_range(const void *base, int64_t bytes);  // a tensor of the current call
void *noalloc_base();                          // stand-in address of the library's scratch array
extern long g_images;                          // images over all launches since reset()
extern long g_launches;
}  // namespace fake
