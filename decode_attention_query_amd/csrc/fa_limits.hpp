// fa_limits.hpp -- constants shared by the host launch plan and the kernels
// (plain C++, no device code).
#pragma once

namespace fa {

// Bits of an arrival counter that count split units (the rest carry the rest
// mark): a request has fewer than 2^24 split units.
constexpr int kCountBits = 24;

// 64-bit words from one arrival counter to the next: 128 bytes, one cache line
// each.  Atomics on one line are serialised where they are performed, and the
// units of one request finish close together, so counters that shared a line
// queued behind each other (a 16-unit request on 8 head blocks: 128 atomics).
constexpr int kArrivalStride = 16;

// Page slots of one split unit staged in LDS (the host caps the split size so
// a unit spans at most 1024 whole pages plus a partial one at each end).
constexpr int kPageTable = 1040;

}  // namespace fa
