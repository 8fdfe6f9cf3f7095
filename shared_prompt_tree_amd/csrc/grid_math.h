// Launch geometry of the element-wise auxiliary kernels (row dot, merge,
// seed and chunk sums, transposed copies).  Plain C++: constexpr functions
// are usable in device code and in a host-only build of the tests.
//
// A dispatch describes its grid in work-items with 32-bit fields, so a
// launch of one thread per element cannot cover every size the library
// accepts (up to 2^31 - 1 rows times 16 lanes).  These kernels instead launch
// at most kAuxMaxBlocks workgroups and walk the elements with a 64-bit
// grid-stride loop: element i is handled by thread i % stride in pass
// i / stride.
#pragma once

#include <stdint.h>

namespace treeattn {

constexpr int kAuxThreads = 256;
constexpr long long kAuxMaxBlocks = 1LL << 22;  // 2^30 work-items per dispatch

// Workgroups for n elements (0 for none).
constexpr long long aux_blocks(long long n) {
  const long long b = (n + kAuxThreads - 1) / kAuxThreads;
  return b < kAuxMaxBlocks ? b : kAuxMaxBlocks;
}

// First element of thread `tid` of workgroup `block`, and the loop stride.
constexpr long long aux_first(long long block, long long tid) { return block * kAuxThreads + tid; }
constexpr long long aux_stride(long long blocks) { return blocks * kAuxThreads; }

}  // namespace treeattn
