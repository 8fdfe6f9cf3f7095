// Host build of the auxiliary kernels' launch geometry (grid_math.h) at the
// largest problem the library accepts: tokens * Hq = 2^31 - 1 rows, 16 lanes
// per row (the row dot product), and the merge's largest element count.
#include <cstdio>

#include "grid_math.h"

using namespace treeattn;

static int check(long long n, long long lanes_per_item) {
  const long long blocks = aux_blocks(n);
  const long long stride = aux_stride(blocks);
  if (n == 0) return blocks == 0 ? 0 : 10;
  if (blocks < 1 || blocks > 0x7FFFFFFFLL) return 1;            // grid x of a launch
  if (blocks * kAuxThreads > 0xFFFFFFFFLL) return 2;            // work-items of a dispatch
  if (aux_first(0, 0) != 0) return 3;
  if (aux_first(blocks - 1, kAuxThreads - 1) != stride - 1) return 4;  // threads cover [0, stride)
  const long long passes = (n + stride - 1) / stride;           // loop trips of thread 0
  if ((passes - 1) * stride >= n || passes * stride < n) return 5;
  if (stride % lanes_per_item != 0) return 6;                   // lanes of an item stay together
  if ((n - 1) / lanes_per_item != n / lanes_per_item - (n % lanes_per_item == 0)) return 7;
  std::printf("n=%lld blocks=%lld passes=%lld\n", n, blocks, passes);
  return 0;
}

int main() {
  const long long max_rows = (1LL << 31) - 1;
  int rc = 0;
  rc |= check(max_rows * 16, 16);           // row dot: 16 lanes per (token, head)
  rc |= check((1LL << 34) * 16, 16) << 8;   // lse_merge: rows * heads up to 2^34 at d = 64
  rc |= check(0, 1);
  rc |= check(1, 1);
  rc |= check(255, 1);
  rc |= check(257, 1);
  if (rc) std::printf("failed %d\n", rc);
  return rc ? 1 : 0;
}
