// Host check of the jagged schedule's sort key: reads "wl wr n" and n lines
// "lq lk" from stdin, prints each sequence's block count, then the indices in
// the order of ascending keys, decoded back from the keys.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "gdpa_kernels.hpp"

int main() {
  int wl = 0, wr = 0, n = 0;
  if (std::scanf("%d %d %d", &wl, &wr, &n) != 3 || n < 0 || n > gdpa::kSortMax) return 2;
  std::vector<uint64_t> keys(n);
  for (int i = 0; i < n; ++i) {
    int lq = 0, lk = 0;
    if (std::scanf("%d %d", &lq, &lk) != 2) return 2;
    std::printf("%lld\n", (long long)gdpa::mask_blocks(lq, lk, wl, wr));
    keys[i] = gdpa::schedule_key(lq, lk, wl, wr, i);
  }
  std::sort(keys.begin(), keys.end());
  for (int i = 0; i < n; ++i) std::printf("%d\n", gdpa::schedule_key_index(keys[i]));
  return 0;
}
