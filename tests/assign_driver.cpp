// CPU driver for the planner's assignment solver: reads "n" then n * n
// integer costs (row-major) per case from stdin until end of input, and
// prints the chosen column of each row, one case per line.
#include <cstdio>
#include <vector>

#include "schedule.h"

int main() {
  int n = 0;
  while (std::scanf("%d", &n) == 1) {
    if (n <= 0 || n > 64) return 2;
    std::vector<int> cost((size_t)n * n), col(n);
    for (auto& v : cost)
      if (std::scanf("%d", &v) != 1) return 2;
    ckhip::assign_min_cost(cost.data(), n, col.data());
    for (int i = 0; i < n; ++i) std::printf(i ? " %d" : "%d", col[i]);
    std::printf("\n");
  }
  return 0;
}
