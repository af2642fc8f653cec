// CPU driver for the resident planner: reads "N ranks max_lens" and the N + 1
// row pointers from stdin; prints "none", or "D ranks max_pieces blk" followed by
// rank_rows, owner_pbeg, piece_row, piece_kbeg, piece_cnt and piece_blk (one
// array per line).
#include <cstdio>
#include <vector>

#include "schedule.h"

static void put(const std::vector<int32_t>& v) {
  for (size_t i = 0; i < v.size(); ++i) std::printf(i ? " %d" : "%d", v[i]);
  std::printf("\n");
}

int main() {
  long long N = 0;
  int ranks = 0, lens = 0;
  if (std::scanf("%lld %d %d", &N, &ranks, &lens) != 3 || N < 0) return 2;
  std::vector<int32_t> ptr(N + 1);
  for (auto& v : ptr)
    if (std::scanf("%d", &v) != 1) return 2;
  ckhip::ResidentPlan plan;
  if (!ckhip::plan_resident(ptr.data(), N, ranks, lens, &plan)) {
    std::printf("none\n");
    return 0;
  }
  std::printf("%d %d %d %d\n", plan.D, plan.ranks, plan.max_pieces, plan.blk);
  put(plan.rank_rows);
  put(plan.owner_pbeg);
  put(plan.piece_row);
  put(plan.piece_kbeg);
  put(plan.piece_cnt);
  put(plan.piece_blk);
  return 0;
}
