// CPU driver for the resident planner: reads "N ranks max_D every order" (every
// = 1: every wave gathers, as in the backward) and the
// N + 1 row pointers from stdin, then (order = 1) the row read by each
// compressed edge; prints "none", or "D ranks max_pieces cost cost_ordered misses"
// (bank-conflict costs of the slot table in compressed order and after
// ordering, and the ordering's slots off their wave's permutation; 0 when
// not ordered) followed by rank_rows, owner_pbeg, piece_row,
// piece_kbeg, piece_cnt and slot_edge (one array per line).
#include <cstdio>
#include <vector>

#include "schedule.h"

static void put(const std::vector<int32_t>& v) {
  for (size_t i = 0; i < v.size(); ++i) std::printf(i ? " %d" : "%d", v[i]);
  std::printf("\n");
}

int main() {
  long long N = 0;
  int ranks = 0, max_D = 0, every = 0, order = 0;
  if (std::scanf("%lld %d %d %d %d", &N, &ranks, &max_D, &every, &order) != 5 || N < 0) return 2;
  std::vector<int32_t> ptr(N + 1);
  for (auto& v : ptr)
    if (std::scanf("%d", &v) != 1) return 2;
  std::vector<int32_t> col;
  if (order) {
    col.resize(ptr[N]);
    for (auto& v : col)
      if (std::scanf("%d", &v) != 1) return 2;
  }
  ckhip::ResidentPlan plan;
  if (!ckhip::plan_resident(ptr.data(), N, ranks, max_D, every != 0, &plan)) {
    std::printf("none\n");
    return 0;
  }
  long long c0 = 0, c1 = 0;
  if (order) {
    c0 = ckhip::resident_conflict_cost(col.data(), N, plan);
    ckhip::order_resident_slots(col.data(), N, &plan);
    c1 = ckhip::resident_conflict_cost(col.data(), N, plan);
  }
  std::printf("%d %d %d %lld %lld %lld\n", plan.D, plan.ranks, plan.max_pieces, c0, c1,
              (long long)plan.order_misses);
  put(plan.rank_rows);
  put(plan.owner_pbeg);
  put(plan.piece_row);
  put(plan.piece_kbeg);
  put(plan.piece_cnt);
  put(plan.slot_edge);
  return 0;
}
