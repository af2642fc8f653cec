// CPU driver for the blocked planner: reads "N num_cus", the N + 1 row
// pointers and the node read by each compressed edge from stdin; prints
// "none", or "num_wgs KB items" followed by row_items, the table as row,
// kbeg, count, id per entry, edge_order and item_ids (one array per line).
#include <cstdio>
#include <vector>

#include "schedule.h"

int main() {
  long long N = 0;
  int cus = 0;
  if (std::scanf("%lld %d", &N, &cus) != 2 || N < 0) return 2;
  std::vector<int32_t> ptr(N + 1);
  for (auto& v : ptr)
    if (std::scanf("%d", &v) != 1) return 2;
  std::vector<int32_t> col(ptr[N]);
  for (auto& v : col)
    if (std::scanf("%d", &v) != 1) return 2;
  ckhip::BlockedPlan plan;
  if (!ckhip::plan_blocked(ptr.data(), col.data(), N, cus, &plan)) {
    std::printf("none\n");
    return 0;
  }
  std::printf("%d %d %lld\n", plan.num_wgs, plan.KB, (long long)plan.items);
  for (size_t i = 0; i < plan.row_items.size(); ++i)
    std::printf(i ? " %d" : "%d", plan.row_items[i]);
  std::printf("\n");
  for (size_t i = 0; i < plan.table.size(); ++i) {
    const ckhip::BlkItem& t = plan.table[i];
    std::printf(i ? " %d %d %d %d" : "%d %d %d %d", t.row, t.kbeg, t.count, t.id);
  }
  std::printf("\n");
  for (size_t i = 0; i < plan.edge_order.size(); ++i)
    std::printf(i ? " %d" : "%d", plan.edge_order[i]);
  std::printf("\n");
  for (size_t i = 0; i < plan.item_ids.size(); ++i)
    std::printf(i ? " %d" : "%d", plan.item_ids[i]);
  std::printf("\n");
  return 0;
}
