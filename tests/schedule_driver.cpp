// CPU driver for the schedule planner: reads "N num_cus waves" and the N + 1
// row pointers from stdin, prints "num_wgs waves KB" and then one batch entry
// (row kbeg count info) per line.
#include <cstdio>
#include <vector>

#include "schedule.h"

int main() {
  long long N = 0;
  int cus = 0, waves = 0;
  if (std::scanf("%lld %d %d", &N, &cus, &waves) != 3 || N < 0) return 2;
  std::vector<int32_t> ptr(N + 1);
  for (auto& v : ptr)
    if (std::scanf("%d", &v) != 1) return 2;
  ckhip::SchedulePlan plan;
  ckhip::plan_schedule(ptr.data(), N, cus, waves, &plan);
  std::printf("%d %d %d\n", plan.num_wgs, plan.waves, plan.KB);
  for (const auto& e : plan.table) std::printf("%d %d %d %d\n", e.row, e.kbeg, e.count, e.info);
  return 0;
}
