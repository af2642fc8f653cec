// schedule.cpp -- host-side planning of the per-wave batch lists (see
// schedule.h); called by ck_graph_create for each orientation and width.
#include "schedule.h"

#include <algorithm>
#include <climits>

namespace ckhip {

// Degree-balanced, XCD-aware schedule (host side, from the row pointers) for
// workgroups of `waves` waves.  The unit of work is a batch: at most
// kBatchEdges edges of one row, one gather round of a wave at B = 32; a row
// without edges takes one empty batch (its epilogue still runs).
//  1. Rows are cut into kXcds contiguous ranges of about equal batch count;
//     workgroup g runs on XCD g % kXcds as that XCD's workgroup g / kXcds.
//  2. Inside an XCD the rows are cut into at most wg_x contiguous workgroup
//     ranges whose largest batch count is as small as possible (bisection on
//     that bound, with greedy packing as the test).
//  3. A workgroup's batches, in row order, are dealt to its waves as
//     contiguous runs whose lengths differ by at most one.  A row whose batches
//     land on several waves is split into pieces (one segment per wave), and
//     its last piece's wave adds the pieces up after the workgroup barrier.
void plan_schedule(const int32_t* ptr, int64_t N, int num_cus, int waves, SchedulePlan* out) {
  constexpr int64_t kMinWaveBatches = 2;  // small graphs: fewer, fuller workgroups
  std::vector<int64_t> nb(N);
  int64_t total = 0;
  for (int64_t i = 0; i < N; ++i) {
    const int64_t d = ptr[i + 1] - ptr[i];
    nb[i] = std::max<int64_t>(1, (d + kBatchEdges - 1) / kBatchEdges);
    total += nb[i];
  }
  std::vector<int64_t> cut(kXcds + 1, N);
  cut[0] = 0;
  {
    int64_t acc = 0;
    int x = 1;
    for (int64_t i = 0; i < N && x < kXcds; ++i) {
      acc += nb[i];
      while (x < kXcds && acc * kXcds >= total * x) cut[x++] = i + 1;
    }
  }
  const int64_t cap = std::max<int64_t>(1, (int64_t)num_cus / kXcds * (kWavesPerCu / waves));
  const int64_t per_x = (total + kXcds - 1) / kXcds;
  const int wg_x = (int)std::min<int64_t>(
      cap, std::max<int64_t>(1, (per_x + kMinWaveBatches * waves - 1) / (kMinWaveBatches * waves)));
  // lists[(wgl * kXcds + x) * waves + wave]: batch entries of one wave
  std::vector<std::vector<BatchEntry>> lists((size_t)wg_x * kXcds * waves);
  for (int x = 0; x < kXcds; ++x) {
    const int64_t r0 = cut[x], r1 = cut[x + 1];
    if (r0 >= r1) continue;
    // number of workgroup ranges greedy packing needs under bound lim
    auto pack = [&](int64_t lim, std::vector<int64_t>* bounds) {
      int64_t groups = 1, sum = 0;
      if (bounds) bounds->assign(1, r0);
      for (int64_t i = r0; i < r1; ++i) {
        if (sum > 0 && sum + nb[i] > lim) {
          ++groups;
          sum = 0;
          if (bounds) bounds->push_back(i);
        }
        sum += nb[i];
      }
      if (bounds) bounds->push_back(r1);
      return groups;
    };
    int64_t sum = 0, big = 0;
    for (int64_t i = r0; i < r1; ++i) {
      sum += nb[i];
      big = std::max(big, nb[i]);
    }
    int64_t lo = std::max(big, (sum + wg_x - 1) / wg_x), hi = std::max(lo, sum);
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo) / 2;
      if (pack(mid, nullptr) <= wg_x)
        hi = mid;
      else
        lo = mid + 1;
    }
    std::vector<int64_t> bounds;
    pack(lo, &bounds);
    for (size_t k = 0; k + 1 < bounds.size(); ++k) {
      std::vector<BatchEntry> bl;  // this workgroup's batches in row order
      for (int64_t i = bounds[k]; i < bounds[k + 1]; ++i)
        for (int64_t j = 0; j < nb[i]; ++j) {
          const int32_t kb = (int32_t)(ptr[i] + j * kBatchEdges);
          const int32_t cnt = std::max(0, std::min<int32_t>(kBatchEdges, ptr[i + 1] - kb));
          bl.push_back({(int32_t)i, kb, cnt, 0});
        }
      const size_t n = bl.size();
      std::vector<size_t> wb(waves + 1);
      for (int w = 0; w <= waves; ++w) wb[w] = n * (size_t)w / (size_t)waves;
      int pieces = 0;
      for (int w = 0; w < waves; ++w) {
        const size_t b0 = wb[w], b1 = wb[w + 1];
        if (b0 == b1) continue;
        for (size_t b = b0; b < b1; ++b) {
          if (b == b0 || bl[b - 1].row != bl[b].row) bl[b].info |= kInfoFirstBit;
          if (b + 1 == b1 || bl[b + 1].row != bl[b].row) bl[b].info |= kInfoLastBit;
        }
        // the first segment continues a row of the previous wave, the last
        // segment continues into the next wave: those segments are pieces
        size_t f1 = b0;
        while (f1 < b1 && bl[f1].row == bl[b0].row) ++f1;
        size_t l0 = b1;
        while (l0 > b0 && bl[l0 - 1].row == bl[b1 - 1].row) --l0;
        const bool piece_first = b0 > 0 && bl[b0 - 1].row == bl[b0].row;
        const bool piece_last = b1 < n && bl[b1].row == bl[b1 - 1].row;
        auto mark = [&](size_t e0, size_t e1) {
          for (size_t b = e0; b < e1; ++b) bl[b].info |= kInfoPieceBit | pieces;
          ++pieces;
        };
        if (piece_first) mark(b0, f1);
        if (piece_last && !(piece_first && l0 == b0)) mark(l0, b1);
      }
      // the last piece of each split row (highest number among the row's
      // consecutive piece numbers) carries the row's piece count
      if (pieces > 0) {
        std::vector<int> row_of(pieces, -1);
        std::vector<size_t> at(pieces, 0);
        for (size_t b = 0; b < n; ++b)
          if ((bl[b].info & kInfoPieceBit) && (bl[b].info & kInfoFirstBit)) {
            const int q = bl[b].info & kInfoSlotMask;
            row_of[q] = bl[b].row;
            at[q] = b;
          }
        for (int q = 0; q < pieces; ++q) {
          const bool last_of_row = q + 1 == pieces || row_of[q + 1] != row_of[q];
          if (!last_of_row) continue;
          int q0 = q;
          while (q0 > 0 && row_of[q0 - 1] == row_of[q]) --q0;
          const int np = q - q0 + 1;
          for (size_t b = at[q]; b < n && bl[b].row == row_of[q] && (bl[b].info & kInfoPieceBit) &&
                                 (bl[b].info & kInfoSlotMask) == q;
               ++b)
            bl[b].info |= kInfoCombineBit | (np << kInfoCountShift);
        }
        for (auto& e : bl) e.info |= kInfoGroupBit;
      }
      for (int w = 0; w < waves; ++w) {
        auto& lst = lists[((size_t)k * kXcds + x) * waves + w];
        lst.assign(bl.begin() + wb[w], bl.begin() + wb[w + 1]);
        // an empty wave of a workgroup with pieces must still reach its barrier
        if (lst.empty() && pieces > 0) lst.push_back({-1, 0, 0, kInfoGroupBit});
      }
    }
  }
  size_t KB = 1;
  for (const auto& l : lists) KB = std::max(KB, l.size());
  const int num_wgs = wg_x * kXcds;
  out->table.assign((size_t)num_wgs * waves * KB, BatchEntry{-1, 0, 0, 0});
  for (size_t v = 0; v < lists.size(); ++v)
    std::copy(lists[v].begin(), lists[v].end(), out->table.begin() + v * KB);
  out->num_wgs = num_wgs;
  out->waves = waves;
  out->KB = (int)KB;
}


// Resident plan (see schedule.h).  For a piece length D, row i has
// p_i = ceil(d_i / D) pieces (none for an empty row, whose owner still runs
// its epilogue).  The rows are cut greedily into contiguous ranges of at most
// `cap` pieces and kResLanes rows; bisection finds the smallest cap that needs
// at most `ranks` ranges.
namespace {

bool pack_ranges(const std::vector<int64_t>& pc, int ranks, int64_t cap, std::vector<int32_t>* cut) {
  const int64_t N = (int64_t)pc.size();
  if (cut) cut->assign(1, 0);
  int used = 1;
  int64_t pieces = 0, rows = 0;
  for (int64_t i = 0; i < N; ++i) {
    if (pc[i] > cap) return false;
    if (pieces + pc[i] > cap || rows + 1 > kResLanes) {
      if (++used > ranks) return false;
      if (cut) cut->push_back((int32_t)i);
      pieces = 0;
      rows = 0;
    }
    pieces += pc[i];
    ++rows;
  }
  if (cut) {
    while ((int)cut->size() < ranks + 1) cut->push_back((int32_t)N);
  }
  return true;
}

}  // namespace

bool plan_resident(const int32_t* ptr, int64_t N, int ranks, int max_D, bool every_wave_gathers,
                   ResidentPlan* out) {
  if (ranks <= 0 || N <= 0) return false;
  int best_D = 0;
  int64_t best_cap = 0, best_cost = -1;
  std::vector<int64_t> pc(N);
  for (int li = 0; li < kResNumPieceLens; ++li) {
    const int D = kResPieceLens[li];
    if (D > max_D) continue;
    int64_t lo = 0;
    for (int64_t i = 0; i < N; ++i) {
      pc[i] = (ptr[i + 1] - ptr[i] + D - 1) / D;
      lo = std::max(lo, pc[i]);
    }
    if (!pack_ranges(pc, ranks, kResLanes, nullptr)) continue;
    int64_t hi = kResLanes;
    while (lo < hi) {
      const int64_t mid = (lo + hi) / 2;
      if (pack_ranges(pc, ranks, mid, nullptr)) hi = mid;
      else lo = mid + 1;
    }
    const int64_t cost = every_wave_gathers ? (int64_t)D * kResLanes + hi : hi * (D + 4);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best_cap = hi;
      best_D = D;
    }
  }
  if (best_cost < 0) return false;
  const int D = best_D;
  for (int64_t i = 0; i < N; ++i) pc[i] = (ptr[i + 1] - ptr[i] + D - 1) / D;
  ResidentPlan& p = *out;
  p = ResidentPlan();
  p.D = D;
  p.ranks = ranks;
  pack_ranges(pc, ranks, best_cap, &p.rank_rows);
  p.owner_pbeg.assign((size_t)ranks * (kResLanes + 1), 0);
  p.piece_row.assign((size_t)ranks * kResLanes, -1);
  p.piece_kbeg.assign((size_t)ranks * kResLanes, 0);
  p.piece_cnt.assign((size_t)ranks * kResLanes, 0);
  for (int r = 0; r < ranks; ++r) {
    const int32_t r0 = p.rank_rows[r], r1 = p.rank_rows[r + 1];
    int32_t* pb = &p.owner_pbeg[(size_t)r * (kResLanes + 1)];
    int lane = 0;
    for (int32_t i = r0; i < r1; ++i) {
      pb[i - r0] = lane;
      for (int32_t k = ptr[i]; k < ptr[i + 1]; k += D, ++lane) {
        const size_t q = (size_t)r * kResLanes + lane;
        p.piece_row[q] = i;
        p.piece_kbeg[q] = k;
        p.piece_cnt[q] = std::min<int32_t>(D, ptr[i + 1] - k);
      }
    }
    for (int o = r1 - r0; o <= kResLanes; ++o) pb[o] = lane;
    p.max_pieces = std::max(p.max_pieces, lane);
  }
  p.slot_edge.assign((size_t)ranks * D * kResLanes, -1);
  for (int r = 0; r < ranks; ++r)
    for (int l = 0; l < kResLanes; ++l) {
      const size_t q = (size_t)r * kResLanes + l;
      for (int j = 0; j < p.piece_cnt[q]; ++j)
        p.slot_edge[((size_t)r * D + j) * kResLanes + l] = p.piece_kbeg[q] + j;
    }
  return true;
}

namespace {

// Distinct rows sharing the most-shared bank group among `rows` (-1 = none).
int group_cost(const int32_t* rows, int n) {
  int cnt[kResBankGroups] = {0};
  int best = 0;
  for (int a = 0; a < n; ++a) {
    if (rows[a] < 0) continue;
    bool dup = false;
    for (int b = 0; b < a && !dup; ++b) dup = rows[b] == rows[a];
    if (dup) continue;
    best = std::max(best, ++cnt[rows[a] % kResBankGroups]);
  }
  return best;
}

}  // namespace

int64_t resident_conflict_cost(const int32_t* col, int64_t N, const ResidentPlan& p) {
  int64_t cost = 0;
  int32_t rows[kResBankGroups];
  for (int r = 0; r < p.ranks; ++r)
    for (int j = 0; j < p.D; ++j)
      for (int g = 0; g < kResLanes; g += kResBankGroups) {
        bool any = false;
        for (int u = 0; u < kResBankGroups; ++u) {
          const int32_t e = p.slot_edge[((size_t)r * p.D + j) * kResLanes + g + u];
          rows[u] = e >= 0 ? col[e] : (int32_t)N - 1 - e;
          any = any || e >= 0;
        }
        if (any) cost += group_cost(rows, kResBankGroups);
      }
  return cost;
}

void assign_min_cost(const int* cost, int n, int* col_of_row) {
  constexpr int kInf = 1 << 29;
  std::vector<int> pu(n + 1, 0), pv(n + 1, 0), row_of(n + 1, 0), way(n + 1, 0), minv(n + 1);
  std::vector<char> used(n + 1);
  for (int i = 1; i <= n; ++i) {
    row_of[0] = i;
    int j0 = 0;
    std::fill(minv.begin(), minv.end(), kInf);
    std::fill(used.begin(), used.end(), 0);
    do {
      used[j0] = 1;
      const int i0 = row_of[j0];
      int delta = kInf, j1 = 0;
      for (int j = 1; j <= n; ++j) {
        if (used[j]) continue;
        const int cur = cost[(i0 - 1) * n + (j - 1)] - pu[i0] - pv[j];
        if (cur < minv[j]) {
          minv[j] = cur;
          way[j] = j0;
        }
        if (minv[j] < delta) {
          delta = minv[j];
          j1 = j;
        }
      }
      for (int j = 0; j <= n; ++j) {
        if (used[j]) {
          pu[row_of[j]] += delta;
          pv[j] -= delta;
        } else {
          minv[j] -= delta;
        }
      }
      j0 = j1;
    } while (row_of[j0] != 0);
    do {
      const int j1 = way[j0];
      row_of[j0] = row_of[j1];
      j0 = j1;
    } while (j0 != 0);
  }
  for (int j = 1; j <= n; ++j) col_of_row[row_of[j] - 1] = j - 1;
}

void order_resident_slots(const int32_t* col, int64_t N, ResidentPlan* out) {
  ResidentPlan& p = *out;
  const int D = p.D;
  constexpr int G = kResBankGroups;
  constexpr int W = 64;                 // lanes per wave
  constexpr int kEdge = 10, kEmpty = 9;  // what a lane can offer a bank group
  const int zero_group = (int)(N % G);  // bank group of zero row N
  std::vector<int32_t> left[W][G];      // per lane: its remaining edges by bank group
  p.order_misses = 0;
  for (int r = 0; r < p.ranks; ++r)
    for (int w0 = 0; w0 < kResLanes; w0 += W) {
      int empty[W];
      bool any = false;
      for (int u = 0; u < W; ++u) {
        for (int b = 0; b < G; ++b) left[u][b].clear();
        const size_t q = (size_t)r * kResLanes + w0 + u;
        for (int j = 0; j < p.piece_cnt[q]; ++j) {
          const int32_t e = p.piece_kbeg[q] + j;
          left[u][col[e] % G].push_back(e);
        }
        empty[u] = D - p.piece_cnt[q];
        any = any || p.piece_cnt[q] > 0;
      }
      if (!any) continue;  // a wave without pieces keeps reading zero row N
      for (int j = 0; j < D; ++j) {
        int cost[G * G];
        for (int c = 0; c < G; ++c)
          for (int b = 0; b < G; ++b) {
            int offer = 0;
            for (int u = c; u < W; u += G)
              offer += !left[u][b].empty() ? kEdge : (empty[u] > 0 ? kEmpty : 0);
            cost[c * G + b] = (W / G) * kEdge - offer;
          }
        int perm[G];
        assign_min_cost(cost, G, perm);
        for (int u = 0; u < W; ++u) {
          int32_t& slot = p.slot_edge[((size_t)r * D + j) * kResLanes + w0 + u];
          int b = perm[u % G];
          if (left[u][b].empty()) {
            if (empty[u] > 0) {
              --empty[u];
              slot = -1 - (b - zero_group + G) % G;
              continue;
            }
            for (int k = 0; k < G; ++k)
              if (left[u][k].size() > left[u][b].size()) b = k;
            ++p.order_misses;
          }
          slot = left[u][b].back();
          left[u][b].pop_back();
        }
      }
    }
}

bool plan_blocked(const int32_t* ptr, const int32_t* col, int64_t N, int num_cus,
                  BlockedPlan* out) {
  if (num_cus <= 0 || num_cus % kBlkBlocks != 0 || N < 0) return false;
  BlockedPlan& p = *out;
  p = BlockedPlan();
  p.num_wgs = num_cus;
  const int64_t bs = std::max<int64_t>(1, (N + kBlkBlocks - 1) / kBlkBlocks);
  // items, numbered row by row
  std::vector<std::vector<BlkItem>> per(kBlkBlocks);
  p.row_items.assign(N + 1, 0);
  int64_t id = 0;
  for (int64_t i = 0; i < N; ++i) {
    p.row_items[i] = (int32_t)id;
    int64_t k = ptr[i];
    while (k < ptr[i + 1]) {
      const int64_t x = col[k] / bs;
      int64_t e = k;
      while (e < ptr[i + 1] && col[e] / bs == x) ++e;
      for (int64_t c = k; c < e; c += kBlkChunk) {
        if (id >= (int64_t)INT32_MAX) return false;
        per[x].push_back(BlkItem{(int32_t)i, (int32_t)c,
                                 (int32_t)std::min<int64_t>(kBlkChunk, e - c), (int32_t)id++});
      }
      k = e;
    }
  }
  p.row_items[N] = (int32_t)id;
  p.items = id;
  // deal each block's items to the waves of its workgroups
  const int wgs_per = num_cus / kBlkBlocks;
  const int nw = wgs_per * kBlkWaves;  // waves per block
  std::vector<std::vector<std::vector<BlkItem>>> lists(kBlkBlocks);
  size_t KB = 0;
  for (int x = 0; x < kBlkBlocks; ++x) {
    std::vector<BlkItem>& it = per[x];
    std::stable_sort(it.begin(), it.end(),
                     [](const BlkItem& a, const BlkItem& b) { return a.count > b.count; });
    lists[x].assign(nw, {});
    // min-heap of (cost so far, wave)
    std::vector<std::pair<int64_t, int>> heap;
    for (int w = 0; w < nw; ++w) heap.emplace_back(0, w);
    auto later = [](const std::pair<int64_t, int>& a, const std::pair<int64_t, int>& b) {
      return a > b;
    };
    std::make_heap(heap.begin(), heap.end(), later);
    for (const BlkItem& item : it) {
      std::pop_heap(heap.begin(), heap.end(), later);
      auto& top = heap.back();
      lists[x][top.second].push_back(item);
      top.first += item.count + kBlkItemCost;
      std::push_heap(heap.begin(), heap.end(), later);
    }
    for (const auto& l : lists[x]) KB = std::max(KB, l.size());
  }
  p.KB = (int)KB;
  // wave v = b * kBlkWaves + w of workgroup b serves block b % kBlkBlocks as
  // that block's wave (b / kBlkBlocks) * kBlkWaves + w
  const size_t stride = KB + kBlkPad;
  p.table.assign((size_t)num_cus * kBlkWaves * stride, BlkItem{-1, 0, 0, 0});
  p.edge_order.assign(ptr[N], 0);
  p.item_ids.assign(id, 0);
  // Positions (of edges and of partial rows) go group by group of kBlkGroup
  // items: all waves' first groups, then all waves' second groups, ... so the
  // waves, which walk their lists at about the same pace, read and write
  // nearby memory at any moment.
  int64_t pos = 0, walk = 0;
  for (size_t g0 = 0; g0 < KB; g0 += kBlkGroup)
    for (int b = 0; b < num_cus; ++b)
      for (int w = 0; w < kBlkWaves; ++w) {
        const auto& l = lists[b % kBlkBlocks][(b / kBlkBlocks) * kBlkWaves + w];
        BlkItem* t = &p.table[((size_t)b * kBlkWaves + w) * stride];
        for (size_t q = g0; q < std::min(l.size(), g0 + kBlkGroup); ++q) {
          t[q] = l[q];
          t[q].kbeg = (int32_t)pos;
          t[q].id = (int32_t)walk;
          p.item_ids[l[q].id] = (int32_t)walk++;  // (l[q].id: the item's number row by row)
          for (int32_t j = 0; j < l[q].count; ++j) p.edge_order[pos++] = l[q].kbeg + j;
        }
      }
  return true;
}

}  // namespace ckhip
