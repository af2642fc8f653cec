// schedule.h -- the row schedule of one orientation of the graph: which
// edge batches each wave of the per-microstep kernels walks.  Plain C++ (no
// HIP calls), so that the CPU tests can build and check it on its own.
#pragma once

#include <cstdint>
#include <vector>

#ifdef __HIPCC__
#define CK_HOST_DEVICE __host__ __device__
#else
#define CK_HOST_DEVICE
#endif

namespace ckhip {

// Workgroup shapes of the per-microstep kernels.  A kernel whose row width
// (L lanes of float4 per row) keeps it within 128 VGPRs runs 16-wave
// workgroups, one per CU; the others run 8-wave workgroups, two per CU when
// their registers allow.  Either way the schedule is sized for 16 resident
// waves per CU, i.e. one round of workgroups.
constexpr int kWavesPerCu = 16;
CK_HOST_DEVICE constexpr int waves_for_lanes(int L) {
  return (L <= 8 && (L & (L - 1)) == 0) ? 16 : 8;
}
constexpr int kMaxWaves = 16;
// Workgroups are dispatched round-robin over the 8 XCDs of an MI355X.
constexpr int kXcds = 8;

// Row schedule of one orientation of the graph for one workgroup width W, as
// edge batches.  Wave v (= workgroup * W + wave index) walks
// batches[v * KB .. v * KB + KB) in order until an entry with row < 0.
// Entry = {row, kbeg, count, info}: edges [kbeg, kbeg + count) (count <=
// kBatchEdges) of the row's compressed list.  (The uploaded device table
// replaces kbeg by the row's input slot, or -1, once the padded edge slots
// are built from it.)  Consecutive batches of one row on
// one wave form a segment; a row whose batches fall on several waves (always
// of one workgroup) is split into pieces, one segment per wave.  A piece is a
// wave's first or last segment, so a workgroup holds at most 2 W pieces; they
// are numbered in row order, so the pieces of one row have consecutive
// numbers, and the last piece of a row is the first segment of its wave.
//   info bits 0..5: piece number (LDS slot of the piece's partial sum);
//   bits 6..11: on the last piece of a row, the row's number of pieces;
//   bit 12: last piece of its row (its wave sums the row's pieces, in piece
//   order, after the workgroup barrier and runs the row's epilogue);
//   bit 16: the workgroup holds pieces (all its waves synchronise once at the
//   end); bit 17: this batch belongs to a piece; bit 18: first batch of its
//   segment; bit 19: last batch of its segment.
constexpr int kBatchEdges = 64;
constexpr int kInfoSlotMask = 63;
constexpr int kInfoCountShift = 6;
constexpr int kInfoCombineBit = 1 << 12;
constexpr int kInfoGroupBit = 1 << 16;
constexpr int kInfoPieceBit = 1 << 17;
constexpr int kInfoFirstBit = 1 << 18;
constexpr int kInfoLastBit = 1 << 19;
// One batch entry; the same 16-byte layout as the int4 the kernels read.
struct BatchEntry {
  int32_t row, kbeg, count, info;
};

// The table of one schedule: wave v (= workgroup * waves + wave index) owns
// entries [v * KB, v * KB + KB), padded with row = -1.
struct SchedulePlan {
  std::vector<BatchEntry> table;
  int num_wgs = 0;
  int waves = 0;
  int KB = 0;
};

// Plan the schedule of a compressed row structure ptr[0..N] (row i holds edges
// [ptr[i], ptr[i+1])) for workgroups of `waves` waves on `num_cus` compute
// units.
void plan_schedule(const int32_t* ptr, int64_t N, int num_cus, int waves, SchedulePlan* out);

// ---------------------------------------------------------------------------
// Resident plan: the split of one orientation's rows over the `ranks`
// workgroups of one XCD for the XCD-resident kernels, which run every
// microstep of a call in one launch.  Each XCD computes all rows for its own
// group of batch columns, so all XCDs share one plan.
//
// A row of degree d is cut into ceil(d / D) pieces of at most D consecutive
// edges; each piece is held by one thread (lane) of a workgroup of kResLanes
// threads, in registers, for the whole launch.  Rows are cut into contiguous
// workgroup ranges; inside a range, the pieces of its rows take consecutive
// lanes in row order, and the row's "owner" (the range's o-th row is owned by
// lane o) forms the row's sum from its pieces' partial sums: a segmented scan
// across each 64-lane wave leaves the sum of the row's pieces in that wave at
// the last of them, and the owner adds these in wave order.
constexpr int kResLanes = 1024;
// Piece lengths the kernels are built for.
constexpr int kResPieceLens[] = {8, 12, 16, 18, 20, 24};
constexpr int kResNumPieceLens = 6;
constexpr int kResFwdMaxD = 24;
// The backward kernel also keeps D edge-gradient sums per lane; past D = 20
// it no longer fits in 128 registers.
constexpr int kResBwdMaxD = 20;

struct ResidentPlan {
  int D = 0;                        // edges per piece
  int ranks = 0;                    // workgroups per XCD
  int max_pieces = 0;               // pieces on the busiest workgroup
  int64_t order_misses = 0;         // slots off their wave's bank-group permutation
                                    // (set by order_resident_slots)
  std::vector<int32_t> rank_rows;   // [ranks + 1]: rows of workgroup r are [rank_rows[r], rank_rows[r+1])
  std::vector<int32_t> owner_pbeg;  // [ranks][kResLanes + 1]: the pieces of the r-th range's row o
                                    // are lanes [owner_pbeg[o], owner_pbeg[o+1]); constant past the range
  std::vector<int32_t> piece_row;   // [ranks][kResLanes]: row of the lane's piece, or -1
  std::vector<int32_t> piece_kbeg;  // [ranks][kResLanes]: first edge (compressed index) of the piece
  std::vector<int32_t> piece_cnt;   // [ranks][kResLanes]: edges in the piece (0 if none)
  std::vector<int32_t> slot_edge;   // [ranks][D][kResLanes]: edge of slot j of lane l, or
                                    // -1 - z for an empty slot, which reads zero row N + z
                                    // (compressed order and z = 0 unless order_resident_slots ran)
};

// LDS rows are 16 bytes; a row's bank group is its index mod kResBankGroups.
// Measured on gfx950: a wave's 16-byte-per-lane read runs at full rate when
// lanes l, l + 16, l + 32 and l + 48 read rows of one bank group and the 16
// lanes of each 16-lane group read 16 different bank groups (one permutation
// of bank groups shared by the wave's four 16-lane groups); distinct bank
// groups chosen separately per 16-lane group run at about 70 % of that rate,
// random rows at about 45 %.
constexpr int kResBankGroups = 16;
// Each plane ends with this many all-zero rows (N, N + 1, ...), one per bank
// group, so that an empty slot can read the bank group its slot wants.
constexpr int kResZeroRows = 16;

// Minimum-cost perfect assignment of the rows of an n x n integer cost
// matrix (row-major, entries below 2^28) to distinct columns: the Hungarian
// method with row and column potentials and shortest augmenting paths,
// O(n^3).  Writes col_of_row[0..n).
void assign_min_cost(const int* cost, int n, int* col_of_row);

// Order the edges inside each piece (slot j of lane l) for the rule above:
// per wave and slot, the permutation of bank groups over the 16 lane classes
// (lane mod 16) that the most lanes can follow (an assignment problem,
// solved exactly: an edge left in that bank group counts more than an empty
// slot), then each lane takes an edge in its class's bank group, else an
// empty slot (the zero row of that bank group), else an edge of its most
// frequent remaining bank group (a miss, counted in out->order_misses).
// col[k] is the row read by compressed edge k.  Fills out->slot_edge.
void order_resident_slots(const int32_t* col, int64_t N, ResidentPlan* out);

// Bank-conflict cost of a slot table: over all slots and 16-lane groups, the
// sum of the largest number of distinct rows sharing one bank group (1 = no
// conflict).  Used to compare orderings.
int64_t resident_conflict_cost(const int32_t* col, int64_t N, const ResidentPlan& p);

// Plan the pieces of ptr[0..N] for `ranks` workgroups, choosing the piece
// length D among kResPieceLens up to max_D.  When only the waves holding
// pieces gather (the forward), D minimises the busiest workgroup's
// pieces x (D + 4), an estimate of its gather work plus the owners'
// combining; when every wave gathers (the backward), the smallest D that
// fits wins (fewer pieces on a tie).  Returns false when no length fits (a
// range needs more than kResLanes pieces or rows).
bool plan_resident(const int32_t* ptr, int64_t N, int ranks, int max_D, bool every_wave_gathers,
                   ResidentPlan* out);

// ---------------------------------------------------------------------------
// Blocked plan: the per-microstep kernels of graphs whose state plane is far
// larger than the L2 caches.  The gathered nodes (the far end of each edge:
// the source in the forward, the destination in the backward) are cut into
// kBlkBlocks contiguous blocks of ceil(N / kBlkBlocks) nodes, one per XCD:
// the workgroups of XCD x gather rows of block x only, so that block's slice
// of the plane stays in that XCD's L2.  A row's edges into one block are one
// contiguous run (each row's edges are sorted by gathered node); the run is
// cut into work items of at most kBlkChunk edges.  An item leaves one partial
// sum row; a second kernel adds each row's partials in item order.
constexpr int kBlkBlocks = 8;
constexpr int kBlkChunk = 64;
constexpr int kBlkWaves = 16;  // waves per workgroup (one workgroup per CU)
// Balancing cost of an item in edge units: its edges plus this much for
// loading the item and storing its partial row.
constexpr int kBlkItemCost = 8;
// Padding entries (row = -1) after each wave's list: at least the widest pass
// (64 items), so a wave may read the pass after its last one.
constexpr int kBlkPad = 64;
// Items per group of the blocked layout (see edge_order).
constexpr int kBlkGroup = 8;

// One work item: `count` edges of `row`, at positions [kbeg, kbeg + count)
// of the blocked edge order (below); its partial row is number `id` (in the
// same order as the edges).  The
// same 16-byte layout as the int4 the kernels read; row = -1 pads a wave's
// list.
struct BlkItem {
  int32_t row, kbeg, count, id;
};

struct BlockedPlan {
  int num_wgs = 0;    // workgroup b serves block b % kBlkBlocks
  int KB = 0;         // items of the longest wave list (shorter lists padded with row = -1)
  int64_t items = 0;
  // Row i's items, blocks ascending and chunks ascending, are entries
  // [row_items[i], row_items[i+1]) of item_ids, which gives each one's id.
  std::vector<int32_t> row_items;  // [N + 1]
  std::vector<int32_t> item_ids;   // [items]
  std::vector<BlkItem> table;      // [num_wgs * kBlkWaves][KB + kBlkPad]: wave v's items, largest first
  // [E] the blocked edge order: position q holds compressed edge
  // edge_order[q].  Items are laid out in groups of kBlkGroup consecutive
  // items of one wave's list (their edges side by side), the first group of
  // every wave, then the second group of every wave, and so on; item ids
  // (partial rows) follow the same order.
  std::vector<int32_t> edge_order;
};

// Plan the blocked schedule of a compressed row structure ptr[0..N] whose
// edge k reads node col[k] (ascending within each row) for num_cus
// workgroups of kBlkWaves waves.  Each block's items are dealt to the waves
// of its workgroups largest first, each to the wave with the least cost so
// far (edges plus kBlkItemCost per item); a wave walks its items largest
// first, 64 / L at a time.  Returns false when num_cus is not a positive
// multiple of kBlkBlocks or the ids would overflow 32 bits.
bool plan_blocked(const int32_t* ptr, const int32_t* col, int64_t N, int num_cus,
                  BlockedPlan* out);

}  // namespace ckhip
