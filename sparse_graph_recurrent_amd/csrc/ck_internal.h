// ck_internal.h -- library-internal declarations shared by the HIP sources.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "ck.h"

namespace ckhip {

// Tuning constants (compile-time; -D overrides exist for sweeps only).
#ifndef CK_WAVES
#define CK_WAVES 8
#endif
#ifndef CK_SPLIT_EDGES
#define CK_SPLIT_EDGES 128
#endif
#ifndef CK_WGS_PER_CU
#define CK_WGS_PER_CU 2
#endif
// Workgroup shape of the per-microstep kernels: kWaves wave64s.
constexpr int kWaves = CK_WAVES;
constexpr int kThreads = kWaves * 64;
// A row is split into pieces (at most kWaves, all in one workgroup) when it
// holds more than max(kSplitEdges, per-wave share) edges.
constexpr int kSplitEdges = CK_SPLIT_EDGES;
// Workgroups per CU the schedule is sized for (one resident round).
constexpr int kWgsPerCu = CK_WGS_PER_CU;
// Workgroups are dispatched round-robin over the 8 XCDs of an MI355X.
constexpr int kXcds = 8;

// Row schedule of one orientation of the graph, as edge batches.  Wave v
// (= workgroup * kWaves + wave index) walks batches[v * KB .. v * KB + KB) in
// order until an entry with row < 0.  Entry = {row, kbeg, count, info}: edges
// [kbeg, kbeg + count) (count <= kBatchEdges) of the row's compressed list.
// A row is one or more consecutive batches of one wave ("segment"), or pieces
// on several waves of one workgroup (split row).
//   info bits 0..7: for a piece of a split row, the wave (inside the
//   workgroup) that combines the pieces; bits 8..15: number of pieces;
//   bit 16: the workgroup holds split rows (all its waves synchronise once at
//   the end); bit 17: this batch belongs to a piece (always a wave's first
//   segment); bit 18: first batch of its segment; bit 19: last batch of its
//   segment (the row, or the piece, is complete after it).
constexpr int kBatchEdges = 64;
constexpr int kInfoGroupBit = 1 << 16;
constexpr int kInfoPieceBit = 1 << 17;
constexpr int kInfoFirstBit = 1 << 18;
constexpr int kInfoLastBit = 1 << 19;
struct Schedule {
  int4* batches = nullptr;  // [num_wgs * kWaves * KB]
  int num_wgs = 0;
  int KB = 0;               // batch entries per wave (padded with row = -1)
};

}  // namespace ckhip

struct ck_graph {
  uint32_t magic;
  int device;
  int64_t N, E, n_in;
  int32_t* row_ptr;    // [N+1] CSR by destination
  int32_t* col_idx;    // [E] source of each CSR edge
  int32_t* perm;       // [E] caller index of each CSR edge
  int32_t* t_row_ptr;  // [N+1] CSR by source (transposed)
  int32_t* t_col_idx;  // [E] destination of each transposed edge
  int32_t* t_perm;     // [E] caller index of each transposed edge
  int32_t* input_slot; // [N] k if the node is input_nodes[k], else -1
  ckhip::Schedule fwd; // rows of the CSR (in-degree)
  ckhip::Schedule bwd; // rows of the transposed CSR (out-degree)
};

namespace ckhip {

constexpr uint32_t kGraphMagic = 0x434B4731u;  // "CKG1"

void set_error(const char* fmt, ...);
void clear_error();
ck_status check_graph(const ck_graph* g);

}  // namespace ckhip

#define CK_HIP_TRY(expr)                                                            \
  do {                                                                              \
    hipError_t ck_e_ = (expr);                                                      \
    if (ck_e_ != hipSuccess) {                                                      \
      ckhip::set_error("%s failed: %s (%s:%d)", #expr, hipGetErrorString(ck_e_),    \
                       __FILE__, __LINE__);                                         \
      return ck_e_ == hipErrorOutOfMemory ? CK_ERR_NOMEM : CK_ERR_HIP;              \
    }                                                                               \
  } while (0)
