// ck_internal.h -- library-internal declarations shared by the HIP sources.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <utility>
#include <vector>

#include "ck.h"
#include "schedule.h"

namespace ckhip {

struct Schedule {
  int4* batches = nullptr;  // [num_wgs * waves * KB]
  int32_t* pcol = nullptr;  // [slots] column of edge k of entry t at t * kBatchEdges + k, or -1
  int32_t* pperm = nullptr; // [slots] caller index of that edge, or -1
  int64_t slots = 0;        // num_wgs * waves * KB * kBatchEdges
  int num_wgs = 0;
  int waves = 0;            // waves per workgroup
  int KB = 0;               // batch entries per wave (padded with row = -1)
};

// Device copy of a BlockedPlan (see schedule.h).
struct Blocked {
  int4* table = nullptr;         // [num_wgs * kBlkWaves][KB + kBlkPad] items {row, kbeg, count, id}
  int32_t* row_items = nullptr;  // [N + 1]: row i's items are item_ids[row_items[i] ..]
  int32_t* item_ids = nullptr;   // [items] partial row of each of a row's items
  int32_t* pnode = nullptr;      // [E] gathered node of the edge at each blocked position
  int32_t* pperm = nullptr;      // [E] caller index of that edge
  int num_wgs = 0;
  int KB = 0;
  int64_t items = 0;
};
// Graphs of at least this many nodes get a blocked plan of the forward at
// creation (CK_BLOCKED: "0" none, "1" the forward's for any graph, "2" both
// directions' for any graph).  Below it the per-microstep kernels' gathers
// mostly hit the L2s already.  The backward keeps the per-microstep kernels
// unless CK_BLOCKED is "2": at whole-connectome size they are faster there
// (416 against 371 + 74 µs per microstep) and sum the edge gradient more
// accurately.
constexpr int64_t kBlkMinN = 100000;

// Largest node count of the XCD-resident kernels: one workgroup holds a
// whole [N + kResZeroRows] x 16-byte state plane plus kResLanes 16-byte partial sums in
// the 160 KiB of LDS of a gfx950 compute unit.
constexpr int64_t kResMaxN = 9184;
// XCDs of an MI355X; a launch deals its workgroups round-robin over them.
constexpr int kResXcds = 8;

// Hardware id of the XCD (accelerator complex die) the calling wave runs on.
__device__ __forceinline__ unsigned xcc_id() {
  unsigned x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  return x & 15u;
}

// Device copy of a ResidentPlan (see schedule.h) with its padded edge slots:
// slot (r, j, l) = ((r * D) + j) * kResLanes + l holds edge j of lane l's
// piece on workgroup r (coalesced per j when the lanes load their pieces).
struct Resident {
  int D = 0;
  int ranks = 0;
  int32_t* rank_rows = nullptr;   // [ranks + 1]
  int32_t* owner_pbeg = nullptr;  // [ranks][kResLanes + 1]
  int32_t* piece_row = nullptr;   // [ranks][kResLanes], -1 for a lane without a piece
  int32_t* pcol = nullptr;        // [slots] node at the other end of the edge, or N + z (all-zero rows)
  int32_t* pperm = nullptr;       // [slots] caller index of the edge, or -1
  int64_t slots = 0;              // ranks * D * kResLanes
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
  ckhip::Schedule fwd[2]; // rows of the CSR (in-degree), for 8- and 16-wave workgroups
  ckhip::Schedule bwd[2]; // rows of the transposed CSR (out-degree), likewise
  // XCD-resident kernels (one launch per call): usable when res_ok is set at
  // creation (the device has 8 XCDs of equal size, N fits the LDS-resident
  // plane, both orientations have a plan, and CK_RESIDENT is not "0").
  int res_ok;
  // polls before a resident kernel's wait gives up (CK_RESIDENT_SPIN_LIMIT
  // at creation, default 2^20 -- about a second; a negative value makes every
  // wait give up at once, which tests use to exercise the failure path)
  int res_spin_limit;
  ckhip::Resident res_fwd;  // rows of the CSR
  ckhip::Resident res_bwd;  // rows of the transposed CSR
  // blocked per-microstep kernels: the forward's when blk_ok is set at
  // creation, the backward's too when blk_bwd_ok is (see kBlkMinN and
  // CK_BLOCKED)
  int blk_ok;
  int blk_bwd_ok;
  ckhip::Blocked blk_fwd;   // rows of the CSR, items over source blocks
  ckhip::Blocked blk_bwd;   // rows of the transposed CSR, items over destination blocks
};

namespace ckhip {

constexpr uint32_t kGraphMagic = 0x434B4731u;  // "CKG1"

void set_error(const char* fmt, ...);
void clear_error();
ck_status check_graph(const ck_graph* g);

// `saved` and workspace buffers start on a 256-byte boundary (as hipMalloc
// and torch allocations do): the kernels address their parts with 16-byte
// vector accesses at offsets that are multiples of 256.
inline ck_status check_aligned(const void* p, const char* what) {
  if (reinterpret_cast<uintptr_t>(p) % 256 != 0) {
    set_error("%s does not start on a 256-byte boundary", what);
    return CK_ERR_BAD_VALUE;
  }
  return CK_OK;
}

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

namespace ckhip {

// Measurement hook state: HIP event pairs around the main kernel launches.
struct Profile {
  bool enabled = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> fwd, bwd, lif_gather, lif_update;
};
extern Profile g_profile;

// Launch `launch()` on `stream`, bracketed by events when profiling is on.
template <typename F>
ck_status timed_launch(std::vector<std::pair<hipEvent_t, hipEvent_t>>& log, hipStream_t stream,
                       F&& launch) {
  if (!g_profile.enabled) {
    launch();
    return CK_OK;
  }
  // timing-only events: no system-scope fence (cache writeback/invalidate)
  // around the kernel they bracket
  hipEvent_t a, b;
  CK_HIP_TRY(hipEventCreateWithFlags(&a, hipEventDisableSystemFence));
  CK_HIP_TRY(hipEventCreateWithFlags(&b, hipEventDisableSystemFence));
  CK_HIP_TRY(hipEventRecord(a, stream));
  launch();
  CK_HIP_TRY(hipEventRecord(b, stream));
  log.emplace_back(a, b);
  return CK_OK;
}

}  // namespace ckhip

namespace ckhip {

// Sizes of one call of the XCD-resident kernels: G = ceil(B / 4) column
// groups (at most kResXcds), Np = N rounded up to 8 rows (a group's plane
// slice is a whole number of 128-byte lines).
struct ResDims {
  int64_t N, Np, B, G, n_in, T, M, S;
};
// Workspace of the resident path, byte offsets.
struct ResWs {
  size_t pedge, h0, ctl, ga, gv, gl, gb, total;
};
// Allows the resident kernels their LDS (once per graph creation).
ck_status res_prepare();
ResWs res_ws_layout(const ck_graph* g, const ResDims& d);
size_t res_saved_bytes(const ResDims& d);
// Reads the error flag of the last resident call that used `workspace`
// (synchronises `stream`).
ck_status res_status(const ck_graph* g, const ResDims& d, const void* workspace,
                     hipStream_t stream, unsigned* err);
// Leading bytes of the workspace a resident forward uses.
size_t res_forward_ws_bytes(const ck_graph* g, const ResDims& d);
// profile: record the measurement hook's events around the main launch.
ck_status res_forward(const ck_graph* g, const ResDims& d, const float* edge_values,
                      const float* leak, const float* bias, const float* drives,
                      const float* state0, float* out, void* saved, void* workspace,
                      hipStream_t stream, bool profile);
// Resolves, once per device, the device address of the allocation-free
// forward's fixed scratch array (called at graph creation, with `device`
// current).
ck_status scratch_prepare(int device);
// Sizes of one call of the blocked kernels (8 <= Bp <= 64, L = Bp / 4).
struct BlkDims {
  int64_t N, E, n_in, T, B, M, S, Bp;
  int L;
  size_t plane;  // floats per [N][Bp] plane
};
// Workspace of the blocked path, byte offsets; a forward uses [0, fwd_end).
struct BlkWs {
  size_t pe, part, h0, fwd_end, gv, gh, ga0, ga1, gt, total;
};
BlkWs blk_ws_layout(const ck_graph* g, const BlkDims& d);
// True when the graph has blocked plans and a call of Bp padded columns fits
// them (8 <= Bp <= 64, buffer byte offsets below 2^32).
bool blk_fits(const ck_graph* g, int64_t Bp);
ck_status blk_forward(const ck_graph* g, const BlkDims& d, const float* edge_values,
                      const float* leak, const float* bias, const float* drives,
                      const float* state0, float* out, void* saved, void* workspace,
                      hipStream_t stream, bool profile);
ck_status blk_backward(const ck_graph* g, const BlkDims& d, const float* edge_values,
                       const float* leak, const float* state0, const void* saved,
                       const float* grad_out, float* grad_edge_values, float* grad_leak,
                       float* grad_bias, float* grad_drives, float* grad_state0,
                       void* workspace, hipStream_t stream);
// Plan and upload the blocked items of one orientation (row pointers ptr;
// gathered node col and caller index perm of each compressed edge, on the
// device); *planned is false when the device shape allows no plan.
ck_status build_blocked(const std::vector<int32_t>& ptr, int64_t N, const int32_t* col,
                        const int32_t* perm, int num_cus, hipStream_t stream, Blocked* out,
                        bool* planned);
void free_blocked(Blocked* b);

ck_status res_backward(const ck_graph* g, const ResDims& d, const float* edge_values,
                       const float* leak, const float* state0, const void* saved,
                       const float* grad_out, float* grad_edge_values, float* grad_leak,
                       float* grad_bias, float* grad_drives, float* grad_state0, void* workspace,
                       hipStream_t stream);

}  // namespace ckhip
