// ck_internal.h -- library-internal declarations shared by the HIP sources.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "ck.h"

namespace ckhip {

// Workgroup shape of every hot-path kernel: 4 wave64s.
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
// Rows with more edges than this are split across all waves of a workgroup.
constexpr int kLongRow = 256;
// Workgroups are dispatched round-robin over the 8 XCDs of an MI355X.
constexpr int kXcds = 8;

// A degree-balanced row schedule for one orientation of the graph.
//   items[w] = {first, count} for workgroup w: count == -1 -> one long row
//   rows[first] split across the waves; count in 1..kWaves -> wave i takes
//   rows[first + i]; count == 0 -> nothing to do (padding).
struct Schedule {
  int2* items = nullptr;
  int32_t* rows = nullptr;
  int num_items = 0;
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
