// ck_internal.h -- library-internal declarations shared by the HIP sources.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

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
