// lif.hip -- deterministic fixed-point leaky integrate-and-fire (LIF) forward
// on the graph handle's CSR by destination (soup-connectome page, "Runtime
// contract": signed int32 membrane potentials, signed int16 synaptic
// impulses, positive integer timestep delays, checked arithmetic with
// rejected overflow, the leak V := V - (V >> k); "Full-scale benchmark": the
// threshold, reset, decay shifts and refractory steps of a run).
//
// Per timestep t, for every neuron i (the update order is the one stated in
// include/ck.h at ck_lif_forward):
//   I = sum of the impulses w[e] of the in-edges e of i whose source spiked at
//       step t - d[e]  (the delay line read as a gather over the spike history)
//   refractory: drop I, count down; otherwise leak, add I (checked), spike at
//   the threshold, reset, start the refractory count.
// Two launches per step:
//   lif_gather   one thread per CSR position: the edge's impulse if its source
//                spiked d steps earlier; a segmented sum over each wave's run
//                of positions of one row, then one 64-bit integer atomic add
//                per run into I[row].  Integer sums are exact and associative,
//                so the result does not depend on the order of the atomics.
//   lif_update   one thread per neuron: the state update above; writes the
//                step's spikes and potentials, clears I.
// A per-call prologue packs {source, impulse, delay} into 8-byte records in
// CSR order (the caller's edge order stays invisible) with each position's
// destination beside it, and validates the delays.
#include <algorithm>
#include <climits>

#include "ck_internal.h"

namespace ckhip {
namespace {

// flags[0]: first timestep whose update left the int32 range (INT_MAX: none)
// flags[1]: set when a delay is outside [1, 32767]
constexpr int kLifFlags = 64;

struct LifWs {
  size_t rec, dst, acc, v, r, flags, total;
};

LifWs lif_layout(int64_t N, int64_t E) {
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  LifWs w;
  size_t o = 0;
  w.rec = o;   o = al(o + (size_t)std::max<int64_t>(E, 1) * 8);
  w.dst = o;   o = al(o + (size_t)std::max<int64_t>(E, 1) * 4);
  w.acc = o;   o = al(o + (size_t)N * 8);
  w.v = o;     o = al(o + (size_t)N * 4);
  w.r = o;     o = al(o + (size_t)N * 4);
  w.flags = o; o = al(o + kLifFlags * 4);
  w.total = o;
  return w;
}

__global__ void lif_init(const int32_t* __restrict__ v0, int64_t N, int32_t* __restrict__ v,
                         int32_t* __restrict__ r, long long* __restrict__ acc,
                         int32_t* __restrict__ flags) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < N) {
    v[i] = v0[i];
    r[i] = 0;
    acc[i] = 0;
  }
  if (i == 0) {
    flags[0] = INT_MAX;
    flags[1] = 0;
  }
}

// Record k of the CSR: {source node, impulse (low 16 bits) | delay << 16} and
// the destination of position k (the row whose range holds k).
__global__ void lif_pack(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
                         const int32_t* __restrict__ perm, const int16_t* __restrict__ impulses,
                         const int32_t* __restrict__ delays, int64_t N, int64_t E,
                         int2* __restrict__ rec, int32_t* __restrict__ dst,
                         int32_t* __restrict__ flags) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= E) return;
  const int32_t e = perm[k];
  const int32_t d = delays[e];
  if (d < 1 || d > 32767) atomicOr(&flags[1], 1);
  const uint32_t w = (uint16_t)impulses[e];
  rec[k] = make_int2(col_idx[k], (int)(w | ((uint32_t)(d & 0x7FFF) << 16)));
  // last row whose start is <= k (rows without edges share their start)
  int64_t lo = 0, hi = N;  // invariant: row_ptr[lo] <= k < row_ptr[hi]
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) >> 1;
    if (row_ptr[mid] <= k) lo = mid;
    else hi = mid;
  }
  dst[k] = (int32_t)lo;
}

__global__ __launch_bounds__(256) void lif_gather(const int2* __restrict__ rec,
                                                  const int32_t* __restrict__ dst, int64_t E,
                                                  int64_t N, int t,
                                                  const uint8_t* __restrict__ spikes,
                                                  long long* __restrict__ acc) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int lane = threadIdx.x & 63;
  int row = -1;
  long long c = 0;
  if (k < E) {
    const int2 x = rec[k];
    row = dst[k];
    const int d = (int)((uint32_t)x.y >> 16);
    if (t >= d && spikes[(size_t)(t - d) * N + x.x]) c = (long long)(int16_t)(x.y & 0xFFFF);
  }
  // inclusive segmented sum over lanes holding the same row (rows are
  // non-decreasing along the positions, so a row's lanes are contiguous)
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long v = __shfl_up(c, off);
    const int rr = __shfl_up(row, off);
    if (lane >= off && rr == row) c += v;
  }
  const int next = __shfl_down(row, 1);
  const bool last = lane == 63 || next != row;
  if (row >= 0 && last && c != 0)
    atomicAdd(reinterpret_cast<unsigned long long*>(&acc[row]), (unsigned long long)c);
}

struct LifParams {
  int32_t threshold, reset, refractory, nshift;
  int32_t shift[8];
};

__global__ __launch_bounds__(256) void lif_update(int64_t N, int t, LifParams p,
                                                  long long* __restrict__ acc,
                                                  int32_t* __restrict__ v, int32_t* __restrict__ r,
                                                  uint8_t* __restrict__ spikes,
                                                  int32_t* __restrict__ potentials,
                                                  int32_t* __restrict__ flags) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  const long long in = acc[i];
  acc[i] = 0;
  int32_t vi = v[i];
  int32_t ri = r[i];
  uint8_t s = 0;
  if (ri > 0) {
    ri -= 1;  // refractory: the arriving impulses are dropped
  } else {
    // arithmetic right shift of a signed int32 = floor division by 2^k
    for (int j = 0; j < p.nshift; ++j) vi -= vi >> p.shift[j];
    const long long x = (long long)vi + in;
    if (x < INT_MIN || x > INT_MAX) atomicMin(&flags[0], t);
    vi = (int32_t)x;
    if (vi >= p.threshold) {
      s = 1;
      vi = p.reset;
      ri = p.refractory;
    }
  }
  v[i] = vi;
  r[i] = ri;
  spikes[(size_t)t * N + i] = s;
  potentials[(size_t)t * N + i] = vi;
}

inline unsigned blocks(int64_t n) { return (unsigned)std::max<int64_t>(1, (n + 255) / 256); }

}  // namespace
}  // namespace ckhip

using namespace ckhip;

extern "C" ck_status ck_lif_workspace_size(ck_graph_t g, size_t* workspace_bytes) {
  clear_error();
  ck_status rc = check_graph(g);
  if (rc != CK_OK) return rc;
  if (!workspace_bytes) {
    set_error("workspace_bytes is NULL");
    return CK_ERR_NULL_ARG;
  }
  *workspace_bytes = lif_layout(g->N, g->E).total;
  return CK_OK;
}

extern "C" ck_status ck_lif_forward(ck_graph_t g, const int16_t* impulses, const int32_t* delays,
                                    const ck_lif_params* params, const int32_t* v0, int64_t T,
                                    uint8_t* spikes, int32_t* potentials, int64_t* overflow_step,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  ck_status rc = check_graph(g);
  if (rc != CK_OK) return rc;
  if (overflow_step) *overflow_step = -1;
  const int64_t N = g->N, E = g->E;
  if (T <= 0 || T > INT_MAX) {
    set_error("T must be in [1, 2^31 - 1] (got %lld)", (long long)T);
    return CK_ERR_BAD_SIZE;
  }
  if ((E > 0 && (!impulses || !delays)) || !params || !v0 || !spikes || !potentials ||
      !workspace) {
    set_error("NULL pointer for a non-empty tensor in the LIF forward");
    return CK_ERR_NULL_ARG;
  }
  if (params->num_decay_shifts < 0 || params->num_decay_shifts > 8 ||
      params->refractory_steps < 0) {
    set_error("num_decay_shifts must be in [0, 8] and refractory_steps >= 0");
    return CK_ERR_BAD_VALUE;
  }
  LifParams p{};
  p.threshold = params->threshold;
  p.reset = params->reset;
  p.refractory = params->refractory_steps;
  p.nshift = params->num_decay_shifts;
  for (int j = 0; j < p.nshift; ++j) {
    if (params->decay_shifts[j] < 0 || params->decay_shifts[j] > 31) {
      set_error("decay shift %d is outside [0, 31]", params->decay_shifts[j]);
      return CK_ERR_BAD_VALUE;
    }
    p.shift[j] = params->decay_shifts[j];
  }
  const LifWs ws = lif_layout(N, E);
  if (workspace_bytes < ws.total) {
    set_error("workspace of %zu bytes is below the %zu required", workspace_bytes, ws.total);
    return CK_ERR_WORKSPACE;
  }
  char* wsb = static_cast<char*>(workspace);
  int2* rec = reinterpret_cast<int2*>(wsb + ws.rec);
  int32_t* dst = reinterpret_cast<int32_t*>(wsb + ws.dst);
  long long* acc = reinterpret_cast<long long*>(wsb + ws.acc);
  int32_t* v = reinterpret_cast<int32_t*>(wsb + ws.v);
  int32_t* r = reinterpret_cast<int32_t*>(wsb + ws.r);
  int32_t* flags = reinterpret_cast<int32_t*>(wsb + ws.flags);
  lif_init<<<blocks(N), 256, 0, stream>>>(v0, N, v, r, acc, flags);
  if (E > 0)
    lif_pack<<<blocks(E), 256, 0, stream>>>(g->row_ptr, g->col_idx, g->perm, impulses, delays, N,
                                            E, rec, dst, flags);
  for (int64_t t = 0; t < T; ++t) {
    if (t >= 1 && E > 0) {
      rc = timed_launch(g_profile.lif_gather, stream, [&] {
        lif_gather<<<blocks(E), 256, 0, stream>>>(rec, dst, E, N, (int)t, spikes, acc);
      });
      if (rc != CK_OK) return rc;
    }
    rc = timed_launch(g_profile.lif_update, stream, [&] {
      lif_update<<<blocks(N), 256, 0, stream>>>(N, (int)t, p, acc, v, r, spikes, potentials, flags);
    });
    if (rc != CK_OK) return rc;
  }
  CK_HIP_TRY(hipGetLastError());
  int32_t fl[2] = {0, 0};
  CK_HIP_TRY(hipMemcpyAsync(fl, flags, sizeof(fl), hipMemcpyDeviceToHost, stream));
  CK_HIP_TRY(hipStreamSynchronize(stream));
  if (fl[1]) {
    set_error("an edge delay is outside [1, 32767]");
    return CK_ERR_BAD_VALUE;
  }
  if (fl[0] != INT_MAX) {
    if (overflow_step) *overflow_step = fl[0];
    set_error("a membrane potential left the int32 range at timestep %d; the run is rejected "
              "(outputs of that step and later are unspecified)", fl[0]);
    return CK_ERR_OVERFLOW;
  }
  return CK_OK;
}
