// resident.hip -- XCD-resident forward and backward of the leaky-tanh
// recurrence on a fixed sparse graph (connectome-kernels README, introduction:
// the proposal and the leaky update repeated `microsteps` times per input
// step, and its gradient for edge values, leak, bias, drives and initial
// state; "Design notes": [N, B] state, transposed CSR in the backward, saved
// state and pre-activation after every microstep).
//
// The per-microstep kernels pay a launch, a cold first round trip and a
// kernel-boundary cache flush every microstep.  Here one launch runs every
// microstep of a call.  Batch columns never interact, so the batch is cut
// into groups of 4 columns and group c is computed entirely by the
// workgroups of XCD c mod 8 (an XCD with several groups computes them in
// turn): those share one L2, so a microstep's new state (written by all of
// them) is exchanged through that L2 behind a counter barrier local to the
// XCD, with no cross-XCD coherence traffic.
//
// Each workgroup (1024 threads, one per CU) keeps the whole state plane of its
// column group ([N + 16] x float4, rows N.. all zeros) in LDS, and holds its share
// of the edges in registers for the whole launch: lane l holds one "piece" of
// at most D edges of one row (host plan in schedule.cpp; a row's pieces take
// consecutive lanes, and each piece's edges are ordered against LDS bank
// conflicts).  A microstep is
//   1. every lane gathers its D source rows from LDS and forms the piece's
//      partial sum (float4 over the group's 4 columns);
//   2. the pieces' partial sums are added per row (a segmented scan across
//      each wave, then the row's owner lane adds one value per wave) and the
//      owner runs the row's epilogue, writing the new row to this
//      microstep's plane in global memory (the saved-state arena, or the
//      exchange planes of the backward);
//   3. the XCD's workgroups meet at a counter barrier, and every workgroup
//      copies the new plane into its LDS (global -> LDS loads, 16 B per lane).
//      What no other workgroup reads -- the saved pre-activation and the
//      outputs of the forward, the drive gradients of the backward -- is
//      stored after the workgroup's arrival, so the barrier does not wait
//      for it.
// Every sum has a fixed order, so results are bitwise reproducible.  Every
// wait is bounded: a workgroup that waits too long raises an error flag and
// leaves; the call's last kernel then writes NaN to every output.
#include <algorithm>
#include <cmath>

#include "ck_internal.h"
#include "device_math.h"

namespace ckhip {
namespace {

// Control block (per call, zeroed by the prologue): tickets and barrier
// counters per XCD, 128 bytes apart, and the error flag.
constexpr int kCtlTicket = 0;
constexpr int kCtlCount = 256;
constexpr int kCtlErr = 512;
// bits of the error flag: a workgroup found an unexpected grouping (1), a wait
// gave up (2), the saved arena came from a forward that failed (4)
constexpr unsigned kErrForward = 4u;
constexpr int kCtlWords = 1024;
constexpr int kCtlStride = 32;

typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

struct ResCommon {
  const int32_t* rank_rows;
  const int32_t* owner_pbeg;
  const int32_t* piece_row;
  const int2* pedge;  // [ranks][D][kResLanes] {node, value bits}
  unsigned* ctl;
  const float* leak;
  const int32_t* input_slot;
  int N, Np, B, G, n_in, M, S, ranks;
  int spin_limit;  // polls before a wait gives up (< 0: every wait gives up at once)
};

struct ResFwdArgs {
  ResCommon c;
  const float* bias;
  const float* drives;  // [T][n_in][B]
  const float* h0;      // [G][Np] float4: the initial state by column group
  float* hplanes;       // [S][G][Np] float4: h^(s)
  float* aplanes;       // [S][G][Np] float4: a^(s)
  float* out;           // [T][B][N]: h at the last microstep of every input step
};

struct ResBwdArgs {
  ResCommon c;
  const float* h0;
  const float* hplanes;
  const float* aplanes;
  const float* grad_out;  // [T][B][N]
  float* gaplanes;        // [S][G][Np] float4: ga^(s), the exchanged plane
  float* gvpart;          // [G][slots] edge-gradient partials by column group
  float* glpart;          // [G][N]
  float* gbpart;          // [G][N]
  float* gdrives;         // [T][n_in][B]
  float* gstate0;         // [B][N]
};

__device__ __forceinline__ float4 ldf4(const float* base, size_t row) {
  return reinterpret_cast<const float4*>(base)[row];
}
__device__ __forceinline__ void stf4(float* base, size_t row, float4 v) {
  reinterpret_cast<float4*>(base)[row] = v;
}

// Buffer accesses: a wave-uniform base (kept in scalar registers), a 32-bit
// per-lane byte offset and a wave-uniform byte offset, so that a lane's
// addresses cost one vector register instead of a 64-bit pair each.  The
// range is the maximum; every offset here is below 2^32 by construction.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ float4 bld4(const void* base, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rsrc(base), voff, soff, 0));
}
__device__ __forceinline__ float bld1(const void* base, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc(base), voff, soff, 0));
}
__device__ __forceinline__ void bst4(float4 v, void* base, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, v), rsrc(base), voff, soff, 0);
}
__device__ __forceinline__ void bst1(float v, void* base, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rsrc(base), voff, soff, 0);
}
// tanh from the identity tanh(a) = sign(a) (1 - e) / (1 + e), e = exp(-2|a|)
// (0 < e <= 1, so nothing overflows), with the hardware exponential and
// reciprocal: absolute error about 2^-23, below the fp32 rounding of the
// row sums that feed it.  The backward shares e between tanh and
// sech^2(a) = 4 e / (1 + e)^2.
__device__ __forceinline__ float ftanh(float a) {
  const float e = __expf(-2.0f * fabsf(a));
  return copysignf((1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e), a);
}
__device__ __forceinline__ float comp(float4 v, int c) {
  return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}

// Join the launch: the workgroup's XCD computes column groups xcc, xcc + 8,
// ..., one after the other; its rank in the XCD comes from the XCD's ticket
// counter.  Returns the rank, or -1 when the workgroup has nothing to do (an
// XCD beyond the column groups) or the grouping is not the expected one
// (error flag raised).
__device__ int res_join(const ResCommon& c, int xcc, int* s_rank) {
  if (threadIdx.x == 0) {
    int rank = -1;
    if (xcc < kResXcds) {
      rank = (int)__hip_atomic_fetch_add(&c.ctl[kCtlTicket + xcc * kCtlStride], 1u,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (rank >= c.ranks) rank = -2;
    } else {
      rank = -2;
    }
    if (rank == -2) {
      __hip_atomic_fetch_or(&c.ctl[kCtlErr], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      rank = -1;
    }
    if (xcc >= c.G) rank = -1;
    *s_rank = rank;
  }
  __syncthreads();
  return *s_rank;
}

// Barrier of the XCD's workgroups, the `round`-th of the launch (1-based),
// in two halves: res_arrive counts the workgroup in once its stores are
// complete in the XCD's L2; res_wait waits for the others and leaves no line
// older than that in this CU's vector L1.  Stores issued between the two are
// not covered (nor waited for).  res_wait returns false (after raising the
// error flag) if the other workgroups did not all arrive in time.
__device__ void res_arrive(const ResCommon& c, int xcc) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(&c.ctl[kCtlCount + xcc * kCtlStride], 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

__device__ bool res_wait(const ResCommon& c, int xcc, int round, volatile int* s_fail) {
  if (threadIdx.x == 0) {
    unsigned* cnt = &c.ctl[kCtlCount + xcc * kCtlStride];
    const unsigned target = (unsigned)c.ranks * (unsigned)round;
    int spins = 0;
    while (c.spin_limit < 0 ||
           __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (++spins > c.spin_limit) {
        __hip_atomic_fetch_or(&c.ctl[kCtlErr], 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_fail = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  if (*s_fail) return false;
  asm volatile("buffer_inv sc0" ::: "memory");
  return true;
}

__device__ bool res_barrier(const ResCommon& c, int xcc, int round, volatile int* s_fail) {
  res_arrive(c, xcc);
  return res_wait(c, xcc, round, s_fail);
}

// Rows [0, N) of a plane of float4 rows into LDS, 64 rows per wave
// instruction (global -> LDS, no registers).  The 64-row chunks are taken in
// an order rotated by `rot`: the XCD's workgroups all copy the same plane at
// the same moment, and starting each at a different place spreads their
// requests over the L2 channels.
__device__ __forceinline__ void res_load_plane(float4* lds, const float* src, int N, int rot = 0) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const float4* s4 = reinterpret_cast<const float4*>(src);
  const int nch = (N + 63) / 64;
  for (int k = wave; k < nch; k += kResLanes / 64) {
    const int ch = (k + rot) % nch;
    const int i = ch * 64 + lane;
    if (i < N)
      __builtin_amdgcn_global_load_lds((const void*)(s4 + i),
                                       (__attribute__((address_space(3))) void*)(lds + ch * 64),
                                       16, 0, 0);
  }
}

// The lane's piece: D {node, value} pairs, nodes packed two per register.
template <int D>
struct Piece {
  uint32_t node[D / 2];
  float val[D];
  __device__ __forceinline__ void load(const int2* pedge, int rank, int tid) {
    const int2* p = pedge + (size_t)rank * D * kResLanes + tid;
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int2 x = p[(size_t)j * kResLanes];
      val[j] = __int_as_float(x.y);
      if (j & 1) node[j / 2] |= (uint32_t)x.x << 16;
      else node[j / 2] = (uint32_t)x.x;
    }
  }
  __device__ __forceinline__ uint32_t at(int j) const {
    return (j & 1) ? (node[j / 2] >> 16) : (node[j / 2] & 0xFFFFu);
  }
  // Hide the packed nodes' values from the optimiser once per microstep, so
  // it unpacks them where they are used instead of keeping D unpacked
  // addresses alive for the whole launch.
  __device__ __forceinline__ void launder() {
#pragma unroll
    for (int k = 0; k < D / 2; ++k) asm volatile("" : "+v"(node[k]));
  }
};

// One step of a segmented scan across a wave with a DPP lane move (CTRL:
// row_shr:n = 0x110 + n, row_bcast:15 = 0x142, row_bcast:31 = 0x143; rows
// outside ROW_MASK and lanes the move brings nothing to read 0): the moved
// value is added where `take` holds.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void seg_step(float4& acc, bool take) {
  const float ux = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc.x), CTRL, ROW_MASK, 0xF, false));
  const float uy = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc.y), CTRL, ROW_MASK, 0xF, false));
  const float uz = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc.z), CTRL, ROW_MASK, 0xF, false));
  const float uw = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc.w), CTRL, ROW_MASK, 0xF, false));
  acc.x = take ? acc.x + ux : acc.x;
  acc.y = take ? acc.y + uy : acc.y;
  acc.z = take ? acc.z + uz : acc.z;
  acc.w = take ? acc.w + uw : acc.w;
}

// First lane of the lane's segment: the run of lanes of its wave holding
// pieces of the same row (a row's pieces take consecutive lanes).
__device__ __forceinline__ int segment_start(int prow) {
  const int lane = threadIdx.x & 63;
  const int before = __shfl_up(prow, 1);
  const unsigned long long starts = __ballot(lane == 0 || before != prow);
  const unsigned long long upto = starts & (lane == 63 ? ~0ull : ((2ull << lane) - 1ull));
  return 63 - __builtin_clzll(upto);
}

// Inclusive scan of the pieces' partial sums inside each segment: the
// segment's last lane ends with the sum of the row's pieces held by its wave.
// DPP moves (within 16-lane rows, then row broadcasts) keep it off the LDS
// pipe, which the gathers saturate (shuffles through LDS permutes cost a
// sixth of the forward).
__device__ __forceinline__ void segmented_scan(float4& acc, int seg0) {
  const int lane = threadIdx.x & 63;
  seg_step<0x111, 0xF>(acc, lane - 1 >= seg0);     // row_shr:1
  seg_step<0x112, 0xF>(acc, lane - 2 >= seg0);     // row_shr:2
  seg_step<0x114, 0xF>(acc, lane - 4 >= seg0);     // row_shr:4
  seg_step<0x118, 0xF>(acc, lane - 8 >= seg0);     // row_shr:8
  seg_step<0x142, 0xA>(acc, seg0 < (lane & ~15));  // row_bcast:15 into rows 1, 3
  seg_step<0x143, 0xC>(acc, seg0 < 32);            // row_bcast:31 into rows 2, 3
}

// The owner's row sum: its pieces are lanes [pb, pe) of `part`, which holds
// every lane's scanned value; one segment end per wave the pieces touch.
__device__ __forceinline__ float4 row_sum(const float4* part, int pb, int pe) {
  float4 sum = f4(0.f);
  for (int q = pb; q < pe; q = (q | 63) + 1) sum = add4(sum, part[min(pe - 1, q | 63)]);
  return sum;
}

// MULTI: more than kResXcds column groups, so each XCD computes several in
// turn (a separate instantiation keeps the one-group kernel's registers).
template <int D, bool MULTI>
__global__ __launch_bounds__(kResLanes) void res_fwd(ResFwdArgs p) {
  extern __shared__ float4 sm[];
  __shared__ int s_rank;
  __shared__ int s_fail;
  const int tid = threadIdx.x;
  const int xcc = (int)xcc_id();
  if (tid == 0) s_fail = 0;
  const int rank = res_join(p.c, xcc, &s_rank);
  if (rank < 0) return;
  const int N = p.c.N, B = p.c.B;
  float4* plane = sm;             // [N + kResZeroRows]
  float4* part = sm + (N + kResZeroRows);  // [kResLanes]
  const int r0 = p.c.rank_rows[rank], r1 = p.c.rank_rows[rank + 1];
  Piece<D> pc;
  pc.load(p.c.pedge, rank, tid);
  const int prow = p.c.piece_row[(size_t)rank * kResLanes + tid];
  const int seg0 = segment_start(prow);
  // a wave whose lanes hold no piece (the plan fills lanes from 0) skips the
  // gathers: reads of the zero row cost the LDS as much as real ones.  (The
  // same skip measured slightly slower in the backward, which has fewer idle
  // waves, so it is not used there.)
  const bool wlive = __ballot(prow >= 0) != 0ull;
  const bool owner = r0 + tid < r1;
  const int row = owner ? r0 + tid : 0;
  const uint32_t rowb = (uint32_t)row * 16u, rowf = (uint32_t)row * 4u;
  const uint32_t colN = (uint32_t)N * 4u;  // bytes between batch columns of [B][N] tensors
  int pb = 0, pe = 0, ks = -1;
  float lam = 0.f, beta = 0.f;
  if (owner) {
    const int32_t* ob = p.c.owner_pbeg + (size_t)rank * (kResLanes + 1);
    pb = ob[tid];
    pe = ob[tid + 1];
    lam = p.c.leak[row];
    beta = p.bias[row];
    ks = p.c.input_slot[row];
  }
  const uint32_t ksb = (uint32_t)(ks >= 0 ? ks : 0) * (uint32_t)B * 4u;
  const size_t gsz = (size_t)p.c.Np * 4;   // floats per column-group slice
  const size_t psz = gsz * p.c.G;          // floats per microstep plane
  int round = 0;
  const int gend = MULTI ? p.c.G : xcc + 1;
  for (int grp = xcc; grp < gend; grp += kResXcds) {
    const int b0 = grp * 4;
    const size_t goff = (size_t)grp * gsz;
    if (grp != xcc) __syncthreads();  // the previous group's last reads of the plane are done
    res_load_plane(plane, p.h0 + goff, N);
    if (tid < kResZeroRows) plane[N + tid] = f4(0.f);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int s = 1; s <= p.c.S; ++s) {
      const int t = (s - 1) / p.c.M;
      // the drive of an input row, requested before the gathers
      float4 drv = f4(0.f);
      if (owner && ks >= 0) {
        const float* dr = p.drives + (size_t)t * p.c.n_in * B;
        if (b0 < B) drv.x = bld1(dr, ksb, (uint32_t)b0 * 4u);
        if (b0 + 1 < B) drv.y = bld1(dr, ksb, (uint32_t)(b0 + 1) * 4u);
        if (b0 + 2 < B) drv.z = bld1(dr, ksb, (uint32_t)(b0 + 2) * 4u);
        if (b0 + 3 < B) drv.w = bld1(dr, ksb, (uint32_t)(b0 + 3) * 4u);
      }
      pc.launder();
      float4 acc = f4(0.f);
      if (wlive) {
#pragma unroll
        for (int j = 0; j < D; ++j) acc = fma4(pc.val[j], plane[pc.at(j)], acc);
        segmented_scan(acc, seg0);
      }
      part[tid] = acc;
      __syncthreads();
      float4 ast = f4(0.f), hst = f4(0.f);
      if (owner) {
        const float4 sum = row_sum(part, pb, pe);
        const float4 hp = plane[row];
        float4 a, h;
        a.x = sum.x + drv.x + beta;
        a.y = sum.y + drv.y + beta;
        a.z = sum.z + drv.z + beta;
        a.w = sum.w + drv.w + beta;
        h.x = (1.0f - lam) * hp.x + lam * ftanh(a.x);
        h.y = (1.0f - lam) * hp.y + lam * ftanh(a.y);
        h.z = (1.0f - lam) * hp.z + lam * ftanh(a.z);
        h.w = (1.0f - lam) * hp.w + lam * ftanh(a.w);
        bst4(h, p.hplanes + (size_t)(s - 1) * psz + goff, rowb, 0);
        ast = a;
        hst = h;
      }
      // only the new state is exchanged: the saved a and the outputs are
      // stored after this workgroup has arrived at the barrier
      if (s < p.c.S) res_arrive(p.c, xcc);
      if (owner) {
        bst4(ast, p.aplanes + (size_t)(s - 1) * psz + goff, rowb, 0);
        if (s % p.c.M == 0) {
          // the output of input step s / M - 1, column by column (consecutive
          // owners hold consecutive rows, so each store is contiguous)
          float* o = p.out + (size_t)(s / p.c.M - 1) * B * N;
          const uint32_t cb = (uint32_t)b0 * colN;
          if (b0 < B) bst1(hst.x, o, rowf, cb);
          if (b0 + 1 < B) bst1(hst.y, o, rowf, cb + colN);
          if (b0 + 2 < B) bst1(hst.z, o, rowf, cb + 2 * colN);
          if (b0 + 3 < B) bst1(hst.w, o, rowf, cb + 3 * colN);
        }
      }
      if (s == p.c.S) break;
      if (!res_wait(p.c, xcc, ++round, &s_fail)) return;
      res_load_plane(plane, p.hplanes + (size_t)(s - 1) * psz + goff, N, rank * ((N + 63) / 64) / p.c.ranks);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }
}

template <int D, bool MULTI>
__global__ __launch_bounds__(kResLanes) void res_bwd(ResBwdArgs p) {
  extern __shared__ float4 sm[];
  __shared__ int s_rank;
  __shared__ int s_fail;
  const int tid = threadIdx.x;
  const int xcc = (int)xcc_id();
  if (tid == 0) s_fail = 0;
  const int rank = res_join(p.c, xcc, &s_rank);
  if (rank < 0) return;
  const int N = p.c.N, B = p.c.B, M = p.c.M, S = p.c.S;
  float4* plane = sm;
  float4* part = sm + (N + kResZeroRows);
  const int r0 = p.c.rank_rows[rank], r1 = p.c.rank_rows[rank + 1];
  Piece<D> pc;
  pc.load(p.c.pedge, rank, tid);
  float gvacc[D];
#pragma unroll
  for (int j = 0; j < D; ++j) gvacc[j] = 0.f;
  const int prow = p.c.piece_row[(size_t)rank * kResLanes + tid];
  const uint32_t prowb = (uint32_t)(prow >= 0 ? prow : 0) * 16u;
  // (every wave runs the gathers here: skipping idle waves measured slower
  // in the backward)
  const int seg0 = segment_start(prow);
  const bool owner = r0 + tid < r1;
  const int row = owner ? r0 + tid : 0;
  const uint32_t rowb = (uint32_t)row * 16u, rowf = (uint32_t)row * 4u;
  int pb = 0, pe = 0, ks = -1;
  float lam = 0.f;
  if (owner) {
    const int32_t* ob = p.c.owner_pbeg + (size_t)rank * (kResLanes + 1);
    pb = ob[tid];
    pe = ob[tid + 1];
    lam = p.c.leak[row];
    ks = p.c.input_slot[row];
  }
  const uint32_t ksb = (uint32_t)(ks >= 0 ? ks : 0) * (uint32_t)B * 4u;
  // the column group being computed (set per pass below): its first batch
  // column, its number of real columns (the rest are padding), its slice
  int b0 = 0, live = 0;
  size_t goff = 0;
  const uint32_t colN = (uint32_t)N * 4u;  // bytes between batch columns of [B][N] tensors
  const size_t gsz = (size_t)p.c.Np * 4;
  const size_t psz = gsz * p.c.G;
  // h^(s) of the group (s = 0: the initial state), a^(s), ga^(s)
  auto hpl = [&](int s) { return s == 0 ? p.h0 + goff : p.hplanes + (size_t)(s - 1) * psz + goff; };
  auto apl = [&](int s) { return p.aplanes + (size_t)(s - 1) * psz + goff; };
  auto gapl = [&](int s) { return p.gaplanes + (size_t)(s - 1) * psz + goff; };
  // upstream gradient entering at microstep k (k % M == 0): G[k/M - 1][b][row]
  auto gin = [&](int k) {
    float4 g = f4(0.f);
    if (k % M == 0) {
      const float* Gt = p.grad_out + (size_t)(k / M - 1) * B * N;
      const uint32_t cb = (uint32_t)b0 * colN;
      if (live > 0) g.x = bld1(Gt, rowf, cb);
      if (live > 1) g.y = bld1(Gt, rowf, cb + colN);
      if (live > 2) g.z = bld1(Gt, rowf, cb + 2 * colN);
      if (live > 3) g.w = bld1(Gt, rowf, cb + 3 * colN);
    }
    return g;
  };
  float4 gh = f4(0.f), gd = f4(0.f);
  float gl = 0.f, gb = 0.f;
  int gd_step = -1;  // input step whose drive gradient gd holds, complete and not yet stored
  // elementwise pass of microstep k on the owner's row, given g^(k) before
  // its seed, the seed, a^(k) and h^(k-1): leak/bias row sums, drive gradient,
  // and ga^(k) to the exchange plane
  auto k1 = [&](int k, float4 g, float4 seed, float4 ak, float4 qk) {
    g = add4(g, seed);
    float ga[4], gg[4] = {g.x, g.y, g.z, g.w};
    const float av[4] = {ak.x, ak.y, ak.z, ak.w}, qv[4] = {qk.x, qk.y, qk.z, qk.w};
    float ls = 0.f, bs = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // every column is computed and padding columns are masked by selects:
      // branches here cost the backward 2.5 %
      const bool on = c < live;
      // e = exp(-2|a|), r = 1/(1+e): tanh(a) = sign(a)(1-e)r, sech^2(a) = 4e r^2
      // (from a itself, not 1 - tanh^2, which cancels once |a| is a few units)
      const float e = __expf(-2.0f * fabsf(av[c]));
      const float r = __builtin_amdgcn_rcpf(1.0f + e);
      const float th = copysignf((1.0f - e) * r, av[c]);
      const float lt = gg[c] * (th - qv[c]);
      const float gt = gg[c] * lam * (4.0f * e * r * r);
      ls += on ? lt : 0.f;
      gg[c] = on ? gg[c] : 0.f;
      ga[c] = on ? gt : 0.f;
      bs += ga[c];
    }
    gl += ls;
    gb += bs;
    gh = make_float4(gg[0], gg[1], gg[2], gg[3]);
    const float4 ga4 = make_float4(ga[0], ga[1], ga[2], ga[3]);
    if (ks >= 0) {
      gd = add4(gd, ga4);
      // the input step's drive gradient is complete: stored by flush_gd,
      // after the barrier's arrival (no other workgroup reads it)
      if ((k - 1) % M == 0) gd_step = (k - 1) / M;
    }
    bst4(ga4, gapl(k), rowb, 0);
  };
  auto flush_gd = [&]() {
    if (gd_step >= 0) {
      float* o = p.gdrives + (size_t)gd_step * p.c.n_in * B;
      if (live > 0) bst1(gd.x, o, ksb, (uint32_t)b0 * 4u);
      if (live > 1) bst1(gd.y, o, ksb, (uint32_t)(b0 + 1) * 4u);
      if (live > 2) bst1(gd.z, o, ksb, (uint32_t)(b0 + 2) * 4u);
      if (live > 3) bst1(gd.w, o, ksb, (uint32_t)(b0 + 3) * 4u);
      gd = f4(0.f);
      gd_step = -1;
    }
  };
  int round = 0;
  const int gend = MULTI ? p.c.G : xcc + 1;
  for (int grp = xcc; grp < gend; grp += kResXcds) {
    b0 = grp * 4;
    live = B - b0 < 4 ? B - b0 : 4;
    goff = (size_t)grp * gsz;
    gh = f4(0.f);
    gd = f4(0.f);
    gl = 0.f;
    gb = 0.f;
#pragma unroll
    for (int j = 0; j < D; ++j) gvacc[j] = 0.f;
    if (grp != xcc) __syncthreads();  // the previous group's last reads of the plane are done
    // the last microstep's elementwise pass seeds the reverse sweep
    if (owner) k1(S, f4(0.f), gin(S), bld4(apl(S), rowb, 0), bld4(hpl(S - 1), rowb, 0));
    float4 hq = prow >= 0 ? bld4(hpl(S - 1), prowb, 0) : f4(0.f);
    res_arrive(p.c, xcc);
    if (owner) flush_gd();
    if (!res_wait(p.c, xcc, ++round, &s_fail)) return;
    res_load_plane(plane, gapl(S), N, rank * ((N + 63) / 64) / p.c.ranks);
    if (tid < kResZeroRows) plane[N + tid] = f4(0.f);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int s = S; s >= 1; --s) {
      // operands of this iteration's elementwise pass (microstep s-1) and of the
      // next iteration's edge pass, requested before the gathers
      float4 seed = f4(0.f), ak = f4(0.f), qk = f4(0.f);
      if (s >= 2 && owner) {
        seed = gin(s - 1);
        ak = bld4(apl(s - 1), rowb, 0);
        qk = bld4(hpl(s - 2), rowb, 0);
      }
      pc.launder();
      // gathers in groups of 4 rows, so that at most 4 gathered rows occupy
      // registers beside the piece and its edge-gradient sums
      float4 acc = f4(0.f);
#pragma unroll
      for (int j0 = 0; j0 < D; j0 += 4) {
        // (the last group holds D mod 4 rows when D is not a multiple of 4)
        float4 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (j0 + u < D) x[u] = plane[pc.at(j0 + u)];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (j0 + u >= D) break;
          acc = fma4(pc.val[j0 + u], x[u], acc);
          gvacc[j0 + u] += dot4(x[u], hq);
          // keep the update here (the optimiser would otherwise sink it past
          // the barrier below and keep every gathered row alive until then)
          asm volatile("" : "+v"(gvacc[j0 + u]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      segmented_scan(acc, seg0);
      part[tid] = acc;
      __syncthreads();
      if (owner) {
        const float4 sum = row_sum(part, pb, pe);
        float4 g;
        g.x = fmaf(1.0f - lam, gh.x, sum.x);
        g.y = fmaf(1.0f - lam, gh.y, sum.y);
        g.z = fmaf(1.0f - lam, gh.z, sum.z);
        g.w = fmaf(1.0f - lam, gh.w, sum.w);
        if (s >= 2) {
          k1(s - 1, g, seed, ak, qk);
        } else {
          const uint32_t cb = (uint32_t)b0 * colN;
          if (live > 0) bst1(g.x, p.gstate0, rowf, cb);
          if (live > 1) bst1(g.y, p.gstate0, rowf, cb + colN);
          if (live > 2) bst1(g.z, p.gstate0, rowf, cb + 2 * colN);
          if (live > 3) bst1(g.w, p.gstate0, rowf, cb + 3 * colN);
        }
      }
      if (s > 1) res_arrive(p.c, xcc);
      if (owner) flush_gd();
      if (s == 1) break;
      // the next iteration's piece rows h^(s-2): a piece's row is one of this
      // workgroup's rows, whose owner has just used that row as qk -- passed
      // through LDS (the partial sums are all read once every wave has
      // arrived) instead of loaded again by every piece lane
      if (owner) part[tid] = qk;
      if (!res_wait(p.c, xcc, ++round, &s_fail)) return;
      if (prow >= 0) hq = part[prow - r0];
      res_load_plane(plane, gapl(s - 1), N, rank * ((N + 63) / 64) / p.c.ranks);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    // partial results of this column group
    const int64_t slots = (int64_t)p.c.ranks * D * kResLanes;
    float* gvp = p.gvpart + (size_t)grp * slots + (size_t)rank * D * kResLanes + tid;
#pragma unroll
    for (int j = 0; j < D; ++j) gvp[(size_t)j * kResLanes] = gvacc[j];
    if (owner) {
      p.glpart[(size_t)grp * N + row] = gl;
      p.gbpart[(size_t)grp * N + row] = gb;
    }
  }
}

// Per call, before the resident kernel: edge values into the padded slots,
// the initial state into column-group planes, the control block to zero.
__global__ void res_prologue(const float* __restrict__ values, const int32_t* __restrict__ pcol,
                             const int32_t* __restrict__ pperm, int64_t slots,
                             int2* __restrict__ pedge, const float* __restrict__ state0, int N,
                             int Np, int B, int G, float* __restrict__ h0, unsigned* __restrict__ ctl) {
  const int64_t n = std::max<int64_t>(slots, (int64_t)G * Np);
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n;
       k += (int64_t)gridDim.x * blockDim.x) {
    if (k < slots) {
      const int32_t e = pperm[k];
      pedge[k] = make_int2(pcol[k], e >= 0 ? __float_as_int(values[e]) : 0);
    }
    if (k < (int64_t)G * Np) {
      const int g = (int)(k / Np), i = (int)(k % Np);
      float4 v = f4(0.f);
      if (i < N) {
        const int b = g * 4;
        v.x = b < B ? state0[(size_t)b * N + i] : 0.f;
        v.y = b + 1 < B ? state0[(size_t)(b + 1) * N + i] : 0.f;
        v.z = b + 2 < B ? state0[(size_t)(b + 2) * N + i] : 0.f;
        v.w = b + 3 < B ? state0[(size_t)(b + 3) * N + i] : 0.f;
      }
      stf4(h0, (size_t)k, v);
    }
    if (k < kCtlWords) ctl[k] = 0u;
  }
}

// After the resident forward (whose owners wrote the outputs): the kernel's
// error flag copied into the saved arena's status word (so that a backward
// given this arena knows), and NaN in every output if the flag is raised.
__global__ void res_fwd_status(const unsigned* __restrict__ ctl, int64_t n,
                               float* __restrict__ out, unsigned* __restrict__ saved_status) {
  const unsigned err = ctl[kCtlErr];
  if (blockIdx.x == 0 && threadIdx.x == 0) saved_status[0] = err;
  if (err == 0u) return;
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n;
       k += (int64_t)gridDim.x * blockDim.x)
    out[k] = NAN;
}

// After the resident backward: edge gradients to caller order and the leak /
// bias gradients, each summed over the column groups in group order; NaN in
// every gradient if the resident kernel raised its error flag or the forward
// that wrote the saved arena did (its status word; then kErrForward is added
// to the error flag, so that the call's status reports it).
__global__ void res_bwd_finish(const float* __restrict__ gvpart, int G, const int32_t* __restrict__ pperm,
                               int64_t slots, float* __restrict__ gv, const float* __restrict__ glpart,
                               const float* __restrict__ gbpart, int N, float* __restrict__ gleak,
                               float* __restrict__ gbias, unsigned* __restrict__ ctl,
                               const unsigned* __restrict__ saved_status,
                               float* __restrict__ gdrives, int64_t nd, float* __restrict__ gstate0,
                               int64_t ns) {
  const bool fwd_bad = saved_status[0] != 0u;
  const bool bad = fwd_bad || ctl[kCtlErr] != 0u;
  if (fwd_bad && blockIdx.x == 0 && threadIdx.x == 0)
    __hip_atomic_fetch_or(&ctl[kCtlErr], kErrForward, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int64_t n = std::max<int64_t>(std::max<int64_t>(slots, N), bad ? std::max(nd, ns) : 0);
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n;
       k += (int64_t)gridDim.x * blockDim.x) {
    if (k < slots) {
      const int32_t e = pperm[k];
      if (e >= 0) {
        float s = gvpart[k];
        for (int g = 1; g < G; ++g) s += gvpart[(size_t)g * slots + k];
        gv[e] = bad ? NAN : s;
      }
    }
    if (k < N) {
      float l = glpart[k], b = gbpart[k];
      for (int g = 1; g < G; ++g) {
        l += glpart[(size_t)g * N + k];
        b += gbpart[(size_t)g * N + k];
      }
      gleak[k] = bad ? NAN : l;
      gbias[k] = bad ? NAN : b;
    }
    if (bad) {
      if (k < nd) gdrives[k] = NAN;
      if (k < ns) gstate0[k] = NAN;
    }
  }
}

inline unsigned res_grid(int64_t n) {
  return (unsigned)std::min<int64_t>(std::max<int64_t>(1, (n + 255) / 256), 8192);
}

using ResFwdFn = void (*)(ResFwdArgs);
using ResBwdFn = void (*)(ResBwdArgs);

ResFwdFn fwd_kernel(int D, bool multi) {
  switch (D) {
    case 8: return multi ? &res_fwd<8, true> : &res_fwd<8, false>;
    case 12: return multi ? &res_fwd<12, true> : &res_fwd<12, false>;
    case 16: return multi ? &res_fwd<16, true> : &res_fwd<16, false>;
    case 18: return multi ? &res_fwd<18, true> : &res_fwd<18, false>;
    case 20: return multi ? &res_fwd<20, true> : &res_fwd<20, false>;
    case 24: return multi ? &res_fwd<24, true> : &res_fwd<24, false>;
  }
  return nullptr;
}
ResBwdFn bwd_kernel(int D, bool multi) {
  switch (D) {
    case 8: return multi ? &res_bwd<8, true> : &res_bwd<8, false>;
    case 12: return multi ? &res_bwd<12, true> : &res_bwd<12, false>;
    case 16: return multi ? &res_bwd<16, true> : &res_bwd<16, false>;
    case 18: return multi ? &res_bwd<18, true> : &res_bwd<18, false>;
    case 20: return multi ? &res_bwd<20, true> : &res_bwd<20, false>;
    case 24: return multi ? &res_bwd<24, true> : &res_bwd<24, false>;
  }
  return nullptr;
}

// LDS of a resident workgroup: the plane with its zero rows and the partial
// sums, and at least 82 KiB so that a CU never holds two of them.
size_t res_lds_bytes(int N) {
  return std::max<size_t>((size_t)(N + kResZeroRows) * 16 + (size_t)kResLanes * 16, 82 * 1024);
}

ResCommon common(const Resident& r, const ResDims& d, const int2* pedge, unsigned* ctl,
                 const float* leak, const int32_t* input_slot, int g_spin_limit) {
  ResCommon c{};
  c.rank_rows = r.rank_rows;
  c.owner_pbeg = r.owner_pbeg;
  c.piece_row = r.piece_row;
  c.pedge = pedge;
  c.ctl = ctl;
  c.leak = leak;
  c.input_slot = input_slot;
  c.N = (int)d.N;
  c.Np = (int)d.Np;
  c.B = (int)d.B;
  c.G = (int)d.G;
  c.n_in = (int)d.n_in;
  c.M = (int)d.M;
  c.S = (int)d.S;
  c.ranks = r.ranks;
  c.spin_limit = g_spin_limit;
  return c;
}

}  // namespace

ck_status res_prepare() {
  // the largest dynamic LDS a resident launch asks for (the plane of
  // kResMaxN nodes and the partial sums), allowed once for every kernel
  const int lds = (int)res_lds_bytes((int)kResMaxN);
  for (int D : kResPieceLens)
    for (bool multi : {false, true}) {
      CK_HIP_TRY(hipFuncSetAttribute((const void*)fwd_kernel(D, multi),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds));
      CK_HIP_TRY(hipFuncSetAttribute((const void*)bwd_kernel(D, multi),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds));
    }
  return CK_OK;
}

ResWs res_ws_layout(const ck_graph* g, const ResDims& d) {
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t plane = (size_t)d.G * d.Np * 16;  // bytes of one microstep plane
  ResWs w;
  size_t o = 0;
  w.pedge = o; o = al(o + (size_t)std::max(g->res_fwd.slots, g->res_bwd.slots) * 8);
  w.h0 = o;    o = al(o + plane);
  w.ctl = o;   o = al(o + kCtlWords * 4);
  w.ga = o;    o = al(o + (size_t)d.S * plane);
  w.gv = o;    o = al(o + (size_t)d.G * g->res_bwd.slots * 4);
  w.gl = o;    o = al(o + (size_t)d.G * d.N * 4);
  w.gb = o;    o = al(o + (size_t)d.G * d.N * 4);
  w.total = o;
  return w;
}

// the h and a planes, then a 256-byte trailer whose first word is the
// forward's error flag
size_t res_saved_bytes(const ResDims& d) { return 2 * (size_t)d.S * d.G * d.Np * 16 + 256; }

static unsigned* saved_status(void* saved, const ResDims& d) {
  return reinterpret_cast<unsigned*>(static_cast<char*>(saved) + 2 * (size_t)d.S * d.G * d.Np * 16);
}

ck_status res_status(const ck_graph* g, const ResDims& d, const void* workspace,
                     hipStream_t stream, unsigned* err) {
  const ResWs ws = res_ws_layout(g, d);
  const unsigned* ctl =
      reinterpret_cast<const unsigned*>(static_cast<const char*>(workspace) + ws.ctl);
  unsigned v = 0;
  CK_HIP_TRY(hipMemcpyAsync(&v, ctl + kCtlErr, sizeof(unsigned), hipMemcpyDeviceToHost, stream));
  CK_HIP_TRY(hipStreamSynchronize(stream));
  *err = v;
  return CK_OK;
}

size_t res_forward_ws_bytes(const ck_graph* g, const ResDims& d) {
  return res_ws_layout(g, d).ga;  // the edge slots, the initial state and the control block
}

ck_status res_forward(const ck_graph* g, const ResDims& d, const float* edge_values,
                      const float* leak, const float* bias, const float* drives,
                      const float* state0, float* out, void* saved, void* workspace,
                      hipStream_t stream, bool profile) {
  const Resident& r = g->res_fwd;
  const ResFwdFn kern = fwd_kernel(r.D, d.G > kResXcds);
  if (!kern) {
    set_error("no resident forward kernel for piece length %d", r.D);
    return CK_ERR_HIP;
  }
  const ResWs ws = res_ws_layout(g, d);
  char* wsb = static_cast<char*>(workspace);
  int2* pedge = reinterpret_cast<int2*>(wsb + ws.pedge);
  float* h0 = reinterpret_cast<float*>(wsb + ws.h0);
  unsigned* ctl = reinterpret_cast<unsigned*>(wsb + ws.ctl);
  res_prologue<<<res_grid(std::max<int64_t>(r.slots, d.G * d.Np)), 256, 0, stream>>>(
      edge_values, r.pcol, r.pperm, r.slots, pedge, state0, (int)d.N, (int)d.Np, (int)d.B,
      (int)d.G, h0, ctl);
  ResFwdArgs a{};
  a.c = common(r, d, pedge, ctl, leak, g->input_slot, g->res_spin_limit);
  a.bias = bias;
  a.drives = drives;
  a.h0 = h0;
  a.hplanes = static_cast<float*>(saved);
  a.aplanes = a.hplanes + (size_t)d.S * d.G * d.Np * 4;
  a.out = out;
  const size_t lds = res_lds_bytes((int)d.N);
  const unsigned wgs = (unsigned)(r.ranks * kResXcds);
  ck_status rc = CK_OK;
  if (profile)
    rc = timed_launch(g_profile.fwd, stream, [&] {
      hipLaunchKernelGGL(kern, dim3(wgs), dim3(kResLanes), lds, stream, a);
    });
  else
    hipLaunchKernelGGL(kern, dim3(wgs), dim3(kResLanes), lds, stream, a);
  if (rc != CK_OK) return rc;
  const int64_t nout = d.T * d.B * d.N;
  res_fwd_status<<<(unsigned)std::min<int64_t>(res_grid(nout), 1024), 256, 0, stream>>>(
      ctl, nout, out, saved_status(saved, d));
  CK_HIP_TRY(hipGetLastError());
  return CK_OK;
}

ck_status res_backward(const ck_graph* g, const ResDims& d, const float* edge_values,
                       const float* leak, const float* state0, const void* saved,
                       const float* grad_out, float* grad_edge_values, float* grad_leak,
                       float* grad_bias, float* grad_drives, float* grad_state0, void* workspace,
                       hipStream_t stream) {
  const Resident& r = g->res_bwd;
  const ResBwdFn kern = bwd_kernel(r.D, d.G > kResXcds);
  if (!kern) {
    set_error("no resident backward kernel for piece length %d", r.D);
    return CK_ERR_HIP;
  }
  const ResWs ws = res_ws_layout(g, d);
  char* wsb = static_cast<char*>(workspace);
  int2* pedge = reinterpret_cast<int2*>(wsb + ws.pedge);
  float* h0 = reinterpret_cast<float*>(wsb + ws.h0);
  unsigned* ctl = reinterpret_cast<unsigned*>(wsb + ws.ctl);
  res_prologue<<<res_grid(std::max<int64_t>(r.slots, d.G * d.Np)), 256, 0, stream>>>(
      edge_values, r.pcol, r.pperm, r.slots, pedge, state0, (int)d.N, (int)d.Np, (int)d.B,
      (int)d.G, h0, ctl);
  ResBwdArgs a{};
  a.c = common(r, d, pedge, ctl, leak, g->input_slot, g->res_spin_limit);
  a.h0 = h0;
  a.hplanes = static_cast<const float*>(saved);
  a.aplanes = a.hplanes + (size_t)d.S * d.G * d.Np * 4;
  a.grad_out = grad_out;
  a.gaplanes = reinterpret_cast<float*>(wsb + ws.ga);
  a.gvpart = reinterpret_cast<float*>(wsb + ws.gv);
  a.glpart = reinterpret_cast<float*>(wsb + ws.gl);
  a.gbpart = reinterpret_cast<float*>(wsb + ws.gb);
  a.gdrives = grad_drives;
  a.gstate0 = grad_state0;
  const size_t lds = res_lds_bytes((int)d.N);
  const unsigned wgs = (unsigned)(r.ranks * kResXcds);
  ck_status rc = timed_launch(g_profile.bwd, stream, [&] {
    hipLaunchKernelGGL(kern, dim3(wgs), dim3(kResLanes), lds, stream, a);
  });
  if (rc != CK_OK) return rc;
  const int64_t nd = d.T * d.n_in * d.B, ns = d.B * d.N;
  res_bwd_finish<<<res_grid(std::max<int64_t>({r.slots, d.N, nd, ns})), 256, 0, stream>>>(
      a.gvpart, (int)d.G, r.pperm, r.slots, grad_edge_values, a.glpart, a.gbpart, (int)d.N,
      grad_leak, grad_bias, ctl, saved_status(const_cast<void*>(saved), d), grad_drives, nd,
      grad_state0, ns);
  CK_HIP_TRY(hipGetLastError());
  return CK_OK;
}

}  // namespace ckhip
