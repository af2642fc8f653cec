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
//   lif_gather   four CSR positions per lane: each edge's impulse if its
//                source spiked d steps earlier (one byte read of the spike
//                history), a DPP prefix sum over the wave's positions, and
//                one 64-bit integer atomic add per run of positions of one
//                row into I[row].  Integer sums are exact and associative,
//                so the result does not depend on the order of the atomics.
//                When the bit rows of the steps the delays reach fit in LDS
//                (lif_gather_lds), each workgroup first copies them there and
//                looks the spikes up in LDS instead of one scattered byte
//                read per edge, and reads 8-byte records that carry the row
//                (no separate destination).
//   lif_update   one thread per neuron: the state update above; writes the
//                step's spikes and potentials (and the step's spike bits into
//                a ring of kLifRing bit rows), clears I.
// A prologue (in every ck_lif_forward, or once in ck_lif_prepare for any
// number of ck_lif_run calls) validates the delays, writes each position's
// destination, and packs {source, impulse, delay} (and, for the LDS lookups,
// the destination) into 8-byte records in CSR order (the caller's edge order
// stays invisible: impulse and delay are first packed into one word per
// caller edge, so the permutation costs one scattered read per position).
#include <algorithm>
#include <climits>
#include <cstdlib>

#include "ck_internal.h"

namespace ckhip {
namespace {

// flags[0]: first timestep whose update left the int32 range (INT_MAX: none)
// flags[1]: set when a delay is outside [1, 32767]
// flags[2]: the largest delay
// flags[3..7]: what a prepare left in the workspace: kLifMark, E and N (low
//   31 bits), the lookup (R: the bit rows' count, 0 for byte lookups) and the
//   low 32 bits of the graph's row-pointer address
constexpr int kLifFlags = 64;
constexpr int32_t kLifMark = 0x4C494650;
// Spike bit rows kept for the LDS lookups: step t's row is slot t % R of the
// ring, R = the largest delay (at most kLifRing); a workgroup holds the
// R rows in LDS, at most kLifLdsBytes.
constexpr int kLifRing = 16;
constexpr int kLifLdsBytes = 128 * 1024;

// Words between two bit rows: one bit per neuron, rounded up to 16 bytes.
inline int64_t lif_row_words(int64_t N) { return ((N + 31) / 32 + 3) & ~int64_t(3); }

struct LifWs {
  size_t rec, dst, words, acc, v, r, bits, flags, total;
};

LifWs lif_layout(int64_t N, int64_t E) {
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  LifWs w;
  size_t o = 0;
  // (32 spare bytes: lif_gather_lds reads positions in groups of 4, and the
  // last group may reach up to 3 positions past the records)
  w.rec = o;   o = al(o + (size_t)std::max<int64_t>(E, 1) * 8 + 32);
  // (16 spare bytes: lif_gather reads the rows of 4 positions at once)
  w.dst = o;   o = al(o + (size_t)std::max<int64_t>(E, 1) * 4 + 16);
  w.words = o; o = al(o + (size_t)std::max<int64_t>(E, 1) * 4);
  w.acc = o;   o = al(o + (size_t)N * 8);
  w.v = o;     o = al(o + (size_t)N * 4);
  w.r = o;     o = al(o + (size_t)N * 4);
  w.bits = o;  o = al(o + (size_t)kLifRing * lif_row_words(N) * 4);
  w.flags = o; o = al(o + kLifFlags * 4);
  w.total = o;
  return w;
}

// Start of a run: potentials from v0, refractory counts and accumulators
// cleared, no overflow seen.
__global__ void lif_init(const int32_t* __restrict__ v0, int64_t N, int32_t* __restrict__ v,
                         int32_t* __restrict__ r, long long* __restrict__ acc,
                         int32_t* __restrict__ flags) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < N) {
    v[i] = v0[i];
    r[i] = 0;
    acc[i] = 0;
  }
  if (i == 0) flags[0] = INT_MAX;
}

// Flags of a prepare: first cleared (mark included), then marked once done.
__global__ void lif_flags(int32_t* __restrict__ flags, int32_t m0, int32_t m1, int32_t m2,
                          int32_t m3, int32_t m4) {
  if (threadIdx.x == 0) {
    flags[1] = 0;
    flags[2] = 0;
    flags[3] = m0;
    flags[4] = m1;
    flags[5] = m2;
    flags[6] = m3;
    flags[7] = m4;
  }
}

// The impulse and delay of every edge in the caller's order packed into one
// word, impulse (low 16 bits) | delay << 16, with the delays validated and the
// largest one found.  Grid-stride, so the largest delay costs one atomic per
// workgroup.
__global__ __launch_bounds__(256) void lif_words(const int16_t* __restrict__ impulses,
                                                 const int32_t* __restrict__ delays, int64_t E,
                                                 uint32_t* __restrict__ words,
                                                 int32_t* __restrict__ flags) {
  __shared__ int32_t s_max[4];
  int32_t dmax = 0;
  bool bad = false;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < E;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int32_t d = delays[e];
    bad |= d < 1 || d > 32767;
    dmax = max(dmax, d);
    words[e] = (uint32_t)(uint16_t)impulses[e] | ((uint32_t)(d & 0x7FFF) << 16);
  }
  if (bad) atomicOr(&flags[1], 1);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) dmax = max(dmax, __shfl_xor(dmax, off));
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = dmax;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax(&flags[2], max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3])));
}

// Record k of the CSR: {source node, the word of its caller edge}: one
// scattered 4-byte read per position.
__global__ __launch_bounds__(256) void lif_pack(const int32_t* __restrict__ col_idx,
                                                const int32_t* __restrict__ perm,
                                                const uint32_t* __restrict__ words, int64_t E,
                                                int2* __restrict__ rec) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k < E) rec[k] = make_int2(col_idx[k], (int)words[perm[k]]);
}

// The records of the LDS-lookup path (every such graph has N <= 2^20 nodes:
// its bit rows fit 128 KB, and the largest delay is at most 16), with the
// destination inside: x = source (bits 0-19) | row bits 0-11 (bits 20-31),
// y = impulse (bits 0-15) | delay - 1 (bits 16-19) | row bits 12-23 (bits
// 20-31).  The per-step gather then reads 8 bytes per position.
__global__ __launch_bounds__(256) void lif_pack_lds(const int32_t* __restrict__ col_idx,
                                                    const int32_t* __restrict__ perm,
                                                    const uint32_t* __restrict__ words,
                                                    const int32_t* __restrict__ dst, int64_t E,
                                                    int2* __restrict__ rec) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= E) return;
  const uint32_t w = words[perm[k]], row = (uint32_t)dst[k];
  const uint32_t x = (uint32_t)col_idx[k] | (row & 0xFFFu) << 20;
  const uint32_t y = (w & 0xFFFFu) | ((w >> 16) - 1u) << 16 | (row >> 12) << 20;
  rec[k] = make_int2((int)x, (int)y);
}

// The destination of every CSR position: one wave per row writes the row's
// index over its range [row_ptr[i], row_ptr[i + 1]).
__global__ __launch_bounds__(256) void lif_rows(const int32_t* __restrict__ row_ptr, int64_t N,
                                                int32_t* __restrict__ dst) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  if (i >= N) return;
  const int lane = threadIdx.x & 63;
  const int32_t b = row_ptr[i], e = row_ptr[i + 1];
  for (int32_t k = b + lane; k < e; k += 64) dst[k] = (int32_t)i;
}

// Inclusive prefix sum over the 64 lanes of a wave: DPP row shifts within
// each row of 16 lanes, then the totals of the earlier rows added.
__device__ __forceinline__ int wave_prefix_sum(int v, int lane) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  return v + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
}

// lif_gather with the spike lookups in LDS: the R bit rows of steps
// t - 1 .. t - R (zero before step 0) are copied into LDS, row d - 1 for
// delay d, then each position tests its source's bit.  Bit rows are `ws`
// words apart (a multiple of 4), so the copy moves 16-byte words, at most
// kLifCopy of them per lane, all loads in flight together.  Grid-stride over
// the positions in chunks of kLifChunk; a lane takes kLifQ neighbouring
// positions in kLifQ / 2 16-byte loads, so a wave covers 64 kLifQ positions
// per group, and each chunk's records are loaded while the previous chunk is
// summed.  Per wave and group: one prefix sum over the lanes' sums (a group
// holds at most 256 impulses, |impulse| < 2^15, so 32 bits are exact) gives
// the prefix at every position; the run starts (the group's first position
// and every row change) come from two ballots, and the last position of each
// run adds its run's total (its prefix minus the prefix before the run's
// first position, found in the lane of the run's start) with one 64-bit
// atomic.
constexpr int kLifQ = 4;       // positions per lane and load group (kLifQ / 2 16-byte loads)
constexpr int kLifGroups = 1;  // load groups per lane and chunk
constexpr int kLifChunk = kLifGroups * kLifQ * 1024;
static_assert(kLifQ % 2 == 0 && 8 * (kLifQ - 1) <= 32,
              "a group's loads reach at most the record region's 32 spare bytes");
constexpr int kLifCopy = kLifLdsBytes / 16 / 1024;

__device__ __forceinline__ int lif_rec_row(int x, int y) {
  return (int)(((uint32_t)x >> 20) | ((uint32_t)y >> 20) << 12);
}

__global__ __launch_bounds__(1024) void lif_gather_lds(const int2* __restrict__ rec,
                                                      int64_t E, int ws, int t, int R,
                                                      const uint4* __restrict__ bits,
                                                      long long* __restrict__ acc) {
  extern __shared__ uint4 sb4[];  // [R][ws / 4]
  const uint32_t* sb = reinterpret_cast<const uint32_t*>(sb4);
  const int lane = threadIdx.x & 63;
  // load group j of a chunk starting at `base`: positions
  // base + kLifQ (1024 j + tid) + i, i < kLifQ; the loads start at a group of
  // positions no later than the last one, which the record region's spare
  // bytes keep in range.  The first chunk's records are requested before the
  // bit rows, so both round trips overlap.
  const int4* rec4 = reinterpret_cast<const int4*>(rec);
  const int64_t last_q = (E - 1) / kLifQ;
  const int64_t stride = (int64_t)gridDim.x * kLifChunk;
  constexpr int NL = kLifQ / 2;
  int4 x[kLifGroups][NL];
  int64_t base = (int64_t)blockIdx.x * kLifChunk;
#pragma unroll
  for (int j = 0; j < kLifGroups; ++j) {
    const int64_t q = std::min<int64_t>(base / kLifQ + j * 1024 + threadIdx.x, last_q);
#pragma unroll
    for (int h = 0; h < NL; ++h) x[j][h] = rec4[NL * q + h];
  }
  {
    const int w4 = ws / 4, n4 = R * w4;
    uint4 tmp[kLifCopy];
#pragma unroll
    for (int j = 0; j < kLifCopy; ++j) {
      const int i = min((int)threadIdx.x + j * 1024, n4 - 1);
      const int d = i / w4 + 1;
      tmp[j] = bits[(size_t)((t - d + R) % R) * w4 + (i - (d - 1) * w4)];
    }
#pragma unroll
    for (int j = 0; j < kLifCopy; ++j) {
      const int i = (int)threadIdx.x + j * 1024;
      if (i < n4) sb4[i] = t >= i / w4 + 1 ? tmp[j] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __syncthreads();
  for (; base < E; base += stride) {
    int4 xn[kLifGroups][NL];
#pragma unroll
    for (int j = 0; j < kLifGroups; ++j) {
      const int64_t q = std::min<int64_t>((base + stride) / kLifQ + j * 1024 + threadIdx.x, last_q);
#pragma unroll
      for (int h = 0; h < NL; ++h) xn[j][h] = rec4[NL * q + h];
    }
    int r[kLifGroups][kLifQ], c[kLifGroups][kLifQ];
#pragma unroll
    for (int j = 0; j < kLifGroups; ++j) {
      const int64_t p = base + kLifQ * (j * 1024 + (int64_t)threadIdx.x);
      int xs[2 * kLifQ];
#pragma unroll
      for (int h = 0; h < NL; ++h) {
        xs[4 * h] = x[j][h].x;
        xs[4 * h + 1] = x[j][h].y;
        xs[4 * h + 2] = x[j][h].z;
        xs[4 * h + 3] = x[j][h].w;
      }
#pragma unroll
      for (int i = 0; i < kLifQ; ++i) {
        // a position past the records reads word 0 and counts nothing
        const bool live = p + i < E;
        const uint32_t xx = live ? (uint32_t)xs[2 * i] : 0u, yy = live ? (uint32_t)xs[2 * i + 1] : 0u;
        r[j][i] = live ? lif_rec_row((int)xx, (int)yy) : -1;
        const uint32_t w = sb[(int)((yy >> 16) & 15u) * ws + (int)((xx & 0xFFFFFu) >> 5)];
        c[j][i] = live && ((w >> (xx & 31u)) & 1u) ? (int)(int16_t)(yy & 0xFFFFu) : 0;
      }
    }
    int rprev[kLifGroups], Pin[kLifGroups];
#pragma unroll
    for (int j = 0; j < kLifGroups; ++j) rprev[j] = __shfl_up(r[j][kLifQ - 1], 1);
#pragma unroll
    for (int j = 0; j < kLifGroups; ++j) {
      int tsum = 0;
#pragma unroll
      for (int i = 0; i < kLifQ; ++i) tsum += c[j][i];
      Pin[j] = wave_prefix_sum(tsum, lane);
    }
#pragma unroll
    for (int j = 0; j < kLifGroups; ++j) {
      // prefixes at each position (Ex: before the lane's first), run starts
      // (the first position against the previous lane's last), the prefix
      // before the lane's last run start (fetched by the lanes whose first
      // run continues from an earlier lane; lane 0 always starts a run)
      int P[kLifQ];
      bool st[kLifQ];
      int run = 0;
#pragma unroll
      for (int i = 0; i < kLifQ; ++i) run += c[j][i];
      const int Ex = Pin[j] - run;
      int acc_i = Ex;
#pragma unroll
      for (int i = 0; i < kLifQ; ++i) {
        acc_i += c[j][i];
        P[i] = acc_i;
        st[i] = i == 0 ? (lane == 0 || rprev[j] != r[j][0]) : r[j][i] != r[j][i - 1];
      }
      bool any = false;
      int before_last = Ex;
#pragma unroll
      for (int i = 0; i < kLifQ; ++i)
        if (st[i]) {
          any = true;
          before_last = i == 0 ? Ex : P[i - 1];
        }
      const unsigned long long S0 = __ballot(st[0]);
      const unsigned long long F = __ballot(any);
      const unsigned long long below = F & ((1ull << lane) - 1ull);
      const int m = below ? 63 - __clzll(below) : 0;
      const int bprev = __shfl(before_last, m);
      int before = bprev;
#pragma unroll
      for (int i = 0; i < kLifQ; ++i) {
        if (st[i]) before = i == 0 ? Ex : P[i - 1];
        // a position ends a run when the next one starts one (for the last
        // position: the next lane's first, or the end of the wave's group)
        const bool end = i + 1 < kLifQ ? st[i + 1] : (lane == 63 || (((S0 >> lane) >> 1) & 1ull) != 0);
        const int sum = P[i] - before;
        if (r[j][i] >= 0 && end && sum != 0)
          atomicAdd(reinterpret_cast<unsigned long long*>(&acc[r[j][i]]),
                    (unsigned long long)(long long)sum);
      }
    }
#pragma unroll
    for (int j = 0; j < kLifGroups; ++j)
#pragma unroll
      for (int h = 0; h < NL; ++h) x[j][h] = xn[j][h];
  }
}


// lif_gather with one byte read of the spike history per position (delays
// beyond the bit ring, or graphs too large for the LDS bit rows): a lane
// takes kLifQ neighbouring positions (their records in kLifQ / 2 16-byte
// loads, their rows in one), and the run sums are formed as in
// lif_gather_lds.
__global__ __launch_bounds__(256) void lif_gather(const int2* __restrict__ rec,
                                                  const int32_t* __restrict__ dst, int64_t E,
                                                  int64_t N, int t,
                                                  const uint8_t* __restrict__ spikes,
                                                  long long* __restrict__ acc) {
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t p = g * kLifQ;
  // (groups past the records load the last group, within the spare bytes)
  const int64_t q = std::min<int64_t>(g, (E - 1) / kLifQ);
  constexpr int NL = kLifQ / 2;
  const int4* rec4 = reinterpret_cast<const int4*>(rec);
  int xs[2 * kLifQ];
#pragma unroll
  for (int h = 0; h < NL; ++h) {
    const int4 v = rec4[NL * q + h];
    xs[4 * h] = v.x;
    xs[4 * h + 1] = v.y;
    xs[4 * h + 2] = v.z;
    xs[4 * h + 3] = v.w;
  }
  static_assert(kLifQ == 4, "one 16-byte load of rows per group");
  const int4 rd = reinterpret_cast<const int4*>(dst)[q];
  const int rows[kLifQ] = {rd.x, rd.y, rd.z, rd.w};
  int r[kLifQ], c[kLifQ];
#pragma unroll
  for (int i = 0; i < kLifQ; ++i) {
    const bool live = p + i < E;
    const uint32_t x = (uint32_t)xs[2 * i], y = (uint32_t)xs[2 * i + 1];
    const int d = (int)(y >> 16);
    r[i] = live ? rows[i] : -1;
    c[i] = live && t >= d && spikes[(size_t)(t - d) * N + x] ? (int)(int16_t)(y & 0xFFFFu) : 0;
  }
  const int rprev = __shfl_up(r[kLifQ - 1], 1);
  int tsum = 0;
#pragma unroll
  for (int i = 0; i < kLifQ; ++i) tsum += c[i];
  const int Pin = wave_prefix_sum(tsum, lane);
  const int Ex = Pin - tsum;
  int P[kLifQ];
  bool st[kLifQ];
  int run = Ex;
#pragma unroll
  for (int i = 0; i < kLifQ; ++i) {
    run += c[i];
    P[i] = run;
    st[i] = i == 0 ? (lane == 0 || rprev != r[0]) : r[i] != r[i - 1];
  }
  bool any = false;
  int before_last = Ex;
#pragma unroll
  for (int i = 0; i < kLifQ; ++i)
    if (st[i]) {
      any = true;
      before_last = i == 0 ? Ex : P[i - 1];
    }
  const unsigned long long S0 = __ballot(st[0]);
  const unsigned long long F = __ballot(any);
  const unsigned long long below = F & ((1ull << lane) - 1ull);
  const int bprev = __shfl(before_last, below ? 63 - __clzll(below) : 0);
  int before = bprev;
#pragma unroll
  for (int i = 0; i < kLifQ; ++i) {
    if (st[i]) before = i == 0 ? Ex : P[i - 1];
    const bool end = i + 1 < kLifQ ? st[i + 1] : (lane == 63 || (((S0 >> lane) >> 1) & 1ull) != 0);
    const int sum = P[i] - before;
    if (r[i] >= 0 && end && sum != 0)
      atomicAdd(reinterpret_cast<unsigned long long*>(&acc[r[i]]),
                (unsigned long long)(long long)sum);
  }
}

struct LifParams {
  int32_t threshold, reset, refractory, nshift;
  int32_t shift[8];
};

// With bits set (the LDS lookups are in use), the step's spikes also go into
// slot t % R of the bit ring (slots ws words apart): one ballot per wave, bit
// i % 32 of word i / 32 for neuron i.  Every lane takes part in the ballot, so no lane returns early.
__global__ __launch_bounds__(256) void lif_update(int64_t N, int t, LifParams p,
                                                  long long* __restrict__ acc,
                                                  int32_t* __restrict__ v, int32_t* __restrict__ r,
                                                  uint8_t* __restrict__ spikes,
                                                  int32_t* __restrict__ potentials,
                                                  uint32_t* __restrict__ bits, int64_t ws,
                                                  int R, int32_t* __restrict__ flags) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint8_t s = 0;
  if (i < N) {
    const long long in = acc[i];
    acc[i] = 0;
    int32_t vi = v[i];
    int32_t ri = r[i];
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
  if (bits != nullptr) {
    const unsigned long long m = __ballot(s != 0);
    const int lane = threadIdx.x & 63;
    const int64_t wd = i >> 5;  // lanes 0 and 32 start a word
    if ((lane & 31) == 0 && wd < (N + 31) / 32)
      bits[(size_t)(t % R) * ws + wd] = (uint32_t)(lane != 0 ? (m >> 32) : m);
  }
}

inline unsigned blocks(int64_t n) { return (unsigned)std::max<int64_t>(1, (n + 255) / 256); }

// CK_LIF_LDS=0 in the environment keeps the byte lookups (lif_gather) for
// every run; read on each call.
bool lif_lds_enabled() {
  const char* e = std::getenv("CK_LIF_LDS");
  return !(e && e[0] == '0' && e[1] == 0);
}

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

namespace {

struct LifBufs {
  int2* rec;
  int32_t* dst;
  uint32_t* words;
  long long* acc;
  int32_t *v, *r, *flags;
  uint32_t* bits;
};

LifBufs lif_bufs(void* workspace, const LifWs& ws) {
  char* b = static_cast<char*>(workspace);
  return LifBufs{reinterpret_cast<int2*>(b + ws.rec),       reinterpret_cast<int32_t*>(b + ws.dst),
                 reinterpret_cast<uint32_t*>(b + ws.words), reinterpret_cast<long long*>(b + ws.acc),
                 reinterpret_cast<int32_t*>(b + ws.v),      reinterpret_cast<int32_t*>(b + ws.r),
                 reinterpret_cast<int32_t*>(b + ws.flags),  reinterpret_cast<uint32_t*>(b + ws.bits)};
}

ck_status lif_check_ws(const ck_graph* g, void* workspace, size_t workspace_bytes, LifWs* ws) {
  if (!workspace) {
    set_error("workspace is NULL");
    return CK_ERR_NULL_ARG;
  }
  const ck_status rc = check_aligned(workspace, "workspace");
  if (rc != CK_OK) return rc;
  *ws = lif_layout(g->N, g->E);
  if (workspace_bytes < ws->total) {
    set_error("workspace of %zu bytes is below the %zu required", workspace_bytes, ws->total);
    return CK_ERR_WORKSPACE;
  }
  return CK_OK;
}

int32_t lif_graph_tag(const ck_graph* g) {
  return (int32_t)(uint32_t)(reinterpret_cast<uintptr_t>(g->row_ptr) & 0xFFFFFFFFu);
}

// Validate the delays, write the destinations and the CSR-order records, and
// leave the mark; *R = the bit rows of the LDS lookups (0: byte lookups).
ck_status lif_prepare_body(const ck_graph* g, const int16_t* impulses, const int32_t* delays,
                           const LifBufs& b, hipStream_t stream, int* R) {
  const int64_t N = g->N, E = g->E;
  *R = 0;
  lif_flags<<<1, 64, 0, stream>>>(b.flags, 0, 0, 0, 0, 0);
  if (E > 0) {
    lif_words<<<std::min(blocks(E), 4096u), 256, 0, stream>>>(impulses, delays, E, b.words,
                                                              b.flags);
    lif_rows<<<blocks(N * 64), 256, 0, stream>>>(g->row_ptr, N, b.dst);
    CK_HIP_TRY(hipGetLastError());
    int32_t fl[3] = {0, 0, 0};
    CK_HIP_TRY(hipMemcpyAsync(fl, b.flags, sizeof(fl), hipMemcpyDeviceToHost, stream));
    CK_HIP_TRY(hipStreamSynchronize(stream));
    if (fl[1]) {
      set_error("an edge delay is outside [1, 32767]");
      return CK_ERR_BAD_VALUE;
    }
    // (the 128 KB bound implies N <= 2^20, which the 20-bit sources and rows
    // of lif_pack_lds need; it is checked on its own all the same)
    if (fl[2] >= 1 && fl[2] <= kLifRing && (int64_t)fl[2] * lif_row_words(N) * 4 <= kLifLdsBytes &&
        N <= (int64_t(1) << 20) && lif_lds_enabled())
      *R = fl[2];
    if (*R > 0)
      lif_pack_lds<<<blocks(E), 256, 0, stream>>>(g->col_idx, g->perm, b.words, b.dst, E, b.rec);
    else
      lif_pack<<<blocks(E), 256, 0, stream>>>(g->col_idx, g->perm, b.words, E, b.rec);
  }
  lif_flags<<<1, 64, 0, stream>>>(b.flags, kLifMark, (int32_t)(E & INT_MAX),
                                  (int32_t)(N & INT_MAX), *R, lif_graph_tag(g));
  CK_HIP_TRY(hipGetLastError());
  return CK_OK;
}

ck_status lif_params(const ck_lif_params* params, LifParams* p) {
  if (params->num_decay_shifts < 0 || params->num_decay_shifts > 8 ||
      params->refractory_steps < 0) {
    set_error("num_decay_shifts must be in [0, 8] and refractory_steps >= 0");
    return CK_ERR_BAD_VALUE;
  }
  *p = LifParams{};
  p->threshold = params->threshold;
  p->reset = params->reset;
  p->refractory = params->refractory_steps;
  p->nshift = params->num_decay_shifts;
  for (int j = 0; j < p->nshift; ++j) {
    if (params->decay_shifts[j] < 0 || params->decay_shifts[j] > 31) {
      set_error("decay shift %d is outside [0, 31]", params->decay_shifts[j]);
      return CK_ERR_BAD_VALUE;
    }
    p->shift[j] = params->decay_shifts[j];
  }
  return CK_OK;
}

// T steps on prepared records (R as the prepare chose), then the overflow
// check.
ck_status lif_run_body(const ck_graph* g, const LifParams& p, const int32_t* v0, int64_t T,
                       uint8_t* spikes, int32_t* potentials, int64_t* overflow_step,
                       const LifBufs& b, int R, hipStream_t stream) {
  const int64_t N = g->N, E = g->E;
  lif_init<<<blocks(N), 256, 0, stream>>>(v0, N, b.v, b.r, b.acc, b.flags);
  const int64_t wsw = lif_row_words(N);
  const int lds = R > 0 ? (int)(R * wsw * 4) : 0;
  unsigned lds_grid = 0;
  if (R > 0) {
    CK_HIP_TRY(hipFuncSetAttribute((const void*)lif_gather_lds,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, lds));
    int cus = 0;
    CK_HIP_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, g->device));
    const int per_cu = lds <= 80 * 1024 ? 2 : 1;  // workgroups whose LDS fits a 160 KB CU
    const int64_t chunks = (E + kLifChunk - 1) / kLifChunk;
    lds_grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>((int64_t)cus * per_cu, chunks));
  }
  ck_status rc = CK_OK;
  for (int64_t t = 0; t < T; ++t) {
    if (t >= 1 && E > 0) {
      rc = timed_launch(g_profile.lif_gather, stream, [&] {
        if (R > 0)
          lif_gather_lds<<<lds_grid, 1024, lds, stream>>>(b.rec, E, (int)wsw, (int)t, R,
                                                          reinterpret_cast<const uint4*>(b.bits),
                                                          b.acc);
        else
          lif_gather<<<blocks((E + kLifQ - 1) / kLifQ), 256, 0, stream>>>(b.rec, b.dst, E, N,
                                                                         (int)t, spikes, b.acc);
      });
      if (rc != CK_OK) return rc;
    }
    rc = timed_launch(g_profile.lif_update, stream, [&] {
      lif_update<<<blocks(N), 256, 0, stream>>>(N, (int)t, p, b.acc, b.v, b.r, spikes, potentials,
                                               R > 0 ? b.bits : nullptr, wsw, std::max(R, 1),
                                               b.flags);
    });
    if (rc != CK_OK) return rc;
  }
  CK_HIP_TRY(hipGetLastError());
  int32_t fl[1] = {0};
  CK_HIP_TRY(hipMemcpyAsync(fl, b.flags, sizeof(fl), hipMemcpyDeviceToHost, stream));
  CK_HIP_TRY(hipStreamSynchronize(stream));
  if (fl[0] != INT_MAX) {
    if (overflow_step) *overflow_step = fl[0];
    set_error("a membrane potential left the int32 range at timestep %d; the run is rejected "
              "(outputs of that step and later are unspecified)", fl[0]);
    return CK_ERR_OVERFLOW;
  }
  return CK_OK;
}

ck_status lif_run_checks(const ck_lif_params* params, const int32_t* v0, int64_t T,
                         uint8_t* spikes, int32_t* potentials) {
  if (T <= 0 || T > INT_MAX) {
    set_error("T must be in [1, 2^31 - 1] (got %lld)", (long long)T);
    return CK_ERR_BAD_SIZE;
  }
  if (!params || !v0 || !spikes || !potentials) {
    set_error("NULL pointer for a non-empty tensor in the LIF run");
    return CK_ERR_NULL_ARG;
  }
  return CK_OK;
}

}  // namespace

extern "C" ck_status ck_lif_prepare(ck_graph_t g, const int16_t* impulses, const int32_t* delays,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  ck_status rc = check_graph(g);
  if (rc != CK_OK) return rc;
  if (g->E > 0 && (!impulses || !delays)) {
    set_error("impulses or delays is NULL");
    return CK_ERR_NULL_ARG;
  }
  LifWs ws;
  rc = lif_check_ws(g, workspace, workspace_bytes, &ws);
  if (rc != CK_OK) return rc;
  int R = 0;
  rc = lif_prepare_body(g, impulses, delays, lif_bufs(workspace, ws), stream, &R);
  if (rc != CK_OK) return rc;
  CK_HIP_TRY(hipStreamSynchronize(stream));
  return CK_OK;
}

extern "C" ck_status ck_lif_run(ck_graph_t g, const ck_lif_params* params, const int32_t* v0,
                                int64_t T, uint8_t* spikes, int32_t* potentials,
                                int64_t* overflow_step, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  clear_error();
  ck_status rc = check_graph(g);
  if (rc != CK_OK) return rc;
  if (overflow_step) *overflow_step = -1;
  rc = lif_run_checks(params, v0, T, spikes, potentials);
  if (rc != CK_OK) return rc;
  LifParams p;
  rc = lif_params(params, &p);
  if (rc != CK_OK) return rc;
  LifWs ws;
  rc = lif_check_ws(g, workspace, workspace_bytes, &ws);
  if (rc != CK_OK) return rc;
  const LifBufs b = lif_bufs(workspace, ws);
  int32_t mk[5] = {0, 0, 0, 0, 0};
  CK_HIP_TRY(hipMemcpyAsync(mk, b.flags + 3, sizeof(mk), hipMemcpyDeviceToHost, stream));
  CK_HIP_TRY(hipStreamSynchronize(stream));
  if (mk[0] != kLifMark || mk[1] != (int32_t)(g->E & INT_MAX) ||
      mk[2] != (int32_t)(g->N & INT_MAX) || mk[3] < 0 || mk[3] > kLifRing ||
      mk[4] != lif_graph_tag(g)) {
    set_error("the workspace holds no prepared synapses of this graph (ck_lif_prepare)");
    return CK_ERR_BAD_VALUE;
  }
  return lif_run_body(g, p, v0, T, spikes, potentials, overflow_step, b, mk[3], stream);
}

extern "C" ck_status ck_lif_forward(ck_graph_t g, const int16_t* impulses, const int32_t* delays,
                                    const ck_lif_params* params, const int32_t* v0, int64_t T,
                                    uint8_t* spikes, int32_t* potentials, int64_t* overflow_step,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  ck_status rc = check_graph(g);
  if (rc != CK_OK) return rc;
  if (overflow_step) *overflow_step = -1;
  rc = lif_run_checks(params, v0, T, spikes, potentials);
  if (rc != CK_OK) return rc;
  if (g->E > 0 && (!impulses || !delays)) {
    set_error("NULL pointer for a non-empty tensor in the LIF forward");
    return CK_ERR_NULL_ARG;
  }
  LifParams p;
  rc = lif_params(params, &p);
  if (rc != CK_OK) return rc;
  LifWs ws;
  rc = lif_check_ws(g, workspace, workspace_bytes, &ws);
  if (rc != CK_OK) return rc;
  const LifBufs b = lif_bufs(workspace, ws);
  int R = 0;
  rc = lif_prepare_body(g, impulses, delays, b, stream, &R);
  if (rc != CK_OK) return rc;
  return lif_run_body(g, p, v0, T, spikes, potentials, overflow_step, b, R, stream);
}
