// blocked.hip -- the recurrence, one microstep per launch pair, for graphs
// whose [N][Bp] state plane is far larger than the L2 caches (the leaky-tanh
// update of the connectome-kernels README introduction; node-major [N, B]
// rows gathered per edge and long rows split, README "Design notes"; the
// whole-connectome scale of soup-connectome, "Status at a glance").
//
// The gathered nodes are cut into 8 blocks, one per XCD (schedule.h, blocked
// plan): the workgroups of XCD x gather only rows of block x, whose slice of
// the plane (N/8 rows) stays in that XCD's 4 MB L2, while the edge list and
// the partial rows stream past it with non-temporal accesses.  A microstep is
// two launches:
//   part: each work item (at most 64 edges of one row into one block) sums
//         its edge terms into one partial row of Bp floats;
//   epi:  each row adds its partial rows in item order and runs the row's
//         elementwise update.
// Forward:  a[i] = sum_k v_k h[src_k] + drive[i] + bias[i] (fp64 item sums,
//           rounded to fp32 per item, added in fp64, rounded once);
//           h'[i] = (1 - leak[i]) h[i] + leak[i] tanh(a[i]).
// Backward (rows of the transposed CSR, per source node j; items over the
// destination blocks): part sums v_k ga[dst_k] into the partial row and adds
// <ga[dst_k], h^(s-1)[j]> to the edge gradient of every edge it holds; epi
// forms g^(s-1)[j] = (1 - leak[j]) g^(s)[j] + sum of partials (+ the upstream
// gradient entering there) and the elementwise pass of microstep s-1 (leak and
// bias row sums, drive gradient), or the initial-state gradient.
// No floating-point atomics; every sum is taken in a fixed order, so results
// are bitwise reproducible.
#include <algorithm>
#include <vector>

#include "ck_internal.h"
#include "device_math.h"

namespace ckhip {
namespace {

// Buffer resource over `bytes` bytes at `base`: an access at an offset past
// the range returns zero (loads) or is dropped (stores) without touching
// memory, so masked lanes pass kOut instead of branching.
constexpr uint32_t kOut = 0xFFFFFFF0u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t brsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ float4 ld_row4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// The streamed accesses (edges, partial rows, edge gradients) are
// non-temporal, so they do not push the gathered slice out of the L2.  They
// are plain global accesses: the same loads as non-temporal buffer loads
// measured twice as slow (the edge loads, whose lanes share addresses).
// (a wave-uniform base and a 32-bit byte offset: one address register)
__device__ __forceinline__ int2 ld_edge(const int2* pe, uint32_t q) {
  const long long v = __builtin_nontemporal_load(
      reinterpret_cast<const long long*>(reinterpret_cast<const char*>(pe) + q * 8u));
  return make_int2((int)(v & 0xffffffffll), (int)(v >> 32));
}
__device__ __forceinline__ float ld_f(const float* p) { return __builtin_nontemporal_load(p); }
// Partial rows: non-temporal stores, issued the same way on every path (a
// lane without an item writes scratch row `items` instead of branching).
// Stores that stay in the L2 measured slower here: they push out the
// gathered slice.
typedef float f4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st_row4(float4 v, float* base, size_t off4) {
  __builtin_nontemporal_store(f4v{v.x, v.y, v.z, v.w}, reinterpret_cast<f4v*>(base) + off4);
}
// Edge gradients: a buffer store, which drops a lane passing kOut (the
// non-temporal form measured slower for these 4-byte stores).
__device__ __forceinline__ void st_fb(float v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
}

constexpr bool pow2(int x) { return (x & (x - 1)) == 0; }

// Sum over the L lanes of this lane's slot (slot = lane / L); every lane of
// the slot receives the same bits.  Powers of two below 32 use DPP lane moves
// inside 16-lane rows; other widths read the slot's lanes in order.
template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               CTRL, 0xF, 0xF, false));
}
template <int L>
__device__ __forceinline__ float slot_total(float x, int slot) {
  if constexpr (L == 1) {
    return x;
  } else if constexpr (pow2(L) && L <= 16) {
    x += dppf<0xB1>(x);                           // quad_perm [1,0,3,2]
    if constexpr (L >= 4) x += dppf<0x4E>(x);     // quad_perm [2,3,0,1]
    if constexpr (L >= 8) x += dppf<0x141>(x);    // row_half_mirror
    if constexpr (L >= 16) x += dppf<0x140>(x);   // row_mirror
    return x;
  } else {
    // (rolled: unrolled, the shuffles of every edge of a round are hoisted
    // together and spill)
    float s = __shfl(x, slot * L);
#pragma unroll 1
    for (int i = 1; i < L; ++i) s += __shfl(x, slot * L + i);
    return s;
  }
}

// Lane roles of both part kernels: a wave takes P = 64 / L items per pass,
// item q on lanes [q L, q L + L), lane sub of it holding columns
// [4 sub, 4 sub + 4) (L = Bp / 4).
struct BlkLanes {
  int lane, wave, slot, sub;
  bool ok;  // the lane belongs to one of the P slots
};
template <int L>
__device__ __forceinline__ BlkLanes blk_lanes() {
  BlkLanes r;
  r.lane = threadIdx.x & 63;
  r.wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  r.slot = r.lane / L;
  r.sub = r.lane % L;
  r.ok = r.slot < 64 / L;
  return r;
}

struct BlkPartArgs {
  const int4* table;     // [num_wgs * kBlkWaves][KB + kBlkPad] items, largest first per wave
  int KB;
  const int2* pe;        // [E + 1] {gathered node, value bits}, blocked edge order, then a sentinel
  uint32_t sentinel;     // E: the sentinel's index
  const float* src;      // gathered plane [N][Bp]: h^(s-1) (forward) or ga^(s) (backward)
  uint32_t src_bytes;
  float* partial;        // [items + 1][Bp] (row `items`: scratch for lanes without an item)
  int64_t items;
  // backward only
  const float* h_sm1;    // h^(s-1) [N][Bp], the row's own state for the edge gradient
  float* gv;             // [E] edge gradient, blocked edge order
  uint32_t gv_bytes;
  int first_gv;          // 1: overwrite gv instead of adding to it
  int Bp;
};

// Both part kernels walk a wave's items P = 64 / L at a time (a pass) in
// rounds of U edges per item, software-pipelined: each round's edges are
// requested one round ahead, with the gathers of the round before, and the
// next pass's first edges during the current pass's last round.  A wave
// stages its item list in LDS, kBlkStage entries at a time, so reading an
// item never waits for vector loads.  A round's edge loads are the same
// whatever its items' counts (lanes past their item's count read the
// sentinel entry), and gathers no item of the pass reaches are skipped by a
// wave-uniform test, so the compiler can wait for exactly the loads a step
// needs instead of for all of them.
constexpr int kBlkStage = 256;  // items a wave stages in LDS at a time (4 KB)

// Stage entries [base, base + n) of the wave's list (n <= kBlkStage; entries
// past the list's padding read as padding) into `my`, and make them visible
// to the wave's own later LDS reads.
__device__ __forceinline__ void blk_stage(int4* my, const int4* tb, int limit, int base, int n,
                                          int lane) {
  for (int i = lane; i < n; i += 64)
    my[i] = base + i < limit ? tb[base + i] : make_int4(-1, 0, 0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
}

// Rounds of the forward part kernel: a round takes U = R * L edges of each
// item of a pass (16 at L = 8 and 16, where the registers allow; at least 8
// otherwise); lane sub of a slot loads edges sub, sub + L, ... of the round,
// and the slot's lanes share them through lane shuffles -- R edge loads per
// round instead of one per edge (the loads are what the address unit spends
// its time on).
template <int L>
constexpr int blk_r() { return L == 8 ? 2 : L >= 8 ? 1 : (8 + L - 1) / L; }

// This lane's edges of round r of an item: edges j = q L + sub (q < R) of
// the round's U, the sentinel past its count or U.
template <int R, int L, int U = R * L>
__device__ __forceinline__ void blk_own(int2 (&own)[R], const int2* pe, int4 item, int r, int sub,
                                        uint32_t sentinel) {
  const int rem = item.x >= 0 ? item.z - r * U : 0;
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const int j = q * L + sub;
    own[q] = ld_edge(pe, j < U && j < rem ? (uint32_t)(item.y + r * U + j) : sentinel);
  }
}

// Forward part: the item's sum of v_k h^(s-1)[src_k] (each round's terms in
// fp32, added to an fp64 sum), stored as one fp32 partial row.
template <int L>
__global__ __launch_bounds__(kBlkWaves * 64) void blk_fwd_part(BlkPartArgs p) {
  constexpr int P = 64 / L, R = blk_r<L>(), U = R * L;
  constexpr int SP = kBlkStage / P * P;  // items staged at a time: whole passes
  __shared__ int4 s_items[kBlkWaves][kBlkStage];
  const BlkLanes ln = blk_lanes<L>();
  const __amdgpu_buffer_rsrc_t hr = brsrc(p.src, p.src_bytes);
  const uint32_t rowb = (uint32_t)p.Bp * 4u, colb = (uint32_t)ln.sub * 16u;
  const int4* tb = p.table + ((size_t)blockIdx.x * kBlkWaves + ln.wave) * (p.KB + kBlkPad);
  int4* my = s_items[ln.wave];
  const int4 idle = make_int4(-1, 0, 0, 0);
  const int sbase = ln.slot * L;  // the slot's first lane
  for (int base = 0; base < p.KB; base += SP) {
    blk_stage(my, tb, p.KB + kBlkPad, base, SP, ln.lane);
    int4 item = ln.ok ? my[ln.slot] : idle;
    int2 own[R];
    blk_own<R, L>(own, p.pe, item, 0, ln.sub, p.sentinel);
    int cm = __builtin_amdgcn_readfirstlane(item.x >= 0 ? item.z : 0);  // slot 0: the largest
    for (int it = 0; it < SP && cm > 0; it += P) {
      const int4 next = (ln.ok && it + P < SP) ? my[it + P + ln.slot] : idle;
      const int rounds = (cm + U - 1) / U;
      double4 acc = d4(0.0);
      for (int r = 0; r < rounds; ++r) {
        // (edges no item of the pass has, j >= cm - r U, cost nothing: the
        // bound is wave-uniform)
        const int live = cm - r * U;
        uint32_t off[U];
        float w[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
          off[j] = __umul24((uint32_t)__shfl(own[j / L].x, sbase + j % L), rowb) + colb;
          w[j] = __int_as_float(__shfl(own[j / L].y, sbase + j % L));
        }
        float4 v[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
          v[j] = f4(0.f);
          if (j < live) v[j] = ld_row4(hr, off[j]);
        }
        if (r + 1 < rounds) blk_own<R, L>(own, p.pe, item, r + 1, ln.sub, p.sentinel);
        else blk_own<R, L>(own, p.pe, next, 0, ln.sub, p.sentinel);
        float4 racc = f4(0.f);
#pragma unroll
        for (int j = 0; j < U; ++j)
          if (j < live) racc = fma4(w[j], v[j], racc);
        acc.x += (double)racc.x;
        acc.y += (double)racc.y;
        acc.z += (double)racc.z;
        acc.w += (double)racc.w;
      }
      st_row4(make_float4((float)acc.x, (float)acc.y, (float)acc.z, (float)acc.w), p.partial,
              (size_t)(item.x >= 0 ? item.w : p.items) * (p.Bp / 4) + ln.sub);
      item = next;
      cm = __builtin_amdgcn_readfirstlane(item.x >= 0 ? item.z : 0);
    }
    if (my[SP - 1].x < 0) break;  // the list (a prefix of the entries) ended in this stage
  }
}

// Backward part: the item's sum of v_k ga^(s)[dst_k] (fp32) as one partial
// row, and gv_k += <ga^(s)[dst_k], h^(s-1)[j]> for each of its edges.  As in
// the forward, lane sub of a slot loads edges sub, sub + L, ... of a round
// (and their old gradients) and shares the edges through lane shuffles; the
// edge dot products are summed over the slot's lanes, and each lane keeps the
// gradients of the edges it loaded.
template <int L>
__global__ __launch_bounds__(kBlkWaves * 64) void blk_bwd_part(BlkPartArgs p) {
  // 8 edges per round from L = 8 up (lanes sub >= 8 load none), else R per lane
  constexpr int P = 64 / L, R = L >= 8 ? 1 : (8 + L - 1) / L, U = L >= 8 ? 8 : R * L;
  constexpr int SP = kBlkStage / P * P;
  __shared__ int4 s_items[kBlkWaves][kBlkStage];
  const BlkLanes ln = blk_lanes<L>();
  const __amdgpu_buffer_rsrc_t gr = brsrc(p.src, p.src_bytes);
  const __amdgpu_buffer_rsrc_t hsr = brsrc(p.h_sm1, p.src_bytes);
  const __amdgpu_buffer_rsrc_t vr = brsrc(p.gv, p.gv_bytes);
  const uint32_t rowb = (uint32_t)p.Bp * 4u, colb = (uint32_t)ln.sub * 16u;
  const int4* tb = p.table + ((size_t)blockIdx.x * kBlkWaves + ln.wave) * (p.KB + kBlkPad);
  int4* my = s_items[ln.wave];
  const int4 idle = make_int4(-1, 0, 0, 0);
  const int sbase = ln.slot * L;
  // the old gradients of this lane's edges of round r (read whether or not
  // the edge exists, from an address inside the item or the sentinel's
  // neighbour 0, so that every round issues the same loads)
  auto olds = [&](float (&gold)[R], int4 it4, int r) {
    const int rem = it4.x >= 0 ? it4.z - r * U : 0;
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int j = q * L + ln.sub;
      gold[q] = ld_f(p.gv + (j < U && j < rem ? it4.y + r * U + j : 0));
    }
  };
  auto own_row = [&](int4 it4) {
    return ld_row4(hsr, it4.x >= 0 ? (uint32_t)it4.x * rowb + colb : kOut);
  };
  for (int base = 0; base < p.KB; base += SP) {
    blk_stage(my, tb, p.KB + kBlkPad, base, SP, ln.lane);
    int4 item = ln.ok ? my[ln.slot] : idle;
    int2 own[R];
    float gold[R];
    blk_own<R, L, U>(own, p.pe, item, 0, ln.sub, p.sentinel);
    olds(gold, item, 0);
    float4 hj = own_row(item);
    int cm = __builtin_amdgcn_readfirstlane(item.x >= 0 ? item.z : 0);
    for (int it = 0; it < SP && cm > 0; it += P) {
      const int4 next = (ln.ok && it + P < SP) ? my[it + P + ln.slot] : idle;
      const int cnt = item.x >= 0 ? item.z : 0;
      const int rounds = (cm + U - 1) / U;
      float4 hn = f4(0.f);  // the next pass's own rows, requested with its first edges
      float4 acc = f4(0.f);
      for (int r = 0; r < rounds; ++r) {
        const int live = cm - r * U;
        uint32_t off[U];
        float w[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
          off[j] = __umul24((uint32_t)__shfl(own[j / L].x, sbase + j % L), rowb) + colb;
          w[j] = __int_as_float(__shfl(own[j / L].y, sbase + j % L));
        }
        float4 g4[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
          g4[j] = f4(0.f);
          if (j < live) g4[j] = ld_row4(gr, off[j]);
        }
        float gcur[R];
#pragma unroll
        for (int q = 0; q < R; ++q) gcur[q] = p.first_gv ? 0.f : gold[q];
        const int4 src4 = r + 1 < rounds ? item : next;
        const int rn = r + 1 < rounds ? r + 1 : 0;
        blk_own<R, L, U>(own, p.pe, src4, rn, ln.sub, p.sentinel);
        olds(gold, src4, rn);
        if (r + 1 == rounds) hn = own_row(next);
        float mine[R];
#pragma unroll
        for (int q = 0; q < R; ++q) mine[q] = 0.f;
#pragma unroll
        for (int j = 0; j < U; ++j) {
          if (j < live) {
            acc = fma4(w[j], g4[j], acc);
            const float tot = slot_total<L>(dot4(g4[j], hj), ln.slot);
            if (ln.sub == j % L) mine[j / L] = tot;
          }
        }
#pragma unroll
        for (int q = 0; q < R; ++q) {
          const int j = q * L + ln.sub, k = r * U + j;
          st_fb(gcur[q] + mine[q], vr, j < U && k < cnt ? (uint32_t)(item.y + k) * 4u : kOut);
        }
      }
      st_row4(acc, p.partial, (size_t)(item.x >= 0 ? item.w : p.items) * (p.Bp / 4) + ln.sub);
      item = next;
      hj = hn;
      cm = __builtin_amdgcn_readfirstlane(item.x >= 0 ? item.z : 0);
    }
    if (my[SP - 1].x < 0) break;
  }
}

// Row mapping of both epilogue kernels: each wave holds 64 / L rows (lanes
// past them idle), so a row's L lanes never straddle two waves.
template <int L>
__device__ __forceinline__ int64_t epi_row(int& sub) {
  constexpr int RW = 64 / L;
  const int lane = threadIdx.x & 63;
  sub = lane % L;
  if (lane / L >= RW) return -1;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  return wave * RW + lane / L;
}
template <int L>
constexpr int64_t epi_threads(int64_t N) {
  return (N + 64 / L - 1) / (64 / L) * 64;
}

struct BlkFwdEpiArgs {
  const int32_t* row_items;  // [N + 1]
  const int32_t* item_ids;   // [items]: row i's partial rows are item_ids[row_items[i] ..]
  const float* partial;      // [items][Bp]
  const float* leak;
  const float* bias;
  const int32_t* input_slot;
  const float* drives_t;     // [n_in][B] of the current input step (nullptr if n_in == 0)
  const float* h_prev;       // [N][Bp]
  float* h_next;             // [N][Bp]
  float* a_next;             // [N][Bp]
  int N, B, Bp;
};

// a = (sum of the row's partial rows, in fp64) + drive + bias, rounded once;
// h' = (1 - leak) h + leak tanh(a); four columns per lane.
template <int L>
__global__ __launch_bounds__(256) void blk_fwd_epi(BlkFwdEpiArgs p) {
  int sub;
  const int64_t row = epi_row<L>(sub);
  if (row < 0 || row >= p.N) return;
  const int i0 = p.row_items[row], i1 = p.row_items[row + 1];
  const size_t w4 = (size_t)p.Bp / 4;  // float4 per row
  const float4* part = reinterpret_cast<const float4*>(p.partial);
  double4 acc = d4(0.0);
  // sixteen partial rows at a time (most rows have at most 16 items), all
  // requested at once (past the row's last item the loads repeat it and the
  // sums skip it); 16 measured faster than 8, 12 or 24
  for (int c = i0; c < i1; c += 16) {
    int id[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) id[u] = p.item_ids[min(c + u, i1 - 1)];
    float4 q[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) q[u] = part[(size_t)id[u] * w4 + sub];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const bool in = c + u < i1;
      acc.x += in ? (double)q[u].x : 0.0;
      acc.y += in ? (double)q[u].y : 0.0;
      acc.z += in ? (double)q[u].z : 0.0;
      acc.w += in ? (double)q[u].w : 0.0;
    }
  }
  const float lam = p.leak[row], bi = p.bias[row];
  const int ks = p.input_slot[row];
  const size_t off = (size_t)row * w4 + sub;
  const float4 hp = reinterpret_cast<const float4*>(p.h_prev)[off];
  const double av[4] = {acc.x, acc.y, acc.z, acc.w};
  const float hv[4] = {hp.x, hp.y, hp.z, hp.w};
  float a[4], h[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = 4 * sub + q;
    const float dv = (ks >= 0 && c < p.B) ? p.drives_t[(size_t)ks * p.B + c] : 0.f;
    a[q] = (float)(av[q] + (double)dv + (double)bi);
    h[q] = (1.0f - lam) * hv[q] + lam * tanhf(a[q]);
  }
  reinterpret_cast<float4*>(p.a_next)[off] = make_float4(a[0], a[1], a[2], a[3]);
  reinterpret_cast<float4*>(p.h_next)[off] = make_float4(h[0], h[1], h[2], h[3]);
}

struct BlkBwdEpiArgs {
  const int32_t* row_items;  // [N + 1]
  const int32_t* item_ids;   // [items]
  const float* partial;      // [items][Bp]; nullptr: no edge pass (the seeding launch)
  const float* leak;
  const int32_t* input_slot;
  float* gh;                 // in: g^(s) (ignored without an edge pass), out: g^(s-1)
  const float* G_t;          // [N][Bp] upstream gradient entering at microstep s-1, or nullptr
  // elementwise pass of microstep s-1 (a_k1 == nullptr when s-1 == 0)
  const float* a_k1;         // a^(s-1)
  const float* h_k1;         // h^(s-2)
  float* ga_out;             // ga^(s-1)
  float* gdrives_t;          // [n_in][B] of input step t(s-1), accumulated
  float* gleak;              // [N] accumulated (overwritten when first_k1)
  float* gbias;              // [N]
  float* gstate0;            // [B][N], written when s-1 == 0
  int first_k1;
  int N, B, Bp;
};

// Sum over the L lanes of a row, exact in lane sub == 0.
template <int L>
__device__ __forceinline__ float row_lanes_sum(float x, int lane) {
  if constexpr (pow2(L)) {
#pragma unroll
    for (int m = 1; m < L; m <<= 1) x += __shfl_xor(x, m);
    return x;
  } else {
    const int base = lane - lane % L;
    float s = __shfl(x, base);
#pragma unroll
    for (int i = 1; i < L; ++i) s += __shfl(x, base + i);
    return s;
  }
}

// g^(s-1) = (1 - leak) g^(s) + (sum of the row's partial rows) (+ G entering
// at s-1), then the elementwise pass of microstep s-1, or the initial-state
// gradient when s-1 == 0; four columns per lane.
template <int L>
__global__ __launch_bounds__(256) void blk_bwd_epi(BlkBwdEpiArgs p) {
  int sub;
  const int64_t row0 = epi_row<L>(sub);
  const bool live = row0 >= 0 && row0 < p.N;
  const int64_t row = live ? row0 : 0;
  const int lane = threadIdx.x & 63;
  const size_t w4 = (size_t)p.Bp / 4;
  const size_t off = (size_t)row * w4 + sub;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f, bsum = 0.f;
  if (live) {
    if (p.partial != nullptr) {
      const float4* part = reinterpret_cast<const float4*>(p.partial);
      const int i0 = p.row_items[row], i1 = p.row_items[row + 1];
      for (int c = i0; c < i1; c += 8) {
        int id[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) id[u] = p.item_ids[min(c + u, i1 - 1)];
        float4 q[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) q[u] = part[(size_t)id[u] * w4 + sub];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const bool in = c + u < i1;
          acc[0] += in ? q[u].x : 0.f;
          acc[1] += in ? q[u].y : 0.f;
          acc[2] += in ? q[u].z : 0.f;
          acc[3] += in ? q[u].w : 0.f;
        }
      }
    }
    const float lam = p.leak[row];
    float gold[4] = {0.f, 0.f, 0.f, 0.f};
    if (p.partial != nullptr) {
      const float4 o = reinterpret_cast<const float4*>(p.gh)[off];
      gold[0] = o.x;
      gold[1] = o.y;
      gold[2] = o.z;
      gold[3] = o.w;
    }
    float gin[4] = {0.f, 0.f, 0.f, 0.f};
    if (p.G_t != nullptr) {  // (padding columns of the planes are zero)
      const float4 o = reinterpret_cast<const float4*>(p.G_t)[off];
      gin[0] = o.x;
      gin[1] = o.y;
      gin[2] = o.z;
      gin[3] = o.w;
    }
    float g[4], ga[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      g[q] = acc[q];
      if (p.partial != nullptr) g[q] = fmaf(1.0f - lam, gold[q], g[q]);
      if (p.G_t) g[q] += gin[q];
      ga[q] = 0.f;
    }
    if (p.a_k1 == nullptr) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 4 * sub + q;
        if (c < p.B) p.gstate0[(size_t)c * p.N + row] = g[q];
      }
    } else {
      const int ks = p.input_slot[row];
      const float4 ak = reinterpret_cast<const float4*>(p.a_k1)[off];
      const float4 qk = reinterpret_cast<const float4*>(p.h_k1)[off];
      const float av[4] = {ak.x, ak.y, ak.z, ak.w}, qv[4] = {qk.x, qk.y, qk.z, qk.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 4 * sub + q;
        if (c < p.B) {
          lsum += g[q] * (tanhf(av[q]) - qv[q]);
          ga[q] = g[q] * lam * sech2f(av[q]);
          bsum += ga[q];
          if (ks >= 0) {
            float* gd = p.gdrives_t + (size_t)ks * p.B + c;
            *gd = *gd + ga[q];
          }
        } else {
          g[q] = 0.f;
        }
      }
      reinterpret_cast<float4*>(p.gh)[off] = make_float4(g[0], g[1], g[2], g[3]);
      reinterpret_cast<float4*>(p.ga_out)[off] = make_float4(ga[0], ga[1], ga[2], ga[3]);
    }
  }
  if (p.a_k1 == nullptr) return;  // uniform over the launch
  lsum = row_lanes_sum<L>(lsum, lane);
  bsum = row_lanes_sum<L>(bsum, lane);
  if (live && sub == 0) {
    p.gleak[row] = p.first_k1 ? lsum : p.gleak[row] + lsum;
    p.gbias[row] = p.first_k1 ? bsum : p.gbias[row] + bsum;
  }
}

// pe[q] = {node[q], bits of values[perm[q]]} for the edges in blocked order,
// then pe[n] = the sentinel {kBlkNoNode, 0}
constexpr int32_t kBlkNoNode = (1 << 24) - 1;
__global__ void blk_pack(const float* __restrict__ values, const int32_t* __restrict__ node,
                         const int32_t* __restrict__ perm, int64_t n, int2* __restrict__ out) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q < n) out[q] = make_int2(node[q], __float_as_int(values[perm[q]]));
  else if (q == n) out[q] = make_int2(kBlkNoNode, 0);
}

// out[q] = a[order[q]]: an edge array of the compressed order in blocked order
__global__ void blk_gather_i32(const int32_t* __restrict__ a, const int32_t* __restrict__ order,
                               int64_t n, int32_t* __restrict__ out) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q < n) out[q] = a[order[q]];
}

// dst[idx[k]] = src[k]
__global__ void blk_scatter(const float* __restrict__ src, const int32_t* __restrict__ idx,
                            int64_t n, float* __restrict__ dst) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k < n) dst[idx[k]] = src[k];
}

__global__ void blk_zero(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// Tiled transposes between [B][N] and [N][Bp] (32 x 32 tiles through LDS).
constexpr int kT = 32;
// (blockIdx.z: the z-th [B][N] matrix, bm_stride floats apart, into the z-th
// plane, plane_stride floats apart)
__global__ __launch_bounds__(256) void blk_to_planes(const float* __restrict__ bm, int N, int B,
                                                     int Bp, float* __restrict__ plane,
                                                     size_t bm_stride = 0,
                                                     size_t plane_stride = 0) {
  __shared__ float tile[kT][kT + 1];
  const int tx = threadIdx.x % kT, ty = threadIdx.x / kT;
  const int n0 = blockIdx.x * kT, b0 = blockIdx.y * kT;
  bm += blockIdx.z * bm_stride;
  plane += blockIdx.z * plane_stride;
  for (int i = ty; i < kT; i += blockDim.x / kT) {
    const int b = b0 + i, n = n0 + tx;
    tile[i][tx] = (b < B && n < N) ? bm[(size_t)b * N + n] : 0.0f;
  }
  __syncthreads();
  for (int i = ty; i < kT; i += blockDim.x / kT) {
    const int n = n0 + i, b = b0 + tx;
    if (n < N && b < Bp) plane[(size_t)n * Bp + b] = tile[tx][i];
  }
}
// bm[t][b][n] = planes[t * pstride + n * Bp + b], t < T
__global__ __launch_bounds__(256) void blk_from_planes(const float* __restrict__ planes,
                                                       size_t pstride, int64_t T, int N, int B,
                                                       int Bp, float* __restrict__ bm) {
  __shared__ float tile[kT][kT + 1];
  const int tx = threadIdx.x % kT, ty = threadIdx.x / kT;
  const int n0 = blockIdx.x * kT, b0 = blockIdx.y * kT;
  for (int64_t t = blockIdx.z; t < T; t += gridDim.z) {
    const float* src = planes + (size_t)t * pstride;
    for (int i = ty; i < kT; i += blockDim.x / kT) {
      const int n = n0 + i, b = b0 + tx;
      tile[i][tx] = (n < N && b < B) ? src[(size_t)n * Bp + b] : 0.0f;
    }
    __syncthreads();
    float* dst = bm + (size_t)t * B * N;
    for (int i = ty; i < kT; i += blockDim.x / kT) {
      const int b = b0 + i, n = n0 + tx;
      if (b < B && n < N) dst[(size_t)b * N + n] = tile[tx][i];
    }
    __syncthreads();
  }
}

inline unsigned blocks_for(int64_t n, int threads = 256) {
  return (unsigned)std::max<int64_t>(1, (n + threads - 1) / threads);
}

using PartFn = void (*)(BlkPartArgs);
using FEpiFn = void (*)(BlkFwdEpiArgs);
using BEpiFn = void (*)(BlkBwdEpiArgs);
template <int... Ls>
struct BlkTables {
  static constexpr PartFn fpart[] = {&blk_fwd_part<Ls>...};
  static constexpr PartFn bpart[] = {&blk_bwd_part<Ls>...};
  static constexpr FEpiFn fepi[] = {&blk_fwd_epi<Ls>...};
  static constexpr BEpiFn bepi[] = {&blk_bwd_epi<Ls>...};
  static constexpr int64_t (*threads[])(int64_t) = {&epi_threads<Ls>...};
};
// (L = 1, B <= 4, is not built: the compiler does not finish the backward
// part kernel at that width; such calls take the per-microstep kernels)
using BT = BlkTables<2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>;

inline size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

BlkWs blk_ws_layout(const ck_graph* g, const BlkDims& d) {
  BlkWs w;
  size_t o = 0;
  const int64_t items = std::max<int64_t>({g->blk_fwd.items, g->blk_bwd.items, 1});
  w.pe = o;   o = al256(o + (size_t)(d.E + 1) * 8);
  w.part = o; o = al256(o + (size_t)(items + 1) * d.Bp * 4);
  w.h0 = o;   o = al256(o + d.plane * 4);
  w.fwd_end = o;
  w.gv = o;   o = al256(o + (size_t)std::max<int64_t>(d.E, 1) * 4);
  w.gh = o;   o = al256(o + d.plane * 4);
  w.ga0 = o;  o = al256(o + d.plane * 4);
  w.ga1 = o;  o = al256(o + d.plane * 4);
  w.gt = o;   o = al256(o + (size_t)d.T * d.plane * 4);  // upstream gradient, node-major
  w.total = o;
  return w;
}

bool blk_fits(const ck_graph* g, int64_t Bp) {
  if (!g->blk_ok || Bp < 8 || Bp > 64) return false;
  const int64_t items = std::max(g->blk_fwd.items, g->blk_bwd.items);  // (0 when not planned)
  const int64_t lim = (int64_t)kOut;  // buffer byte offsets stay below the out-of-range marker
  // nodes below the sentinel, whose gather offset (at least kBlkNoNode * 32
  // bytes) lies past the plane
  return items * Bp * 4 < lim && (g->E + 1) * 8 < lim && g->N < kBlkNoNode &&
         g->N * Bp * 4 <= (int64_t)kBlkNoNode * 32;
}

ck_status blk_forward(const ck_graph* g, const BlkDims& d, const float* edge_values,
                      const float* leak, const float* bias, const float* drives,
                      const float* state0, float* out, void* saved, void* workspace,
                      hipStream_t stream, bool profile) {
  const BlkWs ws = blk_ws_layout(g, d);
  char* wsb = static_cast<char*>(workspace);
  int2* pe = reinterpret_cast<int2*>(wsb + ws.pe);
  float* partial = reinterpret_cast<float*>(wsb + ws.part);
  float* h0 = reinterpret_cast<float*>(wsb + ws.h0);
  float* hplanes = static_cast<float*>(saved);
  float* aplanes = hplanes + (size_t)d.S * d.plane;
  const Blocked& bf = g->blk_fwd;
  if (d.E > 0)
    blk_pack<<<blocks_for(d.E + 1), 256, 0, stream>>>(edge_values, bf.pnode, bf.pperm, d.E, pe);
  blk_to_planes<<<dim3(blocks_for(d.N, kT), (unsigned)((d.Bp + kT - 1) / kT)), 256, 0, stream>>>(
      state0, (int)d.N, (int)d.B, (int)d.Bp, h0);
  const PartFn part = BT::fpart[d.L - 2];
  const FEpiFn epi = BT::fepi[d.L - 2];
  const unsigned epi_blocks = blocks_for(BT::threads[d.L - 2](d.N));
  BlkPartArgs a{};
  a.table = bf.table;
  a.KB = bf.KB;
  a.pe = pe;
  a.sentinel = (uint32_t)d.E;
  a.src_bytes = (uint32_t)(d.plane * 4);
  a.partial = partial;
  a.items = bf.items;
  a.Bp = (int)d.Bp;
  BlkFwdEpiArgs e{};
  e.row_items = bf.row_items;
  e.item_ids = bf.item_ids;
  e.partial = partial;
  e.leak = leak;
  e.bias = bias;
  e.input_slot = g->input_slot;
  e.N = (int)d.N;
  e.B = (int)d.B;
  e.Bp = (int)d.Bp;
  ck_status rc = CK_OK;
  for (int64_t s = 1; s <= d.S; ++s) {
    const int64_t t = (s - 1) / d.M;
    a.src = s == 1 ? h0 : hplanes + (size_t)(s - 2) * d.plane;
    if (bf.KB > 0) {
      auto launch = [&] {
        hipLaunchKernelGGL(part, dim3(bf.num_wgs), dim3(kBlkWaves * 64), 0, stream, a);
      };
      if (profile) rc = timed_launch(g_profile.fwd, stream, launch);
      else launch();
      if (rc != CK_OK) return rc;
    }
    e.drives_t = d.n_in > 0 ? drives + (size_t)t * d.n_in * d.B : nullptr;
    e.h_prev = a.src;
    e.h_next = hplanes + (size_t)(s - 1) * d.plane;
    e.a_next = aplanes + (size_t)(s - 1) * d.plane;
    auto launch_epi = [&] { hipLaunchKernelGGL(epi, dim3(epi_blocks), dim3(256), 0, stream, e); };
    if (profile) rc = timed_launch(g_profile.fwd, stream, launch_epi);
    else launch_epi();
    if (rc != CK_OK) return rc;
  }
  blk_from_planes<<<dim3(blocks_for(d.N, kT), (unsigned)((d.B + kT - 1) / kT),
                         (unsigned)std::min<int64_t>(d.T, 65535)),
                    256, 0, stream>>>(hplanes + (size_t)(d.M - 1) * d.plane,
                                      (size_t)d.M * d.plane, d.T, (int)d.N, (int)d.B,
                                      (int)d.Bp, out);
  CK_HIP_TRY(hipGetLastError());
  return CK_OK;
}

ck_status blk_backward(const ck_graph* g, const BlkDims& d, const float* edge_values,
                       const float* leak, const float* state0, const void* saved,
                       const float* grad_out, float* grad_edge_values, float* grad_leak,
                       float* grad_bias, float* grad_drives, float* grad_state0,
                       void* workspace, hipStream_t stream) {
  const BlkWs ws = blk_ws_layout(g, d);
  char* wsb = static_cast<char*>(workspace);
  int2* pe = reinterpret_cast<int2*>(wsb + ws.pe);
  float* partial = reinterpret_cast<float*>(wsb + ws.part);
  float* h0 = reinterpret_cast<float*>(wsb + ws.h0);
  float* gv = reinterpret_cast<float*>(wsb + ws.gv);
  float* gh = reinterpret_cast<float*>(wsb + ws.gh);
  float* gabuf[2] = {reinterpret_cast<float*>(wsb + ws.ga0), reinterpret_cast<float*>(wsb + ws.ga1)};
  const float* hplanes = static_cast<const float*>(saved);
  const float* aplanes = hplanes + (size_t)d.S * d.plane;
  auto hplane = [&](int64_t s) { return s == 0 ? h0 : hplanes + (size_t)(s - 1) * d.plane; };
  auto aplane = [&](int64_t s) { return aplanes + (size_t)(s - 1) * d.plane; };
  const Blocked& bb = g->blk_bwd;
  if (d.E > 0)
    blk_pack<<<blocks_for(d.E + 1), 256, 0, stream>>>(edge_values, bb.pnode, bb.pperm, d.E, pe);
  blk_to_planes<<<dim3(blocks_for(d.N, kT), (unsigned)((d.Bp + kT - 1) / kT)), 256, 0, stream>>>(
      state0, (int)d.N, (int)d.B, (int)d.Bp, h0);
  // the upstream gradient [T][B][N] as node-major planes: a row's epilogue
  // lane reads its 4 columns with one 16-byte load
  float* gt = reinterpret_cast<float*>(wsb + ws.gt);
  blk_to_planes<<<dim3(blocks_for(d.N, kT), (unsigned)((d.Bp + kT - 1) / kT), (unsigned)d.T), 256,
                  0, stream>>>(grad_out, (int)d.N, (int)d.B, (int)d.Bp, gt,
                               (size_t)d.B * d.N, d.plane);
  if (d.n_in > 0)
    blk_zero<<<blocks_for(d.T * d.n_in * d.B), 256, 0, stream>>>(grad_drives, d.T * d.n_in * d.B);
  const PartFn part = BT::bpart[d.L - 2];
  const BEpiFn epi = BT::bepi[d.L - 2];
  const unsigned epi_blocks = blocks_for(BT::threads[d.L - 2](d.N));
  BlkPartArgs a{};
  a.table = bb.table;
  a.KB = bb.KB;
  a.pe = pe;
  a.sentinel = (uint32_t)d.E;
  a.src_bytes = (uint32_t)(d.plane * 4);
  a.partial = partial;
  a.items = bb.items;
  a.gv = gv;
  a.gv_bytes = (uint32_t)(d.E * 4);
  a.Bp = (int)d.Bp;
  BlkBwdEpiArgs e{};
  e.row_items = bb.row_items;
  e.item_ids = bb.item_ids;
  e.leak = leak;
  e.input_slot = g->input_slot;
  e.gh = gh;
  e.gleak = grad_leak;
  e.gbias = grad_bias;
  e.gstate0 = grad_state0;
  e.N = (int)d.N;
  e.B = (int)d.B;
  e.Bp = (int)d.Bp;
  ck_status rc = CK_OK;
  // Step "s" is the edge pass of microstep s (part) and the elementwise pass
  // of microstep s-1 (epi); step S+1 has no edge pass and seeds g^(S) = G[T-1].
  for (int64_t s = d.S + 1; s >= 1; --s) {
    const bool init = s == d.S + 1;
    if (!init && bb.KB > 0) {
      a.src = gabuf[s % 2];
      a.h_sm1 = hplane(s - 1);
      a.first_gv = s == d.S ? 1 : 0;
      rc = timed_launch(g_profile.bwd, stream, [&] {
        hipLaunchKernelGGL(part, dim3(bb.num_wgs), dim3(kBlkWaves * 64), 0, stream, a);
      });
      if (rc != CK_OK) return rc;
    }
    e.partial = init ? nullptr : partial;
    e.first_k1 = init ? 1 : 0;
    const int64_t k1 = s - 1;  // microstep whose elementwise pass runs here
    e.G_t = (k1 >= 1 && k1 % d.M == 0) ? gt + (size_t)((k1 - 1) / d.M) * d.plane : nullptr;
    if (k1 >= 1) {
      e.a_k1 = aplane(k1);
      e.h_k1 = hplane(k1 - 1);
      e.ga_out = gabuf[k1 % 2];
      e.gdrives_t = d.n_in > 0 ? grad_drives + (size_t)((k1 - 1) / d.M) * d.n_in * d.B : nullptr;
    } else {
      e.a_k1 = nullptr;
      e.h_k1 = nullptr;
      e.ga_out = nullptr;
      e.gdrives_t = nullptr;
    }
    rc = timed_launch(g_profile.bwd, stream, [&] {
      hipLaunchKernelGGL(epi, dim3(epi_blocks), dim3(256), 0, stream, e);
    });
    if (rc != CK_OK) return rc;
  }
  if (d.E > 0) {
    if (bb.KB > 0) {
      blk_scatter<<<blocks_for(d.E), 256, 0, stream>>>(gv, bb.pperm, d.E, grad_edge_values);
    } else {
      blk_zero<<<blocks_for(d.E), 256, 0, stream>>>(grad_edge_values, d.E);
    }
  }
  CK_HIP_TRY(hipGetLastError());
  return CK_OK;
}

ck_status build_blocked(const std::vector<int32_t>& ptr, int64_t N, const int32_t* col,
                        const int32_t* perm, int num_cus, hipStream_t stream, Blocked* out,
                        bool* planned) {
  *planned = false;
  std::vector<int32_t> hcol(std::max<int32_t>(ptr[N], 1));
  if (ptr[N] > 0) {
    CK_HIP_TRY(hipMemcpyAsync(hcol.data(), col, (size_t)ptr[N] * sizeof(int32_t),
                              hipMemcpyDeviceToHost, stream));
    CK_HIP_TRY(hipStreamSynchronize(stream));
  }
  BlockedPlan plan;
  if (!plan_blocked(ptr.data(), hcol.data(), N, num_cus, &plan)) return CK_OK;
  static_assert(sizeof(BlkItem) == sizeof(int4), "items are read as int4");
  out->num_wgs = plan.num_wgs;
  out->KB = plan.KB;
  out->items = plan.items;
  const size_t tb = std::max<size_t>(plan.table.size(), 1) * sizeof(BlkItem);
  CK_HIP_TRY(hipMalloc(&out->table, tb));
  if (!plan.table.empty())
    CK_HIP_TRY(hipMemcpy(out->table, plan.table.data(), plan.table.size() * sizeof(BlkItem),
                         hipMemcpyHostToDevice));
  CK_HIP_TRY(hipMalloc(&out->row_items, plan.row_items.size() * sizeof(int32_t)));
  CK_HIP_TRY(hipMemcpy(out->row_items, plan.row_items.data(),
                       plan.row_items.size() * sizeof(int32_t), hipMemcpyHostToDevice));
  CK_HIP_TRY(hipMalloc(&out->item_ids, std::max<size_t>(plan.item_ids.size(), 1) * sizeof(int32_t)));
  if (!plan.item_ids.empty())
    CK_HIP_TRY(hipMemcpy(out->item_ids, plan.item_ids.data(),
                         plan.item_ids.size() * sizeof(int32_t), hipMemcpyHostToDevice));
  const int64_t E = ptr[N];
  const size_t eb = (size_t)std::max<int64_t>(E, 1) * sizeof(int32_t);
  CK_HIP_TRY(hipMalloc(&out->pnode, eb));
  CK_HIP_TRY(hipMalloc(&out->pperm, eb));
  if (E > 0) {
    int32_t* order = nullptr;
    hipError_t e = hipMalloc(&order, eb);
    if (e == hipSuccess)
      e = hipMemcpy(order, plan.edge_order.data(), E * sizeof(int32_t), hipMemcpyHostToDevice);
    if (e == hipSuccess) {
      blk_gather_i32<<<blocks_for(E), 256, 0, stream>>>(col, order, E, out->pnode);
      blk_gather_i32<<<blocks_for(E), 256, 0, stream>>>(perm, order, E, out->pperm);
      e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    (void)hipFree(order);
    CK_HIP_TRY(e);
  }
  *planned = true;
  return CK_OK;
}

void free_blocked(Blocked* b) {
  (void)hipFree(b->table);
  (void)hipFree(b->row_items);
  (void)hipFree(b->item_ids);
  (void)hipFree(b->pnode);
  (void)hipFree(b->pperm);
  *b = Blocked();
}

}  // namespace ckhip
