// recurrence.hip -- forward and backward of the leaky-tanh recurrence on a
// fixed sparse graph (connectome-kernels README, introduction: the proposal /
// leaky update, repeated `microsteps` times per input step; "Design notes":
// [N, B] state layout, split long rows, transposed CSR in the backward, saved
// state and pre-activation after every microstep).
//
// State layout: [N][Bp] fp32 with Bp = B rounded up to a multiple of 4, so a
// node's batch row is a run of 16-byte vectors (128 bytes at B = 32).
//
// Lane mapping (wave64): a row of Bp columns is covered by L = Bp/4 lanes, each
// holding one float4 of columns; a wave holds P = 64/L such "slots" and so
// gathers P source rows per vector load (8 edges x 32 columns at B = 32).
// Batches wider than 64 columns are cut into 64-column chunks (grid y).
//
// Forward, one launch per microstep s (rows of the CSR by destination):
//   a[i,:] = sum_k v_csr[k] h[col_idx[k],:] + drive[i,:] + bias[i]
//   h'[i,:] = (1 - leak[i]) h[i,:] + leak[i] tanh(a[i,:])
// Backward, one launch per microstep s (rows of the transposed CSR, i.e. per
// source node j), fusing the three backward passes of the README design:
//   g'[j,:] = (1 - leak[j]) g[j,:] + sum_k v_csc[k] ga[t_col_idx[k],:]   (transposed product)
//   gv_csc[k] += <ga[t_col_idx[k],:], h^(s-1)[j,:]>                     (edge gradient, same gather)
//   then the elementwise pass of microstep s-1 on node j with its leak/bias
//   row reductions and the drive gradient.
// No floating-point atomics: every output element has exactly one owner, and
// every sum is taken in a fixed order, so results are bitwise reproducible.
#include <algorithm>
#include <vector>

#include "ck_internal.h"

namespace ckhip {
namespace {

// Measurement hook state: HIP event pairs around per-microstep launches.
struct Profile {
  bool enabled = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> fwd, bwd;
};
Profile g_profile;

// Launch `launch()` on `stream`, bracketed by events when profiling is on.
template <typename F>
ck_status timed_launch(std::vector<std::pair<hipEvent_t, hipEvent_t>>& log, hipStream_t stream,
                       F&& launch) {
  if (!g_profile.enabled) {
    launch();
    return CK_OK;
  }
  hipEvent_t a, b;
  CK_HIP_TRY(hipEventCreate(&a));
  CK_HIP_TRY(hipEventCreate(&b));
  CK_HIP_TRY(hipEventRecord(a, stream));
  launch();
  CK_HIP_TRY(hipEventRecord(b, stream));
  log.emplace_back(a, b);
  return CK_OK;
}

constexpr int kChunkCols = 64;  // columns per grid-y chunk when Bp > 64

__device__ __forceinline__ float4 f4(float x) { return make_float4(x, x, x, x); }
__device__ __forceinline__ float4 fma4(float w, float4 h, float4 acc) {
  acc.x = fmaf(w, h.x, acc.x);
  acc.y = fmaf(w, h.y, acc.y);
  acc.z = fmaf(w, h.z, acc.z);
  acc.w = fmaf(w, h.w, acc.w);
  return acc;
}
__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ __forceinline__ float4 shfl4(float4 v, int src) {
  return make_float4(__shfl(v.x, src), __shfl(v.y, src), __shfl(v.z, src), __shfl(v.w, src));
}
__device__ __forceinline__ float4 shfl_xor4(float4 v, int m) {
  return make_float4(__shfl_xor(v.x, m), __shfl_xor(v.y, m), __shfl_xor(v.z, m),
                     __shfl_xor(v.w, m));
}
__device__ __forceinline__ float dot4(float4 a, float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}
__device__ __forceinline__ float4 tanh4(float4 a) {
  return make_float4(tanhf(a.x), tanhf(a.y), tanhf(a.z), tanhf(a.w));
}
// sech^2(a) = 4 e^{-2|a|} / (1 + e^{-2|a|})^2, from the pre-activation itself
// (not 1 - tanh^2, which cancels badly once |a| is a few units).
__device__ __forceinline__ float sech2f(float a) {
  float e = expf(-2.0f * fabsf(a));
  float d = 1.0f + e;
  return 4.0f * e / (d * d);
}

constexpr bool is_pow2(int x) { return (x & (x - 1)) == 0; }

// Lane geometry for L lanes per slot.
template <int L>
struct Geom {
  static constexpr int P = 64 / L;                        // slots per wave
  static constexpr int I = (64 / P) < L ? (64 / P) : L;   // edge rounds per batch
  static constexpr int EB = P * I;                         // edges per batch (<= 64)
};

// Sum over the P slots for each lane's column group; every lane gets the total
// of its own sub-lane (fixed order: butterfly for powers of two, else ascending).
template <int L>
__device__ __forceinline__ float4 sum_slots(float4 v, int sub) {
  constexpr int P = Geom<L>::P;
  if constexpr (is_pow2(L)) {
#pragma unroll
    for (int m = L; m < 64; m <<= 1) v = add4(v, shfl_xor4(v, m));
    return v;
  } else {
    float4 s = shfl4(v, sub);
#pragma unroll
    for (int p = 1; p < P; ++p) s = add4(s, shfl4(v, p * L + sub));
    return s;
  }
}

// Sum over the L lanes of this lane's slot; every lane of the slot gets it.
template <int L>
__device__ __forceinline__ float sum_in_slot(float x, int slot) {
  if constexpr (L == 1) {
    return x;
  } else if constexpr (is_pow2(L)) {
#pragma unroll
    for (int m = 1; m < L; m <<= 1) x += __shfl_xor(x, m);
    return x;
  } else {
    float s = __shfl(x, slot * L);
#pragma unroll
    for (int i = 1; i < L; ++i) s += __shfl(x, slot * L + i);
    return s;
  }
}

struct FwdArgs {
  const int2* items;
  const int32_t* rows;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const float* v_csr;
  const float* leak;
  const float* bias;
  const int32_t* input_slot;
  const float* drives_t;  // [n_in][B] of the current input step (nullptr if n_in == 0)
  const float* h_prev;    // [N][Bp]
  float* h_next;          // [N][Bp]
  float* a_next;          // [N][Bp]
  float* out_t;           // [B][N] or nullptr when s is not the last microstep of a step
  int N, B, Bp;
};

template <int L>
__global__ __launch_bounds__(kThreads) void fwd_step(FwdArgs p) {
  using G = Geom<L>;
  constexpr int P = G::P, I = G::I, EB = G::EB;
  __shared__ float4 red[kWaves][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane / L, sub = lane % L;
  const int col = blockIdx.y * kChunkCols + sub * 4;
  const bool lane_ok = slot < P && col < p.Bp;
  const int2 it = p.items[blockIdx.x];
  const bool split = it.y < 0;
  if (!split && wave >= it.y) return;
  const int row = p.rows[it.x + (split ? 0 : wave)];
  int kbeg = p.row_ptr[row], kend = p.row_ptr[row + 1];
  if (split) {
    const int n = kend - kbeg, per = (n + kWaves - 1) / kWaves;
    kbeg = min(kend, kbeg + wave * per);
    kend = min(kend, kbeg + per);
  }
  float4 acc = f4(0.f);
  for (int kb = kbeg; kb < kend; kb += EB) {
    const int nb = min(EB, kend - kb);
    int c = 0;
    float w = 0.f;
    if (lane < nb) {
      c = p.col_idx[kb + lane];
      w = p.v_csr[kb + lane];
    }
#pragma unroll
    for (int j = 0; j < I; ++j) {
      const int e = j * P + slot;
      const int cj = __shfl(c, e);
      const float wj = __shfl(w, e);
      if (lane_ok && e < nb) {
        const float4 hv = *reinterpret_cast<const float4*>(p.h_prev + (size_t)cj * p.Bp + col);
        acc = fma4(wj, hv, acc);
      }
    }
  }
  acc = sum_slots<L>(acc, sub);
  if (split) {
    if (slot == 0) red[wave][sub] = acc;
    __syncthreads();
    if (wave != 0) return;
    acc = red[0][sub];
#pragma unroll
    for (int q = 1; q < kWaves; ++q) acc = add4(acc, red[q][sub]);
  }
  if (slot != 0 || !lane_ok) return;
  // elementwise: drive, bias, tanh, leaky mix
  const size_t off = (size_t)row * p.Bp + col;
  const float4 hp = *reinterpret_cast<const float4*>(p.h_prev + off);
  const float lam = p.leak[row], bi = p.bias[row];
  float d[4] = {0.f, 0.f, 0.f, 0.f};
  const int ks = p.input_slot[row];
  if (ks >= 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (col + q < p.B) d[q] = p.drives_t[(size_t)ks * p.B + col + q];
  }
  float4 a;
  a.x = acc.x + d[0] + bi;
  a.y = acc.y + d[1] + bi;
  a.z = acc.z + d[2] + bi;
  a.w = acc.w + d[3] + bi;
  const float4 pr = tanh4(a);
  const float om = 1.0f - lam;
  float4 h;
  h.x = om * hp.x + lam * pr.x;
  h.y = om * hp.y + lam * pr.y;
  h.z = om * hp.z + lam * pr.z;
  h.w = om * hp.w + lam * pr.w;
  *reinterpret_cast<float4*>(p.h_next + off) = h;
  *reinterpret_cast<float4*>(p.a_next + off) = a;
  if (p.out_t) {
    const float hv[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (col + q < p.B) p.out_t[(size_t)(col + q) * p.N + row] = hv[q];
  }
}

struct BwdArgs {
  const int2* items;
  const int32_t* rows;
  const int32_t* t_row_ptr;
  const int32_t* t_col_idx;
  const float* v_csc;
  float* gv_csc;          // [chunks][E] transposed-CSR order, one row per column chunk
  const float* leak;
  const int32_t* input_slot;
  const float* ga_in;     // ga^(s) [N][Bp] (gathered); nullptr: no edge pass (init)
  const float* h_sm1;     // h^(s-1) [N][Bp]
  float* gh;              // in: g^(s) (ignored when ga_in == nullptr), out: g^(s-1)
  const float* G_t;       // [B][N] upstream gradient entering at microstep s-1, or nullptr
  // elementwise pass of microstep s-1 (skipped when a_k1 == nullptr, i.e. s-1 == 0)
  const float* a_k1;      // a^(s-1)
  const float* h_k1;      // h^(s-2)
  float* ga_out;          // ga^(s-1)
  float* gdrives_t;       // [n_in][B] of input step t(s-1), accumulated
  float* gleak;           // [chunks][N] accumulated (written when first_k1)
  float* gbias;           // [chunks][N]
  float* gstate0;         // [B][N], written when s-1 == 0
  int first_k1;           // 1: overwrite gleak/gbias instead of accumulating
  int first_gv;           // 1: overwrite gv_csc instead of accumulating
  int N, B, Bp, E;
};

template <int L>
__global__ __launch_bounds__(kThreads) void bwd_step(BwdArgs p) {
  using G = Geom<L>;
  constexpr int P = G::P, I = G::I, EB = G::EB;
  __shared__ float4 red[kWaves][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane / L, sub = lane % L;
  const int col = blockIdx.y * kChunkCols + sub * 4;
  const bool lane_ok = slot < P && col < p.Bp;
  const int2 it = p.items[blockIdx.x];
  const bool split = it.y < 0;
  if (!split && wave >= it.y) return;
  const int row = p.rows[it.x + (split ? 0 : wave)];
  float4 acc = f4(0.f);
  if (p.ga_in != nullptr) {
    int kbeg = p.t_row_ptr[row], kend = p.t_row_ptr[row + 1];
    if (split) {
      const int n = kend - kbeg, per = (n + kWaves - 1) / kWaves;
      kbeg = min(kend, kbeg + wave * per);
      kend = min(kend, kbeg + per);
    }
    const float4 hj = lane_ok ? *reinterpret_cast<const float4*>(p.h_sm1 + (size_t)row * p.Bp + col)
                              : f4(0.f);
    for (int kb = kbeg; kb < kend; kb += EB) {
      const int nb = min(EB, kend - kb);
      int c = 0;
      float w = 0.f;
      if (lane < nb) {
        c = p.t_col_idx[kb + lane];
        w = p.v_csc[kb + lane];
      }
      float mine = 0.f;  // edge-gradient term kept by this lane: edge kb + sub*P + slot
#pragma unroll
      for (int j = 0; j < I; ++j) {
        const int e = j * P + slot;
        const int cj = __shfl(c, e);
        const float wj = __shfl(w, e);
        float part = 0.f;
        if (lane_ok && e < nb) {
          const float4 gv = *reinterpret_cast<const float4*>(p.ga_in + (size_t)cj * p.Bp + col);
          acc = fma4(wj, gv, acc);
          part = dot4(gv, hj);
        }
        const float tot = sum_in_slot<L>(part, slot);
        if (sub == j) mine = tot;
      }
      if (slot < P && sub < I) {
        const int e = sub * P + slot;
        if (e < nb) {
          float* dst = p.gv_csc + (size_t)blockIdx.y * p.E + kb + e;
          *dst = p.first_gv ? mine : *dst + mine;
        }
      }
    }
    acc = sum_slots<L>(acc, sub);
    if (split) {
      if (slot == 0) red[wave][sub] = acc;
      __syncthreads();
      if (wave != 0) return;
      acc = red[0][sub];
#pragma unroll
      for (int q = 1; q < kWaves; ++q) acc = add4(acc, red[q][sub]);
    }
  } else if (split && wave != 0) {
    return;
  }
  if (slot != 0) return;
  // g^(s-1)[row, cols] = (1 - leak) g^(s) + W^T ga^(s) (+ G entering at s-1)
  const size_t off = (size_t)row * p.Bp + col;
  const float lam = p.leak[row];
  float4 g = acc;
  if (p.ga_in != nullptr && lane_ok) {
    const float4 go = *reinterpret_cast<const float4*>(p.gh + off);
    const float om = 1.0f - lam;
    g.x = fmaf(om, go.x, acc.x);
    g.y = fmaf(om, go.y, acc.y);
    g.z = fmaf(om, go.z, acc.z);
    g.w = fmaf(om, go.w, acc.w);
  }
  float gg[4] = {g.x, g.y, g.z, g.w};
  if (p.G_t) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (lane_ok && col + q < p.B) gg[q] += p.G_t[(size_t)(col + q) * p.N + row];
  }
  if (p.a_k1 == nullptr) {  // s - 1 == 0: gradient of the initial state
    if (lane_ok) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (col + q < p.B) p.gstate0[(size_t)(col + q) * p.N + row] = gg[q];
    }
    return;
  }
  // elementwise pass of microstep s-1 on this node
  float lsum = 0.f, bsum = 0.f;
  float ga[4] = {0.f, 0.f, 0.f, 0.f};
  if (lane_ok) {
    const float4 a4 = *reinterpret_cast<const float4*>(p.a_k1 + off);
    const float4 q4 = *reinterpret_cast<const float4*>(p.h_k1 + off);
    const float av[4] = {a4.x, a4.y, a4.z, a4.w};
    const float qv[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (col + q < p.B) {
        const float pr = tanhf(av[q]);
        lsum += gg[q] * (pr - qv[q]);
        ga[q] = gg[q] * lam * sech2f(av[q]);
        bsum += ga[q];
      } else {
        gg[q] = 0.f;
      }
    }
    *reinterpret_cast<float4*>(p.gh + off) = make_float4(gg[0], gg[1], gg[2], gg[3]);
    *reinterpret_cast<float4*>(p.ga_out + off) = make_float4(ga[0], ga[1], ga[2], ga[3]);
    const int ks = p.input_slot[row];
    if (ks >= 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (col + q < p.B) p.gdrives_t[(size_t)ks * p.B + col + q] += ga[q];
    }
  }
  // per-node leak and bias reductions over the batch (the lanes of slot 0)
  lsum = sum_in_slot<L>(lsum, 0);
  bsum = sum_in_slot<L>(bsum, 0);
  if (sub == 0) {
    float* gl = p.gleak + (size_t)blockIdx.y * p.N + row;
    float* gb = p.gbias + (size_t)blockIdx.y * p.N + row;
    *gl = p.first_k1 ? lsum : *gl + lsum;
    *gb = p.first_k1 ? bsum : *gb + bsum;
  }
}

// ---------------------------------------------------------------- small kernels
__global__ void gather_f32(const float* __restrict__ src, const int32_t* __restrict__ idx,
                           int64_t n, float* __restrict__ dst) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k < n) dst[k] = src[idx[k]];
}

// dst[idx[k]] = sum over chunks c (ascending) of src[c][k]
__global__ void scatter_sum_f32(const float* __restrict__ src, int chunks,
                                const int32_t* __restrict__ idx, int64_t n,
                                float* __restrict__ dst) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= n) return;
  float s = src[k];
  for (int c = 1; c < chunks; ++c) s += src[(size_t)c * n + k];
  dst[idx[k]] = s;
}

// [B][N] -> [N][Bp] with zero padding columns
__global__ void to_node_major(const float* __restrict__ x, int N, int B, int Bp,
                              float* __restrict__ y) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)N * Bp) return;
  const int i = (int)(t / Bp), b = (int)(t % Bp);
  y[t] = b < B ? x[(size_t)b * N + i] : 0.0f;
}

// out[i] = sum over chunks c (ascending) of part[c][i]
__global__ void sum_chunks(const float* __restrict__ part, int chunks, int64_t n,
                           float* __restrict__ out) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = part[i];
  for (int c = 1; c < chunks; ++c) s += part[(size_t)c * n + i];
  out[i] = s;
}

__global__ void zero_f32(float* __restrict__ p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

inline unsigned grid1(int64_t n, int threads = 256) {
  return (unsigned)std::max<int64_t>(1, (n + threads - 1) / threads);
}

// Kernel tables indexed by L - 1 (L = 1..16 lanes per slot).
using FwdFn = void (*)(FwdArgs);
using BwdFn = void (*)(BwdArgs);
template <int... Ls>
struct Tables {
  static constexpr FwdFn fwd[] = {&fwd_step<Ls>...};
  static constexpr BwdFn bwd[] = {&bwd_step<Ls>...};
};
using KT = Tables<1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>;

struct Dims {
  int64_t N, E, n_in, T, B, M, S, Bp;
  int L, chunks;
  size_t plane;  // floats per [N][Bp] plane
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct WsLayout {
  size_t v, gv, h0, gh, ga0, ga1, part, total;
};

WsLayout ws_layout(const Dims& d) {
  WsLayout w;
  size_t o = 0;
  w.v = o;   o = align256(o + (size_t)std::max<int64_t>(d.E, 1) * 4);
  w.gv = o;  o = align256(o + (size_t)d.chunks * std::max<int64_t>(d.E, 1) * 4);
  w.h0 = o;  o = align256(o + d.plane * 4);
  w.gh = o;  o = align256(o + d.plane * 4);
  w.ga0 = o; o = align256(o + d.plane * 4);
  w.ga1 = o; o = align256(o + d.plane * 4);
  w.part = o;  // per-chunk leak/bias partial sums when the batch spans several chunks
  if (d.chunks > 1) o = align256(o + 2 * (size_t)d.chunks * d.N * 4);
  w.total = o;
  return w;
}

ck_status make_dims(const ck_graph* g, int64_t T, int64_t B, int64_t M, Dims* d) {
  if (T <= 0 || B <= 0 || M <= 0) {
    set_error("T, B and microsteps must be positive (got %lld, %lld, %lld)", (long long)T,
              (long long)B, (long long)M);
    return CK_ERR_BAD_SIZE;
  }
  const int64_t Bp = (B + 3) / 4 * 4;
  if (B >= (1LL << 30) || (g->N * Bp) >= (1LL << 31) || T * M >= (1LL << 31) ||
      T * B * g->N >= (1LL << 62) / 8) {
    set_error("sizes overflow 32-bit indexing: N=%lld B=%lld T=%lld M=%lld", (long long)g->N,
              (long long)B, (long long)T, (long long)M);
    return CK_ERR_TOO_LARGE;
  }
  d->N = g->N;
  d->E = g->E;
  d->n_in = g->n_in;
  d->T = T;
  d->B = B;
  d->M = M;
  d->S = T * M;
  d->Bp = Bp;
  d->L = Bp <= kChunkCols ? (int)(Bp / 4) : 16;
  d->chunks = (int)((Bp + kChunkCols - 1) / kChunkCols);
  d->plane = (size_t)g->N * Bp;
  return CK_OK;
}

}  // namespace
}  // namespace ckhip

using namespace ckhip;

extern "C" ck_status ck_recurrence_sizes(ck_graph_t g, int64_t T, int64_t B, int64_t microsteps,
                                         size_t* saved_bytes, size_t* workspace_bytes) {
  clear_error();
  ck_status rc = check_graph(g);
  if (rc != CK_OK) return rc;
  Dims d;
  rc = make_dims(g, T, B, microsteps, &d);
  if (rc != CK_OK) return rc;
  if (saved_bytes) *saved_bytes = 2 * (size_t)d.S * d.plane * sizeof(float);
  if (workspace_bytes) *workspace_bytes = ws_layout(d).total;
  return CK_OK;
}

extern "C" ck_status ck_recurrence_forward(ck_graph_t g, const float* edge_values,
                                           const float* leak, const float* bias,
                                           const float* drives, const float* state0, int64_t T,
                                           int64_t B, int64_t microsteps, float* out, void* saved,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
  clear_error();
  ck_status rc = check_graph(g);
  if (rc != CK_OK) return rc;
  Dims d;
  rc = make_dims(g, T, B, microsteps, &d);
  if (rc != CK_OK) return rc;
  if ((d.E > 0 && !edge_values) || !leak || !bias || (d.n_in > 0 && !drives) || !state0 ||
      !out || !saved || !workspace) {
    set_error("NULL pointer for a non-empty tensor in forward");
    return CK_ERR_NULL_ARG;
  }
  const WsLayout ws = ws_layout(d);
  if (workspace_bytes < ws.total) {
    set_error("workspace of %zu bytes is below the %zu required", workspace_bytes, ws.total);
    return CK_ERR_WORKSPACE;
  }
  char* wsb = static_cast<char*>(workspace);
  float* v_csr = reinterpret_cast<float*>(wsb + ws.v);
  float* h0 = reinterpret_cast<float*>(wsb + ws.h0);
  float* hplanes = static_cast<float*>(saved);
  float* aplanes = hplanes + (size_t)d.S * d.plane;
  if (d.E > 0) gather_f32<<<grid1(d.E), 256, 0, stream>>>(edge_values, g->perm, d.E, v_csr);
  to_node_major<<<grid1((int64_t)d.plane), 256, 0, stream>>>(state0, (int)d.N, (int)d.B,
                                                             (int)d.Bp, h0);
  const FwdFn kern = KT::fwd[d.L - 1];
  const dim3 grid(g->fwd.num_items, d.chunks);
  FwdArgs a{};
  a.items = g->fwd.items;
  a.rows = g->fwd.rows;
  a.row_ptr = g->row_ptr;
  a.col_idx = g->col_idx;
  a.v_csr = v_csr;
  a.leak = leak;
  a.bias = bias;
  a.input_slot = g->input_slot;
  a.N = (int)d.N;
  a.B = (int)d.B;
  a.Bp = (int)d.Bp;
  for (int64_t s = 1; s <= d.S; ++s) {
    const int64_t t = (s - 1) / d.M;
    a.drives_t = d.n_in > 0 ? drives + (size_t)t * d.n_in * d.B : nullptr;
    a.h_prev = s == 1 ? h0 : hplanes + (size_t)(s - 2) * d.plane;
    a.h_next = hplanes + (size_t)(s - 1) * d.plane;
    a.a_next = aplanes + (size_t)(s - 1) * d.plane;
    a.out_t = (s % d.M == 0) ? out + (size_t)t * d.B * d.N : nullptr;
    rc = timed_launch(g_profile.fwd, stream,
                      [&] { hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, stream, a); });
    if (rc != CK_OK) return rc;
  }
  CK_HIP_TRY(hipGetLastError());
  return CK_OK;
}

extern "C" ck_status ck_recurrence_backward(ck_graph_t g, const float* edge_values,
                                            const float* leak, const float* state0, int64_t T,
                                            int64_t B, int64_t microsteps, const void* saved,
                                            const float* grad_out, float* grad_edge_values,
                                            float* grad_leak, float* grad_bias,
                                            float* grad_drives, float* grad_state0,
                                            void* workspace, size_t workspace_bytes,
                                            hipStream_t stream) {
  clear_error();
  ck_status rc = check_graph(g);
  if (rc != CK_OK) return rc;
  Dims d;
  rc = make_dims(g, T, B, microsteps, &d);
  if (rc != CK_OK) return rc;
  if ((d.E > 0 && (!edge_values || !grad_edge_values)) || !leak || !state0 || !saved ||
      !grad_out || !grad_leak || !grad_bias || (d.n_in > 0 && !grad_drives) || !grad_state0 ||
      !workspace) {
    set_error("NULL pointer for a non-empty tensor in backward");
    return CK_ERR_NULL_ARG;
  }
  const WsLayout ws = ws_layout(d);
  if (workspace_bytes < ws.total) {
    set_error("workspace of %zu bytes is below the %zu required", workspace_bytes, ws.total);
    return CK_ERR_WORKSPACE;
  }
  char* wsb = static_cast<char*>(workspace);
  float* v_csc = reinterpret_cast<float*>(wsb + ws.v);
  float* gv_csc = reinterpret_cast<float*>(wsb + ws.gv);
  float* h0 = reinterpret_cast<float*>(wsb + ws.h0);
  float* gh = reinterpret_cast<float*>(wsb + ws.gh);
  float* gabuf[2] = {reinterpret_cast<float*>(wsb + ws.ga0), reinterpret_cast<float*>(wsb + ws.ga1)};
  const float* hplanes = static_cast<const float*>(saved);
  const float* aplanes = hplanes + (size_t)d.S * d.plane;
  auto hplane = [&](int64_t s) { return s == 0 ? h0 : hplanes + (size_t)(s - 1) * d.plane; };
  auto aplane = [&](int64_t s) { return aplanes + (size_t)(s - 1) * d.plane; };
  if (d.E > 0) gather_f32<<<grid1(d.E), 256, 0, stream>>>(edge_values, g->t_perm, d.E, v_csc);
  to_node_major<<<grid1((int64_t)d.plane), 256, 0, stream>>>(state0, (int)d.N, (int)d.B,
                                                             (int)d.Bp, h0);
  if (d.n_in > 0)
    zero_f32<<<grid1(d.T * d.n_in * d.B), 256, 0, stream>>>(grad_drives, d.T * d.n_in * d.B);
  const BwdFn kern = KT::bwd[d.L - 1];
  const dim3 grid(g->bwd.num_items, d.chunks);
  BwdArgs a{};
  a.items = g->bwd.items;
  a.rows = g->bwd.rows;
  a.t_row_ptr = g->t_row_ptr;
  a.t_col_idx = g->t_col_idx;
  a.v_csc = v_csc;
  a.gv_csc = gv_csc;
  a.gh = gh;
  a.leak = leak;
  a.input_slot = g->input_slot;
  float* part = reinterpret_cast<float*>(wsb + ws.part);
  a.gleak = d.chunks > 1 ? part : grad_leak;
  a.gbias = d.chunks > 1 ? part + (size_t)d.chunks * d.N : grad_bias;
  a.gstate0 = grad_state0;
  a.N = (int)d.N;
  a.B = (int)d.B;
  a.Bp = (int)d.Bp;
  a.E = (int)d.E;
  // Launch "s" covers the edge pass of microstep s and the elementwise pass of
  // microstep s-1; launch S+1 has no edge pass and seeds g^(S) = G[T-1].
  for (int64_t s = d.S + 1; s >= 1; --s) {
    const bool init = s == d.S + 1;
    a.ga_in = init ? nullptr : gabuf[s % 2];
    a.h_sm1 = init ? nullptr : hplane(s - 1);
    a.first_gv = s == d.S ? 1 : 0;
    a.first_k1 = init ? 1 : 0;
    const int64_t k1 = s - 1;  // microstep whose elementwise pass runs here
    a.G_t = (k1 >= 1 && k1 % d.M == 0) ? grad_out + (size_t)((k1 - 1) / d.M) * d.B * d.N : nullptr;
    if (k1 >= 1) {
      a.a_k1 = aplane(k1);
      a.h_k1 = hplane(k1 - 1);
      a.ga_out = gabuf[k1 % 2];
      a.gdrives_t = d.n_in > 0 ? grad_drives + (size_t)((k1 - 1) / d.M) * d.n_in * d.B : nullptr;
    } else {
      a.a_k1 = nullptr;
      a.h_k1 = nullptr;
      a.ga_out = nullptr;
      a.gdrives_t = nullptr;
    }
    rc = timed_launch(g_profile.bwd, stream,
                      [&] { hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, stream, a); });
    if (rc != CK_OK) return rc;
  }
  if (d.chunks > 1) {
    sum_chunks<<<grid1(d.N), 256, 0, stream>>>(a.gleak, d.chunks, d.N, grad_leak);
    sum_chunks<<<grid1(d.N), 256, 0, stream>>>(a.gbias, d.chunks, d.N, grad_bias);
  }
  if (d.E > 0)
    scatter_sum_f32<<<grid1(d.E), 256, 0, stream>>>(gv_csc, d.chunks, g->t_perm, d.E,
                                                    grad_edge_values);
  CK_HIP_TRY(hipGetLastError());
  return CK_OK;
}

extern "C" ck_status ck_profile_enable(int enable) {
  clear_error();
  g_profile.enabled = enable != 0;
  return CK_OK;
}

extern "C" ck_status ck_profile_collect(double* fwd_ms, int64_t* fwd_launches, double* bwd_ms,
                                        int64_t* bwd_launches) {
  clear_error();
  ck_status rc = CK_OK;
  auto drain = [&](std::vector<std::pair<hipEvent_t, hipEvent_t>>& log, double* ms,
                   int64_t* n) {
    double total = 0.0;
    for (auto& e : log) {
      float t = 0.f;
      hipError_t err = hipEventSynchronize(e.second);
      if (err == hipSuccess) err = hipEventElapsedTime(&t, e.first, e.second);
      if (err != hipSuccess && rc == CK_OK) {
        set_error("profiling event failed: %s", hipGetErrorString(err));
        rc = CK_ERR_HIP;
      }
      total += t;
      (void)hipEventDestroy(e.first);
      (void)hipEventDestroy(e.second);
    }
    if (ms) *ms = total;
    if (n) *n = (int64_t)log.size();
    log.clear();
  };
  drain(g_profile.fwd, fwd_ms, fwd_launches);
  drain(g_profile.bwd, bwd_ms, bwd_launches);
  return rc;
}
