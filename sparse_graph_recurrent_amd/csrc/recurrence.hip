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
#include <mutex>
#include <vector>

#include "ck_internal.h"
#include "device_math.h"

namespace ckhip {

Profile g_profile;

// Device scratch of the allocation-free forward (ck_recurrence_forward_noalloc):
// one fixed array per GPU the library runs on, held until the process ends.
// Host code never passes the array's name to a kernel (on the host it is only
// a stand-in); it uses the device address resolved by scratch_prepare.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kScratchDevices] = {};

ck_status scratch_prepare(int device) {
  if (device < 0 || device >= kScratchDevices) {
    set_error("device %d is beyond the %d devices the scratch table covers", device,
              kScratchDevices);
    return CK_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device] == nullptr) {
    void* ptr = nullptr;
    CK_HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    g_scratch_ptr[device] = ptr;
  }
  return CK_OK;
}

static void* scratch_ptr(int device) {
  if (device < 0 || device >= kScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[device];
}

namespace {


constexpr int kChunkCols = 64;  // columns per grid-y chunk when Bp > 64

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

// sum_slots for the forward's fp64 row sums (same order)
template <int L>
__device__ __forceinline__ double4 sum_slots_d(double4 v, int sub) {
  constexpr int P = Geom<L>::P;
  if constexpr (is_pow2(L)) {
#pragma unroll
    for (int m = L; m < 64; m <<= 1) v = add4d(v, shfl_xor4d(v, m));
    return v;
  } else {
    double4 s = shfl4d(v, sub);
#pragma unroll
    for (int p = 1; p < P; ++p) s = add4d(s, shfl4d(v, p * L + sub));
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

// Sum over the L lanes of one slot with DPP lane swizzles (no LDS traffic);
// every lane of the slot receives the same bits.  L must be a power of two.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}
template <int L>
__device__ __forceinline__ float slot_sum(float x, int slot) {
  if constexpr (L == 1) {
    return x;
  } else if constexpr (is_pow2(L)) {
    x += dpp<0xB1>(x);                      // quad_perm [1,0,3,2]: pairs
    if constexpr (L >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: quads
    if constexpr (L >= 8) x += dpp<0x141>(x);  // row_half_mirror: 8 lanes
    if constexpr (L >= 16) x += dpp<0x128>(x); // row_ror 8: 16 lanes
    return x;
  } else {
    return sum_in_slot<L>(x, slot);
  }
}

// Sum over the epilogue lanes 0 .. 4L-1 (slots 0..3); exact in lane 0.
template <int L>
__device__ __forceinline__ float epilogue_sum(float x, int slot) {
  if constexpr (is_pow2(L)) {
    x = slot_sum<L>(x, slot);
    x += __shfl_xor(x, L);
    x += __shfl_xor(x, 2 * L);
    return x;
  } else {
    float s = __shfl(x, 0);
    for (int i = 1; i < 4 * L; ++i) s += __shfl(x, i);
    return s;
  }
}

// 16-byte load at a 32-bit byte offset from a uniform base (lets the compiler
// use the scalar-base addressing form: one VGPR per address).
__device__ __forceinline__ float4 ld4(const float* base, uint32_t byte_off) {
  return *reinterpret_cast<const float4*>(reinterpret_cast<const char*>(base) + byte_off);
}

// Bounds-checked build (-DCK_CHECKED, for validating kernel changes): every
// global access goes through CK_AT / ld4c, an out-of-range index sets a site
// bit in g_ck_err and is redirected to a scratch cell instead of faulting.
#ifdef CK_CHECKED
__device__ unsigned g_ck_err;
__device__ float4 g_ck_dummy[2];
template <typename T>
__device__ __forceinline__ T* ck_at(T* base, size_t i, size_t n, int site) {
  if (base == nullptr || i >= n) {
    atomicOr(&g_ck_err, 1u << site);
    return reinterpret_cast<T*>(g_ck_dummy);
  }
  return base + i;
}
#define CK_AT(base, i, n, site) (*ck_at((base), (size_t)(i), (size_t)(n), (site)))
__device__ __forceinline__ float4 ld4c(const float* base, uint32_t byte_off, size_t nfloats,
                                       int site) {
  if (base == nullptr || (size_t)byte_off / 4 + 4 > nfloats || (byte_off & 15u)) {
    atomicOr(&g_ck_err, 1u << site);
    return g_ck_dummy[0];
  }
  return ld4(base, byte_off);
}
#else
#define CK_AT(base, i, n, site) ((base)[(i)])
__device__ __forceinline__ float4 ld4c(const float* base, uint32_t byte_off, size_t, int) {
  return ld4(base, byte_off);
}
#endif

// Row gathers go through a buffer resource over one [N][Bp] plane.  A lane
// with nothing to gather (padded edge slot, idle lane) passes kNoRow, an
// offset past any plane (planes are below 2^32 - 16 bytes): the hardware
// range check returns zero for it without a memory access, so no branch is
// needed around the load.  (Third descriptor word: the gfx9 family's raw
// 32-bit buffer format.)
constexpr uint32_t kNoRow = 0xFFFFFFF0u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t plane_rsrc(const float* plane, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(plane), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ float4 gather4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t bytes,
                                          int site) {
#ifdef CK_CHECKED
  if (off != kNoRow && ((size_t)off + 16 > bytes || (off & 15u))) {
    atomicOr(&g_ck_err, 1u << site);
    return g_ck_dummy[0];
  }
#else
  (void)bytes;
  (void)site;
#endif
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Load of a value that is the same for every lane (a per-row parameter) from
// an array no kernel of the recurrence writes: through the constant address
// space, so it takes the scalar path and no vector memory instruction.
template <typename T>
__device__ __forceinline__ T ld_row(const T* base, size_t i, size_t n, int site) {
#ifdef CK_CHECKED
  if (base == nullptr || i >= n) {
    atomicOr(&g_ck_err, 1u << site);
    return T(0);
  }
#else
  (void)n;
  (void)site;
#endif
  return ((const __attribute__((address_space(4))) T*)base)[i];
}

__device__ __forceinline__ float pick4(float4 v, int q) {
  return q == 0 ? v.x : (q == 1 ? v.y : (q == 2 ? v.z : v.w));
}
__device__ __forceinline__ double pick4d(double4 v, int q) {
  return q == 0 ? v.x : (q == 1 ? v.y : (q == 2 ? v.z : v.w));
}

// Lane roles shared by both kernels.  In the gather loop lane = slot * L + sub
// holds columns [col, col + 4) of one gathered row.  In the per-row epilogue
// lane (slot q < 4, sub s) handles the single column colbase + 4 s + q, so 32
// lanes (not 8) share the transcendental work at B = 32.
struct Lanes {
  int lane, wave, slot, sub, col, ecol;
  bool ok;       // lane takes part in the gather loop
  bool eok;      // lane owns an epilogue column < Bp
};

template <int L>
__device__ __forceinline__ Lanes lanes(int Bp) {
  Lanes r;
  r.lane = threadIdx.x & 63;
  r.wave = threadIdx.x >> 6;
  r.slot = r.lane / L;
  r.sub = r.lane % L;
  const int colbase = blockIdx.y * kChunkCols;
  r.col = colbase + r.sub * 4;
  r.ok = r.slot < Geom<L>::P && r.col < Bp;
  r.ecol = r.col + r.slot;
  r.eok = r.slot < 4 && r.col < Bp;  // ecol < Bp since Bp is a multiple of 4
  return r;
}


// LDS slot of a piece and the slot range of a split row (from the last
// piece's info word); the checked build reports numbers outside [0, 2W).
template <int W>
__device__ __forceinline__ int piece_slot(int info) {
  const int q = info & kInfoSlotMask;
#ifdef CK_CHECKED
  if (q >= 2 * W) {
    atomicOr(&g_ck_err, 1u << 26);
    return 0;
  }
#endif
  return q;
}
template <int W>
__device__ __forceinline__ void piece_range(int info, int& q0, int& q1) {
  q1 = piece_slot<W>(info);
  q0 = q1 - ((info >> kInfoCountShift) & kInfoSlotMask) + 1;
#ifdef CK_CHECKED
  if (q0 < 0) {
    atomicOr(&g_ck_err, 1u << 26);
    q0 = q1;
  }
#endif
}

// A wave walks its schedule in groups of G batch entries.  The group's
// entries (lane q holds entry q) and the padded edge slots of its batches
// (lane k holds edge k of each batch) sit at offsets fixed by the wave's
// index, so both are requested together at the start of the group.  The
// gathers then run as a ring: a unit is one gather round of a batch (I loads
// per lane), TU units are in flight, and units are consumed in order, each
// freed ring slot being refilled with the unit TU places ahead.  The row
// operands of a batch's epilogue are requested with its first unit.
template <int L, int G>
struct Pipe {
  static constexpr int I = Geom<L>::I;
  static constexpr int NSUB = (kBatchEdges + Geom<L>::EB - 1) / Geom<L>::EB;  // units per batch
  static constexpr int NU = G * NSUB;                                          // units per group
  // units in flight: about 32 VGPRs of gathered float4 rows per lane (more
  // in flight measured no faster at B = 32: the gathers are bound by the
  // vector memory pipeline's throughput, not by its latency)
  static constexpr int TU = (8 / I) < 1 ? 1 : ((8 / I) > NU ? NU : 8 / I);
  // batch entries whose operands are in flight with the ring
  static constexpr int TE = (TU - 1) / NSUB + 1;
};
constexpr int kFwdGroup = 8;
constexpr int kBwdGroup = 4;

__device__ __forceinline__ int4 lane_entry(const int4& v, int q) {
  return make_int4(__builtin_amdgcn_readlane(v.x, q), __builtin_amdgcn_readlane(v.y, q),
                   __builtin_amdgcn_readlane(v.z, q), __builtin_amdgcn_readlane(v.w, q));
}

// The value a lane shuffle brought from batch edge e, or `none` past the
// batch's 64 edges.  The shuffle itself must run on every lane (a permute
// reads nothing useful from a lane that is switched off), so it is done
// unconditionally and only its result is selected.
template <typename T>
__device__ __forceinline__ T lane_or(T shuffled, int e, T none) {
  return e < kBatchEdges ? shuffled : none;
}

// Number of entries in use in a group (they form a prefix of lanes 0..G-1).
template <int G>
__device__ __forceinline__ int group_entries(const int4& ent, int lane) {
  return __popcll(__ballot(lane < G && ent.x >= 0));
}

struct FwdArgs {
  const int4* batches;    // schedule: KB batch entries per wave
  const int2* pedge;      // [slots] padded edge slots: {source node or -1, bits of the value}
  int64_t slots;
  int KB;
  const float* leak;
  const float* bias;
  const float* drives_t;  // [n_in][B] of the current input step (nullptr if n_in == 0)
  const float* h_prev;    // [N][Bp]
  float* h_next;          // [N][Bp]
  float* a_next;          // [N][Bp]
  int N, B, Bp, n_in;
};

// Row operands of the forward epilogue (this lane's column).
struct FwdEpi {
  float hp, lam, bi, dv;
};

// row: the node (or -1 for none); ks: its input slot from the schedule entry
__device__ __forceinline__ FwdEpi fwd_epi_load(const FwdArgs& p, const Lanes& ln, int row, int ks) {
  FwdEpi e{0.f, 0.f, 0.f, 0.f};
  if (row < 0) return e;
  // per-row values first (the same for every lane)
  e.lam = ld_row(p.leak, row, p.N, 1);
  e.bi = ld_row(p.bias, row, p.N, 2);
  if (!ln.eok) return e;
  [[maybe_unused]] const size_t NBp = (size_t)p.N * p.Bp;
  e.hp = CK_AT(p.h_prev, (size_t)row * p.Bp + ln.ecol, NBp, 0);
  if (ks >= 0 && ln.ecol < p.B)
    e.dv = CK_AT(p.drives_t, (size_t)ks * p.B + ln.ecol, (size_t)p.n_in * p.B, 4);
  return e;
}

// a = (W h)[row] + drive + bias (summed in fp64, rounded once);
// h' = (1 - leak) h + leak tanh(a)
__device__ __forceinline__ void fwd_epilogue(const FwdArgs& p, const Lanes& ln, int row,
                                             double4 acc, const FwdEpi& e) {
  if (!ln.eok) return;
  const int c = ln.ecol;
  const size_t off = (size_t)row * p.Bp + c;
  const float a = (float)(pick4d(acc, ln.slot) + (double)e.dv + (double)e.bi);
  const float h = (1.0f - e.lam) * e.hp + e.lam * tanhf(a);
  [[maybe_unused]] const size_t NBp = (size_t)p.N * p.Bp;
  CK_AT(p.h_next, off, NBp, 5) = h;
  CK_AT(p.a_next, off, NBp, 6) = a;
}

template <int L>
__global__ __launch_bounds__(waves_for_lanes(L) * 64) void fwd_step(FwdArgs p) {
  using Gm = Geom<L>;
  using Pp = Pipe<L, kFwdGroup>;
  constexpr int W = waves_for_lanes(L);
  constexpr int P = Gm::P, I = Gm::I, EB = Gm::EB;
  constexpr int NSUB = Pp::NSUB, NU = Pp::NU, TU = Pp::TU, TE = Pp::TE;
  __shared__ double4 red[2 * W][16];  // partial sums of pieces, by piece number
  const Lanes ln = lanes<L>(p.Bp);
  const int wave = __builtin_amdgcn_readfirstlane(ln.wave);
  const uint32_t colb = (uint32_t)(ln.ok ? ln.col : 0) * 4u;  // this lane's columns, in bytes
  const uint32_t rowb = (uint32_t)p.Bp * 4u;                   // bytes per state row
  [[maybe_unused]] const size_t NBp = (size_t)p.N * p.Bp;
  const size_t wv = (size_t)blockIdx.x * W + wave;
  const int4* bt = p.batches + wv * p.KB;
  const size_t slot0 = wv * p.KB * kBatchEdges;
  const int4 idle = make_int4(-1, 0, 0, 0);
  const int first_info = p.KB > 0 ? CK_AT(bt, 0, p.KB, 10).w : 0;
  const uint32_t pbytes = (uint32_t)NBp * 4u;
  const __amdgpu_buffer_rsrc_t hsrc = plane_rsrc(p.h_prev, pbytes);
  double4 acc = d4(0.0);  // the row sums are formed in fp64
  FwdEpi eo{0.f, 0.f, 0.f, 0.f};
  for (int g0 = 0; g0 < p.KB; g0 += kFwdGroup) {
    const int4 ent = (ln.lane < kFwdGroup && g0 + ln.lane < p.KB)
                         ? CK_AT(bt, g0 + ln.lane, p.KB, 10) : idle;
    int cb[kFwdGroup];
    float wb[kFwdGroup];
#pragma unroll
    for (int q = 0; q < kFwdGroup; ++q) {
      cb[q] = -1;
      wb[q] = 0.f;
      if (g0 + q < p.KB) {
        const int2 pe = CK_AT(p.pedge, slot0 + (size_t)(g0 + q) * kBatchEdges + ln.lane, p.slots, 8);
        cb[q] = pe.x;
        wb[q] = __int_as_float(pe.y);
      }
    }
    const int nq = group_entries<kFwdGroup>(ent, ln.lane);
    if (nq == 0) break;
    int4 dq[kFwdGroup];  // the entries as wave-uniform values
#pragma unroll
    for (int q = 0; q < kFwdGroup; ++q) dq[q] = lane_entry(ent, q);
    float4 hv[TU][I];
    FwdEpi er[TE];
#pragma unroll
    for (int u = 0; u < NU + TU; ++u) {
      if (u >= TU) {  // consume unit u - TU
        const int uc = u - TU, q = uc / NSUB, sb = uc % NSUB;
        if (q < nq) {
          const int4 d = dq[q];
          if (sb == 0 && (d.w & kInfoFirstBit) && !(d.w & kInfoPieceBit)) eo = er[q % TE];
          if (sb * EB < d.z) {
            // rounds past the batch's last edge hold zero rows and weights,
            // so up to 8 rounds run without a branch and all weight shuffles
            // go first (wider rows keep the register-lean per-round form)
            if constexpr (I <= 8) {
              float wj[I];
#pragma unroll
              for (int j = 0; j < I; ++j) {
                const int e = sb * EB + j * P + ln.slot;
                wj[j] = lane_or(__shfl(wb[q], e & 63), e, 0.f);
              }
#pragma unroll
              for (int j = 0; j < I; ++j) acc = fma4d(wj[j], hv[uc % TU][j], acc);
            } else {
#pragma unroll
              for (int j = 0; j < I; ++j) {
                if (sb * EB + j * P >= d.z) break;  // past the batch's last edge (uniform)
                const int e = sb * EB + j * P + ln.slot;
                acc = fma4d(lane_or(__shfl(wb[q], e & 63), e, 0.f), hv[uc % TU][j], acc);
              }
            }
          }
          if (sb == NSUB - 1 && (d.w & kInfoLastBit)) {  // the row (or piece) is complete
            acc = sum_slots_d<L>(acc, ln.sub);
            if (d.w & kInfoPieceBit) {
              if (ln.slot == 0) red[piece_slot<W>(d.w)][ln.sub] = acc;
            } else {
              fwd_epilogue(p, ln, d.x, acc, eo);
            }
            acc = d4(0.0);
          }
        }
      }
      if (u < NU) {  // issue unit u into the slot just freed
        const int q = u / NSUB, sb = u % NSUB;
        if (q < nq) {
          const int4 d = dq[q];
          if (sb * EB < d.z) {
#pragma unroll
            for (int j = 0; j < I; ++j) {
              if (sb * EB + j * P >= d.z) {  // past the batch's last edge (uniform): no load
                hv[u % TU][j] = f4(0.f);
                continue;
              }
              const int e = sb * EB + j * P + ln.slot;
              const int cj = lane_or(__shfl(cb[q], e & 63), e, -1);
              hv[u % TU][j] = gather4(hsrc, (cj >= 0 && ln.ok) ? (uint32_t)cj * rowb + colb : kNoRow,
                                      pbytes, 11);
            }
          }
          if (sb == 0)
            er[q % TE] = fwd_epi_load(
                p, ln, ((d.w & kInfoFirstBit) && !(d.w & kInfoPieceBit)) ? d.x : -1, d.y);
        }
      }
    }
  }
  if (first_info & kInfoGroupBit) {
    // the wave holding a split row's last piece (its first segment) adds the
    // row's pieces in piece order; its operand loads overlap the barrier
    const int4 d0 = CK_AT(bt, 0, p.KB, 10);
    const bool combine = d0.x >= 0 && (d0.w & kInfoCombineBit);
    const FwdEpi ce = fwd_epi_load(p, ln, combine ? d0.x : -1, d0.y);
    __syncthreads();
    if (combine) {
      int q0, q1;
      piece_range<W>(d0.w, q0, q1);
      double4 a = red[q0][ln.sub];
      for (int q = q0 + 1; q <= q1; ++q) a = add4d(a, red[q][ln.sub]);
      fwd_epilogue(p, ln, d0.x, a, ce);
    }
  }
}

struct BwdArgs {
  const int4* batches;    // schedule of the transposed CSR: KB batch entries per wave
  const int2* pedge;      // [slots] padded edge slots: {destination node or -1, bits of the value}
  float* gv;              // [chunks][slots] edge gradient per slot, one row per column chunk
  int64_t slots;
  int KB;
  const float* leak;
  const float* ga_in;     // ga^(s) [N][Bp] (gathered); nullptr: no edge pass (init)
  const float* h_sm1;     // h^(s-1) [N][Bp]
  float* gh;              // in: g^(s) (ignored when ga_in == nullptr), out: g^(s-1)
  const float* G_t;       // [N][Bp] upstream gradient entering at microstep s-1, or nullptr
  // elementwise pass of microstep s-1 (skipped when a_k1 == nullptr, i.e. s-1 == 0)
  const float* a_k1;      // a^(s-1)
  const float* h_k1;      // h^(s-2)
  float* ga_out;          // ga^(s-1)
  float* gdrives_t;       // [n_in][B] of input step t(s-1), accumulated
  float* gleak;           // [chunks][N] accumulated (written when first_k1)
  float* gbias;           // [chunks][N]
  float* gstate0;         // [B][N], written when s-1 == 0
  int first_k1;           // 1: overwrite gleak/gbias instead of accumulating
  int first_gv;           // 1: overwrite gv instead of accumulating
  int N, B, Bp, n_in;
};

// Row operands of the backward epilogue (this lane's column), including the
// old values of the three sums it accumulates into.
struct BwdEpi {
  float lam, gold, gin, ak, qk, gdo, glo, gbo;
  int ks;
};

// row: the node (or -1 for none); ks: its input slot from the schedule entry
__device__ __forceinline__ BwdEpi bwd_epi_load(const BwdArgs& p, const Lanes& ln, int row, int ks) {
  BwdEpi e{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, -1};
  if (row < 0) return e;
  // per-row values first (the same for every lane)
  e.lam = ld_row(p.leak, row, p.N, 1);
  if (p.a_k1 != nullptr) {
    e.ks = ks;
    // the two row sums this launch adds to (written below by lane 0 only)
    if (!p.first_k1 && ln.lane == 0) {
      e.glo = CK_AT(p.gleak + (size_t)blockIdx.y * p.N, row, p.N, 20);
      e.gbo = CK_AT(p.gbias + (size_t)blockIdx.y * p.N, row, p.N, 20);
    }
  }
  if (!ln.eok) return e;
  const int c = ln.ecol;
  const size_t off = (size_t)row * p.Bp + c;
  [[maybe_unused]] const size_t NBp = (size_t)p.N * p.Bp;
  if (p.ga_in != nullptr) e.gold = CK_AT(p.gh, off, NBp, 12);
  if (c < p.B) {
    if (p.G_t) e.gin = CK_AT(p.G_t, off, NBp, 13);
    if (p.a_k1 != nullptr) {
      e.ak = CK_AT(p.a_k1, off, NBp, 14);
      e.qk = CK_AT(p.h_k1, off, NBp, 15);
      if (e.ks >= 0)
        e.gdo = CK_AT(p.gdrives_t, (size_t)e.ks * p.B + c, (size_t)p.n_in * p.B, 17);
    }
  }
  return e;
}

// g^(s-1) = (1 - leak) g^(s) + (W^T ga^(s))[row] (+ G entering at s-1), then the
// elementwise pass of microstep s-1 (leak/bias row reductions, drive gradient),
// or the initial-state gradient when s-1 == 0.
template <int L>
__device__ __forceinline__ void bwd_epilogue(const BwdArgs& p, const Lanes& ln, int row,
                                             float4 acc, const BwdEpi& e) {
  const int c = ln.ecol;
  const size_t off = (size_t)row * p.Bp + (ln.eok ? c : 0);
  const bool real_col = ln.eok && c < p.B;
  float g = pick4(acc, ln.slot);
  if (p.ga_in != nullptr) g = fmaf(1.0f - e.lam, e.gold, g);
  if (p.G_t && real_col) g += e.gin;
  if (p.a_k1 == nullptr) {
    if (real_col) CK_AT(p.gstate0, (size_t)c * p.N + row, (size_t)p.B * p.N, 16) = g;
    return;
  }
  float lsum = 0.f, bsum = 0.f;
  if (ln.eok) {
    float ga = 0.f;
    if (real_col) {
      lsum = g * (tanhf(e.ak) - e.qk);
      ga = g * e.lam * sech2f(e.ak);
      bsum = ga;
      if (e.ks >= 0)
        CK_AT(p.gdrives_t, (size_t)e.ks * p.B + c, (size_t)p.n_in * p.B, 17) = e.gdo + ga;
    } else {
      g = 0.f;
    }
    CK_AT(p.gh, off, (size_t)p.N * p.Bp, 18) = g;
    CK_AT(p.ga_out, off, (size_t)p.N * p.Bp, 19) = ga;
  }
  lsum = epilogue_sum<L>(lsum, ln.slot);
  bsum = epilogue_sum<L>(bsum, ln.slot);
  if (ln.lane == 0) {
    CK_AT(p.gleak + (size_t)blockIdx.y * p.N, row, p.N, 20) = p.first_k1 ? lsum : e.glo + lsum;
    CK_AT(p.gbias + (size_t)blockIdx.y * p.N, row, p.N, 20) = p.first_k1 ? bsum : e.gbo + bsum;
  }
}

template <int L>
__global__ __launch_bounds__(waves_for_lanes(L) * 64) void bwd_step(BwdArgs p) {
  using Gm = Geom<L>;
  using Pp = Pipe<L, kBwdGroup>;
  constexpr int W = waves_for_lanes(L);
  constexpr int P = Gm::P, I = Gm::I, EB = Gm::EB;
  constexpr int NSUB = Pp::NSUB, NU = Pp::NU, TU = Pp::TU, TE = Pp::TE;
  __shared__ float4 red[2 * W][16];  // partial sums of pieces, by piece number
  const Lanes ln = lanes<L>(p.Bp);
  const int wave = __builtin_amdgcn_readfirstlane(ln.wave);
  const uint32_t colb = (uint32_t)(ln.ok ? ln.col : 0) * 4u;
  const uint32_t rowb = (uint32_t)p.Bp * 4u;
  [[maybe_unused]] const size_t NBp = (size_t)p.N * p.Bp;
  const size_t wv = (size_t)blockIdx.x * W + wave;
  const int4* bt = p.batches + wv * p.KB;
  const size_t slot0 = wv * p.KB * kBatchEdges;
  // the seeding launch (no ga_in) has no edge pass: every batch counts as empty
  const bool edges = p.ga_in != nullptr;
  float* gv = p.gv + (size_t)blockIdx.y * p.slots;
  // in gather round (sb, j) slot q handles batch edge sb*EB + j*P + q; the
  // edge term of round (sb, j = sub) is kept by lane (q, sub)
  const bool keeps = ln.slot < P && ln.sub < I;
  const int4 idle = make_int4(-1, 0, 0, 0);
  const int first_info = p.KB > 0 ? CK_AT(bt, 0, p.KB, 10).w : 0;
  const uint32_t pbytes = (uint32_t)NBp * 4u;
  const __amdgpu_buffer_rsrc_t gsrc = plane_rsrc(p.ga_in, pbytes);
  float4 acc = f4(0.f);
  float4 hj = f4(0.f);
  BwdEpi eo{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, -1};
  for (int g0 = 0; g0 < p.KB; g0 += kBwdGroup) {
    const int4 ent = (ln.lane < kBwdGroup && g0 + ln.lane < p.KB)
                         ? CK_AT(bt, g0 + ln.lane, p.KB, 10) : idle;
    int cb[kBwdGroup];
    float wb[kBwdGroup];
#pragma unroll
    for (int q = 0; q < kBwdGroup; ++q) {
      cb[q] = -1;
      wb[q] = 0.f;
      if (edges && g0 + q < p.KB) {
        const int2 pe = CK_AT(p.pedge, slot0 + (size_t)(g0 + q) * kBatchEdges + ln.lane, p.slots, 8);
        cb[q] = pe.x;
        wb[q] = __int_as_float(pe.y);
      }
    }
    const int nq = group_entries<kBwdGroup>(ent, ln.lane);
    if (nq == 0) break;
    int4 dq[kBwdGroup];  // the entries as wave-uniform values
#pragma unroll
    for (int q = 0; q < kBwdGroup; ++q) dq[q] = lane_entry(ent, q);
    float4 gav[TU][I];
    float gold[TU];
    float4 hr[TE];
#pragma unroll
    for (int u = 0; u < NU + TU; ++u) {
      if (u >= TU) {  // consume unit u - TU
        const int uc = u - TU, q = uc / NSUB, sb = uc % NSUB;
        if (q < nq) {
          const int4 d = dq[q];
          const int cnt = edges ? d.z : 0;
          if (sb == 0 && (d.w & kInfoFirstBit)) {
            hj = hr[q % TE];
            // requested here, they arrive while the row's gathers are consumed
            if (!(d.w & kInfoPieceBit)) eo = bwd_epi_load(p, ln, d.x, d.y);
          }
          if (sb * EB < cnt) {
            // one branch per round: the backward's rounds carry more arithmetic
            // (the edge dot products), which a branch-free form would spend on
            // rounds past the batch's end
            float mine = 0.f;
#pragma unroll
            for (int j = 0; j < I; ++j) {
              if (sb * EB + j * P >= cnt) break;  // past the batch's last edge (uniform)
              const int e = sb * EB + j * P + ln.slot;
              const float4 g4 = gav[uc % TU][j];
              acc = fma4(lane_or(__shfl(wb[q], e & 63), e, 0.f), g4, acc);
              const float tot = slot_sum<L>(dot4(g4, hj), ln.slot);
              if (ln.sub == j) mine = tot;
            }
            const int ek = sb * EB + ln.sub * P + ln.slot;
            if (keeps && ek < cnt)
              CK_AT(gv, slot0 + (size_t)(g0 + q) * kBatchEdges + ek, p.slots, 22) =
                  gold[uc % TU] + mine;
          }
          if (sb == NSUB - 1 && (d.w & kInfoLastBit)) {
            acc = sum_slots<L>(acc, ln.sub);
            if (d.w & kInfoPieceBit) {
              if (ln.slot == 0) red[piece_slot<W>(d.w)][ln.sub] = acc;
            } else {
              bwd_epilogue<L>(p, ln, d.x, acc, eo);
            }
            acc = f4(0.f);
          }
        }
      }
      if (u < NU) {  // issue unit u into the slot just freed
        const int q = u / NSUB, sb = u % NSUB;
        if (q < nq) {
          const int4 d = dq[q];
          const int cnt = edges ? d.z : 0;
          if (sb * EB < cnt) {
#pragma unroll
            for (int j = 0; j < I; ++j) {
              if (sb * EB + j * P >= cnt) break;  // past the batch's last edge (uniform)
              const int e = sb * EB + j * P + ln.slot;
              const int cj = lane_or(__shfl(cb[q], e & 63), e, -1);
              gav[u % TU][j] = gather4(gsrc, (cj >= 0 && ln.ok) ? (uint32_t)cj * rowb + colb : kNoRow,
                                       pbytes, 24);
            }
            const int ek = sb * EB + ln.sub * P + ln.slot;
            gold[u % TU] = (keeps && ek < cnt && !p.first_gv)
                               ? CK_AT(gv, slot0 + (size_t)(g0 + q) * kBatchEdges + ek, p.slots, 21)
                               : 0.f;
          }
          if (sb == 0)  // the row's own h^(s-1), for the edge dot products
            hr[q % TE] = ((d.w & kInfoFirstBit) && cnt > 0)
                             ? ld4c(p.h_sm1, (uint32_t)d.x * rowb + colb, NBp, 23) : f4(0.f);
        }
      }
    }
  }
  if (first_info & kInfoGroupBit) {
    const int4 d0 = CK_AT(bt, 0, p.KB, 10);
    const bool combine = d0.x >= 0 && (d0.w & kInfoCombineBit);
    const BwdEpi ce = bwd_epi_load(p, ln, combine ? d0.x : -1, d0.y);
    __syncthreads();
    if (combine) {
      int q0, q1;
      piece_range<W>(d0.w, q0, q1);
      float4 a = red[q0][ln.sub];
      for (int q = q0 + 1; q <= q1; ++q) a = add4(a, red[q][ln.sub]);
      bwd_epilogue<L>(p, ln, d0.x, a, ce);
    }
  }
}

// ---------------------------------------------------------------- small kernels

// dst[idx[k]] = sum over chunks c (ascending) of src[c][k], for idx[k] >= 0
__global__ void scatter_sum_f32(const float* __restrict__ src, int chunks,
                                const int32_t* __restrict__ idx, int64_t n,
                                float* __restrict__ dst) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= n) return;
  const int32_t i = idx[k];
  if (i < 0) return;
  float s = src[k];
  for (int c = 1; c < chunks; ++c) s += src[(size_t)c * n + k];
  dst[i] = s;
}

// Padded edge slot k of a schedule: {its node (or -1), bits of its edge value
// (0 for an empty slot)}, from the caller-ordered edge values.
__global__ void pack_edges(const float* __restrict__ values, const int32_t* __restrict__ pcol,
                           const int32_t* __restrict__ pperm, int64_t n, int2* __restrict__ out) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= n) return;
  const int32_t i = pperm[k];
  out[k] = make_int2(pcol[k], i >= 0 ? __float_as_int(values[i]) : 0);
}

// Tiled transposes between the node-major state planes [N][Bp] and the
// caller's batch-major [B][N] layout, 32 x 32 tiles through LDS so that both
// the reads and the writes are coalesced.  Plane t of `planes` starts at
// t * pstride floats; grid = (ceil(N / 32), <= ceil(cols / 32), <= T), the y
// and z loops cover what the grid does not.
constexpr int kTile = 32;

// bm[t][b][n] = planes[t][n][b] for b < B
__global__ __launch_bounds__(256) void planes_to_batch_major(const float* __restrict__ planes,
                                                             size_t pstride, int64_t T, int N,
                                                             int B, int Bp, float* __restrict__ bm) {
  __shared__ float tile[kTile][kTile + 1];
  const int tx = threadIdx.x % kTile, ty = threadIdx.x / kTile;
  const int n0 = blockIdx.x * kTile;
  for (int64_t t = blockIdx.z; t < T; t += gridDim.z)
    for (int b0 = blockIdx.y * kTile; b0 < B; b0 += gridDim.y * kTile) {
      const float* src = planes + (size_t)t * pstride;
      for (int i = ty; i < kTile; i += blockDim.x / kTile) {
        const int n = n0 + i, b = b0 + tx;
        tile[i][tx] = (n < N && b < B) ? src[(size_t)n * Bp + b] : 0.0f;
      }
      __syncthreads();
      float* dst = bm + (size_t)t * B * N;
      for (int i = ty; i < kTile; i += blockDim.x / kTile) {
        const int b = b0 + i, n = n0 + tx;
        if (b < B && n < N) dst[(size_t)b * N + n] = tile[tx][i];
      }
      __syncthreads();
    }
}

// planes[t][n][b] = bm[t][b][n] for b < B, 0 for B <= b < Bp
__global__ __launch_bounds__(256) void batch_major_to_planes(const float* __restrict__ bm,
                                                             int64_t T, int N, int B, int Bp,
                                                             size_t pstride,
                                                             float* __restrict__ planes) {
  __shared__ float tile[kTile][kTile + 1];
  const int tx = threadIdx.x % kTile, ty = threadIdx.x / kTile;
  const int n0 = blockIdx.x * kTile;
  for (int64_t t = blockIdx.z; t < T; t += gridDim.z)
    for (int b0 = blockIdx.y * kTile; b0 < Bp; b0 += gridDim.y * kTile) {
      const float* src = bm + (size_t)t * B * N;
      for (int i = ty; i < kTile; i += blockDim.x / kTile) {
        const int b = b0 + i, n = n0 + tx;
        tile[i][tx] = (b < B && n < N) ? src[(size_t)b * N + n] : 0.0f;
      }
      __syncthreads();
      float* dst = planes + (size_t)t * pstride;
      for (int i = ty; i < kTile; i += blockDim.x / kTile) {
        const int n = n0 + i, b = b0 + tx;
        if (n < N && b < Bp) dst[(size_t)n * Bp + b] = tile[tx][i];
      }
      __syncthreads();
    }
}

inline dim3 transpose_grid(int64_t N, int64_t cols, int64_t T) {
  return dim3((unsigned)std::max<int64_t>(1, (N + kTile - 1) / kTile),
              (unsigned)std::min<int64_t>((cols + kTile - 1) / kTile, 65535),
              (unsigned)std::min<int64_t>(T, 65535));
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
  int wide;                // schedule index: 1 for 16-wave workgroups, 0 for 8-wave
  int64_t slots_f, slots_b;  // padded edge slots of the forward / backward schedule
  size_t plane;  // floats per [N][Bp] plane
  bool resident;  // the call runs the XCD-resident kernels (one launch per call)
  bool blocked;   // the forward runs the blocked kernels (two launches per microstep)
  bool blocked_bwd;  // so does the backward (else it runs the per-microstep kernels)
  ResDims rd;
  BlkDims bd;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct WsLayout {
  size_t v, gv, h0, gh, ga0, ga1, part, gt, total;
};

WsLayout ws_layout(const Dims& d) {
  WsLayout w;
  size_t o = 0;
  w.v = o;   o = align256(o + (size_t)std::max<int64_t>({d.slots_f, d.slots_b, 1}) * 8);
  w.gv = o;  o = align256(o + (size_t)d.chunks * std::max<int64_t>(d.slots_b, 1) * 4);
  w.h0 = o;  o = align256(o + d.plane * 4);
  w.gh = o;  o = align256(o + d.plane * 4);
  w.ga0 = o; o = align256(o + d.plane * 4);
  w.ga1 = o; o = align256(o + d.plane * 4);
  w.part = o;  // per-chunk leak/bias partial sums when the batch spans several chunks
  if (d.chunks > 1) o = align256(o + 2 * (size_t)d.chunks * d.N * 4);
  w.gt = o;  // the upstream gradient as T node-major planes (backward only)
  o = align256(o + (size_t)d.T * d.plane * 4);
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
  if (B >= (1LL << 30) || (g->N * Bp) >= (1LL << 30) || T * M >= (1LL << 31) ||
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
  d->wide = waves_for_lanes(d->L) == 16 ? 1 : 0;
  d->slots_f = g->fwd[d->wide].slots;
  d->slots_b = g->bwd[d->wide].slots;
  d->plane = (size_t)g->N * Bp;
  // the resident kernels address the [T][n_in][B] drives and the [B][N]
  // upstream-gradient and initial-state tensors of one step with 32-bit byte
  // offsets below 2^31 (range-checked buffer accesses)
  d->resident = g->res_ok != 0 && std::max(g->N, g->n_in) * B * 4 < (1LL << 31);
  d->rd = ResDims{g->N, (g->N + 7) / 8 * 8, B, Bp / 4, g->n_in, T, M, T * M};
  d->blocked = !d->resident && blk_fits(g, Bp);
  d->blocked_bwd = d->blocked && g->blk_bwd_ok != 0;
  d->bd = BlkDims{g->N, g->E, g->n_in, T, B, M, T * M, Bp, (int)(Bp / 4), d->plane};
  return CK_OK;
}

// Workspace bytes of a call (either direction).
size_t ws_total(const ck_graph* g, const Dims& d) {
  if (d.resident) return res_ws_layout(g, d.rd).total;
  if (d.blocked_bwd) return blk_ws_layout(g, d.bd).total;
  // a blocked forward's regions, then (from offset 0 again) the per-microstep
  // backward's: the backward reads nothing the forward left in the workspace
  if (d.blocked) return std::max(blk_ws_layout(g, d.bd).fwd_end, ws_layout(d).total);
  return ws_layout(d).total;
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
  if (saved_bytes)
    *saved_bytes = d.resident ? res_saved_bytes(d.rd) : 2 * (size_t)d.S * d.plane * sizeof(float);
  if (workspace_bytes) *workspace_bytes = ws_total(g, d);
  return CK_OK;
}

extern "C" ck_status ck_recurrence_path(ck_graph_t g, int64_t B, int* path) {
  clear_error();
  ck_status rc = check_graph(g);
  if (rc != CK_OK) return rc;
  if (!path) {
    set_error("path output pointer is NULL");
    return CK_ERR_NULL_ARG;
  }
  Dims d;
  rc = make_dims(g, 1, B, 1, &d);
  if (rc != CK_OK) return rc;
  *path = d.resident ? 1 : d.blocked_bwd ? 3 : d.blocked ? 2 : 0;
  return CK_OK;
}

namespace {

// Bytes of the workspace a forward call touches (its leading part: the
// backward's regions follow it).
size_t forward_ws_bytes(const ck_graph* g, const Dims& d) {
  if (d.resident) return res_forward_ws_bytes(g, d.rd);
  if (d.blocked) return blk_ws_layout(g, d.bd).fwd_end;
  return ws_layout(d).gh;
}

// Argument checks shared by both forward entry points.
ck_status forward_checks(ck_graph_t g, const float* edge_values, const float* leak,
                         const float* bias, const float* drives, const float* state0, int64_t T,
                         int64_t B, int64_t microsteps, float* out, void* saved, Dims* d) {
  ck_status rc = check_graph(g);
  if (rc != CK_OK) return rc;
  rc = make_dims(g, T, B, microsteps, d);
  if (rc != CK_OK) return rc;
  if ((d->E > 0 && !edge_values) || !leak || !bias || (d->n_in > 0 && !drives) || !state0 ||
      !out || !saved) {
    set_error("NULL pointer for a non-empty tensor in forward");
    return CK_ERR_NULL_ARG;
  }
  return check_aligned(saved, "saved");
}

// The forward once its arguments are checked; `workspace` holds at least
// forward_ws_bytes(g, d) bytes.
// `profile`: false keeps the measurement hook's events out of the call.
ck_status forward_body(const ck_graph* g, const Dims& d, const float* edge_values,
                       const float* leak, const float* bias, const float* drives,
                       const float* state0, float* out, void* saved, void* workspace,
                       hipStream_t stream, bool profile) {
  if (d.resident)
    return res_forward(g, d.rd, edge_values, leak, bias, drives, state0, out, saved, workspace,
                       stream, profile);
  if (d.blocked)
    return blk_forward(g, d.bd, edge_values, leak, bias, drives, state0, out, saved, workspace,
                       stream, profile);
  ck_status rc = CK_OK;
  const WsLayout ws = ws_layout(d);
  char* wsb = static_cast<char*>(workspace);
  int2* pedge = reinterpret_cast<int2*>(wsb + ws.v);
  float* h0 = reinterpret_cast<float*>(wsb + ws.h0);
  float* hplanes = static_cast<float*>(saved);
  float* aplanes = hplanes + (size_t)d.S * d.plane;
  const Schedule& sc = g->fwd[d.wide];
  if (d.E > 0)
    pack_edges<<<grid1(sc.slots), 256, 0, stream>>>(edge_values, sc.pcol, sc.pperm, sc.slots, pedge);
  batch_major_to_planes<<<transpose_grid(d.N, d.Bp, 1), 256, 0, stream>>>(
      state0, 1, (int)d.N, (int)d.B, (int)d.Bp, d.plane, h0);
  const FwdFn kern = KT::fwd[d.L - 1];
  const dim3 grid(sc.num_wgs, d.chunks), block(sc.waves * 64);
  FwdArgs a{};
  a.batches = sc.batches;
  a.KB = sc.KB;
  a.pedge = pedge;
  a.slots = sc.slots;
  a.leak = leak;
  a.bias = bias;
  a.N = (int)d.N;
  a.B = (int)d.B;
  a.Bp = (int)d.Bp;
  a.n_in = (int)d.n_in;
  for (int64_t s = 1; s <= d.S; ++s) {
    const int64_t t = (s - 1) / d.M;
    a.drives_t = d.n_in > 0 ? drives + (size_t)t * d.n_in * d.B : nullptr;
    a.h_prev = s == 1 ? h0 : hplanes + (size_t)(s - 2) * d.plane;
    a.h_next = hplanes + (size_t)(s - 1) * d.plane;
    a.a_next = aplanes + (size_t)(s - 1) * d.plane;
    if (profile)
      rc = timed_launch(g_profile.fwd, stream,
                        [&] { hipLaunchKernelGGL(kern, grid, block, 0, stream, a); });
    else
      hipLaunchKernelGGL(kern, grid, block, 0, stream, a);
    if (rc != CK_OK) return rc;
  }
  // out[t] = the state after the last microstep of step t, in [B][N]
  planes_to_batch_major<<<transpose_grid(d.N, d.B, d.T), 256, 0, stream>>>(
      hplanes + (size_t)(d.M - 1) * d.plane, (size_t)d.M * d.plane, d.T, (int)d.N, (int)d.B,
      (int)d.Bp, out);
  CK_HIP_TRY(hipGetLastError());
#ifdef CK_CHECKED
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  CK_HIP_TRY(hipStreamIsCapturing(stream, &cap));
  if (cap == hipStreamCaptureStatusNone) {
    CK_HIP_TRY(hipStreamSynchronize(stream));
    unsigned flag = 0;
    CK_HIP_TRY(hipMemcpyFromSymbol(&flag, HIP_SYMBOL(g_ck_err), sizeof(unsigned)));
    if (flag) {
      const unsigned zero = 0;
      (void)hipMemcpyToSymbol(HIP_SYMBOL(g_ck_err), &zero, sizeof(unsigned));
      set_error("bounds check failed in %s: site mask 0x%x", "forward", flag);
      return CK_ERR_HIP;
    }
  }
#endif
  return CK_OK;
}

}  // namespace

extern "C" ck_status ck_recurrence_forward(ck_graph_t g, const float* edge_values,
                                           const float* leak, const float* bias,
                                           const float* drives, const float* state0, int64_t T,
                                           int64_t B, int64_t microsteps, float* out, void* saved,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
  clear_error();
  Dims d;
  ck_status rc = forward_checks(g, edge_values, leak, bias, drives, state0, T, B, microsteps, out,
                                saved, &d);
  if (rc != CK_OK) return rc;
  if (!workspace) {
    set_error("NULL workspace in forward");
    return CK_ERR_NULL_ARG;
  }
  rc = check_aligned(workspace, "workspace");
  if (rc != CK_OK) return rc;
  const size_t need = ws_total(g, d);
  if (workspace_bytes < need) {
    set_error("workspace of %zu bytes is below the %zu required", workspace_bytes, need);
    return CK_ERR_WORKSPACE;
  }
  return forward_body(g, d, edge_values, leak, bias, drives, state0, out, saved, workspace,
                      stream, true);
}

extern "C" ck_status ck_recurrence_forward_noalloc(ck_graph_t g, const float* edge_values,
                                                   const float* leak, const float* bias,
                                                   const float* drives, const float* state0,
                                                   int64_t T, int64_t B, int64_t microsteps,
                                                   float* out, void* saved, hipStream_t stream) {
  clear_error();
  Dims d;
  ck_status rc = forward_checks(g, edge_values, leak, bias, drives, state0, T, B, microsteps, out,
                                saved, &d);
  if (rc != CK_OK) return rc;
  const size_t need = forward_ws_bytes(g, d);
  if (need > kScratchBytes) {
    set_error("this forward needs %zu bytes of scratch, above the %zu of the allocation-free "
              "entry point; use ck_recurrence_forward with a workspace", need, kScratchBytes);
    return CK_ERR_TOO_LARGE;
  }
  void* ws = scratch_ptr(g->device);
  if (ws == nullptr) {
    set_error("device scratch of device %d was not resolved at graph creation", g->device);
    return CK_ERR_HIP;
  }
  return forward_body(g, d, edge_values, leak, bias, drives, state0, out, saved, ws, stream,
                      false);
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
  rc = check_aligned(saved, "saved");
  if (rc == CK_OK) rc = check_aligned(workspace, "workspace");
  if (rc != CK_OK) return rc;
  if (d.resident) {
    const size_t need = res_ws_layout(g, d.rd).total;
    if (workspace_bytes < need) {
      set_error("workspace of %zu bytes is below the %zu required", workspace_bytes, need);
      return CK_ERR_WORKSPACE;
    }
    return res_backward(g, d.rd, edge_values, leak, state0, saved, grad_out, grad_edge_values,
                        grad_leak, grad_bias, grad_drives, grad_state0, workspace, stream);
  }
  if (d.blocked_bwd) {
    const size_t need = blk_ws_layout(g, d.bd).total;
    if (workspace_bytes < need) {
      set_error("workspace of %zu bytes is below the %zu required", workspace_bytes, need);
      return CK_ERR_WORKSPACE;
    }
    return blk_backward(g, d.bd, edge_values, leak, state0, saved, grad_out, grad_edge_values,
                        grad_leak, grad_bias, grad_drives, grad_state0, workspace, stream);
  }
  const WsLayout ws = ws_layout(d);
  if (workspace_bytes < ws.total) {
    set_error("workspace of %zu bytes is below the %zu required", workspace_bytes, ws.total);
    return CK_ERR_WORKSPACE;
  }
  char* wsb = static_cast<char*>(workspace);
  int2* pedge = reinterpret_cast<int2*>(wsb + ws.v);
  float* gv = reinterpret_cast<float*>(wsb + ws.gv);
  float* h0 = reinterpret_cast<float*>(wsb + ws.h0);
  float* gh = reinterpret_cast<float*>(wsb + ws.gh);
  float* gabuf[2] = {reinterpret_cast<float*>(wsb + ws.ga0), reinterpret_cast<float*>(wsb + ws.ga1)};
  const float* hplanes = static_cast<const float*>(saved);
  const float* aplanes = hplanes + (size_t)d.S * d.plane;
  auto hplane = [&](int64_t s) { return s == 0 ? h0 : hplanes + (size_t)(s - 1) * d.plane; };
  auto aplane = [&](int64_t s) { return aplanes + (size_t)(s - 1) * d.plane; };
  const Schedule& sc = g->bwd[d.wide];
  if (d.E > 0)
    pack_edges<<<grid1(sc.slots), 256, 0, stream>>>(edge_values, sc.pcol, sc.pperm, sc.slots, pedge);
  batch_major_to_planes<<<transpose_grid(d.N, d.Bp, 1), 256, 0, stream>>>(
      state0, 1, (int)d.N, (int)d.B, (int)d.Bp, d.plane, h0);
  // the upstream gradient [T][B][N] as node-major planes, so each row's
  // epilogue reads its B values from one place instead of B cache lines
  float* gt = reinterpret_cast<float*>(wsb + ws.gt);
  batch_major_to_planes<<<transpose_grid(d.N, d.Bp, d.T), 256, 0, stream>>>(
      grad_out, d.T, (int)d.N, (int)d.B, (int)d.Bp, d.plane, gt);
  if (d.n_in > 0)
    zero_f32<<<grid1(d.T * d.n_in * d.B), 256, 0, stream>>>(grad_drives, d.T * d.n_in * d.B);
  const BwdFn kern = KT::bwd[d.L - 1];
  const dim3 grid(sc.num_wgs, d.chunks), block(sc.waves * 64);
  BwdArgs a{};
  a.batches = sc.batches;
  a.KB = sc.KB;
  a.pedge = pedge;
  a.gv = gv;
  a.slots = sc.slots;
  a.gh = gh;
  a.leak = leak;
  float* part = reinterpret_cast<float*>(wsb + ws.part);
  a.gleak = d.chunks > 1 ? part : grad_leak;
  a.gbias = d.chunks > 1 ? part + (size_t)d.chunks * d.N : grad_bias;
  a.gstate0 = grad_state0;
  a.N = (int)d.N;
  a.B = (int)d.B;
  a.Bp = (int)d.Bp;
  a.n_in = (int)d.n_in;
  // Launch "s" covers the edge pass of microstep s and the elementwise pass of
  // microstep s-1; launch S+1 has no edge pass and seeds g^(S) = G[T-1].
  for (int64_t s = d.S + 1; s >= 1; --s) {
    const bool init = s == d.S + 1;
    a.ga_in = init ? nullptr : gabuf[s % 2];
    a.h_sm1 = init ? nullptr : hplane(s - 1);
    a.first_gv = s == d.S ? 1 : 0;
    a.first_k1 = init ? 1 : 0;
    const int64_t k1 = s - 1;  // microstep whose elementwise pass runs here
    a.G_t = (k1 >= 1 && k1 % d.M == 0) ? gt + (size_t)((k1 - 1) / d.M) * d.plane : nullptr;
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
                      [&] { hipLaunchKernelGGL(kern, grid, block, 0, stream, a); });
    if (rc != CK_OK) return rc;
  }
  if (d.chunks > 1) {
    sum_chunks<<<grid1(d.N), 256, 0, stream>>>(a.gleak, d.chunks, d.N, grad_leak);
    sum_chunks<<<grid1(d.N), 256, 0, stream>>>(a.gbias, d.chunks, d.N, grad_bias);
  }
  if (d.E > 0)
    scatter_sum_f32<<<grid1(sc.slots), 256, 0, stream>>>(gv, d.chunks, sc.pperm, sc.slots,
                                                         grad_edge_values);
  CK_HIP_TRY(hipGetLastError());
#ifdef CK_CHECKED
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  CK_HIP_TRY(hipStreamIsCapturing(stream, &cap));
  if (cap == hipStreamCaptureStatusNone) {
    CK_HIP_TRY(hipStreamSynchronize(stream));
    unsigned flag = 0;
    CK_HIP_TRY(hipMemcpyFromSymbol(&flag, HIP_SYMBOL(g_ck_err), sizeof(unsigned)));
    if (flag) {
      const unsigned zero = 0;
      (void)hipMemcpyToSymbol(HIP_SYMBOL(g_ck_err), &zero, sizeof(unsigned));
      set_error("bounds check failed in %s: site mask 0x%x", "backward", flag);
      return CK_ERR_HIP;
    }
  }
#endif
  return CK_OK;
}

extern "C" ck_status ck_recurrence_status(ck_graph_t g, int64_t T, int64_t B,
                                          int64_t microsteps, const void* workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  ck_status rc = check_graph(g);
  if (rc != CK_OK) return rc;
  Dims d;
  rc = make_dims(g, T, B, microsteps, &d);
  if (rc != CK_OK) return rc;
  if (!d.resident) return CK_OK;  // the per-microstep kernels have no waits
  if (!workspace) {
    set_error("workspace is NULL");
    return CK_ERR_NULL_ARG;
  }
  rc = check_aligned(workspace, "workspace");
  if (rc != CK_OK) return rc;
  const size_t need = res_ws_layout(g, d.rd).total;
  if (workspace_bytes < need) {
    set_error("workspace of %zu bytes is below the %zu required", workspace_bytes, need);
    return CK_ERR_WORKSPACE;
  }
  unsigned err = 0;
  rc = res_status(g, d.rd, workspace, stream, &err);
  if (rc != CK_OK) return rc;
  if (err != 0u) {
    set_error("the last resident call on this workspace failed (flag 0x%x: %s%s%s); its outputs "
              "were set to NaN", err, (err & 1u) ? "unexpected workgroup grouping " : "",
              (err & 2u) ? "a wait between XCD workgroups gave up " : "",
              (err & 4u) ? "the saved arena came from a failed forward" : "");
    return CK_ERR_WAIT;
  }
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
  // the events carry no fence of their own: wait for all recorded work first
  if (!g_profile.fwd.empty() || !g_profile.bwd.empty()) CK_HIP_TRY(hipDeviceSynchronize());
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
  drain(g_profile.lif_gather, nullptr, nullptr);
  drain(g_profile.lif_update, nullptr, nullptr);
  return rc;
}

extern "C" ck_status ck_profile_collect_lif(double* gather_ms, int64_t* gather_launches,
                                            double* update_ms, int64_t* update_launches) {
  clear_error();
  ck_status rc = CK_OK;
  if (!g_profile.lif_gather.empty() || !g_profile.lif_update.empty())
    CK_HIP_TRY(hipDeviceSynchronize());
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
  drain(g_profile.lif_gather, gather_ms, gather_launches);
  drain(g_profile.lif_update, update_ms, update_launches);
  return rc;
}
