// graph_build.hip -- ck_graph_create and friends: validation, CSR / transposed
// CSR construction with a stable LSD radix sort, input-slot map and the upload
// of the row schedules (planned in schedule.cpp).
//
// The graph is given as caller-ordered src/dst lists (connectome-kernels
// README, "Use"); parameters stay in that order and the internal permutation is
// invisible.  The backward's state gradient needs the transposed CSR
// ("Design notes").  Edge order inside a row is (other endpoint, caller index):
// a total order, so every array produced here is unique.
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "ck_internal.h"

namespace ckhip {

static thread_local char g_last_error[1024] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

void clear_error() { g_last_error[0] = '\0'; }

ck_status check_graph(const ck_graph* g) {
  if (g == nullptr || g->magic != kGraphMagic) {
    set_error("invalid or destroyed graph handle");
    return CK_ERR_BAD_HANDLE;
  }
  return CK_OK;
}

namespace {

constexpr int64_t kInt32Limit = 2147483647LL;

// ---------------------------------------------------------------- validation
// flags bit 0: an index outside [0, N); bit 1: a duplicate input node.
__global__ void validate_edges(const int64_t* __restrict__ src, const int64_t* __restrict__ dst,
                               int64_t E, int64_t N, unsigned* flags) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  int64_t s = src[e], d = dst[e];
  if (s < 0 || s >= N || d < 0 || d >= N) atomicOr(flags, 1u);
}

__global__ void validate_inputs(const int64_t* __restrict__ inputs, int64_t n_in, int64_t N,
                                int32_t* __restrict__ seen, unsigned* flags) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= n_in) return;
  int64_t i = inputs[k];
  if (i < 0 || i >= N) {
    atomicOr(flags, 1u);
    return;
  }
  if (atomicAdd(&seen[i], 1) != 0) atomicOr(flags, 2u);
}

__global__ void fill_i32(int32_t* __restrict__ p, int64_t n, int32_t v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void set_input_slots(const int64_t* __restrict__ inputs, int64_t n_in,
                                int32_t* __restrict__ slot) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k < n_in) slot[inputs[k]] = (int32_t)k;
}

// key = major * N + minor, value = caller index (ascending, so ties keep it)
__global__ void make_keys(const int64_t* __restrict__ major, const int64_t* __restrict__ minor,
                          int64_t E, int64_t N, uint64_t* __restrict__ keys,
                          int32_t* __restrict__ vals) {
  int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  keys[e] = (uint64_t)major[e] * (uint64_t)N + (uint64_t)minor[e];
  vals[e] = (int32_t)e;
}

// ---------------------------------------------------------------- radix sort
// Stable LSD radix sort, 4-bit digits, tiles of 2048 keys (256 threads x 8).
constexpr int kRsThreads = 256;
constexpr int kRsItems = 8;
constexpr int kRsTile = kRsThreads * kRsItems;
constexpr int kRsRadix = 16;

__global__ __launch_bounds__(kRsThreads) void rs_histogram(const uint64_t* __restrict__ keys,
                                                           int64_t n, int shift,
                                                           uint32_t* __restrict__ hist,
                                                           int64_t nblocks) {
  __shared__ uint32_t cnt[kRsRadix];
  if (threadIdx.x < kRsRadix) cnt[threadIdx.x] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kRsTile;
  for (int i = threadIdx.x; i < kRsTile; i += kRsThreads) {
    int64_t k = base + i;
    if (k < n) atomicAdd(&cnt[(keys[k] >> shift) & (kRsRadix - 1)], 1u);
  }
  __syncthreads();
  if (threadIdx.x < kRsRadix) hist[threadIdx.x * nblocks + blockIdx.x] = cnt[threadIdx.x];
}

// Exclusive scan of m uint32 values in place, in tiles of kScanTile values
// (256 threads x 16 consecutive values): scan_tile_sums writes each tile's
// total, scan_small scans those totals in one workgroup, scan_tiles scans
// every tile from its total's prefix.  Every load is of 16 consecutive values.
constexpr int kScanPer = 16;
constexpr int kScanTile = 256 * kScanPer;

__device__ __forceinline__ void scan_load(const uint32_t* data, int64_t m, int64_t b,
                                          uint32_t (&x)[kScanPer]) {
  if (b + kScanPer <= m) {
    const uint4* q = reinterpret_cast<const uint4*>(data + b);
#pragma unroll
    for (int i = 0; i < kScanPer / 4; ++i) {
      const uint4 v = q[i];
      x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) x[i] = b + i < m ? data[b + i] : 0u;
  }
}

// Exclusive scan over the 256 threads of a workgroup of one value each.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* sh) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const uint32_t add = t >= off ? sh[t - off] : 0u;
    __syncthreads();
    sh[t] += add;
    __syncthreads();
  }
  const uint32_t r = t ? sh[t - 1] : 0u;
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(256) void scan_tile_sums(const uint32_t* __restrict__ data,
                                                      int64_t m, uint32_t* __restrict__ sums) {
  __shared__ uint32_t sh[256];
  const int64_t b = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanPer;
  uint32_t x[kScanPer];
  scan_load(data, m, b, x);
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) s += x[i];
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) sh[threadIdx.x] += sh[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) sums[blockIdx.x] = sh[0];
}

// Exclusive scan of n values in one workgroup of 256 threads (n up to a few
// thousand: each thread takes a contiguous run).
__global__ __launch_bounds__(256) void scan_small(uint32_t* __restrict__ v, int64_t n) {
  __shared__ uint32_t sh[256];
  const int64_t chunk = (n + 255) / 256;
  const int64_t b = std::min<int64_t>(n, (int64_t)threadIdx.x * chunk);
  const int64_t e = std::min<int64_t>(n, b + chunk);
  uint32_t s = 0;
  for (int64_t i = b; i < e; ++i) s += v[i];
  uint32_t run = block_exclusive_scan(s, sh);
  for (int64_t i = b; i < e; ++i) {
    const uint32_t x = v[i];
    v[i] = run;
    run += x;
  }
}

__global__ __launch_bounds__(256) void scan_tiles(uint32_t* __restrict__ data, int64_t m,
                                                  const uint32_t* __restrict__ sums) {
  __shared__ uint32_t sh[256];
  const int64_t b = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanPer;
  uint32_t x[kScanPer];
  scan_load(data, m, b, x);
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) s += x[i];
  uint32_t run = sums[blockIdx.x] + block_exclusive_scan(s, sh);
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) {
    const uint32_t c = x[i];
    x[i] = run;
    run += c;
  }
  if (b + kScanPer <= m) {
    uint4* q = reinterpret_cast<uint4*>(data + b);
#pragma unroll
    for (int i = 0; i < kScanPer / 4; ++i)
      q[i] = make_uint4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
  } else {
#pragma unroll
    for (int i = 0; i < kScanPer; ++i)
      if (b + i < m) data[b + i] = x[i];
  }
}

__global__ __launch_bounds__(kRsThreads) void rs_scatter(
    const uint64_t* __restrict__ kin, const int32_t* __restrict__ vin, uint64_t* __restrict__ kout,
    int32_t* __restrict__ vout, int64_t n, int shift, const uint32_t* __restrict__ goff,
    int64_t nblocks) {
  // pos[d][t]: elements of this tile with digit < d, plus those with digit d in
  // threads < t.  Thread t owns the items t*8 .. t*8+7 of the tile, in order.
  __shared__ uint32_t pos[kRsRadix][kRsThreads + 1];
  __shared__ uint32_t sums[kRsThreads];
  __shared__ uint32_t dstart[kRsRadix];
  const int t = threadIdx.x;
  for (int d = 0; d < kRsRadix; ++d) pos[d][t] = 0;
  const int64_t base = (int64_t)blockIdx.x * kRsTile + (int64_t)t * kRsItems;
  uint64_t key[kRsItems];
  int32_t val[kRsItems];
#pragma unroll
  for (int i = 0; i < kRsItems; ++i) {
    int64_t idx = base + i;
    if (idx < n) {
      key[i] = kin[idx];
      val[i] = vin[idx];
      pos[(key[i] >> shift) & (kRsRadix - 1)][t] += 1;
    }
  }
  __syncthreads();
  // exclusive scan over the 16 x 256 counts in digit-major order:
  // thread u scans the 16 consecutive entries [16u, 16u + 16)
  const int d0 = t / 16, t0 = (t % 16) * 16;
  uint32_t local = 0;
  for (int j = 0; j < 16; ++j) local += pos[d0][t0 + j];
  sums[t] = local;
  __syncthreads();
  for (int off = 1; off < kRsThreads; off <<= 1) {
    uint32_t add = t >= off ? sums[t - off] : 0u;
    __syncthreads();
    sums[t] += add;
    __syncthreads();
  }
  uint32_t run = t ? sums[t - 1] : 0u;
  for (int j = 0; j < 16; ++j) {
    uint32_t c = pos[d0][t0 + j];
    pos[d0][t0 + j] = run;
    run += c;
  }
  __syncthreads();
  if (t < kRsRadix) dstart[t] = pos[t][0];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kRsItems; ++i) {
    int64_t idx = base + i;
    if (idx < n) {
      int d = (int)((key[i] >> shift) & (kRsRadix - 1));
      uint32_t rank = pos[d][t] - dstart[d];
      pos[d][t] += 1;
      int64_t o = (int64_t)goff[d * nblocks + blockIdx.x] + rank;
      kout[o] = key[i];
      vout[o] = val[i];
    }
  }
}

// row_ptr[i] = number of keys below i * N (keys sorted ascending), i in [0, N]
__global__ void row_starts(const uint64_t* __restrict__ keys, int64_t E, int64_t N,
                           int32_t* __restrict__ ptr) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i > N) return;
  const uint64_t target = (uint64_t)i * (uint64_t)N;
  int64_t lo = 0, hi = E;
  while (lo < hi) {
    int64_t mid = (lo + hi) >> 1;
    if (keys[mid] < target) lo = mid + 1;
    else hi = mid;
  }
  ptr[i] = (int32_t)lo;
}

__global__ void split_keys(const uint64_t* __restrict__ keys, const int32_t* __restrict__ vals,
                           int64_t E, int64_t N, int32_t* __restrict__ minor,
                           int32_t* __restrict__ perm) {
  int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= E) return;
  minor[k] = (int32_t)(keys[k] % (uint64_t)N);
  perm[k] = vals[k];
}

inline unsigned grid_for(int64_t n, int threads) {
  return (unsigned)std::max<int64_t>(1, (n + threads - 1) / threads);
}

// Sort the E edges by key major*N + minor (stable: ties keep caller order) and
// write ptr[N+1], idx[E] = minor, prm[E] = caller index.
ck_status build_compressed(const int64_t* major, const int64_t* minor, int64_t E, int64_t N,
                           int32_t* ptr, int32_t* idx, int32_t* prm, hipStream_t st) {
  if (E == 0) {
    fill_i32<<<grid_for(N + 1, 256), 256, 0, st>>>(ptr, N + 1, 0);
    CK_HIP_TRY(hipGetLastError());
    return CK_OK;
  }
  const int64_t nblocks = (E + kRsTile - 1) / kRsTile;
  uint64_t *k0 = nullptr, *k1 = nullptr;
  int32_t *v0 = nullptr, *v1 = nullptr;
  uint32_t* hist = nullptr;
  // the histogram (digit-major, nblocks per digit) and its tile totals
  const int64_t ntiles = (nblocks * kRsRadix + kScanTile - 1) / kScanTile;
  auto cleanup = [&]() {
    (void)hipFree(k0); (void)hipFree(k1); (void)hipFree(v0); (void)hipFree(v1);
    (void)hipFree(hist);
  };
  if (hipMalloc(&k0, E * 8) != hipSuccess || hipMalloc(&k1, E * 8) != hipSuccess ||
      hipMalloc(&v0, E * 4) != hipSuccess || hipMalloc(&v1, E * 4) != hipSuccess ||
      hipMalloc(&hist, (nblocks * kRsRadix + ntiles) * 4) != hipSuccess) {
    cleanup();
    (void)hipGetLastError();
    set_error("device allocation of %lld bytes of sort scratch failed", (long long)(E * 24));
    return CK_ERR_NOMEM;
  }
  uint32_t* tsum = hist + nblocks * kRsRadix;
  make_keys<<<grid_for(E, 256), 256, 0, st>>>(major, minor, E, N, k0, v0);
  const uint64_t maxkey = (uint64_t)N * (uint64_t)N - 1;
  int bits = 0;
  while (bits < 64 && (maxkey >> bits) != 0) ++bits;
  for (int shift = 0; shift < bits; shift += 4) {
    rs_histogram<<<(unsigned)nblocks, kRsThreads, 0, st>>>(k0, E, shift, hist, nblocks);
    scan_tile_sums<<<(unsigned)ntiles, 256, 0, st>>>(hist, nblocks * kRsRadix, tsum);
    scan_small<<<1, 256, 0, st>>>(tsum, ntiles);
    scan_tiles<<<(unsigned)ntiles, 256, 0, st>>>(hist, nblocks * kRsRadix, tsum);
    rs_scatter<<<(unsigned)nblocks, kRsThreads, 0, st>>>(k0, v0, k1, v1, E, shift, hist, nblocks);
    std::swap(k0, k1);
    std::swap(v0, v1);
  }
  row_starts<<<grid_for(N + 1, 256), 256, 0, st>>>(k0, E, N, ptr);
  split_keys<<<grid_for(E, 256), 256, 0, st>>>(k0, v0, E, N, idx, prm);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess) err = hipStreamSynchronize(st);
  cleanup();
  if (err != hipSuccess) {
    set_error("graph sort failed: %s", hipGetErrorString(err));
    return CK_ERR_HIP;
  }
  return CK_OK;
}

// Padded edge slots of one schedule: slot t * kBatchEdges + k holds edge k of
// batch entry t (its column index and caller index), or -1 past the batch's
// end, so a wave finds the edges of its j-th batch at a fixed offset.
__global__ void pad_edges(const int4* __restrict__ table, int64_t slots,
                          const int32_t* __restrict__ col, const int32_t* __restrict__ perm,
                          int32_t* __restrict__ pcol, int32_t* __restrict__ pperm) {
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= slots) return;
  const int4 t = table[s / kBatchEdges];
  const int k = (int)(s % kBatchEdges);
  const bool live = t.x >= 0 && k < t.z;
  pcol[s] = live ? col[t.y + k] : -1;
  pperm[s] = live ? perm[t.y + k] : -1;
}

// On the device the y field of a table entry carries the row's input slot
// (the kernels find a batch's edges by position in the padded slots, so the
// edge offset is no longer needed there): the row's drive can then be
// requested as soon as the entry arrives.
__global__ void entry_input_slots(int4* __restrict__ table, int64_t n,
                                  const int32_t* __restrict__ input_slot) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  const int4 e = table[t];
  if (e.x >= 0) table[t].y = input_slot[e.x];
}

// Plan and upload the schedule of one orientation (row pointers ptr, edge
// columns col and caller indices perm in compressed order) for `waves`-wave
// workgroups, with its padded edge slots.
ck_status build_schedule(const std::vector<int32_t>& ptr, int64_t N, const int32_t* col,
                         const int32_t* perm, const int32_t* input_slot, int num_cus, int waves,
                         hipStream_t stream, Schedule* out) {
  static_assert(sizeof(BatchEntry) == sizeof(int4), "batch entries are read as int4");
  SchedulePlan plan;
  plan_schedule(ptr.data(), N, num_cus, waves, &plan);
  const int64_t slots = (int64_t)plan.table.size() * kBatchEdges;
  if (slots > kInt32Limit) {
    set_error("padded edge slots (%lld) overflow 32-bit indexing", (long long)slots);
    return CK_ERR_TOO_LARGE;
  }
  out->num_wgs = plan.num_wgs;
  out->waves = plan.waves;
  out->KB = plan.KB;
  out->slots = slots;
  const size_t bytes = plan.table.size() * sizeof(BatchEntry);
  CK_HIP_TRY(hipMalloc(&out->batches, bytes));
  CK_HIP_TRY(hipMemcpy(out->batches, plan.table.data(), bytes, hipMemcpyHostToDevice));
  CK_HIP_TRY(hipMalloc(&out->pcol, slots * sizeof(int32_t)));
  CK_HIP_TRY(hipMalloc(&out->pperm, slots * sizeof(int32_t)));
  pad_edges<<<grid_for(slots, 256), 256, 0, stream>>>(out->batches, slots, col, perm, out->pcol,
                                                       out->pperm);
  const int64_t entries = (int64_t)plan.table.size();
  entry_input_slots<<<grid_for(entries, 256), 256, 0, stream>>>(out->batches, entries, input_slot);
  CK_HIP_TRY(hipGetLastError());
  return CK_OK;
}

// Records the XCD of each workgroup.
__global__ void xcc_of_workgroups(int32_t* __restrict__ out) {
  if (threadIdx.x == 0) out[blockIdx.x] = (int32_t)xcc_id();
}

// Resident slot q = ((r * D) + j) * kResLanes + l (slot j of lane l on
// workgroup r): its compressed edge slot_edge[q], or an empty slot (node N,
// caller index -1).
__global__ void pad_resident(const int32_t* __restrict__ slot_edge, int64_t slots,
                             const int32_t* __restrict__ col, const int32_t* __restrict__ perm,
                             int32_t N, int32_t* __restrict__ pcol, int32_t* __restrict__ pperm) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= slots) return;
  const int32_t k = slot_edge[q];
  pcol[q] = k >= 0 ? col[k] : N - 1 - k;  // an empty slot reads zero row N + z, k = -1 - z
  pperm[q] = k >= 0 ? perm[k] : -1;
}

// True when a launch of num_cus workgroups puts num_cus / kResXcds of them on
// each of kResXcds XCDs: the grouping the resident kernels rely on (they
// check it again themselves).
bool xcds_as_expected(int num_cus, hipStream_t stream) {
  if (num_cus <= 0 || num_cus % kResXcds != 0) return false;
  int32_t* d = nullptr;
  if (hipMalloc(&d, num_cus * sizeof(int32_t)) != hipSuccess) return false;
  std::vector<int32_t> h(num_cus, -1);
  xcc_of_workgroups<<<num_cus, 64, 0, stream>>>(d);
  bool ok = hipGetLastError() == hipSuccess &&
            hipMemcpyAsync(h.data(), d, num_cus * sizeof(int32_t), hipMemcpyDeviceToHost,
                           stream) == hipSuccess &&
            hipStreamSynchronize(stream) == hipSuccess;
  (void)hipFree(d);
  std::vector<int> per(kResXcds, 0);
  for (int b = 0; ok && b < num_cus; ++b) {
    ok = h[b] >= 0 && h[b] < kResXcds;
    if (ok) ++per[h[b]];
  }
  for (int x = 0; ok && x < kResXcds; ++x) ok = per[x] == num_cus / kResXcds;
  return ok;
}

ck_status build_resident(const std::vector<int32_t>& ptr, int64_t N, const int32_t* col,
                         const int32_t* perm, int ranks, int max_D, bool every_wave_gathers,
                         hipStream_t stream, Resident* out, bool* planned) {
  ResidentPlan plan;
  *planned = plan_resident(ptr.data(), N, ranks, max_D, every_wave_gathers, &plan);
  if (!*planned) return CK_OK;
  {
    // order each piece's edges against LDS bank conflicts (needs the rows read)
    std::vector<int32_t> hcol(std::max<int32_t>(ptr[N], 1));
    if (ptr[N] > 0) {
      CK_HIP_TRY(hipMemcpyAsync(hcol.data(), col, (size_t)ptr[N] * sizeof(int32_t),
                                hipMemcpyDeviceToHost, stream));
      CK_HIP_TRY(hipStreamSynchronize(stream));
    }
    order_resident_slots(hcol.data(), N, &plan);
  }
  out->D = plan.D;
  out->ranks = plan.ranks;
  out->slots = (int64_t)plan.ranks * plan.D * kResLanes;
  auto upload = [&](int32_t** dst, const std::vector<int32_t>& src) -> hipError_t {
    hipError_t e = hipMalloc(dst, src.size() * sizeof(int32_t));
    if (e == hipSuccess)
      e = hipMemcpy(*dst, src.data(), src.size() * sizeof(int32_t), hipMemcpyHostToDevice);
    return e;
  };
  CK_HIP_TRY(upload(&out->rank_rows, plan.rank_rows));
  CK_HIP_TRY(upload(&out->owner_pbeg, plan.owner_pbeg));
  CK_HIP_TRY(upload(&out->piece_row, plan.piece_row));
  int32_t* slot_edge = nullptr;
  hipError_t e = upload(&slot_edge, plan.slot_edge);
  if (e == hipSuccess) e = hipMalloc(&out->pcol, out->slots * sizeof(int32_t));
  if (e == hipSuccess) e = hipMalloc(&out->pperm, out->slots * sizeof(int32_t));
  if (e == hipSuccess) {
    pad_resident<<<grid_for(out->slots, 256), 256, 0, stream>>>(
        slot_edge, out->slots, col, perm, (int32_t)N, out->pcol, out->pperm);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  (void)hipFree(slot_edge);
  CK_HIP_TRY(e);
  return CK_OK;
}

void free_resident(Resident* r) {
  (void)hipFree(r->rank_rows);
  (void)hipFree(r->owner_pbeg);
  (void)hipFree(r->piece_row);
  (void)hipFree(r->pcol);
  (void)hipFree(r->pperm);
  *r = Resident();
}

void free_graph_arrays(ck_graph* g) {
  int32_t* arrs[] = {g->row_ptr, g->col_idx, g->perm, g->t_row_ptr, g->t_col_idx, g->t_perm,
                     g->input_slot};
  for (int32_t* p : arrs) (void)hipFree(p);
  for (int k = 0; k < 2; ++k)
    for (Schedule* sc : {&g->fwd[k], &g->bwd[k]}) {
      (void)hipFree(sc->batches);
      (void)hipFree(sc->pcol);
      (void)hipFree(sc->pperm);
    }
  free_resident(&g->res_fwd);
  free_resident(&g->res_bwd);
  free_blocked(&g->blk_fwd);
  free_blocked(&g->blk_bwd);
}

}  // namespace
}  // namespace ckhip

using namespace ckhip;

extern "C" ck_status ck_graph_create(const int64_t* src, const int64_t* dst, int64_t num_edges,
                                     int64_t num_nodes, const int64_t* input_nodes,
                                     int64_t num_inputs, hipStream_t stream, ck_graph_t* out) {
  clear_error();
  if (out == nullptr) {
    set_error("out handle pointer is NULL");
    return CK_ERR_NULL_ARG;
  }
  *out = nullptr;
  const int64_t N = num_nodes, E = num_edges, n_in = num_inputs;
  if (N <= 0 || E < 0 || n_in < 0) {
    set_error("bad sizes: num_nodes=%lld num_edges=%lld num_inputs=%lld", (long long)N,
              (long long)E, (long long)n_in);
    return CK_ERR_BAD_SIZE;
  }
  if (N >= kInt32Limit || E >= kInt32Limit) {
    set_error("num_nodes and num_edges must be below 2^31");
    return CK_ERR_TOO_LARGE;
  }
  if ((E > 0 && (src == nullptr || dst == nullptr)) || (n_in > 0 && input_nodes == nullptr)) {
    set_error("NULL src/dst/input_nodes for a non-empty list");
    return CK_ERR_NULL_ARG;
  }
  ck_graph* g = (ck_graph*)calloc(1, sizeof(ck_graph));
  if (!g) {
    set_error("host allocation failed");
    return CK_ERR_NOMEM;
  }
  g->N = N;
  g->E = E;
  g->n_in = n_in;
  (void)hipGetDevice(&g->device);
  unsigned* flags = nullptr;
  int32_t* seen = nullptr;
  ck_status rc = CK_OK;
  auto fail = [&](ck_status s) {
    (void)hipFree(flags);
    (void)hipFree(seen);
    free_graph_arrays(g);
    free(g);
    return s;
  };
#define CK_GB_TRY(expr)                                                                     \
  do {                                                                                      \
    hipError_t e_ = (expr);                                                                 \
    if (e_ != hipSuccess) {                                                                 \
      set_error("%s failed: %s", #expr, hipGetErrorString(e_));                             \
      return fail(e_ == hipErrorOutOfMemory ? CK_ERR_NOMEM : CK_ERR_HIP);                   \
    }                                                                                       \
  } while (0)
  CK_GB_TRY(hipMalloc(&flags, sizeof(unsigned)));
  CK_GB_TRY(hipMalloc(&seen, N * sizeof(int32_t)));
  fill_i32<<<grid_for(1, 64), 64, 0, stream>>>((int32_t*)flags, 1, 0);
  fill_i32<<<grid_for(N, 256), 256, 0, stream>>>(seen, N, 0);
  if (E > 0) validate_edges<<<grid_for(E, 256), 256, 0, stream>>>(src, dst, E, N, flags);
  if (n_in > 0)
    validate_inputs<<<grid_for(n_in, 256), 256, 0, stream>>>(input_nodes, n_in, N, seen, flags);
  CK_GB_TRY(hipGetLastError());
  unsigned hflags = 0;
  CK_GB_TRY(hipMemcpyAsync(&hflags, flags, sizeof(unsigned), hipMemcpyDeviceToHost, stream));
  CK_GB_TRY(hipStreamSynchronize(stream));
  if (hflags & 1u) {
    set_error("an edge endpoint or input node lies outside [0, %lld)", (long long)N);
    return fail(CK_ERR_INDEX_RANGE);
  }
  if (hflags & 2u) {
    set_error("input_nodes lists a node more than once");
    return fail(CK_ERR_DUP_INPUT);
  }
  const size_t eb = std::max<int64_t>(E, 1) * sizeof(int32_t);
  const size_t nb = (N + 1) * sizeof(int32_t);
  CK_GB_TRY(hipMalloc(&g->row_ptr, nb));
  CK_GB_TRY(hipMalloc(&g->t_row_ptr, nb));
  CK_GB_TRY(hipMalloc(&g->col_idx, eb));
  CK_GB_TRY(hipMalloc(&g->perm, eb));
  CK_GB_TRY(hipMalloc(&g->t_col_idx, eb));
  CK_GB_TRY(hipMalloc(&g->t_perm, eb));
  CK_GB_TRY(hipMalloc(&g->input_slot, N * sizeof(int32_t)));
  rc = build_compressed(dst, src, E, N, g->row_ptr, g->col_idx, g->perm, stream);
  if (rc != CK_OK) return fail(rc);
  rc = build_compressed(src, dst, E, N, g->t_row_ptr, g->t_col_idx, g->t_perm, stream);
  if (rc != CK_OK) return fail(rc);
  fill_i32<<<grid_for(N, 256), 256, 0, stream>>>(g->input_slot, N, -1);
  if (n_in > 0) set_input_slots<<<grid_for(n_in, 256), 256, 0, stream>>>(input_nodes, n_in, g->input_slot);
  CK_GB_TRY(hipGetLastError());
  std::vector<int32_t> hptr(N + 1), htptr(N + 1);
  CK_GB_TRY(hipMemcpyAsync(hptr.data(), g->row_ptr, nb, hipMemcpyDeviceToHost, stream));
  CK_GB_TRY(hipMemcpyAsync(htptr.data(), g->t_row_ptr, nb, hipMemcpyDeviceToHost, stream));
  CK_GB_TRY(hipStreamSynchronize(stream));
  int num_cus = 256;
  {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, g->device) == hipSuccess && prop.multiProcessorCount > 0)
      num_cus = prop.multiProcessorCount;
  }
  for (int k = 0; k < 2; ++k) {
    const int waves = k == 0 ? 8 : 16;
    rc = build_schedule(hptr, N, g->col_idx, g->perm, g->input_slot, num_cus, waves, stream,
                        &g->fwd[k]);
    if (rc != CK_OK) return fail(rc);
    rc = build_schedule(htptr, N, g->t_col_idx, g->t_perm, g->input_slot, num_cus, waves,
                        stream, &g->bwd[k]);
    if (rc != CK_OK) return fail(rc);
  }
  CK_GB_TRY(hipStreamSynchronize(stream));
  // XCD-resident plans (optional: without them every call takes the
  // per-microstep kernels)
  {
    const char* env = getenv("CK_RESIDENT");
    const bool wanted = !(env && env[0] == '0' && env[1] == '\0');
    const char* spin = getenv("CK_RESIDENT_SPIN_LIMIT");
    g->res_spin_limit = spin && spin[0] ? atoi(spin) : (1 << 20);
    // (the resident kernels' progress flags hold at most 32 workgroups per XCD)
    if (wanted && N <= kResMaxN && num_cus <= 32 * kResXcds && xcds_as_expected(num_cus, stream)) {
      const int ranks = num_cus / kResXcds;
      bool pf = false, pb = false;
      // (the forward's waves without pieces skip their gathers; every wave of
      // the backward gathers)
      rc = build_resident(hptr, N, g->col_idx, g->perm, ranks, kResFwdMaxD, false, stream,
                          &g->res_fwd, &pf);
      if (rc != CK_OK) return fail(rc);
      if (pf)
        rc = build_resident(htptr, N, g->t_col_idx, g->t_perm, ranks, kResBwdMaxD, true, stream,
                            &g->res_bwd, &pb);
      if (rc != CK_OK) return fail(rc);
      g->res_ok = pf && pb && res_prepare() == CK_OK ? 1 : 0;
      if (!g->res_ok) {
        free_resident(&g->res_fwd);
        free_resident(&g->res_bwd);
      }
    }
  }
  // blocked plans (optional: for graphs whose state plane dwarfs the L2s)
  {
    const char* env = getenv("CK_BLOCKED");
    const bool set = env && env[0] && env[1] == '\0';
    const bool both = set && env[0] == '2';
    const bool wanted = env && env[0] ? (set && (env[0] == '1' || both)) : N >= kBlkMinN;
    if (wanted) {
      bool pf = false, pb = false;
      rc = build_blocked(hptr, N, g->col_idx, g->perm, num_cus, stream, &g->blk_fwd, &pf);
      if (rc != CK_OK) return fail(rc);
      if (pf && both)
        rc = build_blocked(htptr, N, g->t_col_idx, g->t_perm, num_cus, stream, &g->blk_bwd, &pb);
      if (rc != CK_OK) return fail(rc);
      g->blk_ok = pf ? 1 : 0;
      g->blk_bwd_ok = pf && pb ? 1 : 0;
      if (!g->blk_ok) free_blocked(&g->blk_fwd);
      if (!g->blk_bwd_ok) free_blocked(&g->blk_bwd);
    }
  }
  (void)hipFree(flags);
  (void)hipFree(seen);
  flags = nullptr;
  seen = nullptr;
  rc = scratch_prepare(g->device);
  if (rc != CK_OK) return fail(rc);
  g->magic = kGraphMagic;
  *out = g;
  return CK_OK;
#undef CK_GB_TRY
}

extern "C" ck_status ck_graph_destroy(ck_graph_t g) {
  clear_error();
  if (g == nullptr) return CK_OK;
  ck_status rc = check_graph(g);
  if (rc != CK_OK) return rc;
  (void)hipDeviceSynchronize();
  free_graph_arrays(g);
  g->magic = 0;
  free(g);
  return CK_OK;
}

extern "C" ck_status ck_graph_sizes(ck_graph_t g, int64_t* num_nodes, int64_t* num_edges,
                                    int64_t* num_inputs) {
  clear_error();
  ck_status rc = check_graph(g);
  if (rc != CK_OK) return rc;
  if (num_nodes) *num_nodes = g->N;
  if (num_edges) *num_edges = g->E;
  if (num_inputs) *num_inputs = g->n_in;
  return CK_OK;
}

extern "C" ck_status ck_graph_export(ck_graph_t g, int32_t* row_ptr, int32_t* col_idx,
                                     int32_t* perm, int32_t* t_row_ptr, int32_t* t_col_idx,
                                     int32_t* t_perm, int32_t* input_slot, hipStream_t stream) {
  clear_error();
  ck_status rc = check_graph(g);
  if (rc != CK_OK) return rc;
  const size_t nb = (g->N + 1) * sizeof(int32_t), eb = g->E * sizeof(int32_t);
  struct {
    int32_t* dst;
    const int32_t* src;
    size_t bytes;
  } copies[] = {{row_ptr, g->row_ptr, nb},     {col_idx, g->col_idx, eb},
                {perm, g->perm, eb},           {t_row_ptr, g->t_row_ptr, nb},
                {t_col_idx, g->t_col_idx, eb}, {t_perm, g->t_perm, eb},
                {input_slot, g->input_slot, g->N * sizeof(int32_t)}};
  for (auto& c : copies)
    if (c.dst != nullptr && c.bytes > 0)
      CK_HIP_TRY(hipMemcpyAsync(c.dst, c.src, c.bytes, hipMemcpyDeviceToDevice, stream));
  return CK_OK;
}

extern "C" const char* ck_status_string(ck_status s) {
  switch (s) {
    case CK_OK: return "CK_OK";
    case CK_ERR_NULL_ARG: return "CK_ERR_NULL_ARG";
    case CK_ERR_BAD_SIZE: return "CK_ERR_BAD_SIZE";
    case CK_ERR_INDEX_RANGE: return "CK_ERR_INDEX_RANGE";
    case CK_ERR_DUP_INPUT: return "CK_ERR_DUP_INPUT";
    case CK_ERR_TOO_LARGE: return "CK_ERR_TOO_LARGE";
    case CK_ERR_WORKSPACE: return "CK_ERR_WORKSPACE";
    case CK_ERR_NOMEM: return "CK_ERR_NOMEM";
    case CK_ERR_HIP: return "CK_ERR_HIP";
    case CK_ERR_BAD_HANDLE: return "CK_ERR_BAD_HANDLE";
    case CK_ERR_WAIT: return "CK_ERR_WAIT";
    case CK_ERR_OVERFLOW: return "CK_ERR_OVERFLOW";
    case CK_ERR_BAD_VALUE: return "CK_ERR_BAD_VALUE";
  }
  return "CK_ERR_UNKNOWN";
}

extern "C" const char* ck_last_error(void) { return ckhip::g_last_error; }
