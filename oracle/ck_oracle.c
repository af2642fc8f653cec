/*
 * ck_oracle.c -- plain, slow, fp64 CPU oracle of the leaky-tanh recurrence on a
 * fixed sparse directed graph and of its reverse-mode gradient.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file: only the test suite, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant with the
 * HIP library; the two meet only through the seeded input generators.
 *
 * What it computes (connectome-kernels README, introduction, the two update
 * equations and the paragraph after them; "Use" section for the shapes):
 *
 *   for every input step t = 0..T-1 and microstep m = 0..M-1 (s = t*M + m + 1):
 *     a^(s)_{b,i} = sum_{e : dst[e] = i} v[e] * h^(s-1)_{b,src[e]}
 *                   + (i is input node k ? drives[t][k][b] : 0) + bias[i]
 *     h^(s)_{b,i} = (1 - leak[i]) * h^(s-1)_{b,i} + leak[i] * tanh(a^(s)_{b,i})
 *   h^(0) = state0 ([B][N]),  out[t] = h^((t+1)M)  ([T][B][N]).
 *
 * Every node reads the previous microstep's state (synchronous update), the
 * drive of step t is held for all M microsteps, and an edge e adds v[e] to
 * W[dst[e]][src[e]] (a signal flows from src into dst; "Use" section).
 *
 * The gradient is that of the scalar L = sum(out * G) for a caller-supplied G,
 * derived by hand by reverse-mode differentiation of the two equations above:
 *
 *   g = 0;  for s = S..1 (t = (s-1)/M):
 *     if s % M == 0:  g += G[t]
 *     p = tanh(a^(s)),  q = h^(s-1)
 *     g_leak[i]      += sum_b g * (p - q)
 *     ga              = g * leak * sech^2(a^(s))
 *     g_bias[i]      += sum_b ga
 *     g_drives[t][k] += ga[input_nodes[k]]
 *     g_v[e]         += sum_b ga[dst[e]] * q[src[e]]
 *     g              <- (1 - leak) * g + W^T ga
 *   g_state0 = g.
 *
 * All sums are formed sequentially inside the single thread that owns the
 * result (a batch column, a node, an input slot or an edge), so results do not
 * depend on the OpenMP thread count.  Inputs arrive as fp64; the fp32 values
 * the GPU sees convert to fp64 exactly.
 *
 * The working precision is `real`: double by default.  Built with
 * -DOR_REAL=float the same code evaluates every step in fp32 (inputs rounded
 * to fp32); that build measures the fp32 rounding floor of the method (the
 * parity tests fall back to it only where an element misses the stated bound
 * against the fp64 build).
 *
 * The graph builder orders edges by (dst, src, caller index) for the CSR and by
 * (src, dst, caller index) for the transposed CSR; both are total orders, so the
 * arrays are unique and any correct builder must reproduce them bit for bit.
 */
#include <stdint.h>
#include <tgmath.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Status values: the library's documented error convention, restated here. */
enum {
  OR_OK = 0,
  OR_ERR_NULL_ARG = 1,
  OR_ERR_BAD_SIZE = 2,
  OR_ERR_INDEX_RANGE = 3,
  OR_ERR_DUP_INPUT = 4,
  OR_ERR_TOO_LARGE = 5,
  OR_ERR_NOMEM = 7
};

#ifndef OR_REAL
#define OR_REAL double
#endif
typedef OR_REAL real;

static const int64_t OR_INT32_LIMIT = 2147483647LL; /* sizes must stay below 2^31 */

/* Validation of a graph description, checks taken in a fixed order:
 * sizes, null pointers, edge index range, input index range, duplicate inputs. */
int ckor_validate(int64_t N, int64_t E, const int64_t* src, const int64_t* dst,
                  int64_t n_in, const int64_t* inputs) {
  if (N <= 0 || E < 0 || n_in < 0) return OR_ERR_BAD_SIZE;
  if (N >= OR_INT32_LIMIT || E >= OR_INT32_LIMIT) return OR_ERR_TOO_LARGE;
  if (E > 0 && (src == NULL || dst == NULL)) return OR_ERR_NULL_ARG;
  if (n_in > 0 && inputs == NULL) return OR_ERR_NULL_ARG;
  for (int64_t e = 0; e < E; ++e)
    if (src[e] < 0 || src[e] >= N || dst[e] < 0 || dst[e] >= N) return OR_ERR_INDEX_RANGE;
  for (int64_t k = 0; k < n_in; ++k)
    if (inputs[k] < 0 || inputs[k] >= N) return OR_ERR_INDEX_RANGE;
  char* seen = (char*)calloc((size_t)N, 1);
  if (!seen) return OR_ERR_NOMEM;
  int rc = OR_OK;
  for (int64_t k = 0; k < n_in && rc == OR_OK; ++k) {
    if (seen[inputs[k]]) rc = OR_ERR_DUP_INPUT;
    seen[inputs[k]] = 1;
  }
  free(seen);
  return rc;
}

typedef struct {
  int64_t major, minor, e;
} or_edge_key;

static int or_key_cmp(const void* pa, const void* pb) {
  const or_edge_key* a = (const or_edge_key*)pa;
  const or_edge_key* b = (const or_edge_key*)pb;
  if (a->major != b->major) return a->major < b->major ? -1 : 1;
  if (a->minor != b->minor) return a->minor < b->minor ? -1 : 1;
  if (a->e != b->e) return a->e < b->e ? -1 : 1;
  return 0;
}

/* One compressed-row structure: rows keyed by `major`, ordered inside a row by
 * (minor, caller index).  ptr[N+1], idx[E] = minor, prm[E] = caller index. */
static int or_compress(int64_t N, int64_t E, const int64_t* major, const int64_t* minor,
                       int32_t* ptr, int32_t* idx, int32_t* prm) {
  or_edge_key* keys = (or_edge_key*)malloc(sizeof(or_edge_key) * (size_t)(E > 0 ? E : 1));
  if (!keys) return OR_ERR_NOMEM;
  for (int64_t e = 0; e < E; ++e) {
    keys[e].major = major[e];
    keys[e].minor = minor[e];
    keys[e].e = e;
  }
  qsort(keys, (size_t)E, sizeof(or_edge_key), or_key_cmp);
  for (int64_t i = 0; i <= N; ++i) ptr[i] = 0;
  for (int64_t e = 0; e < E; ++e) ptr[keys[e].major + 1] += 1;
  for (int64_t i = 0; i < N; ++i) ptr[i + 1] += ptr[i];
  for (int64_t k = 0; k < E; ++k) {
    idx[k] = (int32_t)keys[k].minor;
    prm[k] = (int32_t)keys[k].e;
  }
  free(keys);
  return OR_OK;
}

/* Graph build: CSR by destination, transposed CSR by source, input slot map. */
int ckor_build(int64_t N, int64_t E, const int64_t* src, const int64_t* dst, int64_t n_in,
               const int64_t* inputs, int32_t* row_ptr, int32_t* col_idx, int32_t* perm,
               int32_t* t_row_ptr, int32_t* t_col_idx, int32_t* t_perm, int32_t* input_slot) {
  int rc = ckor_validate(N, E, src, dst, n_in, inputs);
  if (rc != OR_OK) return rc;
  rc = or_compress(N, E, dst, src, row_ptr, col_idx, perm);
  if (rc != OR_OK) return rc;
  rc = or_compress(N, E, src, dst, t_row_ptr, t_col_idx, t_perm);
  if (rc != OR_OK) return rc;
  for (int64_t i = 0; i < N; ++i) input_slot[i] = -1;
  for (int64_t k = 0; k < n_in; ++k) input_slot[inputs[k]] = (int32_t)k;
  return OR_OK;
}

/* sech^2(x) = 1 / cosh^2(x); cosh overflows to +inf for large |x| and the
 * result then correctly becomes 0. */
static real or_sech2(real x) {
  real c = cosh(x);
  return (real)1 / (c * c);
}

/*
 * Forward over the whole window and, when G is not NULL, the gradient of
 * L = sum(out * G) with respect to all five inputs.
 *
 * Layouts (all row-major, caller edge order for edge arrays):
 *   v[E], leak[N], bias[N], drives[T][n_in][B], state0[B][N], G[T][B][N]
 *   out[T][B][N], g_v[E], g_leak[N], g_bias[N], g_drives[T][n_in][B], g_state0[B][N]
 * Gradient outputs are overwritten.  nthreads <= 0 uses the OpenMP default.
 */
int ckor_run(int64_t N, int64_t E, const int64_t* src, const int64_t* dst, int64_t n_in,
             const int64_t* inputs, const double* v_in, const double* leak_in,
             const double* bias_in, const double* drives_in, const double* state0, int64_t T,
             int64_t B, int64_t M, const double* G_in, double* out, double* g_v, double* g_leak,
             double* g_bias, double* g_drives, double* g_state0, int nthreads) {
  int rc = ckor_validate(N, E, src, dst, n_in, inputs);
  if (rc != OR_OK) return rc;
  if (T <= 0 || B <= 0 || M <= 0) return OR_ERR_BAD_SIZE;
  if (!leak_in || !bias_in || !state0 || !out || (E > 0 && !v_in) || (n_in > 0 && !drives_in))
    return OR_ERR_NULL_ARG;
  if (G_in && (!g_leak || !g_bias || !g_state0 || (E > 0 && !g_v) || (n_in > 0 && !g_drives)))
    return OR_ERR_NULL_ARG;
#ifdef _OPENMP
  int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
  int nt = 1;
  (void)nthreads;
#endif
  const int64_t S = T * M;
  const int64_t BN = B * N;
  const int64_t ND = T * n_in * B;
  int64_t* slot = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
  real* v = (real*)malloc(sizeof(real) * (size_t)(E > 0 ? E : 1));
  real* leak = (real*)malloc(sizeof(real) * (size_t)N);
  real* bias = (real*)malloc(sizeof(real) * (size_t)N);
  real* drives = (real*)malloc(sizeof(real) * (size_t)(ND > 0 ? ND : 1));
  real* hs = (real*)malloc(sizeof(real) * (size_t)((S + 1) * BN)); /* h^(0..S) */
  real* as = (real*)malloc(sizeof(real) * (size_t)(S * BN));       /* a^(1..S) */
  if (!slot || !v || !leak || !bias || !drives || !hs || !as) {
    free(slot); free(v); free(leak); free(bias); free(drives); free(hs); free(as);
    return OR_ERR_NOMEM;
  }
  for (int64_t e = 0; e < E; ++e) v[e] = (real)v_in[e];
  for (int64_t i = 0; i < N; ++i) {
    leak[i] = (real)leak_in[i];
    bias[i] = (real)bias_in[i];
    slot[i] = -1;
  }
  for (int64_t x = 0; x < ND; ++x) drives[x] = (real)drives_in[x];
  for (int64_t k = 0; k < n_in; ++k) slot[inputs[k]] = k;
  for (int64_t x = 0; x < BN; ++x) hs[x] = (real)state0[x];

  /* ---- forward ---- */
  for (int64_t s = 1; s <= S; ++s) {
    const int64_t t = (s - 1) / M;
    const real* hp = hs + (s - 1) * BN;
    real* hn = hs + s * BN;
    real* a = as + (s - 1) * BN;
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t b = 0; b < B; ++b) {
      real* acc = a + b * N;
      const real* hb = hp + b * N;
      for (int64_t i = 0; i < N; ++i) acc[i] = 0;
      for (int64_t e = 0; e < E; ++e) acc[dst[e]] += v[e] * hb[src[e]];
      for (int64_t i = 0; i < N; ++i) {
        real drive = slot[i] >= 0 ? drives[(t * n_in + slot[i]) * B + b] : (real)0;
        real x = acc[i] + drive + bias[i];
        acc[i] = x;
        hn[b * N + i] = ((real)1 - leak[i]) * hb[i] + leak[i] * tanh(x);
      }
    }
    if (s % M == 0)
      for (int64_t x = 0; x < BN; ++x) out[t * BN + x] = (double)hn[x];
  }

  if (G_in) {
    /* ---- backward ---- */
    real* g = (real*)calloc((size_t)BN, sizeof(real));
    real* gn = (real*)malloc(sizeof(real) * (size_t)BN);
    real* ga = (real*)malloc(sizeof(real) * (size_t)BN);
    real* gv = (real*)calloc((size_t)(E > 0 ? E : 1), sizeof(real));
    real* gl_ = (real*)calloc((size_t)N, sizeof(real));
    real* gb_ = (real*)calloc((size_t)N, sizeof(real));
    real* gd = (real*)calloc((size_t)(ND > 0 ? ND : 1), sizeof(real));
    if (!g || !gn || !ga || !gv || !gl_ || !gb_ || !gd) {
      free(g); free(gn); free(ga); free(gv); free(gl_); free(gb_); free(gd);
      free(slot); free(v); free(leak); free(bias); free(drives); free(hs); free(as);
      return OR_ERR_NOMEM;
    }
    for (int64_t s = S; s >= 1; --s) {
      const int64_t t = (s - 1) / M;
      const real* q = hs + (s - 1) * BN;
      const real* a = as + (s - 1) * BN;
      if (s % M == 0)
        for (int64_t x = 0; x < BN; ++x) g[x] += (real)G_in[t * BN + x];
#pragma omp parallel for num_threads(nt) schedule(static)
      for (int64_t i = 0; i < N; ++i) {
        real gl = 0, gb = 0;
        for (int64_t b = 0; b < B; ++b) {
          const int64_t x = b * N + i;
          const real p = tanh(a[x]);
          gl += g[x] * (p - q[x]);
          ga[x] = g[x] * leak[i] * or_sech2(a[x]);
          gb += ga[x];
        }
        gl_[i] += gl;
        gb_[i] += gb;
      }
#pragma omp parallel for num_threads(nt) schedule(static)
      for (int64_t k = 0; k < n_in; ++k)
        for (int64_t b = 0; b < B; ++b) gd[(t * n_in + k) * B + b] += ga[b * N + inputs[k]];
#pragma omp parallel for num_threads(nt) schedule(static)
      for (int64_t e = 0; e < E; ++e) {
        real d = 0;
        for (int64_t b = 0; b < B; ++b) d += ga[b * N + dst[e]] * q[b * N + src[e]];
        gv[e] += d;
      }
#pragma omp parallel for num_threads(nt) schedule(static)
      for (int64_t b = 0; b < B; ++b) {
        real* gnb = gn + b * N;
        const real* gb_row = g + b * N;
        const real* gab = ga + b * N;
        for (int64_t j = 0; j < N; ++j) gnb[j] = ((real)1 - leak[j]) * gb_row[j];
        for (int64_t e = 0; e < E; ++e) gnb[src[e]] += v[e] * gab[dst[e]];
      }
      real* tmp = g;
      g = gn;
      gn = tmp;
    }
    for (int64_t e = 0; e < E; ++e) g_v[e] = (double)gv[e];
    for (int64_t i = 0; i < N; ++i) {
      g_leak[i] = (double)gl_[i];
      g_bias[i] = (double)gb_[i];
    }
    for (int64_t x = 0; x < ND; ++x) g_drives[x] = (double)gd[x];
    for (int64_t x = 0; x < BN; ++x) g_state0[x] = (double)g[x];
    free(g); free(gn); free(ga); free(gv); free(gl_); free(gb_); free(gd);
  }
  free(slot); free(v); free(leak); free(bias); free(drives); free(hs); free(as);
  return OR_OK;
}
