/*
 * lif_oracle.c -- plain, slow CPU oracle of the deterministic fixed-point
 * leaky integrate-and-fire (LIF) forward on a fixed sparse directed graph.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file: only the test suite and the benchmark's CPU baseline use it.  It
 * shares no code, header, table or constant with the HIP library.
 *
 * What it computes (soup-connectome page, "Runtime contract": signed int32
 * membrane potentials, signed int16 synaptic impulses, positive integer
 * timestep delays, checked arithmetic with rejected overflow, the
 * arithmetic-shift leak V := V - (V >> k); "Full-scale benchmark": the run
 * parameters threshold, reset, decay_shifts, refractory_steps).  The page fixes
 * the representation, not the order of the update; the readings taken here:
 *
 *   state: V[i] (int32), refractory count r[i] (>= 0), and a delay line of
 *   impulses in flight.  V starts at v0, r at 0, the delay line empty.
 *   for every timestep t = 0..T-1, for every neuron i:
 *     I = the sum of the impulses that arrive at i at step t (exact, int64)
 *     if r[i] > 0:   r[i] -= 1; the arriving impulses are dropped; V[i] is
 *                    kept; no spike
 *     else:          for each k in decay_shifts, in order: V := V - floor(V / 2^k)
 *                    V := V + I, rejected (the run fails at step t) if the
 *                    result leaves the int32 range
 *                    if V >= threshold: spike; V := reset; r[i] := refractory_steps
 *     spikes[t][i] = spike ? 1 : 0, potentials[t][i] = V[i]
 *   then every edge e (src[e] -> dst[e], impulse w[e], delay d[e] >= 1) whose
 *   source spiked at step t puts w[e] in flight to dst[e], arriving at step
 *   t + d[e].
 *
 * The delay line is a ring of max_delay + 1 slots of N int64 accumulators
 * (slot (t mod (max_delay + 1)) holds what arrives at step t); edges are
 * visited in the caller's order.  Integer sums are exact, so any correct
 * implementation -- in particular one that gathers, for every neuron and
 * step, the impulses of the in-edges whose source spiked d steps earlier --
 * gives bit-identical spikes and potentials.
 */
#include <stdint.h>
#include <stdlib.h>

enum {
  LOR_OK = 0,
  LOR_ERR_NULL_ARG = 1,
  LOR_ERR_BAD_SIZE = 2,
  LOR_ERR_INDEX_RANGE = 3,
  LOR_ERR_NOMEM = 7,
  LOR_ERR_OVERFLOW = 11,
  LOR_ERR_BAD_VALUE = 12
};

/* floor(v / 2^k) for 0 <= k <= 31, written out with an int64 division
 * (C's division truncates toward zero; floor differs for negative v with a
 * non-zero remainder). */
static int64_t lor_floor_shift(int64_t v, int k) {
  const int64_t d = (int64_t)1 << k;
  int64_t q = v / d;
  if (v % d != 0 && v < 0) q -= 1;
  return q;
}

int lifor_run(int64_t N, int64_t E, const int64_t* src, const int64_t* dst, const int16_t* w,
              const int32_t* delay, int32_t threshold, int32_t reset, int32_t refractory_steps,
              int32_t num_shifts, const int32_t* shifts, const int32_t* v0, int64_t T,
              uint8_t* spikes, int32_t* potentials, int64_t* overflow_step) {
  if (N <= 0 || E < 0 || T <= 0) return LOR_ERR_BAD_SIZE;
  if ((E > 0 && (!src || !dst || !w || !delay)) || !v0 || !spikes || !potentials ||
      (num_shifts > 0 && !shifts))
    return LOR_ERR_NULL_ARG;
  if (num_shifts < 0 || num_shifts > 8 || refractory_steps < 0) return LOR_ERR_BAD_VALUE;
  for (int32_t j = 0; j < num_shifts; ++j)
    if (shifts[j] < 0 || shifts[j] > 31) return LOR_ERR_BAD_VALUE;
  int64_t max_delay = 1;
  for (int64_t e = 0; e < E; ++e) {
    if (src[e] < 0 || src[e] >= N || dst[e] < 0 || dst[e] >= N) return LOR_ERR_INDEX_RANGE;
    if (delay[e] < 1 || delay[e] > 32767) return LOR_ERR_BAD_VALUE;
    if (delay[e] > max_delay) max_delay = delay[e];
  }
  const int64_t H = max_delay + 1;
  int32_t* V = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
  int32_t* r = (int32_t*)calloc((size_t)N, sizeof(int32_t));
  int64_t* line = (int64_t*)calloc((size_t)(H * N), sizeof(int64_t));
  if (!V || !r || !line) {
    free(V); free(r); free(line);
    return LOR_ERR_NOMEM;
  }
  for (int64_t i = 0; i < N; ++i) V[i] = v0[i];
  if (overflow_step) *overflow_step = -1;
  int rc = LOR_OK;
  for (int64_t t = 0; t < T && rc == LOR_OK; ++t) {
    int64_t* arriving = line + (t % H) * N;
    uint8_t* s = spikes + t * N;
    for (int64_t i = 0; i < N; ++i) {
      const int64_t in = arriving[i];
      arriving[i] = 0;
      s[i] = 0;
      if (r[i] > 0) {
        r[i] -= 1;
      } else {
        int64_t v = V[i];
        for (int32_t j = 0; j < num_shifts; ++j) v = v - lor_floor_shift(v, shifts[j]);
        v += in;
        if (v < INT32_MIN || v > INT32_MAX) {
          if (overflow_step) *overflow_step = t;
          rc = LOR_ERR_OVERFLOW;
          break;
        }
        if (v >= threshold) {
          s[i] = 1;
          v = reset;
          r[i] = refractory_steps;
        }
        V[i] = (int32_t)v;
      }
      potentials[t * N + i] = V[i];
    }
    if (rc != LOR_OK) break;
    for (int64_t e = 0; e < E; ++e)
      if (s[src[e]]) line[((t + delay[e]) % H) * N + dst[e]] += w[e];
  }
  free(V); free(r); free(line);
  return rc;
}
