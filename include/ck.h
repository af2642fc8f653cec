/*
 * ck.h -- C ABI of the MI355X (gfx950) leaky-tanh sparse-graph recurrence library.
 *
 * The method (connectome-kernels README, introduction): every node i of a fixed
 * sparse directed graph carries one scalar state per batch column and every
 * edge one trainable scalar value.  For each input step t = 0..T-1 the update
 *
 *     proposal_i = tanh( sum_j W_ij h_j + drive_i + bias_i )
 *     h_i       <- (1 - leak_i) h_i + leak_i * proposal_i
 *
 * is applied `microsteps` (M) times, every node reading the previous
 * microstep's states.  An edge e (src[e] -> dst[e]) contributes its value to
 * W[dst[e]][src[e]]; parallel edges add and self-loops are allowed.  drives
 * enter only at the designated input nodes and are held for all M microsteps
 * of a step.  out[t] is the state after the last microstep of step t.  The
 * gradient (all five inputs: edge values, leak, bias, drives, initial state)
 * is that of a scalar loss given its upstream gradient grad_out = dL/dout.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is caller-owned device memory (hipMalloc'ed or
 *     torch CUDA storage), contiguous, fp32 for values and int64 for indices.
 *     A NULL pointer is accepted only for a tensor of zero elements.
 *   - The `saved` and `workspace` buffers must start on a 256-byte boundary
 *     (hipMalloc and torch allocations do); otherwise CK_ERR_BAD_VALUE.
 *   - Errors are returned as ck_status; no exception crosses the ABI.
 *     ck_last_error() gives a thread-local detail string of the last failure.
 *   - Forward and backward are asynchronous on `stream` and validate only
 *     scalars and pointers on the host.  NaN/Inf inputs are not checked; they
 *     propagate.
 *   - Sizes: num_nodes and num_edges must be below 2^31, and num_nodes times
 *     the padded batch width (B rounded up to a multiple of 4) must be below
 *     2^30 (one state plane under 4 GiB); otherwise CK_ERR_TOO_LARGE.
 *   - A graph handle is immutable after creation.  On the per-microstep and
 *     blocked paths (ck_recurrence_path) it may be used from several streams at once
 *     provided each call has its own `saved` and `workspace`.  An XCD-resident
 *     call occupies every compute unit and its workgroups wait for one
 *     another: issue resident calls on one stream, with no other device work
 *     running beside them (a call that cannot finish its waits sets its
 *     outputs to NaN and ck_recurrence_status reports CK_ERR_WAIT).
 *   - Calls that share a `saved` or `workspace` buffer must be ordered on one
 *     stream (or otherwise synchronised) by the caller.
 */
#ifndef CK_H
#define CK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ck_graph* ck_graph_t;

typedef enum {
  CK_OK = 0,
  CK_ERR_NULL_ARG = 1,    /* NULL pointer for a non-empty tensor or an output handle */
  CK_ERR_BAD_SIZE = 2,    /* num_nodes <= 0, negative counts, T/B/microsteps <= 0 */
  CK_ERR_INDEX_RANGE = 3, /* src/dst/input_nodes outside [0, num_nodes) */
  CK_ERR_DUP_INPUT = 4,   /* the same node listed twice in input_nodes */
  CK_ERR_TOO_LARGE = 5,   /* a size that would overflow 32-bit indexing */
  CK_ERR_WORKSPACE = 6,   /* workspace_bytes below what ck_recurrence_sizes reports */
  CK_ERR_NOMEM = 7,       /* device or host allocation failed */
  CK_ERR_HIP = 8,         /* a HIP runtime call failed; see ck_last_error() */
  CK_ERR_BAD_HANDLE = 9,  /* NULL or destroyed graph handle */
  CK_ERR_WAIT = 10,       /* a wait inside an XCD-resident kernel gave up (ck_recurrence_status) */
  CK_ERR_OVERFLOW = 11,   /* LIF forward: a membrane potential left the int32 range (run rejected) */
  CK_ERR_BAD_VALUE = 12   /* a parameter or per-edge value outside its documented range */
} ck_status;

/*
 * Build the graph structures on the device (connectome-kernels README, "Use":
 * any directed graph as int64 src/dst lists plus num_nodes and input_nodes;
 * "Design notes": the transposed CSR used by the backward).
 *
 *   src, dst     int64[num_edges] device, caller edge order (edge e: src[e] -> dst[e])
 *   input_nodes  int64[num_inputs] device; node input_nodes[k] receives drives[t][k][:]
 *   stream       HIP stream the build runs on; the call synchronises it
 *   out          receives the new handle (owned by the caller; free with ck_graph_destroy)
 *
 * Internally: the CSR by destination (rows ordered by (src, caller index)),
 * the transposed CSR by source (rows ordered by (dst, caller index)), both
 * edge permutations, the input-slot map and the degree-balanced row schedules.
 * When the device deals a launch's workgroups evenly over 8 XCDs, num_nodes
 * is at most 9184 and the environment variable CK_RESIDENT is not "0" at
 * creation, it also plans the XCD-resident kernels (see
 * ck_recurrence_path), which run a whole forward or backward in one launch.
 * When the device's compute units are a multiple of 8 and num_nodes is at
 * least 100000 (or the environment variable CK_BLOCKED is "1" at creation;
 * "0" turns this off), it plans the blocked forward kernels; with CK_BLOCKED
 * "2" it plans the blocked kernels of both directions (ck_recurrence_path).
 * The caller's edge order is kept for edge values and their gradient: the
 * permutation is invisible outside.  Validation failures return
 * CK_ERR_BAD_SIZE, CK_ERR_TOO_LARGE, CK_ERR_NULL_ARG, CK_ERR_INDEX_RANGE or
 * CK_ERR_DUP_INPUT, checked in that order.
 */
ck_status ck_graph_create(const int64_t* src, const int64_t* dst, int64_t num_edges,
                          int64_t num_nodes, const int64_t* input_nodes, int64_t num_inputs,
                          hipStream_t stream, ck_graph_t* out);

/* Release a handle and its device arrays (synchronises the device).  NULL is accepted. */
ck_status ck_graph_destroy(ck_graph_t g);

/* Sizes the graph was created with (any output pointer may be NULL). */
ck_status ck_graph_sizes(ck_graph_t g, int64_t* num_nodes, int64_t* num_edges,
                         int64_t* num_inputs);

/*
 * Copy the internal graph arrays into caller device buffers (int32):
 *   row_ptr[N+1], col_idx[E] (= src), perm[E] (= caller edge index)      CSR by dst
 *   t_row_ptr[N+1], t_col_idx[E] (= dst), t_perm[E]                      CSR by src
 *   input_slot[N] (k if node is input_nodes[k], else -1)
 * Any pointer may be NULL to skip that array.  Asynchronous on `stream`.
 */
ck_status ck_graph_export(ck_graph_t g, int32_t* row_ptr, int32_t* col_idx, int32_t* perm,
                          int32_t* t_row_ptr, int32_t* t_col_idx, int32_t* t_perm,
                          int32_t* input_slot, hipStream_t stream);

/*
 * Buffer sizes for a window of T input steps, batch B and `microsteps` M.
 *   saved_bytes      the saved-activation arena written by forward and read by
 *                    backward: the state and the pre-activation after every
 *                    microstep (connectome-kernels README, "Design notes"),
 *                    2 * T * M * N * Bp * 4 bytes with Bp = B rounded up to a
 *                    multiple of 4 (= 2*T*M*N*B*4 when B % 4 == 0); on the
 *                    XCD-resident path N is first rounded up to a multiple of
 *                    8 and 256 bytes follow (the forward's status word).  Its
 *                    layout is internal.
 *   workspace_bytes  scratch needed by either forward or backward.
 */
ck_status ck_recurrence_sizes(ck_graph_t g, int64_t T, int64_t B, int64_t microsteps,
                              size_t* saved_bytes, size_t* workspace_bytes);

/*
 * Which kernels a call with batch B runs on this graph: *path = 1 for the
 * XCD-resident kernels, 2 for the blocked forward (with the per-microstep
 * backward), 3 for the blocked kernels in both directions, 0 for the
 * per-microstep kernels.  The resident kernels are taken whenever the graph
 * has their plans; else the blocked kernels when the graph has theirs and
 * 5 <= B <= 64.
 *
 * Per-microstep kernels: one fused launch per microstep and direction, the
 * rows of all batch columns spread over every compute unit.
 * XCD-resident kernels (graphs planned for them at creation): one launch per
 * call.  Batch column group c (4 columns) is computed by the compute units of
 * XCD c mod 8 alone (an XCD with several groups computes them in turn), which
 * keep its whole state plane in LDS and
 * their share of the edges in registers, and exchange each microstep's new
 * state through their shared L2 behind a barrier local to the XCD.  Such a
 * launch holds one workgroup on every compute unit and its workgroups wait
 * for one another, so it must not run concurrently with other kernels on the
 * device.  A wait that does not end within about a second raises an internal
 * error flag; the call's outputs (or all five gradients) are then NaN, a
 * backward given the saved arena of such a forward also writes NaN, and
 * ck_recurrence_status reports CK_ERR_WAIT.  (The
 * poll limit of those waits is read from CK_RESIDENT_SPIN_LIMIT at graph
 * creation, default 1048576; a negative value fails every wait at once and
 * exists to test that failure path.)
 * Blocked kernels (graphs of at least 100000 nodes, or CK_BLOCKED set to
 * "1" at creation; 5 <= B <= 64; *path 2): the forward runs two launches per
 * microstep and the backward the per-microstep kernels; with CK_BLOCKED "2"
 * at creation (*path 3) the backward is blocked as well.  The nodes
 * whose rows are gathered are cut into 8 contiguous blocks, one per XCD, so
 * each XCD gathers from a slice of the state plane that stays in its own L2;
 * each row's edges into a block (at most 64 per work item) leave one partial
 * row, and a second launch adds each row's partials in a fixed order and runs
 * the elementwise update.
 * All paths compute the same sums; results agree to rounding.
 */
ck_status ck_recurrence_path(ck_graph_t g, int64_t B, int* path);

/*
 * Forward over the whole window (connectome-kernels README, introduction and
 * "Use"): one fused launch per microstep, or one launch on the XCD-resident
 * path (ck_recurrence_path).
 *
 *   edge_values  fp32[E]           caller edge order
 *   leak, bias   fp32[N]
 *   drives       fp32[T][n_in][B]
 *   state0       fp32[B][N]
 *   out          fp32[T][B][N]     written: the state after each input step
 *   saved        saved_bytes       written; must be kept for backward
 *   workspace    workspace_bytes   scratch, contents undefined afterwards
 */
ck_status ck_recurrence_forward(ck_graph_t g, const float* edge_values, const float* leak,
                                const float* bias, const float* drives, const float* state0,
                                int64_t T, int64_t B, int64_t microsteps, float* out,
                                void* saved, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * Allocation-free variant of ck_recurrence_forward, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): same arguments without the workspace, same
 * kernels and the same results.  Its scratch (the packed edge slots, the
 * initial state in the kernels' layout and, on the XCD-resident path, the
 * control block) lives in a fixed device array of 64 MiB that the library
 * holds on every GPU it runs on until the process ends; its device address is
 * resolved when a graph is created on that GPU.  The call allocates nothing,
 * records no profiling events and returns CK_ERR_TOO_LARGE when the forward
 * needs more than 64 MiB of scratch (e.g. graphs of tens of millions of
 * edges).  Every call on one GPU shares that array and leaves its contents
 * behind (each call rewrites what it reads): calls that overlap in time on
 * one GPU race and must be ordered by the caller (one stream).  `saved` is
 * the caller's, as for ck_recurrence_forward, and serves ck_recurrence_backward
 * unchanged.  ck_recurrence_status does not apply (the control block is not
 * in a caller workspace).
 */
ck_status ck_recurrence_forward_noalloc(ck_graph_t g, const float* edge_values,
                                        const float* leak, const float* bias, const float* drives,
                                        const float* state0, int64_t T, int64_t B,
                                        int64_t microsteps, float* out, void* saved,
                                        hipStream_t stream);

/*
 * Gradient of L given grad_out = dL/dout, for all five inputs
 * (connectome-kernels README, introduction and "Design notes": elementwise
 * gradients with per-node leak/bias reductions, the transposed sparse product
 * for the state gradient, the per-edge batch dot product for the edge
 * gradient; no sparse tensor is formed).  `saved` must come from the forward
 * call with the same graph, edge values, leak, state0, T, B and microsteps.
 *
 *   grad_out          fp32[T][B][N]
 *   grad_edge_values  fp32[E] caller edge order   (all five outputs are
 *   grad_leak         fp32[N]                      overwritten, not
 *   grad_bias         fp32[N]                      accumulated)
 *   grad_drives       fp32[T][n_in][B]
 *   grad_state0       fp32[B][N]
 */
ck_status ck_recurrence_backward(ck_graph_t g, const float* edge_values, const float* leak,
                                 const float* state0, int64_t T, int64_t B, int64_t microsteps,
                                 const void* saved, const float* grad_out,
                                 float* grad_edge_values, float* grad_leak, float* grad_bias,
                                 float* grad_drives, float* grad_state0, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * Status of the last forward or backward call that used `workspace` (same
 * graph, T, B and microsteps).  Synchronises `stream`, then returns CK_OK, or
 * CK_ERR_WAIT if that call ran the XCD-resident kernels and one of their
 * bounded waits gave up -- typically because other device work ran beside
 * the call -- or if the call was a backward whose saved arena came from such
 * a failed forward.  In both cases every output of that call was set to NaN.
 * The per-microstep kernels have no waits: CK_OK.
 */
ck_status ck_recurrence_status(ck_graph_t g, int64_t T, int64_t B, int64_t microsteps,
                               const void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * Measurement hook (changes no result).  While enabled (process-wide),
 * forward and backward record a pair of HIP events on the caller's stream
 * around every launch of the main kernels: the fused forward microstep and
 * backward step kernels, or the XCD-resident forward and backward kernels
 * (timing-only events without a system-scope fence).  ck_profile_collect synchronises the device,
 * returns the summed kernel durations in milliseconds and the launch counts
 * since the last collect, and releases the events.  Any output pointer may be NULL.  Not meant for concurrent use from
 * several threads.
 */
ck_status ck_profile_enable(int enable);
ck_status ck_profile_collect(double* fwd_ms, int64_t* fwd_launches, double* bwd_ms,
                             int64_t* bwd_launches);

/*
 * ---------------------------------------------------------------------------
 * Fixed-point leaky integrate-and-fire (LIF) forward on the same graph handle
 * (soup-connectome page, "Runtime contract": signed int32 membrane potentials,
 * signed int16 synaptic impulses, positive integer timestep delays, checked
 * arithmetic with rejected overflow, the arithmetic-shift leak
 * V := V - (V >> k); "Full-scale benchmark": a run's threshold, reset,
 * decay_shifts and refractory_steps).  The page fixes the representation,
 * not the update order; this library's reading, per timestep t and neuron i:
 *
 *   I = sum of w[e] over the in-edges e of i whose source spiked at t - d[e]
 *       (exact; impulses whose arrival step precedes the run never exist)
 *   if i is refractory (count r > 0): r -= 1, I is dropped, V is kept, no spike
 *   else: for each k in decay_shifts in order, V := V - (V >> k) (arithmetic
 *         shift, i.e. floor(V / 2^k)); V := V + I, rejected if it leaves the
 *         int32 range; if V >= threshold: spike, V := reset, r := refractory_steps
 *   spikes[t][i] = spike, potentials[t][i] = V.
 *
 * The graph's input_nodes play no part.  Integer arithmetic is exact: results
 * are bit-identical to any correct evaluation.
 */
typedef struct {
  int32_t threshold;         /* a neuron spikes when its potential reaches this value */
  int32_t reset;             /* potential right after a spike */
  int32_t refractory_steps;  /* >= 0: steps after a spike that ignore input */
  int32_t num_decay_shifts;  /* 0..8 */
  int32_t decay_shifts[8];   /* each in [0, 31]: V := V - (V >> k), applied in order */
} ck_lif_params;

/* Workspace bytes of ck_lif_forward (and of ck_lif_prepare / ck_lif_run) on
 * this graph. */
ck_status ck_lif_workspace_size(ck_graph_t g, size_t* workspace_bytes);

/*
 *   impulses     int16[E]  device, caller edge order: the impulse edge e delivers
 *   delays       int32[E]  device, caller edge order: steps until it arrives, 1..32767
 *   params       host pointer (above)
 *   v0           int32[N]  device: potentials before step 0 (refractory counts start at 0)
 *   T            timesteps, 1..2^31-1
 *   spikes       uint8[T][N]  device, written (1 = spike)
 *   potentials   int32[T][N]  device, written: V after each step
 *   overflow_step  host, may be NULL: -1, or the first step whose update left
 *                  the int32 range
 * Runs on `stream` and synchronises it twice: once after the delays are
 * validated (before any step runs; the largest delay picks the spike lookup:
 * bit rows of the last max-delay steps held in LDS when max delay <= 16 and
 * they fit 128 KB, else one byte read of `spikes` per edge; the environment
 * variable CK_LIF_LDS set to "0" keeps the byte reads) and once at the end
 * (the overflow check is read back).  Returns CK_ERR_OVERFLOW if a potential left the int32
 * range (outputs of that step and later are unspecified), CK_ERR_BAD_VALUE for
 * a delay outside [1, 32767] (no step is run), more than 8 decay shifts, a
 * shift outside [0, 31] or a negative refractory count.
 */
ck_status ck_lif_forward(ck_graph_t g, const int16_t* impulses, const int32_t* delays,
                         const ck_lif_params* params, const int32_t* v0, int64_t T,
                         uint8_t* spikes, int32_t* potentials, int64_t* overflow_step,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ck_lif_forward in two parts, for many runs over one set of synapses (the
 * soup-connectome page's runtime loads a connectome once and runs it many
 * times).  ck_lif_prepare validates the delays and leaves the synapses,
 * packed in CSR order, in the workspace (which the caller keeps; argument
 * meaning as for ck_lif_forward; synchronises the stream; CK_ERR_BAD_VALUE
 * for a delay outside [1, 32767]).  ck_lif_run runs T steps from v0 on
 * synapses a ck_lif_prepare (or ck_lif_forward) left in that workspace for
 * this graph, with the spike lookup that prepare chose; it leaves them in
 * place, so runs can follow one another.  It returns CK_ERR_BAD_VALUE when the
 * workspace holds no prepared synapses of this graph, and otherwise as
 * ck_lif_forward.  Results equal ck_lif_forward's bit for bit.
 */
ck_status ck_lif_prepare(ck_graph_t g, const int16_t* impulses, const int32_t* delays,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);
ck_status ck_lif_run(ck_graph_t g, const ck_lif_params* params, const int32_t* v0, int64_t T,
                     uint8_t* spikes, int32_t* potentials, int64_t* overflow_step,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Measurement hook for the LIF forward: summed durations (ms) and counts of
 * the per-step gather and update launches recorded while ck_profile_enable
 * is on, since the last collect (synchronises the device). */
ck_status ck_profile_collect_lif(double* gather_ms, int64_t* gather_launches, double* update_ms,
                                 int64_t* update_launches);

/* Static name of a status value. */
const char* ck_status_string(ck_status s);

/* Thread-local detail message of the last failing call on this thread ("" if none). */
const char* ck_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CK_H */
