/*
 * gdr.h - C ABI of the chunked gated delta rule forward pass for AMD MI355X
 * (gfx950, CDNA4).
 *
 * The operation is `chunk_gated_delta_rule`, named on the FlashQLA pages
 * ("FlashQLA GDN backend produces different tokens from FLA Triton", Setup:
 * chunk size 64, varlen API, initial and final state; "Findings from
 * integrating FlashQLA's Blackwell GDN kernels into a JAX trainer", items 1-3).
 * The pages name the op but not its formula; it is the gated delta rule of
 * Gated DeltaNet.  Per sequence and v-head, with the state kept as H = S^T
 * (dk x dv):
 *
 *     S_t = exp(g_t) * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale * S_t q_t
 *
 * evaluated in chunks of 64 tokens (within a chunk: a 64x64 unit lower
 * triangular solve into the WY form, then one state hand-off per chunk).
 *
 * Tensors are passed as plain descriptors (device pointer, dtype, shape and
 * optional strides).  No torch or other framework type appears here.
 *
 * Ownership: the caller owns every buffer.  The library keeps no pointer after
 * a call returns, never frees caller memory, and caches nothing keyed by a
 * tensor's address or by a stream.  Work is enqueued on `stream` and the call
 * returns without synchronising.  cu_seqlens is read only on the device, on
 * every call (no host copy, no cache of derived chunk indices).
 *
 * Errors: every descriptor is validated on the host before anything is
 * enqueued.  On a non-zero status nothing has been enqueued and no output has
 * been touched; gdr_last_error() returns a message for the calling thread.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t; NULL means the default (null) stream. */
struct ihipStream_t;
typedef struct ihipStream_t *hipStream_t;

typedef enum {
    GDR_OK = 0,
    GDR_EINVAL = -1,  /* NULL descriptor / data pointer, non-finite scale, bad argument */
    GDR_ESHAPE = -2,  /* ranks or extents inconsistent with one another or unsupported */
    GDR_EDTYPE = -3,  /* dtype not accepted for that argument */
    GDR_ESTRIDE = -4, /* strides are not compact row-major */
    GDR_EALIAS = -5,  /* an output overlaps an input or another output */
    GDR_EDEVICE = -6, /* current device is not gfx950 or cannot be queried */
    GDR_ELAUNCH = -7, /* a kernel launch or a stream operation failed */
    GDR_ENOMEM = -8   /* device memory for the call's workspace could not be obtained */
} gdr_status;

typedef enum { GDR_F32 = 0, GDR_BF16 = 1, GDR_I32 = 2 } gdr_dtype;

/*
 * A tensor descriptor.  `data` is a device pointer (may be NULL only when the
 * tensor has no elements).  `shape` has `ndim` extents.  `strides` (in
 * elements) may be NULL, meaning compact row-major, as DLPack defines it
 * (the integration report, item 3, notes a generated stub that rejected NULL
 * strides); non-NULL strides must equal the compact row-major ones.
 */
typedef struct {
    void *data;
    int32_t dtype;          /* a gdr_dtype value */
    int32_t ndim;
    const int64_t *shape;
    const int64_t *strides; /* NULL = compact row-major */
} gdr_tensor;

/*
 * gdr_chunk_fwd - forward pass of chunk_gated_delta_rule, chunk size 64.
 *
 *   q, k        [B, T, Hk, dk]   bf16 or f32 (q, k, v, o share one dtype)
 *   v           [B, T, Hv, dv]
 *   g           [B, T, Hv]       log-gate (natural log; decay is exp(g)), bf16 or f32
 *   beta        [B, T, Hv]       same dtype as g
 *   cu_seqlens  [N+1] int32, or NULL.  With cu_seqlens, B must be 1 and
 *               sequence n owns tokens [cu[n], cu[n+1]).  Preconditions (not
 *               checked on the host, since the content stays on the device):
 *               cu[0] == 0, non-decreasing, cu[N] == T.  Repeated offsets are
 *               length-0 ("ghost") segments, allowed anywhere: they read
 *               nothing and write nothing (the integration report, item 2).
 *               NULL means B fixed-length sequences of T tokens (N = B).
 *   h0          [N, Hv, dk, dv] f32 initial state, or NULL for zero.
 *   o           [B, T, Hv, dv]   output, dtype of q.  Rows of tokens outside
 *               every segment are not written.
 *   ht          [N, Hv, dk, dv] f32 final state, or NULL (not written).
 *               Rows of ghost segments keep their previous bytes.
 *   scale       output scale (callers usually pass dk^-0.5).
 *   stream      HIP stream the work is enqueued on.
 *
 * Constraints: dk and dv each 64 or 128 (independently); Hv % Hk == 0 and v-head h reads
 * q/k head h / (Hv / Hk); all tensors compact row-major.  o and ht must not
 * overlap any input or each other.  The current device must be gfx950.
 *
 * Numerics: bf16 inputs run the chunked kernel (512 threads per (sequence,
 * v-head)) with bf16 MFMA operands, fp32 accumulation and an fp32 state; o is
 * rounded once to bf16 (nearest-even).  f32 inputs ask for f32 precision and
 * run a token-serial kernel (256 threads per (sequence, v-head)) in fp32
 * arithmetic throughout: H <- e^g H, d = beta (v - H^T k), H <- H + k d^T,
 * o = scale H^T q for each token in turn, with no bf16 rounding anywhere
 * (error against an fp64 evaluation at fp32 rounding level, about 1e-7
 * relative to the state).  It is latency-bound, one token after another, and
 * meant for checking and for f32 callers, not for throughput.  Results do not
 * depend on scheduling: ghost padding and repeated calls are bitwise
 * reproducible.
 *
 * Uses a small device workspace (4*N + 16 bytes) when cu_seqlens is given.
 * The library keeps, per device, a ring of 8 reusable workspace buffers, all
 * created by the first call on the device in one allocation (1 MiB each at
 * least) and kept until gdr_free_workspaces or the end of the process; a
 * later request larger than a buffer regrows the whole ring once.  A call
 * takes the next buffer of the ring and, if its previous user may still be
 * running, makes `stream` wait for it on the GPU (an event recorded after
 * that user's kernels): no host wait, no allocation or free per call once
 * the ring exists, correct across streams and threads.  The ring is indexed
 * by a counter, not by stream or tensor identity (the review of
 * "feat(cake_kda): add paired recurrent training for SM100a and SM103a" asks
 * for bounded workspace caches that are not keyed by stream handles).
 *
 * Failure reporting inside the kernel: the kernel's two wave roles hand
 * chunks to each other through bounded waits.  A wait that gives up (never
 * expected; see gdr_debug_set) sets GDR_DEVSTAT_WAIT_TIMEOUT in the device
 * status word (gdr_device_status) and writes NaN to the affected rows of ht.
 */
int gdr_chunk_fwd(const gdr_tensor *q, const gdr_tensor *k, const gdr_tensor *v,
                  const gdr_tensor *g, const gdr_tensor *beta, const gdr_tensor *cu_seqlens,
                  const gdr_tensor *h0, const gdr_tensor *o, const gdr_tensor *ht,
                  float scale, hipStream_t stream);

/*
 * gdr_chunk_fwd_noalloc - gdr_chunk_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation.  Same arguments, results and errors as
 * gdr_chunk_fwd, bit for bit; it never calls hipMalloc, hipFree or any
 * allocating routine.  Its workspace (the dispatch order, 4*N + 16 bytes with
 * cu_seqlens) is a static 64 KiB device array that each GPU holds until the
 * process ends, so with cu_seqlens N is limited to 16380 sequences (larger N:
 * GDR_ESHAPE, use gdr_chunk_fwd).  Every call on one GPU shares that array
 * and overwrites it before reading it; calls that overlap on one GPU (on
 * different streams, or from different threads without ordering) race on it
 * and must not be issued.  Calls without cu_seqlens use no workspace.
 */
int gdr_chunk_fwd_noalloc(const gdr_tensor *q, const gdr_tensor *k, const gdr_tensor *v,
                          const gdr_tensor *g, const gdr_tensor *beta, const gdr_tensor *cu_seqlens,
                          const gdr_tensor *h0, const gdr_tensor *o, const gdr_tensor *ht,
                          float scale, hipStream_t stream);

/*
 * gdr_chunk_fwd_checkpoints - gdr_chunk_fwd that also writes the state after
 * every 64-token chunk of every sequence: the per-chunk state checkpoints that
 * the pages' prefill surface keeps for prefix caching (`state_checkpoints`,
 * "feat(cake_kda): add paired recurrent training for SM100a and SM103a", the
 * follow-up's list of kept kwargs).
 *
 *   h_chunks  fp32 [R, Hv, dk, dv] out (device), R = ceil(T/64) + N with
 *             cu_seqlens, else B * ceil(T/64).  Chunk c of sequence n holds
 *             its tokens 64c .. min(64(c+1), L_n) - 1; row off_n + c receives
 *             H (= S^T, [dk][dv]) after the last of them, where off_n = sum
 *             over m < n of ceil(L_m / 64) (the chunk_offsets of
 *             gdr_prepare_chunks).  The last chunk of a sequence holds ht.
 *             Rows past NT = off_N are not written; length-0 sequences own
 *             no rows.
 *
 * Everything else, including o and ht, is exactly gdr_chunk_fwd (f32 inputs:
 * the fp32 kernel, which stores the same rows).  Extra traffic: 4 * dk * dv
 * bytes per (chunk, v-head) written.  With cu_seqlens the
 * workspace is 8*N + 20 bytes (order and chunk offsets); sequences start
 * longest first.  Errors as gdr_chunk_fwd, plus GDR_EINVAL (h_chunks NULL),
 * GDR_EDTYPE / GDR_ESHAPE for h_chunks, GDR_EALIAS when it overlaps any other
 * tensor.
 */
int gdr_chunk_fwd_checkpoints(const gdr_tensor *q, const gdr_tensor *k, const gdr_tensor *v,
                              const gdr_tensor *g, const gdr_tensor *beta,
                              const gdr_tensor *cu_seqlens, const gdr_tensor *h0,
                              const gdr_tensor *o, const gdr_tensor *ht,
                              const gdr_tensor *h_chunks, float scale, hipStream_t stream);

/*
 * gdr_chunk_fwd_checkpoints_n - gdr_chunk_fwd_checkpoints with a checkpoint
 * every `every_n` tokens in place of every 64.  The same kept prefill surface
 * ("feat(cake_kda): add paired recurrent training for SM100a and SM103a", the
 * follow-up's list of kept kwargs) has a `checkpoint_every_n_tokens` argument
 * beside `state_checkpoints`, and keeps checkpoint granularity 16.
 *
 *   every_n   a multiple of 16, 16 <= every_n <= 2^30
 *   h_ckpt    fp32 [R, Hv, dk, dv] out (device), R = ceil(T/every_n) + N with
 *             cu_seqlens, else B * ceil(T/every_n).  Sequence n owns
 *             ceil(L_n / every_n) rows starting at off_n = sum over m < n of
 *             ceil(L_m / every_n); row off_n + j receives H (= S^T, [dk][dv])
 *             after min((j+1) every_n, L_n) tokens, so the last row of a
 *             sequence is its ht.  Rows past off_N are not written; length-0
 *             sequences own no rows.
 *
 * every_n = 64 gives gdr_chunk_fwd_checkpoints bit for bit, and o and ht are
 * gdr_chunk_fwd's for any every_n.  bf16 inputs: a checkpoint inside a
 * 64-token chunk is formed from the state at the chunk's start and the
 * chunk's first 16, 32 or 48 tokens (bf16 MFMA operands, fp32 accumulation;
 * same tolerance as the chunk-end rows).  f32 inputs: the fp32 kernel stores
 * its state after the token.  Extra traffic: 4 * dk * dv bytes per row
 * written.  With cu_seqlens the workspace is 8*N + 20 bytes.  Errors: those of
 * gdr_chunk_fwd_checkpoints (for h_ckpt), plus GDR_EINVAL for every_n.
 */
int gdr_chunk_fwd_checkpoints_n(const gdr_tensor *q, const gdr_tensor *k, const gdr_tensor *v,
                                const gdr_tensor *g, const gdr_tensor *beta,
                                const gdr_tensor *cu_seqlens, const gdr_tensor *h0,
                                const gdr_tensor *o, const gdr_tensor *ht,
                                const gdr_tensor *h_ckpt, int64_t every_n, float scale,
                                hipStream_t stream);

/*
 * gdr_chunk_bwd - backward pass of gdr_chunk_fwd: the gradients of the scalar
 * loss L given dL/do and dL/dht, for every input.  The pages discuss the
 * backward as the other half of the kernel family ("Findings from integrating
 * FlashQLA's Blackwell GDN kernels into a JAX trainer", opening summary and
 * items 3-4) without giving its formula; these are the exact derivatives of
 * the recurrence above, evaluated in chunks of 64 tokens.
 *
 *   q, k, v, g, beta, cu_seqlens, h0   the forward inputs, as in gdr_chunk_fwd
 *   do          [B, T, Hv, dv]   dL/do, dtype of q
 *   dht         [N, Hv, dk, dv]  f32 dL/dht, or NULL for zero
 *   dq, dk      [B, T, Hk, dk]   out, dtype of q (summed over the Hv / Hk
 *                                v-heads that share each q/k head)
 *   dv          [B, T, Hv, dv]   out, dtype of q
 *   dg, dbeta   [B, T, Hv]       out, f32 (dg: gradient of the log-gate)
 *   dh0         [N, Hv, dk, dv]  out, f32, or NULL (not written); written also
 *                                when h0 is NULL (the gradient of the zero state)
 *   scale       the forward's output scale.
 *
 * Rows of tokens outside every segment are not written; length-0 segments
 * read nothing and write nothing (their dh0 rows keep their bytes).  The
 * gradient outputs must not overlap any input or each other.
 *
 * Work: the forward states after every chunk are recomputed (the forward
 * kernel, without o), then three kernels run: a per-chunk preparation, the
 * reverse pass over the chunks of each sequence, and the per-chunk gradients.
 * Numerics: bf16 MFMA operands, fp32 accumulation and fp32 state gradients.
 *
 * Workspace: the library's large per-device buffer (reused like the ring of
 * gdr_chunk_fwd: concurrent backward calls on one device are ordered on the
 * GPU), of
 * R * Hv * (4 d^2 + 128 d + 8192) bytes plus 4 (2N + 1 + 2R) for the
 * chunk indices, R = ceil(T/64) + N with cu_seqlens else B * ceil(T/64).
 * About 3.0 GB for 65536 tokens, 32 v-heads, d = 128.  Errors as
 * gdr_chunk_fwd, with GDR_ENOMEM when the workspace cannot be obtained, and
 * GDR_ESHAPE unless dk == dv (the backward kernels are written for square
 * states).
 */
int gdr_chunk_bwd(const gdr_tensor *q, const gdr_tensor *k, const gdr_tensor *v, const gdr_tensor *g,
                  const gdr_tensor *beta, const gdr_tensor *cu_seqlens, const gdr_tensor *h0,
                  const gdr_tensor *dout, const gdr_tensor *dht, const gdr_tensor *dq, const gdr_tensor *dk,
                  const gdr_tensor *dv, const gdr_tensor *dg, const gdr_tensor *dbeta, const gdr_tensor *dh0,
                  float scale, hipStream_t stream);

/*
 * gdr_chunk_kda_fwd - gdr_chunk_fwd with one log-gate per key channel: the
 * KDA-style variant of "feat(cake_kda): add paired recurrent training for
 * SM100a and SM103a", whose raw gate has one value per key channel.  The
 * scalar decay exp(g_t) becomes diag(exp(g_t)) on the key side:
 *
 *     S_t = S_{t-1} diag(exp(g_t)) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *
 *   g      [B, T, Hv, dk]   per-channel natural-log decay, bf16 or f32 (the
 *                           transform from a raw gate, undefined on the pages,
 *                           is the caller's)
 *   beta   [B, T, Hv]       same dtype as g
 *
 * Everything else (shapes, varlen and ghosts, h0/ht, GQA, errors) is
 * gdr_chunk_fwd, except that dk must equal dv (GDR_ESHAPE otherwise).  bf16 inputs: within one 64-token chunk the gates are
 * folded into the operands with one reference per block of 16 tokens, so a
 * channel's log-decay summed over 16 tokens must stay above about -87 (fp32
 * exponent range), about -5.4 per token: this holds the pages' safe-gate
 * lower bound of -5 ("feat(cake_kda): add paired recurrent training for
 * SM100a and SM103a", the maintainer's section).  A call that meets steeper
 * gates sets GDR_DEVSTAT_KDA_RANGE in the device status word
 * (gdr_device_status).  f32 inputs run the token-serial fp32 kernel of
 * gdr_chunk_fwd with diag(exp(g_t)) in place of exp(g_t): any gate is in
 * range.  With cu_seqlens the workspace is 4*N + 16 bytes (longest sequences
 * start first).
 */
int gdr_chunk_kda_fwd(const gdr_tensor *q, const gdr_tensor *k, const gdr_tensor *v, const gdr_tensor *g,
                      const gdr_tensor *beta, const gdr_tensor *cu_seqlens, const gdr_tensor *h0,
                      const gdr_tensor *o, const gdr_tensor *ht, float scale, hipStream_t stream);

/*
 * gdr_decode_step - one token of the same recurrence for each of B sequences:
 * the decode step that follows this forward pass in inference (the pages'
 * inference surface keeps a decode module beside the prefill, "feat(cake_kda):
 * add paired recurrent training for SM100a and SM103a", the follow-up's list
 * of kept modules), consuming the final state of gdr_chunk_fwd.  With the
 * state H = S^T [dk][dv] of sequence b and v-head h:
 *     H <- e^g H,  d = beta (v - H^T k),  H <- H + k d^T,  o = scale H^T q.
 *
 *   q, k   [B, Hk, dk]  bf16 or f32 (one dtype with v and o)
 *   v      [B, Hv, dv]
 *   g, beta [B, Hv]     bf16 or f32 (g is the log-gate of the token)
 *   h      [B, Hv, dk, dv] fp32, read and overwritten with the new state
 *   o      [B, Hv, dv]  out, rounded once to its dtype
 *   scale  as gdr_chunk_fwd
 *
 * dk and dv each 64 or 128; Hv % Hk == 0 (v-head h reads q/k head h / (Hv/Hk)).  fp32
 * arithmetic throughout.  No workspace.  HBM bound: 8 * dk * dv bytes of state
 * traffic per (sequence, v-head).  Errors: GDR_ESHAPE, GDR_EDTYPE, GDR_EINVAL
 * (alignment: q/k/v 8 bytes, h and o 16 bytes; scale), GDR_EALIAS (o or h
 * overlaps an input or each other), GDR_EDEVICE, GDR_ELAUNCH.
 */
int gdr_decode_step(const gdr_tensor *q, const gdr_tensor *k, const gdr_tensor *v,
                    const gdr_tensor *g, const gdr_tensor *beta, const gdr_tensor *h,
                    const gdr_tensor *o, float scale, hipStream_t stream);

/*
 * Launch plan of a gdr_chunk_fwd call, computed from shapes only (no device
 * access, no allocation).  gdr_plan validates exactly like gdr_chunk_fwd and
 * fills `plan`; it is what gdr_chunk_fwd launches.  It exists so that the
 * validation of every extent can be tested without a GPU: the review of
 * "feat(cake_kda): add paired recurrent training for SM100a and SM103a" asks
 * that every tensor's element count be checked before launch (an undersized
 * tensor must give an error, not out-of-bounds accesses) and tests its
 * bindings against a recording stand-in for the device module.
 *
 *   q .. ht, scale  as gdr_chunk_fwd (data pointers are only compared for
 *                   overlaps, never dereferenced)
 *   plan            out, host memory owned by the caller
 *
 * Returns the status gdr_chunk_fwd would return for these descriptors before
 * touching the device (GDR_OK, GDR_EINVAL, GDR_ESHAPE, GDR_EDTYPE,
 * GDR_ESTRIDE, GDR_EALIAS); GDR_EINVAL when plan is NULL.
 */
typedef struct {
    int64_t n_seq;          /* N */
    int64_t total_tokens;   /* B * T */
    int64_t nt_max;         /* upper bound on the number of 64-token chunks: ceil(B*T/64) + N */
    int32_t hk, hv, d;      /* heads and the key head dim dk */
    int32_t in_dtype;       /* gdr_dtype of q/k/v/o */
    int32_t gate_dtype;     /* gdr_dtype of g/beta */
    int32_t varlen;         /* 1 when cu_seqlens is given */
    int32_t has_h0, has_ht;
    int64_t grid_fwd;       /* work-groups of the forward kernel: N * Hv */
    int32_t block_fwd;      /* threads per work-group: 512 (bf16 inputs), 256 (f32) */
    int32_t lds_fwd;        /* bytes of LDS per work-group */
    int64_t workspace_bytes;/* device workspace per call: 4*N + 16 with cu_seqlens */
    int32_t dv;             /* the value head dim */
} gdr_launch_plan;

int gdr_plan(const gdr_tensor *q, const gdr_tensor *k, const gdr_tensor *v,
             const gdr_tensor *g, const gdr_tensor *beta, const gdr_tensor *cu_seqlens,
             const gdr_tensor *h0, const gdr_tensor *o, const gdr_tensor *ht, float scale,
             gdr_launch_plan *plan);

/*
 * gdr_prepare_chunks - chunk indices derived from the content of cu_seqlens on
 * the device (the integration report, item 1: the indices must follow the
 * content of every call, never a cache keyed by tensor identity).
 *
 *   cu_seqlens     [N+1] int32 (device)
 *   chunk_offsets  [N+1] int32 out: exclusive prefix sum of ceil(L_n / 64)
 *   chunk_map      [nt_max, 2] int32 out, or NULL: entry i < NT holds
 *                  (sequence n, chunk c within n); entries NT..nt_max-1 hold
 *                  (-1, -1).  nt_max = shape[0] must be >= the true NT
 *                  (ceil(T/64) + N always is); extra entries are marked.
 *   seq_order      [N] int32 out, or NULL: sequence indices by length,
 *                  longest first, ties by index (N > 8192: identity order).
 *
 * Work-list only: the forward pass uses seq_order to start long sequences
 * first; results never depend on it.
 */
int gdr_prepare_chunks(const gdr_tensor *cu_seqlens, const gdr_tensor *chunk_offsets,
                       const gdr_tensor *chunk_map, const gdr_tensor *seq_order,
                       hipStream_t stream);

/*
 * gdr_dispatch_order - the order in which gdr_chunk_fwd starts the sequences
 * of a varlen call when there are few of them, derived on the device from the
 * content of cu_seqlens on every call (the integration report, item 1).
 *
 *   cu_seqlens  [N+1] int32 (device), 1 <= N <= 64
 *   groups      machines of the schedule model, 1..16
 *   order       [N] int32 out (device): a permutation of 0..N-1
 *
 * Model: `groups` identical machines (each the CUs that run all v-heads of
 * one sequence at once); sequence n keeps one busy for ceil(L_n / 64) + 1
 * units; work-groups start in grid order on the machine that frees first.
 * The result is the longest-first order (ties by index, length-0 sequences
 * last) unless an order built from a first-fit-decreasing bin packing at
 * the smallest capacity that fits (capacities tried: up to 64 evenly spaced
 * values below the longest-first makespan) has a smaller makespan in that
 * model.  gdr_chunk_fwd uses it with groups = (work-groups resident on the
 * device) / Hv when Hv is a multiple of 8, that ratio is 2..16 and smaller
 * than N, and N <= 64; otherwise it starts sequences longest first.
 * Work-list only: results never depend on it.
 *
 * Errors: GDR_ESHAPE (N outside 1..64, order not [N]), GDR_EINVAL (groups),
 * GDR_EDTYPE, GDR_EALIAS (order overlaps cu_seqlens), GDR_EDEVICE,
 * GDR_ELAUNCH.  Enqueued on `stream`; no workspace.
 */
int gdr_dispatch_order(const gdr_tensor *cu_seqlens, int32_t groups, const gdr_tensor *order,
                       hipStream_t stream);

/*
 * gdr_chunk_local_cumsum - chunk-local inclusive prefix sum of the log-gate:
 * G[t, h] = sum of g[s, h] for s from the start of t's 64-token chunk to t.
 * Chunks restart at every sequence start.  Computed in fp32.
 *
 *   g           [B, T, H] bf16 or f32
 *   cu_seqlens  [N+1] int32 or NULL (B fixed-length rows)
 *   G           [B, T, H] f32 out (rows outside every segment not written)
 *
 * Uses a workspace for the chunk map (8 * nt_max bytes) from the same
 * per-device ring as gdr_chunk_fwd.
 */
int gdr_chunk_local_cumsum(const gdr_tensor *g, const gdr_tensor *cu_seqlens,
                           const gdr_tensor *G, hipStream_t stream);

/*
 * Text of the last non-OK status returned on the calling thread ("" after an
 * OK status).  Every check of every entry point has its own message naming
 * the argument and the values involved (the review of "feat(cake_kda): add
 * paired recurrent training for SM100a and SM103a" asks for a message on
 * every check).  The pointer is owned by the library and stays valid until
 * the calling thread's next call into it.
 */
const char *gdr_last_error(void);

/* Options of gdr_debug_set. */
typedef enum {
    /* value != 0: before every call that takes cu_seqlens, check its content
     * on the device (cu[0] == 0, non-decreasing, cu[N] == T), wait for the
     * stream and return GDR_EINVAL with the first violation (the planned
     * debug check for the content preconditions, which a call cannot check on
     * the host without a device read).  Also on with GDR_DEBUG_CHECK_CU=1 in
     * the environment. */
    GDR_DEBUG_CHECK_CU = 1,
    /* value = n >= 0: the next n kernel launches of the library's entry
     * points fail as if the launch had failed (GDR_ELAUNCH; nothing of the
     * failed kernel runs, outputs stay untouched).  Test hook. */
    GDR_DEBUG_FAIL_LAUNCHES = 2,
    /* value = polls before a hand-off wait inside the forward kernel gives up
     * (each poll sleeps about 64 cycles); value < 0 restores the default
     * 2^18.  A small value makes the waits give up early, which exercises
     * GDR_DEVSTAT_WAIT_TIMEOUT without hanging anything.  Test hook. */
    GDR_DEBUG_SPIN_LIMIT = 3
} gdr_debug_option;

/*
 * gdr_debug_set - process-wide debug and test options (see gdr_debug_option).
 * Returns GDR_OK, or GDR_EINVAL for an unknown option or a value out of range.
 * No device access.
 */
int gdr_debug_set(int option, int64_t value);

/* Bits of the device status word. */
#define GDR_DEVSTAT_WAIT_TIMEOUT 1u /* a forward kernel's hand-off wait gave up: its outputs are wrong */
#define GDR_DEVSTAT_KDA_RANGE 2u    /* gdr_chunk_kda_fwd (bf16 inputs) met a channel whose log-decay over
                                       one 16-token block is below about -87: its outputs are not finite */

/*
 * gdr_device_status - the status word of the current device: bits the
 * kernels set when something went wrong inside them (GDR_DEVSTAT_*), sticky
 * across calls.  Synchronises the current device first.  clear != 0 resets
 * the word to zero after reading it.  bits: host memory, written on GDR_OK.
 * Errors: GDR_EINVAL (bits NULL), GDR_EDEVICE, GDR_ELAUNCH (the
 * synchronisation or copy failed).
 */
int gdr_device_status(uint32_t *bits, int clear);

/*
 * gdr_free_workspaces - release the current device's workspace ring and the
 * backward pass's large buffer (waiting for their last users first).  The
 * next call that needs a workspace creates them again.  Must not run while
 * another thread is inside a call on the same device.  Returns GDR_OK,
 * GDR_EDEVICE or GDR_ELAUNCH.
 */
int gdr_free_workspaces(void);

/* ABI version: major * 10000 + minor * 100 + patch. */
int gdr_version(void);

/*
 * gdr_selftest_mfma - diagnostic: runs one wave of each bf16 MFMA shape the
 * kernels use on the given operands, so a test can check the lane layout the
 * kernels assume.  a, b: 64 lanes x 8 bf16 (device); c: out, 2 x 64 lanes x 4
 * f32 (first block: 16x16x32, second: 16x16x16 using the first 4 values of
 * each lane).  Returns GDR_ELAUNCH on a launch failure.
 */
int gdr_selftest_mfma(const uint16_t *a, const uint16_t *b, float *c, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
