/*
 * libloopspec - the per-step hot path of pipelined self-speculative decoding for looped
 * Transformers on AMD Instinct MI355X (gfx950).
 *
 * Method: "LoopSpec: Pipelined Self-Speculative Decoding for Looped Transformers"
 * (liuzhao09.github.io/papers/loopspec.html, arXiv:2609.17184).  A looped model is
 * H^(0) = P(X), H^(r) = B(H^(r-1)), p_r = C(H^(r)) for 1 <= r <= R (section 2.1, eq. 1).
 * One pipeline step applies the shared block B once to every active branch row, each row
 * at its own loop depth with its own depth-indexed KV cache (section 2.2 and 2.4), reads
 * out C at the proposal depths and at R, and verifies proposals losslessly (eq. 2-6 and the
 * cascade of section 2.3).
 *
 * Conventions shared by every call
 *  - All pointers to tensors are DEVICE pointers unless a field says "host".  The caller
 *    owns every buffer (weights, KV cache, hidden states, workspace, outputs); the library
 *    never allocates, frees or retains device memory.
 *  - Calls are stream-ordered and asynchronous: they validate the host-visible arguments,
 *    enqueue kernels on `stream` and return.  Buffers must stay alive until the stream has
 *    completed the work.  One stream per model at a time; distinct models are independent.
 *  - Every call returns an ls_status.  On failure nothing is enqueued and ls_last_error()
 *    (thread-local) describes the reason.  Malformed device-side descriptors (a slot outside
 *    [0, S), a token outside [0, V)) never cause an out-of-bounds access: the kernels skip
 *    the offending row and record LS_ERR_INVALID in the workspace error word, reported by
 *    ls_sync_status().
 *  - Matrices are row-major [out_features][in_features] (y = x W^T), elements bf16 (bit
 *    patterns in uint16) or fp32 according to the model dtype.  Hidden states are fp32.
 *  - KV caches hold one entry per slot; a slot is the storage of one token position of one
 *    branch.  Entry layout: [2][d] (keys then values), dtype of the model.  Keys are stored
 *    after the rotary embedding.
 */
#ifndef LOOPSPEC_H
#define LOOPSPEC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LS_OK = 0,
  LS_ERR_INVALID = 1,      /* bad argument or descriptor */
  LS_ERR_UNSUPPORTED = 2,  /* shape or option the kernels do not implement */
  LS_ERR_CAPACITY = 3,     /* more rows / keys / jobs than the workspace was sized for */
  LS_ERR_HIP = 4           /* a HIP runtime call failed */
} ls_status;

typedef enum { LS_F32 = 0, LS_BF16 = 1 } ls_dtype;

#define LS_MAX_READOUT_DEPTHS 8
#define LS_MAX_ROWS 128
#define LS_UNIFORMS_PER_JOB 24

/* Model shape.  Block internals: pre-RMSNorm, multi-head attention with rotary position
 * embedding (rotate-half), SwiGLU MLP, no biases; C = [coda layers] + RMSNorm + LM head
 * tied to the embedding.  Raven/Huginn-family models have prelude (L_pre) and coda
 * (L_coda) layers with their own caches (section 2.1, Fig. 2; section 2.4). */
typedef struct {
  int V, d, n_heads, head_dim, F;
  int L;                 /* layers of the shared block B */
  int L_pre, L_coda;     /* prelude / coda layers (0 for Ouro-like models) */
  int R;                 /* full loop depth */
  int n_readout;         /* |D| */
  int readout_depths[LS_MAX_READOUT_DEPTHS];  /* D, ascending, last entry == R */
  int dtype;             /* ls_dtype of weights, GEMM operands and KV cache */
  float rope_theta;
  float norm_eps;
  int slot_capacity;     /* S: slots in every KV cache */
} ls_model_desc;

typedef struct {
  const void *Wq, *Wk, *Wv, *Wo;   /* [d][d] */
  const void *Wg, *Wu;             /* [F][d] */
  const void *Wd;                  /* [d][F] */
  const float *g1, *g2;            /* RMSNorm gains [d] */
} ls_layer_ptrs;

typedef struct {
  const void *emb;                 /* [V][d]; also the LM head */
  const float *g_final;            /* [d] */
  const ls_layer_ptrs *pre;        /* host array [L_pre] */
  const ls_layer_ptrs *core;       /* host array [L] */
  const ls_layer_ptrs *coda;       /* host array [L_coda] */
} ls_weight_ptrs;

typedef struct ls_model ls_model;

/* KV caches (caller-owned; entry = [2][d] of the model dtype).
 *   core: [R][L][S] entries; loop iteration k (1..R) of layer l uses block (k-1, l).
 *   pre:  [L_pre][S] entries (may be NULL when L_pre == 0).
 *   coda: [n_readout][L_coda][S] entries; readout at depth D[j] uses block j (may be NULL
 *         when L_coda == 0).
 * KV of different loop depths is never mixed (section 2.1 on Fig. 2, section 2.4). */
typedef struct {
  void *core;
  void *pre;
  void *coda;
} ls_kv;

/* The rows of one call.  Row i is one branch: the token at absolute position pos[i] whose
 * state lives in slot[i].  Its attention keys, in position order, are the finished prefix
 * fin_slots[0 .. n_fin) shared by all rows, then its speculative ancestors
 * anc_slots[anc_off[i] .. anc_off[i+1]) (the branch mask: the path from the current root
 * to its parent), then slot[i] itself; so pos[i] == n_fin + anc_off[i+1] - anc_off[i].
 * A child reuses its parent's prefix by index, never by copying KV (section 2.4).
 *   n, n_fin, max_anc: host values.  All arrays: device int32.
 *   depth[i]: ls_loop_step - loop iteration to run (1..R);
 *             ls_readout   - index j into D of the readout depth;
 *             ls_prelude   - ignored. */
typedef struct {
  int n;
  int n_fin;
  int max_anc;           /* >= max_i (anc_off[i+1] - anc_off[i]) */
  const int32_t *slot;
  const int32_t *pos;
  const int32_t *depth;
  const int32_t *fin_slots;
  const int32_t *anc_off;    /* [n+1] */
  const int32_t *anc_slots;
} ls_rows;

typedef struct {
  int greedy;            /* nonzero: one-hot at the argmax (lowest id on ties) */
  float temperature;     /* > 0 */
  float top_p;           /* (0, 1]; >= 1 keeps every token */
} ls_sampling;

/* Verification jobs (section 2.2-2.3).  Probabilities are rows of `probs` ([*][V] fp32,
 * as written by ls_readout); each is read in fixed point A(v) = floor(p(v) * 2^40).
 * Uniform words: uniforms[job][k], k = 0 first draw, 1 second draw, 2 first accept,
 * 3 second accept, 4 residual resample, 5 plain draw, 8+j copy candidate j.
 * The second proposal q2 is q2_row (-) q1_row (eq. 5), or, with LS_JOB_NON_RESIDUAL in
 * flags, q2_row with x1 masked out (the non-residual ablation of Table 3, section 3.4);
 * DRAW2 and VERIFY of one branch must use the same form.
 * SCREEN is the shallow screening of copied candidates (CopyLoop page, "shallow screening"):
 * candidate c survives when A(c) >= thr, thr = (uint32)x1 | (uint64)(uint32)x2 << 32 (the
 * fixed-point threshold floor(tau * 2^40)); the survivors, ordered by A descending then id,
 * are written back to the front of the job's range cands[cand_off .. + n_cand), the rest
 * after them in input order; out.aux = number of survivors; with none, the job draws one
 * proposal token ~ p_row with u[0] (outcome DRAWN), else outcome SCREENED (token -1). */
typedef enum {
  LS_JOB_SAMPLE = 0,       /* token ~ p_row                                  (uses u[5]) */
  LS_JOB_DRAW1 = 1,        /* x1 ~ q1 = q1_row                               (u[0])      */
  LS_JOB_DRAW2 = 2,        /* gate (eq. 6) and x2 ~ q2                       (u[1])      */
  LS_JOB_VERIFY = 3,       /* cascade of x1 (and x2 if gate) against p_row   (u[2,3,4])  */
  LS_JOB_VERIFY_COPY = 4,  /* point-mass cascade over cands[cand_off..+n_cand] (u[8+j], u[4]) */
  LS_JOB_SCREEN = 5        /* keep cands with A(c) >= thr, in order; else draw (u[0])      */
} ls_job_op;

#define LS_JOB_NON_RESIDUAL 1   /* flags bit: q2 = q2_row with x1 masked (DRAW2, VERIFY) */

typedef struct {
  int32_t op;
  int32_t p_row, q1_row, q2_row;
  int32_t x1, x2;
  int32_t gate;            /* VERIFY: second candidate present; DRAW2: 1 = gated, 0 = ungated */
  int32_t cand_off, n_cand;
  int32_t flags;           /* LS_JOB_NON_RESIDUAL or 0 */
} ls_verify_job;

typedef enum { LS_OUT_ACC1 = 1, LS_OUT_ACC2 = 2, LS_OUT_RESAMPLED = 3, LS_OUT_DRAWN = 4, LS_OUT_ACC_COPY = 5,
               LS_OUT_SCREENED = 6 } ls_outcome;

typedef struct {
  int32_t token;
  int32_t outcome;         /* ls_outcome */
  int32_t gate;            /* DRAW2: gate open */
  int32_t aux;             /* VERIFY_COPY: index of the accepted candidate or -1; SCREEN: survivors */
} ls_verify_out;

/* Last error message of the calling thread (static storage, never NULL). */
const char *ls_last_error(void);

/* Create a model handle over caller-owned weights (pointers are retained, not copied).
 * Fails with LS_ERR_UNSUPPORTED if head_dim is not a multiple of 16 or exceeds 128, d or F
 * is not a multiple of 32 (bf16) / 16 (fp32), or V exceeds 65536. */
ls_status ls_model_create(const ls_model_desc *desc, const ls_weight_ptrs *w, ls_model **out);
void ls_model_destroy(ls_model *m);

/* Workspace bytes for calls with at most max_rows rows, max_keys attention keys per row and
 * max_jobs verification jobs.  The caller allocates it (device memory, 256-byte aligned). */
size_t ls_workspace_bytes(const ls_model *m, int max_rows, int max_keys, int max_jobs);

/* Bind a workspace of ls_workspace_bytes(m, max_rows, max_keys, max_jobs) bytes and clear
 * its error word (enqueued on stream).  Later calls with more rows/keys/jobs fail with
 * LS_ERR_CAPACITY. */
ls_status ls_bind_workspace(ls_model *m, void *ws, int max_rows, int max_keys, int max_jobs, hipStream_t stream);

/* P (eq. 1): H[slot[i]] = prelude(tokens[i]) for every row: the embedding row, then the
 * prelude layers (Raven/Huginn), which write the prelude cache at slot[i].
 * tokens: device int32 [n].  H: device fp32 [S][d]. */
ls_status ls_prelude(ls_model *m, const ls_rows *rows, const int32_t *tokens, float *H,
                     const ls_kv *kv, hipStream_t stream);

/* B (eq. 1), one loop iteration for every row: H[slot[i]] <- B_k(H[slot[i]]) with
 * k = depth[i], reading and writing the cache of depth k.  Rows may be at different
 * depths; the block weights are streamed from HBM once for all rows. */
ls_status ls_loop_step(ls_model *m, const ls_rows *rows, float *H, const ls_kv *kv, hipStream_t stream);

/* C (eq. 1 and section 2.1) at readout depth D[depth[i]] for every row: coda layers (cache
 * block depth[i]), final RMSNorm, tied LM head, temperature, top-p, normalisation.
 * probs: fp32 [*][V]; row i is written to probs[out_rows ? out_rows[i] : i] (out_rows:
 * device int32 [n] or NULL; entries must lie in [0, n_prob_rows), or be -1 to skip the
 * distribution of that row, e.g. when a readout only fills the coda caches).  argmax: int32 [n]
 * (lowest id on ties) or NULL; logits: fp32 [n][V] raw head outputs or NULL.  H is not
 * modified. */
ls_status ls_readout(ls_model *m, const ls_rows *rows, const float *H, const ls_sampling *smp,
                     float *probs, const int32_t *out_rows, int n_prob_rows, int32_t *argmax, float *logits,
                     const ls_kv *kv, hipStream_t stream);

/* Prefill of a chunk of prompt positions (the step before decoding: section 2.1, eq. 1
 * applied to the prompt; section 2.4 for the prelude, loop and coda caches; section 3.1
 * excludes it from decode timing).  Row i is position n_fin + i of the sequence whose first
 * n_fin positions are committed with their slots in fin_slots[0..n_fin) (device int32, every
 * cache already filled for them).  For every row the call runs P (embedding, prelude layers
 * writing the prelude cache at slots[i]), every loop iteration k = 1..R of B (writing the
 * cache of depth k at slots[i]; causal attention over the committed prefix and rows 0..i of
 * the chunk), and, for each readout depth index j with bit j of coda_mask set, the coda
 * layers on H^(D[j]) (writing the coda cache of that readout depth; their outputs are not
 * kept), and leaves H[slots[i]] = H^(R).  The readout of the last position (its distribution
 * at R) is an ls_readout call afterwards.  Each layer runs as matrix products with the
 * chunk's n rows as M (the weights are streamed once per layer per depth for the chunk).
 * tokens, slots: device int32 [n].  pws: device scratch of ls_prefill_workspace_bytes(m, n)
 * bytes or more, 256-byte aligned, caller-owned (LS_ERR_CAPACITY if smaller).  Requires a
 * bound workspace (its error word and rotary table).  A token outside [0, V) or a slot outside
 * [0, S) raises LS_ERR_INVALID in the error word: such a row's embedding is zero, an invalid
 * row slot stores nothing, an invalid prefix slot is read as slot 0. */
size_t ls_prefill_workspace_bytes(const ls_model *m, int max_n);
ls_status ls_prefill(ls_model *m, const int32_t *tokens, const int32_t *slots, int n, const int32_t *fin_slots,
                     int n_fin, unsigned coda_mask, float *H, const ls_kv *kv, void *pws, size_t pws_bytes,
                     hipStream_t stream);

/* Lossless verification jobs (section 2.2-2.3), one integer pass over V per job; results
 * are bit-identical for identical inputs.  jobs: [n_jobs]; probs: fp32
 * [n_prob_rows][V], each row a probability vector (entries in [0, 1], sum <= ~1; a row whose
 * fixed-point mass reaches 2^41 is rejected); cands: int32 [n_cands] (VERIFY_COPY and SCREEN
 * use cands[cand_off .. cand_off + n_cand), n_cand <= 16; SCREEN rewrites its range, every
 * other job only reads; the ranges of jobs of one call must not overlap); uniforms: uint32
 * [n_jobs][24]; out: [n_jobs].  jobs, cands, uniforms and out may be device memory or pinned
 * host memory (hipHostMalloc): the kernel reads each job, its uniforms and candidates once
 * and writes its results directly; out and the rewritten candidates are complete once the
 * stream is synchronised; the caller keeps host inputs unchanged until then.  A job with an
 * out-of-range row, token or candidate yields token -1, outcome 0 and LS_ERR_INVALID in the
 * error word. */
ls_status ls_verify(ls_model *m, const ls_verify_job *jobs, int n_jobs, const float *probs, int n_prob_rows,
                    int32_t *cands, int n_cands, const uint32_t *uniforms, ls_verify_out *out,
                    hipStream_t stream);

/* Synchronise `stream` and report the first device-side error recorded in the workspace
 * (LS_ERR_INVALID for a rejected descriptor) or LS_ERR_HIP for a runtime error. */
ls_status ls_sync_status(ls_model *m, hipStream_t stream);

/* ls_loop_step without a caller workspace, for callers that cannot allocate device memory
 * (code under graph capture, tight serving loops, harnesses that forbid allocation): the same
 * kernels and results as ls_loop_step, with every buffer the kernels need beyond the caller's
 * inputs and outputs in the library's static scratch (LS_STATIC_SCRATCH_BYTES of device
 * memory per GPU, held until the process ends).  No workspace needs to be bound; the call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).  The model's layer
 * and rotary tables are copied into the scratch when a model other than the last one to use
 * it on this GPU calls.  Calls that would need more scratch than LS_STATIC_SCRATCH_BYTES (many
 * rows with long prefixes) fail with LS_ERR_CAPACITY before anything is enqueued.  Every call on
 * a GPU shares that GPU's scratch: calls that overlap on one GPU (other streams, other threads,
 * other models) race and must be serialised by the caller.  err_out: optional device int32
 * that the caller zeroes; descriptor errors and wait timeouts of this call are recorded there
 * (first error wins, codes as in the workspace error word: 1 rejected descriptor, 5 timeout);
 * with NULL they are recorded in the scratch and not reported. */
#define LS_STATIC_SCRATCH_BYTES (64u << 20)
ls_status ls_loop_step_static(ls_model *m, const ls_rows *rows, float *H, const ls_kv *kv, int *err_out,
                              hipStream_t stream);

/* Bound on every dependency wait inside one layer-kernel launch (default 2 s): workgroups
 * wait for each other's results, and a wait still unmet that long after the launch started
 * gives up, records a timeout in the error word (ls_sync_status then returns LS_ERR_HIP) and
 * lets the launch run to its end without waiting; every later wait of the launch gives up at
 * its first poll.  Results of a launch that timed out are undefined.  seconds in [0, 3600];
 * 0 makes every wait that would block give up at once (a test of the give-up path). */
ls_status ls_set_wait_limit(ls_model *m, double seconds);

/* Diagnostics: while dev_buf is non-NULL, each later layer-kernel launch writes wall-clock
 * stamps (phase begin/end, dependency met, first chunk staged, first tile batch multiplied,
 * first/last weight slab issued; first 4 layers) per workgroup into dev_buf (device int64
 * [grid][4][8][8]); grid_out receives the grid size of the last launch.
 * Pass NULL to stop.  Not needed for decoding. */
ls_status ls_debug_trace(ls_model *m, long long *dev_buf, int *grid_out);

/* Measurement aid (not part of decoding): reads bytes of device memory at src with the loads
 * the layer kernel's producer waves use (16-byte direct-to-LDS, non-temporal, 1 KB per wave
 * instruction, 16 in flight per wave, two waves per workgroup), n_workgroups workgroups (one per
 * CU: the device's multiprocessor count), asynchronously on stream; time it with events to get
 * the streaming-read rate that ls_loop_step's HBM roofline is compared against.  bytes must be
 * a positive multiple of n_workgroups * 2 KiB (else LS_ERR_INVALID); LS_ERR_HIP if the launch
 * fails.  No workspace, no model. */
ls_status ls_measure_stream_read(const void *src, size_t bytes, int n_workgroups, hipStream_t stream);

/* Host-side Philox4x32-10 (Salmon et al., SC'11): word 0 of the block for key
 * (seed mod 2^32, seed >> 32) and counter (pos, purpose, 0, 0).  Fills out[i] for
 * purposes purposes[i]; used by the scheduler to build the uniform rows of ls_verify. */
void ls_philox_uniforms(uint64_t seed, int64_t pos, const int32_t *purposes, int n, uint32_t *out);

#ifdef __cplusplus
}
#endif
#endif /* LOOPSPEC_H */
