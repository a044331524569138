/*
 * dsa.h - C ABI of libdsa: decode-step diagonal-aware sparse attention and its
 * dense comparison point, on AMD MI355X (gfx950).
 *
 * The operation is Algorithm 1 ("Diagonal-Aware Sparse Attention") of
 * "Understanding and Exploiting Diagonal Attention Sparsity in Autoregressive
 * Image Generation" (arxiv 2609.19702, Section 4), for every (sequence, head)
 * lane of one transformer layer; one state per layer.  Per decode step t every
 * lane attends its whole prompt KV (L_p rows) plus N_att of the last N_r
 * decode entries; the skipped set grows by one lowest-score entry per step
 * during phase 2 and moves +1 along the attention diagonal every step; once
 * t >= N_r the oldest decode entry is evicted (Section 4, "Detailed
 * explanation").  sink = 4 selects the Diagonal+Sink4 variant (Section 5.1,
 * "Our methods"): decode positions 0..3 stay attended for good and the
 * algorithm runs on the rest with budgets N_r - 4 and N_att - 4.
 *
 * Conventions
 *   - Lanes: lane = b * heads + h.  All lanes of a state share the step t.
 *   - Tensors passed per step are device pointers, row-major [batch][heads][head_dim]
 *     in the state's KV dtype (q, k, v; bf16 for DSA_MXFP8) or fp32 (out).  The prompt is
 *     [batch][L_p][heads][head_dim].  Pointers must be 16-byte aligned.
 *   - Softmax scale is 1 / sqrt(head_dim); one softmax over prompt + selected
 *     decode rows; accumulation in fp32, the raw q.k logits in fp64.
 *   - Argmin: the lowest raw logit q.k among the attended non-sink window
 *     entries of the step (the current token included); ties go to the lowest
 *     decode position.  Selections happen at t = N_att-1 .. N_r-2.
 *   - Memory: the caller owns the device workspace (size from the
 *     *_workspace_bytes call, 256-byte aligned) and every tensor.  The library
 *     owns only the small host handle, freed by dsa_state_destroy.
 *   - Execution: every call is asynchronous on the state's HIP stream, except
 *     dsa_read_state, which synchronises it.  Arguments are checked on the host
 *     before anything is enqueued; a failing call returns a negative dsa_status,
 *     leaves the state unchanged and enqueues nothing.  dsa_last_error() gives
 *     a message for the calling thread's last failure.
 *   - Order: *_append_prompt once; then for each step one *_append_kv followed
 *     by one *_decode_step.  Anything else returns DSA_E_ORDER.
 *   - dsa_append_kv / dense_append_kv record the pointers only; the following
 *     decode step writes the new row into the cache (overwriting the evicted
 *     entry in phase 3) in the same launch.  k_t and v_t must stay valid until
 *     that step has run on the stream.
 *   - Calls on one state must not run concurrently from several host threads.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dsa_state dsa_state;

typedef enum {
    DSA_OK = 0,
    DSA_E_INVAL = -1,     /* bad argument: sizes, dtype, null or misaligned pointer, capacity */
    DSA_E_ORDER = -2,     /* call out of order (see Order above) */
    DSA_E_WORKSPACE = -3, /* workspace missing, too small or misaligned */
    DSA_E_HIP = -4,       /* the HIP runtime reported an error (detail in dsa_last_error) */
    DSA_E_NOMEM = -5      /* host allocation failed */
} dsa_status;

/*
 * KV dtype of a state.  DSA_F32 / DSA_BF16: q, k, v and the cache in that
 * type.  DSA_MXFP8: q, k, v and the prompt arrive in bf16 and the cache holds
 * MXFP8 rows (OCP Microscaling v1.0: E4M3 elements, one E8M0 power-of-two
 * scale per 32 elements, scale exponent floor(log2(max |v|)) - 8, elements
 * rounded to nearest even and saturated at +-448); every decode row is
 * attended in its quantised form, the current token's included.  The pages
 * call KV quantization stackable with the selection (Section 6) and fix no
 * format.  A row then takes 2 * head_dim bytes of codes instead of 4 * head_dim,
 * plus its 8-byte scale word, kept in a region of its own (one word per cache
 * row, lane-major), so that the codes of a row fill whole 64-byte segments.
 * The *_init calls of DSA_MXFP8 states clear the workspace's cache rows on
 * the state's stream (hipMemsetAsync), so whatever the workspace held before
 * never reaches the attention; the other dtypes enqueue nothing at init.
 */
typedef enum { DSA_F32 = 0, DSA_BF16 = 1, DSA_MXFP8 = 2 } dsa_dtype;

/* Largest N_att - sink the sparse kernel supports (its index list lives in LDS). */
#define DSA_MAX_ATTEND 8192

/*
 * Device workspace bytes of a sparse state: per lane a cache of L_p prompt
 * rows plus an N_r-entry ring of decode rows (each row K then V, head_dim
 * elements each), which is the footprint bound N_r + L_p of Section 4 "Cost
 * analysis", plus the per-lane list of attended window offsets, plus the
 * records of split launches (dsa_set_splits: up to 4 records of
 * 4 * (head_dim + 8) bytes per lane, and one arrival counter per lane).
 * Returns 0 when the parameters are invalid (same rules as dsa_state_init).
 */
size_t dsa_state_workspace_bytes(int batch, int L_p, int N_r, int N_att, int heads, int head_dim, int sink,
                                 int dtype);

/*
 * Create a sparse state.  Parameters: batch >= 1, heads >= 1, head_dim in
 * {64, 128}, L_p >= 0, 1 <= N_att <= N_r <= 32767, sink in {0, 4} (sink = 4
 * needs N_att >= 5), N_att - sink <= DSA_MAX_ATTEND, dtype a dsa_dtype.
 * d_workspace: device memory of at least dsa_state_workspace_bytes(...) bytes,
 * 256-byte aligned, owned by the caller and used by this state alone until
 * destroy.  hip_stream: the hipStream_t every call of this state enqueues on
 * (NULL = the null stream).  On success *out receives the handle.
 */
int dsa_state_init(dsa_state** out, int batch, int L_p, int N_r, int N_att, int heads, int head_dim, int sink,
                   int dtype, void* d_workspace, size_t workspace_bytes, void* hip_stream);

/*
 * KV-selection policies.  DIAGONAL and DIAGONAL_SINK4 are Algorithm 1 and its
 * Diagonal+Sink4 variant (the states dsa_state_init makes).  The others are
 * the baselines the pages compare against, under the same budget accounting
 * (prompt always attended; N_att decode entries attended per step once that
 * many exist, the current token included):
 *   SLIDING_WINDOW - the N_att most recent decode positions (Section 2.3 (2));
 *   STREAMING_LLM  - decode positions 0..3 as attention sinks plus the
 *                    N_att - 4 most recent ones (Section 2.3 (2); Section 5.1
 *                    "Sparse KV baselines": the first 4 decode tokens are the
 *                    sinks since the prompt is kept whole);
 *   TOVA           - a cache of N_att entries; once step t has filled it, the
 *                    entry with the lowest logit q_t . k (the lowest score of
 *                    this step's query; the current token included) leaves
 *                    it, the lowest position among equals (Section 2.3 (3));
 *   H2O            - a cache of N_att entries whose N_r most recent positions
 *                    are protected; every entry accumulates its softmax
 *                    probability (over prompt + cache) at each step it is
 *                    attended, and once step t has filled the cache the
 *                    unprotected entry with the lowest accumulated score
 *                    leaves it, the lowest position among equals (Section 2.3
 *                    (3)).  Scores and their probabilities are fp64.
 * SLIDING_WINDOW and STREAMING_LLM run as Algorithm 1 with a ring of N_att
 * entries (it never selects); TOVA and H2O run on their own kernel modes.
 */
typedef enum {
    DSA_POLICY_DIAGONAL = 0,
    DSA_POLICY_DIAGONAL_SINK4 = 1,
    DSA_POLICY_SLIDING_WINDOW = 2,
    DSA_POLICY_STREAMING_LLM = 3,
    DSA_POLICY_TOVA = 4,
    DSA_POLICY_H2O = 5
} dsa_policy;

/* Largest L_p + N_att of an H2O state (one fp64 logit per attended row lives in LDS). */
#define DSA_MAX_H2O_ROWS 4096

/*
 * Device workspace bytes of a state of the given policy; 0 when the parameters
 * are invalid (same rules as dsa_policy_state_init).  N_r is the ring (DIAGONAL,
 * DIAGONAL_SINK4), must equal N_att (SLIDING_WINDOW, STREAMING_LLM, TOVA), or is
 * H2O's protected recent count in [1, N_att - 1].  TOVA / H2O workspaces hold
 * per lane L_p + N_att cache rows, the slot metadata (N_att + 4 int32) and, for
 * H2O, N_att fp64 scores.
 */
size_t dsa_policy_workspace_bytes(int policy, int batch, int L_p, int N_r, int N_att, int heads, int head_dim,
                                  int dtype);

/*
 * Create a state of the given policy; otherwise as dsa_state_init (no sink
 * argument: the policy fixes it).  N_att <= DSA_MAX_ATTEND for TOVA and H2O,
 * L_p + N_att <= DSA_MAX_H2O_ROWS for H2O.  The state takes the dsa_ calls:
 * dsa_append_prompt, dsa_append_kv, dsa_decode_step, dsa_read_state.  For TOVA
 * and H2O the trace of dsa_decode_step is (position that leaves the cache after
 * this step or -1, -1), and dsa_read_state lists N_att offsets per lane (the
 * cached entries the next step attends, with offset 0 for the next token).
 */
int dsa_policy_state_init(dsa_state** out, int policy, int batch, int L_p, int N_r, int N_att, int heads,
                          int head_dim, int dtype, void* d_workspace, size_t workspace_bytes, void* hip_stream);

/* Change the stream later calls enqueue on. */
int dsa_set_stream(dsa_state* st, void* hip_stream);

/*
 * Copy the prompt KV (Algorithm 1 input K_p, V_p), [batch][L_p][heads][head_dim]
 * each, into the state's cache.  Must be the first call after init; with
 * L_p = 0 the pointers may be NULL.
 */
int dsa_append_prompt(dsa_state* st, const void* k_p, const void* v_p);

/* Record the step's new key and value rows, [batch][heads][head_dim] each. */
int dsa_append_kv(dsa_state* st, const void* k_t, const void* v_t);

/*
 * One decode step t of Algorithm 1 for all lanes, in one kernel launch: write
 * the appended row into the ring (evicting t - N_r in phase 3), gather the
 * prompt rows and the attended window rows, softmax attention into
 * out [batch][heads][head_dim] (fp32), and during t in [N_att-1, N_r-2] pick
 * the window entry with the lowest logit and add it to the skip set (it is
 * skipped from step t+1 on).  q_t: [batch][heads][head_dim] in the KV dtype.
 * trace (nullable, device): [batch][heads][2] int32 = (position selected at
 * this step or -1, position evicted at this step or -1).  Advances t by one.
 */
int dsa_decode_step(dsa_state* st, const void* q_t, float* out, int32_t* trace);

/*
 * dsa_append_kv followed by dsa_decode_step, in one call (same arguments,
 * checks and effects; nothing is recorded if either check fails).  For
 * callers that enqueue many small launches and pay per call.
 */
int dsa_append_decode_step(dsa_state* st, const void* k_t, const void* v_t, const void* q_t, float* out,
                           int32_t* trace);

/*
 * Copy the lane state to the host; synchronises the stream.  h_t receives the
 * index of the next step.  h_offsets ([batch*heads][N_att - sink], nullable)
 * receives, per lane, the window entries the next step will attend, as
 * offsets t - position in ascending order, padded with -1; h_count
 * ([batch*heads], nullable) their number.  Sinks are not listed.
 */
int dsa_read_state(const dsa_state* st, int32_t* h_t, int16_t* h_offsets, int32_t* h_count);

/* Device workspace bytes of a dense state holding L_p + L_max rows per lane; 0 if invalid. */
size_t dense_state_workspace_bytes(int batch, int L_p, int L_max, int heads, int head_dim, int dtype);

/*
 * Create a dense state ("No sparsity", Section 2.3 (1)): step t attends every
 * prompt row and decode positions 0..t.  L_max >= 1 is the number of decode
 * steps the cache holds.  Other parameters as dsa_state_init.
 */
int dense_state_init(dsa_state** out, int batch, int L_p, int L_max, int heads, int head_dim, int dtype,
                     void* d_workspace, size_t workspace_bytes, void* hip_stream);

/* Prompt and per-step rows of a dense state: same contracts as the dsa_ calls. */
int dense_append_prompt(dsa_state* st, const void* k_p, const void* v_p);
int dense_append_kv(dsa_state* st, const void* k_t, const void* v_t);

/* One dense decode step: out [batch][heads][head_dim] fp32.  Fails with
 * DSA_E_INVAL once L_max steps have run. */
int dense_decode_step(dsa_state* st, const void* q_t, float* out);

/* dense_append_kv followed by dense_decode_step, in one call. */
int dense_append_decode_step(dsa_state* st, const void* k_t, const void* v_t, const void* q_t, float* out);

/*
 * Workgroup size of the decode kernels, in 64-wide wavefronts per lane:
 * 1, 2, 4, 8 or 16, or 0 for the library's choice (DSA_MXFP8 states use at
 * most 8).  Results do not depend on it except for fp32 rounding order in
 * the softmax sums.
 */
int dsa_set_waves(dsa_state* st, int waves_per_lane);

/*
 * Workgroups per lane of a sparse state's decode launches: 1, 2 or 4, or 0
 * for the library's choice.  With n > 1, workgroup s of a lane takes the
 * s-th of n contiguous slices of the lane's attended rows (prompt, sinks,
 * window entries) and leaves its partial softmax state (m, l, acc) and argmin
 * candidate in the workspace; the last of the lane's workgroups to finish
 * (a per-lane arrival counter; no workgroup waits) merges the n records in
 * slice order and performs the output, the state update and the append.  This
 * is the split combine of a lane's attention (the pages fuse the whole step
 * into one kernel, Section 5.1).  Choices, evictions and offsets do not depend
 * on n (the argmin order is total); outputs only through fp32 rounding order.
 * Only states with bf16 or fp32 rows split: DSA_MXFP8 and the dense, TOVA and
 * H2O states accept 0 or 1.  The first split launch of a state is preceded
 * by a small kernel that zeroes the counters; every split launch leaves them
 * at zero.  Two launches of one state must not overlap (they share the
 * counters), which the state's single stream ensures.
 */
int dsa_set_splits(dsa_state* st, int splits_per_lane);

/*
 * Attention-map characterization (Section 3.4 of the pages: Fig. 8, attention
 * mass on prompt / local / middle tokens; Fig. 10, vertical vs diagonal
 * cosine similarity of attention score vectors), on the dense decode map of
 * T decode steps: query t attends the prompt and decode positions 0..t, one
 * softmax with scale 1 / sqrt(head_dim).  Per lane (b * heads + h):
 *   mass [lanes][3]  - mean over queries of the mass on the prompt, on the
 *                      local tokens (the ceil((t + 1) / 10) most recent
 *                      decoded tokens, the current one included) and on the
 *                      other decoded tokens;
 *   vert, diag [lanes][max_dist] - for d = 1..max_dist, the mean over
 *                      i in [0, T - d) of cos(P[i][0..i], P[i+d][0..i]) and
 *                      of cos(P[i][0..i], P[i+d][d..i+d]), P the decode
 *                      probabilities (prompt columns left out).
 * q, k: [T][batch][heads][head_dim], k_p: [batch][L_p][heads][head_dim], in
 * dtype DSA_F32 or DSA_BF16, 16-byte aligned.  Outputs: device fp64 arrays,
 * 8-byte aligned.  1 <= max_dist <= min(T - 1, 256).  The workspace (size
 * from dsa_profile_workspace_bytes, 256-byte aligned) holds the fp32 map
 * [lanes][T][T], the per-query mass and per-tile sums; it is the caller's.
 * Asynchronous on hip_stream (NULL = null stream).  The logits and the
 * similarity dot products are MFMA tiles with fp32 sums; the means are fp64.
 */
size_t dsa_profile_workspace_bytes(int batch, int heads, int L_p, int T, int max_dist);
int dsa_attention_profile(const void* q, const void* k, const void* k_p, int batch, int heads, int head_dim, int L_p,
                          int T, int dtype, int max_dist, void* d_workspace, size_t workspace_bytes, double* mass,
                          double* vert, double* diag, void* hip_stream);

/*
 * dsa_attention_profile without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc): the same computation, arguments and
 * outputs, with the scratch (the map, the per-query mass and the per-tile
 * sums, dsa_profile_workspace_bytes(...) bytes) taken from a static device
 * array of DSA_PROFILE_STATIC_SCRATCH_BYTES that the library holds on each GPU
 * it runs on until the process ends.  A profile that needs more scratch
 * fails with DSA_E_WORKSPACE and launches nothing (64 MiB holds, e.g., one
 * sequence of 32 heads over 576 decode steps).  The call allocates nothing;
 * its first call on a device looks up that device's copy of the array (the
 * stream must belong to the current device).  Every call on one GPU shares
 * that GPU's copy: calls that overlap on one GPU (several streams, or several
 * host threads) race on it and must be serialised by the caller; one stream
 * orders them by itself.  No part of the scratch needs to start at zero.
 */
#define DSA_PROFILE_STATIC_SCRATCH_BYTES (64u << 20)
int dsa_attention_profile_static(const void* q, const void* k, const void* k_p, int batch, int heads, int head_dim,
                                 int L_p, int T, int dtype, int max_dist, double* mass, double* vert, double* diag,
                                 void* hip_stream);

/*
 * HBM read probe (a measurement utility, not part of the method): streams
 * `bytes` from src once with 16-byte non-temporal loads, grid-stride over
 * `blocks` workgroups of `threads`, `unroll` loads in flight per thread, the
 * way the decode kernels stream their cache rows.  Gives the practical read
 * ceiling of the device that the decode kernels' bandwidth is read against.
 * src: device, 16-byte aligned, bytes a positive multiple of 16.  sink: one
 * device uint32, written only if a thread's XOR of the words it read equals
 * 0x9e3779b9 (which keeps the loads from being optimised out).  blocks in
 * [1, 65536]; threads a multiple of 64 in [64, 1024]; unroll 1, 4 or 8.
 * Asynchronous on hip_stream; DSA_E_INVAL on bad arguments (nothing launched).
 */
int dsa_hbm_read_probe(const void* src, size_t bytes, int blocks, int threads, int unroll, uint32_t* sink,
                       void* hip_stream);

/* Next step index of a sparse or dense state (or a negative dsa_status). */
int dsa_state_step(const dsa_state* st);

/* Free the host handle (the workspace stays the caller's).  NULL is a no-op. */
int dsa_state_destroy(dsa_state* st);

/* Static name of a dsa_status code. */
const char* dsa_strerror(int code);

/* Message of the calling thread's last failed call ("" if none). */
const char* dsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
