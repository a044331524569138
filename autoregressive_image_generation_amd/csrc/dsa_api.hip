// C ABI of libdsa (declared in include/dsa.h): state sizing and validation,
// the per-step resolution of Algorithm 1's phases (page 4, Section 4), and the
// launches.  Every check runs on the host before anything is enqueued, so a
// failing call has no side effects.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "../../include/dsa.h"
#include "dsa_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(DSA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// SPARSE: Algorithm 1 and its equal-budget cases (SlidingWindow,
// StreamingLLM); DENSE: no sparsity; SCORE: TOVA and H2O over N_att slots.
enum Kind { KIND_SPARSE = 1, KIND_DENSE = 2, KIND_SCORE = 3 };

}  // namespace

struct dsa_state {
    int kind;
    int policy;  // dsa_policy
    int batch, heads, D, L_p, N_r, N_att, S, dtype, L_max;
    int lanes, N_rw, N_attw, list_stride;
    long long lane_rows;
    long long scale_rows;  // MXFP8: scale words per lane (the lane's cache rows)
    size_t scale_off;      // MXFP8: byte offset of the scale-word region (right after the cache rows)
    char* ws;
    size_t ws_bytes;
    size_t list_off;
    size_t ring_off;  // sparse: byte offset of the ring region
    hipStream_t stream;
    int t;
    int prompt_done;
    const void* pend_k;
    const void* pend_v;
    int waves;
    int splits;               // sparse: workgroups per lane requested (0 = the library's choice)
    size_t part_off, ctr_off;  // sparse: split records and per-lane arrival counters
    int counters_clear;       // sparse: the counters were zeroed (before the first split launch)
    int prompt_slot_major;    // sparse: the prompt region is [L_p][lanes] rows (else [lanes][L_p])
    // SCORE states: per-lane slot metadata and (H2O) accumulated scores
    size_t meta_off, score_off;
    int meta_stride, score_stride, n_recent;
};

namespace {

// Bytes of one cache row (K then V): plain elements, or MXFP8 codes (the
// row's 8-byte word of E8M0 block scales is kept in a region of its own).
size_t row_bytes(int D, int dtype) {
    return dtype == DSA_MXFP8 ? (size_t)2 * D : (size_t)2 * D * (dtype == DSA_BF16 ? 2 : 4);
}

// MXFP8 states: one 8-byte scale word per cache row, [lanes][rows per lane].
size_t scale_bytes(long long lanes, long long rows, int dtype) {
    return dtype == DSA_MXFP8 ? ((size_t)lanes * (size_t)rows * 8 + 255) / 256 * 256 : 0;
}

// Per-lane list entries, padded so every lane's list starts on 16 bytes.
int list_stride_for(int n) { return (n + 7) / 8 * 8; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Common shape checks; returns 0 or a status with the message set.
int check_common(int batch, int L_p, int heads, int head_dim, int dtype) {
    if (batch < 1) return fail(DSA_E_INVAL, "batch must be >= 1 (got %d)", batch);
    if (heads < 1) return fail(DSA_E_INVAL, "heads must be >= 1 (got %d)", heads);
    if (head_dim != 64 && head_dim != 128) return fail(DSA_E_INVAL, "head_dim must be 64 or 128 (got %d)", head_dim);
    if (L_p < 0) return fail(DSA_E_INVAL, "L_p must be >= 0 (got %d)", L_p);
    if (dtype != DSA_F32 && dtype != DSA_BF16 && dtype != DSA_MXFP8)
        return fail(DSA_E_INVAL, "dtype must be DSA_F32, DSA_BF16 or DSA_MXFP8");
    if ((long long)batch * heads > (1ll << 30)) return fail(DSA_E_INVAL, "batch * heads too large");
    return 0;
}

int check_sparse(int batch, int L_p, int N_r, int N_att, int heads, int head_dim, int sink, int dtype) {
    int rc = check_common(batch, L_p, heads, head_dim, dtype);
    if (rc) return rc;
    if (sink != 0 && sink != 4) return fail(DSA_E_INVAL, "sink must be 0 or 4 (got %d)", sink);
    if (N_att < 1) return fail(DSA_E_INVAL, "N_att must be >= 1 (got %d)", N_att);
    if (N_r < N_att) return fail(DSA_E_INVAL, "N_r (%d) must be >= N_att (%d)", N_r, N_att);
    if (N_r > 32767) return fail(DSA_E_INVAL, "N_r must be <= 32767 (got %d)", N_r);
    if (sink && N_att <= sink) return fail(DSA_E_INVAL, "sink = %d needs N_att > %d (got %d)", sink, sink, N_att);
    if (N_att - sink > DSA_MAX_ATTEND)
        return fail(DSA_E_INVAL, "N_att - sink must be <= %d (got %d)", DSA_MAX_ATTEND, N_att - sink);
    return 0;
}

size_t kv_bytes(long long lanes, long long lane_rows, int D, int dtype) {
    return align_up((size_t)lanes * (size_t)lane_rows * row_bytes(D, dtype));
}

// Sparse states: the records of split launches (up to kMaxSplits per lane).
size_t split_rec_bytes(long long lanes, int D) {
    return align_up((size_t)lanes * dsa::kMaxSplits * dsa::split_rec_floats(D) * sizeof(float));
}
size_t counter_bytes(long long lanes) { return align_up((size_t)lanes * sizeof(int32_t)); }

int check_workspace(void* ws, size_t have, size_t need) {
    if (!ws) return fail(DSA_E_WORKSPACE, "workspace pointer is NULL");
    if ((uintptr_t)ws % kAlign) return fail(DSA_E_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
    if (have < need) return fail(DSA_E_WORKSPACE, "workspace has %zu bytes, needs %zu", have, need);
    return 0;
}

const char* kind_name(int kind) {
    return kind == KIND_SPARSE ? "sparse" : kind == KIND_DENSE ? "dense" : "score-policy";
}

int check_state(const dsa_state* st, int kind, int kind2 = -1) {
    if (!st) return fail(DSA_E_INVAL, "state is NULL");
    if (kind && st->kind != kind && st->kind != kind2) return fail(DSA_E_INVAL, "state is a %s state", kind_name(st->kind));
    return 0;
}

// MXFP8 states: clear the cache rows on the state's stream, so that every
// row the kernel reads holds zeros or codes the quantiser wrote (finite
// values, scale bytes below 0xFF), including rows no token has reached yet.
int clear_mx_rows(dsa_state* st, size_t kv_region_bytes) {
    if (st->dtype != DSA_MXFP8) return DSA_OK;
    hipError_t e = hipMemsetAsync(st->ws, 0, kv_region_bytes, st->stream);
    return e == hipSuccess ? DSA_OK : hip_fail(e, "MXFP8 cache clear");
}

// Score-policy (TOVA / H2O) sizes: [0] free slot, [4 + j] slot positions, in
// 16-byte chunks; the H2O logits of one lane live in LDS next to them.
int meta_stride_for(int N_att) { return (4 + N_att + 3) / 4 * 4; }
int score_stride_for(int N_att) { return (N_att + 1) / 2 * 2; }
constexpr int kMaxH2oRows = DSA_MAX_H2O_ROWS;

// Prompt region layout of sparse states.  From this many lanes on, every lane
// has one wavefront (choose_waves: lanes * 2 >= 3072), whose four thread groups
// read four rows of the lane at a time while thousands of lanes read the same
// prompt rows: with the rows of one prompt position side by side ([L_p][lanes])
// those reads meet in fewer DRAM pages.  Measured on MI355X (full decodes, the
// two layouts alternating, fraction of 8 TB/s): Janus-Pro-7B two streams (1536
// lanes per launch) 0.843 against 0.821, one stream (3072) 0.702 / 0.704; with
// fewer lanes and several wavefronts per lane, whose groups read many rows of
// one lane at a time, [lanes][L_p] keeps them together: Lumina 1024^2 two
// streams (256 lanes x 8 wavefronts) 0.739 against 0.715 slot-major.  MXFP8
// rows (256 bytes) stay lane-major: slot-major measured 1-3 % slower there.
constexpr int kSlotMajorPromptLanes = 1536;

// Wavefronts per workgroup.  Measured on MI355X: the decode is fastest with
// one to three thousand wavefronts per launch in total (one workgroup per
// lane), so waves doubles while lanes * waves stays below 3072, every thread
// group keeps at least its pipeline depth of rows (dsa::rows_in_flight) of
// work, and the workgroup stays at 8 wavefronts or fewer (16 was slower at
// every measured shape).  Always 1, 2, 4, 8 or 16 (dsa_set_waves accepts no
// other count): the kernel's merges across wavefronts are instantiated for
// those counts only.
int choose_waves(const dsa_state* st, long long rows, int splits = 1) {
    const int max_w = st->dtype == DSA_MXFP8 ? 8 : 16;  // MXFP8 workgroups stop at 8 wavefronts
    if (st->waves) return std::min(st->waves, max_w);
    const int ept = st->dtype == DSA_F32 ? 4 : st->dtype == DSA_MXFP8 ? 16 : 8;  // elements per thread
    const int gpw = 64 / (st->D / ept);
    const long long wgs = (long long)st->lanes * splits;  // workgroups per launch
    const long long per = (rows + splits - 1) / splits;   // rows per workgroup
    int w = 1;
    while (w < 8 && wgs * (2 * w) < 3072 && per >= (long long)dsa::rows_in_flight(wgs, 2 * w) * gpw * (2 * w)) w *= 2;
    return w;
}

// Workgroups per lane of a sparse launch: the state's request, or 1.  Only
// plain-row (bf16 / fp32) sparse states split.
int choose_splits(const dsa_state* st) {
    if (st->kind != KIND_SPARSE || st->dtype == DSA_MXFP8) return 1;
    return st->splits ? st->splits : 1;
}

int launch_prompt(dsa_state* st, const void* k_p, const void* v_p) {
    if (st->prompt_done) return fail(DSA_E_ORDER, "prompt already appended");
    if (st->L_p > 0) {
        if (!k_p || !v_p) return fail(DSA_E_INVAL, "prompt pointers are NULL");
        if (!aligned16(k_p) || !aligned16(v_p)) return fail(DSA_E_INVAL, "prompt pointers must be 16-byte aligned");
    }
    const bool init_list = st->kind == KIND_SPARSE && st->S == 0;  // score states need no initial data
    if (st->L_p > 0 || init_list) {
        dsa::PromptArgs a;
        a.k_p = k_p;
        a.v_p = v_p;
        a.kv = st->ws;
        a.list = init_list ? reinterpret_cast<int16_t*>(st->ws + st->list_off) : nullptr;
        a.counter = nullptr;
        a.lane_rows = st->lane_rows;
        a.slot_major = st->prompt_slot_major;
        a.scales = st->ws + st->scale_off;
        a.scale_rows = st->scale_rows;
        a.B = st->batch;
        a.H = st->heads;
        a.L_p = st->L_p;
        a.list_stride = st->list_stride;
        hipError_t e = dsa::launch_prompt(st->dtype, st->D, a, st->stream);
        if (e != hipSuccess) return hip_fail(e, "prompt copy launch");
    }
    st->prompt_done = 1;
    return DSA_OK;
}

int record_kv(dsa_state* st, const void* k_t, const void* v_t) {
    if (!st->prompt_done) return fail(DSA_E_ORDER, "append the prompt first");
    if (st->pend_k) return fail(DSA_E_ORDER, "a row is already appended for step %d", st->t);
    if (st->kind == KIND_DENSE && st->t >= st->L_max)
        return fail(DSA_E_INVAL, "dense cache full (L_max = %d)", st->L_max);
    if (!k_t || !v_t) return fail(DSA_E_INVAL, "k_t / v_t is NULL");
    if (!aligned16(k_t) || !aligned16(v_t)) return fail(DSA_E_INVAL, "k_t / v_t must be 16-byte aligned");
    st->pend_k = k_t;
    st->pend_v = v_t;
    return DSA_OK;
}

int check_step(const dsa_state* st, const void* q_t, const float* out) {
    if (!st->prompt_done) return fail(DSA_E_ORDER, "append the prompt first");
    if (!st->pend_k) return fail(DSA_E_ORDER, "append the step's K/V before decoding step %d", st->t);
    if (!q_t || !out) return fail(DSA_E_INVAL, "q_t / out is NULL");
    if (!aligned16(q_t) || !aligned16(out)) return fail(DSA_E_INVAL, "q_t / out must be 16-byte aligned");
    if (st->t == 0x7fffffff) return fail(DSA_E_INVAL, "step counter exhausted");
    return 0;
}

void fill_common(const dsa_state* st, const void* q_t, float* out, dsa::DecodeArgs& a) {
    memset(&a, 0, sizeof(a));
    a.kv = st->ws;
    a.q = q_t;
    a.k_new = st->pend_k;
    a.v_new = st->pend_v;
    a.out = out;
    a.lane_rows = st->lane_rows;
    a.scales = st->ws + st->scale_off;
    a.scale_rows = st->scale_rows;
    a.lanes = st->lanes;
    const long long rb = (long long)row_bytes(st->D, st->dtype);
    a.prompt_row_bytes = st->prompt_slot_major ? (long long)st->lanes * rb : rb;
    a.prompt_lane_bytes = st->prompt_slot_major ? rb : st->lane_rows * rb;
    a.L_p = st->L_p;
    a.t = st->t;
    a.scale_log2e = 1.4426950408889634 / sqrt((double)st->D);
    a.splits = 1;
}

// Map a dsa_policy onto a state kind.  Diagonal (with or without sinks)
// takes N_r as given; SlidingWindow and StreamingLLM are Algorithm 1 with the
// ring as long as the attended budget (no selection ever happens), so N_r must
// equal N_att; TOVA keeps N_att slots and N_r must equal N_att too; H2O keeps
// N_att slots of which the N_r most recent positions are protected.
int resolve_policy(int policy, int N_r, int N_att, int* kind, int* sink) {
    switch (policy) {
        case DSA_POLICY_DIAGONAL: *kind = KIND_SPARSE; *sink = 0; return 0;
        case DSA_POLICY_DIAGONAL_SINK4: *kind = KIND_SPARSE; *sink = 4; return 0;
        case DSA_POLICY_SLIDING_WINDOW:
        case DSA_POLICY_STREAMING_LLM:
        case DSA_POLICY_TOVA:
            if (N_r != N_att) return fail(DSA_E_INVAL, "this policy keeps N_att entries: N_r (%d) must equal N_att (%d)", N_r, N_att);
            *kind = policy == DSA_POLICY_TOVA ? KIND_SCORE : KIND_SPARSE;
            *sink = policy == DSA_POLICY_STREAMING_LLM ? 4 : 0;
            return 0;
        case DSA_POLICY_H2O:
            if (N_r < 1 || N_r >= N_att)
                return fail(DSA_E_INVAL, "H2O: the protected recent count N_r (%d) must be in [1, N_att - 1] (N_att = %d)", N_r, N_att);
            *kind = KIND_SCORE;
            *sink = 0;
            return 0;
        default: return fail(DSA_E_INVAL, "unknown policy %d", policy);
    }
}

int check_score(int policy, int batch, int L_p, int N_att, int heads, int head_dim, int dtype) {
    int rc = check_common(batch, L_p, heads, head_dim, dtype);
    if (rc) return rc;
    if (N_att < 1 || N_att > DSA_MAX_ATTEND) return fail(DSA_E_INVAL, "N_att must be in [1, %d] (got %d)", DSA_MAX_ATTEND, N_att);
    if (policy == DSA_POLICY_H2O && (long long)L_p + N_att > kMaxH2oRows)
        return fail(DSA_E_INVAL, "H2O needs L_p + N_att <= %d (got %lld)", kMaxH2oRows, (long long)L_p + N_att);
    return 0;
}

size_t score_workspace_bytes(int policy, int batch, int L_p, int N_att, int heads, int head_dim, int dtype) {
    const long long lanes = (long long)batch * heads;
    size_t b = kv_bytes(lanes, (long long)L_p + N_att, head_dim, dtype) +
               scale_bytes(lanes, (long long)L_p + N_att, dtype) +
               align_up((size_t)lanes * (size_t)meta_stride_for(N_att) * sizeof(int32_t));
    if (policy == DSA_POLICY_H2O) b += align_up((size_t)lanes * (size_t)score_stride_for(N_att) * sizeof(double));
    return b;
}

int score_decode(dsa_state* st, const void* q_t, float* out, int32_t* trace) {
    dsa::DecodeArgs a;
    fill_common(st, q_t, out, a);
    const int t = st->t, N = st->N_att;
    a.trace = trace;
    a.meta = reinterpret_cast<int32_t*>(st->ws + st->meta_off);
    a.score = st->policy == DSA_POLICY_H2O ? reinterpret_cast<double*>(st->ws + st->score_off) : nullptr;
    a.meta_stride = st->meta_stride;
    a.score_stride = st->score_stride;
    a.N_cache = N;
    a.n_occ = std::min(t, N - 1);
    a.n_meta = 4 + std::min(t, N);
    a.free_host = t < N ? t : -1;  // while the cache fills, token t takes slot t
    a.select = t >= N - 1 ? 1 : 0;  // the cache is full once token t is in it
    a.n_recent = st->n_recent;
    a.inv_sqrt_d = 1.0 / sqrt((double)st->D);
    a.evicted = -1;
    const int waves = choose_waves(st, (long long)st->L_p + std::min(t + 1, N));
    const int mode = st->policy == DSA_POLICY_H2O ? dsa::MODE_H2O : dsa::MODE_TOVA;
    hipError_t e = dsa::launch_decode(mode, st->dtype, st->D, waves, a, st->stream);
    if (e != hipSuccess) return hip_fail(e, "score-policy decode launch");
    st->pend_k = st->pend_v = nullptr;
    st->t += 1;
    return DSA_OK;
}

// Attended-entry offsets of the next step of a score state, read from the slot metadata.
int score_read_state(const dsa_state* st, int16_t* h_offsets, int32_t* h_count) {
    const int tn = st->t, N = st->N_att;
    std::vector<int32_t> buf;
    try {
        buf.resize((size_t)st->lanes * st->meta_stride);
    } catch (...) {
        return fail(DSA_E_NOMEM, "host allocation failed");
    }
    hipError_t e = hipStreamSynchronize(st->stream);
    if (e != hipSuccess) return hip_fail(e, "stream synchronize");
    e = hipMemcpy(buf.data(), st->ws + st->meta_off, buf.size() * sizeof(int32_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "slot metadata copy");
    const int occ = std::min(tn, N);  // slots holding a position before step tn
    std::vector<int> offs;
    for (int l = 0; l < st->lanes; ++l) {
        const int32_t* m = buf.data() + (size_t)l * st->meta_stride;
        const int free_slot = tn < N ? tn : m[0];
        offs.clear();
        offs.push_back(0);  // the next token itself
        for (int j = 0; j < occ; ++j)
            if (j != free_slot) offs.push_back(tn - m[4 + j]);
        std::sort(offs.begin(), offs.end());
        if (h_offsets) {
            int16_t* dst = h_offsets + (size_t)l * N;
            for (int j = 0; j < N; ++j) dst[j] = j < (int)offs.size() ? (int16_t)std::min(offs[j], 32767) : (int16_t)-1;
        }
        if (h_count) h_count[l] = (int)offs.size();
    }
    return DSA_OK;
}

}  // namespace

extern "C" {

size_t dsa_state_workspace_bytes(int batch, int L_p, int N_r, int N_att, int heads, int head_dim, int sink,
                                 int dtype) {
    if (check_sparse(batch, L_p, N_r, N_att, heads, head_dim, sink, dtype)) return 0;
    const long long lanes = (long long)batch * heads;
    return kv_bytes(lanes, (long long)L_p + N_r, head_dim, dtype) + scale_bytes(lanes, (long long)L_p + N_r, dtype) +
           align_up((size_t)lanes * (size_t)list_stride_for(N_att - sink) * sizeof(int16_t)) +
           split_rec_bytes(lanes, head_dim) + counter_bytes(lanes);
}

int dsa_state_init(dsa_state** out, int batch, int L_p, int N_r, int N_att, int heads, int head_dim, int sink,
                   int dtype, void* d_workspace, size_t workspace_bytes, void* hip_stream) {
    if (!out) return fail(DSA_E_INVAL, "out handle pointer is NULL");
    int rc = check_sparse(batch, L_p, N_r, N_att, heads, head_dim, sink, dtype);
    if (rc) return rc;
    const size_t need = dsa_state_workspace_bytes(batch, L_p, N_r, N_att, heads, head_dim, sink, dtype);
    rc = check_workspace(d_workspace, workspace_bytes, need);
    if (rc) return rc;
    dsa_state* st = new (std::nothrow) dsa_state();
    if (!st) return fail(DSA_E_NOMEM, "host allocation failed");
    st->kind = KIND_SPARSE;
    st->policy = sink ? DSA_POLICY_DIAGONAL_SINK4 : DSA_POLICY_DIAGONAL;
    st->batch = batch;
    st->heads = heads;
    st->D = head_dim;
    st->L_p = L_p;
    st->N_r = N_r;
    st->N_att = N_att;
    st->S = sink;
    st->dtype = dtype;
    st->L_max = 0;
    st->lanes = batch * heads;
    st->N_rw = N_r - sink;
    st->N_attw = N_att - sink;
    st->list_stride = list_stride_for(N_att - sink);
    st->lane_rows = L_p;  // prompt region (rows of L_p per lane); the ring region [N_r][lanes] follows it
    st->prompt_slot_major = st->lanes >= kSlotMajorPromptLanes && dtype != DSA_MXFP8;
    st->ws = static_cast<char*>(d_workspace);
    st->ws_bytes = workspace_bytes;
    st->ring_off = (size_t)st->lanes * (size_t)L_p * row_bytes(head_dim, dtype);
    st->scale_rows = (long long)L_p + N_r;
    st->scale_off = kv_bytes(st->lanes, (long long)L_p + N_r, head_dim, dtype);
    st->list_off = st->scale_off + scale_bytes(st->lanes, st->scale_rows, dtype);
    st->part_off = st->list_off + align_up((size_t)st->lanes * (size_t)st->list_stride * sizeof(int16_t));
    st->ctr_off = st->part_off + split_rec_bytes(st->lanes, head_dim);
    st->stream = static_cast<hipStream_t>(hip_stream);
    rc = clear_mx_rows(st, st->list_off);
    if (rc) {
        delete st;
        return rc;
    }
    *out = st;
    return DSA_OK;
}

size_t dsa_policy_workspace_bytes(int policy, int batch, int L_p, int N_r, int N_att, int heads, int head_dim,
                                  int dtype) {
    int kind, sink;
    if (resolve_policy(policy, N_r, N_att, &kind, &sink)) return 0;
    if (kind == KIND_SPARSE) return dsa_state_workspace_bytes(batch, L_p, N_r, N_att, heads, head_dim, sink, dtype);
    if (check_score(policy, batch, L_p, N_att, heads, head_dim, dtype)) return 0;
    return score_workspace_bytes(policy, batch, L_p, N_att, heads, head_dim, dtype);
}

int dsa_policy_state_init(dsa_state** out, int policy, int batch, int L_p, int N_r, int N_att, int heads,
                          int head_dim, int dtype, void* d_workspace, size_t workspace_bytes, void* hip_stream) {
    if (!out) return fail(DSA_E_INVAL, "out handle pointer is NULL");
    int kind, sink;
    int rc = resolve_policy(policy, N_r, N_att, &kind, &sink);
    if (rc) return rc;
    if (kind == KIND_SPARSE) {
        rc = dsa_state_init(out, batch, L_p, N_r, N_att, heads, head_dim, sink, dtype, d_workspace, workspace_bytes,
                            hip_stream);
        if (rc == DSA_OK) (*out)->policy = policy;
        return rc;
    }
    rc = check_score(policy, batch, L_p, N_att, heads, head_dim, dtype);
    if (rc) return rc;
    rc = check_workspace(d_workspace, workspace_bytes,
                         score_workspace_bytes(policy, batch, L_p, N_att, heads, head_dim, dtype));
    if (rc) return rc;
    dsa_state* st = new (std::nothrow) dsa_state();
    if (!st) return fail(DSA_E_NOMEM, "host allocation failed");
    st->kind = KIND_SCORE;
    st->policy = policy;
    st->batch = batch;
    st->heads = heads;
    st->D = head_dim;
    st->L_p = L_p;
    st->N_r = N_r;
    st->N_att = N_att;
    st->dtype = dtype;
    st->lanes = batch * heads;
    st->lane_rows = (long long)L_p + N_att;
    st->ws = static_cast<char*>(d_workspace);
    st->ws_bytes = workspace_bytes;
    st->meta_stride = meta_stride_for(N_att);
    st->score_stride = score_stride_for(N_att);
    st->scale_rows = st->lane_rows;
    st->scale_off = kv_bytes(st->lanes, st->lane_rows, head_dim, dtype);
    st->meta_off = st->scale_off + scale_bytes(st->lanes, st->scale_rows, dtype);
    st->score_off = st->meta_off + align_up((size_t)st->lanes * (size_t)st->meta_stride * sizeof(int32_t));
    st->n_recent = policy == DSA_POLICY_H2O ? N_r : 0;
    st->stream = static_cast<hipStream_t>(hip_stream);
    rc = clear_mx_rows(st, st->meta_off);
    if (rc) {
        delete st;
        return rc;
    }
    *out = st;
    return DSA_OK;
}

int dsa_set_stream(dsa_state* st, void* hip_stream) {
    int rc = check_state(st, 0);
    if (rc) return rc;
    st->stream = static_cast<hipStream_t>(hip_stream);
    return DSA_OK;
}

int dsa_append_prompt(dsa_state* st, const void* k_p, const void* v_p) {
    int rc = check_state(st, KIND_SPARSE, KIND_SCORE);
    return rc ? rc : launch_prompt(st, k_p, v_p);
}

int dsa_append_kv(dsa_state* st, const void* k_t, const void* v_t) {
    int rc = check_state(st, KIND_SPARSE, KIND_SCORE);
    return rc ? rc : record_kv(st, k_t, v_t);
}

int dsa_decode_step(dsa_state* st, const void* q_t, float* out, int32_t* trace) {
    int rc = check_state(st, KIND_SPARSE, KIND_SCORE);
    if (rc) return rc;
    rc = check_step(st, q_t, out);
    if (rc) return rc;
    if (trace && ((uintptr_t)trace & 7u)) return fail(DSA_E_INVAL, "trace must be 8-byte aligned");
    if (st->kind == KIND_SCORE) return score_decode(st, q_t, out, trace);

    dsa::DecodeArgs a;
    fill_common(st, q_t, out, a);
    const int t = st->t, S = st->S, N_rw = st->N_rw, N_attw = st->N_attw;
    const int tw = t - S;  // step inside the non-sink sequence
    a.list = reinterpret_cast<int16_t*>(st->ws + st->list_off);
    a.ring = st->ws + st->ring_off;
    a.trace = trace;
    a.S = S;
    a.N_rw = N_rw;
    a.N_attw = N_attw;
    a.list_stride = st->list_stride;
    // Window entries attended at t: min(t' + 1, N_att') (phase 1 grows, then fixed).
    a.n_list = tw < 0 ? 0 : std::min(tw + 1, N_attw);
    a.n_sink = std::min(t + 1, S);
    // Phase 2 selects while |skip_idx| < N_r - N_att: steps N_att-1 .. N_r-2.
    a.select = (t >= st->N_att - 1 && t <= st->N_r - 2) ? 1 : 0;
    // Offset t'+1 enters the window at step t+1 while the window still grows.
    a.add_off = (tw + 1 >= 0 && tw + 1 <= N_rw - 1) ? tw + 1 : -1;
    a.base = tw >= 0 ? tw % N_rw : 0;
    a.self_row = t < S ? t : S + a.base;
    // Phase 3 (t >= N_r): the oldest non-sink entry t - (N_r - S) leaves.
    a.evicted = t >= st->N_r ? t - N_rw : -1;

    const int splits = choose_splits(st);
    if (splits > 1 && !st->counters_clear) {
        // arrivals counted from zero; a fill kernel (the prompt kernel with
        // nothing to copy), not a memset, so the step stays capturable
        dsa::PromptArgs pa;
        memset(&pa, 0, sizeof(pa));
        pa.kv = st->ws;
        pa.counter = reinterpret_cast<int32_t*>(st->ws + st->ctr_off);
        pa.B = st->batch;
        pa.H = st->heads;
        hipError_t e = dsa::launch_prompt(st->dtype, st->D, pa, st->stream);
        if (e != hipSuccess) return hip_fail(e, "split counter clear");
        st->counters_clear = 1;
    }
    a.splits = splits;
    a.partial = reinterpret_cast<float*>(st->ws + st->part_off);
    a.counter = reinterpret_cast<int32_t*>(st->ws + st->ctr_off);
    const int waves = choose_waves(st, (long long)st->L_p + S + N_attw, splits);
    hipError_t e = dsa::launch_decode(dsa::MODE_SPARSE, st->dtype, st->D, waves, a, st->stream);
    if (e != hipSuccess) return hip_fail(e, "sparse decode launch");
    st->pend_k = st->pend_v = nullptr;
    st->t += 1;
    return DSA_OK;
}

int dsa_append_decode_step(dsa_state* st, const void* k_t, const void* v_t, const void* q_t, float* out,
                           int32_t* trace) {
    int rc = dsa_append_kv(st, k_t, v_t);
    if (rc) return rc;
    rc = dsa_decode_step(st, q_t, out, trace);
    if (rc) {  // leave the state as it was: no row recorded
        st->pend_k = st->pend_v = nullptr;
    }
    return rc;
}

int dsa_read_state(const dsa_state* st, int32_t* h_t, int16_t* h_offsets, int32_t* h_count) {
    int rc = check_state(st, KIND_SPARSE, KIND_SCORE);
    if (rc) return rc;
    if (st->kind == KIND_SCORE) {
        rc = (h_offsets || h_count) ? score_read_state(st, h_offsets, h_count) : 0;
        if (rc) return rc;
        if (!h_offsets && !h_count) {
            hipError_t e = hipStreamSynchronize(st->stream);
            if (e != hipSuccess) return hip_fail(e, "stream synchronize");
        }
        if (h_t) *h_t = st->t;
        return DSA_OK;
    }
    const int tw = st->t - st->S;
    const int n = tw < 0 ? 0 : std::min(tw + 1, st->N_attw);
    if (h_offsets || h_count) {
        std::vector<int16_t> buf;
        try {
            buf.resize((size_t)st->lanes * st->list_stride);
        } catch (...) {
            return fail(DSA_E_NOMEM, "host allocation failed");
        }
        hipError_t e = hipStreamSynchronize(st->stream);
        if (e != hipSuccess) return hip_fail(e, "stream synchronize");
        e = hipMemcpy(buf.data(), st->ws + st->list_off, buf.size() * sizeof(int16_t), hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(e, "list copy");
        for (int l = 0; l < st->lanes; ++l) {
            int16_t* src = buf.data() + (size_t)l * st->list_stride;
            std::sort(src, src + n);
            if (h_offsets) {
                int16_t* dst = h_offsets + (size_t)l * st->N_attw;
                for (int j = 0; j < st->N_attw; ++j) dst[j] = j < n ? src[j] : (int16_t)-1;
            }
            if (h_count) h_count[l] = n;
        }
    } else {
        hipError_t e = hipStreamSynchronize(st->stream);
        if (e != hipSuccess) return hip_fail(e, "stream synchronize");
    }
    if (h_t) *h_t = st->t;
    return DSA_OK;
}

size_t dense_state_workspace_bytes(int batch, int L_p, int L_max, int heads, int head_dim, int dtype) {
    if (check_common(batch, L_p, heads, head_dim, dtype) || L_max < 1) return 0;
    return kv_bytes((long long)batch * heads, (long long)L_p + L_max, head_dim, dtype) +
           scale_bytes((long long)batch * heads, (long long)L_p + L_max, dtype);
}

int dense_state_init(dsa_state** out, int batch, int L_p, int L_max, int heads, int head_dim, int dtype,
                     void* d_workspace, size_t workspace_bytes, void* hip_stream) {
    if (!out) return fail(DSA_E_INVAL, "out handle pointer is NULL");
    int rc = check_common(batch, L_p, heads, head_dim, dtype);
    if (rc) return rc;
    if (L_max < 1) return fail(DSA_E_INVAL, "L_max must be >= 1 (got %d)", L_max);
    if ((long long)L_p + L_max > 0x7fffffffll) return fail(DSA_E_INVAL, "L_p + L_max too large");
    rc = check_workspace(d_workspace, workspace_bytes,
                         dense_state_workspace_bytes(batch, L_p, L_max, heads, head_dim, dtype));
    if (rc) return rc;
    dsa_state* st = new (std::nothrow) dsa_state();
    if (!st) return fail(DSA_E_NOMEM, "host allocation failed");
    st->kind = KIND_DENSE;
    st->batch = batch;
    st->heads = heads;
    st->D = head_dim;
    st->L_p = L_p;
    st->dtype = dtype;
    st->L_max = L_max;
    st->lanes = batch * heads;
    st->lane_rows = (long long)L_p + L_max;
    st->ws = static_cast<char*>(d_workspace);
    st->ws_bytes = workspace_bytes;
    st->stream = static_cast<hipStream_t>(hip_stream);
    st->scale_rows = st->lane_rows;
    st->scale_off = kv_bytes(st->lanes, st->lane_rows, head_dim, dtype);
    rc = clear_mx_rows(st, st->scale_off + scale_bytes(st->lanes, st->scale_rows, dtype));
    if (rc) {
        delete st;
        return rc;
    }
    *out = st;
    return DSA_OK;
}

int dense_append_prompt(dsa_state* st, const void* k_p, const void* v_p) {
    int rc = check_state(st, KIND_DENSE);
    return rc ? rc : launch_prompt(st, k_p, v_p);
}

int dense_append_kv(dsa_state* st, const void* k_t, const void* v_t) {
    int rc = check_state(st, KIND_DENSE);
    return rc ? rc : record_kv(st, k_t, v_t);
}

int dense_decode_step(dsa_state* st, const void* q_t, float* out) {
    int rc = check_state(st, KIND_DENSE);
    if (rc) return rc;
    rc = check_step(st, q_t, out);
    if (rc) return rc;
    dsa::DecodeArgs a;
    fill_common(st, q_t, out, a);
    a.self_row = st->t;
    const int waves = choose_waves(st, (long long)st->L_p + st->t + 1);
    hipError_t e = dsa::launch_decode(dsa::MODE_DENSE, st->dtype, st->D, waves, a, st->stream);
    if (e != hipSuccess) return hip_fail(e, "dense decode launch");
    st->pend_k = st->pend_v = nullptr;
    st->t += 1;
    return DSA_OK;
}

int dense_append_decode_step(dsa_state* st, const void* k_t, const void* v_t, const void* q_t, float* out) {
    int rc = dense_append_kv(st, k_t, v_t);
    if (rc) return rc;
    rc = dense_decode_step(st, q_t, out);
    if (rc) st->pend_k = st->pend_v = nullptr;
    return rc;
}

static size_t profile_map_bytes(size_t lanes, int T) { return align_up(lanes * (size_t)T * (size_t)T * sizeof(float)); }
static size_t profile_mass_bytes(size_t lanes, int T) { return align_up(lanes * (size_t)T * 3 * sizeof(float)); }

// Workspace of a profile: the fp32 map [lanes][T][T], the per-query mass
// [lanes][T][3] and the per-row-tile cosine sums [lanes][ceil(T/16)][2 max_dist].
size_t dsa_profile_workspace_bytes(int batch, int heads, int L_p, int T, int max_dist) {
    if (batch < 1 || heads < 1 || L_p < 0 || T < 2 || max_dist < 1 || max_dist > T - 1 ||
        max_dist > dsa::kMaxProfileDist)
        return 0;
    const size_t lanes = (size_t)batch * heads;
    return profile_map_bytes(lanes, T) + profile_mass_bytes(lanes, T) +
           align_up(lanes * (size_t)((T + 15) / 16) * 2 * (size_t)max_dist * sizeof(double));
}

}  // extern "C"

namespace {

// Checks shared by both profile entry points (workspace excluded).
int check_profile(const void* q, const void* k, const void* k_p, int batch, int heads, int head_dim, int L_p, int T,
                  int dtype, int max_dist, const double* mass, const double* vert, const double* diag) {
    int rc = check_common(batch, L_p, heads, head_dim, dtype);
    if (rc) return rc;
    if (dtype == DSA_MXFP8) return fail(DSA_E_INVAL, "the profile takes fp32 or bf16 inputs");
    if (T < 2) return fail(DSA_E_INVAL, "T must be >= 2 (got %d)", T);
    if (max_dist < 1 || max_dist > T - 1 || max_dist > dsa::kMaxProfileDist)
        return fail(DSA_E_INVAL, "max_dist must be in [1, min(T - 1, %d)] (got %d)", dsa::kMaxProfileDist, max_dist);
    const long long lanes = (long long)batch * heads;
    if ((lanes + 7) / 8 * 8 * ((T + 15) / 16) > 0x7fffffffll) return fail(DSA_E_INVAL, "grid too large");
    if (!q || !k || (L_p > 0 && !k_p)) return fail(DSA_E_INVAL, "q / k / k_p is NULL");
    if (!aligned16(q) || !aligned16(k) || (L_p > 0 && !aligned16(k_p)))
        return fail(DSA_E_INVAL, "q / k / k_p must be 16-byte aligned");
    if (!mass || !vert || !diag) return fail(DSA_E_INVAL, "an output pointer is NULL");
    if (((uintptr_t)mass | (uintptr_t)vert | (uintptr_t)diag) & 7u)
        return fail(DSA_E_INVAL, "outputs must be 8-byte aligned");
    return 0;
}

// The three profile kernels over a checked, large enough workspace.
int launch_profile_on(const void* q, const void* k, const void* k_p, int batch, int heads, int head_dim, int L_p,
                      int T, int dtype, int max_dist, char* ws, double* mass, double* vert, double* diag,
                      hipStream_t stream) {
    const long long lanes = (long long)batch * heads;
    dsa::ProfileArgs a;
    a.q = q;
    a.k = k;
    a.k_p = k_p;
    a.P = reinterpret_cast<float*>(ws);
    a.mass_rows = reinterpret_cast<float*>(ws + profile_map_bytes(lanes, T));
    a.partial = reinterpret_cast<double*>(ws + profile_map_bytes(lanes, T) + profile_mass_bytes(lanes, T));
    a.mass = mass;
    a.vert = vert;
    a.diag = diag;
    a.lanes = (int)lanes;
    a.B = batch;
    a.H = heads;
    a.L_p = L_p;
    a.T = T;
    a.max_dist = max_dist;
    hipError_t e = dsa::launch_profile(dtype, head_dim, a, stream);
    if (e != hipSuccess) return hip_fail(e, "profile launch");
    return DSA_OK;
}

}  // namespace

extern "C" {

int dsa_attention_profile(const void* q, const void* k, const void* k_p, int batch, int heads, int head_dim, int L_p,
                          int T, int dtype, int max_dist, void* d_workspace, size_t workspace_bytes, double* mass,
                          double* vert, double* diag, void* hip_stream) {
    int rc = check_profile(q, k, k_p, batch, heads, head_dim, L_p, T, dtype, max_dist, mass, vert, diag);
    if (rc) return rc;
    rc = check_workspace(d_workspace, workspace_bytes, dsa_profile_workspace_bytes(batch, heads, L_p, T, max_dist));
    if (rc) return rc;
    return launch_profile_on(q, k, k_p, batch, heads, head_dim, L_p, T, dtype, max_dist,
                             static_cast<char*>(d_workspace), mass, vert, diag, static_cast<hipStream_t>(hip_stream));
}

int dsa_attention_profile_static(const void* q, const void* k, const void* k_p, int batch, int heads, int head_dim,
                                 int L_p, int T, int dtype, int max_dist, double* mass, double* vert, double* diag,
                                 void* hip_stream) {
    int rc = check_profile(q, k, k_p, batch, heads, head_dim, L_p, T, dtype, max_dist, mass, vert, diag);
    if (rc) return rc;
    const size_t need = dsa_profile_workspace_bytes(batch, heads, L_p, T, max_dist);
    if (need > (size_t)DSA_PROFILE_STATIC_SCRATCH_BYTES)
        return fail(DSA_E_WORKSPACE, "this profile needs %zu bytes of scratch; the static scratch holds %zu "
                    "(use dsa_attention_profile with a workspace)", need, (size_t)DSA_PROFILE_STATIC_SCRATCH_BYTES);
    void* ws = nullptr;
    hipError_t e = dsa::profile_static_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "static profile scratch address");
    return launch_profile_on(q, k, k_p, batch, heads, head_dim, L_p, T, dtype, max_dist, static_cast<char*>(ws), mass,
                             vert, diag, static_cast<hipStream_t>(hip_stream));
}

int dsa_hbm_read_probe(const void* src, size_t bytes, int blocks, int threads, int unroll, uint32_t* sink,
                       void* hip_stream) {
    if (!src || !sink) return fail(DSA_E_INVAL, "src / sink is NULL");
    if (bytes == 0 || bytes % 16 != 0) return fail(DSA_E_INVAL, "bytes must be a positive multiple of 16");
    if (!aligned16(src)) return fail(DSA_E_INVAL, "src must be 16-byte aligned");
    if ((uintptr_t)sink & 3u) return fail(DSA_E_INVAL, "sink must be 4-byte aligned");
    if (blocks < 1 || blocks > 65536) return fail(DSA_E_INVAL, "blocks must be in [1, 65536] (got %d)", blocks);
    if (threads < 64 || threads > 1024 || threads % 64 != 0)
        return fail(DSA_E_INVAL, "threads must be a multiple of 64 in [64, 1024] (got %d)", threads);
    if (unroll != 1 && unroll != 4 && unroll != 8) return fail(DSA_E_INVAL, "unroll must be 1, 4 or 8 (got %d)", unroll);
    hipError_t e = dsa::launch_hbm_read_probe(src, bytes, blocks, threads, unroll, sink,
                                              static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "read probe launch");
    return DSA_OK;
}

int dsa_set_waves(dsa_state* st, int waves_per_lane) {
    int rc = check_state(st, 0);
    if (rc) return rc;
    if (waves_per_lane != 0 && waves_per_lane != 1 && waves_per_lane != 2 && waves_per_lane != 4 &&
        waves_per_lane != 8 && waves_per_lane != 16)
        return fail(DSA_E_INVAL, "waves_per_lane must be 0, 1, 2, 4, 8 or 16 (got %d)", waves_per_lane);
    st->waves = waves_per_lane;
    return DSA_OK;
}

int dsa_set_splits(dsa_state* st, int splits_per_lane) {
    int rc = check_state(st, 0);
    if (rc) return rc;
    if (splits_per_lane != 0 && splits_per_lane != 1 && splits_per_lane != 2 && splits_per_lane != 4)
        return fail(DSA_E_INVAL, "splits_per_lane must be 0, 1, 2 or 4 (got %d)", splits_per_lane);
    if (splits_per_lane > 1 && (st->kind != KIND_SPARSE || st->dtype == DSA_MXFP8))
        return fail(DSA_E_INVAL, "only sparse states with bf16 or fp32 rows split (got a %s state, dtype %d)",
                    kind_name(st->kind), st->dtype);
    if ((long long)st->lanes * splits_per_lane > 0x7fffffffll)
        return fail(DSA_E_INVAL, "lanes * splits_per_lane exceeds the launch grid (%d lanes)", st->lanes);
    st->splits = splits_per_lane;
    return DSA_OK;
}

int dsa_state_step(const dsa_state* st) {
    int rc = check_state(st, 0);
    return rc ? rc : st->t;
}

int dsa_state_destroy(dsa_state* st) {
    delete st;
    return DSA_OK;
}

const char* dsa_strerror(int code) {
    switch (code) {
        case DSA_OK: return "DSA_OK";
        case DSA_E_INVAL: return "DSA_E_INVAL: invalid argument";
        case DSA_E_ORDER: return "DSA_E_ORDER: call out of order";
        case DSA_E_WORKSPACE: return "DSA_E_WORKSPACE: workspace missing, misaligned or too small";
        case DSA_E_HIP: return "DSA_E_HIP: HIP runtime error";
        case DSA_E_NOMEM: return "DSA_E_NOMEM: host allocation failed";
        default: return "unknown dsa_status";
    }
}

const char* dsa_last_error(void) { return g_err; }

}  // extern "C"
