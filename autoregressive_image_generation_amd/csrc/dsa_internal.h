// Internal interface between the C-ABI layer (dsa_api.hip) and the kernels
// (dsa_kernels.hip).  Not installed; the public contract is include/dsa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// SPARSE: Algorithm 1 (also SlidingWindow / StreamingLLM as its equal-budget
// cases); DENSE: no sparsity; TOVA, H2O: the score-based baselines over a
// cache of N_att slots per lane.
enum Mode { MODE_SPARSE = 0, MODE_DENSE = 1, MODE_TOVA = 2, MODE_H2O = 3 };

// Everything one decode launch needs.  Host-computed per step: all lanes of a
// state share t, so the phase logic of Algorithm 1 (page 4, Section 4) is
// resolved here once and the kernel only sees its consequences.
// Cache layout.  A row is K (D elements) then V (D elements).  Dense and
// TOVA / H2O states: [lanes][lane_rows] rows (prompt rows, then decode rows or
// slots).  Sparse states: the prompt region at kv, [lanes][L_p] rows or
// [L_p][lanes] rows (prompt row j of every lane side by side; the prompt
// strides below say which), then the ring region at `ring`: [N_r][lanes]
// rows, i.e. ring index i (sinks 0..S-1,
// then the window slots) of every lane side by side.  A step appends the same
// ring index in every lane, so its writes form one contiguous block, and the
// window reads of all lanes fall into the ring rows of a few indices.
struct DecodeArgs {
    const void* kv;        // cache base (see above); lane_rows = L_p for sparse states
    const void* ring;      // sparse: ring region [N_r][lanes] rows
    int16_t* list;         // sparse: [lanes][list_stride] attended window offsets (t - position)
    const void* q;         // [lanes][D]
    const void* k_new;     // [lanes][D], the step's appended key
    const void* v_new;     // [lanes][D]
    float* out;            // [lanes][D]
    int32_t* trace;        // sparse, nullable: [lanes][2]
    long long lane_rows;   // rows per lane in the cache
    // MXFP8 states: the 8-byte scale word of every cache row, lane-major:
    // [lanes][scale_rows], row index r of the lane's rows (sparse: prompt rows
    // 0 .. L_p-1, then L_p + ring index)
    char* scales;
    long long scale_rows;
    int lanes;
    // sparse: bytes between a lane's prompt rows and between the lanes' first
    // prompt rows (row bytes and L_p row bytes, or lanes row bytes and row
    // bytes for a [L_p][lanes] prompt region)
    long long prompt_row_bytes, prompt_lane_bytes;
    int L_p;
    int S;                 // sink count (0 or 4)
    int N_rw;              // ring length for non-sink entries: N_r - S
    int N_attw;            // attended non-sink budget: N_att - S
    int list_stride;       // entries per lane in the list: N_attw rounded up to 8 (16 bytes)
    int t;                 // decode step
    int n_list;            // sparse: entries of the list valid at this step
    int n_sink;            // sparse: sink positions attended at this step (min(t+1, S))
    int select;            // sparse: 1 if this step picks a new skip entry
    int add_off;           // sparse: offset entering the list for step t+1, or -1
    int base;              // sparse: (t - S) mod N_rw, ring index of the current token
    int self_row;          // sparse: ring index the appended K/V goes to; dense: decode row
    int evicted;           // sparse: position evicted at this step, or -1
    double scale_log2e;    // log2(e) / sqrt(D)
    // TOVA / H2O (slot cache; cache rows L_p .. L_p + N_cache - 1 are the slots)
    int32_t* meta;         // [lanes][meta_stride]: [0] free slot, [4 + j] position held by slot j
    double* score;         // H2O: [lanes][score_stride] accumulated score of slot j
    int meta_stride;       // 4 + N_cache rounded up to 4 (16 bytes)
    int score_stride;      // N_cache rounded up to 2
    int N_cache;           // slots per lane (N_att)
    int n_occ;             // occupied slots attended besides the current token: min(t, N_cache - 1)
    int n_meta;            // meta entries this step reads: 4 + min(t, N_cache)
    int free_host;         // slot of the current token when the host knows it (t < N_cache), else -1
    int n_recent;          // H2O: protected most recent positions
    double inv_sqrt_d;     // H2O: 1 / sqrt(D), for the fp64 probabilities
    // Split launches (sparse, plain rows; 1 otherwise): `splits` workgroups per
    // lane, each over a contiguous slice of the lane's rows.
    int splits;
    float* partial;        // [lanes][splits] records of split_rec_floats(D) floats
    int32_t* counter;      // [lanes] arrivals of the current launch; 0 between launches
};

// A split's partial state: acc[D], m, l, the argmin candidate's fp64 logit,
// its offset and its list index, padded to 16 bytes.
constexpr int split_rec_floats(int D) { return D + 8; }
constexpr int kMaxSplits = 4;

struct PromptArgs {
    const void* k_p;       // [B][L_p][H][D]
    const void* v_p;
    void* kv;
    int16_t* list;         // nullable: when set, list[lane * list_stride] = 0 for every lane
    char* scales;          // MXFP8: scale words [lanes][scale_rows] (as in DecodeArgs)
    long long scale_rows;
    int32_t* counter;      // nullable: when set, counter[lane] = 0 for every lane
    long long lane_rows;
    int B, H, L_p, list_stride;
    int slot_major;        // sparse states: rows go to [L_p][lanes] instead of [lanes][lane_rows]
};

// Attention-map characterization (dsa_profile.hip).
struct ProfileArgs {
    const void* q;         // [T][B][H][D] decode queries
    const void* k;         // [T][B][H][D] decode keys
    const void* k_p;       // [B][L_p][H][D] prompt keys
    float* P;              // workspace: [lanes][T][T] decode weights, each row its probabilities times a row constant (j <= i written)
    float* mass_rows;      // workspace: [lanes][T][3] prompt / local / middle mass per query
    double* mass;          // out: [lanes][3] mean over queries
    double* vert;          // out: [lanes][max_dist] mean vertical cosine similarity, distance 1..max_dist
    double* diag;          // out: [lanes][max_dist] mean diagonal cosine similarity
    double* partial;       // workspace: [lanes][row tiles][max_dist][2] per-tile cosine sums
    int lanes, B, H, L_p, T, max_dist;
};
constexpr int kMaxProfileDist = 256;  // per-distance sums of a row tile live in LDS

// Rows a thread group of a decode launch keeps in flight (the depth of its
// row pipeline), by the launch's workgroups and wavefronts per workgroup: 3
// for one-wavefront workgroups (large batches: many resident wavefronts per
// CU already keep HBM busy, and the shallower pipeline frees registers); for
// larger workgroups 2 when the launch alone brings 2048 wavefronts or more (8
// per CU: enough requests in flight, and deeper pipelines only lengthen the
// queues that the later wavefronts wait in), else 4.  Measured on MI355X at
// 512 x 4 and 256 x 8 wavefronts (depth 2 faster) and at 256 x 4 and 128 x 8
// (depth 4 faster).
constexpr int rows_in_flight(long long workgroups, int waves) {
    return waves == 1 ? 3 : workgroups * waves >= 2048 ? 2 : 4;
}

hipError_t launch_decode(int mode, int dtype, int D, int waves, const DecodeArgs& a, hipStream_t s);
hipError_t launch_profile(int dtype, int D, const ProfileArgs& a, hipStream_t s);
// Device address, on the current device, of the library's static profile
// scratch (DSA_PROFILE_STATIC_SCRATCH_BYTES bytes, 256-byte aligned); looked
// up once per device.
hipError_t profile_static_scratch(void** ptr);
hipError_t launch_prompt(int dtype, int D, const PromptArgs& a, hipStream_t s);
hipError_t launch_hbm_read_probe(const void* src, size_t bytes, int blocks, int threads, int unroll, uint32_t* sink,
                                 hipStream_t s);

}  // namespace dsa
