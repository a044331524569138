// Decode-attention kernels for gfx950 (CDNA4): the fused diagonal-aware sparse
// step of "Understanding and Exploiting Diagonal Attention Sparsity in
// Autoregressive Image Generation" (Section 4, Algorithm 1; Section 5.1 for the
// fused gather + argmin design and the Diagonal+Sink4 variant), the dense
// decode step it is compared with, and the score-based baselines of Sections
// 2.3 and 5.1: TOVA (the lowest-scoring entry of the step leaves the cache)
// and H2O (the unprotected entry with the lowest accumulated score leaves).
//
// One workgroup per lane (one (sequence, head) of the layer), `waves` 64-wide
// wavefronts.  Each thread group of TPR threads holds one cache row at a time,
// 16 (MXFP8), 8 (bf16) or 4 (fp32) elements of K and of V per thread; a
// wavefront works on 64 / TPR rows at a time.  Each group keeps its own online-softmax
// state (m, l, acc) over the rows it visits; groups merge through DPP /
// shuffles inside the wavefront and through LDS across wavefronts (with
// plain rows each wavefront normalises its own slice of the output).
// Single-query decode does about one flop per byte of KV, so the kernel is
// bound by HBM bandwidth; MFMA has no role.
//
// The raw logits q.k that a selection reads are accumulated in fp64: the
// products of bf16 (or fp32, or MXFP8) values are exact in fp64 and their sums
// nearly always are, so the argmin decision matches a fp64 reference up to
// order-of-summation rounding far below the selection's near-tie threshold.
// Logits that only the softmax reads take an fp32 dot product of bf16 pairs
// (bf16 and MXFP8 caches; see consume()).  The softmax runs in fp32 on the
// rounded logits.
//
// Cache row formats:
//   Plain<T>: K then V, D elements of T each (bf16 bit patterns or fp32); a
//     thread's chunk is 16 bytes of K and 16 of V.
//   Mx8 (the low-bit KV cache; Section 6 of the pages calls KV quantization
//     stackable with the selection): MXFP8 of the OCP Microscaling v1.0
//     format.  A row is K codes (D bytes, E4M3) then V codes (D bytes), whole
//     64-byte segments at D = 128; its 8-byte scale word (byte b the E8M0
//     scale of K block b, byte 4 + b that of V block b, blocks of 32
//     elements) lives in a region of its own, one word per cache row,
//     lane-major (DecodeArgs::scales).  A thread's chunk is 16 codes of K, 16
//     of V (16-byte loads) and the row's scale word.  q and the appended K/V
//     arrive in bf16; the appended row is quantised in the launch that
//     appends it, and every decode row the attention reads, the current
//     token's included, is the quantised one.
#include <type_traits>

#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kMaxWaves = 16;
constexpr float kNegBig = -1.0e30f;
// Pipeline depth in rows per thread group: rows_in_flight() (dsa_internal.h).
constexpr int kRowsPerChunkOneWave = 3;
constexpr int kRowsPerChunkBig = 2;
constexpr int kRowsPerChunk = 4;
static_assert(rows_in_flight(1, 1) == kRowsPerChunkOneWave && rows_in_flight(512, 4) == kRowsPerChunkBig &&
                  rows_in_flight(256, 4) == kRowsPerChunk,
              "the launcher's depths are rows_in_flight()'s");

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Cache rows are read once per step and not again before every other layer
// has streamed its own cache, so they bypass the caches' retention.
__device__ __forceinline__ uint4 load16_stream(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load8_stream(const void* p) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return make_uint2(v.x, v.y);
}

template <typename T>
__device__ __forceinline__ void unpack(const uint4& x, float* f) {
    if constexpr (sizeof(T) == 4) {
        f[0] = __uint_as_float(x.x);
        f[1] = __uint_as_float(x.y);
        f[2] = __uint_as_float(x.z);
        f[3] = __uint_as_float(x.w);
    } else {
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
}

// ---------------------------------------------------------------- MXFP8
// E4M3 codes -> floats (gfx950 converts OCP E4M3 in hardware, exactly); 4 codes per word.
__device__ __forceinline__ void unpack_e4m3_word(uint32_t w, float* f) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    f[0] = a[0];
    f[1] = a[1];
    f[2] = b[0];
    f[3] = b[1];
}
__device__ __forceinline__ void unpack_e4m3(const uint4& c, float* f) {
    unpack_e4m3_word(c.x, f);
    unpack_e4m3_word(c.y, f + 4);
    unpack_e4m3_word(c.z, f + 8);
    unpack_e4m3_word(c.w, f + 12);
}

// 2^(s - 127) of an E8M0 byte (s = 0 is 2^-127, a float subnormal).
__device__ __forceinline__ float e8m0_value(uint32_t s) { return __uint_as_float(s ? s << 23 : 0x00400000u); }

// Shared exponent of a block, floor(log2(amax)) - 8 (8: the largest E4M3
// exponent), clamped to the E8M0 range; -127 for an all-zero block.
__device__ __forceinline__ int mx_shared_exp(float amax) {
    if (!(amax > 0.0f)) return -127;
    int e;
    (void)frexpf(amax, &e);  // amax = f * 2^e, f in [0.5, 1)
    return min(max(e - 1 - 8, -127), 127);
}

// The E4M3 code nearest to y, ties to the even code, saturating at +-448.
// |y| < 512 always holds for y = v / 2^X with the block's shared exponent X.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float y) {
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fabsf(y);
    const uint32_t ab = __float_as_uint(a);
    int e = (int)(ab >> 23) - 127;
    uint32_t q = (ab & 0x7fffffu) >> 20;
    const uint32_t rest = ab & 0xfffffu;
    q += (rest > 0x80000u || (rest == 0x80000u && (q & 1u))) ? 1u : 0u;
    e += q == 8u ? 1 : 0;
    q = q == 8u ? 0u : q;
    const uint32_t normal = (e > 8 || (e == 8 && q == 7u)) ? 0x7eu : ((uint32_t)(e + 7) << 3) | q;
    const uint32_t sub = (uint32_t)__builtin_rintf(a * 512.0f);  // multiples of 2^-9; 8 = code 0x08
    return (a >= 0x1p-6f ? normal : sub) | sign;
}

// ---------------------------------------------------------------- row formats
template <typename T>
struct Plain {
    using In = T;
    static constexpr bool MX = false;
    static constexpr int EPT = 16 / (int)sizeof(T);  // elements of K (and of V) per thread
    template <int D>
    static constexpr size_t row_bytes() {
        return (size_t)2 * D * sizeof(T);
    }
    struct Chunk {
        uint4 k, v;
    };
};

struct Mx8 {
    using In = uint16_t;  // q and the appended rows arrive in bf16
    static constexpr bool MX = true;
    static constexpr int EPT = 16;
    template <int D>
    static constexpr size_t row_bytes() {
        return (size_t)2 * D;  // the codes; the scale word lives apart (DecodeArgs::scales)
    }
    struct Chunk {
        uint4 k, v;
        uint2 s;
    };
};

// The value of the lane a DPP pattern names.  Every pattern used here names
// a lane inside the same row of 16 for every lane, so no lane reads out of
// bounds and the moves need no fill value.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, true);
    return __hiloint2double(hi, lo);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over the TPR consecutive lanes of a thread group; every lane of the
// group ends with the same bits (each step adds a value and its partner's,
// and IEEE addition is commutative).
template <int TPR, typename V>
__device__ __forceinline__ V group_sum(V v) {
    if constexpr (sizeof(V) == 8) {
        v += dpp_f64<0xB1>(v);                            // quad_perm [1,0,3,2]
        v += dpp_f64<0x4E>(v);                            // quad_perm [2,3,0,1]
        if constexpr (TPR >= 8) v += dpp_f64<0x141>(v);   // row_half_mirror
        if constexpr (TPR >= 16) v += dpp_f64<0x140>(v);  // row_mirror
    } else {
        v += dpp_f32<0xB1>(v);
        v += dpp_f32<0x4E>(v);
        if constexpr (TPR >= 8) v += dpp_f32<0x141>(v);
        if constexpr (TPR >= 16) v += dpp_f32<0x140>(v);
    }
    if constexpr (TPR >= 32) v += __shfl_xor(v, 16);
    return v;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// q . k over a thread's 8 bf16 elements in fp32 (v_dot2_f32_bf16: two
// products per instruction, accumulated in fp32).
__device__ __forceinline__ float dot8_bf16(const uint4& q, const uint4& k) {
    float p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.x), __builtin_bit_cast(bf16x2, k.x), 0.0f,
                                              false);
    p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.y), __builtin_bit_cast(bf16x2, k.y), p, false);
    p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.z), __builtin_bit_cast(bf16x2, k.z), p, false);
    p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.w), __builtin_bit_cast(bf16x2, k.w), p, false);
    return p;
}

// The same for 16 bf16 q elements (two chunks) and 16 E4M3 codes, unscaled:
// each pair of codes widens exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8 with
// scale 1; every E4M3 value is a bf16 value), then v_dot2_f32_bf16.
__device__ __forceinline__ float dot16_bf16_e4m3(const uint4& q0, const uint4& q1, const uint4& k) {
    const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
    float p = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)kw[i], 1.0f, false);
        const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)kw[i], 1.0f, true);
        p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[2 * i]), lo, p, false);
        p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[2 * i + 1]), hi, p, false);
    }
    return p;
}

// Clamp the 8 int16 offsets of a list chunk into [0, hi].
__device__ __forceinline__ uint4 clamp_offsets(uint4 c, int hi) {
    uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int a = min(max((int)(int16_t)(w[i] & 0xffffu), 0), hi);
        const int b = min(max((int)(int16_t)(w[i] >> 16), 0), hi);
        w[i] = (uint32_t)a | ((uint32_t)b << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Maximum over the 4 lanes of a quad (every lane ends with it).
__device__ __forceinline__ float quad_max(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
    return v;
}

struct Softmax {
    float m, l;
};

// Merge (m2, l2, acc2) into (m, l, acc).  Symmetric in its two operands.
template <int EPT>
__device__ __forceinline__ void merge(Softmax& a, float* acc, float m2, float l2, const float* acc2) {
    float mn = fmaxf(a.m, m2);
    float c1 = __builtin_amdgcn_exp2f(a.m - mn);
    float c2 = __builtin_amdgcn_exp2f(m2 - mn);
    a.l = a.l * c1 + l2 * c2;
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = acc[e] * c1 + acc2[e] * c2;
    a.m = mn;
}

// Argmin candidate order: lower logit first; among equal logits the larger
// offset, i.e. the lower (older) position.
__device__ __forceinline__ bool better(double s, int d, double bs, int bd) {
    return s < bs || (s == bs && d > bd);
}

// Calls f with the workgroup's wavefront count (2, 4, 8 or 16) as a compile-time
// constant, so that a loop over the wavefronts' partial states unrolls and
// all of its LDS reads are issued at once.
template <typename Fn>
__device__ __forceinline__ void with_wave_count(int nwaves, Fn&& f) {
    switch (nwaves) {
        case 2: f(std::integral_constant<int, 2>{}); break;
        case 4: f(std::integral_constant<int, 4>{}); break;
        case 8: f(std::integral_constant<int, 8>{}); break;
        case 16: f(std::integral_constant<int, 16>{}); break;
        default: break;
    }
}

// Wavefront-wide reductions of doubles (butterfly: every lane ends with the result).
__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Marks the current token's row in the MXFP8 row stream: it is taken from
// registers after the merge, not read from the cache (d is the offset t -
// position for window entries, -1 for prompt and sink rows).
constexpr int kSelfOutOfStream = -2;

// NE: how many of every thread group's first U rows are requested before the
// lane's index data has arrived (rows g + u * G with u < NE need no list or
// slot entry: NE * G <= number of prompt + sink rows).
// MXFP8 holds 16 elements per thread and needs more than 128 VGPRs, so its
// workgroups stop at 8 wavefronts.
// SPLIT: a split launch (a.splits workgroups per lane; sparse, plain rows).
template <typename F, int D, int MODE, int U, int NE, bool SPLIT = false>
__global__ void __launch_bounds__(F::MX ? 512 : 1024) decode_kernel(DecodeArgs a) {
    using T = typename F::In;
    constexpr bool MX = F::MX;
    constexpr int EPT = F::EPT;
    constexpr int TPR = D / EPT;          // threads per half-row
    constexpr int GPW = 64 / TPR;         // thread groups per wavefront
    constexpr size_t RB = F::template row_bytes<D>();
    constexpr bool SLOTS = MODE == MODE_TOVA || MODE == MODE_H2O;
    constexpr int IEPT = 16 / (int)sizeof(T);     // input elements per 16-byte chunk
    constexpr int CH = 2 * D / IEPT;              // 16-byte chunks of an input K|V row
    static_assert(CH <= 64, "the lanes of wave 0 hold the appended row");

    // Dynamic LDS: the lane's index data, staged once per launch.  Sparse: the
    // attended window offsets (int16).  TOVA / H2O: the slot metadata (int32:
    // [0] the free slot, [4 + j] the position slot j holds), then for H2O the
    // fp64 logit of every attended row.
    extern __shared__ uint4 s_dyn16[];
    int16_t* s_list = reinterpret_cast<int16_t*>(s_dyn16);
    const int32_t* s_meta = reinterpret_cast<const int32_t*>(s_dyn16);
    double* s_logit = reinterpret_cast<double*>(s_dyn16 + a.meta_stride / 4);
    __shared__ float s_m[kMaxWaves], s_l[kMaxWaves];
    __shared__ float s_acc[kMaxWaves][D];
    __shared__ double s_bs[kMaxWaves];
    __shared__ int s_bd[kMaxWaves], s_bj[kMaxWaves];
    __shared__ int s_self_j;  // MXFP8 sparse: list index of the current token, -1 if not attended

    // Split launches (sparse, plain rows): workgroup x takes a contiguous
    // slice of the rows of lane x / splits, and the last of the lane's
    // workgroups to finish combines their partial states.
    static_assert(!SPLIT || (MODE == MODE_SPARSE && !MX && NE == 0), "split launches: sparse, plain rows");
    const int nsplit = SPLIT ? a.splits : 1;
    const int lane = SPLIT ? (int)blockIdx.x / nsplit : (int)blockIdx.x;
    const int split = SPLIT ? (int)blockIdx.x % nsplit : 0;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int wl = tid & 63;
    const int nwaves = blockDim.x >> 6;
    const int sl = wl % TPR;              // position inside the group
    const int g = wave * GPW + wl / TPR;  // group index in the workgroup
    const int G = nwaves * GPW;

    // sparse: this lane's first prompt row (prompt rows prompt_row_bytes apart);
    // other modes: the lane's cache rows
    const char* lane_kv = reinterpret_cast<const char*>(a.kv) +
                          (size_t)lane * (MODE == MODE_SPARSE ? (size_t)a.prompt_lane_bytes : (size_t)a.lane_rows * RB);
    const char* ring = reinterpret_cast<const char*>(a.ring);
    const char* k_self = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.k_new) + (size_t)lane * D);
    const char* v_self = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.v_new) + (size_t)lane * D);

    // Rows [0, R): prompt rows, then sinks (sparse) or cached decode positions
    // (dense), then from win0 on the listed window entries (sparse) or the
    // occupied slots and the current token (TOVA / H2O).
    const int R = MODE == MODE_SPARSE ? a.L_p + a.n_sink + a.n_list
                  : MODE == MODE_DENSE ? a.L_p + a.t + 1
                                       : a.L_p + a.n_occ + 1;
    const int win0 = MODE == MODE_SPARSE ? a.L_p + a.n_sink : MODE == MODE_DENSE ? R : a.L_p;
    // this workgroup's rows [r0, r1) (all of them unless split)
    const int per = (R + nsplit - 1) / nsplit;
    const int r0 = min(R, split * per), r1 = min(R, r0 + per);

    // Requests in the order their data is needed: the index data (16-byte
    // chunks; strides are padded to whole chunks), the query chunk, the
    // appended row, then (NE > 0) the first prompt rows.  Vector loads complete
    // in issue order, so waiting for the index data only waits for what was
    // issued before it.
    const int nch = MODE == MODE_SPARSE ? (a.n_list + 7) / 8 : SLOTS ? (a.n_meta + 3) / 4 : 0;
    const uint4* idx16 = MODE == MODE_SPARSE ? reinterpret_cast<const uint4*>(a.list + (size_t)lane * a.list_stride)
                                             : reinterpret_cast<const uint4*>(a.meta + (size_t)lane * a.meta_stride);
    uint4 lc0 = make_uint4(0, 0, 0, 0), lc1 = make_uint4(0, 0, 0, 0);
    if constexpr (MODE != MODE_DENSE) {
        if (tid < nch) lc0 = load16(idx16 + tid);
        if (tid + (int)blockDim.x < nch) lc1 = load16(idx16 + tid + blockDim.x);
    }
    constexpr int QCH = EPT / IEPT > 0 ? EPT / IEPT : 1;  // 16-byte chunks of q per thread
    uint4 qx[QCH];
#pragma unroll
    for (int c = 0; c < QCH; ++c) qx[c] = load16(reinterpret_cast<const T*>(a.q) + (size_t)lane * D + sl * EPT + c * IEPT);
    uint4 ax = make_uint4(0, 0, 0, 0);
    if (tid < CH) ax = load16((tid < CH / 2 ? k_self : v_self) + (tid % (CH / 2)) * 16);

    // TOVA / H2O: the slot the current token takes (the one freed by the last
    // eviction, or the next empty one while the cache fills).
    int fslot = SLOTS && a.free_host >= 0 ? a.free_host : 0;

    // Source of row r in [0, R): the addresses of this thread's K and V
    // chunks (and, MXFP8, of the row's scale word).  Sparse: offset d = t -
    // position of the listed entry, ring index S + (t' - d) mod N_rw.  TOVA /
    // H2O: the j-th occupied slot skips the free one; the last row is the
    // current token.  The current token is read from k_new / v_new (plain
    // rows) or taken out of the stream (MXFP8).  Branch-free, so that the row
    // loads below are straight-line code and every wait on them is exact.
    auto row_src = [&](int r, const char*& kr, const char*& vr, const char*& sr, int& d) {
        const bool listed = r >= win0;
        bool self;
        const char* row;
        long long sidx;  // MXFP8: the row's index among the lane's scale words
        d = -1;
        if constexpr (MODE == MODE_SPARSE) {
            const int dl = s_list[max(r - win0, 0)];  // clamped into [0, N_rw) when staged
            int slot = a.base - dl;
            slot += slot < 0 ? a.N_rw : 0;
            // the current token is a listed entry (offset 0) or, while t < S, a sink
            self = listed ? dl == 0 : (r >= a.L_p && r - a.L_p == a.t);
            const int ri = listed ? a.S + slot : max(r - a.L_p, 0);  // ring index of a sink or window entry
            const char* prow = lane_kv + (size_t)min(r, max(a.L_p - 1, 0)) * (size_t)a.prompt_row_bytes;
            const char* rrow = ring + ((size_t)ri * a.lanes + lane) * RB;
            row = r < a.L_p ? prow : rrow;
            sidx = r < a.L_p ? min(r, max(a.L_p - 1, 0)) : a.L_p + ri;
            d = listed ? dl : -1;
        } else if constexpr (MODE == MODE_DENSE) {
            self = r >= a.L_p && r - a.L_p == a.t;
            row = lane_kv + (size_t)r * RB;
            sidx = r;
        } else {
            const int j = max(r - win0, 0);
            const bool me = j == a.n_occ;
            const int slot = min(j + (j >= fslot ? 1 : 0), a.N_cache - 1);
            self = listed && me;
            sidx = listed ? a.L_p + slot : r;
            row = lane_kv + (size_t)sidx * RB;
            d = listed ? (me ? 0 : a.t - s_meta[4 + slot]) : -1;
        }
        if constexpr (MX) {
            d = self ? kSelfOutOfStream : d;  // the row address stays a valid cache row
            kr = row + sl * 16;
            vr = row + D + sl * 16;
            sr = a.scales + ((size_t)lane * a.scale_rows + sidx) * 8;
        } else {
            kr = (self ? k_self : row) + sl * 16;
            vr = (self ? v_self : row + D * sizeof(T)) + sl * 16;
            sr = nullptr;
            (void)sidx;
        }
    };
    auto load_row = [&](const char* kr, const char* vr, const char* sr) {
        typename F::Chunk c;
        if constexpr (MX) {
            c.k = load16_stream(kr);
            c.v = load16_stream(vr);
            c.s = load8_stream(sr);
        } else {
            (void)sr;
            c.k = load16_stream(kr);
            c.v = load16_stream(vr);
        }
        return c;
    };

    // Rows of this group: r_k = g + k * G.  Every group of a wavefront runs the
    // trip count of the wavefront's first group; rows past R re-read row R-1
    // (cached) and are not consumed.
    const int nk = (r1 - r0 - g + G - 1) / G;                // rows this group consumes
    const int nkw = (r1 - r0 - wave * GPW + G - 1) / G;       // trip count of the wavefront

    typename F::Chunk cx[U];
    int dd[U];
    // the group's first rows u in [u0, u1) (constants at both call sites)
    auto first_rows = [&](int u0, int u1) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u < u0 || u >= u1) continue;
            const char *kr, *vr, *sr;
            row_src(min(r0 + g + u * G, r1 - 1), kr, vr, sr, dd[u]);
            cx[u] = load_row(kr, vr, sr);
        }
    };
    if constexpr (NE > 0) first_rows(0, NE);  // prompt rows only: no index data read
    if constexpr (MODE != MODE_DENSE) {
        if constexpr (MX && MODE == MODE_SPARSE) {
            if (tid == 0) s_self_j = -1;
        }
        // Sparse offsets are written only by this kernel and lie in [0, N_rw);
        // they are clamped once here so that a damaged workspace cannot turn
        // into stray reads.  The slot metadata of TOVA / H2O is clamped where
        // it is used.
        auto stage = [&](uint4 c) { return MODE == MODE_SPARSE ? clamp_offsets(c, a.N_rw - 1) : c; };
        if (tid < nch) s_dyn16[tid] = stage(lc0);
        if (tid + (int)blockDim.x < nch) s_dyn16[tid + blockDim.x] = stage(lc1);
        for (int c = tid + 2 * (int)blockDim.x; c < nch; c += blockDim.x) s_dyn16[c] = stage(load16(idx16 + c));
        __syncthreads();
    }
    if constexpr (SLOTS) {
        // free slot: clamped like the offsets above
        if (a.free_host < 0) fslot = min(max(s_meta[0], 0), a.N_cache - 1);
    }
    if constexpr (NE < U) first_rows(NE, U);

    double qd[EPT];
    {
        float qf[EPT];
#pragma unroll
        for (int c = 0; c < QCH; ++c) unpack<T>(qx[c], qf + c * IEPT);
#pragma unroll
        for (int e = 0; e < EPT; ++e) qd[e] = (double)qf[e];
    }

    Softmax sm{kNegBig, 0.0f};
    float acc[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = 0.0f;
    double best_s = __builtin_inf();
    int best_d = -1, best_j = -1;

    // Logits the argmin reads (the window rows of a selection step: the
    // argmin candidates of Algorithm 1 and TOVA) and all of H2O's rows (its
    // scores are fp64 probabilities) are exact fp64 dot products.  The other
    // rows of bf16 and MXFP8 caches feed only the softmax and take an fp32
    // dot product of bf16 pairs (v_dot2_f32_bf16; MXFP8 codes widened to
    // bf16 first, the block scale applied to the sum).  The choice is made
    // per wavefront and iteration (uniform), from the wavefront's last row of
    // the iteration.  MXFP8 takes it at pipeline depth 3 only: at depth 4 the
    // two paths together need more registers than 3 wavefronts per SIMD
    // leave (measured slower).
    constexpr bool FAST = sizeof(T) == 2 && MODE != MODE_H2O && (!MX || U <= 3);
    const float scale_f = (float)a.scale_log2e;

    // Consume one row: logit, argmin candidate, online softmax.  Rows past
    // this group's share (k >= nk), and the out-of-stream current token of
    // MXFP8, enter with logit -inf and weight 0: selects instead of branches,
    // so the loop below stays straight-line apart from the uniform choice of
    // the logit's precision.
    auto consume = [&](int k, const typename F::Chunk& ch, int d) {
        const int r = r0 + g + k * G;
        int jj = r - win0;  // sparse: list index; TOVA: the slot (below)
        if constexpr (MODE == MODE_TOVA) jj = jj == a.n_occ ? fslot : jj + (jj >= fslot ? 1 : 0);
        float kf[EPT], vf[EPT];
        bool valid = k < nk;
        float x = -__builtin_inff();  // the logit in log2 units, scaled by 1 / sqrt(D)
        const bool exact = !FAST || ((MODE == MODE_SPARSE || MODE == MODE_TOVA) && a.select &&
                                     r0 + wave * GPW + GPW - 1 + k * G >= win0);
        if constexpr (FAST && !MX) {
            if (!exact) {
                const float s32 = group_sum<TPR>(dot8_bf16(qx[0], ch.k));
                x = valid ? s32 * scale_f : -__builtin_inff();
            }
        }
        double kscale = 1.0;
        float vscale = 1.0f;
        if constexpr (MX) {
            if constexpr (MODE == MODE_SPARSE) {
                // the list index of the current token; a sink (t < S, never a
                // selection step) records 0 just to mark it attended
                if (valid && d == kSelfOutOfStream && sl == 0) s_self_j = max(jj, 0);
            }
            valid = valid && d != kSelfOutOfStream;
            // A row that does not count (the current token's placeholder, a
            // row past the group's share) enters with weight 0.  Every cache
            // row holds zeros (cleared at state init) or the quantiser's codes
            // (no NaN code, scale bytes below 0xFF), so 0 times its values is 0.
            unpack_e4m3(ch.v, vf);
            const int b = sl * EPT / 32;  // this thread's elements lie in block b of 32
            const float kscale_f = e8m0_value(ch.s.x >> (8 * b) & 0xffu);
            kscale = (double)kscale_f;
            vscale = e8m0_value(ch.s.y >> (8 * b) & 0xffu);
            if constexpr (FAST) {
                if (exact) {
                    unpack_e4m3(ch.k, kf);
                } else {
                    // the block scale is a power of two: scaling each thread's
                    // partial sum before the group sum is exact
                    const float s32 = group_sum<TPR>(dot16_bf16_e4m3(qx[0], qx[1], ch.k) * kscale_f);
                    x = valid ? s32 * scale_f : -__builtin_inff();
                }
            } else {
                unpack_e4m3(ch.k, kf);
            }
        } else {
            unpack<T>(ch.v, vf);
        }
        if (exact) {
            if constexpr (!MX) unpack<T>(ch.k, kf);
            double part = 0.0;
#pragma unroll
            for (int e = 0; e < EPT; ++e) part = fma(qd[e], (double)kf[e], part);
            if constexpr (MX) part *= kscale;  // a power of two: exact
            const double s = group_sum<TPR>(part);
            if constexpr (MODE == MODE_SPARSE || MODE == MODE_TOVA) {
                const bool cand = valid && a.select && d >= 0 && better(s, d, best_s, best_d);
                best_s = cand ? s : best_s;
                best_d = cand ? d : best_d;
                best_j = cand ? jj : best_j;
            }
            if constexpr (MODE == MODE_H2O) {
                if (valid && sl == 0) s_logit[r] = s;
            }
            x = valid ? (float)(s * a.scale_log2e) : -__builtin_inff();
        }
        if constexpr (MX) {
            // 16 accumulators per thread: the running maximum moves only when
            // a logit exceeds it by more than 8 (log2 units), so weights stay
            // below 2^8 and the accumulators are rescaled only when some group
            // of the wavefront needs it (the state (m, l, acc) stays exact for
            // any m it holds)
            const bool need = x > sm.m + 8.0f;
            if (__builtin_amdgcn_ballot_w64(need)) {
                const float mn = need ? x : sm.m;
                const float c = __builtin_amdgcn_exp2f(sm.m - mn);
                sm.l *= c;
#pragma unroll
                for (int e = 0; e < EPT; ++e) acc[e] *= c;
                sm.m = mn;
            }
            const float p = __builtin_amdgcn_exp2f(x - sm.m);
            sm.l += p;
            const float pv = p * vscale;
#pragma unroll
            for (int e = 0; e < EPT; ++e) acc[e] = fmaf(pv, vf[e], acc[e]);
        } else {
            const float mn = fmaxf(sm.m, x);
            const float c = __builtin_amdgcn_exp2f(sm.m - mn);
            const float p = __builtin_amdgcn_exp2f(x - mn);
            sm.l = sm.l * c + p;
#pragma unroll
            for (int e = 0; e < EPT; ++e) acc[e] = acc[e] * c + p * vf[e];
            sm.m = mn;
        }
    };

    // Rolling pipeline: consume row k from its buffer, then refill that buffer
    // with row k + U, so U - 1 rows stay in flight while one is computed.
    int k0 = 0;
    for (; k0 + U < nkw; k0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            consume(k0 + u, cx[u], dd[u]);
            const char *kr, *vr, *sr;
            row_src(min(r0 + g + (k0 + u + U) * G, r1 - 1), kr, vr, sr, dd[u]);
            cx[u] = load_row(kr, vr, sr);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) consume(k0 + u, cx[u], dd[u]);

    // Append: the new K/V row goes to its cache row.  Nothing this launch
    // reads lives there (it is empty, holds the entry evicted at this step, or
    // is the free slot); the current token itself is read from k_new / v_new
    // (plain) or from the registers below (MXFP8).  Loaded at the start and
    // stored by wave 0 after its last global load: loads and stores share one
    // counter whose wait cannot tell them apart, so a store issued before a
    // load would make the wait for that load also wait for the store.
    char* dst_row;
    if constexpr (MODE == MODE_SPARSE)
        dst_row = const_cast<char*>(ring) + ((size_t)a.self_row * a.lanes + lane) * RB;
    else
        dst_row = const_cast<char*>(lane_kv) + (size_t)(a.L_p + (SLOTS ? fslot : a.self_row)) * RB;
    uint2 qcode = make_uint2(0, 0);  // MXFP8: this lane's 8 codes of the new row (lanes < CH of wave 0)
    uint32_t qscale = 0;             // and the E8M0 scale of its block
    uint32_t qw0 = 0, qw1 = 0;       // the row's scale word: K block b at byte b, V block b at byte 4 + b
    if constexpr (MX) {
        if (wave == 0) {
            // lanes 0 .. CH/2-1 hold K, CH/2 .. CH-1 hold V, 8 elements each;
            // a block of 32 is a quad of lanes
            float xf[8];
            unpack<uint16_t>(ax, xf);
            float am = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(xf[e]));
            const int X = mx_shared_exp(quad_max(am));
            uint32_t c[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) c[e] = e4m3_rne_sat(ldexpf(xf[e], -X));
            qcode = make_uint2(c[0] | c[1] << 8 | c[2] << 16 | c[3] << 24, c[4] | c[5] << 8 | c[6] << 16 | c[7] << 24);
            qscale = (uint32_t)(X + 127);
#pragma unroll
            for (int b = 0; b < D / 32; ++b) {
                qw0 |= (uint32_t)__shfl((int)qscale, 4 * b) << (8 * b);
                qw1 |= (uint32_t)__shfl((int)qscale, CH / 2 + 4 * b) << (8 * b);
            }
        }
    }
    auto store_append = [&]() {
        if constexpr (MX) {
            if (tid < CH) {
                const int off = tid < CH / 2 ? 8 * tid : D + 8 * (tid - CH / 2);
                *reinterpret_cast<uint2*>(dst_row + off) = qcode;
            }
            if (tid == 0) {
                const long long sidx = a.L_p + (MODE == MODE_SPARSE ? a.self_row : SLOTS ? fslot : a.self_row);
                *reinterpret_cast<uint2*>(a.scales + ((size_t)lane * a.scale_rows + sidx) * 8) = make_uint2(qw0, qw1);
            }
        } else {
            if (tid < CH) *reinterpret_cast<uint4*>(dst_row + tid * 16) = ax;
        }
    };

    // Merge the groups of this wavefront (butterfly over lanes TPR apart).
#pragma unroll
    for (int o = TPR; o < 64; o <<= 1) {
        const float m2 = __shfl_xor(sm.m, o);
        const float l2 = __shfl_xor(sm.l, o);
        float acc2[EPT];
#pragma unroll
        for (int e = 0; e < EPT; ++e) acc2[e] = __shfl_xor(acc[e], o);
        merge<EPT>(sm, acc, m2, l2, acc2);
        if constexpr (MODE == MODE_SPARSE || MODE == MODE_TOVA) {
            const double bs2 = __shfl_xor(best_s, o);
            const int bd2 = __shfl_xor(best_d, o);
            const int bj2 = __shfl_xor(best_j, o);
            if (bd2 >= 0 && (best_d < 0 || better(bs2, bd2, best_s, best_d))) {
                best_s = bs2;
                best_d = bd2;
                best_j = bj2;
            }
        }
    }

    // Across wavefronts: through LDS (MXFP8, H2O and split launches: merged in
    // wave order by wave 0; otherwise by output slices, below).
    if (wl < TPR) {
#pragma unroll
        for (int e = 0; e < EPT; ++e) s_acc[wave][sl * EPT + e] = acc[e];
        if (wl == 0) {
            s_m[wave] = sm.m;
            s_l[wave] = sm.l;
            s_bs[wave] = best_s;
            s_bd[wave] = best_d;
            s_bj[wave] = best_j;
        }
    }
    __syncthreads();

    // Plain rows in a workgroup of several wavefronts: every wavefront
    // normalises and stores its own D / nwaves output dimensions, each the
    // sum over the wavefronts' partial states weighted by 2^(m_w - max m),
    // divided by the same sum of the l_w.  All partial states are read at
    // once (the wavefront count a constant of the instance), so the last
    // lane of a launch does not wait for a merge chained through one
    // wavefront.  Wave 0 then stores the appended row and takes the selection.
    constexpr bool SLICED = !MX && !SPLIT && MODE != MODE_H2O;
    const bool sliced = SLICED && nwaves > 1;
    if constexpr (SLICED) {
        auto slice_out = [&](auto nw) {
            constexpr int NW = decltype(nw)::value;
            constexpr int DPW = D / NW;
            static_assert(DPW <= 64, "one dimension per thread");
            float mw[NW], lw[NW];
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                mw[w] = s_m[w];
                lw[w] = s_l[w];
            }
            if (wl < DPW) {
                const int dim = wave * DPW + wl;
                float ow[NW];
#pragma unroll
                for (int w = 0; w < NW; ++w) ow[w] = s_acc[w][dim];
                float mx = mw[0];
#pragma unroll
                for (int w = 1; w < NW; ++w) mx = fmaxf(mx, mw[w]);
                float l = 0.0f, o = 0.0f;
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    const float c = __builtin_amdgcn_exp2f(mw[w] - mx);
                    l = fmaf(c, lw[w], l);
                    o = fmaf(c, ow[w], o);
                }
                a.out[(size_t)lane * D + dim] = o / l;
            }
        };
        with_wave_count(nwaves, slice_out);
    }
    if (wave != 0) return;

    // MXFP8: the current token's row, quantised above, enters after the merge
    // of all other rows, in the lanes of wave 0's first group.  Lane c < CH/2
    // holds K codes 8c .. 8c+7 and lane CH/2 + c the same V codes, so group
    // lane sl gathers chunks 2 sl and 2 sl + 1 of each half.
    bool self_in = false;
    int self_j = -1;
    double self_s = 0.0;
    float self_vf[EPT];
    float self_vs = 1.0f;
    if constexpr (MX) {
        static_assert(EPT == 16, "two 8-code chunks per thread");
        const int k0l = 2 * wl, v0l = CH / 2 + 2 * wl;  // source lanes (only lanes < TPR use them)
        const uint4 kcode = make_uint4(__shfl((int)qcode.x, k0l), __shfl((int)qcode.y, k0l),
                                       __shfl((int)qcode.x, k0l + 1), __shfl((int)qcode.y, k0l + 1));
        const uint4 vcode = make_uint4(__shfl((int)qcode.x, v0l), __shfl((int)qcode.y, v0l),
                                       __shfl((int)qcode.x, v0l + 1), __shfl((int)qcode.y, v0l + 1));
        const float self_ks = e8m0_value((uint32_t)__shfl((int)qscale, k0l));
        self_vs = e8m0_value((uint32_t)__shfl((int)qscale, v0l));
        if constexpr (MODE == MODE_SPARSE) {
            self_j = s_self_j;
            self_in = self_j >= 0;
        } else {
            self_in = true;
            self_j = MODE == MODE_TOVA ? fslot : -1;
        }
        float kf[EPT];
        unpack_e4m3(kcode, kf);
        unpack_e4m3(vcode, self_vf);
        double part = 0.0;
#pragma unroll
        for (int e = 0; e < EPT; ++e) part = fma(qd[e], (double)kf[e], part);
        self_s = group_sum<TPR>(part * (double)self_ks);
    }

    if constexpr (!SLICED) {
        if (wl < TPR && nwaves > 1) {
            // wave 0's state and the others' from LDS, weighted by 2^(m_w -
            // max m): the maximum over all partial states at once, then the
            // sums two wavefronts at a time
            float mx = sm.m;
            with_wave_count(nwaves, [&](auto nw) {
                constexpr int NW = decltype(nw)::value;
                float mw[NW];
#pragma unroll
                for (int w = 1; w < NW; ++w) mw[w] = s_m[w];
#pragma unroll
                for (int w = 1; w < NW; ++w) mx = fmaxf(mx, mw[w]);
            });
            const float c0 = __builtin_amdgcn_exp2f(sm.m - mx);
            float l = sm.l * c0;
#pragma unroll
            for (int e = 0; e < EPT; ++e) acc[e] *= c0;
#pragma unroll 2
            for (int w = 1; w < nwaves; ++w) {
                const float c = __builtin_amdgcn_exp2f(s_m[w] - mx);
                l = fmaf(c, s_l[w], l);
#pragma unroll
                for (int e = 0; e < EPT; ++e) acc[e] = fmaf(c, s_acc[w][sl * EPT + e], acc[e]);
            }
            sm.m = mx;
            sm.l = l;
        }
    }
    if constexpr (MX) {
        if (wl < TPR && self_in) {
            const float x = (float)(self_s * a.scale_log2e);
            const float mn = fmaxf(sm.m, x);
            const float c = __builtin_amdgcn_exp2f(sm.m - mn);
            const float p = __builtin_amdgcn_exp2f(x - mn);
            sm.l = sm.l * c + p;
#pragma unroll
            for (int e = 0; e < EPT; ++e) acc[e] = acc[e] * c + (p * self_vs) * self_vf[e];
            sm.m = mn;
        }
    }
    if constexpr (SPLIT) {
        {
            // This workgroup's partial state: (m, l, acc) and its argmin
            // candidate over all its wavefronts, as one record.
#pragma unroll 1
            for (int w = 1; w < nwaves; ++w) {
                if (s_bd[w] >= 0 && (best_d < 0 || better(s_bs[w], s_bd[w], best_s, best_d))) {
                    best_s = s_bs[w];
                    best_d = s_bd[w];
                    best_j = s_bj[w];
                }
            }
            // Publication by release / acquire at device (agent) scope: the
            // record's stores, an agent-scope release fence executed by the
            // whole of wave 0 (the lanes that stored), then the arrival as an
            // acq_rel read-modify-write of the lane's counter.  The workgroup
            // whose arrival completes the count takes an agent-scope acquire
            // fence before it reads the other records, so every record it reads
            // happens-before its loads (the counter's RMWs form one release
            // sequence).
            float* rec = a.partial + (size_t)blockIdx.x * split_rec_floats(D);
            if (wl < TPR) {
#pragma unroll
                for (int e = 0; e < EPT; ++e) rec[sl * EPT + e] = acc[e];
            }
            if (wl == 0) {
                rec[D] = sm.m;
                rec[D + 1] = sm.l;
                *reinterpret_cast<double*>(rec + D + 2) = best_s;
                reinterpret_cast<int*>(rec)[D + 4] = best_d;
                reinterpret_cast<int*>(rec)[D + 5] = best_j;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            int arrived = 0;
            if (wl == 0)
                arrived = __hip_atomic_fetch_add(a.counter + lane, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            arrived = __shfl(arrived, 0);
            if (arrived != nsplit - 1) return;
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            if (wl == 0) __hip_atomic_store(a.counter + lane, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            // the records merged in split order (the argmin order is total)
            sm = Softmax{kNegBig, 0.0f};
#pragma unroll
            for (int e = 0; e < EPT; ++e) acc[e] = 0.0f;
            best_s = __builtin_inf();
            best_d = best_j = -1;
            for (int s2 = 0; s2 < nsplit; ++s2) {
                const float* r2 = a.partial + ((size_t)lane * nsplit + s2) * split_rec_floats(D);
                if (wl < TPR) {
                    float acc2[EPT];
#pragma unroll
                    for (int e = 0; e < EPT; ++e) acc2[e] = r2[sl * EPT + e];
                    merge<EPT>(sm, acc, r2[D], r2[D + 1], acc2);
                }
                const double bs2 = *reinterpret_cast<const double*>(r2 + D + 2);
                const int bd2 = reinterpret_cast<const int*>(r2)[D + 4];
                const int bj2 = reinterpret_cast<const int*>(r2)[D + 5];
                if (bd2 >= 0 && (best_d < 0 || better(bs2, bd2, best_s, best_d))) {
                    best_s = bs2;
                    best_d = bd2;
                    best_j = bj2;
                }
            }
        }
    }

    // The output and the appended row are stored once no global load is left
    // (H2O: after its score update).
    auto store_results = [&]() {
        if (wl < TPR && !sliced) {
            const float inv = 1.0f / sm.l;
            float4* o4 = reinterpret_cast<float4*>(a.out + (size_t)lane * D + sl * EPT);
#pragma unroll
            for (int e = 0; e < EPT; e += 4)
                o4[e / 4] = make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
        }
        store_append();
    };
    if constexpr (MODE != MODE_H2O) store_results();

    if constexpr (MODE == MODE_SPARSE || MODE == MODE_TOVA) {
        if (a.select && nwaves > 1) {
            // Wavefront w's candidate in lane w of wave 0 (lane 0: its own),
            // reduced over the first 16 lanes by rotations of 1, 2, 4 and 8
            // (the candidate order is total, so the minimum is the same in
            // any order of merging).
            if (wl >= nwaves) best_d = -1;
            if (wl >= 1 && wl < nwaves) {
                best_s = s_bs[wl];
                best_d = s_bd[wl];
                best_j = s_bj[wl];
            }
            auto rotate = [&](auto cc) {
                constexpr int CTRL = decltype(cc)::value;
                const double bs2 = dpp_f64<CTRL>(best_s);
                const int bd2 = __builtin_amdgcn_mov_dpp(best_d, CTRL, 0xF, 0xF, true);
                const int bj2 = __builtin_amdgcn_mov_dpp(best_j, CTRL, 0xF, 0xF, true);
                if (bd2 >= 0 && (best_d < 0 || better(bs2, bd2, best_s, best_d))) {
                    best_s = bs2;
                    best_d = bd2;
                    best_j = bj2;
                }
            };
            rotate(std::integral_constant<int, 0x121>{});  // row_ror:1
            rotate(std::integral_constant<int, 0x122>{});  // row_ror:2
            rotate(std::integral_constant<int, 0x124>{});  // row_ror:4
            rotate(std::integral_constant<int, 0x128>{});  // row_ror:8
        }
        if (wl != 0) return;
        if constexpr (MX) {
            // the current token as a candidate: offset 0
            if (self_in && a.select && (best_d < 0 || better(self_s, 0, best_s, best_d))) {
                best_s = self_s;
                best_d = 0;
                best_j = self_j;
            }
        }
        int chosen = -1;
        if constexpr (MODE == MODE_SPARSE) {
            int16_t* lst = a.list + (size_t)lane * a.list_stride;
            if (a.select) {
                // The lowest-scoring entry joins the skipped set: its offset best_d
                // leaves the attended list for good (a skip keeps its offset as it
                // moves along the diagonal), and the offset entering the window at
                // t+1 takes its list entry.
                if (best_j >= 0) {
                    chosen = a.t - best_d;
                    lst[best_j] = (int16_t)a.add_off;
                }
            } else if (a.add_off >= 0 && a.n_list < a.N_attw) {
                lst[a.n_list] = (int16_t)a.add_off;
            }
        } else {
            // TOVA: the current token holds its slot; with a full cache the
            // lowest-logit entry leaves and its slot is the next free one.
            int32_t* meta = a.meta + (size_t)lane * a.meta_stride;
            meta[4 + fslot] = a.t;
            if (a.select && best_j >= 0) {
                chosen = a.t - best_d;
                meta[0] = best_j;
            }
        }
        if (a.trace) {
            a.trace[2 * lane] = chosen;
            a.trace[2 * lane + 1] = MODE == MODE_SPARSE ? a.evicted : -1;
        }
    }

    if constexpr (MODE == MODE_H2O) {
        // Accumulated scores in fp64: each attended decode entry adds its
        // probability under this step's softmax (prompt rows included in the
        // normalisation); then, with a full cache, the unprotected entry
        // (position <= t - n_recent) with the lowest score leaves, the lowest
        // position among equals.  Wave 0 does this for the lane.
        const double c = a.inv_sqrt_d;
        const double self_logit = __shfl(self_s, 0);  // MXFP8: the current token's logit
        auto logit = [&](int r) { return MX && r == R - 1 ? self_logit : s_logit[r]; };
        double m = -__builtin_inf();
        for (int r = wl; r < R; r += 64) m = fmax(m, logit(r));
        m = wave_max(m);
        double l = 0.0;
        for (int r = wl; r < R; r += 64) l += exp((logit(r) - m) * c);
        l = wave_sum(l);
        double* sc = a.score + (size_t)lane * a.score_stride;
        const int lim = a.t - a.n_recent;
        double bkey = __builtin_inf();
        int bpos = 0x7fffffff, bslot = -1;
        for (int j = wl; j <= a.n_occ; j += 64) {
            const bool me = j == a.n_occ;
            const int slot = me ? fslot : min(j + (j >= fslot ? 1 : 0), a.N_cache - 1);
            const double p = exp((logit(win0 + j) - m) * c) / l;
            const double ns = (me ? 0.0 : sc[slot]) + p;
            sc[slot] = ns;
            const int pos = me ? a.t : s_meta[4 + slot];
            if (a.select && pos <= lim && (ns < bkey || (ns == bkey && pos < bpos))) {
                bkey = ns;
                bpos = pos;
                bslot = slot;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const double k2 = __shfl_xor(bkey, o);
            const int p2 = __shfl_xor(bpos, o);
            const int s2 = __shfl_xor(bslot, o);
            if (k2 < bkey || (k2 == bkey && p2 < bpos)) {
                bkey = k2;
                bpos = p2;
                bslot = s2;
            }
        }
        if (wl == 0) {
            int32_t* meta = a.meta + (size_t)lane * a.meta_stride;
            meta[4 + fslot] = a.t;
            int chosen = -1;
            if (a.select && bslot >= 0) {
                chosen = bpos;
                meta[0] = bslot;
            }
            if (a.trace) {
                a.trace[2 * lane] = chosen;
                a.trace[2 * lane + 1] = -1;
            }
        }
        store_results();
    }
}

// Prompt rows into the cache ([lanes][lane_rows], or [L_p][lanes] for
// slot-major sparse prompt regions; plain: a copy; MXFP8: one block of 32
// values per thread, quantised), and the initial list entry {offset 0} of
// sink-free sparse states.
template <typename F, int D>
__global__ void prompt_kernel(PromptArgs a) {
    using T = typename F::In;
    constexpr size_t RB = F::template row_bytes<D>();
    if constexpr (F::MX) {
        constexpr int NB = D / 32;  // blocks per half-row
        const long long total = (long long)a.B * a.H * a.L_p * 2 * NB;
        for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
             i += (long long)gridDim.x * blockDim.x) {
            long long x = i;
            const int blk = (int)(x % NB);
            x /= NB;
            const int h = (int)(x % a.H);
            x /= a.H;
            const int half = (int)(x % 2);
            x /= 2;
            const int j = (int)(x % a.L_p);
            const int b = (int)(x / a.L_p);
            const T* src = reinterpret_cast<const T*>(half ? a.v_p : a.k_p) +
                           (((size_t)b * a.L_p + j) * a.H + h) * D + blk * 32;
            float v[32];
#pragma unroll
            for (int c = 0; c < 4; ++c) unpack<uint16_t>(load16(src + 8 * c), v + 8 * c);
            float am = 0.0f;
#pragma unroll
            for (int e = 0; e < 32; ++e) am = fmaxf(am, fabsf(v[e]));
            const int X = mx_shared_exp(am);
            uint32_t w[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                w[q] = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[q] |= e4m3_rne_sat(ldexpf(v[4 * q + e], -X)) << (8 * e);
            }
            const size_t lane = (size_t)b * a.H + h;
            const size_t ri = a.slot_major ? (size_t)j * ((size_t)a.B * a.H) + lane : lane * (size_t)a.lane_rows + j;
            char* row = reinterpret_cast<char*>(a.kv) + ri * RB;
            uint4* dst = reinterpret_cast<uint4*>(row + half * D + blk * 32);
            dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
            dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
            a.scales[(lane * (size_t)a.scale_rows + j) * 8 + half * 4 + blk] = (char)(X + 127);
        }
    } else {
        constexpr int CPR = D * (int)sizeof(T) / 16;  // 16-byte chunks per half-row
        const long long total = (long long)a.B * a.H * a.L_p * 2 * CPR;
        for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
             i += (long long)gridDim.x * blockDim.x) {
            long long x = i;
            const int c = (int)(x % CPR);
            x /= CPR;
            const int h = (int)(x % a.H);
            x /= a.H;
            const int half = (int)(x % 2);
            x /= 2;
            const int j = (int)(x % a.L_p);
            const int b = (int)(x / a.L_p);
            const char* src = reinterpret_cast<const char*>(half ? a.v_p : a.k_p) +
                              (((size_t)b * a.L_p + j) * a.H + h) * D * sizeof(T) + c * 16;
            const size_t lane = (size_t)b * a.H + h;
            const size_t ri = a.slot_major ? (size_t)j * ((size_t)a.B * a.H) + lane : lane * (size_t)a.lane_rows + j;
            char* dst = reinterpret_cast<char*>(a.kv) + ri * RB + half * D * sizeof(T) + c * 16;
            *reinterpret_cast<uint4*>(dst) = load16(src);
        }
    }
    if (a.list || a.counter) {
        const int lanes = a.B * a.H;
        for (int l = blockIdx.x * blockDim.x + threadIdx.x; l < lanes; l += gridDim.x * blockDim.x) {
            if (a.list) a.list[(size_t)l * a.list_stride] = 0;
            if (a.counter) a.counter[l] = 0;
        }
    }
}

template <typename F, int D, int U, int MODE>
void launch_decode_m(int G, int win0, dim3 grid, dim3 block, size_t lds, const DecodeArgs& a, hipStream_t s) {
    if constexpr (MODE == MODE_SPARSE && !F::MX) {
        // split launches issue no row before the index list: a slice past the
        // first may start inside the window
        if (a.splits > 1) {
            hipLaunchKernelGGL((decode_kernel<F, D, MODE, U, 0, true>), grid, block, lds, s, a);
            return;
        }
    }
    // rows per group that need no index data: all U, one, or none
    const int ne = win0 / G;
    if (ne >= U)
        hipLaunchKernelGGL((decode_kernel<F, D, MODE, U, U>), grid, block, lds, s, a);
    else if (ne >= 1)
        hipLaunchKernelGGL((decode_kernel<F, D, MODE, U, 1>), grid, block, lds, s, a);
    else
        hipLaunchKernelGGL((decode_kernel<F, D, MODE, U, 0>), grid, block, lds, s, a);
}

template <typename F, int D, int U>
hipError_t launch_decode_u(int mode, int waves, const DecodeArgs& a, hipStream_t s) {
    constexpr int TPR = D / F::EPT;
    const int G = waves * (64 / TPR);
    dim3 grid(a.lanes * a.splits), block(64 * waves);
    switch (mode) {
        case MODE_SPARSE: {
            const size_t lds = (size_t)((a.n_list + 7) / 8 > 0 ? (a.n_list + 7) / 8 : 1) * 16;
            launch_decode_m<F, D, U, MODE_SPARSE>(G, a.L_p + a.n_sink, grid, block, lds, a, s);
            break;
        }
        case MODE_DENSE:
            hipLaunchKernelGGL((decode_kernel<F, D, MODE_DENSE, U, U>), grid, block, 0, s, a);
            break;
        case MODE_TOVA:
            launch_decode_m<F, D, U, MODE_TOVA>(G, a.L_p, grid, block, (size_t)a.meta_stride * 4, a, s);
            break;
        default:  // MODE_H2O: slot metadata, then one fp64 logit per attended row
            launch_decode_m<F, D, U, MODE_H2O>(G, a.L_p, grid, block,
                                               (size_t)a.meta_stride * 4 + (size_t)(a.L_p + a.N_cache) * 8, a, s);
            break;
    }
    return hipGetLastError();
}

template <typename F, int D>
hipError_t launch_decode_t(int mode, int waves, const DecodeArgs& a, hipStream_t s) {
    switch (rows_in_flight((long long)a.lanes * a.splits, waves)) {
        case kRowsPerChunkOneWave:
            return launch_decode_u<F, D, kRowsPerChunkOneWave>(mode, waves, a, s);
        case kRowsPerChunkBig:
            return launch_decode_u<F, D, kRowsPerChunkBig>(mode, waves, a, s);
        default:
            return launch_decode_u<F, D, kRowsPerChunk>(mode, waves, a, s);
    }
}

template <typename F, int D>
hipError_t launch_prompt_t(const PromptArgs& a, hipStream_t s) {
    const long long units =
        (long long)a.B * a.H * a.L_p * 2 * (F::MX ? D / 32 : D * (int)sizeof(typename F::In) / 16);
    long long blocks = (units + 255) / 256;
    const long long lane_blocks = ((long long)a.B * a.H + 255) / 256;
    if (blocks < lane_blocks) blocks = lane_blocks;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL((prompt_kernel<F, D>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <typename F>
hipError_t decode_for(int mode, int D, int waves, const DecodeArgs& a, hipStream_t s) {
    return D == 128 ? launch_decode_t<F, 128>(mode, waves, a, s) : launch_decode_t<F, 64>(mode, waves, a, s);
}

template <typename F>
hipError_t prompt_for(int D, const PromptArgs& a, hipStream_t s) {
    return D == 128 ? launch_prompt_t<F, 128>(a, s) : launch_prompt_t<F, 64>(a, s);
}

}  // namespace

hipError_t launch_decode(int mode, int dtype, int D, int waves, const DecodeArgs& a, hipStream_t s) {
    if (dtype == 2) return decode_for<Mx8>(mode, D, waves, a, s);
    if (dtype == 1) return decode_for<Plain<uint16_t>>(mode, D, waves, a, s);
    return decode_for<Plain<float>>(mode, D, waves, a, s);
}

hipError_t launch_prompt(int dtype, int D, const PromptArgs& a, hipStream_t s) {
    if (dtype == 2) return prompt_for<Mx8>(D, a, s);
    if (dtype == 1) return prompt_for<Plain<uint16_t>>(D, a, s);
    return prompt_for<Plain<float>>(D, a, s);
}

}  // namespace dsa
