// Decode-attention kernels for gfx950 (CDNA4): the fused diagonal-aware sparse
// step of "Understanding and Exploiting Diagonal Attention Sparsity in
// Autoregressive Image Generation" (Section 4, Algorithm 1; Section 5.1 for the
// fused gather + argmin design and the Diagonal+Sink4 variant), the dense
// decode step it is compared with, and the score-based baselines of Sections
// 2.3 and 5.1: TOVA (the lowest-scoring entry of the step leaves the cache)
// and H2O (the unprotected entry with the lowest accumulated score leaves).
//
// One workgroup per lane (one (sequence, head) of the layer), `waves` 64-wide
// wavefronts.  A row of the cache is K (D elements) followed by V (D
// elements); TPR = D * sizeof(T) / 16 threads cover one half-row with one
// 16-byte load each, so a wavefront works on 64 / TPR rows at a time.  Each
// such thread group keeps its own online-softmax state (m, l, acc) over the
// rows it visits; groups merge through DPP / shuffles inside the wavefront and
// through LDS across wavefronts.  Single-query decode does about one flop per
// byte of KV, so the kernel is bound by HBM bandwidth; MFMA has no role.
//
// The raw logits q.k are accumulated in fp64: bf16 x bf16 products are exact
// in fp64 and their sums nearly always are, so the argmin decision matches a
// fp64 reference up to order-of-summation rounding far below the selection's
// near-tie threshold.  The softmax runs in fp32 on the rounded logits.
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kMaxWaves = 16;
constexpr float kNegBig = -1.0e30f;
#ifndef DSA_ROWS_PER_CHUNK
#define DSA_ROWS_PER_CHUNK 4
#endif
constexpr int kRowsPerChunk = DSA_ROWS_PER_CHUNK;  // pipeline depth in rows per thread group

template <typename T>
struct Traits;
template <>
struct Traits<float> {
    static constexpr int EPT = 4;  // elements per 16-byte chunk
};
template <>
struct Traits<uint16_t> {  // bf16 bit patterns
    static constexpr int EPT = 8;
};

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

__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Cache rows are read once per step and not again before every other layer
// has streamed its own cache, so they bypass the caches' retention.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_stream(const void* p) {
#ifdef DSA_CACHED_ROWS
    return *reinterpret_cast<const uint4*>(p);
#else
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
#endif
}

// Exchange a double with the lane a DPP pattern names (both halves moved).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    int lo = __double2loint(v);
    int hi = __double2hiint(v);
    lo = __builtin_amdgcn_update_dpp(0, lo, CTRL, 0xF, 0xF, false);
    hi = __builtin_amdgcn_update_dpp(0, hi, CTRL, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}

// Sum over the TPR consecutive lanes of a thread group; every lane of the
// group ends with the same bits (each step adds a value and its partner's,
// and IEEE addition is commutative).
template <int TPR>
__device__ __forceinline__ double group_sum(double v) {
    v += dpp_f64<0xB1>(v);                            // quad_perm [1,0,3,2]
    v += dpp_f64<0x4E>(v);                            // quad_perm [2,3,0,1]
    if constexpr (TPR >= 8) v += dpp_f64<0x141>(v);   // row_half_mirror
    if constexpr (TPR >= 16) v += dpp_f64<0x140>(v);  // row_mirror
    if constexpr (TPR >= 32) v += __shfl_xor(v, 16);
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

// EARLY: every thread group's first U rows need no list or slot entry (U * G
// <= number of prompt + sink rows), so they are requested before the lane's
// index data has arrived.
template <typename T, int D, int MODE, int U, bool EARLY>
__global__ void __launch_bounds__(1024) decode_kernel(DecodeArgs a) {
    constexpr int EPT = Traits<T>::EPT;
    constexpr int TPR = D / EPT;          // threads per half-row
    constexpr int GPW = 64 / TPR;         // thread groups per wavefront
    constexpr int ROW = 2 * D;            // elements per cache row
    constexpr bool SLOTS = MODE == MODE_TOVA || MODE == MODE_H2O;

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

    const int lane = blockIdx.x;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int wl = tid & 63;
    const int nwaves = blockDim.x >> 6;
    const int sl = wl % TPR;              // position inside the group
    const int g = wave * GPW + wl / TPR;  // group index in the workgroup
    const int G = nwaves * GPW;

    const T* lane_kv = reinterpret_cast<const T*>(a.kv) + (size_t)lane * (size_t)a.lane_rows * ROW;
    const T* k_self = reinterpret_cast<const T*>(a.k_new) + (size_t)lane * D;
    const T* v_self = reinterpret_cast<const T*>(a.v_new) + (size_t)lane * D;

    // Rows [0, R): prompt rows, then sinks (sparse) or cached decode positions
    // (dense), then from win0 on the listed window entries (sparse) or the
    // occupied slots and the current token (TOVA / H2O).
    const int R = MODE == MODE_SPARSE ? a.L_p + a.n_sink + a.n_list
                  : MODE == MODE_DENSE ? a.L_p + a.t + 1
                                       : a.L_p + a.n_occ + 1;
    const int win0 = MODE == MODE_SPARSE ? a.L_p + a.n_sink : MODE == MODE_DENSE ? R : a.L_p;
    constexpr int CH = ROW * (int)sizeof(T) / 16;                // 16-byte chunks per row

    // Requests in the order their data is needed: the index data (16-byte
    // chunks; strides are padded to whole chunks), the query chunk, the
    // appended row, then (EARLY) the first prompt rows.  Vector loads complete
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
    const uint4 qx = load16(reinterpret_cast<const T*>(a.q) + (size_t)lane * D + sl * EPT);
    uint4 ax = make_uint4(0, 0, 0, 0);
    if (tid < CH) ax = load16((tid < CH / 2 ? k_self : v_self) + (tid % (CH / 2)) * EPT);

    // TOVA / H2O: the slot the current token takes (the one freed by the last
    // eviction, or the next empty one while the cache fills).
    int fslot = SLOTS && a.free_host >= 0 ? a.free_host : 0;

    // Source of row r in [0, R).  Sparse: offset d = t - position of the
    // listed entry, ring slot S + (t' - d) mod N_rw.  TOVA / H2O: the j-th
    // occupied slot skips the free one; the last row is the current token.
    // The current token is read from k_new / v_new.  Branch-free, so that the
    // row loads below are straight-line code and every wait on them is exact.
    auto row_src = [&](int r, const T*& kr, const T*& vr, int& d) {
        const bool listed = r >= win0;
        bool self;
        const T* base;
        d = -1;
        if constexpr (MODE == MODE_SPARSE) {
            // Offsets are written only by this kernel and lie in [0, N_rw);
            // the clamp keeps a damaged workspace from turning into stray reads.
            const int dl = min(max((int)s_list[max(r - win0, 0)], 0), a.N_rw - 1);
            int slot = a.base - dl;
            slot += slot < 0 ? a.N_rw : 0;
            // the current token is a listed entry (offset 0) or, while t < S, a sink
            self = listed ? dl == 0 : (r >= a.L_p && r - a.L_p == a.t);
            const int ri = listed ? a.S + slot : max(r - a.L_p, 0);  // ring index of a sink or window entry
            const T* prow = lane_kv + (size_t)min(r, max(a.L_p - 1, 0)) * ROW;
            const T* rrow = reinterpret_cast<const T*>(a.ring) + ((size_t)ri * a.lanes + lane) * ROW;
            base = r < a.L_p ? prow : rrow;
            d = listed ? dl : -1;
        } else if constexpr (MODE == MODE_DENSE) {
            self = r >= a.L_p && r - a.L_p == a.t;
            base = lane_kv + (size_t)r * ROW;
        } else {
            const int j = max(r - win0, 0);
            const bool me = j == a.n_occ;
            const int slot = min(j + (j >= fslot ? 1 : 0), a.N_cache - 1);
            self = listed && me;
            base = lane_kv + (size_t)(listed ? a.L_p + slot : r) * ROW;
            d = listed ? (me ? 0 : a.t - s_meta[4 + slot]) : -1;
        }
        kr = self ? k_self : base;
        vr = self ? v_self : base + D;
    };

    // Rows of this group: r_k = g + k * G.  Every group of a wavefront runs the
    // trip count of the wavefront's first group; rows past R re-read row R-1
    // (cached) and are not consumed.
    const int nk = (R - g + G - 1) / G;                      // rows this group consumes
    const int nkw = (R - wave * GPW + G - 1) / G;             // trip count of the wavefront

    uint4 kx[U], vx[U];
    int dd[U];
    auto first_rows = [&]() {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const T* kr;
            const T* vr;
            row_src(min(g + u * G, R - 1), kr, vr, dd[u]);
            kx[u] = load16_stream(kr + sl * EPT);
            vx[u] = load16_stream(vr + sl * EPT);
        }
    };
    if constexpr (EARLY) first_rows();  // prompt rows only: no index data read
    if constexpr (MODE != MODE_DENSE) {
        if (tid < nch) s_dyn16[tid] = lc0;
        if (tid + (int)blockDim.x < nch) s_dyn16[tid + blockDim.x] = lc1;
        for (int c = tid + 2 * (int)blockDim.x; c < nch; c += blockDim.x) s_dyn16[c] = load16(idx16 + c);
        __syncthreads();
    }
    if constexpr (SLOTS) {
        // free slot: clamped like the offsets above
        if (a.free_host < 0) fslot = min(max(s_meta[0], 0), a.N_cache - 1);
    }
    if constexpr (!EARLY) first_rows();

    double qd[EPT];
    {
        float qf[EPT];
        unpack<T>(qx, qf);
#pragma unroll
        for (int e = 0; e < EPT; ++e) qd[e] = (double)qf[e];
    }

    Softmax sm{kNegBig, 0.0f};
    float acc[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = 0.0f;
    double best_s = __builtin_inf();
    int best_d = -1, best_j = -1;

    // Consume one row: logit in fp64, argmin candidate, online softmax.  Rows
    // past this group's share (k >= nk) enter with logit -inf and weight 0:
    // selects instead of branches, so the loop below stays straight-line.
    auto consume = [&](int k, const uint4& kq, const uint4& vq, int d) {
        const bool valid = k < nk;
        const int r = g + k * G;
        float kf[EPT], vf[EPT];
        unpack<T>(kq, kf);
        unpack<T>(vq, vf);
        double part = 0.0;
#pragma unroll
        for (int e = 0; e < EPT; ++e) part = fma(qd[e], (double)kf[e], part);
        const double s = group_sum<TPR>(part);
        if constexpr (MODE == MODE_SPARSE || MODE == MODE_TOVA) {
            const bool cand = valid && a.select && d >= 0 && better(s, d, best_s, best_d);
            int jj = r - win0;  // sparse: list index
            if constexpr (MODE == MODE_TOVA) jj = jj == a.n_occ ? fslot : jj + (jj >= fslot ? 1 : 0);  // slot
            best_s = cand ? s : best_s;
            best_d = cand ? d : best_d;
            best_j = cand ? jj : best_j;
        }
        if constexpr (MODE == MODE_H2O) {
            if (valid && sl == 0) s_logit[r] = s;
        }
        const float x = valid ? (float)(s * a.scale_log2e) : -__builtin_inff();
        const float mn = fmaxf(sm.m, x);
        const float c = __builtin_amdgcn_exp2f(sm.m - mn);
        const float p = __builtin_amdgcn_exp2f(x - mn);
        sm.l = sm.l * c + p;
#pragma unroll
        for (int e = 0; e < EPT; ++e) acc[e] = acc[e] * c + p * vf[e];
        sm.m = mn;
    };

    // Rolling pipeline: consume row k from its buffer, then refill that buffer
    // with row k + U, so U - 1 rows stay in flight while one is computed.
    int k0 = 0;
    for (; k0 + U < nkw; k0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            consume(k0 + u, kx[u], vx[u], dd[u]);
            const T* kr;
            const T* vr;
            row_src(min(g + (k0 + u + U) * G, R - 1), kr, vr, dd[u]);
            kx[u] = load16_stream(kr + sl * EPT);
            vx[u] = load16_stream(vr + sl * EPT);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) consume(k0 + u, kx[u], vx[u], dd[u]);

    // Append: the new K/V row goes to its cache row.  Nothing this launch
    // reads lives there (it is empty, holds the entry evicted at this step, or
    // is the free slot); the current token itself is read from k_new / v_new.
    // Loaded at the start, stored here, so it adds no latency of its own.
    if (tid < CH) {
        T* row;
        if constexpr (MODE == MODE_SPARSE)
            row = const_cast<T*>(reinterpret_cast<const T*>(a.ring)) + ((size_t)a.self_row * a.lanes + lane) * ROW;
        else
            row = const_cast<T*>(lane_kv) + (size_t)(a.L_p + (SLOTS ? fslot : a.self_row)) * ROW;
        *reinterpret_cast<uint4*>(row + (tid / (CH / 2)) * D + (tid % (CH / 2)) * EPT) = ax;
    }

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

    // Across wavefronts: through LDS, merged in wave order by wave 0.
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
    if (wave != 0) return;

    if (wl < TPR) {
        for (int w = 1; w < nwaves; ++w) {
            float acc2[EPT];
#pragma unroll
            for (int e = 0; e < EPT; ++e) acc2[e] = s_acc[w][sl * EPT + e];
            merge<EPT>(sm, acc, s_m[w], s_l[w], acc2);
        }
        const float inv = 1.0f / sm.l;
        float4* o4 = reinterpret_cast<float4*>(a.out + (size_t)lane * D + sl * EPT);
#pragma unroll
        for (int e = 0; e < EPT; e += 4)
            o4[e / 4] = make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
    }

    if constexpr (MODE == MODE_SPARSE || MODE == MODE_TOVA) {
        if (wl != 0) return;
        for (int w = 1; w < nwaves; ++w) {
            if (s_bd[w] >= 0 && (best_d < 0 || better(s_bs[w], s_bd[w], best_s, best_d))) {
                best_s = s_bs[w];
                best_d = s_bd[w];
                best_j = s_bj[w];
            }
        }
        int chosen = -1;
        if constexpr (MODE == MODE_SPARSE) {
            int16_t* lst = a.list + (size_t)lane * a.list_stride;
            if (a.select) {
                // skip_idx.append(idx[j*]): offset best_d leaves the attended list
                // for good; the offset entering the window at t+1 takes its place.
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
        double m = -__builtin_inf();
        for (int r = wl; r < R; r += 64) m = fmax(m, s_logit[r]);
        m = wave_max(m);
        double l = 0.0;
        for (int r = wl; r < R; r += 64) l += exp((s_logit[r] - m) * c);
        l = wave_sum(l);
        double* sc = a.score + (size_t)lane * a.score_stride;
        const int lim = a.t - a.n_recent;
        double bkey = __builtin_inf();
        int bpos = 0x7fffffff, bslot = -1;
        for (int j = wl; j <= a.n_occ; j += 64) {
            const bool me = j == a.n_occ;
            const int slot = me ? fslot : min(j + (j >= fslot ? 1 : 0), a.N_cache - 1);
            const double p = exp((s_logit[win0 + j] - m) * c) / l;
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
    }
}

template <typename T, int D>
__global__ void prompt_kernel(PromptArgs a) {
    constexpr int EPT = Traits<T>::EPT;
    constexpr int CPR = D / EPT;  // 16-byte chunks per half-row
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
        const T* src = reinterpret_cast<const T*>(half ? a.v_p : a.k_p) +
                       (((size_t)b * a.L_p + j) * a.H + h) * D + c * EPT;
        const size_t lane = (size_t)b * a.H + h;
        T* dst = reinterpret_cast<T*>(a.kv) + (lane * (size_t)a.lane_rows + j) * 2 * D + half * D + c * EPT;
        *reinterpret_cast<uint4*>(dst) = load16(src);
    }
    if (a.list) {
        const int lanes = a.B * a.H;
        for (int l = blockIdx.x * blockDim.x + threadIdx.x; l < lanes; l += gridDim.x * blockDim.x)
            a.list[(size_t)l * a.list_stride] = 0;
    }
}

template <typename T, int D>
hipError_t launch_decode_t(int mode, int waves, const DecodeArgs& a, hipStream_t s) {
    constexpr int U = kRowsPerChunk;
    constexpr int TPR = D / Traits<T>::EPT;
    const int G = waves * (64 / TPR);
    dim3 grid(a.lanes), block(64 * waves);
    switch (mode) {
        case MODE_SPARSE: {
            const size_t lds = (size_t)((a.n_list + 7) / 8 > 0 ? (a.n_list + 7) / 8 : 1) * 16;
            if (U * G <= a.L_p + a.n_sink)
                hipLaunchKernelGGL((decode_kernel<T, D, MODE_SPARSE, U, true>), grid, block, lds, s, a);
            else
                hipLaunchKernelGGL((decode_kernel<T, D, MODE_SPARSE, U, false>), grid, block, lds, s, a);
            break;
        }
        case MODE_DENSE:
            hipLaunchKernelGGL((decode_kernel<T, D, MODE_DENSE, U, true>), grid, block, 0, s, a);
            break;
        case MODE_TOVA: {
            const size_t lds = (size_t)a.meta_stride * 4;
            if (U * G <= a.L_p)
                hipLaunchKernelGGL((decode_kernel<T, D, MODE_TOVA, U, true>), grid, block, lds, s, a);
            else
                hipLaunchKernelGGL((decode_kernel<T, D, MODE_TOVA, U, false>), grid, block, lds, s, a);
            break;
        }
        default: {  // MODE_H2O: slot metadata, then one fp64 logit per attended row
            const size_t lds = (size_t)a.meta_stride * 4 + (size_t)(a.L_p + a.N_cache) * 8;
            if (U * G <= a.L_p)
                hipLaunchKernelGGL((decode_kernel<T, D, MODE_H2O, U, true>), grid, block, lds, s, a);
            else
                hipLaunchKernelGGL((decode_kernel<T, D, MODE_H2O, U, false>), grid, block, lds, s, a);
            break;
        }
    }
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_prompt_t(const PromptArgs& a, hipStream_t s) {
    const long long chunks = (long long)a.B * a.H * a.L_p * 2 * (D / Traits<T>::EPT);
    long long blocks = (chunks + 255) / 256;
    const long long lane_blocks = ((long long)a.B * a.H + 255) / 256;
    if (blocks < lane_blocks) blocks = lane_blocks;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL((prompt_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(int mode, int dtype, int D, int waves, const DecodeArgs& a, hipStream_t s) {
    if (dtype == 1) {
        if (D == 128) return launch_decode_t<uint16_t, 128>(mode, waves, a, s);
        return launch_decode_t<uint16_t, 64>(mode, waves, a, s);
    }
    if (D == 128) return launch_decode_t<float, 128>(mode, waves, a, s);
    return launch_decode_t<float, 64>(mode, waves, a, s);
}

hipError_t launch_prompt(int dtype, int D, const PromptArgs& a, hipStream_t s) {
    if (dtype == 1) {
        if (D == 128) return launch_prompt_t<uint16_t, 128>(a, s);
        return launch_prompt_t<uint16_t, 64>(a, s);
    }
    if (D == 128) return launch_prompt_t<float, 128>(a, s);
    return launch_prompt_t<float, 64>(a, s);
}

}  // namespace dsa
