// Attention-map characterization on gfx950: the measurements of Section 3.4
// of "Understanding and Exploiting Diagonal Attention Sparsity in
// Autoregressive Image Generation" on the dense decode attention map of a
// workload (Fig. 8: attention mass on prompt / local / middle tokens; Fig. 10:
// vertical vs diagonal cosine similarity of attention score vectors).
//
// profile_map_kernel: one wavefront per (lane, 16 queries), four per
// workgroup sharing each 16-key tile through LDS.  The logits Q K^T are a
// dense contraction, computed in 16 x 16 tiles with MFMA (bf16:
// v_mfma_f32_16x16x16_bf16, fp32: v_mfma_f32_16x16x4_f32; fp32 sums), the
// query operand held in registers.  Pass 1 takes each query's maximum logit
// m over its key columns; pass 2 recomputes the tiles and writes the decode
// weights P[i][j] = 2^(x - m) (j <= i; x the logit in base 2): each row is
// the row of probabilities times the row's softmax sum, which leaves every
// cosine below unchanged.  The mass split divides each key group's sum of
// weights by the row's total.
//
// profile_gram_kernel: every similarity term is a band of a Gram matrix.
// With Q[i][o] = P[i][i - o] (the map in offset coordinates: o = i - j),
//   vertical dot   sum_j P[i][j] P[i+d][j]        = (P P^T)[i][i+d]
//   diagonal dot   sum_j P[i][j] P[i+d][j+d]      = (Q Q^T)[i][i+d]
//   |P[i+d][0..i]|^2                             = (L (P.P)^T)[i][i+d]
//   |P[i+d][d..i+d]|^2                           = (L (Q.Q)^T)[i][i+d]
//   |P[i][0..i]|^2                               = (P P^T)[i][i]
// with L[i][k] = 1 for k <= i (P[i][k] = 0 beyond k = i).  A workgroup of
// four wavefronts takes 64 rows; each wavefront computes the 16 x 16 tiles
// of the four products for its 16 rows and the columns i + 1 .. i +
// max_dist, four column tiles per pass, from 16-column chunks of the rows
// staged once for all four wavefronts in LDS (padded strides: no bank
// conflicts; the next chunk is loaded into registers while the current one
// is consumed), and adds each cosine into per-distance sums.  The two Gram
// products take each value split into two bf16 parts (hi = bf16(x), lo =
// bf16(x - hi), so x = hi + lo + r with |r| <= 2^-18 |x|) and sum hi.hi +
// hi.lo + lo.hi with bf16 MFMA (v_mfma_f32_16x16x16_bf16, one step per
// 16-column chunk): every partial product is exact in fp32, and each term
// x y is missed by less than 2^-16 |x y| (the dropped lo.lo and r terms).  The norms stay in fp32 (plain sums of squares left of a tile,
// v_mfma_f32_16x16x4_f32 with L across it).
// profile_reduce_kernel: per lane, the sums over row tiles in order, the
// means, and the mean mass split.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/dsa.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short bf16x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct MfmaIn;
template <>
struct MfmaIn<uint16_t> {  // bf16: 16 dimensions per step, 4 per lane
    using Op = bf16x4;
    static constexpr int STEP = 16, PER = 4;
    __device__ static Op load(const uint16_t* p) { return *reinterpret_cast<const bf16x4*>(p); }
    __device__ static f32x4 mfma(Op a, Op b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0); }
};
template <>
struct MfmaIn<float> {  // fp32: 4 dimensions per step, 1 per lane
    using Op = float;
    static constexpr int STEP = 4, PER = 1;
    __device__ static Op load(const float* p) { return *p; }
    __device__ static f32x4 mfma(Op a, Op b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }
};

// Each wavefront of a workgroup takes 16 consecutive queries (kMapWaves x 16
// per workgroup); keys are staged in LDS kMapKeys at a time, once per
// workgroup (coalesced 16-byte loads), and read by every wavefront as
// 16-key MFMA tiles; the next stage is loaded into registers while the
// current one is consumed.  Lane l supplies tile row / column l % 16 and
// dimensions by l / 16 of each MFMA step.  The tile is computed as K Q^T
// (keys the A operand), so lane l receives the logits of query l % 16 with
// the four consecutive keys 4 (l / 16) + e, e = 0..3: one 16-byte store of
// the row's weights per lane and tile.
constexpr int kMapWaves = 4;
constexpr int kMapKeys = 64;  // keys per LDS stage: four 16-key tiles

// One LDS stage of keys c0 .. c0 + kMapKeys - 1 of a lane (past the last key
// of the group: repeats it; prompt keys first, then decode keys) held in
// registers between its load and its store into LDS: 16-byte chunk x of the
// stage (key x / RCH, part x % RCH) is thread x mod 256's entry x / 256.
template <typename T, int D>
struct KeyStage {
    static constexpr int RCH = D * (int)sizeof(T) / 16;  // 16-byte chunks of a key row
    // LDS row stride in 8-byte units: a key row plus 8 bytes, so that the 16
    // rows of an MFMA operand read start in different banks
    static constexpr int RSTR = 2 * RCH + 1;
    static constexpr int NPF = kMapKeys * RCH / (64 * kMapWaves);
    static_assert(kMapKeys * RCH % (64 * kMapWaves) == 0, "whole chunks per thread");
    u32x4 v[NPF];  // a native vector type (HIP's uint4 is a union wrapper that kept the array in scratch)

    __device__ __forceinline__ void load(const T* kp, const T* k, int L_p, int B, int H, int b, int h, int ncols,
                                         int c0) {
#pragma unroll
        for (int n = 0; n < NPF; ++n) {
            const int x = threadIdx.x + n * 64 * kMapWaves;
            const int c = min(c0 + x / RCH, ncols - 1);
            const T* prow = kp + (((size_t)b * L_p + min(c, max(L_p - 1, 0))) * H + h) * D;
            const T* drow = k + (((size_t)max(c - L_p, 0) * B + b) * H + h) * D;
            const T* krow = c < L_p ? prow : drow;
            v[n] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(krow) + (x % RCH) * 16);
        }
    }
    __device__ __forceinline__ void store(u32x2* s_kt) const {
#pragma unroll
        for (int n = 0; n < NPF; ++n) {
            const int x = threadIdx.x + n * 64 * kMapWaves;
            u32x2* dst = s_kt + (x / RCH) * RSTR + 2 * (x % RCH);  // 8-byte aligned: two stores
            dst[0] = v[n].xy;
            dst[1] = v[n].zw;
        }
    }
};

// Logits of a staged 16-key tile against a wavefront's 16 queries (operand
// qa), keys as the rows of the product; krow: this lane's key row and
// dimension offset in LDS.
template <typename T, int D>
__device__ __forceinline__ f32x4 map_tile(const T* krow, const typename MfmaIn<T>::Op (&qa)[D / MfmaIn<T>::STEP]) {
    using M = MfmaIn<T>;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < D / M::STEP; ++s) acc = M::mfma(M::load(krow + s * M::STEP), qa[s], acc);
    return acc;
}

template <typename T, int D>
__global__ void __launch_bounds__(64 * kMapWaves) profile_map_kernel(ProfileArgs a) {
    using M = MfmaIn<T>;
    constexpr int NS = D / M::STEP;
    constexpr int RSTR = KeyStage<T, D>::RSTR;      // LDS row stride in 8-byte units
    // blockIdx -> (lane, query tile) with all query tiles of a lane on one
    // XCD (workgroup x runs on XCD x % 8; lanes are padded to a multiple of
    // 8): the tiles read overlapping key ranges, from one L2.
    const int tiles = (a.T + 16 * kMapWaves - 1) / (16 * kMapWaves);
    const int x = blockIdx.x;
    const int lane = (x % 8) + 8 * (x / (8 * tiles));
    const int tile = (x / 8) % tiles;
    if (lane >= a.lanes) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);  // uniform: scalar branches below
    const int i0 = tile * 16 * kMapWaves + 16 * wave;  // this wavefront's first query
    const int l = threadIdx.x % 64;
    const int col = l % 16, quarter = l / 16;
    const int b = lane / a.H, h = lane % a.H;
    const T* q = reinterpret_cast<const T*>(a.q);
    const T* k = reinterpret_cast<const T*>(a.k);
    const T* kp = reinterpret_cast<const T*>(a.k_p);
    __shared__ u32x2 s_kt[kMapKeys * RSTR];  // the current stage of keys, key-major
    const T* s_k = reinterpret_cast<const T*>(s_kt);
    // the query operand: row i0 + col (rows past T repeat T - 1 and are not stored)
    typename M::Op qa[NS];
    {
        const T* qrow = q + (((size_t)min(i0 + col, a.T - 1) * a.B + b) * a.H + h) * D + M::PER * quarter;
#pragma unroll
        for (int s = 0; s < NS; ++s) qa[s] = M::load(qrow + s * M::STEP);
    }
    const int ncols = a.L_p + min(tile * 16 * kMapWaves + 16 * kMapWaves, a.T);  // keys of the group
    // (the stage is used directly, not through lambdas: captured by
    // reference, its registers would be demoted to scratch memory)
    KeyStage<T, D> pf;
    const float scale = (float)(1.4426950408889634 / sqrt((double)D));  // log2(e) / sqrt(D)
    // The keys causal for all of this wavefront's queries (0 .. first_key) and
    // for any of them (0 .. last_key); a wavefront wholly past T has none.
    const int first_key = i0 + 15 < a.T ? min(a.L_p + i0, ncols - 1) : -1;
    const int last_key = a.L_p + min(i0 + 15, a.T - 1);

    // this lane's query, and its keys c = cmin + 4 quarter + e of each tile
    const int i = i0 + col;

    // pass 1: the maximum logit of this lane's query over its columns (this
    // lane's four keys per tile, then the four lanes of the query merged)
    float m = -INFINITY;
    pf.load(kp, k, a.L_p, a.B, a.H, b, h, ncols, 0);
    for (int c0 = 0; c0 < ncols; c0 += kMapKeys) {
        __syncthreads();
        pf.store(s_kt);
        __syncthreads();
        // unconditional (past the last key it rereads it): no merge of old and new registers
        pf.load(kp, k, a.L_p, a.B, a.H, b, h, ncols, c0 + kMapKeys);
#pragma unroll
        for (int tp = 0; tp < kMapKeys / 16; tp += 2) {
            // two tiles' MFMA chains, then their softmax work
            f32x4 ts[2];
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2)
                ts[q2] = map_tile<T, D>(s_k + (16 * (tp + q2) + col) * (RSTR * 8 / (int)sizeof(T)) + M::PER * quarter, qa);
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
                const int cmin = c0 + 16 * (tp + q2);
                if (cmin >= ncols || cmin > last_key) break;
                const int c = cmin + 4 * quarter;
                const f32x4 t = ts[q2];
                if (cmin + 15 <= first_key) {  // every key causal for every query (uniform)
                    m = fmaxf(m, fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])));
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool ok = c + e < ncols && c + e <= a.L_p + i;
                        m = ok ? fmaxf(m, t[e]) : m;
                    }
                }
            }
        }
    }
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    m *= scale;  // scale > 0: the maximum of the scaled logits

    // pass 2: the weights 2^(x - m) of the decode keys (the probabilities up to
    // the row's normaliser: the cosines do not depend on a row's scale) and
    // the mass of each key group, divided by the row's total at the end
    float* const Prow = a.P + ((size_t)lane * a.T + min(i, a.T - 1)) * a.T;  // stored only for i < T
    // 16-byte stores where every row and every decode quad starts 16-byte
    // aligned (then no quad mixes prompt and decode keys), else per element
    const bool vec = a.T % 4 == 0 && a.L_p % 4 == 0;
    // the decode columns j0 .. j0 + 3 of this lane's query, up to the causal
    // limit j <= i (and j < T)
    auto store_quad = [&](int j0, float p0, float p1, float p2, float p3) {
        if (vec && j0 >= 0 && j0 + 3 <= i) {
            *reinterpret_cast<float4*>(Prow + j0) = make_float4(p0, p1, p2, p3);
        } else {
            const float pe[4] = {p0, p1, p2, p3};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (j0 + e >= 0 && j0 + e <= i && j0 + e < a.T) Prow[j0 + e] = pe[e];
        }
    };
    float mp = 0.0f, ml = 0.0f, mm = 0.0f;
    pf.load(kp, k, a.L_p, a.B, a.H, b, h, ncols, 0);
    for (int c0 = 0; c0 < ncols; c0 += kMapKeys) {
        __syncthreads();
        pf.store(s_kt);
        __syncthreads();
        // unconditional (past the last key it rereads it): no merge of old and new registers
        pf.load(kp, k, a.L_p, a.B, a.H, b, h, ncols, c0 + kMapKeys);
#pragma unroll
        for (int tp = 0; tp < kMapKeys / 16; tp += 2) {
            f32x4 ts[2];
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2)
                ts[q2] = map_tile<T, D>(s_k + (16 * (tp + q2) + col) * (RSTR * 8 / (int)sizeof(T)) + M::PER * quarter, qa);
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
                const int cmin = c0 + 16 * (tp + q2);
                if (cmin >= ncols || cmin > last_key) break;
                const int c = cmin + 4 * quarter;
                const f32x4 t = ts[q2];
                const int j0 = c - a.L_p;  // decode position of this lane's first key
                // Uniform over the wavefront: every key of the tile causal for every
                // query, and then all prompt keys, or all decode keys of every query's
                // middle group (at most i - ceil((i + 1) / 10), which does not decrease
                // with i): no masks, no mass-split selects.  Else the general path.
                const bool full = cmin + 15 <= first_key;
                if (full && cmin + 15 < a.L_p) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) mp += __builtin_amdgcn_exp2f(t[e] * scale - m);
                } else if (full && cmin >= a.L_p && cmin + 15 - a.L_p <= i0 - (i0 + 10) / 10) {
                    float p[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        p[e] = __builtin_amdgcn_exp2f(t[e] * scale - m);
                        mm += p[e];
                    }
                    store_quad(j0, p[0], p[1], p[2], p[3]);
                } else {
                    const int n_loc = (i + 10) / 10;  // local group: ceil((i + 1) / 10) most recent
                    float p[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = j0 + e;
                        const bool ok = i < a.T && c + e < ncols && j <= i;
                        p[e] = ok ? __builtin_amdgcn_exp2f(t[e] * scale - m) : 0.0f;
                        mp += j < 0 ? p[e] : 0.0f;
                        ml += j >= 0 && j > i - n_loc ? p[e] : 0.0f;
                        mm += j >= 0 && j <= i - n_loc ? p[e] : 0.0f;
                    }
                    if (i < a.T && c < ncols) store_quad(j0, p[0], p[1], p[2], p[3]);
                }
            }
        }
    }
    // the query's sums over its four lanes
    mp += __shfl_xor(mp, 16);
    ml += __shfl_xor(ml, 16);
    mm += __shfl_xor(mm, 16);
    mp += __shfl_xor(mp, 32);
    ml += __shfl_xor(ml, 32);
    mm += __shfl_xor(mm, 32);
    if (quarter == 0 && i < a.T) {
        const float inv = 1.0f / (mp + ml + mm);
        float* r = a.mass_rows + ((size_t)lane * a.T + i) * 3;
        r[0] = mp * inv;
        r[1] = ml * inv;
        r[2] = mm * inv;
    }
}

constexpr int kGramWaves = 4;  // row tiles per workgroup (one per wavefront)
constexpr int kGramJ = 4;      // column tiles per pass (accumulators: 4 products x 4 tiles)
constexpr int kGChunk = 16;    // staged columns per LDS chunk: one bf16 MFMA step
// A staged row in LDS, per form (P or Q): the chunk's 16 values as four
// quads of 4 columns, each quad its 4 bf16 hi parts then its 4 bf16 lo parts
// (one 16-byte read is a lane's operand pair), then 16 bytes of padding, so
// that the 16 rows of an operand read fall into different banks.
constexpr int kGRow = 80;  // bytes per staged row and form

typedef short bf16x4v __attribute__((ext_vector_type(4)));

// Four fp32 values split into bf16 hi = bf16(x) and lo = bf16(x - hi) (round
// to nearest even), so x = hi + lo + r with |r| <= 2^-18 |x|: the words
// (hi0 hi1, hi2 hi3, lo0 lo1, lo2 lo3), element 0 in the low half.
__device__ __forceinline__ u32x4 split_quad(f32x4 x) {
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    const bf16x2v h01 = {(__bf16)x[0], (__bf16)x[1]};
    const bf16x2v h23 = {(__bf16)x[2], (__bf16)x[3]};
    const uint32_t h0 = __builtin_bit_cast(uint32_t, h01), h1 = __builtin_bit_cast(uint32_t, h23);
    const bf16x2v l01 = {(__bf16)(x[0] - __uint_as_float(h0 << 16)), (__bf16)(x[1] - __uint_as_float(h0 & 0xffff0000u))};
    const bf16x2v l23 = {(__bf16)(x[2] - __uint_as_float(h1 << 16)), (__bf16)(x[3] - __uint_as_float(h1 & 0xffff0000u))};
    return u32x4{h0, h1, __builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23)};
}

// The hi (words 0, 1) and lo (words 2, 3) halves of a staged quad as MFMA
// operands.  The halves go through named temporaries: this compiler's
// __builtin_bit_cast of a swizzle such as w.zw reads w.xy instead.
__device__ __forceinline__ bf16x4v quad_hi(const u32x4& w) {
    const u32x2 h = {w[0], w[1]};
    return __builtin_bit_cast(bf16x4v, h);
}
__device__ __forceinline__ bf16x4v quad_lo(const u32x4& w) {
    const u32x2 l = {w[2], w[3]};
    return __builtin_bit_cast(bf16x4v, l);
}

// hi + lo of element e of a staged quad (exact in fp32: both parts are bf16
// values 8 bits apart at most).
__device__ __forceinline__ float quad_value(const u32x4& w, int e) {
    const uint32_t h = e < 2 ? w[0] : w[1], l = e < 2 ? w[2] : w[3];
    const uint32_t hb = e % 2 ? (h & 0xffff0000u) : (h << 16), lb = e % 2 ? (l & 0xffff0000u) : (l << 16);
    return __uint_as_float(hb) + __uint_as_float(lb);
}

// The value of lane CTRL names inside this lane's quad (DPP quad_perm; every
// lane of the quad is active where it is used).
template <int CTRL>
__device__ __forceinline__ float quad_swap(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Four consecutive floats at a 4-byte aligned address (one 16-byte load).
__device__ __forceinline__ f32x4 load_f4(const float* p) {
    f32x4 v;
    __builtin_memcpy(&v, p, sizeof(v));
    return v;
}

// Columns [k0, k0 + kGChunk) of NROWS rows r0.. of the map, as P (row-major,
// zero beyond the causal part and past T) and as Q (offset coordinates:
// Q[r][o] = P[r][r - o], zero for o > r), held in registers as quads: quad u
// of the chunk (row u / 4, columns or offsets 4 (u % 4) .. + 3) is thread
// u mod 256's entry u / 256.  A quad whose four entries are all causal is one
// 16-byte load (the Q quad reversed), the others are loaded entry by entry.
template <int NROWS>
struct Staged {
    static constexpr int NQ = NROWS * kGChunk / 4;
    static constexpr int N = (NQ + 64 * kGramWaves - 1) / (64 * kGramWaves);
    f32x4 p[N], q[N];

    // Issue the loads (they complete while the current chunk is consumed).
    __device__ __forceinline__ void load(const float* P, int T, int r0, int k0) {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const int u = threadIdx.x + 64 * kGramWaves * n;
            const int r = r0 + u / 4, c0 = k0 + 4 * (u % 4);
            p[n] = q[n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (u < NQ && r < T) {
                const float* row = P + (size_t)r * T;
                if (c0 + 3 <= r) {
                    p[n] = load_f4(row + c0);
                    const f32x4 v = load_f4(row + (r - c0 - 3));
                    q[n] = f32x4{v[3], v[2], v[1], v[0]};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (c0 + e <= r) {
                            p[n][e] = row[c0 + e];
                            q[n][e] = row[r - c0 - e];
                        }
                    }
                }
            }
        }
    }
    // Store the quads split into bf16 hi / lo: one 16-byte store per form.
    // With SQ, also each row's sum of squares over the chunk (fp32, of the
    // unsplit values), per form: the four quads of a row sit in four
    // consecutive lanes, which DPP adds.
    template <bool SQ>
    __device__ __forceinline__ void store(char* sp, char* sq, float* ssp, float* ssq) const {
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const int u = threadIdx.x + 64 * kGramWaves * n;
            if (u < NQ) {  // NQ is a multiple of 4: whole rows, so all four lanes of a quad group take part
                const int off = (u / 4) * kGRow + (u % 4) * 16;
                *reinterpret_cast<u32x4*>(sp + off) = split_quad(p[n]);
                *reinterpret_cast<u32x4*>(sq + off) = split_quad(q[n]);
                if constexpr (SQ) {
                    float a = 0.0f, b = 0.0f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        a = fmaf(p[n][e], p[n][e], a);
                        b = fmaf(q[n][e], q[n][e], b);
                    }
                    a += quad_swap<0xB1>(a);  // quad_perm [1,0,3,2]
                    b += quad_swap<0xB1>(b);
                    a += quad_swap<0x4E>(a);  // quad_perm [2,3,0,1]
                    b += quad_swap<0x4E>(b);
                    if (u % 4 == 0) {
                        ssp[u / 4] = a;
                        ssq[u / 4] = b;
                    }
                }
            }
        }
    }
};

// A workgroup takes 64 rows I0 .. I0+63, wavefront w the row tile I = I0 +
// 16 w.  A pass covers the column tiles J = I + 64 g + 16 c (c < 4) of every
// wavefront: their rows, I0 + 64 g .. I0 + 64 g + 111, are staged once per
// chunk for all four wavefronts (pass 0 holds the A rows among them; later
// passes stage the A rows apart).  Dynamic LDS: (112 [+ 64]) rows x 2 forms x
// kGRow bytes.
// MULTI: distances beyond one pass (max_dist > 16 kGramJ - 15): later passes
// stage the A rows apart.  The one-pass form holds no registers for them and
// fits three wavefronts per SIMD.
template <bool MULTI>
__global__ void __launch_bounds__(64 * kGramWaves) __attribute__((amdgpu_waves_per_eu(3)))
profile_gram_kernel(ProfileArgs a) {
    // blockIdx -> (lane, row block) with all row blocks of a lane on one XCD
    // (workgroup x runs on XCD x % 8; lanes are padded to a multiple of 8):
    // they reread the lane's map from one L2.
    const int tiles = (a.T + 15) / 16;
    const int blocks = (tiles + kGramWaves - 1) / kGramWaves;
    const int x = blockIdx.x;
    const int lane = (x % 8) + 8 * (x / (8 * blocks));
    const int bi = (x / 8) % blocks;
    if (lane >= a.lanes) return;
    const int I0 = bi * 16 * kGramWaves;
    const int wave = threadIdx.x / 64, l = threadIdx.x % 64, col = l % 16, quarter = l / 16;
    const int I = I0 + 16 * wave;
    const float* P = a.P + (size_t)lane * a.T * a.T;

    constexpr int NB = 16 * (kGramWaves + kGramJ - 1);  // B rows of a pass: 112
    constexpr int NA = 16 * kGramWaves;  // A rows staged apart (later passes only)
    extern __shared__ u32x4 s_gram[];    // 16-byte aligned
    char* const sPB = reinterpret_cast<char*>(s_gram);
    char* const sQB = sPB + NB * kGRow;
    char* const sPA = sQB + NB * kGRow;
    char* const sQA = sPA + NA * kGRow;
    __shared__ double s_sum[2 * kMaxProfileDist];  // per distance: vertical, diagonal
    __shared__ float s_na[16 * kGramWaves];        // |P[i][0..i]|^2 of the block's rows
    __shared__ float s_sqP[NB], s_sqQ[NB];         // each B row's sum of squares over the staged chunk
    for (int d = threadIdx.x; d < 2 * a.max_dist; d += 64 * kGramWaves) s_sum[d] = 0.0;

    const int kend = min(I0 + 16 * kGramWaves, a.T);                 // P[i][k] = 0 for k > i
    const int span = 15 + a.max_dist;                                // columns i' - I needed: 0 .. span
    const int passes = MULTI ? span / (16 * kGramJ) + 1 : 1;
    for (int g = 0; g < passes; ++g) {
        const int J0 = I + 16 * kGramJ * g;  // this wavefront's first column tile of the pass
        f32x4 gv[kGramJ], gd[kGramJ], nb[kGramJ], nc[kGramJ];
        float sb[kGramJ], sc[kGramJ];  // sums of squares of the B rows over the chunks left of the tile
#pragma unroll
        for (int c = 0; c < kGramJ; ++c) {
            gv[c] = gd[c] = nb[c] = nc[c] = f32x4{0, 0, 0, 0};
            sb[c] = sc[c] = 0.0f;
        }
        const int aoff = 16 * wave;            // this wavefront's A rows in that buffer
        const char* const saP = g == 0 ? sPB : sPA;
        const char* const saQ = g == 0 ? sQB : sQA;
        // The chunk's Gram products, all 16 columns in one step per product:
        // bf16 MFMA (16 x 16 x 16) of the split operands, hi.hi + hi.lo + lo.hi.
        // Lane l holds columns 4 (l / 16) .. + 3 of row l % 16 of A and of B.
        auto gram_chunk = [&]() {
            const int ao = (aoff + col) * kGRow + 16 * quarter;
            const u32x4 pa = *reinterpret_cast<const u32x4*>(saP + ao);
            const u32x4 qa = *reinterpret_cast<const u32x4*>(saQ + ao);
            const bf16x4v pah = quad_hi(pa), pal = quad_lo(pa);
            const bf16x4v qah = quad_hi(qa), qal = quad_lo(qa);
#pragma unroll
            for (int c = 0; c < kGramJ; ++c) {
                const int bo = (16 * (wave + c) + col) * kGRow + 16 * quarter;
                const u32x4 pb = *reinterpret_cast<const u32x4*>(sPB + bo);
                const u32x4 qb = *reinterpret_cast<const u32x4*>(sQB + bo);
                const bf16x4v pbh = quad_hi(pb), pbl = quad_lo(pb);
                const bf16x4v qbh = quad_hi(qb), qbl = quad_lo(qb);
                gv[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pah, pbh, gv[c], 0, 0, 0);
                gd[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(qah, qbh, gd[c], 0, 0, 0);
                gv[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pah, pbl, gv[c], 0, 0, 0);
                gd[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(qah, qbl, gd[c], 0, 0, 0);
                gv[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pal, pbh, gv[c], 0, 0, 0);
                gd[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(qal, qbh, gd[c], 0, 0, 0);
            }
        };
        // the next chunk's rows are loaded into registers while this one is
        // consumed from LDS
        Staged<NB> nxB;
        Staged<16 * kGramWaves> nxA;
        nxB.load(P, a.T, I0 + 16 * kGramJ * g, 0);
        if (MULTI && g > 0) nxA.load(P, a.T, I0, 0);
        for (int k0 = 0; k0 < kend; k0 += kGChunk) {
            __syncthreads();
            nxB.template store<true>(sPB, sQB, s_sqP, s_sqQ);
            if (MULTI && g > 0) nxA.template store<false>(sPA, sQA, nullptr, nullptr);
            __syncthreads();
            if (k0 + kGChunk < kend) {
                nxB.load(P, a.T, I0 + 16 * kGramJ * g, k0 + kGChunk);
                if (MULTI && g > 0) nxA.load(P, a.T, I0, k0 + kGChunk);
            }
            if (I < a.T && k0 + kGChunk - 1 < I) {
                // every column of the chunk lies left of the tile's first row:
                // L is 1 for all (i, k), so the prefix norms add the B rows'
                // sums of squares over the chunk, taken at staging (the lanes
                // of quarter 0 add them; the quarters are summed at the end)
                gram_chunk();
                if (quarter == 0) {
#pragma unroll
                    for (int c = 0; c < kGramJ; ++c) {
                        sb[c] += s_sqP[16 * (wave + c) + col];
                        sc[c] += s_sqQ[16 * (wave + c) + col];
                    }
                }
            } else if (I < a.T && k0 <= I + 15) {  // past I + 15 this wavefront's A rows are zero
                // A rows are zero past column I + 15, so the Gram step may
                // run over all 16 columns
                // (the staged entries past T or past a row's causal part are
                // zero, so the steps run over all 16 columns)
                gram_chunk();
                u32x4 pbq[kGramJ], qbq[kGramJ];  // this lane's quads of the B rows J0 + 16 c + col
#pragma unroll
                for (int c = 0; c < kGramJ; ++c) {
                    const int bo = (16 * (wave + c) + col) * kGRow + 16 * quarter;
                    pbq[c] = *reinterpret_cast<const u32x4*>(sPB + bo);
                    qbq[c] = *reinterpret_cast<const u32x4*>(sQB + bo);
                }
                // step e: lane (col, quarter) supplies L[I + col][k] and the B
                // rows' squares at column k = k0 + 4 quarter + e (its k index
                // is quarter in both operands), so the four steps cover the
                // chunk's 16 columns once
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float ind = (k0 + 4 * quarter + e <= I + col) ? 1.0f : 0.0f;  // L[I + col][k]
#pragma unroll
                    for (int c = 0; c < kGramJ; ++c) {
                        const float xp = quad_value(pbq[c], e), xq = quad_value(qbq[c], e);
                        nb[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(ind, xp * xp, nb[c], 0, 0, 0);
                        nc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(ind, xq * xq, nc[c], 0, 0, 0);
                    }
                }
            }
        }
        // the plain sums: over the four quarters of each column, added to
        // every row of the tile
#pragma unroll
        for (int c = 0; c < kGramJ; ++c) {
            float tb = sb[c] + __shfl_xor(sb[c], 16);
            float tc = sc[c] + __shfl_xor(sc[c], 16);
            tb += __shfl_xor(tb, 32);
            tc += __shfl_xor(tc, 32);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                nb[c][e] += tb;
                nc[c][e] += tc;
            }
        }
        // lane holds entries (i, i') = (I + 4 quarter + e, J0 + 16 c + col)
        if (g == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * quarter + e == col) s_na[16 * wave + col] = gv[0][e];
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < kGramJ; ++c) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = I + 4 * quarter + e, ip = J0 + 16 * c + col, d = ip - i;
                if (i < a.T && ip < a.T && d >= 1 && d <= a.max_dist) {
                    // fp32 cosines of the fp32 sums (v_rsq_f32 is within about
                    // one ulp, far below the sums' own rounding); fp64 means
                    const float ra = __builtin_amdgcn_rsqf(s_na[16 * wave + 4 * quarter + e]);
                    atomicAdd(&s_sum[2 * (d - 1)], (double)(gv[c][e] * ra * __builtin_amdgcn_rsqf(nb[c][e])));
                    atomicAdd(&s_sum[2 * (d - 1) + 1], (double)(gd[c][e] * ra * __builtin_amdgcn_rsqf(nc[c][e])));
                }
            }
        }
    }
    __syncthreads();
    // one partial row per 16-row tile keeps the reduce kernel's layout: the
    // block's sums go to its first tile, the others are zero
    const int nt = min(kGramWaves, tiles - bi * kGramWaves);
    for (int t = 0; t < nt; ++t) {
        double* part = a.partial + ((size_t)lane * tiles + bi * kGramWaves + t) * 2 * a.max_dist;
        for (int d = threadIdx.x; d < 2 * a.max_dist; d += 64 * kGramWaves) part[d] = t == 0 ? s_sum[d] : 0.0;
    }
}

size_t gram_lds_bytes(int max_dist) {
    const int passes = (15 + max_dist) / (16 * kGramJ) + 1;
    const int rows = 16 * (kGramWaves + kGramJ - 1) + (passes > 1 ? 16 * kGramWaves : 0);
    return (size_t)rows * 2 * kGRow;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__global__ void __launch_bounds__(64) profile_reduce_kernel(ProfileArgs a) {
    const int lane = blockIdx.x;
    const int l = threadIdx.x;
    const int tiles = (a.T + 15) / 16;
    const double* part = a.partial + (size_t)lane * tiles * 2 * a.max_dist;
    for (int x = l; x < 2 * a.max_dist; x += 64) {
        double sum = 0.0;
        for (int t = 0; t < tiles; ++t) sum += part[(size_t)t * 2 * a.max_dist + x];
        const int d = x / 2 + 1, n = a.T - d;
        (x % 2 ? a.diag : a.vert)[(size_t)lane * a.max_dist + d - 1] = sum / n;
    }
    const float* r = a.mass_rows + (size_t)lane * a.T * 3;
    double g[3] = {0, 0, 0};
    for (int i = l; i < a.T; i += 64) {
        g[0] += r[3 * i];
        g[1] += r[3 * i + 1];
        g[2] += r[3 * i + 2];
    }
    for (int c = 0; c < 3; ++c) {
        const double v = wave_sum_d(g[c]);
        if (l == 0) a.mass[(size_t)lane * 3 + c] = v / a.T;
    }
}

template <typename T, int D>
hipError_t launch_profile_t(const ProfileArgs& a, hipStream_t s) {
    const int tiles = (a.T + 15) / 16;
    const int map_tiles = (a.T + 16 * kMapWaves - 1) / (16 * kMapWaves);
    const long long lanes8 = ((long long)a.lanes + 7) / 8 * 8;  // both grids: lanes padded to whole XCD rounds
    hipLaunchKernelGGL((profile_map_kernel<T, D>), dim3((unsigned)(lanes8 * map_tiles)), dim3(64 * kMapWaves), 0, s,
                       a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int blocks = (tiles + kGramWaves - 1) / kGramWaves;
    const bool multi = (15 + a.max_dist) / (16 * kGramJ) + 1 > 1;
    if (multi)
        hipLaunchKernelGGL(profile_gram_kernel<true>, dim3((unsigned)(lanes8 * blocks)), dim3(64 * kGramWaves),
                           gram_lds_bytes(a.max_dist), s, a);
    else
        hipLaunchKernelGGL(profile_gram_kernel<false>, dim3((unsigned)(lanes8 * blocks)), dim3(64 * kGramWaves),
                           gram_lds_bytes(a.max_dist), s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(profile_reduce_kernel, dim3((unsigned)a.lanes), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace

// Scratch of dsa_attention_profile_static: the map, the per-query mass and
// the per-tile sums of a profile, in device memory the library itself holds
// (each GPU the library runs on keeps its own copy until the process ends),
// for callers that cannot allocate a workspace.  Host code never passes this
// name to a kernel: its device address comes from hipGetSymbolAddress, once
// per device, below.
static __device__ __align__(256) char scratch[DSA_PROFILE_STATIC_SCRATCH_BYTES];

hipError_t profile_static_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_profile(int dtype, int D, const ProfileArgs& a, hipStream_t s) {
    if (dtype == 1) return D == 128 ? launch_profile_t<uint16_t, 128>(a, s) : launch_profile_t<uint16_t, 64>(a, s);
    return D == 128 ? launch_profile_t<float, 128>(a, s) : launch_profile_t<float, 64>(a, s);
}

}  // namespace dsa
