// Attention-map characterization on gfx950: the measurements of Section 3.4
// of "Understanding and Exploiting Diagonal Attention Sparsity in
// Autoregressive Image Generation" on the dense decode attention map of a
// workload (Fig. 8: attention mass on prompt / local / middle tokens; Fig. 10:
// vertical vs diagonal cosine similarity of attention score vectors).
//
// profile_map_kernel: one wavefront per (lane, 16 queries).  The logits
// Q K^T are a dense contraction, computed in 16 x 16 tiles with MFMA (bf16:
// v_mfma_f32_16x16x16_bf16, fp32: v_mfma_f32_16x16x4_f32; fp32 accumulation).
// Pass 1 keeps an online (max, sum) per query over the key tiles, pass 2
// recomputes the tiles, writes the decode probabilities P[i][j] (j <= i) and
// the per-query mass split.  No LDS holds a whole row, so T is not limited
// by LDS.
//
// profile_sim_kernel: one workgroup per (lane, query distance d); its
// wavefronts take queries i in turn and reduce the five dot products of
// rows i and i + d (P[i][0..i] against P[i+d][0..i] and P[i+d][d..i+d]).
// Workgroups go to the 8 XCDs round-robin, so the grid is ordered to give all
// distances of a lane the same XCD: they reread the lane's map from one L2.
#include <math.h>
#include <stdint.h>

#include "dsa_internal.h"

namespace dsa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short bf16x4 __attribute__((ext_vector_type(4)));

// 16 x 16 logit tile S[r][c] = q_{i0+r} . k_{c0+c} over D dimensions.  Lane l
// supplies row / column l % 16 and dimensions by l / 16; it receives
// S[4 (l / 16) + e][l % 16], e = 0..3.
template <typename T, int D>
__device__ __forceinline__ f32x4 logit_tile(const T* qrow, const T* krow) {
    const int quarter = threadIdx.x / 16;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int kk = 0; kk < D; kk += 16) {
            const bf16x4 a = *reinterpret_cast<const bf16x4*>(qrow + kk + 4 * quarter);
            const bf16x4 b = *reinterpret_cast<const bf16x4*>(krow + kk + 4 * quarter);
            acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
        }
    } else {
#pragma unroll
        for (int kk = 0; kk < D; kk += 4) {
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qrow[kk + quarter], krow[kk + quarter], acc, 0, 0, 0);
        }
    }
    return acc;
}

// Reductions over the 16 lanes that hold one query's tile columns.
__device__ __forceinline__ float max16(float v) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float sum16(float v) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
    return v;
}

template <typename T, int D>
__global__ void __launch_bounds__(64) profile_map_kernel(ProfileArgs a) {
    const int tiles = (a.T + 15) / 16;
    const int lane = blockIdx.x / tiles;
    const int i0 = (blockIdx.x % tiles) * 16;
    const int l = threadIdx.x;
    const int col = l % 16, quarter = l / 16;
    const int b = lane / a.H, h = lane % a.H;
    const T* q = reinterpret_cast<const T*>(a.q);
    const T* k = reinterpret_cast<const T*>(a.k);
    const T* kp = reinterpret_cast<const T*>(a.k_p);
    // A operand row: query i0 + col (rows past T repeat T - 1 and are not stored)
    const T* qrow = q + (((size_t)min(i0 + col, a.T - 1) * a.B + b) * a.H + h) * D;
    auto key_row = [&](int c) {  // key c: prompt row, then decode position c - L_p
        return c < a.L_p ? kp + (((size_t)b * a.L_p + c) * a.H + h) * D
                         : k + (((size_t)(c - a.L_p) * a.B + b) * a.H + h) * D;
    };
    const float scale = (float)(1.4426950408889634 / sqrt((double)D));  // log2(e) / sqrt(D)
    const int ncols = a.L_p + min(i0 + 16, a.T);                         // keys any of the 16 queries sees

    // pass 1: online (max, sum) in base 2 for the 4 queries 4 quarter + e
    float m[4], s[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        m[e] = -INFINITY;
        s[e] = 0.0f;
    }
    for (int c0 = 0; c0 < ncols; c0 += 16) {
        const int c = c0 + col;
        const f32x4 t = logit_tile<T, D>(qrow, key_row(min(c, ncols - 1)));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = i0 + 4 * quarter + e;
            const bool ok = c < ncols && c <= a.L_p + i;  // causal: keys up to decode position i
            const float x = ok ? t[e] * scale : -INFINITY;
            const float mn = fmaxf(m[e], max16(x));
            const float add = sum16(ok ? exp2f(x - mn) : 0.0f);
            s[e] = (m[e] == -INFINITY ? 0.0f : s[e] * exp2f(m[e] - mn)) + add;
            m[e] = mn;
        }
    }

    // pass 2: probabilities of the decode keys and the mass split
    float* P = a.P + (size_t)lane * a.T * a.T;
    float mp[4] = {0, 0, 0, 0}, ml[4] = {0, 0, 0, 0}, mm[4] = {0, 0, 0, 0};
    for (int c0 = 0; c0 < ncols; c0 += 16) {
        const int c = c0 + col;
        const f32x4 t = logit_tile<T, D>(qrow, key_row(min(c, ncols - 1)));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = i0 + 4 * quarter + e;
            const bool ok = i < a.T && c < ncols && c <= a.L_p + i;
            const float p = ok ? exp2f(t[e] * scale - m[e]) / s[e] : 0.0f;
            const int j = c - a.L_p;  // decode position of the key
            const int n_loc = (i + 10) / 10;
            mp[e] += c < a.L_p ? p : 0.0f;
            ml[e] += j >= 0 && j > i - n_loc ? p : 0.0f;
            mm[e] += j >= 0 && j <= i - n_loc ? p : 0.0f;
            if (ok && j >= 0) P[(size_t)i * a.T + j] = p;
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = i0 + 4 * quarter + e;
        const float vp = sum16(mp[e]), vl = sum16(ml[e]), vm = sum16(mm[e]);
        if (col == 0 && i < a.T) {
            float* r = a.mass_rows + ((size_t)lane * a.T + i) * 3;
            r[0] = vp;
            r[1] = vl;
            r[2] = vm;
        }
    }
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

constexpr int kSimWaves = 4;

__global__ void __launch_bounds__(64 * kSimWaves) profile_sim_kernel(ProfileArgs a) {
    // blockIdx -> (lane, distance) with every distance of a lane on one XCD:
    // block x goes to XCD x % 8; lanes are padded to a multiple of 8.
    const int x = blockIdx.x;
    const int lane = (x % 8) + 8 * (x / (8 * a.max_dist));
    const int dd = 1 + (x / 8) % a.max_dist;
    if (lane >= a.lanes) return;
    const int wave = threadIdx.x / 64, wl = threadIdx.x % 64;
    const float* P = a.P + (size_t)lane * a.T * a.T;
    const int n = a.T - dd;
    double sv = 0.0, sd = 0.0;
    for (int i = wave; i < n; i += kSimWaves) {
        const float* ra = P + (size_t)i * a.T;
        const float* rb = P + (size_t)(i + dd) * a.T;
        double ab = 0, ac = 0, aa = 0, bb = 0, cc = 0;
        for (int j = wl; j <= i; j += 64) {
            const double va = ra[j], vb = rb[j], vc = rb[j + dd];
            ab += va * vb;
            ac += va * vc;
            aa += va * va;
            bb += vb * vb;
            cc += vc * vc;
        }
        ab = wave_sum_d(ab);
        ac = wave_sum_d(ac);
        aa = wave_sum_d(aa);
        bb = wave_sum_d(bb);
        cc = wave_sum_d(cc);
        sv += ab / sqrt(aa * bb);
        sd += ac / sqrt(aa * cc);
    }
    __shared__ double s_v[kSimWaves], s_d[kSimWaves];
    if (wl == 0) {
        s_v[wave] = sv;
        s_d[wave] = sd;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double tv = 0, td = 0;
        for (int w = 0; w < kSimWaves; ++w) {
            tv += s_v[w];
            td += s_d[w];
        }
        a.vert[(size_t)lane * a.max_dist + dd - 1] = n > 0 ? tv / n : NAN;
        a.diag[(size_t)lane * a.max_dist + dd - 1] = n > 0 ? td / n : NAN;
    }
    if (dd == 1) {
        // the lane's mean mass split over its queries
        __syncthreads();
        if (wave == 0) {
            const float* r = a.mass_rows + (size_t)lane * a.T * 3;
            double g[3] = {0, 0, 0};
            for (int i = wl; i < a.T; i += 64) {
                g[0] += r[3 * i];
                g[1] += r[3 * i + 1];
                g[2] += r[3 * i + 2];
            }
            for (int c = 0; c < 3; ++c) {
                const double v = wave_sum_d(g[c]);
                if (wl == 0) a.mass[(size_t)lane * 3 + c] = v / a.T;
            }
        }
    }
}

template <typename T, int D>
hipError_t launch_profile_t(const ProfileArgs& a, hipStream_t s) {
    const int tiles = (a.T + 15) / 16;
    hipLaunchKernelGGL((profile_map_kernel<T, D>), dim3((unsigned)((long long)a.lanes * tiles)), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long lanes8 = ((long long)a.lanes + 7) / 8 * 8;
    hipLaunchKernelGGL(profile_sim_kernel, dim3((unsigned)(lanes8 * a.max_dist)), dim3(64 * kSimWaves), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_profile(int dtype, int D, const ProfileArgs& a, hipStream_t s) {
    if (dtype == 1) return D == 128 ? launch_profile_t<uint16_t, 128>(a, s) : launch_profile_t<uint16_t, 64>(a, s);
    return D == 128 ? launch_profile_t<float, 128>(a, s) : launch_profile_t<float, 64>(a, s);
}

}  // namespace dsa
