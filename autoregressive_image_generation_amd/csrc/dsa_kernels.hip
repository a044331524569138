// Decode-attention kernels for gfx950 (CDNA4): the fused diagonal-aware sparse
// step of "Understanding and Exploiting Diagonal Attention Sparsity in
// Autoregressive Image Generation" (Section 4, Algorithm 1; Section 5.1 for the
// fused gather + argmin design and the Diagonal+Sink4 variant) and the dense
// decode step it is compared with.
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
constexpr int kMaxList = 8192;  // DSA_MAX_ATTEND
constexpr float kNegBig = -1.0e30f;

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

template <typename T, int D, int MODE>
__global__ void __launch_bounds__(1024) decode_kernel(DecodeArgs a) {
    constexpr int EPT = Traits<T>::EPT;
    constexpr int TPR = D / EPT;          // threads per half-row
    constexpr int GPW = 64 / TPR;         // thread groups per wavefront
    constexpr int ROW = 2 * D;            // elements per cache row

    __shared__ int16_t s_list[MODE == MODE_SPARSE ? kMaxList : 1];
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

    // Append: the new K/V row goes to its cache row.  Nothing this launch
    // reads lives there (it is empty, or holds the entry evicted at this step);
    // the current token itself is read from k_new / v_new.
    {
        constexpr int CH = ROW * (int)sizeof(T) / 16;
        if (tid < CH) {
            const int half = tid / (CH / 2);
            const int c = tid % (CH / 2);
            const T* src = (half ? v_self : k_self) + c * EPT;
            T* dst = const_cast<T*>(lane_kv) + (size_t)(a.L_p + a.self_row) * ROW + half * D + c * EPT;
            *reinterpret_cast<uint4*>(dst) = load16(src);
        }
    }

    int R;
    if constexpr (MODE == MODE_SPARSE) {
        const int16_t* lst = a.list + (size_t)lane * a.N_attw;
        for (int j = tid; j < a.n_list; j += blockDim.x) s_list[j] = lst[j];
        R = a.L_p + a.n_sink + a.n_list;
        __syncthreads();
    } else {
        R = a.L_p + a.t + 1;
    }

    // The query chunk this thread multiplies, in fp64.
    double qd[EPT];
    {
        float qf[EPT];
        unpack<T>(load16(reinterpret_cast<const T*>(a.q) + (size_t)lane * D + sl * EPT), qf);
#pragma unroll
        for (int e = 0; e < EPT; ++e) qd[e] = (double)qf[e];
    }

    Softmax sm{kNegBig, 0.0f};
    float acc[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = 0.0f;
    double best_s = __builtin_inf();
    int best_d = -1, best_j = -1;

    const int win0 = a.L_p + a.n_sink;  // first window row (sparse)

    constexpr int U = 2;
    for (int r0 = g; r0 < R; r0 += G * U) {
        uint4 kx[U], vx[U];
        int dd[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = r0 + u * G;
            dd[u] = -1;
            if (r < R) {
                const T* kr;
                const T* vr;
                if (r < a.L_p) {
                    kr = lane_kv + (size_t)r * ROW;
                    vr = kr + D;
                } else if constexpr (MODE == MODE_DENSE) {
                    const int p = r - a.L_p;
                    if (p == a.t) {
                        kr = k_self;
                        vr = v_self;
                    } else {
                        kr = lane_kv + (size_t)r * ROW;
                        vr = kr + D;
                    }
                } else if (r < win0) {
                    const int p = r - a.L_p;  // sink position = sink slot
                    if (p == a.t) {
                        kr = k_self;
                        vr = v_self;
                    } else {
                        kr = lane_kv + (size_t)(a.L_p + p) * ROW;
                        vr = kr + D;
                    }
                } else {
                    // Offsets are written only by this kernel and lie in
                    // [0, N_rw); the clamp keeps a damaged workspace from
                    // turning into out-of-bounds reads.
                    const int d = min(max((int)s_list[r - win0], 0), a.N_rw - 1);
                    dd[u] = d;
                    if (d == 0) {
                        kr = k_self;
                        vr = v_self;
                    } else {
                        int slot = a.base - d;
                        if (slot < 0) slot += a.N_rw;
                        kr = lane_kv + (size_t)(a.L_p + a.S + slot) * ROW;
                        vr = kr + D;
                    }
                }
                kx[u] = load16(kr + sl * EPT);
                vx[u] = load16(vr + sl * EPT);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = r0 + u * G;
            if (r < R) {
                float kf[EPT], vf[EPT];
                unpack<T>(kx[u], kf);
                unpack<T>(vx[u], vf);
                double part = 0.0;
#pragma unroll
                for (int e = 0; e < EPT; ++e) part = fma(qd[e], (double)kf[e], part);
                const double s = group_sum<TPR>(part);
                if constexpr (MODE == MODE_SPARSE) {
                    if (a.select && dd[u] >= 0 && better(s, dd[u], best_s, best_d)) {
                        best_s = s;
                        best_d = dd[u];
                        best_j = r - win0;
                    }
                }
                const float x = (float)(s * a.scale_log2e);
                const float mn = fmaxf(sm.m, x);
                const float c = __builtin_amdgcn_exp2f(sm.m - mn);
                const float p = __builtin_amdgcn_exp2f(x - mn);
                sm.l = sm.l * c + p;
#pragma unroll
                for (int e = 0; e < EPT; ++e) acc[e] = acc[e] * c + p * vf[e];
                sm.m = mn;
            }
        }
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
        if constexpr (MODE == MODE_SPARSE) {
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
    if (wave != 0 || wl >= TPR) return;

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

    if constexpr (MODE == MODE_SPARSE) {
        if (wl != 0) return;
        for (int w = 1; w < nwaves; ++w) {
            if (s_bd[w] >= 0 && (best_d < 0 || better(s_bs[w], s_bd[w], best_s, best_d))) {
                best_s = s_bs[w];
                best_d = s_bd[w];
                best_j = s_bj[w];
            }
        }
        int16_t* lst = a.list + (size_t)lane * a.N_attw;
        int chosen = -1;
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
        if (a.trace) {
            a.trace[2 * lane] = chosen;
            a.trace[2 * lane + 1] = a.evicted;
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
            a.list[(size_t)l * a.N_attw] = 0;
    }
}

template <typename T, int D>
hipError_t launch_decode_t(int mode, int waves, const DecodeArgs& a, hipStream_t s) {
    dim3 grid(a.lanes), block(64 * waves);
    if (mode == MODE_SPARSE)
        hipLaunchKernelGGL((decode_kernel<T, D, MODE_SPARSE>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((decode_kernel<T, D, MODE_DENSE>), grid, block, 0, s, a);
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
