/*
 * Seeded synthetic Q/K/V for decode-attention workloads shaped like the
 * autoregressive image models of "Understanding and Exploiting Diagonal
 * Attention Sparsity in Autoregressive Image Generation" (arxiv 2609.19702).
 *
 * The pages publish no activations; this generator stands in for them.  It
 * holds none of the attention method's arithmetic: it only produces inputs,
 * and both the CPU oracle and the GPU library consume exactly these values.
 *
 * Recipe (one value per (stream, layer, batch, head, token, dim)):
 *   * Decode token n sits on a grid of width W at (r, c) = (n / W, n % W);
 *     every prompt token sits at (-1, -1).  Page 4, Table 1 gives the grid
 *     sizes (576 = 24x24, 4096 = 64x64, 8100 = 90x90).
 *   * Per (layer, head) base vectors a, b ~ N(0, 1)^d.  Q and K share a, V
 *     uses b, so q.k depends on the relative grid position of query and key:
 *     the spatial-locality origin of the diagonal pattern (page 4, Sec. 3.4,
 *     Fig. 11).
 *   * 2D rotary map Rot(r, c): the d/2 adjacent pairs (2i, 2i+1) are rotated,
 *     the first d/4 pairs by r * theta_m, the last d/4 by c * theta_m, with
 *     theta_m = 10000^(-m / (d/4)) and m the pair index inside its half.
 *   * x = Rot(r, c) base + 0.1 z, z ~ N(0, 1) i.i.d.
 *   * Normals: a counter hash H = mix(mix(mix(seed) ^ key1) ^ key2), mix being
 *     the splitmix64 finaliser (Steele, Lea, Flood 2014), gives 64 bits per
 *     group of four dims 4j .. 4j+3; its 16-bit fields, high to low, pick
 *     Phi^-1((i + 0.5) / 65536) from a table (quantised inverse-CDF sampling,
 *     tails cut at about 4.3 sigma).  All of it runs in fp64.
 *       key1 = stream << 56 | layer << 40 | head << 24 | batch
 *       key2 = token << 32 | j
 *   * The fp64 value is rounded to fp32 (round to nearest even) and, for
 *     bf16 output, the fp32 value is rounded again to bf16 (nearest even).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { SYN_Q = 0, SYN_K = 1, SYN_V = 2, SYN_KP = 3, SYN_VP = 4, SYN_BASE_A = 5, SYN_BASE_B = 6 };
enum { SYN_F32 = 0, SYN_BF16 = 1 };

static inline uint64_t mix64(uint64_t z) {
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint64_t counter_hash(uint64_t seed, uint64_t stream, uint64_t layer, uint64_t batch,
                                    uint64_t head, uint64_t token, uint64_t pair) {
    uint64_t key1 = (stream << 56) | (layer << 40) | (head << 24) | batch;
    uint64_t key2 = (token << 32) | pair;
    return mix64(mix64(mix64(seed) ^ key1) ^ key2);
}

/*
 * N(0, 1) by quantised inverse-CDF sampling: a 16-bit field i gives
 * Phi^-1((i + 0.5) / 65536), so one 64-bit hash yields four normals.  The
 * table is filled once by bisection on Phi(x) = erfc(-x / sqrt 2) / 2.
 */
static double normal_table[65536];
static int normal_table_ready = 0;

static void build_normal_table(void) {
    if (normal_table_ready) return;
    for (int i = 0; i < 65536; ++i) {
        double p = ((double)i + 0.5) / 65536.0;
        double lo = -12.0, hi = 12.0;
        for (int it = 0; it < 200; ++it) {
            double mid = 0.5 * (lo + hi);
            if (0.5 * erfc(-mid / sqrt(2.0)) < p) lo = mid; else hi = mid;
        }
        normal_table[i] = 0.5 * (lo + hi);
    }
    normal_table_ready = 1;
}

static inline void normal_quad(uint64_t h, double z[4]) {
    z[0] = normal_table[(h >> 48) & 0xffff];
    z[1] = normal_table[(h >> 32) & 0xffff];
    z[2] = normal_table[(h >> 16) & 0xffff];
    z[3] = normal_table[h & 0xffff];
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static void base_vector(uint64_t seed, int stream, int layer, int head, int d, double* out) {
    for (int j = 0; j < d / 4; ++j) {
        uint64_t h = counter_hash(seed, (uint64_t)stream, (uint64_t)layer, 0, (uint64_t)head, 0, (uint64_t)j);
        normal_quad(h, &out[4 * j]);
    }
}

/* Rot(r, c) applied to base, written to y. */
static void rotate(const double* base, int d, int r, int c, double* y) {
    int quarter = d / 4;
    for (int p = 0; p < d / 2; ++p) {
        int m = p < quarter ? p : p - quarter;
        double theta = pow(10000.0, -(double)m / (double)quarter);
        double phi = (p < quarter ? (double)r : (double)c) * theta;
        double cs = cos(phi), sn = sin(phi);
        double x0 = base[2 * p], x1 = base[2 * p + 1];
        y[2 * p] = x0 * cs - x1 * sn;
        y[2 * p + 1] = x0 * sn + x1 * cs;
    }
}

/*
 * Fill out[(tok - tok0) * s_tok + (b - b0) * s_b + (h - h0) * s_h + i] for
 * tokens tok0 .. tok0 + ntok - 1, batches b0 .. b0 + nb - 1, heads h0 .. h0 + nh - 1,
 * dims i < d.  Strides are in elements.  Decode streams (Q, K, V) place token n
 * on a grid of width grid_w; prompt streams (KP, VP) place every token at (-1, -1).
 * Returns 0, or -1 on bad arguments.
 */
int synth_fill(uint64_t seed, int stream, int layer, int d, int grid_w, int b0, int nb, int h0, int nh,
               int tok0, int ntok, long long s_tok, long long s_b, long long s_h, int dtype, void* out,
               int nthreads) {
    if (stream < SYN_Q || stream > SYN_VP || d < 4 || d % 4 || nb < 0 || nh < 0 || ntok < 0 || tok0 < 0 ||
        b0 < 0 || h0 < 0 || layer < 0 || layer >= 65536 || h0 + nh > 65536 || b0 + nb > (1 << 24) ||
        (dtype != SYN_F32 && dtype != SYN_BF16) || !out)
        return -1;
    int prompt = (stream == SYN_KP || stream == SYN_VP);
    if (!prompt && grid_w < 1) return -1;
    int base_stream = (stream == SYN_V || stream == SYN_VP) ? SYN_BASE_B : SYN_BASE_A;
    build_normal_table();
    double* bases = (double*)malloc(sizeof(double) * (size_t)d * (size_t)(nh > 0 ? nh : 1));
    if (!bases) return -1;
    for (int h = 0; h < nh; ++h) base_vector(seed, base_stream, layer, h0 + h, d, bases + (size_t)h * d);
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double* rot = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(static)
        for (int n = 0; n < ntok; ++n) {
            int tok = tok0 + n;
            int r = prompt ? -1 : tok / grid_w;
            int c = prompt ? -1 : tok % grid_w;
            for (int h = 0; h < nh; ++h) {
                rotate(bases + (size_t)h * d, d, r, c, rot);
                for (int b = 0; b < nb; ++b) {
                    long long o = (long long)n * s_tok + (long long)b * s_b + (long long)h * s_h;
                    for (int j = 0; j < d / 4; ++j) {
                        uint64_t hh = counter_hash(seed, (uint64_t)stream, (uint64_t)layer, (uint64_t)(b0 + b),
                                                   (uint64_t)(h0 + h), (uint64_t)tok, (uint64_t)j);
                        double z[4];
                        normal_quad(hh, z);
                        for (int e = 0; e < 4; ++e) {
                            float v = (float)(rot[4 * j + e] + 0.1 * z[e]);
                            if (dtype == SYN_F32)
                                ((float*)out)[o + 4 * j + e] = v;
                            else
                                ((uint16_t*)out)[o + 4 * j + e] = f32_to_bf16_rne(v);
                        }
                    }
                }
            }
        }
        free(rot);
    }
    free(bases);
    return 0;
}
