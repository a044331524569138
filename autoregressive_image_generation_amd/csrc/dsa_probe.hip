// HBM read probe: the practical read-bandwidth ceiling of the device, against
// which the decode kernels' achieved bandwidth is read (a measurement utility,
// not part of the attention method).
//
// Every thread streams 16-byte chunks with a grid-stride loop, UNR chunks in
// flight per iteration, loaded non-temporal like the decode kernels' cache
// rows.  Each thread's XOR of what it read decides a store to one 32-bit sink
// word that real data practically never triggers (a magic value), so the
// loads cannot be dropped and the kernel normally writes nothing.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "dsa_internal.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kProbeMagic = 0x9e3779b9u;

template <int UNR>
__global__ void hbm_read_probe_kernel(const u32x4* __restrict__ src, size_t n16, uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (size_t)(UNR - 1) * stride < n16; i += (size_t)UNR * stride) {
        u32x4 v[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) v[u] = __builtin_nontemporal_load(src + i + (size_t)u * stride);
#pragma unroll
        for (int u = 0; u < UNR; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == kProbeMagic) *sink = acc;  // every thread that matches stores the same value
}

}  // namespace

namespace dsa {

hipError_t launch_hbm_read_probe(const void* src, size_t bytes, int blocks, int threads, int unroll, uint32_t* sink,
                                 hipStream_t s) {
    const size_t n16 = bytes / 16;
    const auto* p = reinterpret_cast<const u32x4*>(src);
    if (unroll == 1)
        hipLaunchKernelGGL(hbm_read_probe_kernel<1>, dim3(blocks), dim3(threads), 0, s, p, n16, sink);
    else if (unroll == 4)
        hipLaunchKernelGGL(hbm_read_probe_kernel<4>, dim3(blocks), dim3(threads), 0, s, p, n16, sink);
    else
        hipLaunchKernelGGL(hbm_read_probe_kernel<8>, dim3(blocks), dim3(threads), 0, s, p, n16, sink);
    return hipGetLastError();
}

}  // namespace dsa
