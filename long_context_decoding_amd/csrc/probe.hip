// probe.hip -- a plain streaming read (measurement aid, not part of the decode path).
//
// The achievable HBM read bandwidth of the chip, measured with the simplest possible kernel, is
// the ceiling the decode kernels are compared with beside the vendor peak.  Each work-group
// reads one contiguous chunk of the buffer with 16-byte loads (eight in flight per lane) and
// writes the XOR of the 16-byte words it read, so that no load can be optimised away and the
// result can be checked.  The loads use the streaming (non-temporal) cache policy, which reads
// faster on this chip than the default one (as the decode kernels' streamed reads do).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ffd_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ src,
                                                               size_t n16, size_t chunk16,
                                                               uint4* __restrict__ sink)
{
    const size_t base = (size_t)blockIdx.x * chunk16;
    const size_t end = base + chunk16 < n16 ? base + chunk16 : n16;
    uint4 acc = make_uint4(0u, 0u, 0u, 0u);
    for (size_t i = base + threadIdx.x; i < end; i += (size_t)kThreads * kUnroll) {
        uint4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t k = i + (size_t)u * kThreads;
            if (k < end) {
                typedef unsigned v4u_t __attribute__((ext_vector_type(4)));
                const v4u_t x = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(src + k));
                v[u] = make_uint4(x[0], x[1], x[2], x[3]);
            } else {
                v[u] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            acc.x ^= v[u].x;
            acc.y ^= v[u].y;
            acc.z ^= v[u].z;
            acc.w ^= v[u].w;
        }
    }
    // XOR over the work-group: within each wave by shuffles, then across the waves in LDS
    __shared__ uint4 part[kThreads / 64];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        acc.x ^= __shfl_xor(acc.x, d);
        acc.y ^= __shfl_xor(acc.y, d);
        acc.z ^= __shfl_xor(acc.z, d);
        acc.w ^= __shfl_xor(acc.w, d);
    }
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint4 r = part[0];
        for (int w = 1; w < kThreads / 64; ++w) {
            r.x ^= part[w].x;
            r.y ^= part[w].y;
            r.z ^= part[w].z;
            r.w ^= part[w].w;
        }
        sink[blockIdx.x] = r;
    }
}

}  // namespace

extern "C" int32_t ffd_probe_stream_read(const void* src, size_t bytes, int32_t n_groups,
                                         void* sink, hipStream_t stream)
{
    if (!src || !sink || (reinterpret_cast<uintptr_t>(src) & 15u) ||
        (reinterpret_cast<uintptr_t>(sink) & 15u) || (bytes & 15u) || bytes == 0 ||
        n_groups < 1 || n_groups > 65535)
        return 1;
    const size_t n16 = bytes / 16;
    const size_t chunk16 = (n16 + (size_t)n_groups - 1) / (size_t)n_groups;
    hipLaunchKernelGGL(stream_read_kernel, dim3(n_groups), dim3(kThreads), 0, stream,
                       static_cast<const uint4*>(src), n16, chunk16, static_cast<uint4*>(sink));
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
