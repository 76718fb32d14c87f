// probe.hip -- a plain streaming read of a device buffer (16-byte loads, four
// in flight per thread, grid-stride), for measuring the HBM read rate a
// buffer of a given size attains on this device: the practical ceiling the
// decode kernels are compared with.  It computes nothing the method needs.
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {

typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fold(const u32x4v_t v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4v_t* __restrict__ p, long long n16,
                                                         uint32_t* sink) {
    const long long stride = (long long)gridDim.x * 256;
    long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4v_t a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
    }
    for (; i < n16; i += stride) acc ^= fold(p[i]);
    // the loads must not be dropped: their folded value decides a store that
    // in practice never happens (sink is one valid word either way)
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

hipError_t launch_read_probe(const void* buf, long long bytes, uint32_t* sink, int grid, hipStream_t stream) {
    if (bytes <= 0 || grid <= 0) return hipSuccess;
    hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(256), 0, stream, (const u32x4v_t*)buf, bytes / 16,
                       sink);
    return hipGetLastError();
}

}  // namespace kvq
