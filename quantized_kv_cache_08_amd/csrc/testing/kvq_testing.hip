// kvq_testing.hip -- libkvq_testing.so (include/kvq_testing.h): device
// conversions and a streaming read for tests and measurement, and the decode
// kernels' split plan evaluated on the host.  Not part of the method.
#include "kvq_testing.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "split_plan.h"

#pragma clang fp contract(off)

namespace kvq {

// The encoders of the append kernel (kvq_device.h) on plain float arrays.
__global__ __launch_bounds__(256) void e4m3_encode_kernel(const float* x, uint8_t* codes,
                                                          long long n) {
    const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i + 3 < n) {
        const float* p = x + i;
        uint32_t w = e4m3_encode4(p[0], p[1], p[2], p[3]);
        codes[i] = (uint8_t)w;
        codes[i + 1] = (uint8_t)(w >> 8);
        codes[i + 2] = (uint8_t)(w >> 16);
        codes[i + 3] = (uint8_t)(w >> 24);
    } else {
        for (long long j = i; j < n; ++j) codes[j] = (uint8_t)e4m3_encode4(x[j], 0.f, 0.f, 0.f);
    }
}

__global__ __launch_bounds__(256) void e5m2_encode_kernel(const float* x, uint8_t* codes,
                                                          long long n) {
    const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i + 3 < n) {
        const float* p = x + i;
        uint32_t w = e5m2_encode4(p[0], p[1], p[2], p[3]);
        codes[i] = (uint8_t)w;
        codes[i + 1] = (uint8_t)(w >> 8);
        codes[i + 2] = (uint8_t)(w >> 16);
        codes[i + 3] = (uint8_t)(w >> 24);
    } else {
        for (long long j = i; j < n; ++j) codes[j] = (uint8_t)e5m2_encode4(x[j], 0.f, 0.f, 0.f);
    }
}

typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fold(const u32x4v_t v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Plain streaming read: workgroup windows of L x 256 16-byte elements, thread t
// loading elements t, t + 256, ... of its window (L loads in flight), windows
// grid-stride.  A window cut by the end of the buffer is read up to the end.
template <int L>
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4v_t* __restrict__ p, long long n16,
                                                         uint32_t* sink) {
    const long long step = (long long)gridDim.x * 256 * L;
    long long i = (long long)blockIdx.x * 256 * L + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 256 * (L - 1) < n16; i += step) {
        u32x4v_t v[L];
#pragma unroll
        for (int k = 0; k < L; ++k) v[k] = p[i + 256 * k];
#pragma unroll
        for (int k = 0; k < L; ++k) acc ^= fold(v[k]);
    }
    for (; i < n16; i += 256) acc ^= fold(p[i]);   // the last, partial window
    // the loads must not be dropped: their folded value decides a store that
    // in practice never happens (sink is one valid word either way)
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace kvq

using namespace kvq;

extern "C" {

kvq_status kvq_e4m3_encode(const float* x, uint8_t* codes, int64_t n, hipStream_t stream) {
    if (n < 0) return KVQ_EINVAL;
    if (n == 0) return KVQ_OK;
    if (!x || !codes) return KVQ_EINVAL;
    const long long grid = (n + 1023) / 1024;
    hipLaunchKernelGGL(e4m3_encode_kernel, dim3((unsigned)grid), dim3(256), 0, stream, x, codes, (long long)n);
    return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EHIP;
}

kvq_status kvq_e5m2_encode(const float* x, uint8_t* codes, int64_t n, hipStream_t stream) {
    if (n < 0) return KVQ_EINVAL;
    if (n == 0) return KVQ_OK;
    if (!x || !codes) return KVQ_EINVAL;
    const long long grid = (n + 1023) / 1024;
    hipLaunchKernelGGL(e5m2_encode_kernel, dim3((unsigned)grid), dim3(256), 0, stream, x, codes, (long long)n);
    return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EHIP;
}

kvq_status kvq_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int32_t blocks_per_cu,
                          int32_t loads_per_thread, hipStream_t stream) {
    const bool loads_ok = loads_per_thread >= 1 && loads_per_thread <= 8 && loads_per_thread != 5 &&
                          loads_per_thread != 7;
    if (bytes < 0 || (bytes & 15) || blocks_per_cu <= 0 || blocks_per_cu > 32 || !loads_ok) return KVQ_EINVAL;
    if (bytes == 0) return KVQ_OK;
    if (!buf || !sink) return KVQ_EINVAL;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return KVQ_EHIP;
    const dim3 grid(cus * blocks_per_cu);
    const u32x4v_t* b = (const u32x4v_t*)buf;
    const long long n16 = bytes / 16;
    switch (loads_per_thread) {
        case 1: hipLaunchKernelGGL(read_probe_kernel<1>, grid, dim3(256), 0, stream, b, n16, sink); break;
        case 2: hipLaunchKernelGGL(read_probe_kernel<2>, grid, dim3(256), 0, stream, b, n16, sink); break;
        case 3: hipLaunchKernelGGL(read_probe_kernel<3>, grid, dim3(256), 0, stream, b, n16, sink); break;
        case 4: hipLaunchKernelGGL(read_probe_kernel<4>, grid, dim3(256), 0, stream, b, n16, sink); break;
        case 6: hipLaunchKernelGGL(read_probe_kernel<6>, grid, dim3(256), 0, stream, b, n16, sink); break;
        default: hipLaunchKernelGGL(read_probe_kernel<8>, grid, dim3(256), 0, stream, b, n16, sink); break;
    }
    return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EHIP;
}

kvq_status kvq_plan_stats(int32_t page_size, int32_t num_kv_heads, int32_t total_waves,
                          const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                          int32_t partition_pages, kvq_plan_info* info) {
    if (!info || page_size <= 0 || num_kv_heads <= 0 || total_waves <= 0 || num_seqs < 0 ||
        max_context_len < 0 || partition_pages < 0 || (num_seqs > 0 && !context_lens))
        return KVQ_EINVAL;
    *info = kvq_plan_info{};
    const int B = num_seqs;
    const int max_pages = (max_context_len + page_size - 1) / page_size;
    int pmin = 0x7FFFFFFF, pmax = 0;
    for (int i = 0; i < B; ++i) {
        const int pg = pages_of(context_lens[i], max_context_len, page_size);
        pmin = std::min(pmin, pg);
        pmax = std::max(pmax, pg);
    }
    const int cost = segment_cost(pmin, pmax);
    std::vector<long long> pfx(B + 1, 0);
    for (int i = 0; i < B; ++i)
        pfx[i + 1] = pfx[i] + item_weight(pages_of(context_lens[i], max_context_len, page_size), cost);
    const long long S = pfx[B];
    const int min_chunk = partition_pages > 0 ? partition_pages : plan_min_chunk(max_pages);
    const long long chunk = plan_chunk(S, total_waves, num_kv_heads, min_chunk, partition_pages);
    const long long R = (S + chunk - 1) / chunk;
    info->chunk = chunk;
    info->ranges_per_head = R;
    info->cost = cost;
    info->slots = plan_slots(B, num_kv_heads, std::max(1, max_pages), partition_pages);
    auto pf = [&](int i) { return pfx[i]; };
    auto uni = [](int v) { return v; };
    for (long long r = 0; r < R; ++r) {
        bool busy = false;
        walk_range(r, chunk, S, B, cost, pf, uni, [&](int, int page0, int page1, int slot, int n_seg) {
            if (page1 > page0) busy = true;
            info->segments_per_head += 1;
            info->slots_used = std::max<int64_t>(info->slots_used, (int64_t)slot + 1);
            info->max_segments_per_item = std::max(info->max_segments_per_item, n_seg);
        });
        info->busy_ranges_per_head += busy ? 1 : 0;
    }
    return KVQ_OK;
}

}  // extern "C"
