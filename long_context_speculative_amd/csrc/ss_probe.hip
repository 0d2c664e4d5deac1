// Same-run HBM read reference of libssverify's measurement: how fast this
// device streams a buffer it only reads, with the history kernels' load
// shape (16-byte non-temporal loads, eight in flight per lane) and either
// their launch shape (one work-group per CU, each a contiguous span) or
// more work-groups. The history kernels' bandwidth is reported against it.

#include "ss_common.h"

namespace ssv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kDepth = 8;

__global__ __launch_bounds__(kThreads) void read_probe_kernel(const u32x4* __restrict__ src, int64_t n_vec,
                                                              int64_t per_wg, uint32_t* sink) {
    const int64_t begin = (int64_t)blockIdx.x * per_wg;
    int64_t end = begin + per_wg;
    if (end > n_vec) end = n_vec;
    uint32_t acc = 0;
    for (int64_t i = begin + threadIdx.x; i < end; i += (int64_t)kThreads * kDepth) {
        u32x4 v[kDepth];
#pragma unroll
        for (int j = 0; j < kDepth; ++j) {
            const int64_t k = i + (int64_t)j * kThreads;
            v[j] = k < end ? __builtin_nontemporal_load(&src[k]) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < kDepth; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    // keeps the loads alive; the sink is written only for one specific value
    if (acc == 0x9e3779b9u) sink[blockIdx.x & 255] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* src, int64_t bytes, int32_t n_wg, uint32_t* sink, hipStream_t stream) {
    const int64_t n_vec = bytes / 16;
    if (n_wg <= 0 || n_vec <= 0) return hipErrorInvalidValue;
    const int64_t per = (n_vec + n_wg - 1) / n_wg;
    hipLaunchKernelGGL(read_probe_kernel, dim3(n_wg), dim3(kThreads), 0, stream, static_cast<const u32x4*>(src), n_vec,
                       per, sink);
    return hipGetLastError();
}

}  // namespace ssv
