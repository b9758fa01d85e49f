// probe.hip -- measurement probes for the benchmark (libtb_probe.so), not part of the path.
//
//   tbp_stream_read: reads a device buffer once with 16-byte non-temporal loads (the same
//                    load the GEMV kernels use) and folds it into one word per workgroup,
//                    to measure the achievable HBM read bandwidth.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4 *__restrict__ buf,
                                                               size_t n16, uint32_t *sink)
{
    const size_t stride = (size_t)gridDim.x * kThreads;
    size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(buf + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // fold the workgroup so the loads stay live; one store per workgroup
    __shared__ uint32_t red[kThreads];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
        for (int t = 0; t < kThreads; ++t)
            s ^= red[t];
        sink[blockIdx.x] = s;
    }
}

}  // namespace

extern "C" {

// buf: device buffer of `bytes` bytes (16-byte aligned, bytes % 16 == 0);
// sink: device uint32 array of at least `grid` entries. Returns 0 or a HIP error code.
int tbp_stream_read(const void *buf, size_t bytes, uint32_t *sink, int grid, void *stream)
{
    if (!buf || !sink || grid < 1 || (bytes & 15) || ((uintptr_t)buf & 15))
        return -1;
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(buf),
                       bytes / 16, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
