// probe.hip -- measurement probes for the benchmark (libtb_probe.so), not part of the path.
//
//   tbp_stream_read: reads a device buffer once with 16-byte non-temporal loads (the same
//                    load the GEMV kernels use) and folds it into one word per workgroup,
//                    to measure the achievable HBM read bandwidth.
//   tbp_clock:       per workgroup, shader-clock ticks (s_memtime) over a span of real-time
//                    ticks (s_memrealtime, 100 MHz): launched beside running kernels, the
//                    ratio is the shader clock they run at.
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

// One wave per workgroup; its first lane records the shader ticks that pass while the real-time
// counter advances by `ticks` (a bounded wait: it ends after ticks / 100 MHz).
__global__ __launch_bounds__(64) void clock_kernel(uint32_t ticks, unsigned long long *out)
{
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    unsigned long long r1 = r0;
    while (r1 - r0 < ticks) {
        __builtin_amdgcn_s_sleep(2);
        r1 = __builtin_amdgcn_s_memrealtime();
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    if (threadIdx.x == 0) {
        out[2 * blockIdx.x] = t1 - t0;
        out[2 * blockIdx.x + 1] = r1 - r0;
    }
}

}  // namespace

extern "C" {

// out: device uint64 array of 2 * grid entries (shader ticks, real-time ticks per workgroup);
// 1 <= ticks <= 10^7 (at most 0.1 s). Returns 0 or a HIP error code.
int tbp_clock(uint32_t ticks, unsigned long long *out, int grid, void *stream)
{
    if (!out || grid < 1 || ticks < 1 || ticks > 10000000u)
        return -1;
    hipLaunchKernelGGL(clock_kernel, dim3(grid), dim3(64), 0, static_cast<hipStream_t>(stream),
                       ticks, out);
    return (int)hipGetLastError();
}


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
