// Streaming-rate calibration for gfx950: a plain read of a buffer, or a plain
// copy, in the access pattern the state kernels use for their largest stream
// (16-byte nontemporal loads and stores, 256 threads per workgroup, the
// workgroup's U loads per thread 4 KiB apart).  It is not part of the method:
// it measures what the memory system delivers to a kernel that does nothing
// else, the practical ceiling to set beside the published peak.
#include "dl_common.hpp"

namespace dl {

typedef float f32x4p __attribute__((ext_vector_type(4)));

// Each workgroup reads 256 * RU float4 and writes their sum (one float).
constexpr int RU = 8;
// Each workgroup copies 256 * CU float4 (all loads issued before the stores).
constexpr int CU = 4;

__global__ void __launch_bounds__(256) probe_read_kernel(const f32x4p *__restrict__ x, size_t n4,
                                                         float *__restrict__ out) {
    __shared__ float part[4];
    const size_t base = (size_t)blockIdx.x * 256 * RU + threadIdx.x;
    f32x4p acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < RU; ++u) {
        const size_t i = base + (size_t)u * 256;
        if (i < n4)
            acc += __builtin_nontemporal_load(x + i);
    }
    float s = (acc.x + acc.y) + (acc.z + acc.w);
    for (int off = 32; off > 0; off >>= 1)
        s += __shfl_xor(s, off);
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0)
        out[blockIdx.x] = (part[0] + part[1]) + (part[2] + part[3]);
}

__global__ void __launch_bounds__(256) probe_copy_kernel(const f32x4p *__restrict__ x,
                                                         f32x4p *__restrict__ y, size_t n4) {
    const size_t base = (size_t)blockIdx.x * 256 * CU + threadIdx.x;
    f32x4p v[CU];
#pragma unroll
    for (int u = 0; u < CU; ++u) {
        const size_t i = base + (size_t)u * 256;
        v[u] = i < n4 ? __builtin_nontemporal_load(x + i) : f32x4p{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < CU; ++u) {
        const size_t i = base + (size_t)u * 256;
        if (i < n4)
            __builtin_nontemporal_store(v[u], y + i);
    }
}

size_t probe_read_outputs(size_t bytes) {
    const size_t n4 = bytes / 16;
    return (n4 + 256 * (size_t)RU - 1) / (256 * (size_t)RU);
}

hipError_t launch_stream_probe(int mode, const void *src, void *dst, size_t bytes, const Launch &ln) {
    const size_t n4 = bytes / 16;
    if (mode == 0) {
        const dim3 grid((unsigned)probe_read_outputs(bytes));
        hipExtLaunchKernelGGL(probe_read_kernel, grid, dim3(256), 0, ln.stream, ln.start, ln.stop, 0,
                              static_cast<const f32x4p *>(src), n4, static_cast<float *>(dst));
    } else {
        const dim3 grid((unsigned)((n4 + 256 * (size_t)CU - 1) / (256 * (size_t)CU)));
        hipExtLaunchKernelGGL(probe_copy_kernel, grid, dim3(256), 0, ln.stream, ln.start, ln.stop, 0,
                              static_cast<const f32x4p *>(src), static_cast<f32x4p *>(dst), n4);
    }
    return hipGetLastError();
}

}  // namespace dl
