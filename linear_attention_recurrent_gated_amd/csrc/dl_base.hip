// Base import and export for gfx950: write the dense bases of a state block
// from fp32 states, or read them back as fp32 (the dense base of the DeltaLog
// page, "DeltaLog: Deferred Materialization of Recurrent States for Linear
// Attention Decoding", Technical Summary, Core Mechanism).  An fp32 base is a
// copy.  An INT8 base (DL_BASE_I8, a reading of the DAMP abstract: most of a
// recurrent state in INT8, a few channels chosen offline at higher precision)
// is quantised on import with the same row quantiser the merges use
// (q8_quantize_row in dl_common.hpp) and dequantised on export.
//
// One workgroup of 256 threads per (row, head); for an INT8 base the 8 lanes
// of a row group hold one value row (lane s: columns QW s .. QW s + QW - 1),
// 32 rows per pass.
#include "dl_common.hpp"

namespace dl {

template <int D>
__global__ void __launch_bounds__(256) base_import_kernel(Params P, const int *__restrict__ slot_idx,
                                                          const float *__restrict__ src) {
    const int H = P.heads;
    const int pr = blockIdx.x;
    const int r = pr / H, h = pr - r * H;
    const int tid = threadIdx.x;
    const int unit = slot_idx ? slot_idx[r] : r;
    if (unit < 0 || unit >= P.units) {
        reject_row(P, nullptr, D, DL_FLAG_BAD_SLOT);
        return;
    }
    const size_t pair = (size_t)unit * H + h;
    const float *in = src + (size_t)pr * D * D;
    if (!P.q8) {
        float4 *out = reinterpret_cast<float4 *>(P.base + pair * D * D);
        const float4 *x4 = reinterpret_cast<const float4 *>(in);
        for (int i = tid; i < D * D / 4; i += 256)
            out[i] = x4[i];
        return;
    }
    constexpr int QW = Q8Row<D>::QW;
    const int s = tid & 7;
    bool ok;
    const uint32_t kbits = q8_kept_bits<D>(P, h, s, ok);
    if (!ok) {
        reject_row(P, nullptr, D, DL_FLAG_BAD_KEPT);
        return;
    }
    for (int row = tid >> 3; row < D; row += 32) {
        float x[QW];
#pragma unroll
        for (int f = 0; f < QW; f += 4)
            f4_to(x + f, *reinterpret_cast<const float4 *>(in + (size_t)row * D + QW * s + f));
        uint32_t w[QW / 4];
        const float sc = q8_quantize_row<QW>(x, kbits, w);
        int8_t *cp = P.codes + (pair * D + row) * D + QW * s;
        if constexpr (QW == 16)
            *reinterpret_cast<uint4 *>(cp) = make_uint4(w[0], w[1], w[2], w[3]);
        else
            *reinterpret_cast<uint2 *>(cp) = make_uint2(w[0], w[1]);
        if (s == 0)
            P.scale[pair * D + row] = sc;
        for (int m = 0; m < P.M; ++m) {
            const int c = P.kidx[h * P.M + m];
            if (c / QW == s) {
                float v = 0.f;
#pragma unroll
                for (int f = 0; f < QW; ++f)
                    v = (f == c % QW) ? x[f] : v;
                P.kept[(pair * D + row) * P.M + m] = v;
            }
        }
    }
}

template <int D>
__global__ void __launch_bounds__(256) base_export_kernel(Params P, const int *__restrict__ slot_idx,
                                                          float *__restrict__ dst) {
    const int H = P.heads;
    const int pr = blockIdx.x;
    const int r = pr / H, h = pr - r * H;
    const int tid = threadIdx.x;
    float *out = dst + (size_t)pr * D * D;
    const int unit = slot_idx ? slot_idx[r] : r;
    if (unit < 0 || unit >= P.units) {
        for (int i = tid; i < D * D; i += 256)
            out[i] = __builtin_nanf("");
        reject_row(P, nullptr, D, DL_FLAG_BAD_SLOT);
        return;
    }
    const size_t pair = (size_t)unit * H + h;
    if (!P.q8) {
        const float4 *in = reinterpret_cast<const float4 *>(P.base + pair * D * D);
        float4 *o4 = reinterpret_cast<float4 *>(out);
        for (int i = tid; i < D * D / 4; i += 256)
            o4[i] = in[i];
        return;
    }
    constexpr int QW = Q8Row<D>::QW;
    const int s = tid & 7;
    for (int row = tid >> 3; row < D; row += 32) {
        uint32_t w[QW / 4];
        const int8_t *cp = P.codes + (pair * D + row) * D + QW * s;
        if constexpr (QW == 16) {
            const uint4 u = *reinterpret_cast<const uint4 *>(cp);
            w[0] = u.x, w[1] = u.y, w[2] = u.z, w[3] = u.w;
        } else {
            const uint2 u = *reinterpret_cast<const uint2 *>(cp);
            w[0] = u.x, w[1] = u.y;
        }
        float x[QW];
        q8_unpack<QW>(w, x);
        const float sc = P.scale[pair * D + row];
#pragma unroll
        for (int f = 0; f < QW; ++f)
            x[f] *= sc;
        for (int m = 0; m < P.M; ++m) {
            const int c = P.kidx[h * P.M + m];
            if (c >= 0 && c < D && c / QW == s) {
                const float v = P.kept[(pair * D + row) * P.M + m];
#pragma unroll
                for (int f = 0; f < QW; ++f)
                    x[f] = (f == c % QW) ? v : x[f];
            }
        }
#pragma unroll
        for (int f = 0; f < QW; f += 4)
            *reinterpret_cast<float4 *>(out + (size_t)row * D + QW * s + f) =
                make_float4(x[f], x[f + 1], x[f + 2], x[f + 3]);
    }
}

// Evenly spaced kept channels m D / M + D / (2 M) for every head.
__global__ void __launch_bounds__(256) kept_default_kernel(int *kidx, int heads, int M, int D) {
    for (int i = threadIdx.x; i < heads * M; i += 256) {
        const int m = i % M;
        kidx[i] = m * (D / M) + D / (2 * M);
    }
}

hipError_t launch_base_import(const Params &P, int rows, const int *slot_idx, const float *src,
                              const Launch &ln) {
    const dim3 grid(rows * P.heads), block(256);
    if (P.D == 128)
        hipExtLaunchKernelGGL(base_import_kernel<128>, grid, block, 0, ln.stream, ln.start, ln.stop, 0,
                              P, slot_idx, src);
    else
        hipExtLaunchKernelGGL(base_import_kernel<64>, grid, block, 0, ln.stream, ln.start, ln.stop, 0,
                              P, slot_idx, src);
    return hipGetLastError();
}

hipError_t launch_base_export(const Params &P, int rows, const int *slot_idx, float *dst,
                              const Launch &ln) {
    const dim3 grid(rows * P.heads), block(256);
    if (P.D == 128)
        hipExtLaunchKernelGGL(base_export_kernel<128>, grid, block, 0, ln.stream, ln.start, ln.stop, 0,
                              P, slot_idx, dst);
    else
        hipExtLaunchKernelGGL(base_export_kernel<64>, grid, block, 0, ln.stream, ln.start, ln.stop, 0,
                              P, slot_idx, dst);
    return hipGetLastError();
}

hipError_t launch_kept_default(const Params &P, const Launch &ln) {
    if (!P.q8 || P.M == 0)
        return hipSuccess;
    hipExtLaunchKernelGGL(kept_default_kernel, dim3(1), dim3(256), 0, ln.stream, ln.start, ln.stop, 0,
                          P.kidx, P.heads, P.M, P.D);
    return hipGetLastError();
}

}  // namespace dl
