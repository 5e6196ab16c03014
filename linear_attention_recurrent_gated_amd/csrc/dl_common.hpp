// Internal device/host definitions of the gfx950 decode-state library.
//
// State of one (unit, head): S, d_v x d_k fp32, row-major (row = value
// channel).  A workgroup of 256 threads (4 wave64s) owns one (unit, head) in
// the step and merge kernels.  Inside a wave, lanes form 8 groups of 8: a
// group owns one state row at a time; lane s of the group holds the columns
// {4s + 32m + e : m < D/32, e < 4}, i.e. D/8 floats per row loaded as float4
// chunks, so one load instruction of a group reads 128 contiguous bytes of
// a row and every group holds a whole key-dimension vector.  Row dot
// products end in an 8-lane DPP butterfly that leaves the bitwise-identical
// sum in all 8 lanes.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "deltalog.h"

namespace dl {

enum Variant { GDN = DL_GDN, KDA = DL_KDA, RWKV6 = DL_RWKV6 };

// Device-side view of one state block (all pointers into caller memory).
struct Params {
    int variant, units, heads, D, L, dtype;
    float *base;
    void *log_k;
    void *log_v;
    float *log_g;
    float *log_beta;
    int *fill;
    int *flags;
};

template <int D>
struct Shape {
    static constexpr int NW = 4;               // waves per workgroup
    static constexpr int NT = 64 * NW;         // threads per workgroup
    static constexpr int NCH = D / 32;         // float4 chunks per lane per row
    static constexpr int FPL = 4 * NCH;        // floats per lane per row
    static constexpr int RPW = D / NW;         // rows per wave
    static constexpr int ITER = RPW / 8;       // rows per lane group
    static_assert(D == 64 || D == 128, "d must be 64 or 128");
};

__device__ __forceinline__ int col_of(int s, int m, int e) { return 4 * s + 32 * m + e; }

// ---------------------------------------------------------------------------
// input element access: fp32 or bf16 (stored as uint16 bit patterns)
// ---------------------------------------------------------------------------
template <typename T>
struct Elem;

template <>
struct Elem<float> {
    __device__ static __forceinline__ float4 load4(const float *p) {
        return *reinterpret_cast<const float4 *>(p);
    }
    __device__ static __forceinline__ float load1(const float *p) { return *p; }
};

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

template <>
struct Elem<uint16_t> {
    __device__ static __forceinline__ float4 load4(const uint16_t *p) {
        const uint2 u = *reinterpret_cast<const uint2 *>(p);
        return make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
    }
    __device__ static __forceinline__ float load1(const uint16_t *p) {
        return __uint_as_float(static_cast<uint32_t>(*p) << 16);
    }
};

__device__ __forceinline__ void f4_to(float *dst, float4 x) {
    dst[0] = x.x; dst[1] = x.y; dst[2] = x.z; dst[3] = x.w;
}

// ---------------------------------------------------------------------------
// 8-lane butterfly sum with DPP: quad xor 1, quad xor 2, half-row mirror.
// All 8 lanes of the group end with the same bits (the adds commute).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float sum8(float x) {
    x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp_mov<0x141>(x);   // row_half_mirror
    return x;
}

// ---------------------------------------------------------------------------
// LDS carve-up for staged log entries (step, readout and merge kernels).
// k entries in the input dtype, decays already exponentiated (alpha), betas.
// ---------------------------------------------------------------------------
struct LdsPlan {
    int off_k, off_a, off_b, off_v, off_q, off_c, bytes;
    int v_stride;  // bytes per staged value row (padded against bank conflicts)
};

__host__ __device__ inline int align16(int x) { return (x + 15) & ~15; }

// entries: number of log rows the plan must hold; with_v: stage values too.
__host__ __device__ inline LdsPlan lds_plan(int variant, int D, int esize, int entries,
                                            int L, bool with_v) {
    LdsPlan p;
    const int ach = (variant == DL_GDN) ? 1 : D;
    p.off_k = 0;
    p.off_a = align16(p.off_k + entries * D * esize);
    p.off_b = align16(p.off_a + entries * ach * 4);
    p.v_stride = D * esize + 16;
    p.off_v = align16(p.off_b + entries * 4);
    p.off_q = align16(p.off_v + (with_v ? entries * p.v_stride : 0));
    p.off_c = align16(p.off_q + D * 4);
    p.bytes = align16(p.off_c + (L + 1) * 4);
    return p;
}

// Raise a device flag and poison a row's outputs (a rejected row).
__device__ __forceinline__ void reject_row(const Params &P, float *orow, int D, int flag) {
    if (orow)
        for (int i = threadIdx.x; i < D; i += blockDim.x)
            orow[i] = __builtin_nanf("");
    if (threadIdx.x == 0)
        atomicOr(P.flags, flag);
}

// ---------------------------------------------------------------------------
// staging of logged entries into LDS (keys in input dtype, exp'd decays,
// betas; values optional).  Entries j0..j0+n-1 of `pair` go to LDS rows 0..n-1.
// ---------------------------------------------------------------------------
template <int V, int D, typename T, bool WITH_V>
__device__ __forceinline__ void stage_entries(const Params &P, size_t pair, int j0, int n,
                                              unsigned char *smem, const LdsPlan &lp) {
    const int tid = threadIdx.x;
    const size_t e0 = pair * P.L + j0;
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const T *>(P.log_k) + e0 * D);
        uint4 *dst = reinterpret_cast<uint4 *>(smem + lp.off_k);
        const int nch = n * D * (int)sizeof(T) / 16;
        for (int i = tid; i < nch; i += 256)
            dst[i] = src[i];
    }
    {
        constexpr int ACH = (V == GDN) ? 1 : D;
        const float *src = P.log_g + e0 * ACH;
        float *dst = reinterpret_cast<float *>(smem + lp.off_a);
        for (int i = tid; i < n * ACH; i += 256)
            dst[i] = expf(src[i]);
    }
    if constexpr (V != RWKV6) {
        float *dst = reinterpret_cast<float *>(smem + lp.off_b);
        for (int i = tid; i < n; i += 256)
            dst[i] = P.log_beta[e0 + i];
    }
    if constexpr (WITH_V) {
        constexpr int CPR = D * (int)sizeof(T) / 16;
        const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const T *>(P.log_v) + e0 * D);
        for (int i = tid; i < n * CPR; i += 256) {
            const int j = i / CPR, c = i - j * CPR;
            *reinterpret_cast<uint4 *>(smem + lp.off_v + j * lp.v_stride + c * 16) = src[i];
        }
    }
}

template <typename T>
__device__ __forceinline__ float4 lds_load4(const unsigned char *base, int elem) {
    if constexpr (sizeof(T) == 4) {
        return *reinterpret_cast<const float4 *>(base + 4 * elem);
    } else {
        const uint2 u = *reinterpret_cast<const uint2 *>(base + 2 * elem);
        return make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
    }
}

// ---------------------------------------------------------------------------
// host launchers (defined in dl_step.hip / dl_merge.hip).  Every kernel goes
// through hipExtLaunchKernelGGL so that optional start/stop events are
// recorded by the dispatch itself.
// ---------------------------------------------------------------------------
struct Launch {
    hipStream_t stream;
    hipEvent_t start, stop;
};

hipError_t launch_zero(void *p, size_t bytes, const Launch &ln);
hipError_t launch_eager(const Params &P, int rows, const int *slot_idx, const void *q,
                        const void *k, const void *v, const float *g, const float *beta,
                        float *o, const Launch &ln);
hipError_t launch_log_step(const Params &P, int rows, const int *slot_idx, const void *q,
                           const void *k, const void *v, const float *g, const float *beta,
                           float *o, const Launch &ln);
hipError_t launch_readout(const Params &P, int rows, const int *slot_idx, const void *q,
                          float *o, const Launch &ln);
hipError_t launch_merge_replay(const Params &P, int rows, const int *slot_idx, int mode,
                               const Launch &ln);
hipError_t launch_merge_wy(const Params &P, int rows, const int *slot_idx, int mode,
                           const Launch &ln);

}  // namespace dl
