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

enum Variant { GDN = DL_GDN, KDA = DL_KDA, RWKV6 = DL_RWKV6, GDN2 = DL_GDN2 };

// Device-side view of one state block (all pointers into caller memory).
struct Params {
    int variant, units, heads, D, L, dtype;
    float *base;
    void *log_k;
    void *log_v;
    float *log_g;
    float *log_beta;
    float *log_t;      // packed columns of the compact-WY factor R (delta-rule variants)
    int *fill;
    int *flags;
    int stream;        // 1: state loads and stores carry the nontemporal hint
    int fuse;          // 1: the log step that fills a log merges it
    int af;            // 1: additive-factor log (delta-rule variants): log_v holds
                       //    the fp32 factors a_j, no betas, no R
    // per launch: the rows of this call and, optionally, the order the step
    // workgroups take them in (a device permutation of 0 .. rows - 1)
    int rows;
    const int *row_order;
    // DL_BASE_I8 (q8 = 1): INT8 codes, row scales, the M kept key channels'
    // fp32 values and their column indices (per head); base is NULL
    int q8, M;
    int8_t *codes;
    float *scale;
    float *kept;
    int *kidx;
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
// v_mfma_f32_16x16x4_f32: D(16x16) += A(16x4) B(4x16); lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16] and holds D[4 (l / 16) + r][l % 16].
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma16x16x4(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// State tiles.  When a call's states are larger than the last-level cache
// can usefully hold (NT), every state is read (and written) once per kernel
// with the nontemporal hint: the lines do not displace reusable data and the
// streaming read rate rises measurably on gfx950.  Smaller state sets keep
// ordinary cacheable accesses, so repeated calls can hit the cache.
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ float4 load_state4(const float *p) {
    if constexpr (NT) {
        const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
        return make_float4(t.x, t.y, t.z, t.w);
    } else {
        return *reinterpret_cast<const float4 *>(p);
    }
}
template <bool NT>
__device__ __forceinline__ void store_state4(float *p, float4 v) {
    if constexpr (NT) {
        const f32x4 t = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(t, reinterpret_cast<f32x4 *>(p));
    } else {
        *reinterpret_cast<float4 *>(p) = v;
    }
}

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

// Eight bf16 values (one 16-byte word) as floats.
__device__ __forceinline__ void unpack_bf16x8(const uint4 &u, float *x) {
    x[0] = bf16_lo(u.x), x[1] = bf16_hi(u.x), x[2] = bf16_lo(u.y), x[3] = bf16_hi(u.y);
    x[4] = bf16_lo(u.z), x[5] = bf16_hi(u.z), x[6] = bf16_lo(u.w), x[7] = bf16_hi(u.w);
}

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

// Orders this wave's LDS stores before its later LDS loads of other lanes'
// data.  A wave's LDS instructions execute in issue order, so the fences
// (wavefront scope, no instructions) only stop the compiler from moving
// memory accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Key side of the DeltaLog step (dl_step.hip).
//
// Chunk layout: lane l covers the eight key channels 8 (l % G) .. + 7 of the
// rows RP u + l / G (u < NU) of a pass over 16 logged entries.
// ---------------------------------------------------------------------------
template <int D>
struct KeyLayout {
    static constexpr int G = D / 8;      // lanes across one row
    static constexpr int RP = 64 / G;    // rows per lane step
    static constexpr int NU = 16 / RP;   // lane steps per 16-row pass
};

// LDS carve-up of the step kernel.  The staging regions are whole multiples
// of one wave's direct-to-LDS load (64 lanes x 16 or 4 bytes).
struct StepPlan {
    int off_k;     // staged keys, rows of D elements in the input dtype
    int off_v;     // staged values, rows of D elements in the input dtype
    int off_lam;   // staged cumulative log-decays, rows of D floats (per-key decays)
    int off_t;     // staged columns of R, packed
    int off_r, off_u, off_f, off_l;   // per-entry scalars, 64 floats each
    int off_bn;    // beta of the appended entry
    int off_c, off_e;                 // per-wave coefficients, 4 x 64 floats each
    int off_qin;   // q as floats, D
    int off_q;     // q0, D floats
    int off_y;     // merge in the step: 16 rows of Y = R Q, D floats each
                   // (in the staged values' place when they are large enough)
    int bytes;
};

// LDS carve-up of the additive-factor step, readout and merge kernels.  Only
// the factors a_j are staged for every step: each logged key and decay is
// used by one lane of the step, which loads it straight from the log.
struct AfPlan {
    int off_a;     // staged factors a_j, rows of D floats
    int off_kd;    // merges only: decayed keys k_j D(j, c), rows of D floats
    int off_r, off_u, off_f;          // per-entry r_j, u_j, (GDN) D(j, c); 64 floats each
    int off_s;     // GDN: Lam of the newest entry
    int off_lc;    // per-key decays: Lam of the newest entry, D floats
    int off_qe, off_ke;               // E q and E k, D floats each
    int off_v;     // the step's value row, D elements (up to 4 bytes each)
    int off_w;     // gated form: the write gate row, D floats
    int off_ek;    // gated form: the erase-gated key e * k, D floats
    int bytes;
};

__host__ __device__ inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

__host__ __device__ inline AfPlan af_plan(int D, int L, bool merges) {
    AfPlan p;
    p.off_a = 0;
    p.off_kd = round_up(L * D * 4, 1024);
    p.off_r = p.off_kd + (merges ? round_up(L * D * 4, 1024) : 0);
    p.off_u = p.off_r + 256;
    p.off_f = p.off_u + 256;
    p.off_s = p.off_f + 256;
    p.off_lc = p.off_s + 16;
    p.off_qe = p.off_lc + D * 4;
    p.off_ke = p.off_qe + D * 4;
    p.off_v = p.off_ke + D * 4;
    p.off_w = p.off_v + D * 4;
    p.off_ek = p.off_w + D * 4;
    p.bytes = p.off_ek + D * 4;
    return p;
}

__host__ __device__ inline int packed_t_len(int variant, int L) {
    return variant == DL_RWKV6 ? 0 : L * (L - 1) / 2;
}


__host__ __device__ inline StepPlan step_plan(int variant, int D, int esize, int L, bool fuse) {
    StepPlan p;
    p.off_k = 0;
    p.off_v = round_up(L * D * esize, 1024);
    p.off_lam = p.off_v + round_up(L * D * esize, 1024);
    p.off_t = p.off_lam + (variant == DL_GDN ? 0 : round_up(L * D * 4, 1024));
    p.off_r = p.off_t + round_up(packed_t_len(variant, L) * 4, 256);
    p.off_u = p.off_r + 256;
    p.off_f = p.off_u + 256;
    p.off_l = p.off_f + 256;
    p.off_bn = p.off_l + 256;
    p.off_c = p.off_bn + 16;
    p.off_e = p.off_c + 4 * 256;
    p.off_qin = p.off_e + 4 * 256;
    p.off_q = p.off_qin + D * 4;
    // Y is built after the merge has read every logged value, so it can take
    // the staged values' place when they span at least 16 rows of D floats
    const bool y_in_v = round_up(L * D * esize, 1024) >= 16 * D * 4;
    p.off_y = y_in_v ? p.off_v : p.off_q + D * 4;
    p.bytes = p.off_q + D * 4 + ((fuse && !y_in_v) ? 16 * D * 4 : 0);
    return p;
}

// LDS carve-up of the chunked compact-WY step (per-key decays at d = 128,
// logs of 33 to 64 entries, no merge in the step): keys and decays of 32
// entries at a time, the values later in their place, the appended entry on
// its own, R whole.
struct ChunkPlan {
    int off_kc;    // keys of one chunk: 32 rows of D elements (input dtype)
    int off_lc;    // cumulative log-decays of that chunk: 32 rows of D floats
    int off_v;     // after q0: the logged values, rows of D elements (over kc, lc)
    int off_kn, off_ln, off_vn;       // the appended entry's key, decays, value
    int off_t;     // packed columns of R
    int off_r, off_u, off_f;          // per-entry scalars, 64 floats each
    int off_bn;    // beta of the appended entry
    int off_c;     // per-wave coefficients, 4 x 64 floats
    int off_qin, off_q;               // q as floats and q0, D floats each
    int bytes;
};

__host__ __device__ inline ChunkPlan chunk_plan(int D, int esize, int L) {
    ChunkPlan p;
    p.off_kc = 0;
    p.off_lc = round_up(32 * D * esize, 256);
    p.off_v = 0;
    const int chunk_end = p.off_lc + round_up(32 * D * 4, 256);
    const int values_end = round_up(L * D * esize, 256);
    p.off_kn = chunk_end > values_end ? chunk_end : values_end;
    p.off_ln = p.off_kn + round_up(D * esize, 16);
    p.off_vn = p.off_ln + D * 4;
    p.off_t = round_up(p.off_vn + D * esize, 256);
    p.off_r = p.off_t + round_up(packed_t_len(DL_KDA, L) * 4, 256);
    p.off_u = p.off_r + 256;
    p.off_f = p.off_u + 256;
    p.off_bn = p.off_f + 256;
    p.off_c = p.off_bn + 16;
    p.off_qin = p.off_c + 4 * 256;
    p.off_q = p.off_qin + D * 4;
    p.bytes = p.off_q + D * 4;
    return p;
}

// e^x through the hardware base-2 exponential: about 1 ulp plus the rounding
// of x log2(e) (relative error near |x| 2^-24); results below the normal
// range flush to zero.
__device__ __forceinline__ float fast_exp(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// Eight consecutive elements as floats (global memory or LDS).
template <typename T>
__device__ __forceinline__ void load8(const T *p, float *x) {
    if constexpr (sizeof(T) == 4) {
        const float4 a = reinterpret_cast<const float4 *>(p)[0];
        const float4 b = reinterpret_cast<const float4 *>(p)[1];
        x[0] = a.x, x[1] = a.y, x[2] = a.z, x[3] = a.w;
        x[4] = b.x, x[5] = b.y, x[6] = b.z, x[7] = b.w;
    } else {
        const uint4 u = *reinterpret_cast<const uint4 *>(p);
        x[0] = bf16_lo(u.x), x[1] = bf16_hi(u.x), x[2] = bf16_lo(u.y), x[3] = bf16_hi(u.y);
        x[4] = bf16_lo(u.z), x[5] = bf16_hi(u.z), x[6] = bf16_lo(u.w), x[7] = bf16_hi(u.w);
    }
}

// Stores eight floats that were widened from T (so the bf16 narrowing is exact).
template <typename T>
__device__ __forceinline__ void store8(T *p, const float *x) {
    if constexpr (sizeof(T) == 4) {
        reinterpret_cast<float4 *>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
        reinterpret_cast<float4 *>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
    } else {
        uint4 u;
        u.x = (__float_as_uint(x[0]) >> 16) | (__float_as_uint(x[1]) & 0xffff0000u);
        u.y = (__float_as_uint(x[2]) >> 16) | (__float_as_uint(x[3]) & 0xffff0000u);
        u.z = (__float_as_uint(x[4]) >> 16) | (__float_as_uint(x[5]) & 0xffff0000u);
        u.w = (__float_as_uint(x[6]) >> 16) | (__float_as_uint(x[7]) & 0xffff0000u);
        *reinterpret_cast<uint4 *>(p) = u;
    }
}

// Sum over aligned groups of G lanes, G = 8 or 16 (every lane gets its group's sum).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    x = sum8(x);
    if constexpr (G == 16)
        x += dpp_mov<0x140>(x);   // row_mirror
    return x;
}

// x(l) + x(l ^ 16) and x(l) + x(l ^ 32): the gfx950 permlane swaps hand each
// lane its partner's value alongside its own.
__device__ __forceinline__ float xor16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the lanes that share l % M (M = 2 or 4): rotations inside each
// 16-lane row, then the permlane swaps across rows.
template <int M>
__device__ __forceinline__ float sum_mod(float x) {
    static_assert(M == 2 || M == 4, "M = 2 or 4");
    if constexpr (M == 2)
        x += dpp_mov<0x122>(x);   // row_ror:2
    x += dpp_mov<0x124>(x);       // row_ror:4
    x += dpp_mov<0x128>(x);       // row_ror:8
    return xor32_sum(xor16_sum(x));
}

// One wave's direct global -> LDS load of 16 (or 4) bytes per lane: lane l's
// bytes land at lds + l * SIZE; lanes outside EXEC load and write nothing.
// `lds` must be wave-uniform.
template <int SIZE>
__device__ __forceinline__ void load_to_lds(const void *src, unsigned char *lds) {
    static_assert(SIZE == 16 || SIZE == 4, "16- or 4-byte loads");
    auto *dst = (__attribute__((address_space(3))) void *)lds;
    if constexpr (SIZE == 16)
        __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
    else
        __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
}

// s_waitcnt vmcnt(0), leaving the other counters free (gfx9 encoding:
// vmcnt bits 3:0 and 15:14 zero, expcnt 6:4 and lgkmcnt 11:8 at their maxima).
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier for data staged with direct-to-LDS loads while at most N
// later loads of each wave (e.g. of a tile that is used after the barrier)
// stay in flight: each wave waits until at most N of its loads are
// outstanding -- loads complete in issue order, so its staging has landed --
// and its LDS stores have completed, then all waves meet.  Unlike
// __syncthreads() this does not wait for the N later loads (a workgroup
// fence would, since the staging loads write LDS).  The asm's memory clobber
// keeps the compiler from moving memory accesses across it.
template <int N>
__device__ __forceinline__ void barrier_after_staging() {
    static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 3) << 14) | 0x0070);
    asm volatile("s_barrier" ::: "memory");
}

// s_waitcnt vmcnt(N): wait until at most N of this wave's vector memory
// loads are outstanding (they complete in issue order), other counters free.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 3) << 14) | 0x0F70);
}

// The input row and head a step workgroup serves.  Workgroups are
// dispatched in block order, so a caller-supplied row_order decides which
// rows start first (e.g. rows whose log merges in this step, which run
// longer, ahead of the rest); without one, block b serves row b / heads.
// Returns -1 for an order entry outside [0, rows).
__device__ __forceinline__ int step_row(const Params &P, int &h) {
    const int b = blockIdx.x;
    const int rb = b / P.heads;
    h = b - rb * P.heads;
    if (!P.row_order)
        return rb;
    const int r = P.row_order[rb];
    return (r >= 0 && r < P.rows) ? r : -1;
}

// Raise a device flag and poison a row's outputs (a rejected row).
__device__ __forceinline__ void reject_row(const Params &P, float *orow, int D, int flag) {
    if (orow)
        for (int i = threadIdx.x; i < D; i += blockDim.x)
            orow[i] = __builtin_nanf("");
    if (threadIdx.x == 0)
        atomicOr(P.flags, flag);
}

// The (unit, head) pair a merge workgroup owns and its log fill; false when
// there is nothing to merge (empty log, or not full under DL_MERGE_FULL) or
// the slot index is out of range (flagged).
__device__ __forceinline__ bool resolve_merge_pair(const Params &P, const int *slot_idx, int mode,
                                                   size_t &pair, int &n) {
    const int H = P.heads;
    const int pr = blockIdx.x;
    const int r = pr / H, h = pr - r * H;
    const int unit = slot_idx ? slot_idx[r] : r;
    if (unit < 0 || unit >= P.units) {
        reject_row(P, nullptr, P.D, DL_FLAG_BAD_SLOT);
        return false;
    }
    pair = (size_t)unit * H + h;
    n = P.fill[pair];
    if (n <= 0 || n > P.L)
        return false;
    if (mode == DL_MERGE_FULL && n != P.L)
        return false;
    return true;
}

// ---------------------------------------------------------------------------
// staging of logged entries into LDS (keys in input dtype, per-entry decays
// alpha_j, betas; values optional).  Entries j0..j0+n-1 of `pair` go to LDS rows 0..n-1.
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
        // the log keeps the decay accumulated since its first entry:
        // alpha_j = exp(Lam_j - Lam_{j-1}), Lam_{-1} = 0
        constexpr int ACH = (V == GDN) ? 1 : D;
        const float *src = P.log_g + e0 * ACH;
        float *dst = reinterpret_cast<float *>(smem + lp.off_a);
        for (int i = tid; i < n * ACH; i += 256) {
            const float prev = (j0 * ACH + i >= ACH) ? src[i - ACH] : 0.f;
            dst[i] = expf(src[i] - prev);
        }
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
// INT8 base (DL_BASE_I8).  A value row is held by the 8 lanes of a row group,
// lane s taking the QW = D / 8 consecutive columns QW s .. QW s + QW - 1, so
// that a row's codes are one 16-byte (D = 128) or 8-byte (D = 64) load per
// lane.  Kept key channels are coded 0 and carry their fp32 value apart.
// ---------------------------------------------------------------------------
template <int D>
struct Q8Row {
    static constexpr int QW = D / 8;           // columns per lane
    static constexpr int NW = QW / 4;          // 32-bit words of codes per lane
};

// This lane's codes of one row as floats.
template <int QW>
__device__ __forceinline__ void q8_unpack(const uint32_t *w, float *x) {
#pragma unroll
    for (int f = 0; f < QW; ++f)
        x[f] = (float)(int)(int8_t)((w[f >> 2] >> (8 * (f & 3))) & 0xff);
}

// Maximum over the 8 lanes of a row group; all 8 end with the same value.
__device__ __forceinline__ float max8(float x) {
    x = fmaxf(x, dpp_mov<0xB1>(x));
    x = fmaxf(x, dpp_mov<0x4E>(x));
    x = fmaxf(x, dpp_mov<0x141>(x));
    return x;
}

// Quantise one row held as x[QW] on each lane of its row group: the scale is
// the maximum |x| over the coded columns (this lane's kept columns are the
// set bits of kbits) divided by 127, each code rint(x / scale) clipped to
// +-127, kept columns and zero rows coded 0.  Every operation is an IEEE
// fp32 operation (correctly rounded divisions, ties-to-even rounding), so an
// fp32 reference taking the same steps decides the same codes.  Returns the
// scale; writes the lane's codes to w[QW / 4].
template <int QW>
__device__ __forceinline__ float q8_quantize_row(const float *x, uint32_t kbits, uint32_t *w) {
    float amax = 0.f;
#pragma unroll
    for (int f = 0; f < QW; ++f)
        amax = ((kbits >> f) & 1u) ? amax : fmaxf(amax, fabsf(x[f]));
    amax = max8(amax);
    const float scale = amax / 127.0f;
#pragma unroll
    for (int i = 0; i < QW / 4; ++i)
        w[i] = 0u;
    if (scale > 0.f) {
#pragma unroll
        for (int f = 0; f < QW; ++f) {
            float c = __builtin_rintf(x[f] / scale);
            c = fminf(fmaxf(c, -127.f), 127.f);
            const int ci = ((kbits >> f) & 1u) ? 0 : (int)c;
            w[f >> 2] |= (uint32_t)(ci & 0xff) << (8 * (f & 3));
        }
    }
    return scale;
}

// The kept channels of head h that fall on lane s's columns, as a bit mask,
// and whether the index list is valid (strictly increasing in [0, D)).
template <int D>
__device__ __forceinline__ uint32_t q8_kept_bits(const Params &P, int h, int s, bool &ok) {
    constexpr int QW = Q8Row<D>::QW;
    uint32_t bits = 0u;
    ok = true;
    int prev = -1;
    for (int m = 0; m < P.M; ++m) {
        const int c = P.kidx[h * P.M + m];
        ok = ok && c > prev && c < D;
        prev = c;
        if (c >= 0 && c < D && c / QW == s)
            bits |= 1u << (c % QW);
    }
    return bits;
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
// additive-factor log (dl_step_af.hip)
hipError_t launch_af_step(const Params &P, int rows, const int *slot_idx, const void *q,
                          const void *k, const void *v, const float *g, const float *beta,
                          float *o, const Launch &ln);
hipError_t launch_af_readout(const Params &P, int rows, const int *slot_idx, const void *q,
                             float *o, const Launch &ln);
hipError_t launch_af_merge(const Params &P, int rows, const int *slot_idx, int mode,
                           const Launch &ln);
// base import / export (dl_base.hip)
hipError_t launch_base_import(const Params &P, int rows, const int *slot_idx, const float *src,
                              const Launch &ln);
hipError_t launch_base_export(const Params &P, int rows, const int *slot_idx, float *dst,
                              const Launch &ln);
hipError_t launch_kept_default(const Params &P, const Launch &ln);
// streaming-rate calibration (dl_probe.hip): mode 0 reads, mode 1 copies
size_t probe_read_outputs(size_t bytes);
hipError_t launch_stream_probe(int mode, const void *src, void *dst, size_t bytes, const Launch &ln);

}  // namespace dl
