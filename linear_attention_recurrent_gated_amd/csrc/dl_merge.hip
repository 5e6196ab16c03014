// Merge kernels for gfx950: materialise base + log into a new base and empty
// the log (the Merge Phase of the DeltaLog page, "DeltaLog: Deferred
// Materialization of Recurrent States for Linear Attention Decoding",
// Technical Summary, Core Mechanism).
//
// merge_wy_kernel -- the logged transforms folded in WY/UT form, the block
// form the CARVE page (abstract: WY-form triangular chunk solver) and Gated
// DeltaNet-2 (chunkwise WY algorithm) use.  For a chunk of C = 16 entries
// with chunk-local cumulative log-decay Lam_j (per key channel):
//   Kt_j = k_j exp(Lam_j)                         (decayed keys)
//   W    = S Kt^T                                 (d_v x C, MFMA)
//   M_ij = beta_j sum_c k_i k_j exp(Lam_j - Lam_i)   for i < j
//   Kh_j = k_j exp(Lam_C - Lam_j)
//   Y    = diag(beta) (I + M)^{-1} Kh             (C x d_k, back substitution)
//   S'   = S diag(exp(Lam_C)) + (V^T - W) Y       (MFMA)
// (additive variant: S' = S diag(exp(Lam_C)) + V^T Kh).  This is the
// recurrence unrolled over the chunk: with u_j = beta_j (v_j - S_{j-1}
// diag(alpha_j) k_j), S_C = S_0 diag(exp Lam_C) + sum_j u_j Kh_j^T and the
// u_j solve U (I + M) = (V^T - W) diag(beta).  Chunks run one after the
// other; decays never exceed 1 inside a chunk, so nothing overflows.
//
// The base stays in registers for the whole merge, in the MFMA operand
// layout of v_mfma_f32_16x16x4_f32 (lane l: row l % 16 of a 16-row value
// tile, column sub-block l / 16): those registers are the B operand of
// W^T = Kt S^T and, read as 16 x 16 output tiles, the accumulators of the
// update S'^T = diag(exp Lam_C) S^T + Y^T Z^T -- no transposes, no reloads.
//
// merge_replay_kernel -- the same result by replaying the logged steps one
// by one on the vector ALUs (cross-check).
#include "dl_common.hpp"

namespace dl {


// ---------------------------------------------------------------------------
// replay merge (VALU)
// ---------------------------------------------------------------------------
template <int V, int D, typename T, bool NT>
__global__ void __launch_bounds__(256) merge_replay_kernel(Params P, const int *__restrict__ slot_idx,
                                                           int mode) {
    using SH = Shape<D>;
    extern __shared__ __align__(16) unsigned char smem[];
    size_t pair;
    int n;
    if (!resolve_merge_pair(P, slot_idx, mode, pair, n))
        return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = lane >> 3, s = lane & 7;
    const int CH = P.L < 32 ? P.L : 32;
    const LdsPlan lp = lds_plan(V, D, (int)sizeof(T), CH, P.L, true);

    float *Sp = P.base + pair * D * D;
    float4 st[SH::ITER][SH::NCH];
#pragma unroll
    for (int it = 0; it < SH::ITER; ++it) {
        const int row = wave * SH::RPW + it * 8 + grp;
#pragma unroll
        for (int m = 0; m < SH::NCH; ++m)
            st[it][m] = load_state4<NT>(Sp + (size_t)row * D + col_of(s, m, 0));
    }
    const unsigned char *sk = smem + lp.off_k;
    const float *sa = reinterpret_cast<const float *>(smem + lp.off_a);
    const float *sb = reinterpret_cast<const float *>(smem + lp.off_b);

    for (int j0 = 0; j0 < n; j0 += CH) {
        const int cnt = (n - j0) < CH ? (n - j0) : CH;
        __syncthreads();
        stage_entries<V, D, T, true>(P, pair, j0, cnt, smem, lp);
        __syncthreads();
        for (int j = 0; j < cnt; ++j) {
            float kj[SH::FPL], ak[SH::FPL], aj[SH::FPL];
            float a_s = 1.f;
#pragma unroll
            for (int m = 0; m < SH::NCH; ++m) {
                f4_to(kj + 4 * m, lds_load4<T>(sk, j * D + col_of(s, m, 0)));
                if constexpr (V != GDN)
                    f4_to(aj + 4 * m, *reinterpret_cast<const float4 *>(sa + j * D + col_of(s, m, 0)));
            }
            if constexpr (V == GDN)
                a_s = sa[j];
#pragma unroll
            for (int f = 0; f < SH::FPL; ++f)
                ak[f] = (V == GDN) ? kj[f] : aj[f] * kj[f];
            const float bj = (V == RWKV6) ? 1.f : sb[j];
            const unsigned char *vrow = smem + lp.off_v + j * lp.v_stride;
#pragma unroll
            for (int it = 0; it < SH::ITER; ++it) {
                const int row = wave * SH::RPW + it * 8 + grp;
                float u = 0.f;
                if constexpr (V != RWKV6) {
#pragma unroll
                    for (int m = 0; m < SH::NCH; ++m)
                        u += st[it][m].x * ak[4 * m] + st[it][m].y * ak[4 * m + 1] +
                             st[it][m].z * ak[4 * m + 2] + st[it][m].w * ak[4 * m + 3];
                    u = sum8(u);
                    if constexpr (V == GDN)
                        u *= a_s;
                }
                const float vj = Elem<T>::load1(reinterpret_cast<const T *>(vrow) + row);
                const float d = (V == RWKV6) ? vj : bj * (vj - u);
#pragma unroll
                for (int m = 0; m < SH::NCH; ++m) {
                    float sv[4] = {st[it][m].x, st[it][m].y, st[it][m].z, st[it][m].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int f = 4 * m + e;
                        sv[e] = ((V == GDN) ? a_s * sv[e] : sv[e] * aj[f]) + d * kj[f];
                    }
                    st[it][m] = make_float4(sv[0], sv[1], sv[2], sv[3]);
                }
            }
        }
    }
#pragma unroll
    for (int it = 0; it < SH::ITER; ++it) {
        const int row = wave * SH::RPW + it * 8 + grp;
#pragma unroll
        for (int m = 0; m < SH::NCH; ++m)
            store_state4<NT>(Sp + (size_t)row * D + col_of(s, m, 0), st[it][m]);
    }
    if (tid == 0)
        P.fill[pair] = 0;
}

// ---------------------------------------------------------------------------
// WY merge (MFMA).  Four waves per (unit, head); each holds D/4 value rows of
// the base in MFMA layout for the whole merge.  Per chunk, the key side
// (decayed keys, pairwise-decay Gram, Y by back substitution) is built in
// LDS by all threads in three short phases, then each wave runs the two
// contractions on its rows.  The value loads of the chunk are issued before
// the key-side phases so they overlap them.
// ---------------------------------------------------------------------------
template <int V, int D, typename T, bool NT>
__global__ void __launch_bounds__(256, (V == KDA && D == 128) ? 3 : 1)
merge_wy_kernel(Params P, const int *__restrict__ slot_idx, int mode) {
    constexpr int C = 16;               // entries per WY chunk
    constexpr int NIT = D / 64;         // 16-row value tiles per wave
    constexpr int NM = D / 16;          // 16-column blocks
    constexpr int KS = D + 4;           // padded LDS row stride (floats)
    __shared__ __align__(16) float sKt[C * KS];   // k_j exp(Lam_j)
    __shared__ __align__(16) float sY[C * KS];    // rows of diag(beta)(I+M)^{-1} Kh
    __shared__ __align__(16) float sK[C * KS];    // keys, fp32
    __shared__ __align__(16) float sLam[C * KS];  // chunk-local cumulative log-decay
    __shared__ float sM[C * C];                   // beta_j G_ij, i < j
    __shared__ float sB[C];
    __shared__ __align__(16) float sELC[D];       // exp(Lam_C) per key channel

    size_t pair;
    int n;
    if (!resolve_merge_pair(P, slot_idx, mode, pair, n))
        return;
    const int L = P.L;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, kg = lane >> 4;
    float *Sp = P.base + pair * D * D;
    const T *Kl = static_cast<const T *>(P.log_k) + pair * L * D;
    const T *Vl = static_cast<const T *>(P.log_v) + pair * L * D;
    const float *Gl = P.log_g + pair * L * ((V == GDN) ? 1 : D);
    const float *Bl = P.log_beta + pair * L;

    // base rows in MFMA operand layout: st[it][m][e] = S[16 (wave NIT + it) + li][4 kg + 16 m + e]
    floatx4 st[NIT][NM];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int row = 16 * (wave * NIT + it) + li;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const float4 x = load_state4<NT>(Sp + (size_t)row * D + 4 * kg + 16 * m);
            st[it][m] = floatx4{x.x, x.y, x.z, x.w};
        }
    }

    for (int j0 = 0; j0 < n; j0 += C) {
        const int cnt = (n - j0) < C ? (n - j0) : C;
        // this chunk's logged values for the Z tiles (clamped, branch-free loads)
        floatx4 vv[NIT];
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int row = 16 * (wave * NIT + it) + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 4 * kg + r;
                const float x = Elem<T>::load1(Vl + (size_t)(j0 + (j < cnt ? j : cnt - 1)) * D + row);
                vv[it][r] = (j < cnt) ? x : 0.f;
            }
        }
        __syncthreads();   // the previous chunk's LDS operands are consumed

        // ---- phase 1: keys of the chunk (zeros past cnt) and the decay
        //      accumulated since the chunk's start, Lam_j - Lam_{j0-1} (the log
        //      stores Lam since its first entry; entries past cnt repeat the
        //      last one, so their decay adds nothing)
        for (int idx = tid; idx < C * (D / 4); idx += 256) {
            const int j = idx / (D / 4), c = 4 * (idx - j * (D / 4));
            const int e = j0 + (j < cnt ? j : cnt - 1);
            float4 kv = Elem<T>::load4(Kl + (size_t)e * D + c);
            float4 lv, lb = make_float4(0.f, 0.f, 0.f, 0.f);
            if constexpr (V == GDN) {
                lv = make_float4(Gl[e], Gl[e], Gl[e], Gl[e]);
                if (j0 > 0)
                    lb = make_float4(Gl[j0 - 1], Gl[j0 - 1], Gl[j0 - 1], Gl[j0 - 1]);
            } else {
                lv = *reinterpret_cast<const float4 *>(Gl + (size_t)e * D + c);
                if (j0 > 0)
                    lb = *reinterpret_cast<const float4 *>(Gl + (size_t)(j0 - 1) * D + c);
            }
            if (j >= cnt)
                kv = make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 lam = make_float4(lv.x - lb.x, lv.y - lb.y, lv.z - lb.z, lv.w - lb.w);
            *reinterpret_cast<float4 *>(&sK[j * KS + c]) = kv;
            *reinterpret_cast<float4 *>(&sLam[j * KS + c]) = lam;
            *reinterpret_cast<float4 *>(&sKt[j * KS + c]) =
                make_float4(kv.x * expf(lam.x), kv.y * expf(lam.y), kv.z * expf(lam.z), kv.w * expf(lam.w));
            if (j == C - 1)
                *reinterpret_cast<float4 *>(&sELC[c]) =
                    make_float4(expf(lam.x), expf(lam.y), expf(lam.z), expf(lam.w));
        }
        if (tid < C) {
            const int e = j0 + (tid < cnt ? tid : cnt - 1);
            sB[tid] = (V != RWKV6 && tid < cnt) ? Bl[e] : 0.f;
        }
        __syncthreads();

        // ---- phase 2: Gram with pairwise decay, two lanes per pair (i < j), halves of the channels
        if constexpr (V != RWKV6) {
            const int p = tid >> 1, half = tid & 1;
            int i = 0, j = 1;
            const bool inpair = p < C * (C - 1) / 2;
            if (inpair) {
                int base = 0;
                while (base + j <= p) {
                    base += j;
                    ++j;
                }
                i = p - base;
            }
            const bool valid = inpair && j < cnt;
            float gsum = 0.f;
            if (valid) {
                const int c0 = half * (D / 2);
#pragma unroll 2
                for (int c = c0; c < c0 + D / 2; c += 4) {
                    const float4 a = *reinterpret_cast<const float4 *>(&sK[i * KS + c]);
                    const float4 b = *reinterpret_cast<const float4 *>(&sK[j * KS + c]);
                    if constexpr (V == GDN) {
                        gsum += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
                    } else {
                        const float4 l1 = *reinterpret_cast<const float4 *>(&sLam[i * KS + c]);
                        const float4 l2 = *reinterpret_cast<const float4 *>(&sLam[j * KS + c]);
                        gsum += a.x * b.x * expf(l2.x - l1.x) + a.y * b.y * expf(l2.y - l1.y) +
                                a.z * b.z * expf(l2.z - l1.z) + a.w * b.w * expf(l2.w - l1.w);
                    }
                }
            }
            gsum += dpp_mov<0xB1>(gsum);   // add the other half (adjacent lane)
            if (V == GDN && valid)
                gsum *= expf(sLam[j * KS] - sLam[i * KS]);
            if (inpair && half == 0)
                sM[i * C + j] = valid ? sB[j] * gsum : 0.f;
        }
        __syncthreads();

        // ---- phase 3: Y = diag(beta) (I + M)^{-1} Kh, Kh_j = k_j exp(Lam_C - Lam_j)
        if (tid < D) {
            const int c = tid;
            const float lamC = sLam[(C - 1) * KS + c];
            float x[C];
#pragma unroll
            for (int j = C - 1; j >= 0; --j) {
                __builtin_amdgcn_sched_barrier(0);   // keep this row's LDS reads from being hoisted
                float kh = sK[j * KS + c] * expf(lamC - sLam[j * KS + c]);
                if constexpr (V != RWKV6) {
#pragma unroll
                    for (int m = j + 1; m < C; ++m)
                        kh -= sM[j * C + m] * x[m];
                    x[j] = kh;
                    sY[j * KS + c] = sB[j] * kh;
                } else {
                    sY[j * KS + c] = kh;
                }
            }
        }
        __syncthreads();

        // ---- W^T = Kt S^T (MFMA); Z^T = V^T - W^T: z[it][r] = Z[row 16 (wave NIT + it) + li][entry 4 kg + r]
        floatx4 z[NIT];
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            if constexpr (V != RWKV6) {
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    if (m % 2 == 0)
                        __builtin_amdgcn_sched_barrier(0);   // bound the LDS reads in flight
                    const float4 a = *reinterpret_cast<const float4 *>(&sKt[li * KS + 4 * kg + 16 * m]);
                    acc = mfma16x16x4(a.x, st[it][m][0], acc);
                    acc = mfma16x16x4(a.y, st[it][m][1], acc);
                    acc = mfma16x16x4(a.z, st[it][m][2], acc);
                    acc = mfma16x16x4(a.w, st[it][m][3], acc);
                }
            }
            z[it] = vv[it] - acc;
        }
        // ---- S'^T = diag(exp Lam_C) S^T + Y^T Z^T (MFMA, accumulating in place)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if (m % 2 == 0)
                __builtin_amdgcn_sched_barrier(0);   // bound the LDS reads in flight
            const float4 el = *reinterpret_cast<const float4 *>(&sELC[4 * kg + 16 * m]);
            float a[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                a[r] = sY[(4 * kg + r) * KS + 16 * m + li];
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                floatx4 acc = st[it][m];
                acc[0] *= el.x;
                acc[1] *= el.y;
                acc[2] *= el.z;
                acc[3] *= el.w;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc = mfma16x16x4(a[r], z[it][r], acc);
                st[it][m] = acc;
            }
        }
    }

#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int row = 16 * (wave * NIT + it) + li;
#pragma unroll
        for (int m = 0; m < NM; ++m)
            store_state4<NT>(Sp + (size_t)row * D + 4 * kg + 16 * m,
                          make_float4(st[it][m][0], st[it][m][1], st[it][m][2], st[it][m][3]));
    }
    if (tid == 0)
        P.fill[pair] = 0;
}

// ---------------------------------------------------------------------------
#define DL_DISPATCH_M(P, FN, ...)                                                        \
    do {                                                                                 \
        const bool bf = (P).dtype == DL_BF16;                                            \
        if ((P).D == 128) {                                                              \
            if (bf) {                                                                    \
                if ((P).variant == DL_GDN) return FN<GDN, 128, uint16_t>(__VA_ARGS__);   \
                if ((P).variant == DL_KDA) return FN<KDA, 128, uint16_t>(__VA_ARGS__);   \
                return FN<RWKV6, 128, uint16_t>(__VA_ARGS__);                            \
            }                                                                            \
            if ((P).variant == DL_GDN) return FN<GDN, 128, float>(__VA_ARGS__);          \
            if ((P).variant == DL_KDA) return FN<KDA, 128, float>(__VA_ARGS__);          \
            return FN<RWKV6, 128, float>(__VA_ARGS__);                                   \
        }                                                                                \
        if (bf) {                                                                        \
            if ((P).variant == DL_GDN) return FN<GDN, 64, uint16_t>(__VA_ARGS__);        \
            if ((P).variant == DL_KDA) return FN<KDA, 64, uint16_t>(__VA_ARGS__);        \
            return FN<RWKV6, 64, uint16_t>(__VA_ARGS__);                                 \
        }                                                                                \
        if ((P).variant == DL_GDN) return FN<GDN, 64, float>(__VA_ARGS__);               \
        if ((P).variant == DL_KDA) return FN<KDA, 64, float>(__VA_ARGS__);               \
        return FN<RWKV6, 64, float>(__VA_ARGS__);                                        \
    } while (0)

template <int V, int D, typename T>
static hipError_t replay_t(const Params &P, int rows, const int *slot_idx, int mode,
                           const Launch &ln) {
    const int CH = P.L < 32 ? P.L : 32;
    const LdsPlan lp = lds_plan(V, D, (int)sizeof(T), CH, P.L, true);
    if (P.stream)
        hipExtLaunchKernelGGL((merge_replay_kernel<V, D, T, true>), dim3(rows * P.heads), dim3(256), lp.bytes,
                              ln.stream, ln.start, ln.stop, 0, P, slot_idx, mode);
    else
        hipExtLaunchKernelGGL((merge_replay_kernel<V, D, T, false>), dim3(rows * P.heads), dim3(256), lp.bytes,
                              ln.stream, ln.start, ln.stop, 0, P, slot_idx, mode);
    return hipGetLastError();
}

template <int V, int D, typename T>
static hipError_t wy_t(const Params &P, int rows, const int *slot_idx, int mode,
                       const Launch &ln) {
    if (P.stream)
        hipExtLaunchKernelGGL((merge_wy_kernel<V, D, T, true>), dim3(rows * P.heads), dim3(256), 0, ln.stream, ln.start,
                              ln.stop, 0, P, slot_idx, mode);
    else
        hipExtLaunchKernelGGL((merge_wy_kernel<V, D, T, false>), dim3(rows * P.heads), dim3(256), 0, ln.stream, ln.start,
                              ln.stop, 0, P, slot_idx, mode);
    return hipGetLastError();
}

hipError_t launch_merge_replay(const Params &P, int rows, const int *slot_idx, int mode,
                               const Launch &ln) {
    DL_DISPATCH_M(P, replay_t, P, rows, slot_idx, mode, ln);
}

hipError_t launch_merge_wy(const Params &P, int rows, const int *slot_idx, int mode,
                           const Launch &ln) {
    DL_DISPATCH_M(P, wy_t, P, rows, slot_idx, mode, ln);
}

}  // namespace dl
