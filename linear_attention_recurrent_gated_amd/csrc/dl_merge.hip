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
// WY merge (MFMA).
//
// A pair's D value rows are split over NS = D / ROWS workgroups of NW waves
// (ROWS = 16 NW NIT rows each, NIT 16-row tiles per wave), so that a launch
// over few pairs -- the handful of logs that fill at one step of a ragged
// batch -- still spreads over every CU.  Each workgroup builds the chunk's key
// side (decayed keys, pairwise-decay Gram, Y by back substitution) for itself:
// it depends on the keys only, which the NS workgroups of a pair read from the
// L2 of one XCD (they are dispatched 8 blocks apart, and blocks go round-robin
// over the 8 XCDs).  A chunk's keys, decays and values are loaded before the
// base, and its key side is built while the base is still in flight; the next
// chunk's are loaded before the current chunk's two contractions.
//
// The fill count is read and reset through tickets in its upper half: every
// workgroup of a pair adds 1 << 16 and reads the count in the lower half; the
// one that takes the last ticket writes the count back (0 when the pair
// merges), so no workgroup of the pair can read a count another one reset.
// ---------------------------------------------------------------------------
template <int V, int D, typename T, int NW, int NIT>
struct WyShape {
    static constexpr int C = 16;                  // entries per WY chunk
    static constexpr int NTH = 64 * NW;           // threads per workgroup
    static constexpr int ROWS = 16 * NW * NIT;    // value rows per workgroup
    static constexpr int NS = D / ROWS;           // workgroups per pair
    static constexpr int NM = D / 16;             // 16-column blocks
    static constexpr int KS = D + 4;              // padded LDS row stride (floats)
    static constexpr bool PK = V != GDN;          // per-key decays
    static constexpr int CPE = D / 8;             // 8-channel items per entry
    static constexpr int NI = (C * CPE + NTH - 1) / NTH;   // key items per thread
    static constexpr int KW = sizeof(T) == 2 ? 1 : 2;       // 16-byte words per item's keys
    static_assert(NS >= 1 && NS * ROWS == D, "the rows of a pair split evenly");
    static_assert(NTH >= D, "one thread per key channel in the back substitution");
};

// One chunk's key side and values as loaded (registers), before they go to LDS.
template <int V, int D, typename T, int NW, int NIT>
struct WyChunk {
    using WS = WyShape<V, D, T, NW, NIT>;
    uint4 k[WS::NI][WS::KW];       // keys of this thread's items
    float4 l[WS::NI][2];           // per-key decays: Lam of the item's entry
    float lg[WS::NI];              // head-wise decay: Lam of the item's entry
    float4 lb[WS::NI][2];          // per-key decays: Lam before the chunk
    float lbg;                     // head-wise decay: Lam before the chunk
    float b;                       // beta of entry tid (tid < C)
    float vv[NIT][4];              // values of the Z tiles
};

template <int V, int D, typename T, int NW, int NIT>
__device__ __forceinline__ void wy_load_chunk(const Params &P, size_t pair, int split, int j0, int n,
                                              WyChunk<V, D, T, NW, NIT> &c) {
    using WS = WyShape<V, D, T, NW, NIT>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, kg = lane >> 4;
    const int L = P.L;
    const int cnt = (n - j0) < WS::C ? (n - j0) : WS::C;
    const T *Kl = static_cast<const T *>(P.log_k) + pair * L * D;
    const T *Vl = static_cast<const T *>(P.log_v) + pair * L * D;
    const float *Gl = P.log_g + pair * L * (WS::PK ? D : 1);
#pragma unroll
    for (int i = 0; i < WS::NI; ++i) {
        const int idx0 = tid + WS::NTH * i;
        const int idx = idx0 < WS::C * WS::CPE ? idx0 : 0;
        const int j = idx / WS::CPE, ch = 8 * (idx - j * WS::CPE);
        // entries past the chunk's last repeat it (their keys are zeroed later)
        const int e = j0 + (j < cnt ? j : cnt - 1);
        const uint4 *kp = reinterpret_cast<const uint4 *>(Kl + (size_t)e * D + ch);
#pragma unroll
        for (int w = 0; w < WS::KW; ++w)
            c.k[i][w] = kp[w];
        if constexpr (WS::PK) {
            const float4 *lp = reinterpret_cast<const float4 *>(Gl + (size_t)e * D + ch);
            c.l[i][0] = lp[0];
            c.l[i][1] = lp[1];
            if (j0 > 0) {
                const float4 *bp = reinterpret_cast<const float4 *>(Gl + (size_t)(j0 - 1) * D + ch);
                c.lb[i][0] = bp[0];
                c.lb[i][1] = bp[1];
            } else {
                c.lb[i][0] = c.lb[i][1] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        } else {
            c.lg[i] = Gl[e];
        }
    }
    if constexpr (!WS::PK)
        c.lbg = j0 > 0 ? Gl[j0 - 1] : 0.f;
    c.b = 0.f;
    if (V != RWKV6 && tid < WS::C && tid < cnt)
        c.b = P.log_beta[pair * L + j0 + tid];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int row = split * WS::ROWS + 16 * (wave * NIT + it) + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = 4 * kg + r;
            const float x = Elem<T>::load1(Vl + (size_t)(j0 + (j < cnt ? j : cnt - 1)) * D + row);
            c.vv[it][r] = (j < cnt) ? x : 0.f;
        }
    }
}

// Waves per SIMD each shape is held to (registers): the base tiles take 32 NIT
// VGPRs at d = 128, the per-key decays of a chunk about 16 more.
template <int V, int D, int NW, int NIT>
constexpr int wy_waves_per_simd() {
    if constexpr (D == 64)
        return NW == 4 ? 5 : 6;
    else if constexpr (NIT == 2)
        return V == GDN ? 4 : 3;
    else if constexpr (NW == 4)
        return V == GDN ? 5 : 4;
    else
        return V == GDN ? 6 : 5;
}

template <int V, int D, typename T, bool NTS, int NW, int NIT>
__global__ void __launch_bounds__(64 * NW, (wy_waves_per_simd<V, D, NW, NIT>()))
merge_wy_kernel(Params P, const int *__restrict__ slot_idx, int mode, int npairs) {
    using WS = WyShape<V, D, T, NW, NIT>;
    constexpr int C = WS::C, NM = WS::NM, KS = WS::KS, NTH = WS::NTH;
    __shared__ __align__(16) float sKt[C * KS];                // k_j exp(Lam_j)
    __shared__ __align__(16) float sKY[C * KS];                // keys (fp32), then Y in place
    __shared__ __align__(16) float sLam[WS::PK ? C * KS : C];  // chunk-local cumulative log-decay
    __shared__ float sM[C * C];                                // beta_j G_ij, i < j
    __shared__ float sB[C];
    __shared__ __align__(16) float sELC[D];                    // exp(Lam_C) per key channel
    __shared__ int sN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, kg = lane >> 4;
    // block -> (pair, split): the NS workgroups of a pair are 8 blocks apart
    const int xcd = blockIdx.x & 7, qb = blockIdx.x >> 3;
    const int split = qb % WS::NS;
    const int pr = (qb / WS::NS) * 8 + xcd;
    if (pr >= npairs)
        return;
    const int H = P.heads, L = P.L;
    const int r = pr / H, h = pr - r * H;
    const int unit = slot_idx ? slot_idx[r] : r;
    if (unit < 0 || unit >= P.units) {
        if (split == 0)
            reject_row(P, nullptr, D, DL_FLAG_BAD_SLOT);
        return;
    }
    const size_t pair = (size_t)unit * H + h;
    if (tid == 0) {
        const int old = atomicAdd(P.fill + pair, 1 << 16);
        const int n0 = old & 0xffff;
        const bool go = n0 > 0 && n0 <= L && (mode != DL_MERGE_FULL || n0 == L);
        if ((old >> 16) == WS::NS - 1)
            P.fill[pair] = go ? 0 : n0;
        sN = go ? n0 : 0;
    }
    __syncthreads();
    const int n = sN;
    if (n == 0)
        return;

    // chunk 0's key side and values first, then this workgroup's rows of the
    // base in MFMA operand layout: st[it][m][e] = S[row0 + 16 (wave NIT + it) + li][4 kg + 16 m + e]
    WyChunk<V, D, T, NW, NIT> cur;
    wy_load_chunk<V, D, T, NW, NIT>(P, pair, split, 0, n, cur);
    float *Sp = P.base + pair * D * D;
    const int row0 = split * WS::ROWS;
    floatx4 st[NIT][NM];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int row = row0 + 16 * (wave * NIT + it) + li;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const float4 x = load_state4<NTS>(Sp + (size_t)row * D + 4 * kg + 16 * m);
            st[it][m] = floatx4{x.x, x.y, x.z, x.w};
        }
    }

    for (int j0 = 0; j0 < n; j0 += C) {
        const int cnt = (n - j0) < C ? (n - j0) : C;
        if (j0 > 0)
            __syncthreads();   // the previous chunk's LDS operands are consumed

        // ---- phase 1: keys of the chunk (zeros past cnt), the decay accumulated
        //      since the chunk's start, Lam_j - Lam_{j0-1}, and the decayed keys
#pragma unroll
        for (int i = 0; i < WS::NI; ++i) {
            const int idx = tid + NTH * i;
            if (idx < C * WS::CPE) {
                const int j = idx / WS::CPE, ch = 8 * (idx - j * WS::CPE);
                float kv[8], lam[8];
                if constexpr (sizeof(T) == 2) {
                    unpack_bf16x8(cur.k[i][0], kv);
                } else {
                    const uint4 a = cur.k[i][0], b = cur.k[i][WS::KW - 1];
                    kv[0] = __uint_as_float(a.x), kv[1] = __uint_as_float(a.y);
                    kv[2] = __uint_as_float(a.z), kv[3] = __uint_as_float(a.w);
                    kv[4] = __uint_as_float(b.x), kv[5] = __uint_as_float(b.y);
                    kv[6] = __uint_as_float(b.z), kv[7] = __uint_as_float(b.w);
                }
                if constexpr (WS::PK) {
                    const float4 l0 = cur.l[i][0], l1 = cur.l[i][1], b0 = cur.lb[i][0], b1 = cur.lb[i][1];
                    lam[0] = l0.x - b0.x, lam[1] = l0.y - b0.y, lam[2] = l0.z - b0.z, lam[3] = l0.w - b0.w;
                    lam[4] = l1.x - b1.x, lam[5] = l1.y - b1.y, lam[6] = l1.z - b1.z, lam[7] = l1.w - b1.w;
                } else {
                    const float lj = cur.lg[i] - cur.lbg;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        lam[e] = lj;
                    if (ch == 0)
                        sLam[j] = lj;
                }
                if (j >= cnt)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        kv[e] = 0.f;
                float kt[8], el[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    el[e] = expf(lam[e]);
                    kt[e] = kv[e] * el[e];
                }
                store8<float>(sKY + j * KS + ch, kv);
                store8<float>(sKt + j * KS + ch, kt);
                if constexpr (WS::PK)
                    store8<float>(sLam + j * KS + ch, lam);
                if (j == C - 1)
                    store8<float>(sELC + ch, el);
            }
        }
        if (tid < C)
            sB[tid] = cur.b;
        __syncthreads();

        // ---- phase 2: Gram with pairwise decay, two lanes per pair (i < j),
        //      halves of the channels
        if constexpr (V != RWKV6) {
            constexpr int NPAIR = C * (C - 1) / 2;
#pragma unroll
            for (int pass = 0; pass < (2 * NPAIR + NTH - 1) / NTH; ++pass) {
                const int w = tid + NTH * pass;
                const int p = w >> 1, half = w & 1;
                int i = 0, j = 1;
                const bool inpair = p < NPAIR;
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
                        const float4 a = *reinterpret_cast<const float4 *>(&sKY[i * KS + c]);
                        const float4 b = *reinterpret_cast<const float4 *>(&sKY[j * KS + c]);
                        if constexpr (!WS::PK) {
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
                if (!WS::PK && valid)
                    gsum *= expf(sLam[j] - sLam[i]);
                if (inpair && half == 0)
                    sM[i * C + j] = valid ? sB[j] * gsum : 0.f;
            }
        }
        __syncthreads();

        // ---- phase 3: Y = diag(beta) (I + M)^{-1} Kh, Kh_j = k_j exp(Lam_C - Lam_j),
        //      one key channel per thread, in place of the keys
        if (tid < D) {
            const int c = tid;
            const float lamC = WS::PK ? sLam[(C - 1) * KS + c] : sLam[C - 1];
            float x[C];
#pragma unroll
            for (int j = C - 1; j >= 0; --j) {
                __builtin_amdgcn_sched_barrier(0);   // keep this row's LDS reads from being hoisted
                const float lj = WS::PK ? sLam[j * KS + c] : sLam[j];
                float kh = sKY[j * KS + c] * expf(lamC - lj);
                if constexpr (V != RWKV6) {
#pragma unroll
                    for (int m = j + 1; m < C; ++m)
                        kh -= sM[j * C + m] * x[m];
                    x[j] = kh;
                    sKY[j * KS + c] = sB[j] * kh;
                } else {
                    sKY[j * KS + c] = kh;
                }
            }
        }
        __syncthreads();

        // the next chunk's key side and values, in flight during the contractions
        WyChunk<V, D, T, NW, NIT> nxt;
        if (j0 + C < n)
            wy_load_chunk<V, D, T, NW, NIT>(P, pair, split, j0 + C, n, nxt);

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
            const floatx4 vz = {cur.vv[it][0], cur.vv[it][1], cur.vv[it][2], cur.vv[it][3]};
            z[it] = vz - acc;
        }
        // ---- S'^T = diag(exp Lam_C) S^T + Y^T Z^T (MFMA, accumulating in place)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if (m % 2 == 0)
                __builtin_amdgcn_sched_barrier(0);   // bound the LDS reads in flight
            const float4 el = *reinterpret_cast<const float4 *>(&sELC[4 * kg + 16 * m]);
            float a[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                a[rr] = sKY[(4 * kg + rr) * KS + 16 * m + li];
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                floatx4 acc = st[it][m];
                acc[0] *= el.x;
                acc[1] *= el.y;
                acc[2] *= el.z;
                acc[3] *= el.w;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    acc = mfma16x16x4(a[rr], z[it][rr], acc);
                st[it][m] = acc;
            }
        }
        cur = nxt;
    }

#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int row = row0 + 16 * (wave * NIT + it) + li;
#pragma unroll
        for (int m = 0; m < NM; ++m)
            store_state4<NTS>(Sp + (size_t)row * D + 4 * kg + 16 * m,
                              make_float4(st[it][m][0], st[it][m][1], st[it][m][2], st[it][m][3]));
    }
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

// Workgroups per pair for a merge over `pairs` pairs: enough that the launch
// has about eight workgroups per CU of the 256 CUs, the rows of a pair split
// two or four ways when there are few pairs.
template <int V, int D, typename T, bool NTS, int NW, int NIT>
static void wy_launch(const Params &P, int pairs, const int *slot_idx, int mode, const Launch &ln) {
    using WS = WyShape<V, D, T, NW, NIT>;
    const int groups = (pairs + 7) / 8;
    hipExtLaunchKernelGGL((merge_wy_kernel<V, D, T, NTS, NW, NIT>), dim3(groups * 8 * WS::NS),
                          dim3(WS::NTH), 0, ln.stream, ln.start, ln.stop, 0, P, slot_idx, mode, pairs);
}

template <int V, int D, typename T, bool NTS>
static void wy_split(const Params &P, int pairs, const int *slot_idx, int mode, const Launch &ln) {
    constexpr int WAVES = 8 * 256 * 4;          // about eight 4-wave workgroups per CU
    if constexpr (D == 128) {
        if (pairs * 4 >= WAVES)
            wy_launch<V, D, T, NTS, 4, 2>(P, pairs, slot_idx, mode, ln);    // one workgroup per pair
        else if (pairs * 8 >= WAVES)
            wy_launch<V, D, T, NTS, 4, 1>(P, pairs, slot_idx, mode, ln);    // two, 64 rows each
        else
            wy_launch<V, D, T, NTS, 2, 1>(P, pairs, slot_idx, mode, ln);    // four, 32 rows each
    } else {
        if (pairs * 4 >= WAVES)
            wy_launch<V, D, T, NTS, 4, 1>(P, pairs, slot_idx, mode, ln);
        else
            wy_launch<V, D, T, NTS, 2, 1>(P, pairs, slot_idx, mode, ln);    // two, 32 rows each
    }
}

template <int V, int D, typename T>
static hipError_t wy_t(const Params &P, int rows, const int *slot_idx, int mode,
                       const Launch &ln) {
    const int pairs = rows * P.heads;
    if (P.stream)
        wy_split<V, D, T, true>(P, pairs, slot_idx, mode, ln);
    else
        wy_split<V, D, T, false>(P, pairs, slot_idx, mode, ln);
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
