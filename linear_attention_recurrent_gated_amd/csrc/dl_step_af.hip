// Additive-factor DeltaLog for the delta-rule operators (GDN, KDA) on gfx950.
//
// The log holds the compact update factors (a_j, b_j = k_j) of each pending
// step with its log-decay snapshot Lam_j (the DeltaLog page, "DeltaLog:
// Deferred Materialization of Recurrent States for Linear Attention
// Decoding", Technical Summary, Core Mechanism: Base + Log).  A delta-rule
// step is  S_t = S_{t-1} diag(alpha_t) + a_t k_t^T  with
//   a_t = beta_t (v_t - S_{t-1} (alpha_t k_t)),
// so with E_c = exp(Lam_c) and D(j, c) = exp(Lam_c - Lam_j) the logical state
// over a read-only base S0 is
//   S_c = S0 diag(E_c) + sum_j a_j (k_j D(j, c))^T.
// A step that appends entry n (Lam_n = Lam_{n-1} + g) computes
//   u_j = (k_j D(j, n)) . k,   r_j = (k_j D(j, n)) . q      (j < n; r_n = k . q)
//   x   = S0 (E_n k) + sum_{j<n} u_j a_j                      (= S_{n-1}(alpha k))
//   a_n = beta (v - x)
//   o   = S0 (E_n q) + sum_{j<n} r_j a_j + r_n a_n
// -- independent dot products per entry, no triangular solve, no chain --
// and a merge is the single contraction S0' = S0 diag(E_c) + sum_j a_j
// (k_j D(j, c))^T.  The factors are fp32 (they are results, not copies of
// inputs); the keys stay bit copies.
//
// Same workgroup shape as the compact-WY step (dl_step.hip): one workgroup of
// four waves per (row, head), S0 rows in registers (lane groups of 8, lane s
// holding the columns 4s + 32m + e), the key side of the log staged in LDS by
// direct-to-LDS loads and shared by all waves through per-entry scalars.
#include "dl_common.hpp"

namespace dl {

// This wave's share of the staging of entries [0, n): keys, factors and
// (per-key decays) cumulative log-decays.  Lanes past the last element are
// masked off.
template <int V, int D, typename T>
__device__ __forceinline__ void af_stage(const Params &P, size_t pair, int n, unsigned char *smem,
                                         const AfPlan &ap, int lane, int wave) {
    const size_t e0 = pair * P.L;
    constexpr int CPK = D * (int)sizeof(T) / 16;   // 16-byte chunks per key row
    constexpr int CPF = D / 4;                     // per fp32 row
    const int nk = n * CPK, nf = n * CPF;
    const uint4 *ks = reinterpret_cast<const uint4 *>(static_cast<const T *>(P.log_k) + e0 * D);
    const uint4 *as = reinterpret_cast<const uint4 *>(static_cast<const float *>(P.log_v) + e0 * D);
    for (int b = 64 * wave; b < nk; b += 256) {
        const int idx = b + lane;
        if (idx < nk)
            load_to_lds<16>(ks + idx, smem + ap.off_k + 16 * b);
    }
    for (int b = 64 * wave; b < nf; b += 256) {
        const int idx = b + lane;
        if (idx < nf)
            load_to_lds<16>(as + idx, smem + ap.off_a + 16 * b);
    }
    if constexpr (V != GDN) {
        const uint4 *ls = reinterpret_cast<const uint4 *>(P.log_g + e0 * D);
        for (int b = 64 * wave; b < nf; b += 256) {
            const int idx = b + lane;
            if (idx < nf)
                load_to_lds<16>(ls + idx, smem + ap.off_lam + 16 * b);
        }
    }
}

// S0 <- S0 diag(E_c) + sum_{j < ct} a_j kd_j^T on this wave's rows, then the
// rows go back to the base.  kd_j = k_j D(j, c): GDN scales the staged key by
// the per-entry factor; KDA finds rows j < ct - 1 already decayed in the
// log-decay region (row ct - 1, D = 1, is the key itself).
template <int V, int D, typename T, bool NT>
__device__ __forceinline__ void af_merge_rows(const Params &P, size_t pair, int ct,
                                              const unsigned char *smem, const AfPlan &ap,
                                              float4 (&st)[Shape<D>::ITER][Shape<D>::NCH]) {
    using SH = Shape<D>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane >> 3, s = lane & 7;
    const float *sa = reinterpret_cast<const float *>(smem + ap.off_a);
    const float *slam = reinterpret_cast<const float *>(smem + ap.off_lam);
    const float *sf = reinterpret_cast<const float *>(smem + ap.off_f);
    const unsigned char *sk = smem + ap.off_k;
    float ec[SH::FPL];
    if constexpr (V == GDN) {
        const float e = fast_exp(reinterpret_cast<const float *>(smem + ap.off_s)[0]);
#pragma unroll
        for (int i = 0; i < SH::FPL; ++i)
            ec[i] = e;
    } else {
#pragma unroll
        for (int m = 0; m < SH::NCH; ++m) {
            const float4 l = *reinterpret_cast<const float4 *>(slam + (ct - 1) * D + col_of(s, m, 0));
            ec[4 * m] = fast_exp(l.x), ec[4 * m + 1] = fast_exp(l.y);
            ec[4 * m + 2] = fast_exp(l.z), ec[4 * m + 3] = fast_exp(l.w);
        }
    }
#pragma unroll
    for (int it = 0; it < SH::ITER; ++it)
#pragma unroll
        for (int m = 0; m < SH::NCH; ++m) {
            st[it][m].x *= ec[4 * m], st[it][m].y *= ec[4 * m + 1];
            st[it][m].z *= ec[4 * m + 2], st[it][m].w *= ec[4 * m + 3];
        }
    for (int j = 0; j < ct; ++j) {
        float kd[SH::FPL];
        if (V == GDN || j == ct - 1) {
            const float f = (V == GDN) ? sf[j] : 1.f;
#pragma unroll
            for (int m = 0; m < SH::NCH; ++m) {
                const float4 kk = lds_load4<T>(sk + (size_t)j * D * sizeof(T), col_of(s, m, 0));
                kd[4 * m] = f * kk.x, kd[4 * m + 1] = f * kk.y;
                kd[4 * m + 2] = f * kk.z, kd[4 * m + 3] = f * kk.w;
            }
        } else {
#pragma unroll
            for (int m = 0; m < SH::NCH; ++m)
                f4_to(kd + 4 * m, *reinterpret_cast<const float4 *>(slam + j * D + col_of(s, m, 0)));
        }
#pragma unroll
        for (int it = 0; it < SH::ITER; ++it) {
            const float aj = sa[j * D + wave * SH::RPW + it * 8 + grp];
#pragma unroll
            for (int m = 0; m < SH::NCH; ++m) {
                st[it][m].x += aj * kd[4 * m], st[it][m].y += aj * kd[4 * m + 1];
                st[it][m].z += aj * kd[4 * m + 2], st[it][m].w += aj * kd[4 * m + 3];
            }
        }
    }
    float *Sp = P.base + pair * D * D;
#pragma unroll
    for (int it = 0; it < SH::ITER; ++it) {
        const int row = wave * SH::RPW + it * 8 + grp;
#pragma unroll
        for (int m = 0; m < SH::NCH; ++m)
            store_state4<NT>(Sp + (size_t)row * D + col_of(s, m, 0), st[it][m]);
    }
}

// One workgroup per (row, head).  APPEND: the step (append + readout);
// otherwise a readout of base + log.  FUSE: the step that fills the log
// also merges it (fill back to 0).  Logs of up to 32 bf16 entries fit four
// workgroups per CU in LDS; the kernel is then held to the registers of four
// waves per SIMD as well.
template <int V, int D, typename T, bool APPEND, int MV, bool NT, bool FUSE>
__global__ void __launch_bounds__(256, (MV <= 4 && sizeof(T) == 2) ? 4 : 1)
af_step_kernel(Params P, const int *__restrict__ slot_idx, const T *__restrict__ q,
               const T *__restrict__ k, const T *__restrict__ v, const float *__restrict__ g,
               const float *__restrict__ beta, float *__restrict__ o) {
    static_assert(V == GDN || V == KDA, "delta-rule variants only");
    using SH = Shape<D>;
    using KL = KeyLayout<D>;
    constexpr int G = KL::G, RP = KL::RP, PASS = 4 * RP;   // entries per pass of the four waves
    extern __shared__ __align__(16) unsigned char smem[];
    const int H = P.heads, L = P.L;
    const int pr = blockIdx.x;
    const int r = pr / H, h = pr - r * H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float *orow = o + (size_t)pr * D;

    const int unit = slot_idx ? slot_idx[r] : r;
    if (unit < 0 || unit >= P.units) {
        reject_row(P, orow, D, DL_FLAG_BAD_SLOT);
        return;
    }
    const size_t pair = (size_t)unit * H + h;
    const size_t io = (size_t)pr * D;
    const size_t e0 = pair * L;
    const AfPlan ap = af_plan(V, D, (int)sizeof(T), L);
    T *sk = reinterpret_cast<T *>(smem + ap.off_k);
    float *sa = reinterpret_cast<float *>(smem + ap.off_a);
    float *slam = reinterpret_cast<float *>(smem + ap.off_lam);
    float *sr = reinterpret_cast<float *>(smem + ap.off_r);
    float *su = reinterpret_cast<float *>(smem + ap.off_u);
    float *sf = reinterpret_cast<float *>(smem + ap.off_f);
    float *ss = reinterpret_cast<float *>(smem + ap.off_s);
    float *sqe = reinterpret_cast<float *>(smem + ap.off_qe);
    float *ske = reinterpret_cast<float *>(smem + ap.off_ke);

    // ---- loads that need nothing: fill, this wave's rows of S0, the inputs
    const int n = P.fill[pair];
    const int grp = lane >> 3, s = lane & 7;
    const float *Sp = P.base + pair * D * D;
    float4 st[SH::ITER][SH::NCH];
#pragma unroll
    for (int it = 0; it < SH::ITER; ++it) {
        const int row = wave * SH::RPW + it * 8 + grp;
#pragma unroll
        for (int m = 0; m < SH::NCH; ++m)
            st[it][m] = load_state4<NT>(Sp + (size_t)row * D + col_of(s, m, 0));
    }
    const int cg = lane % G, ro = lane / G, ch0 = 8 * cg;
    float qv[8], kn[8];
    load8<T>(q + io + ch0, qv);
    if constexpr (APPEND)
        load8<T>(k + io + ch0, kn);
    __builtin_amdgcn_sched_barrier(0);
    if (APPEND ? (n >= L || n < 0) : (n > L || n < 0)) {
        reject_row(P, orow, D, DL_FLAG_LOG_FULL);
        return;
    }

    // ---- loads that need n: the new value on this lane's rows, beta, the
    //      staging, and (wave 0) Lam and the decayed q and k
    float vc[SH::ITER];
#pragma unroll
    for (int it = 0; it < SH::ITER; ++it)
        vc[it] = APPEND ? Elem<T>::load1(v + io + wave * SH::RPW + it * 8 + grp) : 0.f;
    const float b_in = APPEND ? beta[pr] : 0.f;
    if (n > 0)
        af_stage<V, D, T>(P, pair, n, smem, ap, lane, wave);
    const int ct = APPEND ? n + 1 : n;   // entries the readout sees
    if (wave == 0) {
        float en[8];                     // E_c on this lane's channels
        if constexpr (V == GDN) {
            const int jl = lane < n ? lane : (n > 0 ? n - 1 : 0);
            float lam_j = n > 0 ? P.log_g[e0 + jl] : 0.f;
            const float prev = n > 0 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam_j), n - 1)) : 0.f;
            const float lam_c = APPEND ? prev + g[pr] : prev;
            if (APPEND && lane == n)
                lam_j = lam_c;
            if (lane < ct)
                sf[lane] = fast_exp(lam_c - lam_j);
            if (lane == 0)
                ss[0] = lam_c;
            const float e = fast_exp(lam_c);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                en[i] = e;
        } else {
            float lc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                lc[i] = 0.f;
            if (n > 0)
                load8<float>(P.log_g + (e0 + n - 1) * D + ch0, lc);
            if constexpr (APPEND) {
                float gn[8];
                load8<float>(g + io + ch0, gn);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    lc[i] += gn[i];
                if (ro == 0)
                    store8<float>(slam + n * D + ch0, lc);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                en[i] = fast_exp(lc[i]);
        }
        if (ro == 0) {
            float t[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                t[i] = en[i] * qv[i];
            store8<float>(sqe + ch0, t);
            if constexpr (APPEND) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    t[i] = en[i] * kn[i];
                store8<float>(ske + ch0, t);
                store8<T>(sk + n * D + ch0, kn);
            }
        }
    }
    wait_vm_all();      // this wave's staging (and everything before it) has landed
    __syncthreads();    // 1: staged entries, the new entry, Lam, E q, E k

    const bool merging = FUSE && APPEND && n == L - 1;
    float lc[8];
    if constexpr (V != GDN) {
        if (ct > 0)
            load8<float>(slam + (ct - 1) * D + ch0, lc);
        else
#pragma unroll
            for (int i = 0; i < 8; ++i)
                lc[i] = 0.f;
    }

    // ---- r_j = (k_j D(j, c)) . q and u_j = (k_j D(j, c)) . k for this
    //      wave's entries of each pass; a merging step keeps k_j D(j, c)
    //      (per-key decays) in place of Lam_j for the merge
    const int npass = (ct + PASS - 1) / PASS;
    for (int p = 0; p < npass; ++p) {
        const int j = PASS * p + RP * wave + ro;
        const int jc = j < ct ? j : ct - 1;
        float kd[8];
        load8<T>(sk + jc * D + ch0, kd);
        if constexpr (V != GDN) {
            float lr[8];
            load8<float>(slam + jc * D + ch0, lr);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                kd[i] *= fast_exp(lc[i] - lr[i]);
            if (FUSE && merging && j < n)
                store8<float>(slam + j * D + ch0, kd);
        }
        float ar = 0.f, au = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            ar += kd[i] * qv[i];
            if constexpr (APPEND)
                au += kd[i] * kn[i];
        }
        ar = group_sum<G>(ar);
        if constexpr (APPEND)
            au = group_sum<G>(au);
        const float f = (V == GDN) ? sf[jc] : 1.f;
        if (cg == 0 && j < ct) {
            sr[j] = f * ar;
            if constexpr (APPEND)
                su[j] = f * au;
        }
    }
    __syncthreads();    // 2: r and u of every entry (and the merge's decayed keys)

    // ---- per row: x = S0 (E k) + sum u_j a_j, a_n = beta (v - x),
    //      o = S0 (E q) + sum r_j a_j + r_n a_n
    float qt[SH::FPL], kt[SH::FPL];
#pragma unroll
    for (int m = 0; m < SH::NCH; ++m) {
        f4_to(qt + 4 * m, *reinterpret_cast<const float4 *>(sqe + col_of(s, m, 0)));
        if constexpr (APPEND)
            f4_to(kt + 4 * m, *reinterpret_cast<const float4 *>(ske + col_of(s, m, 0)));
    }
    float cr[MV], cu[MV];
#pragma unroll
    for (int mm = 0; mm < MV; ++mm) {
        const int j = s + 8 * mm;
        const int jc = j < n ? j : 0;
        cr[mm] = j < n ? sr[jc] : 0.f;
        cu[mm] = (APPEND && j < n) ? su[jc] : 0.f;
    }
    const float rn = APPEND ? sr[n] : 0.f;      // r_n = k . q (D(n, n) = 1)
    float *alog = static_cast<float *>(P.log_v) + (e0 + n) * D;
#pragma unroll
    for (int it = 0; it < SH::ITER; ++it) {
        const int row = wave * SH::RPW + it * 8 + grp;
        float ao = 0.f, ax = 0.f;
#pragma unroll
        for (int m = 0; m < SH::NCH; ++m) {
            ao += st[it][m].x * qt[4 * m] + st[it][m].y * qt[4 * m + 1] +
                  st[it][m].z * qt[4 * m + 2] + st[it][m].w * qt[4 * m + 3];
            if constexpr (APPEND)
                ax += st[it][m].x * kt[4 * m] + st[it][m].y * kt[4 * m + 1] +
                      st[it][m].z * kt[4 * m + 2] + st[it][m].w * kt[4 * m + 3];
        }
#pragma unroll
        for (int mm = 0; mm < MV; ++mm) {
            const int j = s + 8 * mm;
            const float aj = j < n ? sa[(j < n ? j : 0) * D + row] : 0.f;
            ao += cr[mm] * aj;
            if constexpr (APPEND)
                ax += cu[mm] * aj;
        }
        ao = sum8(ao);
        if constexpr (APPEND) {
            ax = sum8(ax);
            const float an = b_in * (vc[it] - ax);
            ao += rn * an;
            if (s == 1)
                alog[row] = an;
            if (FUSE && merging && s == 0)
                sa[n * D + row] = an;
        }
        if (s == 0)
            orow[row] = ao;
    }
    if constexpr (APPEND) {
        // the rest of entry n: the key (bit copy) and Lam_n
        if (wave == 0) {
            constexpr int CPK = D * (int)sizeof(T) / 16;
            if (lane < CPK)
                reinterpret_cast<uint4 *>(static_cast<T *>(P.log_k) + (e0 + n) * D)[lane] =
                    reinterpret_cast<const uint4 *>(sk + n * D)[lane];
            if constexpr (V == GDN) {
                if (lane == 0)
                    P.log_g[e0 + n] = ss[0];
            } else {
                if (lane < D / 4)
                    reinterpret_cast<float4 *>(P.log_g + (e0 + n) * D)[lane] =
                        reinterpret_cast<const float4 *>(slam + n * D)[lane];
            }
        }
        if constexpr (FUSE) {
            if (merging) {
                wave_lds_sync();   // this wave's rows of a_n are in LDS
                af_merge_rows<V, D, T, NT>(P, pair, ct, smem, ap, st);
                if (tid == 0)
                    P.fill[pair] = 0;
                return;
            }
        }
        if (tid == 0)
            P.fill[pair] = n + 1;
    }
}

// Merge of the selected units' logs into their bases (DL_MERGE_FULL: full
// logs; DL_MERGE_ALL: every non-empty log).
template <int V, int D, typename T, bool NT>
__global__ void __launch_bounds__(256) af_merge_kernel(Params P, const int *__restrict__ slot_idx,
                                                       int mode) {
    static_assert(V == GDN || V == KDA, "delta-rule variants only");
    using SH = Shape<D>;
    extern __shared__ __align__(16) unsigned char smem[];
    size_t pair;
    int n;
    if (!resolve_merge_pair(P, slot_idx, mode, pair, n))
        return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = lane >> 3, s = lane & 7;
    const AfPlan ap = af_plan(V, D, (int)sizeof(T), P.L);
    const size_t e0 = pair * P.L;
    const float *Sp = P.base + pair * D * D;
    float4 st[SH::ITER][SH::NCH];
#pragma unroll
    for (int it = 0; it < SH::ITER; ++it) {
        const int row = wave * SH::RPW + it * 8 + grp;
#pragma unroll
        for (int m = 0; m < SH::NCH; ++m)
            st[it][m] = load_state4<NT>(Sp + (size_t)row * D + col_of(s, m, 0));
    }
    af_stage<V, D, T>(P, pair, n, smem, ap, lane, wave);
    if constexpr (V == GDN) {
        if (wave == 0) {
            const int jl = lane < n ? lane : n - 1;
            const float lam_j = P.log_g[e0 + jl];
            const float lam_c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam_j), n - 1));
            if (lane < n)
                reinterpret_cast<float *>(smem + ap.off_f)[lane] = fast_exp(lam_c - lam_j);
            if (lane == 0)
                reinterpret_cast<float *>(smem + ap.off_s)[0] = lam_c;
        }
    }
    wait_vm_all();
    __syncthreads();
    if constexpr (V != GDN) {
        // decayed keys k_j D(j, c) in place of Lam_j, j < n - 1
        constexpr int CPR = D / 8;
        const T *sk = reinterpret_cast<const T *>(smem + ap.off_k);
        float *slam = reinterpret_cast<float *>(smem + ap.off_lam);
        for (int idx = tid; idx < (n - 1) * CPR; idx += 256) {
            const int j = idx / CPR, c = 8 * (idx - j * CPR);
            float kr[8], lr[8], lc[8];
            load8<T>(sk + j * D + c, kr);
            load8<float>(slam + j * D + c, lr);
            load8<float>(slam + (n - 1) * D + c, lc);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                kr[i] *= fast_exp(lc[i] - lr[i]);
            store8<float>(slam + j * D + c, kr);
        }
        __syncthreads();
    }
    af_merge_rows<V, D, T, NT>(P, pair, n, smem, ap, st);
    if (tid == 0)
        P.fill[pair] = 0;
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
#define DL_DISPATCH_AF(P, FN, ...)                                                       \
    do {                                                                                 \
        const bool bf = (P).dtype == DL_BF16;                                            \
        const bool gdn = (P).variant == DL_GDN;                                          \
        if ((P).D == 128) {                                                              \
            if (bf) {                                                                    \
                if (gdn) return FN<GDN, 128, uint16_t>(__VA_ARGS__);                     \
                return FN<KDA, 128, uint16_t>(__VA_ARGS__);                              \
            }                                                                            \
            if (gdn) return FN<GDN, 128, float>(__VA_ARGS__);                            \
            return FN<KDA, 128, float>(__VA_ARGS__);                                     \
        }                                                                                \
        if (bf) {                                                                        \
            if (gdn) return FN<GDN, 64, uint16_t>(__VA_ARGS__);                          \
            return FN<KDA, 64, uint16_t>(__VA_ARGS__);                                   \
        }                                                                                \
        if (gdn) return FN<GDN, 64, float>(__VA_ARGS__);                                 \
        return FN<KDA, 64, float>(__VA_ARGS__);                                          \
    } while (0)

template <int V, int D, typename T, bool APPEND, int MV>
static void af_launch(const Params &P, int rows, const int *slot_idx, const void *q,
                      const void *k, const void *v, const float *g, const float *beta, float *o,
                      const Launch &ln) {
    const bool fuse = APPEND && P.fuse;
    const AfPlan ap = af_plan(V, D, (int)sizeof(T), P.L);
    const dim3 grid(rows * P.heads), block(256);
#define DL_AF_LAUNCH(NTV, FV)                                                                          \
    hipExtLaunchKernelGGL((af_step_kernel<V, D, T, APPEND, MV, NTV, FV>), grid, block, ap.bytes,       \
                          ln.stream, ln.start, ln.stop, 0, P, slot_idx, static_cast<const T *>(q),     \
                          static_cast<const T *>(k), static_cast<const T *>(v), g, beta, o)
    if constexpr (APPEND) {
        if (P.stream) {
            if (fuse) DL_AF_LAUNCH(true, true); else DL_AF_LAUNCH(true, false);
        } else {
            if (fuse) DL_AF_LAUNCH(false, true); else DL_AF_LAUNCH(false, false);
        }
    } else {
        if (P.stream) DL_AF_LAUNCH(true, false); else DL_AF_LAUNCH(false, false);
    }
#undef DL_AF_LAUNCH
}

template <int V, int D, typename T, bool APPEND>
static hipError_t af_t(const Params &P, int rows, const int *slot_idx, const void *q,
                       const void *k, const void *v, const float *g, const float *beta, float *o,
                       const Launch &ln) {
    // MV = logged factors per lane per row = ceil(L / 8), rounded up to 2, 4 or 8
    if (P.L <= 16)
        af_launch<V, D, T, APPEND, 2>(P, rows, slot_idx, q, k, v, g, beta, o, ln);
    else if (P.L <= 32)
        af_launch<V, D, T, APPEND, 4>(P, rows, slot_idx, q, k, v, g, beta, o, ln);
    else
        af_launch<V, D, T, APPEND, 8>(P, rows, slot_idx, q, k, v, g, beta, o, ln);
    return hipGetLastError();
}

template <int V, int D, typename T>
static hipError_t af_step_t(const Params &P, int rows, const int *slot_idx, const void *q,
                            const void *k, const void *v, const float *g, const float *beta,
                            float *o, const Launch &ln) {
    return af_t<V, D, T, true>(P, rows, slot_idx, q, k, v, g, beta, o, ln);
}

template <int V, int D, typename T>
static hipError_t af_readout_t(const Params &P, int rows, const int *slot_idx, const void *q,
                               float *o, const Launch &ln) {
    return af_t<V, D, T, false>(P, rows, slot_idx, q, nullptr, nullptr, nullptr, nullptr, o, ln);
}

template <int V, int D, typename T>
static hipError_t af_merge_t(const Params &P, int rows, const int *slot_idx, int mode,
                             const Launch &ln) {
    const AfPlan ap = af_plan(V, D, (int)sizeof(T), P.L);
    if (P.stream)
        hipExtLaunchKernelGGL((af_merge_kernel<V, D, T, true>), dim3(rows * P.heads), dim3(256), ap.bytes,
                              ln.stream, ln.start, ln.stop, 0, P, slot_idx, mode);
    else
        hipExtLaunchKernelGGL((af_merge_kernel<V, D, T, false>), dim3(rows * P.heads), dim3(256), ap.bytes,
                              ln.stream, ln.start, ln.stop, 0, P, slot_idx, mode);
    return hipGetLastError();
}

hipError_t launch_af_step(const Params &P, int rows, const int *slot_idx, const void *q,
                          const void *k, const void *v, const float *g, const float *beta,
                          float *o, const Launch &ln) {
    DL_DISPATCH_AF(P, af_step_t, P, rows, slot_idx, q, k, v, g, beta, o, ln);
}

hipError_t launch_af_readout(const Params &P, int rows, const int *slot_idx, const void *q,
                             float *o, const Launch &ln) {
    DL_DISPATCH_AF(P, af_readout_t, P, rows, slot_idx, q, o, ln);
}

hipError_t launch_af_merge(const Params &P, int rows, const int *slot_idx, int mode,
                           const Launch &ln) {
    DL_DISPATCH_AF(P, af_merge_t, P, rows, slot_idx, mode, ln);
}

}  // namespace dl
