// Decode-step kernels for gfx950: the eager update and the DeltaLog
// append + deferred readout (also used, without the append, for readout).
//
// Operators (the DeltaLog page, "DeltaLog: Deferred Materialization of
// Recurrent States for Linear Attention Decoding", Technical Summary, Kernel
// Implementation): GDN (head-wise scalar decay + delta-rule correction), KDA
// (per-key decay + correction), RWKV6 (per-key decay, raw-value update).
// Written with S (d_v x d_k), alpha = exp(g):
//   delta rule: u = S (alpha.k), p = S (alpha.q), delta = beta (v - u),
//               S' = S diag(alpha) + delta k^T,  o = p + delta (k.q)
//   additive:   S' = S diag(w) + v k^T,          o = S (w.q) + v (k.q)
// Both are the update formulas multiplied out so that the state is read and
// written exactly once per step.
//
// The DeltaLog step leaves the base S0 untouched (Core Mechanism: appends of
// compact factors instead of dense write-back).  Its readout pulls q back
// through the logged transforms, newest first -- the key-side work the
// page's Kernel Implementation stages once per slot and head ("ReplayPrep")
// and shares with the value-side work ("AppendDecode"):
//   coef_j = beta_j k_j.q_j (additive: k_j.q_j),
//   q_{j-1} = alpha_j (q_j - coef_j k_j) (additive: w_j q_j),
//   o = S0 q_0 + sum_j coef_j v_j.
// Wave 0 runs that chain while the other waves' S0 loads are in flight and
// they append the new entry; all four waves then read out their value rows.
#include "dl_common.hpp"

namespace dl {

// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) zero_kernel(uint4 *p, size_t n16) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_zero(void *p, size_t bytes, const Launch &ln) {
    const size_t n16 = bytes / 16;
    if (n16 == 0)
        return hipSuccess;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    hipExtLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, ln.stream, ln.start, ln.stop, 0,
                       static_cast<uint4 *>(p), n16);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// eager step
// ---------------------------------------------------------------------------
template <int V, int D, typename T>
__global__ void __launch_bounds__(256)
eager_step_kernel(Params P, const int *__restrict__ slot_idx, const T *__restrict__ q,
                  const T *__restrict__ k, const T *__restrict__ v, const float *__restrict__ g,
                  const float *__restrict__ beta, float *__restrict__ o) {
    using SH = Shape<D>;
    const int H = P.heads;
    const int pr = blockIdx.x;                  // input row * H + head
    const int r = pr / H, h = pr - r * H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = lane >> 3, s = lane & 7;
    float *orow = o + (size_t)pr * D;

    const int unit = slot_idx ? slot_idx[r] : r;
    if (unit < 0 || unit >= P.units) {
        reject_row(P, orow, D, DL_FLAG_BAD_SLOT);
        return;
    }
    const size_t pair = (size_t)unit * H + h;
    const size_t io = (size_t)pr * D;
    // Issue every load before the first wait: the fill counter first, then
    // this lane's state rows, then the per-token inputs.
    const int fill = P.fill[pair];
    float *Sp = P.base + pair * D * D;
    float4 st[SH::ITER][SH::NCH];
#pragma unroll
    for (int it = 0; it < SH::ITER; ++it) {
        const int row = wave * SH::RPW + it * 8 + grp;
#pragma unroll
        for (int m = 0; m < SH::NCH; ++m)
            st[it][m] = *reinterpret_cast<const float4 *>(Sp + (size_t)row * D + col_of(s, m, 0));
    }
    float kc[SH::FPL], qc[SH::FPL], ac[SH::FPL];
#pragma unroll
    for (int m = 0; m < SH::NCH; ++m) {
        f4_to(kc + 4 * m, Elem<T>::load4(k + io + col_of(s, m, 0)));
        f4_to(qc + 4 * m, Elem<T>::load4(q + io + col_of(s, m, 0)));
        if constexpr (V != GDN)
            f4_to(ac + 4 * m, *reinterpret_cast<const float4 *>(g + io + col_of(s, m, 0)));
    }
    const float g_s = (V == GDN) ? g[pr] : 0.f;
    const float b = (V == RWKV6) ? 1.f : beta[pr];
    float vr[SH::ITER];
#pragma unroll
    for (int it = 0; it < SH::ITER; ++it)
        vr[it] = Elem<T>::load1(v + io + wave * SH::RPW + it * 8 + grp);
    __builtin_amdgcn_sched_barrier(0);
    if (fill != 0) {
        reject_row(P, orow, D, DL_FLAG_LOG_NONEMPTY);
        return;
    }
    float alpha = 1.f;
    if constexpr (V == GDN) {
        alpha = expf(g_s);
    } else {
#pragma unroll
        for (int f = 0; f < SH::FPL; ++f)
            ac[f] = expf(ac[f]);
    }

    // k.q, and the decayed key / query the row dots use
    float kq = 0.f;
    float ak[SH::FPL], aq[SH::FPL];
#pragma unroll
    for (int f = 0; f < SH::FPL; ++f) {
        kq += kc[f] * qc[f];
        ak[f] = (V == GDN) ? kc[f] : ac[f] * kc[f];
        aq[f] = (V == GDN) ? qc[f] : ac[f] * qc[f];
    }
    kq = sum8(kq);

#pragma unroll
    for (int it = 0; it < SH::ITER; ++it) {
        const int row = wave * SH::RPW + it * 8 + grp;
        float u = 0.f, p = 0.f;
#pragma unroll
        for (int m = 0; m < SH::NCH; ++m) {
            const float sv[4] = {st[it][m].x, st[it][m].y, st[it][m].z, st[it][m].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                u += sv[e] * ak[4 * m + e];
                p += sv[e] * aq[4 * m + e];
            }
        }
        u = sum8(u);
        p = sum8(p);
        if constexpr (V == GDN) {
            u *= alpha;
            p *= alpha;
        }
        const float d = (V == RWKV6) ? vr[it] : b * (vr[it] - u);
#pragma unroll
        for (int m = 0; m < SH::NCH; ++m) {
            float sv[4] = {st[it][m].x, st[it][m].y, st[it][m].z, st[it][m].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int f = 4 * m + e;
                const float decayed = (V == GDN) ? alpha * sv[e] : sv[e] * ac[f];
                sv[e] = decayed + d * kc[f];
            }
            *reinterpret_cast<float4 *>(Sp + (size_t)row * D + col_of(s, m, 0)) =
                make_float4(sv[0], sv[1], sv[2], sv[3]);
        }
        if (s == 0)
            orow[row] = p + d * kq;
    }
}

// One pull-back of the query through logged transform j (lane columns only).
// Returns coef_j; the dot ends in the 8-lane butterfly so every group agrees.
template <int V, int D>
__device__ __forceinline__ float pull_back(float *qv, const float *kj, const float *aj,
                                           float a_scalar, float bj) {
    using SH = Shape<D>;
    float d = 0.f;
#pragma unroll
    for (int f = 0; f < SH::FPL; ++f)
        d += kj[f] * qv[f];
    d = sum8(d);
    const float coef = (V == RWKV6) ? d : bj * d;
#pragma unroll
    for (int f = 0; f < SH::FPL; ++f) {
        const float a = (V == GDN) ? a_scalar : aj[f];
        qv[f] = (V == RWKV6) ? a * qv[f] : a * (qv[f] - coef * kj[f]);
    }
    return coef;
}

// ---------------------------------------------------------------------------
// Key-side staging for the chain, done by one wave: logged keys (input
// dtype), alpha = exp(g) and beta of entries [0, n) into LDS.  Loads use
// clamped in-range addresses so that a batch issues without branches and
// waits only once.
// ---------------------------------------------------------------------------
template <int V, int D, typename T>
__device__ __forceinline__ void stage_key_side(const Params &P, size_t pair, int n,
                                               unsigned char *smem, const LdsPlan &lp, int lane) {
    constexpr int B = 8;
    // An empty log reads nothing: a state without a log (L = 0) has no log
    // arrays at all, so even the clamped loads below must not run.
    if (n <= 0)
        return;
    const size_t e0 = pair * P.L;
    float *sa = reinterpret_cast<float *>(smem + lp.off_a);
    float *sb = reinterpret_cast<float *>(smem + lp.off_b);
    const int nl = n;
    // scalar decays and betas: one entry per lane (n <= 64)
    float gs = 0.f, bs = 0.f;
    if constexpr (V == GDN)
        gs = P.log_g[e0 + (lane < nl ? lane : nl - 1)];
    if constexpr (V != RWKV6)
        bs = P.log_beta[e0 + (lane < nl ? lane : nl - 1)];
    // keys: n * D * sizeof(T) contiguous bytes
    const int nk = n * D * (int)sizeof(T) / 16;
    const uint4 *ksrc = reinterpret_cast<const uint4 *>(static_cast<const T *>(P.log_k) + e0 * D);
    uint4 *kdst = reinterpret_cast<uint4 *>(smem + lp.off_k);
    for (int base = 0; base < nk; base += 64 * B) {
        uint4 tmp[B];
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const int idx = base + u * 64 + lane;
            tmp[u] = ksrc[idx < nk ? idx : nk - 1];
        }
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const int idx = base + u * 64 + lane;
            if (idx < nk)
                kdst[idx] = tmp[u];
        }
    }
    if constexpr (V != GDN) {
        const int ng = n * D / 4;
        const float4 *gsrc = reinterpret_cast<const float4 *>(P.log_g + e0 * D);
        float4 *gdst = reinterpret_cast<float4 *>(sa);
        for (int base = 0; base < ng; base += 64 * B) {
            float4 tmp[B];
#pragma unroll
            for (int u = 0; u < B; ++u) {
                const int idx = base + u * 64 + lane;
                tmp[u] = gsrc[idx < ng ? idx : ng - 1];
            }
#pragma unroll
            for (int u = 0; u < B; ++u) {
                const int idx = base + u * 64 + lane;
                if (idx < ng)
                    gdst[idx] = make_float4(expf(tmp[u].x), expf(tmp[u].y), expf(tmp[u].z), expf(tmp[u].w));
            }
        }
    }
    if (lane < n) {
        if constexpr (V == GDN)
            sa[lane] = expf(gs);
        if constexpr (V != RWKV6)
            sb[lane] = bs;
    }
}

// ---------------------------------------------------------------------------
// DeltaLog step (APPEND) / readout (!APPEND).  Five waves per (unit, head):
// wave 0 is the key side (stages the logged keys and decays, pulls q back
// through them -- computed once and shared by all value rows); waves 1..4
// each own D/4 value rows of the base, whose loads they issue before
// anything else, and do the append.
// MV: value-log entries each lane reads per row (entries s, s+8, ...).
// ---------------------------------------------------------------------------
template <int V, int D, typename T, bool APPEND, int MV>
__global__ void __launch_bounds__(320)
log_step_kernel(Params P, const int *__restrict__ slot_idx, const T *__restrict__ q,
                const T *__restrict__ k, const T *__restrict__ v, const float *__restrict__ g,
                const float *__restrict__ beta, float *__restrict__ o) {
    using SH = Shape<D>;
    extern __shared__ __align__(16) unsigned char smem[];
    const int H = P.heads, L = P.L;
    const int pr = blockIdx.x;
    const int r = pr / H, h = pr - r * H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = lane >> 3, s = lane & 7;
    const int vw = wave - 1;                         // value wave index
    float *orow = o + (size_t)pr * D;

    const int unit = slot_idx ? slot_idx[r] : r;
    if (unit < 0 || unit >= P.units) {
        reject_row(P, orow, D, DL_FLAG_BAD_SLOT);
        return;
    }
    const size_t pair = (size_t)unit * H + h;
    const size_t io = (size_t)pr * D;
    const int n = P.fill[pair];                      // entries already logged
    const float *Sp = P.base + pair * D * D;
    float4 st[SH::ITER][SH::NCH];
    if (wave > 0) {
#pragma unroll
        for (int it = 0; it < SH::ITER; ++it) {
            const int row = vw * SH::RPW + it * 8 + grp;
#pragma unroll
            for (int m = 0; m < SH::NCH; ++m)
                st[it][m] = *reinterpret_cast<const float4 *>(Sp + (size_t)row * D + col_of(s, m, 0));
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (APPEND ? (n >= L || n < 0) : (n > L || n < 0)) {
        reject_row(P, orow, D, DL_FLAG_LOG_FULL);
        return;
    }
    const LdsPlan lp = lds_plan(V, D, (int)sizeof(T), L, L, false);
    float *sq = reinterpret_cast<float *>(smem + lp.off_q);
    float *sc = reinterpret_cast<float *>(smem + lp.off_c);
    float vl[SH::ITER][MV];
    float vc[SH::ITER];

    if (wave == 0) {
        // ---- key side: pull q back through every logged transform, newest first
        float qv[SH::FPL], kj[SH::FPL], aj[SH::FPL];
        float a_s = 1.f, bj = 1.f;
#pragma unroll
        for (int m = 0; m < SH::NCH; ++m) {
            f4_to(qv + 4 * m, Elem<T>::load4(q + io + col_of(s, m, 0)));
            if constexpr (APPEND) {
                f4_to(kj + 4 * m, Elem<T>::load4(k + io + col_of(s, m, 0)));
                if constexpr (V != GDN)
                    f4_to(aj + 4 * m, *reinterpret_cast<const float4 *>(g + io + col_of(s, m, 0)));
            }
        }
        if constexpr (APPEND) {
            if constexpr (V == GDN)
                a_s = g[pr];
            if constexpr (V != RWKV6)
                bj = beta[pr];
        }
        stage_key_side<V, D, T>(P, pair, n, smem, lp, lane);
        if constexpr (APPEND) {
            if constexpr (V == GDN) {
                a_s = expf(a_s);
            } else {
#pragma unroll
                for (int f = 0; f < SH::FPL; ++f)
                    aj[f] = expf(aj[f]);
            }
            const float coef = pull_back<V, D>(qv, kj, aj, a_s, bj);
            if (lane == 0)
                sc[n] = coef;
        }
        const unsigned char *sk = smem + lp.off_k;
        const float *sa = reinterpret_cast<const float *>(smem + lp.off_a);
        const float *sb = reinterpret_cast<const float *>(smem + lp.off_b);
        for (int j = n - 1; j >= 0; --j) {
#pragma unroll
            for (int m = 0; m < SH::NCH; ++m) {
                f4_to(kj + 4 * m, lds_load4<T>(sk, j * D + col_of(s, m, 0)));
                if constexpr (V != GDN)
                    f4_to(aj + 4 * m, *reinterpret_cast<const float4 *>(sa + j * D + col_of(s, m, 0)));
            }
            if constexpr (V == GDN)
                a_s = sa[j];
            if constexpr (V != RWKV6)
                bj = sb[j];
            const float coef = pull_back<V, D>(qv, kj, aj, a_s, bj);
            if (lane == 0)
                sc[j] = coef;
        }
        if (grp == 0) {
#pragma unroll
            for (int m = 0; m < SH::NCH; ++m)
                *reinterpret_cast<float4 *>(sq + col_of(s, m, 0)) =
                    make_float4(qv[4 * m], qv[4 * m + 1], qv[4 * m + 2], qv[4 * m + 3]);
        }
    } else {
        // ---- value side: logged values of this lane's rows (clamped, branch-free
        //      loads; none at all for an empty log, whose arrays may not exist)
        const T *Vp = static_cast<const T *>(P.log_v) + pair * L * D;
        const int nl = n - 1;
#pragma unroll
        for (int it = 0; it < SH::ITER; ++it) {
            const int row = vw * SH::RPW + it * 8 + grp;
#pragma unroll
            for (int mm = 0; mm < MV; ++mm)
                vl[it][mm] = 0.f;
            if (n > 0) {
#pragma unroll
                for (int mm = 0; mm < MV; ++mm) {
                    const int j = s + 8 * mm;
                    const float x = Elem<T>::load1(Vp + (size_t)(j < n ? j : nl) * D + row);
                    vl[it][mm] = (j < n) ? x : 0.f;
                }
            }
            vc[it] = APPEND ? Elem<T>::load1(v + io + row) : 0.f;
        }
        if constexpr (APPEND) {
            // append (k, v, g, beta) at slot n: bit copies of the inputs
            const int t = tid - 64;
            const size_t e = pair * L + n;
            T *lk = static_cast<T *>(P.log_k) + e * D;
            T *lv = static_cast<T *>(P.log_v) + e * D;
            for (int i = t; i < D; i += 256) {
                lk[i] = k[io + i];
                lv[i] = v[io + i];
            }
            if constexpr (V == GDN) {
                if (t == 0)
                    P.log_g[e] = g[pr];
            } else {
                for (int i = t; i < D; i += 256)
                    P.log_g[e * D + i] = g[io + i];
            }
            if constexpr (V != RWKV6) {
                if (t == 0)
                    P.log_beta[e] = beta[pr];
            }
        }
    }
    __syncthreads();
    if (wave == 0)
        return;

    // ---- value side: o = S0 q0 + sum_j coef_j v_j for this lane's rows
    float qt[SH::FPL];
#pragma unroll
    for (int m = 0; m < SH::NCH; ++m)
        f4_to(qt + 4 * m, *reinterpret_cast<const float4 *>(sq + col_of(s, m, 0)));
    float cf[MV];
#pragma unroll
    for (int mm = 0; mm < MV; ++mm) {
        const int j = s + 8 * mm;
        cf[mm] = (j < n) ? sc[j < n ? j : 0] : 0.f;
    }
    const float ccur = (APPEND && s == 0) ? sc[n] : 0.f;
#pragma unroll
    for (int it = 0; it < SH::ITER; ++it) {
        const int row = vw * SH::RPW + it * 8 + grp;
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < SH::NCH; ++m) {
            acc += st[it][m].x * qt[4 * m] + st[it][m].y * qt[4 * m + 1] +
                   st[it][m].z * qt[4 * m + 2] + st[it][m].w * qt[4 * m + 3];
        }
#pragma unroll
        for (int mm = 0; mm < MV; ++mm)
            acc += cf[mm] * vl[it][mm];
        if (APPEND)
            acc += ccur * vc[it];
        acc = sum8(acc);
        if (s == 0)
            orow[row] = acc;
    }
    if (APPEND && tid == 64)
        P.fill[pair] = n + 1;
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
#define DL_DISPATCH(P, FN, ...)                                                          \
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
static hipError_t eager_t(const Params &P, int rows, const int *slot_idx, const void *q,
                          const void *k, const void *v, const float *g, const float *beta,
                          float *o, const Launch &ln) {
    hipExtLaunchKernelGGL((eager_step_kernel<V, D, T>), dim3(rows * P.heads), dim3(256), 0, ln.stream, ln.start, ln.stop, 0,
                       P, slot_idx, static_cast<const T *>(q), static_cast<const T *>(k),
                       static_cast<const T *>(v), g, beta, o);
    return hipGetLastError();
}

template <int V, int D, typename T, bool APPEND>
static hipError_t log_t(const Params &P, int rows, const int *slot_idx, const void *q,
                        const void *k, const void *v, const float *g, const float *beta,
                        float *o, const Launch &ln) {
    const LdsPlan lp = lds_plan(V, D, (int)sizeof(T), P.L, P.L, false);
    const dim3 grid(rows * P.heads), block(320);
    if (P.L <= 16) {
        hipExtLaunchKernelGGL((log_step_kernel<V, D, T, APPEND, 2>), grid, block, lp.bytes, ln.stream, ln.start, ln.stop, 0,
                           P, slot_idx, static_cast<const T *>(q), static_cast<const T *>(k),
                           static_cast<const T *>(v), g, beta, o);
    } else {
        hipExtLaunchKernelGGL((log_step_kernel<V, D, T, APPEND, 8>), grid, block, lp.bytes, ln.stream, ln.start, ln.stop, 0,
                           P, slot_idx, static_cast<const T *>(q), static_cast<const T *>(k),
                           static_cast<const T *>(v), g, beta, o);
    }
    return hipGetLastError();
}

template <int V, int D, typename T>
static hipError_t log_append_t(const Params &P, int rows, const int *slot_idx, const void *q,
                               const void *k, const void *v, const float *g, const float *beta,
                               float *o, const Launch &ln) {
    return log_t<V, D, T, true>(P, rows, slot_idx, q, k, v, g, beta, o, ln);
}

template <int V, int D, typename T>
static hipError_t readout_t(const Params &P, int rows, const int *slot_idx, const void *q,
                            float *o, const Launch &ln) {
    return log_t<V, D, T, false>(P, rows, slot_idx, q, nullptr, nullptr, nullptr, nullptr, o, ln);
}

hipError_t launch_eager(const Params &P, int rows, const int *slot_idx, const void *q,
                        const void *k, const void *v, const float *g, const float *beta,
                        float *o, const Launch &ln) {
    DL_DISPATCH(P, eager_t, P, rows, slot_idx, q, k, v, g, beta, o, ln);
}

hipError_t launch_log_step(const Params &P, int rows, const int *slot_idx, const void *q,
                           const void *k, const void *v, const float *g, const float *beta,
                           float *o, const Launch &ln) {
    DL_DISPATCH(P, log_append_t, P, rows, slot_idx, q, k, v, g, beta, o, ln);
}

hipError_t launch_readout(const Params &P, int rows, const int *slot_idx, const void *q,
                          float *o, const Launch &ln) {
    DL_DISPATCH(P, readout_t, P, rows, slot_idx, q, o, ln);
}

}  // namespace dl
