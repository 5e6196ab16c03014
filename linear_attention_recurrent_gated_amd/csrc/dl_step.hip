// Decode-step kernels for gfx950: the eager update and the DeltaLog
// append + deferred readout (also used, without the append, for readout).
//
// Operators (the DeltaLog page, "DeltaLog: Deferred Materialization of
// Recurrent States for Linear Attention Decoding", Technical Summary, Kernel
// Implementation): GDN (head-wise scalar decay + delta-rule correction), KDA
// (per-key decay + correction), RWKV6 (per-key decay, raw-value update); and
// the gated form of the Gated DeltaNet-2 abstract (CARVE page, Explore
// similar work), KDA with a channel-wise erase gate e and write gate w.
// Written with S (d_v x d_k), alpha = exp(g):
//   delta rule: u = S (alpha.k), p = S (alpha.q), delta = beta (v - u),
//               S' = S diag(alpha) + delta k^T,  o = p + delta (k.q)
//   gated:      u = S (alpha.e.k), delta = w.v - u, the rest as above
//   additive:   S' = S diag(w) + v k^T,          o = S (w.q) + v (k.q)
// Both are the update formulas multiplied out so that the state is read and
// written exactly once per step.
//
// The DeltaLog step leaves the base S0 untouched (Core Mechanism: appends of
// compact factors instead of dense write-back) and reads out S0 q0 plus a
// combination of the logged values, with q0 and the coefficients formed by
// the key side in compact WY form (see the log step kernel below).  Four
// waves per (row, head) hold S0 in registers while they share that key-side
// work through LDS.
#include "dl_common.hpp"

namespace dl {

// Eight input elements (bf16 pairs or floats) loaded as they are; converted
// where they are used, so that the conversion does not make the compiler
// wait for the load (and for every load issued before it) any earlier.
template <typename T>
__device__ __forceinline__ void load_bits8(const T *p, uint4 (&r)[2]) {
    r[0] = reinterpret_cast<const uint4 *>(p)[0];
    if constexpr (sizeof(T) == 4)
        r[1] = reinterpret_cast<const uint4 *>(p)[1];
}

template <typename T>
__device__ __forceinline__ void bits8_to_float(const uint4 (&r)[2], float *x) {
    if constexpr (sizeof(T) == 4) {
        x[0] = __uint_as_float(r[0].x), x[1] = __uint_as_float(r[0].y);
        x[2] = __uint_as_float(r[0].z), x[3] = __uint_as_float(r[0].w);
        x[4] = __uint_as_float(r[1].x), x[5] = __uint_as_float(r[1].y);
        x[6] = __uint_as_float(r[1].z), x[7] = __uint_as_float(r[1].w);
    } else {
        x[0] = bf16_lo(r[0].x), x[1] = bf16_hi(r[0].x), x[2] = bf16_lo(r[0].y), x[3] = bf16_hi(r[0].y);
        x[4] = bf16_lo(r[0].z), x[5] = bf16_hi(r[0].z), x[6] = bf16_lo(r[0].w), x[7] = bf16_hi(r[0].w);
    }
}

}  // namespace dl

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
template <int V, int D, typename T, bool NT>
__global__ void __launch_bounds__(256)
eager_step_kernel(Params P, const int *__restrict__ slot_idx, const T *__restrict__ q,
                  const T *__restrict__ k, const T *__restrict__ v, const float *__restrict__ g,
                  const float *__restrict__ beta, float *__restrict__ o) {
    using SH = Shape<D>;
    const int H = P.heads;
    int h;
    const int r = step_row(P, h);
    if (r < 0) {
        reject_row(P, nullptr, D, DL_FLAG_BAD_SLOT);
        return;
    }
    const int pr = r * H + h;                   // input row * H + head
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
            st[it][m] = load_state4<NT>(Sp + (size_t)row * D + col_of(s, m, 0));
    }
    float kc[SH::FPL], qc[SH::FPL], ac[SH::FPL], ec[SH::FPL];
    const float *gate = beta + (size_t)pr * 2 * D;   // gated: erase gate, then write gate
#pragma unroll
    for (int m = 0; m < SH::NCH; ++m) {
        f4_to(kc + 4 * m, Elem<T>::load4(k + io + col_of(s, m, 0)));
        f4_to(qc + 4 * m, Elem<T>::load4(q + io + col_of(s, m, 0)));
        if constexpr (V != GDN)
            f4_to(ac + 4 * m, *reinterpret_cast<const float4 *>(g + io + col_of(s, m, 0)));
        if constexpr (V == GDN2)
            f4_to(ec + 4 * m, *reinterpret_cast<const float4 *>(gate + col_of(s, m, 0)));
    }
    const float g_s = (V == GDN) ? g[pr] : 0.f;
    const float b = (V == RWKV6 || V == GDN2) ? 1.f : beta[pr];
    float vr[SH::ITER], wr[SH::ITER];
#pragma unroll
    for (int it = 0; it < SH::ITER; ++it) {
        vr[it] = Elem<T>::load1(v + io + wave * SH::RPW + it * 8 + grp);
        wr[it] = (V == GDN2) ? gate[D + wave * SH::RPW + it * 8 + grp] : 1.f;
    }
    __builtin_amdgcn_sched_barrier(0);
    if (fill != 0) {
        reject_row(P, orow, D, DL_FLAG_LOG_NONEMPTY);
        return;
    }
    // The gated form scales this lane's state columns by alpha once, in
    // place: its row dots and update then read S diag(alpha), and the decay
    // vector is dead before the row loop.  (The other per-key-decay
    // variants measured faster folding alpha into the key and query.)
    constexpr bool FOLD = V == GDN2;
    float alpha = 1.f;
    if constexpr (V == GDN) {
        alpha = expf(g_s);
    } else {
#pragma unroll
        for (int f = 0; f < SH::FPL; ++f)
            ac[f] = expf(ac[f]);
    }
    if constexpr (FOLD) {
#pragma unroll
        for (int it = 0; it < SH::ITER; ++it) {
#pragma unroll
            for (int m = 0; m < SH::NCH; ++m) {
                st[it][m].x *= ac[4 * m];
                st[it][m].y *= ac[4 * m + 1];
                st[it][m].z *= ac[4 * m + 2];
                st[it][m].w *= ac[4 * m + 3];
            }
        }
    }

    // k.q, and the key / query the row dots read
    float kq = 0.f;
    float ak[SH::FPL], aq[SH::FPL];
#pragma unroll
    for (int f = 0; f < SH::FPL; ++f) {
        kq += kc[f] * qc[f];
        ak[f] = (V == GDN) ? kc[f] : (V == GDN2) ? ec[f] * kc[f] : ac[f] * kc[f];
        aq[f] = (V == GDN || FOLD) ? qc[f] : ac[f] * qc[f];
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
        const float d = (V == RWKV6) ? vr[it] : (V == GDN2) ? wr[it] * vr[it] - u : b * (vr[it] - u);
#pragma unroll
        for (int m = 0; m < SH::NCH; ++m) {
            float sv[4] = {st[it][m].x, st[it][m].y, st[it][m].z, st[it][m].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int f = 4 * m + e;
                const float decayed = (V == GDN) ? alpha * sv[e] : FOLD ? sv[e] : sv[e] * ac[f];
                sv[e] = decayed + d * kc[f];
            }
            store_state4<NT>(Sp + (size_t)row * D + col_of(s, m, 0), make_float4(sv[0], sv[1], sv[2], sv[3]));
        }
        if (s == 0)
            orow[row] = p + d * kq;
    }
}

// ---------------------------------------------------------------------------
// DeltaLog step / readout.
//
// The log holds entries j = 0..c (the newest last) with Lam_j, the log-decay
// accumulated from the first entry through entry j (stored cumulative).
// With E_j = exp(Lam_j), D(j, i) = exp(Lam_i - Lam_j) and R = (I + N)^{-1}
// for the couplings N_ij = beta_i k_i.(D(i, j) k_j) (i < j), the pending
// transforms pull q back in compact WY form:
//   r_j   = beta_j k_j.(D(j, c) q)           (additive variant: beta = 1)
//   coef  = R r                              (additive: coef = r)
//   q0    = E_c q - sum_j coef_j E_j k_j     (additive: no k terms)
//   o     = S0 q0 + sum_j coef_j v_j
// which equals pulling q back through the transforms one at a time, newest
// first (coef_j = beta_j k_j.q_j, q_{j-1} = alpha_j (q_j - coef_j k_j)),
// without that chain of dependent steps.  R gains one column per appended
// entry, R[:n, n] = -R[:n, :n] N[:n, n], kept in the log beside the keys:
// key-side factors computed once per slot and head, as the DeltaLog page's
// Kernel Implementation describes.
//
// One workgroup of four waves per (row, head).  Every wave holds D/4 rows of
// S0 in registers (loads issued first) and takes a quarter of the key side:
// the dot products and q0 run in the chunk layout (eight channels of one
// entry per lane, DPP / permlane reductions), R r with one entry per lane
// (each wave computes it for itself, so no barrier separates it from q0).
// ---------------------------------------------------------------------------

// This wave's share of the staging of entries [0, n) of `pair` into LDS
// (direct-to-LDS loads, every fourth batch of 64 lanes): keys, values,
// cumulative log-decays (per-key decays) and the packed R columns.  Lanes past the last
// element are masked off, so nothing is written past entry n - 1.
template <int V, int D, typename T>
__device__ __forceinline__ void stage_log(const Params &P, size_t pair, int n, unsigned char *smem,
                                          const StepPlan &sp, int lane, int wave) {
    const size_t e0 = pair * P.L;
    constexpr int CPR = D * (int)sizeof(T) / 16;
    const int nk = n * CPR;
    const uint4 *ks = reinterpret_cast<const uint4 *>(static_cast<const T *>(P.log_k) + e0 * D);
    const uint4 *vs = reinterpret_cast<const uint4 *>(static_cast<const T *>(P.log_v) + e0 * D);
    for (int b = 64 * wave; b < nk; b += 256) {
        const int idx = b + lane;
        if (idx < nk) {
            load_to_lds<16>(ks + idx, smem + sp.off_k + 16 * b);
            load_to_lds<16>(vs + idx, smem + sp.off_v + 16 * b);
        }
    }
    if constexpr (V != GDN) {
        const int nl = n * (D / 4);
        const float4 *ls = reinterpret_cast<const float4 *>(P.log_g + e0 * D);
        for (int b = 64 * wave; b < nl; b += 256) {
            const int idx = b + lane;
            if (idx < nl)
                load_to_lds<16>(ls + idx, smem + sp.off_lam + 16 * b);
        }
    }
    if constexpr (V != RWKV6) {
        const int nt = n * (n - 1) / 2;
        const float *ts = P.log_t + pair * packed_t_len(V, P.L);
        for (int b = 64 * wave; b < nt; b += 256) {
            const int idx = b + lane;
            if (idx < nt)
                load_to_lds<4>(ts + idx, smem + sp.off_t + 4 * b);
        }
    }
}

// Merge in the step that fills the log (all ct = L entries staged, R
// complete in LDS, this wave's rows of S0 in registers):
//   S' = S0 diag(E_c) + (V^T - S0 Kt^T) Y,   Kt_j = E_j k_j,   Y = R Q,
//   Q_i = beta_i k_i D(i, c)   (additive variant: R = I, beta = 1),
// the readout formula written for every q at once.  Z = V^T - S0 Kt^T is
// formed first, while S0 is intact, and kept in registers (lane s of a row
// group holds the entries j = s + 8 mm); then S0 diag(E_c) + Z Y, with Y
// built 16 rows at a time by all waves, becomes the new base; fill = 0.
template <int V, int D, typename T, int MV, bool NT>
__device__ __forceinline__ void merge_in_step(const Params &P, size_t pair, int ct, unsigned char *smem,
                                              const StepPlan &sp,
                                              float4 (&st)[Shape<D>::ITER][Shape<D>::NCH],
                                              const float (&vc)[Shape<D>::ITER], float lam_c) {
    using SH = Shape<D>;
    constexpr int ITER = SH::ITER, NCH = SH::NCH;
    const int n = ct - 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = lane >> 3, s = lane & 7;
    const float *slam = reinterpret_cast<const float *>(smem + sp.off_lam);
    const float *sT = reinterpret_cast<const float *>(smem + sp.off_t);
    const float *sf = reinterpret_cast<const float *>(smem + sp.off_f);
    const float *sl = reinterpret_cast<const float *>(smem + sp.off_l);
    const T *vr = reinterpret_cast<const T *>(smem + sp.off_v);
    float *sy = reinterpret_cast<float *>(smem + sp.off_y);
    const unsigned char *kbase = smem + sp.off_k;
    auto krow = [&](int j) { return kbase + (size_t)j * D * sizeof(T); };

    // ---- Z[row][j] = v_j[row] - S0[row, :] . (E_j k_j), one entry at a time
    float zr[ITER][MV];
#pragma unroll
    for (int it = 0; it < ITER; ++it)
#pragma unroll
        for (int mm = 0; mm < MV; ++mm)
            zr[it][mm] = 0.f;
#pragma unroll
    for (int mm = 0; mm < MV; ++mm) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = 8 * mm + u;
            if (j >= ct)
                break;
            float w[ITER];
#pragma unroll
            for (int it = 0; it < ITER; ++it)
                w[it] = 0.f;
            if constexpr (V != RWKV6) {
#pragma unroll
                for (int m = 0; m < NCH; ++m) {
                    float4 kt = lds_load4<T>(krow(j), col_of(s, m, 0));
                    if constexpr (V == GDN) {
                        const float e = fast_exp(sl[j]);
                        kt.x *= e, kt.y *= e, kt.z *= e, kt.w *= e;
                    } else {
                        const float4 l4 = *reinterpret_cast<const float4 *>(slam + j * D + col_of(s, m, 0));
                        kt.x *= fast_exp(l4.x), kt.y *= fast_exp(l4.y);
                        kt.z *= fast_exp(l4.z), kt.w *= fast_exp(l4.w);
                    }
#pragma unroll
                    for (int it = 0; it < ITER; ++it)
                        w[it] += st[it][m].x * kt.x + st[it][m].y * kt.y + st[it][m].z * kt.z + st[it][m].w * kt.w;
                }
            }
#pragma unroll
            for (int it = 0; it < ITER; ++it) {
                const int row = wave * SH::RPW + it * 8 + grp;
                const float wsum = (V == RWKV6) ? 0.f : sum8(w[it]);
                const float vj = (j < n) ? Elem<T>::load1(vr + j * D + row) : vc[it];
                zr[it][mm] = (s == u) ? vj - wsum : zr[it][mm];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---- S' = S0 diag(E_c) + Z Y
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
        if constexpr (V == GDN) {
            const float e = fast_exp(lam_c);
#pragma unroll
            for (int it = 0; it < ITER; ++it)
                st[it][m].x *= e, st[it][m].y *= e, st[it][m].z *= e, st[it][m].w *= e;
        } else {
            const float4 l4 = *reinterpret_cast<const float4 *>(slam + n * D + col_of(s, m, 0));
            const float4 e = make_float4(fast_exp(l4.x), fast_exp(l4.y), fast_exp(l4.z), fast_exp(l4.w));
#pragma unroll
            for (int it = 0; it < ITER; ++it)
                st[it][m].x *= e.x, st[it][m].y *= e.y, st[it][m].z *= e.z, st[it][m].w *= e.w;
        }
    }
    constexpr int TPC = 256 / D;          // threads per key channel building Y
    constexpr int JPT = 16 / TPC;         // rows of the Y chunk per thread
    const int ych = tid % D, ysub = tid / D;
    const float lc_y = (V == GDN) ? 0.f : slam[n * D + ych];
    const int gbase = lane & ~7;
#pragma unroll
    for (int c = 0; c < MV / 2; ++c) {
        const int j0 = 16 * c;
        if (j0 >= ct)
            break;
        __syncthreads();   // the previous chunk of Y is consumed
        {
            // Y_j[ch] = sum_{i >= j} R[j, i] Q_i[ch] for j = jb .. jb + JPT - 1
            const int jb = j0 + JPT * ysub;
            float acc[JPT];
#pragma unroll
            for (int u = 0; u < JPT; ++u)
                acc[u] = 0.f;
            // the additive variant has R = I: only i = j contributes
            const int iend = (V == RWKV6) ? (jb + JPT < ct ? jb + JPT : ct) : ct;
            for (int i = jb; i < iend; ++i) {
                float qi = sf[i] * Elem<T>::load1(reinterpret_cast<const T *>(krow(i)) + ych);
                if constexpr (V != GDN)
                    qi *= fast_exp(lc_y - slam[i * D + ych]);
#pragma unroll
                for (int u = 0; u < JPT; ++u) {
                    const int j = jb + u;
                    float r = (j == i) ? 1.f : 0.f;
                    if constexpr (V != RWKV6)
                        r = (j < i) ? sT[i * (i - 1) / 2 + j] : r;
                    acc[u] += r * qi;
                }
            }
#pragma unroll
            for (int u = 0; u < JPT; ++u)
                sy[(JPT * ysub + u) * D + ych] = acc[u];
        }
        __syncthreads();
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int mm = 2 * c + h;
            for (int u = 0; u < 8; ++u) {
                const int j = 8 * mm + u;
                if (j >= ct)
                    break;
                float4 y[NCH];
#pragma unroll
                for (int m = 0; m < NCH; ++m)
                    y[m] = *reinterpret_cast<const float4 *>(sy + (j - j0) * D + col_of(s, m, 0));
#pragma unroll
                for (int it = 0; it < ITER; ++it) {
                    const float z = __shfl(zr[it][mm], gbase | u);
#pragma unroll
                    for (int m = 0; m < NCH; ++m) {
                        st[it][m].x += z * y[m].x, st[it][m].y += z * y[m].y;
                        st[it][m].z += z * y[m].z, st[it][m].w += z * y[m].w;
                    }
                }
            }
        }
    }

    float *Sp = P.base + pair * D * D;
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int row = wave * SH::RPW + it * 8 + grp;
#pragma unroll
        for (int m = 0; m < NCH; ++m)
            store_state4<NT>(Sp + (size_t)row * D + col_of(s, m, 0), st[it][m]);
    }
    if (tid == 0)
        P.fill[pair] = 0;
}

// Entry n of the log, from its LDS copies to HBM (wave 0, after the last
// barrier): k and v (bit copies of the inputs), the decay accumulated through
// it, beta, and column n of R.
template <int V, int D, typename T>
__device__ __forceinline__ void log_append(const Params &P, size_t pair, int n, const unsigned char *smem,
                                           const StepPlan &sp, int lane) {
    const size_t e = pair * P.L + n;
    constexpr int CPR = D * (int)sizeof(T) / 16;     // 16-byte chunks per row
    if (lane < CPR) {
        const uint4 *kr = reinterpret_cast<const uint4 *>(smem + sp.off_k + (size_t)n * D * sizeof(T));
        const uint4 *vr = reinterpret_cast<const uint4 *>(smem + sp.off_v + (size_t)n * D * sizeof(T));
        reinterpret_cast<uint4 *>(static_cast<T *>(P.log_k) + e * D)[lane] = kr[lane];
        reinterpret_cast<uint4 *>(static_cast<T *>(P.log_v) + e * D)[lane] = vr[lane];
    }
    if constexpr (V == GDN) {
        if (lane == 0)
            P.log_g[e] = reinterpret_cast<const float *>(smem + sp.off_l)[n];
    } else {
        if (lane < D / 4) {
            const float4 *lr = reinterpret_cast<const float4 *>(smem + sp.off_lam + (size_t)n * D * 4);
            reinterpret_cast<float4 *>(P.log_g + e * D)[lane] = lr[lane];
        }
    }
    if constexpr (V != RWKV6) {
        if (lane == 0)
            P.log_beta[e] = *reinterpret_cast<const float *>(smem + sp.off_bn);
        if (lane < n)
            P.log_t[pair * packed_t_len(V, P.L) + n * (n - 1) / 2 + lane] =
                reinterpret_cast<const float *>(smem + sp.off_t)[n * (n - 1) / 2 + lane];
    }
}

// With the merge fused in (bf16 inputs, logs of up to 32 entries) the kernel
// is held to four waves per SIMD, i.e. four workgroups per CU, like the
// plain step.
template <int V, int D, typename T, bool APPEND, int MV, bool NT, bool FUSE>
__global__ void __launch_bounds__(256, (FUSE && MV <= 4 && sizeof(T) == 2) ? 4 : 1)
log_step_kernel(Params P, const int *__restrict__ slot_idx, const T *__restrict__ q,
                const T *__restrict__ k, const T *__restrict__ v, const float *__restrict__ g,
                const float *__restrict__ beta, float *__restrict__ o) {
    using SH = Shape<D>;
    using KL = KeyLayout<D>;
    constexpr int G = KL::G, RP = KL::RP, PASS = 4 * RP;   // entries per pass of the four waves
    constexpr bool DELTA = V != RWKV6;
    extern __shared__ __align__(16) unsigned char smem[];
    const int H = P.heads, L = P.L;
    int h;
    const int r = step_row(P, h);
    if (r < 0) {
        reject_row(P, nullptr, D, DL_FLAG_BAD_SLOT);
        return;
    }
    const int pr = r * H + h;                   // input row * H + head
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
    const StepPlan sp = step_plan(V, D, (int)sizeof(T), L, FUSE);
    float *slam = reinterpret_cast<float *>(smem + sp.off_lam);
    float *sT = reinterpret_cast<float *>(smem + sp.off_t);
    float *sr = reinterpret_cast<float *>(smem + sp.off_r);
    float *su = reinterpret_cast<float *>(smem + sp.off_u);
    float *sf = reinterpret_cast<float *>(smem + sp.off_f);
    float *sl = reinterpret_cast<float *>(smem + sp.off_l);
    float *sb_new = reinterpret_cast<float *>(smem + sp.off_bn);
    float *sc = reinterpret_cast<float *>(smem + sp.off_c) + 64 * wave;
    float *se = reinterpret_cast<float *>(smem + sp.off_e) + 64 * wave;
    float *sq = reinterpret_cast<float *>(smem + sp.off_q);
    float *sqin = reinterpret_cast<float *>(smem + sp.off_qin);
    auto krow = [&](int j) { return reinterpret_cast<T *>(smem + sp.off_k) + j * D; };

    // ---- loads that need nothing: fill, this wave's rows of S0, the inputs
    const int n = P.fill[pair];
    const int grp = lane >> 3, s = lane & 7;
    // logged value v_j[row] (staged); 0 past the n stored entries
    auto vlog = [&](int j, int row) {
        const T *vr = reinterpret_cast<const T *>(smem + sp.off_v);
        return j < n ? Elem<T>::load1(vr + (j < n ? j : 0) * D + row) : 0.f;
    };
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
    // q and k on this lane's channels, kept as loaded until they are used: a
    // conversion here would make the compiler wait for them, and so for the
    // base loads issued before them, ahead of the loads below
    uint4 qbits[2] = {}, kbits[2] = {};
    load_bits8<T>(q + io + ch0, qbits);
    if constexpr (APPEND)
        load_bits8<T>(k + io + ch0, kbits);
    __builtin_amdgcn_sched_barrier(0);
    if (APPEND ? (n >= L || n < 0) : (n > L || n < 0)) {
        reject_row(P, orow, D, DL_FLAG_LOG_FULL);
        return;
    }

    // ---- loads that need n: logged values of this wave's rows (clamped,
    //      branch-free; an empty log reads a dummy in-range address instead),
    //      the per-entry scalars and the append's inputs, then the staging.
    //      At d = 128 every wave loads the scalars and inputs, without a
    //      condition, ahead of the staging, so that they are in flight with the
    //      base and nothing waits for them before wave 0 uses them (entry 0 of
    //      an empty log is a valid address); at d = 64, where a workgroup's
    //      loads are few, the extra loads cost more than they hide, and wave 0
    //      loads them after the staging.
    constexpr bool EARLY = D == 128;
    float vc[SH::ITER];       // the new entry's value on this lane's rows
#pragma unroll
    for (int it = 0; it < SH::ITER; ++it)
        vc[it] = APPEND ? Elem<T>::load1(v + io + wave * SH::RPW + it * 8 + grp) : 0.f;
    // A state without a log (an eager state's readout runs here with L = 0)
    // has no log arrays: its early loads read this workgroup's output row
    // instead, a valid address, and go unused (n = 0).
    const bool has_log = L > 0;
    const int jl = lane < n ? lane : (n > 0 ? n - 1 : 0);
    float lam_raw = 0.f, b_raw = 1.f, g_s = 0.f, b_in = 1.f;
    uint4 lbits[2] = {}, vbits[2] = {}, gbits[2] = {};   // Lam_{n-1}, v and g on this lane's channels
    if constexpr (EARLY) {
        if constexpr (V == GDN)
            lam_raw = (has_log ? P.log_g + e0 + jl : orow)[0];
        if constexpr (DELTA)
            b_raw = (has_log ? P.log_beta + e0 + jl : orow)[0];
        if constexpr (V != GDN)
            load_bits8<float>(has_log ? P.log_g + (e0 + (n > 0 ? n - 1 : 0)) * D + ch0 : orow + ch0, lbits);
        if constexpr (APPEND) {
            load_bits8<T>(v + io + ch0, vbits);
            if constexpr (V == GDN)
                g_s = g[pr];
            else
                load_bits8<float>(g + io + ch0, gbits);
            if constexpr (DELTA)
                b_in = beta[pr];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (n > 0)
        stage_log<V, D, T>(P, pair, n, smem, sp, lane, wave);
    if (wave == 0) {
        float qv[8], kn[8];
        bits8_to_float<T>(qbits, qv);
        if constexpr (APPEND)
            bits8_to_float<T>(kbits, kn);
        float lam_j = 0.f, b_j = 1.f;     // entry `lane`: Lam (GDN) and beta
        float lc[8];                      // Lam_c on this lane's channels (per-key decays)
        float gn[8], vv[8];
        if constexpr (EARLY) {
            lam_j = n > 0 ? lam_raw : 0.f;
            b_j = n > 0 ? b_raw : 1.f;
            bits8_to_float<float>(lbits, lc);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                lc[i] = n > 0 ? lc[i] : 0.f;
            if constexpr (APPEND) {
                bits8_to_float<T>(vbits, vv);
                bits8_to_float<float>(gbits, gn);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                lc[i] = 0.f;
            if (n > 0) {
                if constexpr (V == GDN)
                    lam_j = P.log_g[e0 + jl];
                if constexpr (DELTA)
                    b_j = P.log_beta[e0 + jl];
                if constexpr (V != GDN)
                    load8<float>(P.log_g + (e0 + n - 1) * D + ch0, lc);
            }
            if constexpr (APPEND) {
                load8<T>(v + io + ch0, vv);
                if constexpr (V == GDN)
                    g_s = g[pr];
                else
                    load8<float>(g + io + ch0, gn);
                if constexpr (DELTA)
                    b_in = beta[pr];
            }
        }
        // Lam_c, then the append of entry n: bit copies of k and v, the decay
        // accumulated through it, beta
        float lam_c = 0.f;
        if constexpr (V == GDN) {
            const float prev = n > 0 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam_j), n - 1)) : 0.f;
            lam_c = APPEND ? prev + g_s : prev;
        } else if constexpr (APPEND) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                lc[i] += gn[i];
        }
        if constexpr (APPEND) {
            // entry n goes to LDS now and to the log in HBM at the end of the
            // kernel, so that no barrier waits for those stores
            if (ro == 0) {
                store8<T>(krow(n) + ch0, kn);
                store8<T>(reinterpret_cast<T *>(smem + sp.off_v) + n * D + ch0, vv);
                if constexpr (V != GDN)
                    store8<float>(slam + n * D + ch0, lc);
            }
            if (lane == 0)
                sb_new[0] = b_in;
            if (lane == n) {
                lam_j = lam_c;
                b_j = b_in;
            }
        }
        // per-entry factor of the dot products: beta_j (GDN: times D(j, c)),
        // and (GDN) Lam_j for the other waves
        const int ct = APPEND ? n + 1 : n;
        if (lane < ct) {
            float f = b_j;
            if constexpr (V == GDN) {
                f *= fast_exp(lam_c - lam_j);
                sl[lane] = lam_j;
            }
            sf[lane] = f;
        }
        if (ro == 0)
            store8<float>(sqin + ch0, qv);
    }
    wait_vm_all();      // this wave's staging (and everything before it) has landed
    __syncthreads();    // 1: staged entries, the new entry, per-entry factors

    const int ct = APPEND ? n + 1 : n;   // entries the readout sees
    const int npass = (ct + PASS - 1) / PASS;
    float qv[8], kn[8];
    bits8_to_float<T>(qbits, qv);
    if constexpr (APPEND)
        bits8_to_float<T>(kbits, kn);

    float lam_c = 0.f, lc[8];
    if constexpr (V == GDN) {
        lam_c = ct > 0 ? sl[ct - 1] : 0.f;
    } else {
        if (ct > 0)
            load8<float>(slam + (ct - 1) * D + ch0, lc);
        else
#pragma unroll
            for (int i = 0; i < 8; ++i)
                lc[i] = 0.f;
    }

    // ---- r_j = f_j k_j.(D q) and, for the appended entry, u_j = f_j k_j.(D k_n)
    //      (the decays D(j, c) inside the dot for the per-key variants); this
    //      wave's entries of each pass
    for (int p = 0; p < npass; ++p) {
        const int j = PASS * p + RP * wave + ro;
        const int jc = j < ct ? j : ct - 1;
        float kr[8], lr[8];
        load8<T>(krow(jc) + ch0, kr);
        if constexpr (V != GDN)
            load8<float>(slam + jc * D + ch0, lr);
        const float fr = DELTA ? sf[jc] : 1.f;
        float ar = 0.f, au = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float kd = kr[i];
            if constexpr (V != GDN)
                kd *= fast_exp(lc[i] - lr[i]);
            ar += kd * qv[i];
            if constexpr (APPEND && DELTA)
                au += kd * kn[i];
        }
        ar = group_sum<G>(ar);
        if constexpr (APPEND && DELTA)
            au = group_sum<G>(au);
        if (cg == 0 && j < ct) {
            sr[j] = fr * ar;
            if constexpr (APPEND && DELTA)
                su[j] = fr * au;
        }
    }
    __syncthreads();    // 2: r and u of every entry

    // ---- lane i: the new column R[i, n] = -(u_i + sum_{i<m<n} R[i, m] u_m)
    //      and coef_i = (R r)_i, sharing the loads of R (every wave for itself;
    //      wave 0 stores the new column)
    float coef = 0.f;
    if (lane < ct) {
        const int i = lane;
        coef = sr[i];
        if constexpr (DELTA) {
            float acc_u = APPEND ? su[i] : 0.f;
            const int mend = APPEND ? n : ct;     // stored columns m < mend
            for (int m0 = 0; m0 < mend; m0 += 8) {
                float rv[8], uv[8], Rv[8];
                // sr and su hold entries < ct only: the batch's tail past mend is
                // whatever the LDS held before, so it is selected away, not
                // multiplied by zero (a stale Inf or NaN would survive that)
#pragma unroll
                for (int t = 0; t < 8; t += 4) {
                    const float4 a = *reinterpret_cast<const float4 *>(sr + m0 + t);
                    const float ra[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        rv[t + e] = (m0 + t + e < mend) ? ra[e] : 0.f;
                    if constexpr (APPEND) {
                        const float4 b = *reinterpret_cast<const float4 *>(su + m0 + t);
                        const float ub[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            uv[t + e] = (m0 + t + e < mend) ? ub[e] : 0.f;
                    }
                }
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int m = m0 + t;
                    // column m holds rows 0..m-1; other lanes read an in-range dummy
                    const int lim = m < mend ? m : 0;
                    const int col = m < mend ? m * (m - 1) / 2 : 0;
                    Rv[t] = sT[col + (i < lim ? i : 0)];
                    Rv[t] = i < lim ? Rv[t] : 0.f;
                }
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    coef += Rv[t] * rv[t];
                    if constexpr (APPEND)
                        acc_u += Rv[t] * uv[t];
                }
            }
            if constexpr (APPEND) {
                if (i < n) {
                    const float w = -acc_u;
                    if (wave == 0)
                        sT[n * (n - 1) / 2 + i] = w;   // logged at the end; read by a merge
                    coef += w * sr[n];
                }
            }
        }
    }
    if (lane < PASS * npass) {
        sc[lane] = coef;                    // zero past the last entry
        if constexpr (V == GDN)
            se[lane] = lane < ct ? coef * fast_exp(sl[lane]) : 0.f;
    }
    wave_lds_sync();

    // ---- q0 = E_c q - sum_j coef_j E_j k_j on this wave's quarter of the
    //      channels: lane l takes channels 8 (l % LQ) .. + 7 of the quarter for
    //      the entries RQ p + l / LQ
    {
        constexpr int LQ = D / 32, RQ = 64 / LQ;   // lanes across the quarter, entries per step
        const int c4 = lane % LQ, jr = lane / LQ;
        const int chq = (D / 4) * wave + 8 * c4;
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[i] = 0.f;
        if constexpr (DELTA) {
            for (int p = 0; p < ct; p += RQ) {
                const int j = p + jr;
                const int jc = j < ct ? j : ct - 1;
                float kr[8], lr[8];
                load8<T>(krow(jc) + chq, kr);
                if constexpr (V != GDN)
                    load8<float>(slam + jc * D + chq, lr);
                const float cr = j < ct ? ((V == GDN) ? se[jc] : sc[jc]) : 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    float x = cr * kr[i];
                    if constexpr (V != GDN)
                        x *= fast_exp(lr[i]);
                    acc[i] += x;
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] = sum_mod<LQ>(acc[i]);
        }
        if (jr == 0) {
            float qq[8], lq[8], out[8];
            load8<float>(sqin + chq, qq);
            if constexpr (V != GDN) {
                if (ct > 0)
                    load8<float>(slam + (ct - 1) * D + chq, lq);
                else
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        lq[i] = 0.f;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                out[i] = fast_exp((V == GDN) ? lam_c : lq[i]) * qq[i] - acc[i];
            store8<float>(sq + chq, out);
        }
    }
    __syncthreads();    // 3: q0

    // ---- o = S0 q0 + sum_j coef_j v_j for this wave's rows
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
        const int row = wave * SH::RPW + it * 8 + grp;
        float acc_o = 0.f;
#pragma unroll
        for (int m = 0; m < SH::NCH; ++m) {
            acc_o += st[it][m].x * qt[4 * m] + st[it][m].y * qt[4 * m + 1] +
                     st[it][m].z * qt[4 * m + 2] + st[it][m].w * qt[4 * m + 3];
        }
#pragma unroll
        for (int mm = 0; mm < MV; ++mm)
            acc_o += cf[mm] * vlog(s + 8 * mm, row);
        if (APPEND)
            acc_o += ccur * vc[it];
        acc_o = sum8(acc_o);
        if (s == 0)
            orow[row] = acc_o;
    }
    if constexpr (APPEND) {
        if constexpr (FUSE) {
            // the entry that fills the log goes straight into the merged base;
            // the emptied log keeps no copy of it
            if (n == L - 1) {
                merge_in_step<V, D, T, MV, NT>(P, pair, ct, smem, sp, st, vc, lam_c);
                return;
            }
        }
        if (wave == 0)
            log_append<V, D, T>(P, pair, n, smem, sp, lane);
        if (tid == 0)
            P.fill[pair] = n + 1;
    }
}

// ---------------------------------------------------------------------------
// Chunked compact-WY step for per-key decays at d = 128 with logs of 33 to 64
// entries (no merge in the step).  The same arithmetic as log_step_kernel,
// but its 64 staged keys, values and decay rows (72 KiB of LDS, two
// workgroups per CU) become 32 keys and decay rows at a time, the values
// staged in their place once q0 is formed and the appended entry kept apart:
// 36 KiB, four workgroups per CU.  The dot products run over the first 32
// entries, then the rest once they are staged; q0 over the entries still
// staged, then over the first 32 staged again; the readout after the values.
// ---------------------------------------------------------------------------

// Direct-to-LDS staging of rows [j0, j0 + cnt) of a log array of `row`
// 16-byte chunks per entry into `dst` (this wave's batches of 64 lanes).
__device__ __forceinline__ void stage_rows(const void *base, size_t e0, int j0, int cnt, int row,
                                           unsigned char *dst, int lane, int wave) {
    const uint4 *src = reinterpret_cast<const uint4 *>(base) + (e0 + j0) * row;
    const int nchunk = cnt * row;
    for (int b = 64 * wave; b < nchunk; b += 256) {
        const int idx = b + lane;
        if (idx < nchunk)
            load_to_lds<16>(src + idx, dst + 16 * b);
    }
}

template <int D, typename T, bool APPEND, bool NT>
__global__ void __launch_bounds__(256, 4)
log_step_chunked_kernel(Params P, const int *__restrict__ slot_idx, const T *__restrict__ q,
                        const T *__restrict__ k, const T *__restrict__ v, const float *__restrict__ g,
                        const float *__restrict__ beta, float *__restrict__ o) {
    using SH = Shape<D>;
    using KL = KeyLayout<D>;
    constexpr int G = KL::G, RP = KL::RP, PASS = 4 * RP;   // entries per pass of the four waves
    constexpr int CH = 32;                                // entries per staged chunk
    constexpr int MV = 8;                                 // value entries per lane per row
    constexpr int KROW = D * (int)sizeof(T) / 16;         // 16-byte chunks per key / value row
    constexpr int LROW = D / 4;                           // 16-byte chunks per decay row
    extern __shared__ __align__(16) unsigned char smem[];
    const int H = P.heads, L = P.L;
    int h;
    const int r = step_row(P, h);
    if (r < 0) {
        reject_row(P, nullptr, D, DL_FLAG_BAD_SLOT);
        return;
    }
    const int pr = r * H + h;
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
    const ChunkPlan cp = chunk_plan(D, (int)sizeof(T), L);
    float *sT = reinterpret_cast<float *>(smem + cp.off_t);
    float *sr = reinterpret_cast<float *>(smem + cp.off_r);
    float *su = reinterpret_cast<float *>(smem + cp.off_u);
    float *sf = reinterpret_cast<float *>(smem + cp.off_f);
    float *sb_new = reinterpret_cast<float *>(smem + cp.off_bn);
    float *sc = reinterpret_cast<float *>(smem + cp.off_c) + 64 * wave;
    float *sq = reinterpret_cast<float *>(smem + cp.off_q);
    float *sqin = reinterpret_cast<float *>(smem + cp.off_qin);
    float *sln = reinterpret_cast<float *>(smem + cp.off_ln);   // Lam_c (the appended entry's, or the newest's)

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
    // q and k on this lane's channels, kept as loaded until they are used
    // (as in the log step kernel)
    uint4 qbits[2] = {}, kbits[2] = {};
    load_bits8<T>(q + io + ch0, qbits);
    if constexpr (APPEND)
        load_bits8<T>(k + io + ch0, kbits);
    __builtin_amdgcn_sched_barrier(0);
    if (APPEND ? (n >= L || n < 0) : (n > L || n < 0)) {
        reject_row(P, orow, D, DL_FLAG_LOG_FULL);
        return;
    }
    const int ct = APPEND ? n + 1 : n;       // entries the readout sees
    const int na = n < CH ? n : CH;          // logged entries in the first chunk

    // ---- loads that need n: this lane's rows of the new value, the
    //      per-entry scalars and the append's inputs (every wave, without a
    //      condition, so that they fly with the base; this kernel serves logs
    //      of more than 32 entries, so the log arrays exist), then the first
    //      chunk and R
    float vc[SH::ITER];
#pragma unroll
    for (int it = 0; it < SH::ITER; ++it)
        vc[it] = APPEND ? Elem<T>::load1(v + io + wave * SH::RPW + it * 8 + grp) : 0.f;
    const int jl = lane < n ? lane : (n > 0 ? n - 1 : 0);
    const float b_raw = P.log_beta[e0 + jl];
    uint4 lbits[2] = {}, vbits[2] = {}, gbits[2] = {};   // Lam_{n-1}, v and g on this lane's channels
    load_bits8<float>(P.log_g + (e0 + (n > 0 ? n - 1 : 0)) * D + ch0, lbits);
    float b_in = 1.f;
    if constexpr (APPEND) {
        load_bits8<T>(v + io + ch0, vbits);
        load_bits8<float>(g + io + ch0, gbits);
        b_in = beta[pr];
    }
    __builtin_amdgcn_sched_barrier(0);
    stage_rows(P.log_k, e0, 0, na, KROW, smem + cp.off_kc, lane, wave);
    stage_rows(P.log_g, e0, 0, na, LROW, smem + cp.off_lc, lane, wave);
    {
        const int nt = n * (n - 1) / 2;
        const float *ts = P.log_t + pair * packed_t_len(DL_KDA, L);
        for (int b = 64 * wave; b < nt; b += 256)
            if (b + lane < nt)
                load_to_lds<4>(ts + b + lane, smem + cp.off_t + 4 * b);
    }
    if (wave == 0) {
        float qv[8], kn[8];
        bits8_to_float<T>(qbits, qv);
        if constexpr (APPEND)
            bits8_to_float<T>(kbits, kn);
        float b_j = n > 0 ? b_raw : 1.f, lc[8], gn[8], vv[8];
        bits8_to_float<float>(lbits, lc);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            lc[i] = n > 0 ? lc[i] : 0.f;
        if constexpr (APPEND) {
            bits8_to_float<T>(vbits, vv);
            bits8_to_float<float>(gbits, gn);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                lc[i] += gn[i];
        }
        if (ro == 0) {
            store8<float>(sln + ch0, lc);      // Lam_c
            if constexpr (APPEND) {
                store8<T>(reinterpret_cast<T *>(smem + cp.off_kn) + ch0, kn);
                store8<T>(reinterpret_cast<T *>(smem + cp.off_vn) + ch0, vv);
            }
            store8<float>(sqin + ch0, qv);
        }
        if constexpr (APPEND) {
            if (lane == 0)
                sb_new[0] = b_in;
            if (lane == n)
                b_j = b_in;
        }
        if (lane < ct)
            sf[lane] = b_j;
    }
    wait_vm_all();
    __syncthreads();    // 1: the first chunk, R, the new entry, per-entry factors
    float qv[8], kn[8];
    bits8_to_float<T>(qbits, qv);
    if constexpr (APPEND)
        bits8_to_float<T>(kbits, kn);

    // key and decay rows of entry j: the appended entry's own copies, or
    // row j - c0 of the staged chunk
    auto krow = [&](int j, int c0) {
        return (APPEND && j == n) ? reinterpret_cast<const T *>(smem + cp.off_kn)
                                  : reinterpret_cast<const T *>(smem + cp.off_kc) + (j - c0) * D;
    };
    auto lrow = [&](int j, int c0) {
        return (APPEND && j == n) ? static_cast<const float *>(sln)
                                  : reinterpret_cast<const float *>(smem + cp.off_lc) + (j - c0) * D;
    };
    float lc[8];
    load8<float>(sln + ch0, lc);

    // ---- r_j = f_j k_j.(D q) and u_j = f_j k_j.(D k_n): passes 0, 1 over the
    //      first chunk, passes 2, 3 over the second once it is staged
    auto dots = [&](int p, int c0) {
        const int j = PASS * p + RP * wave + ro;
        const int jc = j < ct ? j : ct - 1;
        float kr[8], lr[8];
        load8<T>(krow(jc, c0) + ch0, kr);
        load8<float>(lrow(jc, c0) + ch0, lr);
        const float fr = sf[jc];
        float ar = 0.f, au = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float kd = kr[i] * fast_exp(lc[i] - lr[i]);
            ar += kd * qv[i];
            if constexpr (APPEND)
                au += kd * kn[i];
        }
        ar = group_sum<G>(ar);
        if constexpr (APPEND)
            au = group_sum<G>(au);
        if (cg == 0 && j < ct) {
            sr[j] = fr * ar;
            if constexpr (APPEND)
                su[j] = fr * au;
        }
    };
    const int npass = (ct + PASS - 1) / PASS;
    for (int p = 0; p < 2 && p < npass; ++p)
        dots(p, 0);
    if (ct > CH) {
        __syncthreads();    // every wave is done with the first chunk
        stage_rows(P.log_k, e0, CH, n - CH, KROW, smem + cp.off_kc, lane, wave);
        stage_rows(P.log_g, e0, CH, n - CH, LROW, smem + cp.off_lc, lane, wave);
        wait_vm_all();
        __syncthreads();    // the second chunk
        for (int p = 2; p < npass; ++p)
            dots(p, CH);
    }
    __syncthreads();    // 2: r and u of every entry

    // ---- lane i: the new column R[i, n] and coef_i = (R r)_i (every wave
    //      for itself; wave 0 stores the new column)
    float coef = 0.f;
    if (lane < ct) {
        const int i = lane;
        coef = sr[i];
        float acc_u = APPEND ? su[i] : 0.f;
        const int mend = APPEND ? n : ct;     // stored columns m < mend
        for (int m0 = 0; m0 < mend; m0 += 8) {
            float rv[8], uv[8], Rv[8];
#pragma unroll
            for (int t = 0; t < 8; t += 4) {
                const float4 a = *reinterpret_cast<const float4 *>(sr + m0 + t);
                const float ra[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    rv[t + e] = (m0 + t + e < mend) ? ra[e] : 0.f;
                if constexpr (APPEND) {
                    const float4 b = *reinterpret_cast<const float4 *>(su + m0 + t);
                    const float ub[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        uv[t + e] = (m0 + t + e < mend) ? ub[e] : 0.f;
                }
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int m = m0 + t;
                const int lim = m < mend ? m : 0;
                const int col = m < mend ? m * (m - 1) / 2 : 0;
                Rv[t] = sT[col + (i < lim ? i : 0)];
                Rv[t] = i < lim ? Rv[t] : 0.f;
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                coef += Rv[t] * rv[t];
                if constexpr (APPEND)
                    acc_u += Rv[t] * uv[t];
            }
        }
        if constexpr (APPEND) {
            if (i < n) {
                const float w = -acc_u;
                if (wave == 0)
                    sT[n * (n - 1) / 2 + i] = w;
                coef += w * sr[n];
            }
        }
    }
    if (lane < PASS * npass)
        sc[lane] = coef;
    wave_lds_sync();

    // ---- q0 = E_c q - sum_j coef_j E_j k_j on this wave's quarter of the
    //      channels: over the entries of the staged chunk, then (longer logs)
    //      over the first chunk staged again
    constexpr int LQ = D / 32, RQ = 64 / LQ;
    const int c4 = lane % LQ, jr = lane / LQ;
    const int chq = (D / 4) * wave + 8 * c4;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        acc[i] = 0.f;
    auto q0_part = [&](int jbeg, int jend, int c0) {
        for (int p = jbeg; p < jend; p += RQ) {
            const int j = p + jr;
            const int jc = j < ct ? j : ct - 1;
            float kr[8], lr[8];
            load8<T>(krow(jc, c0) + chq, kr);
            load8<float>(lrow(jc, c0) + chq, lr);
            const float cr = j < jend ? sc[jc] : 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] += cr * kr[i] * fast_exp(lr[i]);
        }
    };
    if (ct > CH) {
        q0_part(CH, ct, CH);
        __syncthreads();    // every wave is done with the second chunk
        stage_rows(P.log_k, e0, 0, CH, KROW, smem + cp.off_kc, lane, wave);
        stage_rows(P.log_g, e0, 0, CH, LROW, smem + cp.off_lc, lane, wave);
        wait_vm_all();
        __syncthreads();    // the first chunk again
        q0_part(0, CH, 0);
    } else {
        q0_part(0, ct, 0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
        acc[i] = sum_mod<LQ>(acc[i]);
    if (jr == 0) {
        float qq[8], lq[8], out[8];
        load8<float>(sqin + chq, qq);
        load8<float>(sln + chq, lq);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            out[i] = fast_exp(lq[i]) * qq[i] - acc[i];
        store8<float>(sq + chq, out);
    }
    __syncthreads();    // 3: q0; the chunks are free

    // ---- the logged values, in the chunks' place
    stage_rows(P.log_v, e0, 0, n, KROW, smem + cp.off_v, lane, wave);
    wait_vm_all();
    __syncthreads();    // 4: values

    // ---- o = S0 q0 + sum_j coef_j v_j for this wave's rows
    const T *vrows = reinterpret_cast<const T *>(smem + cp.off_v);
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
        const int row = wave * SH::RPW + it * 8 + grp;
        float acc_o = 0.f;
#pragma unroll
        for (int m = 0; m < SH::NCH; ++m)
            acc_o += st[it][m].x * qt[4 * m] + st[it][m].y * qt[4 * m + 1] +
                     st[it][m].z * qt[4 * m + 2] + st[it][m].w * qt[4 * m + 3];
#pragma unroll
        for (int mm = 0; mm < MV; ++mm) {
            const int j = s + 8 * mm;
            const float x = Elem<T>::load1(vrows + (j < n ? j : 0) * D + row);
            acc_o += cf[mm] * (j < n ? x : 0.f);
        }
        if (APPEND)
            acc_o += ccur * vc[it];
        acc_o = sum8(acc_o);
        if (s == 0)
            orow[row] = acc_o;
    }

    // ---- append entry n: k and v (bit copies), Lam_n, beta, column n of R
    if constexpr (APPEND) {
        if (wave == 0) {
            const size_t e = e0 + n;
            if (lane < KROW) {
                reinterpret_cast<uint4 *>(static_cast<T *>(P.log_k) + e * D)[lane] =
                    reinterpret_cast<const uint4 *>(smem + cp.off_kn)[lane];
                reinterpret_cast<uint4 *>(static_cast<T *>(P.log_v) + e * D)[lane] =
                    reinterpret_cast<const uint4 *>(smem + cp.off_vn)[lane];
            }
            if (lane < LROW)
                reinterpret_cast<float4 *>(P.log_g + e * D)[lane] = reinterpret_cast<const float4 *>(sln)[lane];
            if (lane == 0)
                P.log_beta[e] = sb_new[0];
            if (lane < n)
                P.log_t[pair * packed_t_len(DL_KDA, L) + n * (n - 1) / 2 + lane] = sT[n * (n - 1) / 2 + lane];
        }
        if (tid == 0)
            P.fill[pair] = n + 1;
    }
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

// the eager step also runs the gated form
#define DL_DISPATCH_EAGER(P, FN, ...)                                                    \
    do {                                                                                 \
        if ((P).variant == DL_GDN2) {                                                    \
            const bool bf = (P).dtype == DL_BF16;                                        \
            if ((P).D == 128) {                                                          \
                if (bf) return FN<GDN2, 128, uint16_t>(__VA_ARGS__);                     \
                return FN<GDN2, 128, float>(__VA_ARGS__);                                \
            }                                                                            \
            if (bf) return FN<GDN2, 64, uint16_t>(__VA_ARGS__);                          \
            return FN<GDN2, 64, float>(__VA_ARGS__);                                     \
        }                                                                                \
        DL_DISPATCH(P, FN, __VA_ARGS__);                                                 \
    } while (0)

template <int V, int D, typename T>
static hipError_t eager_t(const Params &P, int rows, const int *slot_idx, const void *q,
                          const void *k, const void *v, const float *g, const float *beta,
                          float *o, const Launch &ln) {
    if (P.stream)
        hipExtLaunchKernelGGL((eager_step_kernel<V, D, T, true>), dim3(rows * P.heads), dim3(256), 0, ln.stream, ln.start,
                              ln.stop, 0, P, slot_idx, static_cast<const T *>(q), static_cast<const T *>(k),
                              static_cast<const T *>(v), g, beta, o);
    else
        hipExtLaunchKernelGGL((eager_step_kernel<V, D, T, false>), dim3(rows * P.heads), dim3(256), 0, ln.stream, ln.start,
                              ln.stop, 0, P, slot_idx, static_cast<const T *>(q), static_cast<const T *>(k),
                              static_cast<const T *>(v), g, beta, o);
    return hipGetLastError();
}

template <int V, int D, typename T, bool APPEND, int MV>
static void log_launch(const Params &P, int rows, const int *slot_idx, const void *q,
                       const void *k, const void *v, const float *g, const float *beta,
                       float *o, const Launch &ln) {
    const bool fuse = APPEND && P.fuse;
    const StepPlan sp = step_plan(V, D, (int)sizeof(T), P.L, fuse);
    const dim3 grid(rows * P.heads), block(256);
#define DL_LOG_LAUNCH(NTV, FV)                                                                         \
    hipExtLaunchKernelGGL((log_step_kernel<V, D, T, APPEND, MV, NTV, FV>), grid, block, sp.bytes,      \
                          ln.stream, ln.start, ln.stop, 0, P, slot_idx, static_cast<const T *>(q),     \
                          static_cast<const T *>(k), static_cast<const T *>(v), g, beta, o)
    if constexpr (APPEND) {
        if (P.stream) {
            if (fuse) DL_LOG_LAUNCH(true, true); else DL_LOG_LAUNCH(true, false);
        } else {
            if (fuse) DL_LOG_LAUNCH(false, true); else DL_LOG_LAUNCH(false, false);
        }
    } else {
        if (P.stream) DL_LOG_LAUNCH(true, false); else DL_LOG_LAUNCH(false, false);
    }
#undef DL_LOG_LAUNCH
}

template <int V, int D, typename T, bool APPEND>
static hipError_t log_t(const Params &P, int rows, const int *slot_idx, const void *q,
                        const void *k, const void *v, const float *g, const float *beta,
                        float *o, const Launch &ln) {
    // per-key decays at d = 128 with more than 32 entries and no merge in the
    // step: the chunked kernel (four workgroups per CU instead of two)
    if constexpr (V == KDA && D == 128) {
        if (P.L > 32 && !(APPEND && P.fuse)) {
            const ChunkPlan cp = chunk_plan(D, (int)sizeof(T), P.L);
            const dim3 grid(rows * P.heads), block(256);
#define DL_CHUNK_LAUNCH(NTV)                                                                          \
    hipExtLaunchKernelGGL((log_step_chunked_kernel<D, T, APPEND, NTV>), grid, block, cp.bytes, ln.stream, \
                          ln.start, ln.stop, 0, P, slot_idx, static_cast<const T *>(q),               \
                          static_cast<const T *>(k), static_cast<const T *>(v), g, beta, o)
            if (P.stream) DL_CHUNK_LAUNCH(true); else DL_CHUNK_LAUNCH(false);
#undef DL_CHUNK_LAUNCH
            return hipGetLastError();
        }
    }
    // MV = value-log entries per lane per row = ceil(L / 8), rounded up to 2, 4 or 8
    if (P.L <= 16)
        log_launch<V, D, T, APPEND, 2>(P, rows, slot_idx, q, k, v, g, beta, o, ln);
    else if (P.L <= 32)
        log_launch<V, D, T, APPEND, 4>(P, rows, slot_idx, q, k, v, g, beta, o, ln);
    else
        log_launch<V, D, T, APPEND, 8>(P, rows, slot_idx, q, k, v, g, beta, o, ln);
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
    DL_DISPATCH_EAGER(P, eager_t, P, rows, slot_idx, q, k, v, g, beta, o, ln);
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
