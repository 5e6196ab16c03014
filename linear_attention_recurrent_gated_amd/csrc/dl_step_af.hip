// Additive-factor DeltaLog for the delta-rule operators (GDN, KDA and the
// gated form) on gfx950.
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
// The gated form (Gated DeltaNet-2 abstract, CARVE page, Explore similar
// work: a channel-wise erase gate e on the key channels and write gate w on
// the value channels) keeps the update rank one along k:
//   a_t = w_t * v_t - S_{t-1} (alpha_t e_t k_t),
// so only the read direction (e k for k in x and u_j) and the value term
// change; the log, readout and merge are the same as KDA's.
//
// Same workgroup shape as the compact-WY step (dl_step.hip): one workgroup of
// four waves per (row, head), S0 rows in registers (lane groups of 8, lane s
// holding the columns 4s + 32m + e).  Each logged key and decay is used by
// exactly one lane (the dot products above, eight channels per lane), so that
// lane loads it straight from the log into registers -- the first pass (two
// for head-wise decay) in flight with S0, the rest issued right after the
// first barrier -- and only the factors a_j, which every lane group of a row
// reads, are staged in LDS (direct-to-LDS loads).
#include "dl_common.hpp"

namespace dl {

// This wave's share of the staging of the factors of entries [0, n).  Lanes
// past the last element are masked off.
__device__ __forceinline__ void af_stage_factors(const Params &P, size_t pair, int n, int D,
                                                 unsigned char *smem, const AfPlan &ap, int lane,
                                                 int wave) {
    const int nf = n * (D / 4);
    const uint4 *as = reinterpret_cast<const uint4 *>(static_cast<const float *>(P.log_v) + pair * P.L * D);
    for (int b = 64 * wave; b < nf; b += 256) {
        const int idx = b + lane;
        if (idx < nf)
            load_to_lds<16>(as + idx, smem + ap.off_a + 16 * b);
    }
}

// Raw key-side data of one logged entry on one lane: eight channels of the
// key (input dtype) and, for per-key decays, of the cumulative log-decay.
struct KeyRaw {
    uint4 k0, k1;
    float4 l0, l1;
};

template <int V, int D, typename T>
__device__ __forceinline__ void load_key_raw(const Params &P, size_t e, int ch0, KeyRaw &rw) {
    const uint4 *kp = reinterpret_cast<const uint4 *>(static_cast<const T *>(P.log_k) + e * D + ch0);
    rw.k0 = kp[0];
    if constexpr (sizeof(T) == 4)
        rw.k1 = kp[1];
    if constexpr (V != GDN) {
        const float4 *lp = reinterpret_cast<const float4 *>(P.log_g + e * D + ch0);
        rw.l0 = lp[0];
        rw.l1 = lp[1];
    }
}

// Eight input elements kept as loaded (bf16 pairs or floats) until use.
struct Raw8 {
    uint4 a, b;
};

template <typename T>
__device__ __forceinline__ void load_raw8(const T *p, Raw8 &r) {
    r.a = reinterpret_cast<const uint4 *>(p)[0];
    if constexpr (sizeof(T) == 4)
        r.b = reinterpret_cast<const uint4 *>(p)[1];
}

template <typename T>
__device__ __forceinline__ void unpack8(const uint4 &a, const uint4 &b, float *x) {
    if constexpr (sizeof(T) == 4) {
        x[0] = __uint_as_float(a.x), x[1] = __uint_as_float(a.y);
        x[2] = __uint_as_float(a.z), x[3] = __uint_as_float(a.w);
        x[4] = __uint_as_float(b.x), x[5] = __uint_as_float(b.y);
        x[6] = __uint_as_float(b.z), x[7] = __uint_as_float(b.w);
    } else {
        x[0] = bf16_lo(a.x), x[1] = bf16_hi(a.x), x[2] = bf16_lo(a.y), x[3] = bf16_hi(a.y);
        x[4] = bf16_lo(a.z), x[5] = bf16_hi(a.z), x[6] = bf16_lo(a.w), x[7] = bf16_hi(a.w);
    }
}

// S0 <- S0 diag(E_c) + sum_{j < ct} a_j kd_j^T on this wave's rows, then the
// rows go back to the base; kd_j = k_j D(j, c) is staged in LDS.
template <int V, int D, bool NT>
__device__ __forceinline__ void af_merge_rows(const Params &P, size_t pair, int ct,
                                              const unsigned char *smem, const AfPlan &ap,
                                              float4 (&st)[Shape<D>::ITER][Shape<D>::NCH]) {
    using SH = Shape<D>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane >> 3, s = lane & 7;
    const float *sa = reinterpret_cast<const float *>(smem + ap.off_a);
    const float *skd = reinterpret_cast<const float *>(smem + ap.off_kd);
    float ec[SH::FPL];
    if constexpr (V == GDN) {
        const float e = fast_exp(reinterpret_cast<const float *>(smem + ap.off_s)[0]);
#pragma unroll
        for (int i = 0; i < SH::FPL; ++i)
            ec[i] = e;
    } else {
        const float *slc = reinterpret_cast<const float *>(smem + ap.off_lc);
#pragma unroll
        for (int m = 0; m < SH::NCH; ++m) {
            const float4 l = *reinterpret_cast<const float4 *>(slc + col_of(s, m, 0));
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
#pragma unroll
        for (int m = 0; m < SH::NCH; ++m)
            f4_to(kd + 4 * m, *reinterpret_cast<const float4 *>(skd + j * D + col_of(s, m, 0)));
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

// q8_kept_bits from the kept-channel indices the step has already loaded
// (lane s: index s and s + 8) instead of a second read of the list, whose
// wait would also wait for the base codes issued after it.
template <int D>
__device__ __forceinline__ uint32_t kept_bits_from_lanes(const int (&kc)[2], int M, int s, bool &ok) {
    constexpr int QW = Q8Row<D>::QW;
    uint32_t bits = 0u;
    ok = true;
    int prev = -1;
    for (int m = 0; m < M; ++m) {
        const int c = __builtin_amdgcn_readlane(m < 8 ? kc[0] : kc[1], m & 7);
        ok = ok && c > prev && c < D;
        prev = c;
        if (c >= 0 && c < D && c / QW == s)
            bits |= 1u << (c % QW);
    }
    return bits;
}

// This lane's codes of one INT8 base row (QW bytes), optionally nontemporal.
template <int D, bool NT>
__device__ __forceinline__ void load_codes(const int8_t *p, uint32_t *w) {
    if constexpr (Q8Row<D>::QW == 16) {
        uint4 u;
        if constexpr (NT) {
            typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
            u = make_uint4(t.x, t.y, t.z, t.w);
        } else {
            u = *reinterpret_cast<const uint4 *>(p);
        }
        w[0] = u.x, w[1] = u.y, w[2] = u.z, w[3] = u.w;
    } else {
        const uint2 u = *reinterpret_cast<const uint2 *>(p);
        w[0] = u.x, w[1] = u.y;
    }
}

template <int D, bool NT>
__device__ __forceinline__ void store_codes(int8_t *p, const uint32_t *w) {
    if constexpr (Q8Row<D>::QW == 16) {
        if constexpr (NT) {
            typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 t = {w[0], w[1], w[2], w[3]};
            __builtin_nontemporal_store(t, reinterpret_cast<u32x4 *>(p));
        } else {
            *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    } else {
        *reinterpret_cast<uint2 *>(p) = make_uint2(w[0], w[1]);
    }
}

// The INT8-base merge of this wave's rows: S' = S0 diag(E_c) + sum_{j < ct}
// a_j kd_j^T with S0 = code * scale (kept channels: their fp32 values), then
// each row re-quantised (q8_quantize_row) and written back with its scale
// and kept values.  Rows go RB at a time (RB QW fp32 registers per lane in
// flight); the codes are read again here (the step that merges in place has
// just read them, so they come from the cache) to keep them out of the
// registers the step's readout holds; kd_j is staged in LDS.
template <int V, int D, bool NT, int RB>
__device__ __forceinline__ void af_merge_rows_q8(const Params &P, size_t pair, int h, int ct,
                                                 const unsigned char *smem, const AfPlan &ap,
                                                 uint32_t kbits) {
    using SH = Shape<D>;
    constexpr int QW = Q8Row<D>::QW;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane >> 3, s = lane & 7;
    const float *sa = reinterpret_cast<const float *>(smem + ap.off_a);
    const float *skd = reinterpret_cast<const float *>(smem + ap.off_kd);
    float ec[QW];
    if constexpr (V == GDN) {
        const float e = fast_exp(reinterpret_cast<const float *>(smem + ap.off_s)[0]);
#pragma unroll
        for (int f = 0; f < QW; ++f)
            ec[f] = e;
    } else {
        const float *slc = reinterpret_cast<const float *>(smem + ap.off_lc);
#pragma unroll
        for (int f = 0; f < QW; ++f)
            ec[f] = fast_exp(slc[QW * s + f]);
    }
#pragma unroll
    for (int it0 = 0; it0 < SH::ITER; it0 += RB) {
        float x[RB][QW];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            const int row = wave * SH::RPW + (it0 + b) * 8 + grp;
            uint32_t cw[Q8Row<D>::NW];
            load_codes<D, false>(P.codes + (pair * D + row) * D + QW * s, cw);
            const float sc = P.scale[pair * D + row];
            q8_unpack<QW>(cw, x[b]);
#pragma unroll
            for (int f = 0; f < QW; ++f)
                x[b][f] *= sc;
            for (int m = 0; m < P.M; ++m) {
                const int c = P.kidx[h * P.M + m];
                if (c / QW == s) {
                    const float v = P.kept[(pair * D + row) * P.M + m];
#pragma unroll
                    for (int f = 0; f < QW; ++f)
                        x[b][f] = (f == c % QW) ? v : x[b][f];
                }
            }
#pragma unroll
            for (int f = 0; f < QW; ++f)
                x[b][f] *= ec[f];
        }
        for (int j = 0; j < ct; ++j) {
            float kd[QW];
#pragma unroll
            for (int f = 0; f < QW; f += 4)
                f4_to(kd + f, *reinterpret_cast<const float4 *>(skd + j * D + QW * s + f));
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                const float aj = sa[j * D + wave * SH::RPW + (it0 + b) * 8 + grp];
#pragma unroll
                for (int f = 0; f < QW; ++f)
                    x[b][f] += aj * kd[f];
            }
        }
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            const int row = wave * SH::RPW + (it0 + b) * 8 + grp;
            uint32_t w[QW / 4];
            const float scale = q8_quantize_row<QW>(x[b], kbits, w);
            store_codes<D, NT>(P.codes + (pair * D + row) * D + QW * s, w);
            if (s == 0)
                P.scale[pair * D + row] = scale;
            for (int m = 0; m < P.M; ++m) {
                const int c = P.kidx[h * P.M + m];
                if (c / QW == s) {
                    float v = 0.f;
#pragma unroll
                    for (int f = 0; f < QW; ++f)
                        v = (f == c % QW) ? x[b][f] : v;
                    P.kept[(pair * D + row) * P.M + m] = v;
                }
            }
        }
    }
}

// One workgroup per (row, head).  APPEND: the step (append + readout);
// otherwise a readout of base + log.  FUSE: the step that fills the log
// also merges it (fill back to 0).  With bf16 inputs and logs of up to 32
// entries the kernel is held to the registers of four waves per SIMD (four
// workgroups per CU), except where that spills on the hot path (32 entries
// with per-key decays and the merge in the step, or with gates), which runs
// three.  Over an INT8 base, whose codes take a quarter of the registers,
// logs of up to 16 entries run five (the build that merges in place keeps
// one value per lane in scratch across the barriers, and still gains 2-3%;
// the gated form measured slower at five).
template <int V, int D, typename T, bool APPEND, int MV, bool NT, bool FUSE, bool Q8>
__global__ void __launch_bounds__(256, (MV <= 4 && sizeof(T) == 2)
                                          ? (Q8 ? ((MV == 2 && V != GDN2) ? 5 : 4)
                                                : ((MV == 4 && (V == GDN2 || (V == KDA && FUSE))) ? 3 : 4))
                                          : 1)
af_step_kernel(Params P, const int *__restrict__ slot_idx, const T *__restrict__ q,
               const T *__restrict__ k, const T *__restrict__ v, const float *__restrict__ g,
               const float *__restrict__ beta, float *__restrict__ o) {
    static_assert(V == GDN || V == KDA || V == GDN2, "delta-rule variants only");
    using SH = Shape<D>;
    using KL = KeyLayout<D>;
    constexpr int G = KL::G, RP = KL::RP, PASS = 4 * RP;   // entries per pass of the four waves
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
    const AfPlan ap = af_plan(D, L, FUSE);
    float *sa = reinterpret_cast<float *>(smem + ap.off_a);
    float *skd = reinterpret_cast<float *>(smem + ap.off_kd);
    float *sr = reinterpret_cast<float *>(smem + ap.off_r);
    float *su = reinterpret_cast<float *>(smem + ap.off_u);
    float *sf = reinterpret_cast<float *>(smem + ap.off_f);
    float *ss = reinterpret_cast<float *>(smem + ap.off_s);
    float *slc = reinterpret_cast<float *>(smem + ap.off_lc);
    float *sqe = reinterpret_cast<float *>(smem + ap.off_qe);
    float *ske = reinterpret_cast<float *>(smem + ap.off_ke);

    // ---- loads that need nothing: fill, this wave's rows of S0, the inputs
    const int n = P.fill[pair];
    const int grp = lane >> 3, s = lane & 7;
    // Head-wise decay: E_n is one scalar, so S0 q and S0 k are formed while
    // S0 streams in (q and k in S0's column layout, loaded ahead of it) and
    // scaled by E_n after the barriers.  Only where the registers allow it
    // (bf16 inputs, logs of up to 16 entries).
    constexpr bool EARLY_DOT = !Q8 && V == GDN && sizeof(T) == 2 && MV <= 2;
    float4 qs[SH::NCH], ks[SH::NCH];
    if constexpr (EARLY_DOT) {
#pragma unroll
        for (int m = 0; m < SH::NCH; ++m) {
            qs[m] = Elem<T>::load4(q + io + col_of(s, m, 0));
            if constexpr (APPEND)
                ks[m] = Elem<T>::load4(k + io + col_of(s, m, 0));
        }
    }
    // the base rows: fp32 (8 lanes per row, lane s holding the columns
    // 4 s + 32 m + e), or INT8 codes (lane s holding the QW columns from
    // QW s), their row scales and, on lanes s and s + 8, the kept channels
    // m = s, s + 8 with their column indices
    constexpr int QW = Q8Row<D>::QW;
    float4 st[Q8 ? 1 : SH::ITER][SH::NCH];
    uint32_t cw[SH::ITER][Q8Row<D>::NW];
    float sc[SH::ITER], kv[SH::ITER][2];
    int kc[2] = {0, 0};
    if constexpr (Q8) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            // read unconditionally (index 0 past M; with M = 0 that is the
            // first word after the indices, the log's, which an INT8 state
            // always has), so that no wait for it lands before the codes
            const int m = s + 8 * i;
            const int raw = P.kidx[h * P.M + (m < P.M ? m : 0)];
            kc[i] = m < P.M ? raw : 0;
        }
#pragma unroll
        for (int it = 0; it < SH::ITER; ++it) {
            const int row = wave * SH::RPW + it * 8 + grp;
            load_codes<D, NT>(P.codes + (pair * D + row) * D + QW * s, cw[it]);
            sc[it] = P.scale[pair * D + row];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int m = s + 8 * i;
                // unconditional, as the indices above (index 0 past M)
                const float raw = P.kept[(pair * D + row) * P.M + (m < P.M ? m : 0)];
                kv[it][i] = m < P.M ? raw : 0.f;
            }
        }
    } else {
        const float *Sp = P.base + pair * D * D;
#pragma unroll
        for (int it = 0; it < SH::ITER; ++it) {
            const int row = wave * SH::RPW + it * 8 + grp;
#pragma unroll
            for (int m = 0; m < SH::NCH; ++m)
                st[it][m] = load_state4<NT>(Sp + (size_t)row * D + col_of(s, m, 0));
        }
    }
    const int cg = lane % G, ro = lane / G, ch0 = 8 * cg;
    Raw8 qr = {}, kr = {};               // q and k on this lane's channels, as loaded
    load_raw8<T>(q + io + ch0, qr);
    if constexpr (APPEND)
        load_raw8<T>(k + io + ch0, kr);
    __builtin_amdgcn_sched_barrier(0);
    if (APPEND ? (n >= L || n < 0) : (n > L || n < 0)) {
        reject_row(P, orow, D, DL_FLAG_LOG_FULL);
        return;
    }
    uint32_t kbits = 0u;
    if constexpr (Q8) {
        bool ok;
        kbits = kept_bits_from_lanes<D>(kc, P.M, s, ok);
        if (!ok) {
            reject_row(P, orow, D, DL_FLAG_BAD_KEPT);
            return;
        }
    }

    // ---- loads that need n: beta, this lane's logged keys (and decays) of
    //      the first pass(es), the staging of the factors and of the new
    //      value row, and (wave 0) Lam and the decayed q and k
    const float b_in = (APPEND && V != GDN2) ? beta[pr] : 0.f;
    const float *gate = beta + (size_t)pr * 2 * D;   // gated: erase gate, then write gate
    if constexpr (APPEND) {
        constexpr int CPV = D * (int)sizeof(T) / 16;
        if (wave == 0 && lane < CPV)
            load_to_lds<16>(reinterpret_cast<const uint4 *>(v + io) + lane, smem + ap.off_v);
        if constexpr (V == GDN2) {
            if (wave == 1 && lane < D / 4)
                load_to_lds<16>(reinterpret_cast<const uint4 *>(gate + D) + lane, smem + ap.off_w);
        }
    }
    const int ct = APPEND ? n + 1 : n;   // entries the readout sees
    const int npass = (ct + PASS - 1) / PASS;
    // logged entry j of pass p on this lane (clamped to the last logged one)
    // (slot 0 of an empty log: a valid address whose data no lane uses)
    auto entry_of = [&](int p) {
        const int j = PASS * p + RP * wave + ro;
        return e0 + (j < n ? j : (n > 0 ? n - 1 : 0));
    };
    // Every pass gets its own registers (NP passes cover MV * 8 >= L
    // entries).  Before the barrier: two passes of keys (head-wise decay) or
    // one pass of keys and decays (per-key decays, twice the data); the rest
    // right after it, all in flight together.
    constexpr int NP = (8 * MV + PASS - 1) / PASS;
    constexpr int EARLY = (V == GDN && NP > 1) ? 2 : 1;
    // Over an INT8 base every pass is loaded whatever the fill (passes past
    // the log read its last entry again, a cache hit, and are never used): a
    // load under a condition leaves its result to be merged with the other
    // branch's value, and the compiler waits for every load in flight (the
    // base codes included) before that copy, which holds back the factor
    // staging (C4 INT8 step 106 -> 93 us with the kept-channel reads below).
    // With an fp32 base the same change measured no faster and slower for
    // per-key decays at 64 entries, so there the passes stay conditional.
    KeyRaw pre[NP] = {};
    if constexpr (Q8) {
#pragma unroll
        for (int p = 0; p < EARLY; ++p)
            load_key_raw<V, D, T>(P, entry_of(p), ch0, pre[p]);
        af_stage_factors(P, pair, n, D, smem, ap, lane, wave);
    } else if (n > 0) {
#pragma unroll
        for (int p = 0; p < EARLY; ++p)
            if (p < npass)
                load_key_raw<V, D, T>(P, entry_of(p), ch0, pre[p]);
        af_stage_factors(P, pair, n, D, smem, ap, lane, wave);
    }
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
            }
            if (ro == 0)
                store8<float>(slc + ch0, lc);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                en[i] = fast_exp(lc[i]);
        }
        if (!EARLY_DOT && ro == 0) {
            float t[8];
            unpack8<T>(qr.a, qr.b, t);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                t[i] *= en[i];
            store8<float>(sqe + ch0, t);
            if constexpr (APPEND) {
                unpack8<T>(kr.a, kr.b, t);
                if constexpr (V == GDN2) {
                    // the read direction of the gated form: e * k
                    float e[8];
                    load8<float>(gate + ch0, e);
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        t[i] *= e[i];
                    store8<float>(reinterpret_cast<float *>(smem + ap.off_ek) + ch0, t);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    t[i] *= en[i];
                store8<float>(ske + ch0, t);
            }
        }
    }
    float p0[SH::ITER], x0[SH::ITER];   // S0 q and S0 k per row (head-wise decay)
    if constexpr (EARLY_DOT) {
#pragma unroll
        for (int it = 0; it < SH::ITER; ++it) {
            float ap = 0.f, ax = 0.f;
#pragma unroll
            for (int m = 0; m < SH::NCH; ++m) {
                ap += st[it][m].x * qs[m].x + st[it][m].y * qs[m].y + st[it][m].z * qs[m].z +
                      st[it][m].w * qs[m].w;
                if constexpr (APPEND)
                    ax += st[it][m].x * ks[m].x + st[it][m].y * ks[m].y + st[it][m].z * ks[m].z +
                          st[it][m].w * ks[m].w;
            }
            p0[it] = ap;
            x0[it] = ax;
        }
    }
    wait_vm_all();      // this wave's loads and staging have landed
    __syncthreads();    // 1: staged factors, Lam_c, per-entry factors, E q, E k

    const bool merging = FUSE && APPEND && n == L - 1;
    // This lane's first channel, recomputed from the thread index at each use
    // from here on (an empty asm hides it from common-subexpression
    // elimination), so that the compiler neither keeps nor spills it.
    auto chan = [] {
        int t = threadIdx.x;
        asm volatile("" : "+v"(t));
        return 8 * ((t & 63) % G);
    };
    const int chl = chan();
    float ekv[8];                        // gated: this lane's channels of e * k
    if constexpr (APPEND && V == GDN2)
        load8<float>(reinterpret_cast<const float *>(smem + ap.off_ek) + chl, ekv);
    if constexpr (Q8) {
#pragma unroll
        for (int p = EARLY; p < NP; ++p)
            load_key_raw<V, D, T>(P, entry_of(p), chl, pre[p]);
    } else if (n > 0) {
#pragma unroll
        for (int p = EARLY; p < NP; ++p)
            if (p < npass)
                load_key_raw<V, D, T>(P, entry_of(p), chl, pre[p]);
    }
    float lc[8];
    if constexpr (V != GDN)
        load8<float>(slc + chl, lc);

    // ---- r_j = (k_j D(j, c)) . q and u_j = (k_j D(j, c)) . k for this lane's
    //      entry of each pass (the new entry n is this step's k, D = 1); a
    //      merging step also keeps k_j D(j, c) for the merge
    auto process = [&](int p, const KeyRaw &rw) {
        const int j = PASS * p + RP * wave + ro;
        float kd[8], qv[8], kn[8];
        unpack8<T>(rw.k0, rw.k1, kd);
        unpack8<T>(qr.a, qr.b, qv);
        if constexpr (APPEND)
            unpack8<T>(kr.a, kr.b, kn);
        if constexpr (V != GDN) {
            const float lr[8] = {rw.l0.x, rw.l0.y, rw.l0.z, rw.l0.w, rw.l1.x, rw.l1.y, rw.l1.z, rw.l1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
                kd[i] *= fast_exp(lc[i] - lr[i]);
        }
        if (APPEND && j == n)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                kd[i] = kn[i];
        float ar = 0.f, au = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            ar += kd[i] * qv[i];
            if constexpr (APPEND)
                au += kd[i] * ((V == GDN2) ? ekv[i] : kn[i]);
        }
        ar = group_sum<G>(ar);
        if constexpr (APPEND)
            au = group_sum<G>(au);
        const float f = (V == GDN) ? sf[j < ct ? j : ct - 1] : 1.f;
        if (cg == 0 && j < ct) {
            sr[j] = f * ar;
            if constexpr (APPEND)
                su[j] = f * au;
        }
        if (FUSE && merging && j < ct) {
            if constexpr (V == GDN)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    kd[i] *= f;
            store8<float>(skd + j * D + chan(), kd);
        }
    };
#pragma unroll
    for (int p = 0; p < NP; ++p)
        if (p < npass)
            process(p, pre[p]);
    __syncthreads();    // 2: r and u of every entry (and the merge's decayed keys)

    // ---- per row: x = S0 (E k) + sum u_j a_j, a_n = beta (v - x),
    //      o = S0 (E q) + sum r_j a_j + r_n a_n
    float qt[SH::FPL], kt[SH::FPL];
    float qk[2] = {0.f, 0.f}, kk[2] = {0.f, 0.f};   // INT8 base: E q, E k at the kept channels
    if constexpr (Q8) {
        static_assert(QW == SH::FPL, "the INT8 lane layout holds as many columns as the fp32 one");
#pragma unroll
        for (int f = 0; f < QW; f += 4) {
            f4_to(qt + f, *reinterpret_cast<const float4 *>(sqe + QW * s + f));
            if constexpr (APPEND)
                f4_to(kt + f, *reinterpret_cast<const float4 *>(ske + QW * s + f));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            qk[i] = s + 8 * i < P.M ? sqe[kc[i]] : 0.f;
            if constexpr (APPEND)
                kk[i] = s + 8 * i < P.M ? ske[kc[i]] : 0.f;
        }
    } else if constexpr (!EARLY_DOT) {
#pragma unroll
        for (int m = 0; m < SH::NCH; ++m) {
            f4_to(qt + 4 * m, *reinterpret_cast<const float4 *>(sqe + col_of(s, m, 0)));
            if constexpr (APPEND)
                f4_to(kt + 4 * m, *reinterpret_cast<const float4 *>(ske + col_of(s, m, 0)));
        }
    }
    const float e_n = EARLY_DOT ? fast_exp(ss[0]) : 0.f;
    float cr[MV], cu[MV];
#pragma unroll
    for (int mm = 0; mm < MV; ++mm) {
        const int j = s + 8 * mm;
        const int jc = j < n ? j : 0;
        cr[mm] = j < n ? sr[jc] : 0.f;
        cu[mm] = (APPEND && j < n) ? su[jc] : 0.f;
    }
    // r_n = k . q (D(n, n) = 1), the same for the whole workgroup: kept in a
    // scalar register
    const float rn = APPEND ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sr[n]))) : 0.f;
    float *alog = static_cast<float *>(P.log_v) + (e0 + n) * D;
#pragma unroll
    for (int it = 0; it < SH::ITER; ++it) {
        const int row = wave * SH::RPW + it * 8 + grp;
        float ao = 0.f, ax = 0.f;
        if constexpr (Q8) {
            float xc[QW];
            q8_unpack<QW>(cw[it], xc);
#pragma unroll
            for (int f = 0; f < QW; ++f) {
                ao += xc[f] * qt[f];
                if constexpr (APPEND)
                    ax += xc[f] * kt[f];
            }
            ao *= sc[it];
            ax *= sc[it];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                ao += kv[it][i] * qk[i];
                if constexpr (APPEND)
                    ax += kv[it][i] * kk[i];
            }
        } else if constexpr (EARLY_DOT) {
            ao = e_n * p0[it];
            ax = e_n * x0[it];
        } else {
#pragma unroll
            for (int m = 0; m < SH::NCH; ++m) {
                ao += st[it][m].x * qt[4 * m] + st[it][m].y * qt[4 * m + 1] +
                      st[it][m].z * qt[4 * m + 2] + st[it][m].w * qt[4 * m + 3];
                if constexpr (APPEND)
                    ax += st[it][m].x * kt[4 * m] + st[it][m].y * kt[4 * m + 1] +
                          st[it][m].z * kt[4 * m + 2] + st[it][m].w * kt[4 * m + 3];
            }
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
            const float vr = Elem<T>::load1(reinterpret_cast<const T *>(smem + ap.off_v) + row);
            const float an = (V == GDN2)
                                 ? reinterpret_cast<const float *>(smem + ap.off_w)[row] * vr - ax
                                 : b_in * (vr - ax);
            ao += rn * an;
            if (s == 1 && !merging)
                alog[row] = an;
            if (FUSE && merging && s == 0)
                sa[n * D + row] = an;
        }
        if (s == 0)
            orow[row] = ao;
    }
    if constexpr (APPEND) {
        // the rest of entry n: the key (bit copy) and Lam_n (not for the entry
        // that fills the log when it merges in place: it goes straight into
        // the merged base and the emptied log keeps no copy of it)
        if (wave == 0 && !merging) {
            if (ro == 0) {
                uint4 *dst = reinterpret_cast<uint4 *>(static_cast<T *>(P.log_k) + (e0 + n) * D + chan());
                dst[0] = kr.a;
                if constexpr (sizeof(T) == 4)
                    dst[1] = kr.b;
            }
            if constexpr (V == GDN) {
                if (lane == 0)
                    P.log_g[e0 + n] = ss[0];
            } else {
                if (lane < D / 4)
                    reinterpret_cast<float4 *>(P.log_g + (e0 + n) * D)[lane] =
                        reinterpret_cast<const float4 *>(slc)[lane];
            }
        }
        if constexpr (FUSE) {
            if (merging) {
                wave_lds_sync();   // this wave's rows of a_n are in LDS
                if constexpr (Q8)
                    af_merge_rows_q8<V, D, NT, 1>(P, pair, h, ct, smem, ap, kbits);
                else
                    af_merge_rows<V, D, NT>(P, pair, ct, smem, ap, st);
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
template <int V, int D, typename T, bool NT, bool Q8>
__global__ void __launch_bounds__(256) af_merge_kernel(Params P, const int *__restrict__ slot_idx,
                                                       int mode) {
    static_assert(V == GDN || V == KDA || V == GDN2, "delta-rule variants only");
    using SH = Shape<D>;
    extern __shared__ __align__(16) unsigned char smem[];
    size_t pair;
    int n;
    if (!resolve_merge_pair(P, slot_idx, mode, pair, n))
        return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = lane >> 3, s = lane & 7;
    const int h = (int)(pair % (size_t)P.heads);
    const AfPlan ap = af_plan(D, P.L, true);
    const size_t e0 = pair * P.L;
    float4 st[Q8 ? 1 : SH::ITER][SH::NCH];
    uint32_t kbits = 0u;
    if constexpr (Q8) {
        bool ok;
        kbits = q8_kept_bits<D>(P, h, s, ok);
        if (!ok) {
            reject_row(P, nullptr, D, DL_FLAG_BAD_KEPT);
            return;
        }
    } else {
        const float *Sp = P.base + pair * D * D;
#pragma unroll
        for (int it = 0; it < SH::ITER; ++it) {
            const int row = wave * SH::RPW + it * 8 + grp;
#pragma unroll
            for (int m = 0; m < SH::NCH; ++m)
                st[it][m] = load_state4<NT>(Sp + (size_t)row * D + col_of(s, m, 0));
        }
    }
    af_stage_factors(P, pair, n, D, smem, ap, lane, wave);
    float *sf = reinterpret_cast<float *>(smem + ap.off_f);
    float *slc = reinterpret_cast<float *>(smem + ap.off_lc);
    if (wave == 0) {
        if constexpr (V == GDN) {
            const int jl = lane < n ? lane : n - 1;
            const float lam_j = P.log_g[e0 + jl];
            const float lam_c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam_j), n - 1));
            if (lane < n)
                sf[lane] = fast_exp(lam_c - lam_j);
            if (lane == 0)
                reinterpret_cast<float *>(smem + ap.off_s)[0] = lam_c;
        } else {
            if (lane < D / 4)
                reinterpret_cast<float4 *>(slc)[lane] =
                    reinterpret_cast<const float4 *>(P.log_g + (e0 + n - 1) * D)[lane];
        }
    }
    wait_vm_all();
    __syncthreads();
    // decayed keys k_j D(j, c), eight channels per thread and step
    {
        constexpr int CPR = D / 8;
        float *skd = reinterpret_cast<float *>(smem + ap.off_kd);
        for (int idx = tid; idx < n * CPR; idx += 256) {
            const int j = idx / CPR, c = 8 * (idx - j * CPR);
            float kr[8];
            load8<T>(static_cast<const T *>(P.log_k) + (e0 + j) * D + c, kr);
            if constexpr (V == GDN) {
                const float f = sf[j];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    kr[i] *= f;
            } else {
                float lr[8], lcv[8];
                load8<float>(P.log_g + (e0 + j) * D + c, lr);
                load8<float>(slc + c, lcv);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    kr[i] *= fast_exp(lcv[i] - lr[i]);
            }
            store8<float>(skd + j * D + c, kr);
        }
    }
    __syncthreads();
    if constexpr (Q8)
        af_merge_rows_q8<V, D, NT, 2>(P, pair, h, n, smem, ap, kbits);
    else
        af_merge_rows<V, D, NT>(P, pair, n, smem, ap, st);
    if (tid == 0)
        P.fill[pair] = 0;
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
#define DL_DISPATCH_AF(P, FN, ...)                                                       \
    do {                                                                                 \
        const bool bf = (P).dtype == DL_BF16;                                            \
        const int var = (P).variant;                                                     \
        if ((P).D == 128) {                                                              \
            if (bf) {                                                                    \
                if (var == DL_GDN) return FN<GDN, 128, uint16_t>(__VA_ARGS__);           \
                if (var == DL_KDA) return FN<KDA, 128, uint16_t>(__VA_ARGS__);           \
                return FN<GDN2, 128, uint16_t>(__VA_ARGS__);                             \
            }                                                                            \
            if (var == DL_GDN) return FN<GDN, 128, float>(__VA_ARGS__);                  \
            if (var == DL_KDA) return FN<KDA, 128, float>(__VA_ARGS__);                  \
            return FN<GDN2, 128, float>(__VA_ARGS__);                                    \
        }                                                                                \
        if (bf) {                                                                        \
            if (var == DL_GDN) return FN<GDN, 64, uint16_t>(__VA_ARGS__);                \
            if (var == DL_KDA) return FN<KDA, 64, uint16_t>(__VA_ARGS__);                \
            return FN<GDN2, 64, uint16_t>(__VA_ARGS__);                                  \
        }                                                                                \
        if (var == DL_GDN) return FN<GDN, 64, float>(__VA_ARGS__);                       \
        if (var == DL_KDA) return FN<KDA, 64, float>(__VA_ARGS__);                       \
        return FN<GDN2, 64, float>(__VA_ARGS__);                                         \
    } while (0)

template <int V, int D, typename T, bool APPEND, int MV>
static void af_launch(const Params &P, int rows, const int *slot_idx, const void *q,
                      const void *k, const void *v, const float *g, const float *beta, float *o,
                      const Launch &ln) {
    const bool fuse = APPEND && P.fuse;
    const AfPlan ap = af_plan(D, P.L, fuse);
    const dim3 grid(rows * P.heads), block(256);
#define DL_AF_LAUNCH(NTV, FV, QV)                                                                      \
    hipExtLaunchKernelGGL((af_step_kernel<V, D, T, APPEND, MV, NTV, FV, QV>), grid, block, ap.bytes,   \
                          ln.stream, ln.start, ln.stop, 0, P, slot_idx, static_cast<const T *>(q),     \
                          static_cast<const T *>(k), static_cast<const T *>(v), g, beta, o)
#define DL_AF_LAUNCH_Q(NTV, FV)                                                                        \
    do {                                                                                               \
        if (P.q8) DL_AF_LAUNCH(NTV, FV, true); else DL_AF_LAUNCH(NTV, FV, false);                      \
    } while (0)
    if constexpr (APPEND) {
        if (P.stream) {
            if (fuse) DL_AF_LAUNCH_Q(true, true); else DL_AF_LAUNCH_Q(true, false);
        } else {
            if (fuse) DL_AF_LAUNCH_Q(false, true); else DL_AF_LAUNCH_Q(false, false);
        }
    } else {
        if (P.stream) DL_AF_LAUNCH_Q(true, false); else DL_AF_LAUNCH_Q(false, false);
    }
#undef DL_AF_LAUNCH_Q
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
    const AfPlan ap = af_plan(D, P.L, true);
#define DL_AFM_LAUNCH(NTV, QV)                                                                         \
    hipExtLaunchKernelGGL((af_merge_kernel<V, D, T, NTV, QV>), dim3(rows * P.heads), dim3(256), ap.bytes, \
                          ln.stream, ln.start, ln.stop, 0, P, slot_idx, mode)
    if (P.stream) {
        if (P.q8) DL_AFM_LAUNCH(true, true); else DL_AFM_LAUNCH(true, false);
    } else {
        if (P.q8) DL_AFM_LAUNCH(false, true); else DL_AFM_LAUNCH(false, false);
    }
#undef DL_AFM_LAUNCH
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
