// Merge kernels for gfx950: materialise base + log into a new base and empty
// the log (the Merge Phase of the DeltaLog page, "DeltaLog: Deferred
// Materialization of Recurrent States for Linear Attention Decoding",
// Technical Summary, Core Mechanism).
//
// merge_wy_kernel -- the logged transforms folded in WY/UT form, the block
// form the CARVE page (abstract: WY-form triangular chunk solver) and Gated
// DeltaNet-2 (chunkwise WY algorithm) use.  The log step already keeps the
// triangular factor of that form, R = (I + N)^{-1}, one column per appended
// entry, so the merge only contracts: with u_j = beta_j (v_j - S_{j-1}
// diag(alpha_j) k_j) the recurrence unrolls to S_c = S_0 diag(E_c) + sum_j
// u_j (k_j D(j, c))^T, and the u_j are the columns of (V^T - S_0 Kt^T) R
// diag(beta) -- see the kernel below.  With decays of at most 1 (g <= 0) every
// decay factor is exp of a non-positive difference of the cumulative
// log-decays, so nothing overflows.
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
// With n logged entries, E_j = exp(Lam_j), D(j, c) = exp(Lam_c - Lam_j) and
// the key-side factor R = (I + N)^{-1} that the log step keeps (packed
// columns, one appended per entry), the merged base is
//   S' = S0 diag(E_c) + Z Y,   Z = V^T - S0 Kt^T,   Kt_j = E_j k_j,
//   Y = R Q,                   Q_i = beta_i k_i D(i, c)
// (additive variant: R = I, beta = 1, Z = V^T) -- the readout formula of the
// log step written for every query at once, so the merge needs no Gram
// matrix and no triangular solve: R is read back from the log.  All three
// products run on v_mfma_f32_16x16x4_f32 in 16-entry chunks:
//   phase A  z_c = V_c^T - S0 Kt_c^T for every chunk, with the original base;
//   phase B  S0 <- S0 diag(E_c), then per chunk Y_c = R_c Q (each wave a
//            share of its column blocks, through LDS) and S0 += z_c Y_c.
// The base stays in registers in the MFMA operand layout (lane l: row l % 16
// of a 16-row value tile, column sub-block l / 16): the B operand of W^T =
// Kt S0^T and, read as 16 x 16 tiles of S0^T, the accumulators of the
// update -- no transposes, no reloads.
//
// A pair's D value rows may be split over NS = D / (16 NW NIT) workgroups
// (the longest logs, whose chunk tiles do not fit beside a whole base in
// registers); every workgroup of a pair stages the pair's key side and builds
// Y for itself (cheap next to the base traffic), and they are dispatched 8
// blocks apart -- on one XCD, whose L2 then serves the repeated key reads.  The log's keys, decays and R go to LDS
// with direct-to-LDS loads issued before the base loads, so the key side is
// ready while the base is still in flight.
//
// The fill count is read and reset through tickets in its upper half: each
// workgroup of a pair adds 1 << 16 and reads the count in the lower half; the
// one that takes the last ticket writes the count back (0 when the pair
// merges), so no workgroup of a pair can read a count another one reset.
// ---------------------------------------------------------------------------
template <int V, int D, typename T, int NW, int NIT, int NE>
struct WyShape {
    static constexpr int NTH = 64 * NW;           // threads per workgroup
    static constexpr int ROWS = 16 * NW * NIT;    // value rows per workgroup
    static constexpr int NS = D / ROWS;           // workgroups per pair
    static constexpr int NM = D / 16;             // 16-column blocks
    static constexpr int KS = D + 4;              // padded LDS row stride of Y (floats)
    static constexpr bool PK = V != GDN;          // per-key decays
    static_assert(NS >= 1 && NS * ROWS == D, "the rows of a pair split evenly");
    static_assert(NM % NW == 0, "Y's column blocks split evenly over the waves");
    static_assert(NE == 1 || NE == 2 || NE == 4, "chunks of 16 entries: L <= 16 NE");
};

// LDS carve-up of the WY merge for logs of up to L entries.
struct WyPlan {
    int off_k;     // keys, [L][D] in the input dtype
    int off_lam;   // per-key decays: Lam, [L][D] fp32
    int off_t;     // packed columns of R
    int off_f;     // per entry: beta_j (head-wise decay: times D(j, c)), 64 floats
    int off_e;     // per entry (head-wise decay): E_j, 64 floats
    int off_ec;    // E_c per key channel, D floats
    int off_y;     // one chunk of Y: 16 rows of D + 4 floats
    int off_n;     // the fill count read by the workgroup
    int bytes;
};

__host__ __device__ inline WyPlan wy_plan(int variant, int D, int esize, int L) {
    WyPlan p;
    p.off_k = 0;
    p.off_lam = round_up(L * D * esize, 256);
    p.off_t = p.off_lam + (variant == DL_GDN ? 0 : round_up(L * D * 4, 256));
    p.off_f = p.off_t + round_up(packed_t_len(variant, L) * 4, 256);
    p.off_e = p.off_f + 256;
    p.off_ec = p.off_e + 256;
    p.off_y = p.off_ec + D * 4;
    p.off_n = p.off_y + 16 * (D + 4) * 4;
    p.bytes = p.off_n + 16;
    return p;
}

template <int V, int D, typename T, bool NTS, int NW, int NIT, int NE>
__global__ void __launch_bounds__(64 * NW, (NIT == 2 ? 4 : 1))
merge_wy_kernel(Params P, const int *__restrict__ slot_idx, int mode, int npairs) {
    using WS = WyShape<V, D, T, NW, NIT, NE>;
    constexpr int NM = WS::NM, KS = WS::KS, NTH = WS::NTH;
    constexpr bool PK = WS::PK, DELTA = V != RWKV6;
    extern __shared__ __align__(16) unsigned char smem[];
    const int L = P.L;
    const WyPlan wp = wy_plan(V, D, (int)sizeof(T), L);
    const T *sk = reinterpret_cast<const T *>(smem + wp.off_k);
    const float *slam = reinterpret_cast<const float *>(smem + wp.off_lam);
    const float *sT = reinterpret_cast<const float *>(smem + wp.off_t);
    float *sf = reinterpret_cast<float *>(smem + wp.off_f);
    float *se = reinterpret_cast<float *>(smem + wp.off_e);
    float *sec = reinterpret_cast<float *>(smem + wp.off_ec);
    float *sy = reinterpret_cast<float *>(smem + wp.off_y);
    int *sn = reinterpret_cast<int *>(smem + wp.off_n);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, kg = lane >> 4;
    // block -> (pair, split): the NS workgroups of a pair are 8 blocks apart
    const int xcd = blockIdx.x & 7, qb = blockIdx.x >> 3;
    const int split = qb % WS::NS;
    const int pr = (qb / WS::NS) * 8 + xcd;
    if (pr >= npairs)
        return;
    const int H = P.heads;
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
        sn[0] = go ? n0 : 0;
    }
    __syncthreads();
    const int n = sn[0];
    if (n == 0)
        return;
    const int nch = (n + 15) >> 4;       // chunks of 16 entries
    const size_t e0 = pair * L;

    // ---- loads, in the order they are needed: per-entry scalars (wave 0),
    //      the staging of keys, decays and R, the base rows, chunk 0's values
    float b_j = 1.f, lam_j = 0.f;
    if (wave == 0 && lane < n) {
        if constexpr (DELTA)
            b_j = P.log_beta[e0 + lane];
        if constexpr (!PK)
            lam_j = P.log_g[e0 + lane];
    }
    {
        const int nk = n * D * (int)sizeof(T) / 16;
        const uint4 *ks = reinterpret_cast<const uint4 *>(static_cast<const T *>(P.log_k) + e0 * D);
        for (int b = 64 * wave; b < nk; b += NTH)
            if (b + lane < nk)
                load_to_lds<16>(ks + b + lane, smem + wp.off_k + 16 * b);
        if constexpr (PK) {
            const int nl = n * D / 4;
            const float4 *ls = reinterpret_cast<const float4 *>(P.log_g + e0 * D);
            for (int b = 64 * wave; b < nl; b += NTH)
                if (b + lane < nl)
                    load_to_lds<16>(ls + b + lane, smem + wp.off_lam + 16 * b);
        }
        if constexpr (DELTA) {
            const int nt = n * (n - 1) / 2;
            const float *ts = P.log_t + pair * packed_t_len(V, L);
            for (int b = 64 * wave; b < nt; b += NTH)
                if (b + lane < nt)
                    load_to_lds<4>(ts + b + lane, smem + wp.off_t + 4 * b);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
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
    // values of chunk c on this lane: V[entry 16 c + 4 kg + rr][row], loaded
    // as they are (the last entry again past n) and masked where used, so
    // that nothing waits for them before then
    const T *Vl = static_cast<const T *>(P.log_v) + e0 * D;
    auto load_values = [&](int c, float (&vr)[NIT][4]) {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int row = row0 + 16 * (wave * NIT + it) + li;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int j = 16 * c + 4 * kg + rr;
                vr[it][rr] = Elem<T>::load1(Vl + (size_t)(j < n ? j : n - 1) * D + row);
            }
        }
    };
    float vv[NIT][4];
    load_values(0, vv);
    __builtin_amdgcn_sched_barrier(0);
    // the staging has landed once at most the base and value loads are outstanding
    barrier_after_staging<NIT * (NM + 4)>();    // staged keys, decays and R

    // ---- per-entry factors and E_c
    if (wave == 0) {
        if constexpr (!PK) {
            const float lam_c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam_j), n - 1));
            if (lane < n) {
                sf[lane] = b_j * fast_exp(lam_c - lam_j);
                se[lane] = fast_exp(lam_j);
            }
            const float ec = fast_exp(lam_c);
            for (int c = lane; c < D; c += 64)
                sec[c] = ec;
        } else {
            if (lane < n)
                sf[lane] = b_j;
            for (int c = lane; c < D; c += 64)
                sec[c] = fast_exp(slam[(n - 1) * D + c]);
        }
    }
    __syncthreads();

    // ---- phase A: z_c = V_c^T - S0 Kt_c^T (MFMA, accumulator initialised
    //      with the values): z[c][it][rr] = Z[row][entry 16 c + 4 kg + rr]
    floatx4 z[NE][NIT];
#pragma unroll
    for (int c = 0; c < NE; ++c) {
        if (c >= nch)
            break;
        // the next chunk's values, in flight (not under a condition: past
        // the last chunk they read the last entry again and go unused; a load
        // under one is waited for before its register is merged)
        float vn[NIT][4];
        load_values(c + 1, vn);
#pragma unroll
        for (int it = 0; it < NIT; ++it)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                z[c][it][rr] = 16 * c + 4 * kg + rr < n ? vv[it][rr] : 0.f;
        if constexpr (DELTA) {
            const int j = 16 * c + li;            // this lane's entry of the A operand
            const bool live = j < n;
            const int jc = live ? j : n - 1;
            const float ej = PK ? 1.f : (live ? se[jc] : 0.f);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                if (m % 2 == 0)
                    __builtin_amdgcn_sched_barrier(0);   // bound the LDS reads in flight
                const int col = 4 * kg + 16 * m;
                float4 kt = lds_load4<T>(reinterpret_cast<const unsigned char *>(sk), jc * D + col);
                if constexpr (PK) {
                    const float4 l4 = *reinterpret_cast<const float4 *>(slam + jc * D + col);
                    kt.x *= fast_exp(l4.x), kt.y *= fast_exp(l4.y);
                    kt.z *= fast_exp(l4.z), kt.w *= fast_exp(l4.w);
                }
                const float s = live ? -ej : 0.f;   // -Kt (head-wise: E_j; per-key: folded above)
                const float f = PK ? (live ? -1.f : 0.f) : s;
                const float a0 = f * kt.x, a1 = f * kt.y, a2 = f * kt.z, a3 = f * kt.w;
#pragma unroll
                for (int it = 0; it < NIT; ++it) {
                    z[c][it] = mfma16x16x4(a0, st[it][m][0], z[c][it]);
                    z[c][it] = mfma16x16x4(a1, st[it][m][1], z[c][it]);
                    z[c][it] = mfma16x16x4(a2, st[it][m][2], z[c][it]);
                    z[c][it] = mfma16x16x4(a3, st[it][m][3], z[c][it]);
                }
            }
        }
#pragma unroll
        for (int it = 0; it < NIT; ++it)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                vv[it][rr] = vn[it][rr];
    }

    // ---- phase B: S0 diag(E_c), then S0 += z_c Y_c chunk by chunk
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const float4 el = *reinterpret_cast<const float4 *>(sec + 4 * kg + 16 * m);
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            st[it][m][0] *= el.x;
            st[it][m][1] *= el.y;
            st[it][m][2] *= el.z;
            st[it][m][3] *= el.w;
        }
    }
    // Q[i][ch] = f_i k_i[ch] (per-key: times D(i, c) on the channel); 0 past n
    auto qval = [&](int i, int ch) {
        const int ic = i < n ? i : n - 1;
        float q = Elem<T>::load1(sk + ic * D + ch) * sf[ic];
        if constexpr (PK)
            q *= fast_exp(slam[(n - 1) * D + ch] - slam[ic * D + ch]);
        return i < n ? q : 0.f;
    };
#pragma unroll
    for (int c = 0; c < NE; ++c) {
        if (c >= nch)
            break;
        const int j0 = 16 * c;
        if (c > 0)
            __syncthreads();    // the previous chunk's Y is consumed
        // Y_c = R_c Q on this wave's column blocks: Y[j0 + 4 kg + rr][16 m + li]
#pragma unroll
        for (int mb = 0; mb < NM / NW; ++mb) {
            const int m = wave * (NM / NW) + mb;
            const int ch = 16 * m + li;
            floatx4 y = {0.f, 0.f, 0.f, 0.f};
            if constexpr (DELTA) {
                const int j = j0 + li;                 // this lane's row of R
                for (int i0 = j0; i0 < n; i0 += 4) {
                    const int i = i0 + kg;
                    // R[j][i]: 1 on the diagonal, column i's packed entry above it
                    float rji = (i == j) ? 1.f : 0.f;
                    if (j < i && i < n)
                        rji = sT[i * (i - 1) / 2 + j];
                    rji = (j < n) ? rji : 0.f;
                    y = mfma16x16x4(rji, qval(i, ch), y);
                }
            } else {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    y[rr] = qval(j0 + 4 * kg + rr, ch);
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                sy[(4 * kg + rr) * KS + ch] = y[rr];
        }
        __syncthreads();
        // S'^T += Y_c^T z_c^T (MFMA, accumulating in place)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if (m % 2 == 0)
                __builtin_amdgcn_sched_barrier(0);   // bound the LDS reads in flight
            float a[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                a[rr] = sy[(4 * kg + rr) * KS + 16 * m + li];
#pragma unroll
            for (int it = 0; it < NIT; ++it)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    st[it][m] = mfma16x16x4(a[rr], z[c][it][rr], st[it][m]);
        }
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
// WY merge for long logs at d = 128 (more than 32 entries): the same
// products as merge_wy_kernel, with the key side staged 16 entries at a time
// instead of whole.  A log of 64 entries with per-key decays has 48 KiB of
// keys and decays; staged whole beside R they leave room for two workgroups
// per CU, staged a chunk at a time (double-buffered: the next chunk loads
// while this one is used) for four.  Everything that needs the key side is
// done while its chunk is in LDS:
//   phase A  z_c = V_c^T - S0 Kt_c^T            (chunk c's keys),
//   Y        Y_t += R[t, c] Q_c for every t <= c (R is upper triangular, so
//            chunk c's entries reach the rows of Y up to chunk c),
// with the Y_t of every chunk accumulating in registers (each wave its share
// of the column blocks); then S0 diag(E_c) + sum_t z_t Y_t as before, each
// Y_t passing through LDS.  R stays whole in LDS (8 KiB at 64 entries), and
// the Lam row of the last entry, which every D(i, c) needs, is staged apart.
// A pair's rows split over two workgroups (64 rows each).
// ---------------------------------------------------------------------------
struct WyChunkPlan {
    int off_t;     // packed columns of R, whole log
    int off_buf;   // two staging buffers of one 16-entry chunk: keys, then Lam
    int buf;       // bytes per buffer
    int lam;       // offset of Lam inside a buffer
    int off_y;     // one chunk of Y, 16 rows of D + 4 floats (over the buffers)
    int off_ll;    // per-key decays: Lam of the last entry, D floats
    int off_f;     // per entry: beta_j (head-wise decay: times D(j, c)), 64 floats
    int off_e;     // per entry (head-wise decay): E_j, 64 floats
    int off_ec;    // E_c per key channel, D floats
    int off_n;     // the fill count read by the workgroup
    int bytes;
};

__host__ __device__ inline WyChunkPlan wy_chunk_plan(int variant, int D, int esize, int L) {
    WyChunkPlan p;
    p.off_t = 0;
    p.off_buf = round_up(packed_t_len(variant, L) * 4, 256);
    p.lam = round_up(16 * D * esize, 256);
    const int stage = p.lam + (variant == DL_GDN ? 0 : round_up(16 * D * 4, 256));
    const int ybytes = round_up(16 * (D + 4) * 4, 256);
    p.buf = stage;
    p.off_y = p.off_buf;
    const int end = p.off_buf + (2 * stage > ybytes ? 2 * stage : ybytes);
    p.off_ll = end;
    p.off_f = p.off_ll + (variant == DL_GDN ? 0 : D * 4);
    p.off_e = p.off_f + 256;
    p.off_ec = p.off_e + 256;
    p.off_n = p.off_ec + D * 4;
    p.bytes = p.off_n + 16;
    return p;
}

template <int V, int D, typename T, bool NTS>
__global__ void __launch_bounds__(256, 4)
merge_wy_chunked_kernel(Params P, const int *__restrict__ slot_idx, int mode, int npairs) {
    static_assert(D == 128, "long-log WY merge at d = 128");
    constexpr int NW = 4, ROWS = 16 * NW, NS = D / ROWS, NM = D / 16, KS = D + 4, MAXC = 4;
    constexpr bool PK = V != GDN, DELTA = V != RWKV6;
    extern __shared__ __align__(16) unsigned char smem[];
    const int L = P.L;
    const WyChunkPlan wp = wy_chunk_plan(V, D, (int)sizeof(T), L);
    const float *sT = reinterpret_cast<const float *>(smem + wp.off_t);
    const float *sll = reinterpret_cast<const float *>(smem + wp.off_ll);
    float *sf = reinterpret_cast<float *>(smem + wp.off_f);
    float *se = reinterpret_cast<float *>(smem + wp.off_e);
    float *sec = reinterpret_cast<float *>(smem + wp.off_ec);
    float *sy = reinterpret_cast<float *>(smem + wp.off_y);
    int *sn = reinterpret_cast<int *>(smem + wp.off_n);
    auto kbuf = [&](int c) { return smem + wp.off_buf + (c & 1) * wp.buf; };
    auto lbuf = [&](int c) { return reinterpret_cast<const float *>(smem + wp.off_buf + (c & 1) * wp.buf + wp.lam); };

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, kg = lane >> 4;
    // block -> (pair, split): the two workgroups of a pair are 8 blocks apart
    const int xcd = blockIdx.x & 7, qb = blockIdx.x >> 3;
    const int split = qb % NS;
    const int pr = (qb / NS) * 8 + xcd;
    if (pr >= npairs)
        return;
    const int H = P.heads;
    const int r = pr / H, h = pr - r * H;
    const int unit = slot_idx ? slot_idx[r] : r;
    if (unit < 0 || unit >= P.units) {
        if (split == 0)
            reject_row(P, nullptr, D, DL_FLAG_BAD_SLOT);
        return;
    }
    const size_t pair = (size_t)unit * H + h;
    if (tid == 0) {
        // the fill count through tickets in its upper half (as merge_wy_kernel)
        const int old = atomicAdd(P.fill + pair, 1 << 16);
        const int n0 = old & 0xffff;
        const bool go = n0 > 0 && n0 <= L && (mode != DL_MERGE_FULL || n0 == L);
        if ((old >> 16) == NS - 1)
            P.fill[pair] = go ? 0 : n0;
        sn[0] = go ? n0 : 0;
    }
    __syncthreads();
    const int n = sn[0];
    if (n == 0)
        return;
    const int nch = (n + 15) >> 4;       // chunks of 16 entries
    const size_t e0 = pair * L;

    // chunk c's keys (and per-key Lam) into its buffer, entries past n left
    // out (a direct-to-LDS load writes lane l at its wave-uniform address +
    // size * l, so each wave takes 64 consecutive elements of a pass)
    auto stage_chunk = [&](int c) {
        const int cnt = (n - 16 * c) < 16 ? (n - 16 * c) : 16;
        const int nk = cnt * D * (int)sizeof(T) / 16;
        const uint4 *ks = reinterpret_cast<const uint4 *>(static_cast<const T *>(P.log_k) + (e0 + 16 * c) * D);
        unsigned char *kd = kbuf(c);
        for (int b = 64 * wave; b < nk; b += 256)
            if (b + lane < nk)
                load_to_lds<16>(ks + b + lane, kd + 16 * b);
        if constexpr (PK) {
            const int nl = cnt * D / 4;
            const float4 *ls = reinterpret_cast<const float4 *>(P.log_g + (e0 + 16 * c) * D);
            for (int b = 64 * wave; b < nl; b += 256)
                if (b + lane < nl)
                    load_to_lds<16>(ls + b + lane, kd + wp.lam + 16 * b);
        }
    };

    // ---- loads: per-entry scalars (wave 0), R, the last entry's Lam, chunk
    //      0's key side, then the base rows and chunk 0's values
    float b_j = 1.f, lam_j = 0.f;
    if (wave == 0 && lane < n) {
        if constexpr (DELTA)
            b_j = P.log_beta[e0 + lane];
        if constexpr (!PK)
            lam_j = P.log_g[e0 + lane];
    }
    if constexpr (DELTA) {
        const int nt = n * (n - 1) / 2;
        const float *ts = P.log_t + pair * packed_t_len(V, L);
        for (int b = 64 * wave; b < nt; b += 256)
            if (b + lane < nt)
                load_to_lds<4>(ts + b + lane, smem + wp.off_t + 4 * b);
    }
    if constexpr (PK) {
        if (wave == 0 && lane < D / 4)
            load_to_lds<16>(reinterpret_cast<const float4 *>(P.log_g + (e0 + n - 1) * D) + lane,
                            smem + wp.off_ll);
    }
    stage_chunk(0);
    __builtin_amdgcn_sched_barrier(0);
    float *Sp = P.base + pair * D * D;
    const int row = split * ROWS + 16 * wave + li;
    floatx4 st[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const float4 x = load_state4<NTS>(Sp + (size_t)row * D + 4 * kg + 16 * m);
        st[m] = floatx4{x.x, x.y, x.z, x.w};
    }
    // values of chunk c on this lane: V[entry 16 c + 4 kg + rr][row], loaded
    // as they are (the last entry again past n) and masked where used, so
    // that nothing waits for them before then
    const T *Vl = static_cast<const T *>(P.log_v) + e0 * D;
    auto load_values = [&](int c, float (&vr)[4]) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int j = 16 * c + 4 * kg + rr;
            vr[rr] = Elem<T>::load1(Vl + (size_t)(j < n ? j : n - 1) * D + row);
        }
    };
    auto masked = [&](int c, const float (&vr)[4]) {
        floatx4 v;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            v[rr] = 16 * c + 4 * kg + rr < n ? vr[rr] : 0.f;
        return v;
    };
    float vv[4];
    load_values(0, vv);
    __builtin_amdgcn_sched_barrier(0);
    barrier_after_staging<NM + 4>();     // R, the last Lam row and chunk 0 staged

    // ---- per-entry factors and E_c
    if (wave == 0) {
        if constexpr (!PK) {
            const float lam_c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam_j), n - 1));
            if (lane < n) {
                sf[lane] = b_j * fast_exp(lam_c - lam_j);
                se[lane] = fast_exp(lam_j);
            }
            const float ec = fast_exp(lam_c);
            for (int c = lane; c < D; c += 64)
                sec[c] = ec;
        } else {
            if (lane < n)
                sf[lane] = b_j;
            for (int c = lane; c < D; c += 64)
                sec[c] = fast_exp(sll[c]);
        }
    }
    __syncthreads();

    // Q[i][ch] = f_i k_i[ch] (per-key: times D(i, c) on the channel) from
    // chunk c's buffer; 0 past n
    auto qval = [&](int c, int i, int ch) {
        const int ic = i < n ? i : n - 1;
        const int il = ic - 16 * c;
        float q = Elem<T>::load1(reinterpret_cast<const T *>(kbuf(c)) + il * D + ch) * sf[ic];
        if constexpr (PK)
            q *= fast_exp(sll[ch] - lbuf(c)[il * D + ch]);
        return i < n ? q : 0.f;
    };

    floatx4 z[MAXC], yacc[MAXC][NM / NW];
#pragma unroll
    for (int t = 0; t < MAXC; ++t)
#pragma unroll
        for (int mb = 0; mb < NM / NW; ++mb)
            yacc[t][mb] = floatx4{0.f, 0.f, 0.f, 0.f};
    // ---- phase A for chunk c: z_c = V_c^T - S0 Kt_c^T
    auto phase_a = [&](int c) {
        z[c] = masked(c, vv);
        if constexpr (DELTA) {
            const int j = 16 * c + li;            // this lane's entry of the A operand
            const bool live = j < n;
            const int jl = (live ? j : n - 1) - 16 * c;
            const float ej = PK ? 1.f : (live ? se[16 * c + jl] : 0.f);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                if (m % 2 == 0)
                    __builtin_amdgcn_sched_barrier(0);   // bound the LDS reads in flight
                const int col = 4 * kg + 16 * m;
                float4 kt = lds_load4<T>(kbuf(c), jl * D + col);
                if constexpr (PK) {
                    const float4 l4 = *reinterpret_cast<const float4 *>(lbuf(c) + jl * D + col);
                    kt.x *= fast_exp(l4.x), kt.y *= fast_exp(l4.y);
                    kt.z *= fast_exp(l4.z), kt.w *= fast_exp(l4.w);
                }
                const float f = live ? -ej : 0.f;   // -Kt (head-wise: E_j; per-key: folded above)
                z[c] = mfma16x16x4(f * kt.x, st[m][0], z[c]);
                z[c] = mfma16x16x4(f * kt.y, st[m][1], z[c]);
                z[c] = mfma16x16x4(f * kt.z, st[m][2], z[c]);
                z[c] = mfma16x16x4(f * kt.w, st[m][3], z[c]);
            }
        }
    };
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        if (c >= nch)
            break;
        // The next chunk's key side and values load while this one is used;
        // its buffer held chunk c - 1, consumed before the last barrier.  For
        // chunk 0 they are issued after phase A, which waits for the base
        // rows: issued before it, they would be waited for with them.
        // The value loads are not under a condition (past the last chunk they
        // read the last entry again and go unused): a load under one leaves
        // its register to be merged with the other path's, and the compiler
        // waits for every load in flight before that copy.  A chunk past the
        // log stages nothing.
        float vn[4];
        if (c > 0) {
            stage_chunk(c + 1);
            load_values(c + 1, vn);
        }
        phase_a(c);
        if (c == 0) {
            stage_chunk(1);
            load_values(1, vn);
        }
        // ---- Y_t += R[t rows, chunk c columns] Q_c for t <= c, on this
        //      wave's column blocks: Y_t[16 t + 4 kg + rr][16 m + li]
#pragma unroll
        for (int mb = 0; mb < NM / NW; ++mb) {
            const int m = wave * (NM / NW) + mb;
            const int ch = 16 * m + li;
            if constexpr (DELTA) {
                // this lane's Q operands of the chunk's four k-steps, shared
                // by every row block t
                float qv[4];
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4)
                    qv[s4] = qval(c, 16 * c + 4 * s4 + kg, ch);
#pragma unroll
                for (int t = 0; t <= c; ++t) {
                    const int j = 16 * t + li;             // this lane's row of R
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) {
                        const int i0 = 16 * c + 4 * s4;
                        if (i0 >= n)
                            break;
                        const int i = i0 + kg;
                        // R[j][i]: 1 on the diagonal, column i's packed entry above it
                        float rji = (i == j) ? 1.f : 0.f;
                        if (j < i && i < n)
                            rji = sT[i * (i - 1) / 2 + j];
                        rji = (j < n) ? rji : 0.f;
                        yacc[t][mb] = mfma16x16x4(rji, qv[s4], yacc[t][mb]);
                    }
                }
            } else {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    yacc[c][mb][rr] = qval(c, 16 * c + 4 * kg + rr, ch);
            }
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            vv[rr] = vn[rr];
        wait_vm_all();      // the next chunk has landed in its buffer
        __syncthreads();    // and this chunk's buffer is consumed
    }

    // ---- S0 diag(E_c), then S0 += z_t Y_t chunk by chunk
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const float4 el = *reinterpret_cast<const float4 *>(sec + 4 * kg + 16 * m);
        st[m][0] *= el.x;
        st[m][1] *= el.y;
        st[m][2] *= el.z;
        st[m][3] *= el.w;
    }
#pragma unroll
    for (int t = 0; t < MAXC; ++t) {
        if (t >= nch)
            break;
        if (t > 0)
            __syncthreads();    // the previous Y_t is consumed
#pragma unroll
        for (int mb = 0; mb < NM / NW; ++mb) {
            const int ch = 16 * (wave * (NM / NW) + mb) + li;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                sy[(4 * kg + rr) * KS + ch] = yacc[t][mb][rr];
        }
        __syncthreads();
        // S'^T += Y_t^T z_t^T (MFMA, accumulating in place)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if (m % 2 == 0)
                __builtin_amdgcn_sched_barrier(0);   // bound the LDS reads in flight
            float a[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                a[rr] = sy[(4 * kg + rr) * KS + 16 * m + li];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                st[m] = mfma16x16x4(a[rr], z[t][rr], st[m]);
        }
    }

#pragma unroll
    for (int m = 0; m < NM; ++m)
        store_state4<NTS>(Sp + (size_t)row * D + 4 * kg + 16 * m,
                          make_float4(st[m][0], st[m][1], st[m][2], st[m][3]));
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

template <int V, int D, typename T, int NW, int NIT, int NE>
static void wy_launch(const Params &P, int pairs, const int *slot_idx, int mode, const Launch &ln) {
    using WS = WyShape<V, D, T, NW, NIT, NE>;
    const WyPlan wp = wy_plan(V, D, (int)sizeof(T), P.L);
    const dim3 grid(((pairs + 7) / 8) * 8 * WS::NS), block(WS::NTH);
    if (P.stream)
        hipExtLaunchKernelGGL((merge_wy_kernel<V, D, T, true, NW, NIT, NE>), grid, block, wp.bytes,
                              ln.stream, ln.start, ln.stop, 0, P, slot_idx, mode, pairs);
    else
        hipExtLaunchKernelGGL((merge_wy_kernel<V, D, T, false, NW, NIT, NE>), grid, block, wp.bytes,
                              ln.stream, ln.start, ln.stop, 0, P, slot_idx, mode, pairs);
}

// d = 128: with per-key decays, one workgroup per pair, holding the pair's
// whole base, while the chunks' z tiles fit beside it in registers (logs of
// up to 32 entries); with head-wise decay, a pair's rows split over two
// workgroups of half the registers (twice the workgroups per CU, each
// staging the pair's key side again: about 4% faster for GDN at 16 and 32
// entries, 20% slower for per-key decays at 32, whose key side is twice as
// large).  Longer logs take the chunked kernel (two workgroups per pair).  Splitting further (four workgroups of two waves) measured
// slower everywhere: a workgroup's time is set by its chain of loads,
// barriers and contractions, not by its share of the base.
template <int V, int D, typename T>
static hipError_t wy_t(const Params &P, int rows, const int *slot_idx, int mode,
                       const Launch &ln) {
    const int pairs = rows * P.heads;
    if constexpr (D == 128) {
        if (P.L <= 16) {
            if constexpr (V == GDN)
                wy_launch<V, D, T, 4, 1, 1>(P, pairs, slot_idx, mode, ln);
            else
                wy_launch<V, D, T, 4, 2, 1>(P, pairs, slot_idx, mode, ln);
        } else if (P.L <= 32) {
            if constexpr (V == GDN)
                wy_launch<V, D, T, 4, 1, 2>(P, pairs, slot_idx, mode, ln);
            else
                wy_launch<V, D, T, 4, 2, 2>(P, pairs, slot_idx, mode, ln);
        } else {
            const WyChunkPlan wp = wy_chunk_plan(V, D, (int)sizeof(T), P.L);
            const dim3 grid(((pairs + 7) / 8) * 8 * 2), block(256);
            if (P.stream)
                hipExtLaunchKernelGGL((merge_wy_chunked_kernel<V, D, T, true>), grid, block, wp.bytes,
                                      ln.stream, ln.start, ln.stop, 0, P, slot_idx, mode, pairs);
            else
                hipExtLaunchKernelGGL((merge_wy_chunked_kernel<V, D, T, false>), grid, block, wp.bytes,
                                      ln.stream, ln.start, ln.stop, 0, P, slot_idx, mode, pairs);
        }
    } else {
        wy_launch<V, D, T, 4, 1, 4>(P, pairs, slot_idx, mode, ln);
    }
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
