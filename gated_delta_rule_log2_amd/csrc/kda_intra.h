// kda_intra.h -- intra-chunk stage of the KDA forward, one workgroup per
// (chunk, value head), one wave per 16-row sub-chunk.
//
// Per chunk, with G the base-2 chunk-local cumulative gate, q^ = scale*q/|q|,
// k^ = k/|k| and beta b ("Reading Notes: Implementation Notes for KDA in FLA",
// forward steps 1-3):
//   Aqk[i][j]  = sum_d q^_id k^_jd 2^(G_id - G_jd)          (j <= i)
//   Akk0[i][j] = b_i sum_d k^_id k^_jd 2^(G_id - G_jd)      (j <  i)
//   A = (I + Akk0)^-1,  W = A (b * 2^G * k^),  U = A (b * v)
//   Qg = 2^G * q^,  KgT = (2^(G_last - G) * k^)^T,  d = 2^G_last
// which the recurrence kernel consumes, stored in the fragment-major layouts below.
//
// Exponent handling ("flash-linear-attention KDA 内核工程实践…", §3.1 and §3.2):
//   - sub-chunk pairs (p > s) factor 2^(G_i - G_j) as 2^(G_i - G_n) * 2^(G_n - G_j)
//     with n the first row of sub-chunk p; every exponent is <= 0.  Here the
//     second factor is split once more, 2^(G_n - G_e) * 2^(G_e - G_j) with e the
//     last row of sub-chunk s, so each element needs two exp2 of its own
//     (Rf = 2^(G - G_n), Cf = 2^(G_e - G)) and everything pair-dependent is a
//     per-column scalar, computed once per chunk in a column pass.
//   - diagonal sub-chunks subtract the cumulative gate at the sub-chunk midpoint
//     (row min(8, rows left - 1)), so both operand exponents stay small.  The
//     kernel checks that |G - G_mid| <= 60 over the sub-chunk (always true for
//     the bounded gate with lower_bound >= -5, where it is at most 8*5*log2(e));
//     otherwise that block falls back to element-wise exp2 of non-positive
//     differences, the token-parallel form of §4.
//   - the diagonal 16x16 blocks of I + Akk0 are inverted by forward substitution
//     in fp32 and merged into the full inverse block by block (§3.1, §4), here on
//     fp32 matrix cores.
// Products are formed with the operand roles chosen so that each lane's share of
// a result tile is 4 contiguous elements of an output row.
#pragma once

#include "kda_gate.h"

namespace kda {

constexpr float kDiagSpanLimit = 60.f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int C, typename T>
struct IntraLds {
    static constexpr int NB = C / 16;
    // per-column reference rows of G: Gn[NB] (first row), Ge[NB] (last valid row),
    // Gm[NB] (midpoint row), Glast
    static constexpr int NGR = 3 * NB + 1;
    // per-column scalars: En[NB] = 2^Gn, sa[NB] = 2^(Gn-Gm), sb[NB] = 2^(Gm-Ge),
    // kgf[NB] = 2^(Glast-Ge), sig[NB(NB-1)/2] = 2^(Gn[p]-Ge[s]) for s < p
    static constexpr int NSC = 4 * NB + NB * (NB - 1) / 2;
    static constexpr int LDA = C + 4;
    static __host__ __device__ int ldk(int K) { return K + 8; }
    static __host__ __device__ int ldc() { return C + 8; }
    static __host__ __device__ size_t tot(int) { return 0; }
    static __host__ __device__ size_t gr(int K) { return tot(K) + sizeof(float) * NB * K; }
    static __host__ __device__ size_t sc(int K) { return gr(K) + sizeof(float) * NGR * K; }
    static __host__ __device__ size_t ainv(int K) { return sc(K) + sizeof(float) * NSC * K; }
    static __host__ __device__ size_t region(int K) { return ainv(K) + sizeof(float) * C * LDA; }
    // phase 1 of the region: KCs [C][K+8] and Akk [C][LDA]
    static __host__ __device__ size_t kcs(int K) { return region(K); }
    static __host__ __device__ size_t akk(int K) { return (kcs(K) + sizeof(T) * C * ldk(K) + 15) / 16 * 16; }
    // phase 2: XT [K][C+8] and VT [V][C+8]
    static __host__ __device__ size_t xt(int K) { return region(K); }
    static __host__ __device__ size_t vt(int K) { return xt(K) + sizeof(T) * K * ldc(); }
    static __host__ __device__ size_t bytes(int K, int V) {
        const size_t p1 = akk(K) + sizeof(float) * C * LDA;
        const size_t p2 = vt(K) + sizeof(T) * V * ldc();
        return p1 > p2 ? p1 : p2;
    }
};

// 16x16x16 fp32 product on matrix cores: acc += X(16x16) * Y(16x16), X row-major
// in LDS with stride ldx, Y row-major with stride ldy.  Lane group cg supplies
// contraction indices 4*cg + q (q < 4).
__device__ __forceinline__ f32x4 mma16_f32_lds(f32x4 acc, const float *X, int ldx, const float *Y, int ldy) {
    const int l = lane_id(), r = l & 15, cg = l >> 4;
    const float4 a = *reinterpret_cast<const float4 *>(X + r * ldx + 4 * cg);
    const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], Y[(4 * cg + q) * ldy + r], acc, 0, 0, 0);
    return acc;
}

// Fragment-major layouts of the per-chunk intermediates, in exactly the order the
// recurrence kernel's lanes load them (each wave-wide load is one contiguous 1 KB
// (bf16) run instead of 16 partial cache lines):
//   row fragments (W, Qg [C][K]; Aqk [C][C]; KgT [K][C]): element (row, col) at
//     ((row/16 * (ncols/32) + col/32) * 64 + row%16 + 16 * ((col%32)/8)) * 8 + col%8
//   U in accumulator quads: element U[m][v] at
//     ((v/16 * (C/16) + m/16) * 64 + v%16 + 16 * ((m%16)/4)) * 4 + m%4
//   permuted row fragments: as row fragments, but the 8 contraction indices of lane
//     group g inside a 32-column block are {4g..4g+3} and {16+4g..16+4g+3}, i.e.
//     element (row, col) at
//     ((row/16 * (ncols/32) + col/32) * 64 + row%16 + 16 * ((col%16)/4)) * 8 + 4 * ((col%32)/16) + col%4
//     With this order the accumulator layout of a 16x16 product (lane group g holds
//     rows 4g..4g+3) is, two tiles at a time, already the contraction-operand layout
//     of the next product, so results feed matrix cores without a lane exchange.
__host__ __device__ __forceinline__ size_t frag_off(int row, int col, int ncols) {
    return ((size_t)((row >> 4) * (ncols >> 5) + (col >> 5)) * 64 + (row & 15) + 16 * ((col & 31) >> 3)) * 8 + (col & 7);
}
__host__ __device__ __forceinline__ size_t quad_off(int m, int v, int C) {
    return ((size_t)((v >> 4) * (C >> 4) + (m >> 4)) * 64 + (v & 15) + 16 * ((m & 15) >> 2)) * 4 + (m & 3);
}
__host__ __device__ __forceinline__ size_t pfrag_off(int row, int col, int ncols) {
    return ((size_t)((row >> 4) * (ncols >> 5) + (col >> 5)) * 64 + (row & 15) + 16 * ((col & 15) >> 2)) * 8 +
           4 * ((col & 31) >> 4) + (col & 3);
}

template <int C, typename T, int NKK>
__global__ void __launch_bounds__(C / 16 * 64) intra_kernel(Params p) {
    constexpr int NB = C / 16;
    constexpr bool F32 = sizeof(T) == 4;
    using L_ = IntraLds<C, T>;
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr int K = 32 * NKK;
    const int V = p.V;
    constexpr int nkk = NKK;
    const int nvk = V / 32;
    float *tot = reinterpret_cast<float *>(lds + L_::tot(K));
    float *GR = reinterpret_cast<float *>(lds + L_::gr(K));
    float *SC = reinterpret_cast<float *>(lds + L_::sc(K));
    float *Ainv = reinterpret_cast<float *>(lds + L_::ainv(K));
    T *KCs = reinterpret_cast<T *>(lds + L_::kcs(K));
    float *Akk = reinterpret_cast<float *>(lds + L_::akk(K));
    T *XT = reinterpret_cast<T *>(lds + L_::xt(K));
    T *VTs = reinterpret_cast<T *>(lds + L_::vt(K));
    const int LDK = L_::ldk(K), LDC = L_::ldc();
    constexpr int LDA = L_::LDA;
    // row indices into GR / SC
    auto gr_n = [](int b) { return b; };
    auto gr_e = [](int b) { return NB + b; };
    auto gr_m = [](int b) { return 2 * NB + b; };
    constexpr int gr_last = 3 * NB;
    auto sc_en = [](int b) { return b; };
    auto sc_sa = [](int b) { return NB + b; };
    auto sc_sb = [](int b) { return 2 * NB + b; };
    auto sc_kg = [](int b) { return 3 * NB + b; };
    auto sc_sig = [](int pp, int s) { return 4 * NB + pp * (pp - 1) / 2 + s; };

    const int hv = blockIdx.x % p.HV;
    const int gc = blockIdx.x / p.HV;
    const int h = hv / p.group;
    const ChunkInfo ci = chunk_info(p, gc);
    const int w = threadIdx.x >> 6;  // this wave's 16-row sub-chunk
    const int l = lane_id();
    const int lr = l & 15, cg = l >> 4;
    const int r = 16 * w + lr;       // chunk row held by this lane
    const bool valid = r < ci.L;
    const size_t slot = (size_t)gc * p.HV + hv;
    T *Wg = static_cast<T *>(p.w_W) + slot * C * K;
    T *UTg = static_cast<T *>(p.w_U) + slot * (size_t)V * C;
    T *KgTg = static_cast<T *>(p.w_KgT) + slot * K * C;
    T *Qgg = static_cast<T *>(p.w_Qg) + slot * C * K;
    T *Aqkg = static_cast<T *>(p.w_Aqk) + slot * C * C;
    float *dg = p.w_d + slot * K;

    // raw q, k rows (loads issued before the gate so their latency overlaps it)
    float qh[NKK][8], kh[NKK][8];
    const int64_t qrow = ((ci.tok0 + r) * p.H + h) * (int64_t)K;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if (kk < nkk) {
            if (valid) {
                load8(static_cast<const T *>(p.q) + qrow + 32 * kk + 8 * cg, qh[kk]);
                load8(static_cast<const T *>(p.k) + qrow + 32 * kk + 8 * cg, kh[kk]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) qh[kk][i] = kh[kk][i] = 0.f;
            }
        }
    }
    const float b_r = valid ? beta_act(p.beta_mode, load_any(p.beta, (ci.tok0 + r) * p.HV + hv, p.beta_bf16)) : 0.f;

    // ---- step 1: gate activation + base-2 chunk-local cumsum (row fragment) ----
    float G[NKK][8], tmp[NKK][8];
    gate_cumsum_block<NKK>(p, ci, hv, w, nkk, G, tot, tmp);

    // reference rows of this sub-chunk (clamped for sub-chunks past the end)
    int e_loc = ci.L - 1 - 16 * w;
    e_loc = e_loc > 15 ? 15 : (e_loc < 0 ? 0 : e_loc);
    const int mid_loc = e_loc < 8 ? e_loc : 8;
    const bool last_here = (16 * w + e_loc == ci.L - 1);

    // ---- step 2: reference rows -> LDS; norms ----
    float ssq = 0.f, ssk = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if (kk < nkk) {
            const int d0 = 32 * kk + 8 * cg;
            if (lr == 0) store8(GR + gr_n(w) * K + d0, G[kk]);
            if (lr == e_loc) {
                store8(GR + gr_e(w) * K + d0, G[kk]);
                if (last_here) store8(GR + gr_last * K + d0, G[kk]);
            }
            if (lr == mid_loc) store8(GR + gr_m(w) * K + d0, G[kk]);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                ssq += qh[kk][i] * qh[kk][i];
                ssk += kh[kk][i] * kh[kk][i];
            }
        }
    }
    float rq = p.scale, rk = 1.f;
    if (p.qk_l2norm) {
        ssq = sum_col_groups(ssq);
        ssk = sum_col_groups(ssk);
        rq *= rsqrtf(ssq + 1e-6f);
        rk = rsqrtf(ssk + 1e-6f);
    }
    __syncthreads();

    // ---- step 3: per-column scalars (one pass over the K columns) ----
    for (int e = threadIdx.x; e < L_::NSC * K; e += blockDim.x) {
        const int row = e / K, d = e % K;
        float x;
        if (row < NB) x = GR[gr_n(row) * K + d];
        else if (row < 2 * NB) x = GR[gr_n(row - NB) * K + d] - GR[gr_m(row - NB) * K + d];
        else if (row < 3 * NB) x = GR[gr_m(row - 2 * NB) * K + d] - GR[gr_e(row - 2 * NB) * K + d];
        else if (row < 4 * NB) x = GR[gr_last * K + d] - GR[gr_e(row - 3 * NB) * K + d];
        else {
            int q = row - 4 * NB, pp = 1;
            while (q >= pp) { q -= pp; ++pp; }
            x = GR[gr_n(pp) * K + d] - GR[gr_e(q) * K + d];
        }
        SC[row * K + d] = fast_exp2(x);
    }
    for (int d = threadIdx.x; d < K; d += blockDim.x) dg[d] = fast_exp2(GR[gr_last * K + d]);

    // ---- step 4: per-element factors and operands (row fragment) ----
    //   QR = q^ 2^(G - G_n), KR = k^ 2^(G - G_n), KC = k^ 2^(G_e - G)
    float QR[NKK][8], KR[NKK][8], KC[NKK][8];
    bool wide = false;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if (kk < nkk) {
            const int d0 = 32 * kk + 8 * cg;
            float gn[8], ge[8], gm[8];
            load8(GR + gr_n(w) * K + d0, gn);
            load8(GR + gr_e(w) * K + d0, ge);
            load8(GR + gr_m(w) * K + d0, gm);
            float kc8[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float g = G[kk][i];
                wide |= fabsf(g - gm[i]) > kDiagSpanLimit;
                const float qn = qh[kk][i] * rq, kn = kh[kk][i] * rk;
                const float rf = fast_exp2(g - gn[i]);
                QR[kk][i] = qn * rf;
                KR[kk][i] = kn * rf;
                KC[kk][i] = kn * fast_exp2(ge[i] - g);
                kc8[i] = KC[kk][i];
            }
            store8(KCs + r * LDK + d0, kc8);
        }
    }
    const bool diag_fallback = __any(wide);
    __syncthreads();  // KCs, SC complete

    // Qg = QR 2^G_n (row-major, 16-byte stores)
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if (kk < nkk) {
            const int d0 = 32 * kk + 8 * cg;
            float en[8], qg8[8];
            load8(SC + sc_en(w) * K + d0, en);
#pragma unroll
            for (int i = 0; i < 8; ++i) qg8[i] = QR[kk][i] * en[i];
            store8(Qgg + frag_off(r, d0, K), qg8);
        }
    }

    // ---- step 5: Aqk^T and Akk0^T tiles of row block w (lane: row i = 16w+lr,
    //      columns j = 16s + 4cg .. +3) ----
    f32x4 accQ[NB], accK[NB], accQd = zero4(), accKd = zero4();
#pragma unroll
    for (int s = 0; s < NB; ++s) accQ[s] = accK[s] = zero4();
#pragma unroll
    for (int s = 0; s < NB; ++s) {
        if (s < w) {
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                if (kk < nkk) {
                    const int d0 = 32 * kk + 8 * cg;
                    float bq[8], bk[8], kc[8], sig[8];
                    load8(KCs + (16 * s + lr) * LDK + d0, kc);
                    load8(SC + sc_sig(w, s) * K + d0, sig);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        bq[i] = QR[kk][i] * sig[i];
                        bk[i] = KR[kk][i] * sig[i];
                    }
                    accQ[s] = mma32<F32>(accQ[s], kc, bq);
                    accK[s] = mma32<F32>(accK[s], kc, bk);
                }
            }
        }
    }
    if (!diag_fallback) {
        // midpoint split: (k^ 2^(G_mid - G_j)) . (q^ 2^(G_i - G_mid))
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            if (kk < nkk) {
                const int d0 = 32 * kk + 8 * cg;
                float sa[8], sb[8], aq[8], ak[8], bk[8];
                load8(SC + sc_sa(w) * K + d0, sa);
                load8(SC + sc_sb(w) * K + d0, sb);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    aq[i] = QR[kk][i] * sa[i];
                    ak[i] = KR[kk][i] * sa[i];
                    bk[i] = KC[kk][i] * sb[i];
                }
                accQd = mma32<F32>(accQd, bk, aq);
                accKd = mma32<F32>(accKd, bk, ak);
            }
        }
    }
    // mask, beta, store: Aqk -> global, Akk0 -> LDS (fp32)
#pragma unroll
    for (int s = 0; s < NB; ++s) {
        float aq[4], ak[4];
        const f32x4 vq = (s == w) ? accQd : accQ[s], vk = (s == w) ? accKd : accK[s];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int jl = 4 * cg + jj;  // column inside block s
            aq[jj] = (s < w || (s == w && jl <= lr)) ? vq[jj] : 0.f;
            ak[jj] = (s < w || (s == w && jl < lr)) ? b_r * vk[jj] : 0.f;
        }
        if (!(s == w && diag_fallback)) {
            store4(Aqkg + frag_off(r, 16 * s + 4 * cg, C), aq[0], aq[1], aq[2], aq[3]);
            store4(Akk + r * LDA + 16 * s + 4 * cg, ak[0], ak[1], ak[2], ak[3]);
        }
    }
    if (diag_fallback) {
        // element-wise diagonal block: every factor is 2^(G_i - G_j) with j <= i (<= 1).
        // G, q and k are recomputed (same arithmetic, same values) rather than kept live.
        float Gf[NKK][8], q2[NKK][8], k2[NKK][8];
        gate_scan_block<NKK>(p, ci, hv, w, nkk, Gf, q2);
        gate_add_prefix<NKK>(tot, K, w, nkk, Gf);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            if (kk < nkk) {
                if (valid) {
                    load8(static_cast<const T *>(p.q) + qrow + 32 * kk + 8 * cg, q2[kk]);
                    load8(static_cast<const T *>(p.k) + qrow + 32 * kk + 8 * cg, k2[kk]);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) q2[kk][i] = k2[kk][i] = 0.f;
                }
            }
        }
        for (int jr = 0; jr < 16; ++jr) {
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                if (kk < nkk) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float kn = k2[kk][i] * rk;
                        const float kj = shfl(kn, (l & 0x30) + jr);
                        const float gj = shfl(Gf[kk][i], (l & 0x30) + jr);
                        const float f = lr >= jr ? fast_exp2(Gf[kk][i] - gj) : 0.f;
                        sq += q2[kk][i] * rq * kj * f;
                        sk += kn * kj * f;
                    }
                }
            }
            sq = sum_col_groups(sq);
            sk = sum_col_groups(sk);
            if (cg == 0) {
                Aqkg[frag_off(r, 16 * w + jr, C)] = Store<T>::to(lr >= jr ? sq : 0.f);
                Akk[r * LDA + 16 * w + jr] = lr > jr ? b_r * sk : 0.f;
            }
        }
    }
    // X = b k^ 2^G = b KR 2^G_n, kept (as fp32) for W after the solve
    float X[NKK][8];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if (kk < nkk) {
            float en[8];
            load8(SC + sc_en(w) * K + 32 * kk + 8 * cg, en);
#pragma unroll
            for (int i = 0; i < 8; ++i) X[kk][i] = b_r * KR[kk][i] * en[i];
        }
    }
    __syncthreads();  // Akk complete; KCs no longer written

    // ---- step 6: KgT[d][m] = KC[m][d] 2^(G_last - G_e(m)) -> global, via LDS columns ----
    for (int e = threadIdx.x; e < K * (C / 8); e += blockDim.x) {
        const int d = e / (C / 8), mo = e % (C / 8);
        const float kg = SC[sc_kg((8 * mo) / 16) * K + d];
        float v8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v8[i] = Store<T>::from(KCs[(8 * mo + i) * LDK + d]) * kg;
        store8(KgTg + frag_off(d, 8 * mo, C), v8);
    }

    // ---- step 7: A = (I + Akk0)^-1, fp32 ----
    // diagonal blocks: lane j of wave w holds column j of D_w = (I + L_ww)^-1
    if (l < 16) {
        float col[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) col[m] = (m == l) ? 1.f : 0.f;
        const float *Lb = Akk + (16 * w) * LDA + 16 * w;
#pragma unroll
        for (int i = 1; i < 16; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) acc += Lb[i * LDA + m] * col[m];
            if (i > l) col[i] = -acc;
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) Ainv[(16 * w + m) * LDA + 16 * w + l] = col[m];
    }
    for (int s = w + 1; s < NB; ++s)
        for (int e = l; e < 256; e += 64) Ainv[(16 * w + (e >> 4)) * LDA + 16 * s + (e & 15)] = 0.f;
    __syncthreads();
#pragma unroll
    for (int dist = 1; dist < NB; ++dist) {
        if (w >= dist) {
            const int s = w - dist;
            f32x4 t = zero4();
            for (int m = s; m < w; ++m)
                t = mma16_f32_lds(t, Akk + (16 * w) * LDA + 16 * m, LDA, Ainv + (16 * m) * LDA + 16 * s, LDA);
            const float4 a = *reinterpret_cast<const float4 *>(Ainv + (16 * w + lr) * LDA + 16 * w + 4 * cg);
            const float av[4] = {a.x, a.y, a.z, a.w};
            f32x4 uu = zero4();
#pragma unroll
            for (int q = 0; q < 4; ++q) uu = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], t[q], uu, 0, 0, 0);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) Ainv[(16 * w + 4 * cg + jj) * LDA + 16 * s + lr] = -uu[jj];
        }
        __syncthreads();
    }

    // ---- step 8: XT[d][m] = X[m][d], VT[n][m] = b_m v_mn (LDS, transposed) ----
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if (kk < nkk) {
#pragma unroll
            for (int i = 0; i < 8; ++i) XT[(32 * kk + 8 * cg + i) * LDC + r] = Store<T>::to(X[kk][i]);
        }
    }
    const int64_t vrow = ((ci.tok0 + r) * p.HV + hv) * (int64_t)V;
    for (int vk = 0; vk < nvk; ++vk) {
        float x[8];
        if (valid) load8(static_cast<const T *>(p.v) + vrow + 32 * vk + 8 * cg, x);
        else {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) VTs[(32 * vk + 8 * cg + i) * LDC + r] = Store<T>::to(b_r * x[i]);
    }
    __syncthreads();

    // ---- step 9: W = A X (as W^T tiles: lane row m = 16w+lr, columns d = 16dt+4cg..),
    //      U = A (b v) (as U tiles, stored U^T: lane row v = 16vt+lr, columns m) ----
    {
        const int nms = (16 * w + 16 + 31) / 32;
        float am[2][8];
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
            if (ms < nms) load8(Ainv + (16 * w + lr) * LDA + 32 * ms + 8 * cg, am[ms]);
        for (int dt = 0; dt < K / 16; ++dt) {
            f32x4 acc = zero4();
#pragma unroll
            for (int ms = 0; ms < 2; ++ms) {
                if (ms < nms) {
                    float bx[8];
                    load8(XT + (16 * dt + lr) * LDC + 32 * ms + 8 * cg, bx);
                    acc = mma32<F32>(acc, bx, am[ms]);
                }
            }
            store4(Wg + frag_off(r, 16 * dt + 4 * cg, K), acc[0], acc[1], acc[2], acc[3]);
        }
        for (int vt = 0; vt < V / 16; ++vt) {
            f32x4 acc = zero4();
#pragma unroll
            for (int ms = 0; ms < 2; ++ms) {
                if (ms < nms) {
                    float bx[8];
                    load8(VTs + (16 * vt + lr) * LDC + 32 * ms + 8 * cg, bx);
                    acc = mma32<F32>(acc, am[ms], bx);
                }
            }
            store4(UTg + quad_off(16 * w + 4 * cg, 16 * vt + lr, C), acc[0], acc[1], acc[2], acc[3]);
        }
    }
}

template <int C, typename T, int NKK>
hipError_t launch_intra_t(const Params &p, hipStream_t s) {
    const size_t lds = IntraLds<C, T>::bytes(p.K, p.V);
    auto kern = intra_kernel<C, T, NKK>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)p.total_chunks * (unsigned)p.HV), dim3(64 * (C / 16)), lds, s, p);
    return hipGetLastError();
}

// Exact-K dispatch (K = 32 * NKK) for one (chunk size, storage type).
template <int C, typename T>
hipError_t launch_intra_ct(const Params &p, hipStream_t s) {
    switch (p.K / 32) {
    case 1: return launch_intra_t<C, T, 1>(p, s);
    case 2: return launch_intra_t<C, T, 2>(p, s);
    case 3: return launch_intra_t<C, T, 3>(p, s);
    case 4: return launch_intra_t<C, T, 4>(p, s);
    case 5: return launch_intra_t<C, T, 5>(p, s);
    case 6: return launch_intra_t<C, T, 6>(p, s);
    case 7: return launch_intra_t<C, T, 7>(p, s);
    case 8: return launch_intra_t<C, T, 8>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
