// kda_bwd_local.h -- the per-chunk gradients of the KDA backward ("Reading Notes:
// Implementation Notes for KDA in FLA", backward steps 3, 5, 6 and 7), for K <= 128.
//
// One workgroup of C/16 waves per (chunk, value head); wave w owns the chunk rows
// 16w..16w+15.  With the forward's quantities of the chunk (natural-log cumulative gate
// G, E = e^G, F = e^(gamma - G), gamma = G at the last row, normalised q^ k^, beta b,
// M[i][j] = sum_d k^_id k^_jd e^(G_id - G_jd) for j < i, Akk0 = Diag(b) M,
// A = (I + Akk0)^-1, X = Diag(b) (k^ E), Y = Diag(b) v - X S_prev, V_new = A Y), the
// state S_prev the chunk starts from, the gradient dS of the state after it and
// dU = dL/dV_new (both from the reverse chunk recurrence) and dO:
//   dQg = dO S_prev^T,   dW = -dU S_prev^T,   dKg = V_new dS^T,   dd = rowsum(S_prev o dS)
//   dAqk = tril(dO V_new^T)                                        (step 3)
//   dv = b o (A^T dU),   dX = A^T dW,   dA = dU (b v)^T + dW X^T     (step 5, the WY chain)
//   dAkk0 = -A^T dA A^T (strictly lower),   dM = Diag(b) dAkk0
//   db = rowsum(v o A^T dU) + rowsum(dAkk0 o M) + rowsum(dX o k^ o E)
//   dq^ = dQg o E + (dAqk through Aqk),   dk^ = dKg o F + b dX o E + (dAqk, dM through Aqk, M)
//   dG = dQg o Qg - dKg o Kg + b dX o k^ o E + (pairwise terms) ;  dgamma = colsum(dKg o Kg) + dd o e^gamma
//   dg' = suffix cumsum over the chunk of dG, with dgamma added at the last row   (step 7)
// The pairwise terms of Aqk and M (step 6) are formed per 16-row block pair with the
// exponents split as in the forward: the first row of the later block as the offset for
// pairs of different blocks ("flash-linear-attention KDA 内核工程实践…", §3.2) and the
// midpoint row for a diagonal block (§3.1), or element by element for a diagonal block
// whose midpoint factors would exceed 2^60 (§4).
//
// Layouts: every per-element quantity of a wave lives in registers in the "T layout":
// lane (lr, cg) holds row 16w + lr and, for each 16-column tile t, columns 16t + 4cg ..
// +3.  Products whose result has that layout are formed as transposed tiles.  The
// state-side products run over 32-column blocks of V staged in LDS.
#pragma once

#include "kda_bwd_dhu.h"

namespace kda {

// Sum over the 16 lanes of each DPP row, in every lane of the row.
__device__ __forceinline__ float row_sum16_all(float x) {
    auto dpp = [](float v, auto ctrl_tag) {
        constexpr int CTRL = decltype(ctrl_tag)::value;
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
    };
    x += dpp(x, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
    x += dpp(x, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
    x += dpp(x, std::integral_constant<int, 0x124>{});  // row_ror 4
    x += dpp(x, std::integral_constant<int, 0x128>{});  // row_ror 8
    return x;
}

// Value of lane (l + n) within the same 16-lane row, 0 past the row's end (DPP row_shl).
template <int N>
__device__ __forceinline__ float row_shl(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x100 + N, 0xf, 0xf, false));
}
// Inclusive suffix sum over the 16 lanes of each DPP row.
__device__ __forceinline__ float row_suffix16(float x) {
    x += row_shl<1>(x);
    x += row_shl<2>(x);
    x += row_shl<4>(x);
    x += row_shl<8>(x);
    return x;
}

// Precision of a product in this kernel.  The gate gradient is a difference of terms of
// similar size (the query side minus the key side, per element), so operand rounding
// in them is amplified in dg and further in dA_log and dt_bias, which sum dg over
// tokens.  With every operand rounded to bf16 the error of dg is about 1e-2 relative;
// kMmaSplit writes each fp32 operand as hi + lo, hi = bf16(x) and lo = bf16(x - hi),
// and forms hi*hi + hi*lo + lo*hi on the bf16 matrix cores (the dropped lo*lo term is
// about 2^-16 relative), which brings dg to the level that the forward's own bf16
// rounding leaves.  kMmaF32 uses the fp32 matrix cores (fp32 inputs).
enum { kMmaBf16 = 0, kMmaSplit = 1, kMmaF32 = 2 };

__device__ __forceinline__ void split_bf16(float x, __bf16 &hi, __bf16 &lo) {
    hi = (__bf16)x;
    lo = (__bf16)(x - (float)hi);
}

// 16x16 tile, contraction 32: acc += A(16x32) B(32x16) with a[i], b[i] the lane's
// elements of one k-set (any fixed assignment of the 32 k values to (lane group, i)
// that a and b share).
template <int MP>
__device__ __forceinline__ f32x4 mmap32(f32x4 acc, const float (&a)[8], const float (&b)[8]) {
    if constexpr (MP == kMmaF32) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], acc, 0, 0, 0);
        return acc;
    } else if constexpr (MP == kMmaSplit) {
        bf16x8 ah, al, bh, bl;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __bf16 h, l;
            split_bf16(a[i], h, l);
            ah[i] = h;
            al[i] = l;
            split_bf16(b[i], h, l);
            bh[i] = h;
            bl[i] = l;
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
    } else {
        bf16x8 x, y;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[i] = (__bf16)a[i];
            y[i] = (__bf16)b[i];
        }
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc, 0, 0, 0);
    }
}

// 16x16 tile, contraction 16: acc += A(16x16) B(16x16); a[e] = A[lr][4cg + e],
// b[e] = B[4cg + e][lr].
template <int MP>
__device__ __forceinline__ f32x4 mma16(f32x4 acc, const float (&a)[4], const float (&b)[4]) {
    typedef __attribute__((ext_vector_type(4))) short s16x4;
    if constexpr (MP == kMmaF32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], acc, 0, 0, 0);
        return acc;
    } else if constexpr (MP == kMmaSplit) {
        s16x4 ah, al, bh, bl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            __bf16 h, l;
            split_bf16(a[i], h, l);
            ah[i] = __builtin_bit_cast(short, h);
            al[i] = __builtin_bit_cast(short, l);
            split_bf16(b[i], h, l);
            bh[i] = __builtin_bit_cast(short, h);
            bl[i] = __builtin_bit_cast(short, l);
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, acc, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, acc, 0, 0, 0);
    } else {
        s16x4 x, y;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = (short)f2bf(a[i]);
            y[i] = (short)f2bf(b[i]);
        }
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(x, y, acc, 0, 0, 0);
    }
}

template <int C, int K>
struct LocalLds {
    static constexpr int NB = C / 16, NPAIR = NB * (NB - 1) / 2, KH = K / 2;
    static constexpr int LDM = C + 4, LDK = K + 4, LDV = 36, LDH = KH + 4;
    // tables (whole kernel)
    static constexpr size_t kBeta = 0;                             // [C]
    static constexpr size_t kDBeta = kBeta + C;                     // [C] db from tile-layout terms
    static constexpr size_t kWide = kDBeta + C;                     // [NB] (int)
    static constexpr size_t kGF = kWide + 4 * ((NB + 3) / 4);       // [NB][K] log2 G at a block's first row
    static constexpr size_t kGM = kGF + NB * K;                     // [NB][K] ... at its midpoint row
    static constexpr size_t kGE = kGM + NB * K;                     // [NB][K] ... at its last row
    static constexpr size_t kGL = kGE + NB * K;                     // [K]     ... at the chunk's last row
    static constexpr size_t kSA = kGL + K;                          // [NB][K] 2^(GF - GM)
    static constexpr size_t kSB = kSA + NB * K;                     // [NB][K] 2^(GM - GE)
    static constexpr size_t kSIG = kSB + NB * K;                    // [NPAIR][K] 2^(GF[p] - GE[s])
    static constexpr size_t kTOT = kSIG + NPAIR * K;                // [NB][K] block totals (scan, suffix)
    static constexpr size_t kDD = kTOT + NB * K;                    // [K] rowsum(S_prev o dS)
    static constexpr size_t kDGAM = kDD + K;                        // [NB][K] dgamma partials; [K] the total after
    static constexpr size_t t_end = kDGAM + NB * K;
    // A, A^T (and Akk0 while A is formed), M  [C][LDM]  (phases 1-3)
    static constexpr size_t kAI = (t_end + 3) / 4 * 4;
    static constexpr size_t kAT = kAI + (size_t)C * LDM;
    static constexpr size_t kMM = kAT + (size_t)C * LDM;
    static constexpr size_t kQ = kMM + (size_t)C * LDM;
    // region Q, by phase
    //   1: KC [C][LDK]
    static constexpr size_t kKCS = kQ;
    static constexpr size_t q1 = (size_t)C * LDK;
    //   2: S_prev, dS [K][LDV]; dO, dU, v, Y, V_new [C][LDV]
    static constexpr size_t kSP = kQ, kDS = kSP + (size_t)K * LDV, kDO = kDS + (size_t)K * LDV;
    static constexpr size_t kDU = kDO + (size_t)C * LDV, kVV = kDU + (size_t)C * LDV;
    static constexpr size_t kY = kVV + (size_t)C * LDV, kVN = kY + (size_t)C * LDV;
    static constexpr size_t q2 = 2 * (size_t)K * LDV + 5 * (size_t)C * LDV;
    //   3: dW, X [C][LDK]; dA, then T1 = dA A^T [C][LDM]
    static constexpr size_t kDWS = kQ, kXXS = kDWS + (size_t)C * LDK, kDA = kXXS + (size_t)C * LDK;
    static constexpr size_t q3 = 2 * (size_t)C * LDK + (size_t)C * LDM;
    //   4: QR, KR, KC on one key half [C][LDH]; D1 = dAqk, D2 = dM [C][LDM]
    static constexpr size_t kQRL = kQ, kKRL = kQRL + (size_t)C * LDH, kKCL = kKRL + (size_t)C * LDH;
    static constexpr size_t kD1 = kKCL + (size_t)C * LDH, kD2 = kD1 + (size_t)C * LDM;
    static constexpr size_t q4 = 3 * (size_t)C * LDH + 2 * (size_t)C * LDM;
    static constexpr size_t qmax = q1 > q2 ? (q1 > q3 ? (q1 > q4 ? q1 : q4) : (q3 > q4 ? q3 : q4))
                                           : (q2 > q3 ? (q2 > q4 ? q2 : q4) : (q3 > q4 ? q3 : q4));
    static constexpr size_t floats = kQ + qmax;
    static constexpr size_t bytes = floats * 4;
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

// Four consecutive values as fp32 from storage type T (uint16_t: bf16; float).
template <typename T>
__device__ __forceinline__ float4 load4_t(const void *base, int64_t idx) {
    if constexpr (sizeof(T) == 2) {
        const uint2 u = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(base) + idx);
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                           __uint_as_float(u.y & 0xffff0000u));
    } else {
        return *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + idx);
    }
}

// The gate input and its bias for this lane's NT groups of four columns of one row:
// every load issued before any is used (one dtype branch for the whole row).
template <int NT>
__device__ __forceinline__ void load_gate_row(const Params &p, int64_t grow, int hv, int cg, float4 (&gv)[NT],
                                              float4 (&dbv)[NT]) {
    if (p.g_bf16) {
#pragma unroll
        for (int t = 0; t < NT; ++t) gv[t] = load4_t<uint16_t>(p.g, grow + 16 * t + 4 * cg);
    } else {
#pragma unroll
        for (int t = 0; t < NT; ++t) gv[t] = load4_t<float>(p.g, grow + 16 * t + 4 * cg);
    }
    if (p.dt_bias && p.gate_mode != kGatePre) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            dbv[t] = *reinterpret_cast<const float4 *>(p.dt_bias + (int64_t)hv * p.K + 16 * t + 4 * cg);
    } else {
#pragma unroll
        for (int t = 0; t < NT; ++t) dbv[t] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

template <int C, typename T, int NKK>
__global__ void __launch_bounds__(C / 16 * 64) bwd_local_kernel(BwdChunkParams P) {
    constexpr int MP = sizeof(T) == 4 ? kMmaF32 : kMmaSplit;
    constexpr int K = 32 * NKK, NB = C / 16, NT = K / 16, NTH = NT / 2;
    using L_ = LocalLds<C, K>;
    constexpr int LDM = L_::LDM, LDK = L_::LDK, LDV = L_::LDV, LDH = L_::LDH;
    const Params &p = P.f;
    const BwdParams &bp = P.b;
    extern __shared__ __align__(16) float sm[];
    float *betas = sm + L_::kBeta, *DBETA = sm + L_::kDBeta;
    int *wideflag = reinterpret_cast<int *>(sm + L_::kWide);
    float *GF = sm + L_::kGF, *GM = sm + L_::kGM, *GE = sm + L_::kGE, *GL = sm + L_::kGL;
    float *SA = sm + L_::kSA, *SB = sm + L_::kSB, *SIG = sm + L_::kSIG, *TOT = sm + L_::kTOT;
    float *DD = sm + L_::kDD, *DGAM = sm + L_::kDGAM;
    float *AI = sm + L_::kAI, *AT = sm + L_::kAT, *MM = sm + L_::kMM;
    auto pair_of = [](int pb, int sb) { return pb * (pb - 1) / 2 + sb; };

    const int hv = blockIdx.x % p.HV, gc = blockIdx.x / p.HV;
    const int hq = hv / p.group;
    const ChunkInfo ci = chunk_info(p, gc);
    const size_t slot = (size_t)gc * p.HV + hv;
    const int V = p.V;
    const int w = threadIdx.x >> 6, l = lane_id(), lr = l & 15, cg = l >> 4;
    const int i = 16 * w + lr;  // this lane's chunk row
    const bool valid = i < ci.L;
    const int il = valid ? i : ci.L - 1;
    const int64_t tok = ci.tok0 + il;

    for (int e = threadIdx.x; e < C; e += blockDim.x) DBETA[e] = 0.f;
    for (int e = threadIdx.x; e < K; e += blockDim.x) DD[e] = 0.f;
    if (threadIdx.x < NB) wideflag[threadIdx.x] = 0;

    // ---- phase 0: q^, k^, the log2 cumulative gate G2 (T layout), beta ----
    float qh[NT][4], kh[NT][4], G2[NT][4];
    {
        float ssq = 0.f, ssk = 0.f;
        const int64_t qrow = (tok * p.H + hq) * (int64_t)K, grow = (tok * p.HV + hv) * (int64_t)K;
        const float a = p.A_log ? expf(p.A_log[hv]) : 1.f;
        const float unit = valid ? kLog2e : 0.f;
        float4 qv[NT], kv[NT], gv[NT], dbv[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            qv[t] = load4_t<T>(p.q, qrow + 16 * t + 4 * cg);
            kv[t] = load4_t<T>(p.k, qrow + 16 * t + 4 * cg);
        }
        load_gate_row<NT>(p, grow, hv, cg, gv, dbv);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float qa[4] = {qv[t].x, qv[t].y, qv[t].z, qv[t].w}, ka[4] = {kv[t].x, kv[t].y, kv[t].z, kv[t].w};
            const float ga[4] = {gv[t].x, gv[t].y, gv[t].z, gv[t].w}, ba[4] = {dbv[t].x, dbv[t].y, dbv[t].z, dbv[t].w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                qh[t][jj] = qa[jj];
                kh[t][jj] = ka[jj];
                ssq += qa[jj] * qa[jj];
                ssk += ka[jj] * ka[jj];
                G2[t][jj] = gate_act(p.gate_mode, ga[jj], ba[jj], a, p.lower_bound, unit);
            }
        }
        float rq = p.scale, rk = 1.f;
        if (p.qk_l2norm) {
            ssq = sum_col_groups(ssq);
            ssk = sum_col_groups(ssk);
            rq *= rsqrtf(ssq + 1e-6f);
            rk = rsqrtf(ssk + 1e-6f);
        }
        if (!valid) rq = rk = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                qh[t][jj] *= rq;
                kh[t][jj] *= rk;
                G2[t][jj] = row_scan16(G2[t][jj]);
            }
        if (lr == 15) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
                *reinterpret_cast<float4 *>(TOT + w * K + 16 * t + 4 * cg) = make_float4(G2[t][0], G2[t][1], G2[t][2], G2[t][3]);
        }
        if (cg == 0) betas[i] = valid ? beta_act(p.beta_mode, load_any(p.beta, tok * p.HV + hv, p.beta_bf16)) : 0.f;
    }
    __syncthreads();
    {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                float pre = 0.f;
                for (int bb = 0; bb < w; ++bb) pre += TOT[bb * K + 16 * t + 4 * cg + jj];
                G2[t][jj] += pre;
            }
        int e_loc = ci.L - 1 - 16 * w;
        e_loc = e_loc > 15 ? 15 : (e_loc < 0 ? 0 : e_loc);
        const int m_loc = e_loc < 8 ? e_loc : 8;
        const bool last_here = 16 * w + e_loc == ci.L - 1;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float4 gv = make_float4(G2[t][0], G2[t][1], G2[t][2], G2[t][3]);
            const int d0 = 16 * t + 4 * cg;
            if (lr == 0) *reinterpret_cast<float4 *>(GF + w * K + d0) = gv;
            if (lr == m_loc) *reinterpret_cast<float4 *>(GM + w * K + d0) = gv;
            if (lr == e_loc) {
                *reinterpret_cast<float4 *>(GE + w * K + d0) = gv;
                if (last_here) *reinterpret_cast<float4 *>(GL + d0) = gv;
            }
        }
    }
    __syncthreads();
    for (int d = threadIdx.x; d < K; d += blockDim.x) {
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
            const float gf = GF[bb * K + d], gm = GM[bb * K + d], ge = GE[bb * K + d];
            if (fabsf(gf - gm) > kDiagSpanLimit || fabsf(gm - ge) > kDiagSpanLimit) wideflag[bb] = 1;
            SA[bb * K + d] = fast_exp2(gf - gm);
            SB[bb * K + d] = fast_exp2(gm - ge);
        }
#pragma unroll
        for (int pb = 1; pb < NB; ++pb)
#pragma unroll
            for (int sb = 0; sb < pb; ++sb) SIG[pair_of(pb, sb) * K + d] = fast_exp2(GF[pb * K + d] - GE[sb * K + d]);
    }
    // KC = k^ 2^(GE - G2) of this wave's rows -> LDS, for the other blocks' pair products
    float *KCS = sm + L_::kKCS;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int d0 = 16 * t + 4 * cg;
        float kc[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) kc[jj] = kh[t][jj] * fast_exp2(GE[w * K + d0 + jj] - G2[t][jj]);
        *reinterpret_cast<float4 *>(KCS + i * LDK + d0) = make_float4(kc[0], kc[1], kc[2], kc[3]);
    }
    __syncthreads();
    const bool wide = wideflag[w] != 0;
    const float b_i = betas[i];

    // ---- phase 1: M = strict-lower k^ k^T e^(G_i - G_j) (row block w), Akk0 = b M, A ----
    {
        f32x4 accM[NB];
#pragma unroll
        for (int s = 0; s < NB; ++s) accM[s] = zero4();
        // row operand KR = k^ 2^(G2 - GF) (this lane's row), permuted contraction sets
        float KR[NT][4];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) KR[t][jj] = kh[t][jj] * fast_exp2(G2[t][jj] - GF[w * K + 16 * t + 4 * cg + jj]);
#pragma unroll
        for (int s = 0; s < NB; ++s) {
            if (s < w) {
                const float *sg = SIG + pair_of(w, s) * K;
#pragma unroll
                for (int m = 0; m < NT / 2; ++m) {
                    float a[8], bk[8];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int d0 = 32 * m + 16 * hh + 4 * cg;
                        const float4 kc = *reinterpret_cast<const float4 *>(KCS + (16 * s + lr) * LDK + d0);
                        const float4 sgv = *reinterpret_cast<const float4 *>(sg + d0);
                        a[4 * hh + 0] = kc.x * sgv.x, a[4 * hh + 1] = kc.y * sgv.y;
                        a[4 * hh + 2] = kc.z * sgv.z, a[4 * hh + 3] = kc.w * sgv.w;
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) bk[4 * hh + jj] = KR[2 * m + hh][jj];
                    }
                    accM[s] = mmap32<MP>(accM[s], a, bk);
                }
            }
        }
        if (!wide) {
#pragma unroll
            for (int m = 0; m < NT / 2; ++m) {
                float a[8], bk[8];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int t = 2 * m + hh, d0 = 16 * t + 4 * cg;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        a[4 * hh + jj] = KCS[i * LDK + d0 + jj] * SB[w * K + d0 + jj];
                        bk[4 * hh + jj] = KR[t][jj] * SA[w * K + d0 + jj];
                    }
                }
                accM[w] = mmap32<MP>(accM[w], a, bk);
            }
        } else {
            // element-wise diagonal block: sum_d k^_id k^_jd 2^(G_id - G_jd), j < i
            for (int jr = 0; jr < 16; ++jr) {
                float sk = 0.f;
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const float kj = shfl(kh[t][jj], (l & 0x30) + jr);
                        const float gj = shfl(G2[t][jj], (l & 0x30) + jr);
                        sk += lr > jr ? kh[t][jj] * kj * fast_exp2(G2[t][jj] - gj) : 0.f;
                    }
                sk = sum_col_groups(sk);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    if (4 * cg + jj == jr) accM[w][jj] = sk;
            }
        }
        // lane: row i, columns 16s + 4cg + jj; strict lower
#pragma unroll
        for (int s = 0; s < NB; ++s) {
            float mv[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) mv[jj] = (s < w || (s == w && 4 * cg + jj < lr)) ? accM[s][jj] : 0.f;
            *reinterpret_cast<float4 *>(MM + i * LDM + 16 * s + 4 * cg) = make_float4(mv[0], mv[1], mv[2], mv[3]);
            *reinterpret_cast<float4 *>(AT + i * LDM + 16 * s + 4 * cg) =
                make_float4(b_i * mv[0], b_i * mv[1], b_i * mv[2], b_i * mv[3]);  // Akk0 while A is formed
        }
    }
    __syncthreads();
    {
        // A = (I + Akk0)^-1: diagonal blocks by forward substitution (lane l < 16 of wave w
        // holds column l of block w), then the off-diagonal blocks by distance
        const float *Akk = AT;
        if (l < 16) {
            float col[16];
#pragma unroll
            for (int m = 0; m < 16; ++m) col[m] = (m == l) ? 1.f : 0.f;
            const float *Lb = Akk + (16 * w) * LDM + 16 * w;
#pragma unroll
            for (int r2 = 1; r2 < 16; ++r2) {
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < r2; ++m) acc += Lb[r2 * LDM + m] * col[m];
                if (r2 > l) col[r2] = -acc;
            }
#pragma unroll
            for (int m = 0; m < 16; ++m) AI[(16 * w + m) * LDM + 16 * w + l] = col[m];
        }
        for (int s = w + 1; s < NB; ++s)
            for (int e = l; e < 256; e += 64) AI[(16 * w + (e >> 4)) * LDM + 16 * s + (e & 15)] = 0.f;
        __syncthreads();
#pragma unroll
        for (int dist = 1; dist < NB; ++dist) {
            if (w >= dist) {
                const int s = w - dist;
                f32x4 t = zero4();
                for (int m = s; m < w; ++m)
                    t = mma16_f32_lds(t, Akk + (16 * w) * LDM + 16 * m, LDM, AI + (16 * m) * LDM + 16 * s, LDM);
                const float4 av4 = *reinterpret_cast<const float4 *>(AI + (16 * w + lr) * LDM + 16 * w + 4 * cg);
                const float av[4] = {av4.x, av4.y, av4.z, av4.w};
                f32x4 uu = zero4();
#pragma unroll
                for (int q = 0; q < 4; ++q) uu = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], t[q], uu, 0, 0, 0);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) AI[(16 * w + 4 * cg + jj) * LDM + 16 * s + lr] = -uu[jj];
            }
            __syncthreads();
        }
        // A^T (over the Akk0 copy, which the merges no longer read)
        for (int e = threadIdx.x; e < C * C; e += blockDim.x) {
            const int r2 = e / C, c2 = e % C;
            AT[c2 * LDM + r2] = AI[r2 * LDM + c2];
        }
    }
    __syncthreads();

    // ---- phase 2: state-side products over 32-column blocks of V ----
    float X[NT][4];  // X = b k^ E
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) X[t][jj] = b_i * kh[t][jj] * fast_exp2(G2[t][jj]);
    float dQg[NT][4], dW[NT][4], dKg[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) dQg[t][jj] = dW[t][jj] = dKg[t][jj] = 0.f;
    f32x4 dAq[NB], dA1[NB];
#pragma unroll
    for (int s = 0; s < NB; ++s) dAq[s] = dA1[s] = zero4();
    float dbeta_acc[4] = {0.f, 0.f, 0.f, 0.f};  // rows 16w + 4cg + jj, this lane's columns
    {
        float *SP = sm + L_::kSP, *DS = sm + L_::kDS, *DO = sm + L_::kDO, *DU = sm + L_::kDU;
        float *VV = sm + L_::kVV, *YY = sm + L_::kY, *VN = sm + L_::kVN;
        const float *hs = bp.states + slot * (size_t)K * V;
        const float *dh = P.dh + slot * (size_t)K * V;
        const float *du = P.dU + slot * (size_t)C * V;
        for (int v0 = 0; v0 < V; v0 += 32) {
            // stage (rows past the chunk's end as zeros): every load of the block first
            constexpr int NTHR = 64 * NB, NSD = K * 8 / NTHR, NCV = C * 8 / NTHR;
            static_assert(K * 8 % NTHR == 0 && C * 8 % NTHR == 0, "staging split");
            float4 sp4[NSD], ds4[NSD], do4[NCV], vv4[NCV], du4[NCV];
#pragma unroll
            for (int q = 0; q < NSD; ++q) {
                const int e = threadIdx.x + q * NTHR, d = e >> 3, c4 = 4 * (e & 7);
                sp4[q] = *reinterpret_cast<const float4 *>(hs + (size_t)d * V + v0 + c4);
                ds4[q] = *reinterpret_cast<const float4 *>(dh + (size_t)d * V + v0 + c4);
            }
#pragma unroll
            for (int q = 0; q < NCV; ++q) {
                const int e = threadIdx.x + q * NTHR, r2 = e >> 3, c4 = 4 * (e & 7);
                const int rr = r2 < ci.L ? r2 : ci.L - 1;  // in-bounds row, zeroed below
                const int64_t row = ((ci.tok0 + rr) * p.HV + hv) * (int64_t)V + v0 + c4;
                do4[q] = load4_t<T>(bp.dout, row);
                vv4[q] = load4_t<T>(p.v, row);
                du4[q] = *reinterpret_cast<const float4 *>(du + (size_t)r2 * V + v0 + c4);
            }
#pragma unroll
            for (int q = 0; q < NSD; ++q) {
                const int e = threadIdx.x + q * NTHR, d = e >> 3, c4 = 4 * (e & 7);
                *reinterpret_cast<float4 *>(SP + d * LDV + c4) = sp4[q];
                *reinterpret_cast<float4 *>(DS + d * LDV + c4) = ds4[q];
            }
#pragma unroll
            for (int q = 0; q < NCV; ++q) {
                const int e = threadIdx.x + q * NTHR, r2 = e >> 3, c4 = 4 * (e & 7);
                const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
                *reinterpret_cast<float4 *>(DO + r2 * LDV + c4) = r2 < ci.L ? do4[q] : z;
                *reinterpret_cast<float4 *>(VV + r2 * LDV + c4) = r2 < ci.L ? vv4[q] : z;
                *reinterpret_cast<float4 *>(DU + r2 * LDV + c4) = du4[q];
            }
            __syncthreads();
            // Y = b v - X S_prev (lane: rows 16w + 4cg + jj, column 16vt + lr)
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) {
                f32x4 acc = zero4();
#pragma unroll
                for (int m = 0; m < NT / 2; ++m) {
                    float a[8], bb[8];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            a[4 * hh + jj] = X[2 * m + hh][jj];
                            bb[4 * hh + jj] = SP[(32 * m + 16 * hh + 4 * cg + jj) * LDV + 16 * vt + lr];
                        }
                    acc = mmap32<MP>(acc, a, bb);
                }
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int r2 = 16 * w + 4 * cg + jj;
                    YY[r2 * LDV + 16 * vt + lr] = betas[r2] * VV[r2 * LDV + 16 * vt + lr] - acc[jj];
                }
            }
            if (threadIdx.x < K) {  // rowsum(S_prev o dS) of this block
                const int d = threadIdx.x;
                float sacc = 0.f;
#pragma unroll 8
                for (int c = 0; c < 32; ++c) sacc += SP[d * LDV + c] * DS[d * LDV + c];
                DD[d] += sacc;
            }
            __syncthreads();
            // V_new = A Y (lane: rows 16w + 4cg + jj, column 16vt + lr)
            const int njm = (16 * w + 16 + 31) / 32;
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) {
                f32x4 acc = zero4();
                for (int jm = 0; jm < njm; ++jm) {
                    float a[8], bb[8];
                    load8(AI + (16 * w + lr) * LDM + 32 * jm + 8 * cg, a);
#pragma unroll
                    for (int e = 0; e < 8; ++e) bb[e] = YY[(32 * jm + 8 * cg + e) * LDV + 16 * vt + lr];
                    acc = mmap32<MP>(acc, a, bb);
                }
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) VN[(16 * w + 4 * cg + jj) * LDV + 16 * vt + lr] = acc[jj];
            }
            __syncthreads();
            // dQg^T, dW^T, dKg^T tiles (T layout: rows d = 16t + 4cg + jj, column i = 16w + lr)
            {
                float bo[8], bu[8], bn[8];
                load8(DO + (16 * w + lr) * LDV + 8 * cg, bo);
                load8(DU + (16 * w + lr) * LDV + 8 * cg, bu);
                load8(VN + (16 * w + lr) * LDV + 8 * cg, bn);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    float as[8], ad[8];
                    load8(SP + (16 * t + lr) * LDV + 8 * cg, as);
                    load8(DS + (16 * t + lr) * LDV + 8 * cg, ad);
                    f32x4 q4 = {dQg[t][0], dQg[t][1], dQg[t][2], dQg[t][3]};
                    f32x4 w4 = {dW[t][0], dW[t][1], dW[t][2], dW[t][3]};
                    f32x4 k4 = {dKg[t][0], dKg[t][1], dKg[t][2], dKg[t][3]};
                    q4 = mmap32<MP>(q4, as, bo);
                    w4 = mmap32<MP>(w4, as, bu);
                    k4 = mmap32<MP>(k4, ad, bn);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        dQg[t][jj] = q4[jj];
                        dW[t][jj] = w4[jj];  // (sign applied after the last block)
                        dKg[t][jj] = k4[jj];
                    }
                }
                // dAqk = dO V_new^T, dA1 = dU (b v)^T (tiles s <= w; lane: rows 16w + 4cg + jj,
                // column 16s + lr)
#pragma unroll
                for (int s = 0; s < NB; ++s) {
                    if (s <= w) {
                        float bvn[8], bvv[8];
                        load8(VN + (16 * s + lr) * LDV + 8 * cg, bvn);
                        load8(VV + (16 * s + lr) * LDV + 8 * cg, bvv);
                        const float bj = betas[16 * s + lr];
#pragma unroll
                        for (int e = 0; e < 8; ++e) bvv[e] *= bj;
                        float ao[8], au[8];
                        load8(DO + (16 * w + lr) * LDV + 8 * cg, ao);
                        load8(DU + (16 * w + lr) * LDV + 8 * cg, au);
                        dAq[s] = mmap32<MP>(dAq[s], ao, bvn);
                        dA1[s] = mmap32<MP>(dA1[s], au, bvv);
                    }
                }
            }
            // A^T dU (lane: rows 16w + 4cg + jj, column 16vt + lr): dv and the v term of db
            const int jm0 = (16 * w) / 32;
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) {
                f32x4 acc = zero4();
                for (int jm = jm0; jm < C / 32; ++jm) {
                    float a[8], bb[8];
                    load8(AT + (16 * w + lr) * LDM + 32 * jm + 8 * cg, a);
#pragma unroll
                    for (int e = 0; e < 8; ++e) bb[e] = DU[(32 * jm + 8 * cg + e) * LDV + 16 * vt + lr];
                    acc = mmap32<MP>(acc, a, bb);
                }
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int r2 = 16 * w + 4 * cg + jj;
                    if (r2 < ci.L)
                        bp.dv[((ci.tok0 + r2) * p.HV + hv) * (int64_t)V + v0 + 16 * vt + lr] = betas[r2] * acc[jj];
                    dbeta_acc[jj] += VV[r2 * LDV + 16 * vt + lr] * acc[jj];
                }
            }
            __syncthreads();  // the next block's staging overwrites these buffers
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) dW[t][jj] = -dW[t][jj];
    // db from the v term: rows 16w + 4cg + jj, summed over the 16 columns of the DPP row
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const float s = row_sum16_all(dbeta_acc[jj]);
        if (lr == 0) DBETA[16 * w + 4 * cg + jj] += s;
    }

    // ---- phase 3: the WY chain: dX = A^T dW, dA = dU (b v)^T + dW X^T, dAkk0, dM ----
    float dX[NT][4];
    f32x4 dMt[NB];
    {
        float *DWS = sm + L_::kDWS, *XXS = sm + L_::kXXS, *DA = sm + L_::kDA;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            *reinterpret_cast<float4 *>(DWS + i * LDK + 16 * t + 4 * cg) = make_float4(dW[t][0], dW[t][1], dW[t][2], dW[t][3]);
            *reinterpret_cast<float4 *>(XXS + i * LDK + 16 * t + 4 * cg) = make_float4(X[t][0], X[t][1], X[t][2], X[t][3]);
        }
        __syncthreads();
        // dX^T tiles (T layout): sum over rows j >= 16w of dW[j][d] A[j][i]
        const int jm0 = (16 * w) / 32;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            f32x4 acc = zero4();
            for (int jm = jm0; jm < C / 32; ++jm) {
                float a[8], bb[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] = DWS[(32 * jm + 8 * cg + e) * LDK + 16 * t + lr];
                load8(AT + (16 * w + lr) * LDM + 32 * jm + 8 * cg, bb);
                acc = mmap32<MP>(acc, a, bb);
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) dX[t][jj] = acc[jj];
        }
        // dA2 = dW X^T (tiles s <= w), dA = mask(dA1 + dA2) strictly lower -> LDS
#pragma unroll
        for (int s = 0; s < NB; ++s) {
            f32x4 dA = zero4();
            if (s <= w) {
                f32x4 acc = dA1[s];
#pragma unroll
                for (int m = 0; m < NT / 2; ++m) {
                    float a[8], bb[8];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const float4 xv = *reinterpret_cast<const float4 *>(XXS + (16 * s + lr) * LDK + 32 * m + 16 * hh + 4 * cg);
                        bb[4 * hh + 0] = xv.x, bb[4 * hh + 1] = xv.y, bb[4 * hh + 2] = xv.z, bb[4 * hh + 3] = xv.w;
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) a[4 * hh + jj] = dW[2 * m + hh][jj];
                    }
                    acc = mmap32<MP>(acc, a, bb);
                }
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) dA[jj] = (s < w || lr < 4 * cg + jj) ? acc[jj] : 0.f;
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) DA[(16 * w + 4 * cg + jj) * LDM + 16 * s + lr] = dA[jj];
        }
        __syncthreads();
        // T1 = dA A^T on this wave's rows (all column blocks), then over its own rows of dA
        f32x4 T1[NB];
        const int njm = (16 * w + 16 + 31) / 32;
#pragma unroll
        for (int lb = 0; lb < NB; ++lb) {
            T1[lb] = zero4();
            for (int jm = 0; jm < njm; ++jm) {
                float a[8], bb[8];
                load8(DA + (16 * w + lr) * LDM + 32 * jm + 8 * cg, a);
                load8(AI + (16 * lb + lr) * LDM + 32 * jm + 8 * cg, bb);
                T1[lb] = mmap32<MP>(T1[lb], a, bb);
            }
        }
        // (each wave read only its own rows of dA above; the LDS reads complete in order
        // before these writes of the same rows)
#pragma unroll
        for (int lb = 0; lb < NB; ++lb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) DA[(16 * w + 4 * cg + jj) * LDM + 16 * lb + lr] = T1[lb][jj];
        __syncthreads();
        // dAkk0 = -A^T T1 (rows 16w.., column blocks lb <= w), strictly lower; dM = b dAkk0;
        // db from rowsum(dAkk0 o M)
        const int im0 = (16 * w) / 32;
        float dbm[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int lb = 0; lb < NB; ++lb) {
            dMt[lb] = zero4();
            if (lb <= w) {
                f32x4 acc = zero4();
                for (int im = im0; im < C / 32; ++im) {
                    float a[8], bb[8];
                    load8(AT + (16 * w + lr) * LDM + 32 * im + 8 * cg, a);
#pragma unroll
                    for (int e = 0; e < 8; ++e) bb[e] = DA[(32 * im + 8 * cg + e) * LDM + 16 * lb + lr];
                    acc = mmap32<MP>(acc, a, bb);
                }
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int r2 = 16 * w + 4 * cg + jj, c2 = 16 * lb + lr;
                    const float dak = (r2 > c2) ? -acc[jj] : 0.f;
                    dbm[jj] += dak * MM[r2 * LDM + c2];
                    dMt[lb][jj] = betas[r2] * dak;
                }
            }
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float s = row_sum16_all(dbm[jj]);
            if (lr == 0) DBETA[16 * w + 4 * cg + jj] += s;
        }
    }
    __syncthreads();  // region Q is rewritten below

    // ---- phase 4: per-element terms, the pairwise terms of Aqk and M, dgamma, suffix sum ----
    float *QRL = sm + L_::kQRL, *KRL = sm + L_::kKRL, *KCL = sm + L_::kKCL;
    float *D1 = sm + L_::kD1, *D2 = sm + L_::kD2;
#pragma unroll
    for (int s = 0; s < NB; ++s)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int r2 = 16 * w + 4 * cg + jj, c2 = 16 * s + lr;
            D1[r2 * LDM + c2] = (s <= w && c2 <= r2) ? dAq[s][jj] : 0.f;
            D2[r2 * LDM + c2] = (s <= w) ? dMt[s][jj] : 0.f;
        }
    float dqh[NT][4], dkh[NT][4], dG[NT][4];
    float db3 = 0.f;
    {
        float gam[NT][4];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d = 16 * t + 4 * cg + jj;
                const float E = fast_exp2(G2[t][jj]), F = fast_exp2(GL[d] - G2[t][jj]);
                dqh[t][jj] = dQg[t][jj] * E;
                dkh[t][jj] = dKg[t][jj] * F + b_i * dX[t][jj] * E;
                dG[t][jj] = dQg[t][jj] * qh[t][jj] * E - dKg[t][jj] * kh[t][jj] * F + b_i * dX[t][jj] * kh[t][jj] * E;
                gam[t][jj] = row_sum16_all(dKg[t][jj] * kh[t][jj] * F);
                db3 += dX[t][jj] * kh[t][jj] * E;
            }
        if (lr == 0) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
                *reinterpret_cast<float4 *>(DGAM + w * K + 16 * t + 4 * cg) = make_float4(gam[t][0], gam[t][1], gam[t][2], gam[t][3]);
        }
        db3 = sum_col_groups(db3);
    }
    // pairwise terms, one key half at a time (QR, KR, KC of every block through LDS)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        __syncthreads();  // D1, D2 written; the previous half's operands no longer read
#pragma unroll
        for (int tl = 0; tl < NTH; ++tl) {
            const int t = NTH * hh + tl, d0 = 16 * t + 4 * cg;
            float qr[4], kr[4], kc[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float rf = fast_exp2(G2[t][jj] - GF[w * K + d0 + jj]);
                qr[jj] = qh[t][jj] * rf;
                kr[jj] = kh[t][jj] * rf;
                kc[jj] = kh[t][jj] * fast_exp2(GE[w * K + d0 + jj] - G2[t][jj]);
            }
            *reinterpret_cast<float4 *>(QRL + i * LDH + 16 * tl + 4 * cg) = make_float4(qr[0], qr[1], qr[2], qr[3]);
            *reinterpret_cast<float4 *>(KRL + i * LDH + 16 * tl + 4 * cg) = make_float4(kr[0], kr[1], kr[2], kr[3]);
            *reinterpret_cast<float4 *>(KCL + i * LDH + 16 * tl + 4 * cg) = make_float4(kc[0], kc[1], kc[2], kc[3]);
        }
        __syncthreads();
#pragma unroll
        for (int tl = 0; tl < NTH; ++tl) {
            const int t = NTH * hh + tl;
            // row role (rows i of block w): R1 = sum_j dAqk[i][j] k^_jd e^(G_i - G_j), R2 likewise with dM
            f32x4 r1 = zero4(), r2 = zero4();
#pragma unroll
            for (int s = 0; s < NB; ++s) {
                if (s <= w && !(s == w && wide)) {
                    float a[4], b1[4], b2[4];
                    const float sbd = (s == w) ? SB[w * K + 16 * t + lr] : 1.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        a[e] = KCL[(16 * s + 4 * cg + e) * LDH + 16 * tl + lr] * sbd;
                        b1[e] = D1[(16 * w + lr) * LDM + 16 * s + 4 * cg + e];
                        b2[e] = D2[(16 * w + lr) * LDM + 16 * s + 4 * cg + e];
                    }
                    const f32x4 t1 = mma16<MP>(zero4(), a, b1), t2 = mma16<MP>(zero4(), a, b2);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int d = 16 * t + 4 * cg + jj;
                        const float f = (s == w) ? SA[w * K + d] : SIG[pair_of(w, s) * K + d];
                        r1[jj] += f * t1[jj];
                        r2[jj] += f * t2[jj];
                    }
                }
            }
            // column role (rows j of block w): C1 = sum_i dAqk[i][j] q^_id e^(G_i - G_j), C2 with dM, k^
            f32x4 c1 = zero4(), c2 = zero4();
#pragma unroll
            for (int pb = 0; pb < NB; ++pb) {
                if (pb >= w && !(pb == w && wide)) {
                    float aq[4], ak[4], b1[4], b2[4];
                    const float sad = (pb == w) ? SA[w * K + 16 * t + lr] : 1.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        aq[e] = QRL[(16 * pb + 4 * cg + e) * LDH + 16 * tl + lr] * sad;
                        ak[e] = KRL[(16 * pb + 4 * cg + e) * LDH + 16 * tl + lr] * sad;
                        b1[e] = D1[(16 * pb + 4 * cg + e) * LDM + 16 * w + lr];
                        b2[e] = D2[(16 * pb + 4 * cg + e) * LDM + 16 * w + lr];
                    }
                    const f32x4 t1 = mma16<MP>(zero4(), aq, b1), t2 = mma16<MP>(zero4(), ak, b2);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int d = 16 * t + 4 * cg + jj;
                        const float f = (pb == w) ? SB[w * K + d] : SIG[pair_of(pb, w) * K + d];
                        c1[jj] += f * t1[jj];
                        c2[jj] += f * t2[jj];
                    }
                }
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d = 16 * t + 4 * cg + jj;
                const float rf = fast_exp2(G2[t][jj] - GF[w * K + d]);
                const float cf = fast_exp2(GE[w * K + d] - G2[t][jj]);
                float R1 = rf * r1[jj], R2 = rf * r2[jj], C1 = cf * c1[jj], C2 = cf * c2[jj];
                if (wide) {
                    // element-wise diagonal block: exponents G_i - G_j <= 0 taken directly
                    for (int o = 0; o < 16; ++o) {
                        const float ko = shfl(kh[t][jj], (l & 0x30) + o), qo = shfl(qh[t][jj], (l & 0x30) + o);
                        const float go = shfl(G2[t][jj], (l & 0x30) + o);
                        if (o <= lr) {  // j = o <= i = lr: row role
                            const float f = fast_exp2(G2[t][jj] - go);
                            R1 += D1[(16 * w + lr) * LDM + 16 * w + o] * ko * f;
                            R2 += D2[(16 * w + lr) * LDM + 16 * w + o] * ko * f;
                        }
                        if (o >= lr) {  // i = o >= j = lr: column role
                            const float f = fast_exp2(go - G2[t][jj]);
                            C1 += D1[(16 * w + o) * LDM + 16 * w + lr] * qo * f;
                            C2 += D2[(16 * w + o) * LDM + 16 * w + lr] * ko * f;
                        }
                    }
                }
                dqh[t][jj] += R1;
                dkh[t][jj] += R2 + C1 + C2;
                dG[t][jj] += qh[t][jj] * R1 + kh[t][jj] * R2 - kh[t][jj] * (C1 + C2);
            }
        }
    }
    __syncthreads();  // DGAM complete
    for (int d = threadIdx.x; d < K; d += blockDim.x) {
        float s = DD[d] * fast_exp2(GL[d]);
        for (int bb = 0; bb < NB; ++bb) s += DGAM[bb * K + d];
        TOT[d] = s;  // dgamma (TOT's scan totals are no longer needed)
    }
    __syncthreads();
    // dgamma at the chunk's last row, rows past the end zero, then the suffix sum over rows
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            if (i == ci.L - 1) dG[t][jj] += TOT[16 * t + 4 * cg + jj];
            if (!valid) dG[t][jj] = 0.f;
            dG[t][jj] = row_suffix16(dG[t][jj]);
        }
    __syncthreads();  // TOT read
    if (lr == 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            *reinterpret_cast<float4 *>(TOT + w * K + 16 * t + 4 * cg) = make_float4(dG[t][0], dG[t][1], dG[t][2], dG[t][3]);
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            float suf = 0.f;
            for (int bb = w + 1; bb < NB; ++bb) suf += TOT[bb * K + 16 * t + 4 * cg + jj];
            dG[t][jj] += suf;
        }
    // the gate's chain rule (dg w.r.t. the g given), this chunk's sums for dt_bias and
    // A_log, and dbeta through the beta transform
    const size_t o = (size_t)tok * p.HV + hv;
    const float a_h = p.A_log ? expf(p.A_log[hv]) : 1.f;
    float sda = 0.f;
    {
        float4 gv[NT], dbv[NT];
        load_gate_row<NT>(p, (int64_t)o * K, hv, cg, gv, dbv);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float ga[4] = {gv[t].x, gv[t].y, gv[t].z, gv[t].w}, ba[4] = {dbv[t].x, dbv[t].y, dbv[t].z, dbv[t].w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                float da;
                dG[t][jj] = gate_act_grad(p.gate_mode, valid ? dG[t][jj] : 0.f, ga[jj], ba[jj], a_h, p.lower_bound, da);
                sda += da;
            }
        }
    }
    if (valid) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int d0 = 16 * t + 4 * cg;
            *reinterpret_cast<float4 *>(bp.p_dq + o * K + d0) = make_float4(dqh[t][0], dqh[t][1], dqh[t][2], dqh[t][3]);
            *reinterpret_cast<float4 *>(bp.p_dk + o * K + d0) = make_float4(dkh[t][0], dkh[t][1], dkh[t][2], dkh[t][3]);
            *reinterpret_cast<float4 *>(bp.dg + o * K + d0) = make_float4(dG[t][0], dG[t][1], dG[t][2], dG[t][3]);
        }
        if (cg == 0) {
            float dbv = DBETA[i] + db3;
            if (p.beta_mode != kBetaGiven) {
                const float s = 1.f / (1.f + expf(-load_any(p.beta, (int64_t)o, p.beta_bf16)));
                dbv *= (p.beta_mode == kBetaTwoSigmoid ? 2.f : 1.f) * s * (1.f - s);
            }
            bp.dbeta[o] = dbv;
        }
    }
    if (p.gate_mode != kGatePre) {
        // column sums over the chunk's rows (rows past the end hold dg = 0), then over waves
        __syncthreads();  // TOT's suffix totals read
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float cs = row_sum16_all(dG[t][jj]);
                if (lr == 0) TOT[w * K + 16 * t + 4 * cg + jj] = cs;
            }
        sda = sum_col_groups(row_sum16_all(sda));
        if (l == 0) DGAM[w] = sda;
        __syncthreads();
        float *part = P.cparam + slot * (K + 1);
        for (int d = threadIdx.x; d <= K; d += blockDim.x) {
            float acc = 0.f;
            if (d < K) {
                for (int bb = 0; bb < NB; ++bb) acc += TOT[bb * K + d];
            } else {
                for (int bb = 0; bb < NB; ++bb) acc += DGAM[bb];
            }
            part[d] = acc;
        }
    }
}

}  // namespace kda
