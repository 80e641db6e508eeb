// kda_bwd_local2.h -- the per-chunk gradients of the KDA backward for bf16 inputs: the
// same quantities, in the same order, as bwd_local_kernel (kda_bwd_local.h, which holds
// the formulas and the fp32 form), with operands staged once in LDS as split bf16.
//
// Every fp32 operand of a product is written to LDS as two bf16 planes, hi = bf16(x) and
// lo = bf16(x - hi), laid out so that the contraction index is contiguous for each use,
// and the products read whole fragments (8 or 4 bf16 per lane) from both planes: hi*hi +
// hi*lo + lo*hi on the bf16 matrix cores (bf16 inputs such as dO and v are exact and
// take one plane).  Splitting once per element instead of at every use removes most of
// the vector work of the fp32 form's operand conversions.  An accumulator tile (lane:
// rows 4cg + jj, column lr) is written to the transposed matrix as four contiguous
// values, so a product whose result is needed with a given contiguous index is formed
// as the transposed product where that helps.
//
// Phases as in bwd_local_kernel:
//   0, 1  q^, k^, G (T layout), the block tables, M, A = (I + Diag(b) M)^-1 (fp32); A and
//         A^T are then kept as split planes.
//   2     per 32-column block of V: S_prev (both orientations) and v staged,
//         Y = b v - X S_prev (X from registers, pre-split), V_new^T = Y^T A^T; then dS,
//         dO, dU, dU^T staged over S_prev^T and Y^T, and dQg^T, dW^T, dKg^T (T layout
//         accumulators), dAqk, dU (b v)^T and (A^T dU)^T (for dv and db) formed.
//   3     the WY chain (fp32 staging of dW, X, dA as in the fp32 form; A, A^T split).
//   4     the pairwise terms with Kc^T, Qr^T, Kr^T (one key half at a time) and dAqk, dM
//         in both orientations as split planes; the block factors are applied to the
//         products' rows.
#pragma once

#include "kda_bwd_local.h"

namespace kda {

// hi = bf16(x), lo = bf16(x - hi), packed in pairs (element 2e in the low half).
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t &h, uint32_t &l) {
    const uint16_t h0 = f2bf(x0), h1 = f2bf(x1);
    h = (uint32_t)h0 | ((uint32_t)h1 << 16);
    l = (uint32_t)f2bf(x0 - bf2f(h0)) | ((uint32_t)f2bf(x1 - bf2f(h1)) << 16);
}
__device__ __forceinline__ void split_store1(uint16_t *hp, uint16_t *lp, int idx, float x) {
    const uint16_t h = f2bf(x);
    hp[idx] = h;
    lp[idx] = f2bf(x - bf2f(h));
}
// four consecutive elements (8 bytes per plane)
__device__ __forceinline__ void split_store4(uint16_t *hp, uint16_t *lp, int idx, float x0, float x1, float x2,
                                             float x3) {
    uint32_t h0, l0, h1, l1;
    split_pair(x0, x1, h0, l0);
    split_pair(x2, x3, h1, l1);
    *reinterpret_cast<uint2 *>(hp + idx) = make_uint2(h0, h1);
    *reinterpret_cast<uint2 *>(lp + idx) = make_uint2(l0, l1);
}
__device__ __forceinline__ float split_load1(const uint16_t *hp, const uint16_t *lp, int idx) {
    return bf2f(hp[idx]) + bf2f(lp[idx]);
}

// 16x16x32 products of split operands (3 instructions), or with one exact operand (2).
__device__ __forceinline__ f32x4 mma32_ss(f32x4 acc, uint4 ah, uint4 al, uint4 bh, uint4 bl) {
    acc = mma32_bf16(acc, al, bh);
    acc = mma32_bf16(acc, ah, bl);
    return mma32_bf16(acc, ah, bh);
}
__device__ __forceinline__ f32x4 mma32_se(f32x4 acc, uint4 ah, uint4 al, uint4 b) {
    acc = mma32_bf16(acc, al, b);
    return mma32_bf16(acc, ah, b);
}
__device__ __forceinline__ f32x4 mma32_es(f32x4 acc, uint4 a, uint4 bh, uint4 bl) {
    acc = mma32_bf16(acc, a, bl);
    return mma32_bf16(acc, a, bh);
}
// 16x16x32 with one fp32 operand split here (a) and one pre-split (b), or the reverse.
__device__ __forceinline__ void split8(const float (&x)[8], uint4 &h, uint4 &l) {
    split_pair(x[0], x[1], h.x, l.x);
    split_pair(x[2], x[3], h.y, l.y);
    split_pair(x[4], x[5], h.z, l.z);
    split_pair(x[6], x[7], h.w, l.w);
}
__device__ __forceinline__ f32x4 mma32_fs(f32x4 acc, const float (&a)[8], uint4 bh, uint4 bl) {
    uint4 ah, al;
    split8(a, ah, al);
    return mma32_ss(acc, ah, al, bh, bl);
}
__device__ __forceinline__ f32x4 mma32_sf(f32x4 acc, uint4 ah, uint4 al, const float (&b)[8]) {
    uint4 bh, bl;
    split8(b, bh, bl);
    return mma32_ss(acc, ah, al, bh, bl);
}
// 16x16x16 product of split operands (4 bf16 per lane and plane).
__device__ __forceinline__ f32x4 mma16_ss(f32x4 acc, uint2 ah, uint2 al, uint2 bh, uint2 bl) {
    typedef __attribute__((ext_vector_type(4))) short s16x4;
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, al), __builtin_bit_cast(s16x4, bh), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, ah), __builtin_bit_cast(s16x4, bl), acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, ah), __builtin_bit_cast(s16x4, bh), acc, 0, 0, 0);
}

// The chunk-start state, the state gradient and dU arrive in the fragment order of the
// recurrences that wrote them: within a (chunk, value head) block of R rows and V
// columns, float4 index (vs * 2 + j) * (R / 16) * 64 + f' with f' = t * 64 + lane holds
// rows 16t + 4cg .. +3 of one column of the 32-column slice vs.  frag_rows_col gives,
// for the float4 index f within a slice, its first row and its column in the slice:
// the forward recurrence's state waves hold column 8 (lr / 4) + 4 j + lr % 4 (HM =
// false), the reverse recurrence's column 16 j + lr (HM = true).
template <int R, bool HM>
__device__ __forceinline__ void frag_rows_col(int f, int &row0, int &col) {
    const int ln = f & 63, tj = f >> 6, t = tj % (R / 16), j = tj / (R / 16), lr = ln & 15;
    row0 = 16 * t + 4 * (ln >> 4);
    col = HM ? 16 * j + lr : 8 * (lr >> 2) + 4 * j + (lr & 3);
}

template <int C, int K>
struct LocalLds2 {
    static constexpr int NB = C / 16, NPAIR = NB * (NB - 1) / 2, KH = K / 2;
    static constexpr int LDM = C + 4, LDK = K + 4;                 // fp32 rows
    static constexpr int LB32 = 40, LBC = C + 8, LBK = K + 8;      // bf16 plane rows
    // tables (floats), as in the fp32 form
    static constexpr size_t kBeta = 0, kDBeta = kBeta + C, kWide = kDBeta + C;
    static constexpr size_t kGF = kWide + 4 * ((NB + 3) / 4), kGM = kGF + NB * K, kGE = kGM + NB * K;
    static constexpr size_t kGL = kGE + NB * K, kSA = kGL + K, kSB = kSA + NB * K, kSIG = kSB + NB * K;
    static constexpr size_t kTOT = kSIG + NPAIR * K, kDD = kTOT + NB * K, kDGAM = kDD + K;
    static constexpr size_t t_end = kDGAM + NB * K;
    // M (fp32, phases 1-3), then A and A^T as split planes (phases 2-3); byte offsets
    static constexpr size_t kMM = (t_end + 3) / 4 * 4;             // floats
    static constexpr size_t bMM = kMM * 4;
    static constexpr size_t PA = (size_t)C * LBC * 2;              // one [C][C] plane
    static constexpr size_t bAIh = bMM + (size_t)C * LDM * 4, bAIl = bAIh + PA, bATh = bAIl + PA, bATl = bATh + PA;
    static constexpr size_t bQ = bATl + PA;
    // phase 1: A (fp32), Akk0 (fp32), KC (fp32)
    static constexpr size_t bAI = bQ, bAKK = bAI + (size_t)C * LDM * 4, bKCS = bAKK + (size_t)C * LDM * 4;
    static constexpr size_t q1 = 2 * (size_t)C * LDM * 4 + (size_t)C * LDK * 4;
    // phase 2: v (bf16), V_new (split) for the whole block; then S_prev^T and Y^T (split),
    // later overlaid by S_prev, dS, dO, dU, dU^T
    static constexpr size_t P32C = (size_t)C * LB32 * 2, P32K = (size_t)K * LB32 * 2;
    static constexpr size_t PT_K = 32 * (size_t)LBK * 2, PT_C = 32 * (size_t)LBC * 2;
    static constexpr size_t bVV = bQ, bVNh = bVV + P32C, bVNl = bVNh + P32C;
    static constexpr size_t bSPh = bVNl + P32C, bSPl = bSPh + P32K, bU = bSPl + P32K;
    static constexpr size_t bSPTh = bU, bSPTl = bSPTh + PT_K, bYTh = bSPTl + PT_K, bYTl = bYTh + PT_C;
    static constexpr size_t ua = 2 * PT_K + 2 * PT_C;
    static constexpr size_t bDSh = bU, bDSl = bDSh + P32K;
    static constexpr size_t bDO = bDSl + P32K, bDUh = bDO + P32C, bDUl = bDUh + P32C;
    static constexpr size_t bDUTh = bDUl + P32C, bDUTl = bDUTh + PT_C;
    static constexpr size_t ub = 2 * P32K + 3 * P32C + 2 * PT_C;
    static constexpr size_t q2 = 3 * P32C + 2 * P32K + (ua > ub ? ua : ub);
    // phase 3: dW, X (fp32 [C][K]), dA then T1 (fp32 [C][C])
    static constexpr size_t bDWS = bQ, bXXS = bDWS + (size_t)C * LDK * 4, bDA = bXXS + (size_t)C * LDK * 4;
    static constexpr size_t q3 = 2 * (size_t)C * LDK * 4 + (size_t)C * LDM * 4;
    // phase 4 (from bMM: M, A are dead): Kc^T, Qr^T, Kr^T of one key half ([KH][C]) and
    // dAqk, dM, dAqk^T, dM^T ([C][C]), all split planes
    static constexpr size_t PH = (size_t)KH * LBC * 2;
    static constexpr size_t bKCTh = bMM, bKCTl = bKCTh + PH, bQRTh = bKCTl + PH, bQRTl = bQRTh + PH;
    static constexpr size_t bKRTh = bQRTl + PH, bKRTl = bKRTh + PH;
    static constexpr size_t bD1h = bKRTl + PH, bD1l = bD1h + PA, bD2h = bD1l + PA, bD2l = bD2h + PA;
    static constexpr size_t bD1Th = bD2l + PA, bD1Tl = bD1Th + PA, bD2Th = bD1Tl + PA, bD2Tl = bD2Th + PA;
    static constexpr size_t end4 = bD2Tl + PA;
    static constexpr size_t qmax = q1 > q2 ? (q1 > q3 ? q1 : q3) : (q2 > q3 ? q2 : q3);
    static constexpr size_t bytes = (bQ + qmax > end4) ? bQ + qmax : end4;
    static_assert(bytes <= 160 * 1024, "LDS budget");
    static_assert(bMM % 16 == 0 && PA % 16 == 0 && P32C % 16 == 0 && P32K % 16 == 0 && PT_K % 16 == 0 &&
                      PT_C % 16 == 0 && PH % 16 == 0 && bQ % 16 == 0,
                  "16-byte aligned planes");
};

template <int C, int NKK>
__global__ void __launch_bounds__(C / 16 * 64) bwd_local2_kernel(BwdChunkParams P) {
    using T = uint16_t;
    constexpr int MP = kMmaSplit;
    constexpr int K = 32 * NKK, NB = C / 16, NT = K / 16, NTH = NT / 2;
    using L_ = LocalLds2<C, K>;
    constexpr int LDM = L_::LDM, LDK = L_::LDK;
    const Params &p = P.f;
    const BwdParams &bp = P.b;
    extern __shared__ __align__(16) float sm[];
    unsigned char *smc = reinterpret_cast<unsigned char *>(sm);
    float *betas = sm + L_::kBeta, *DBETA = sm + L_::kDBeta;
    int *wideflag = reinterpret_cast<int *>(sm + L_::kWide);
    float *GF = sm + L_::kGF, *GM = sm + L_::kGM, *GE = sm + L_::kGE, *GL = sm + L_::kGL;
    float *SA = sm + L_::kSA, *SB = sm + L_::kSB, *SIG = sm + L_::kSIG, *TOT = sm + L_::kTOT;
    float *DD = sm + L_::kDD, *DGAM = sm + L_::kDGAM;
    float *MM = reinterpret_cast<float *>(smc + L_::bMM);
    float *AI = reinterpret_cast<float *>(smc + L_::bAI), *AKK = reinterpret_cast<float *>(smc + L_::bAKK);
    uint16_t *AIh = reinterpret_cast<uint16_t *>(smc + L_::bAIh), *AIl = reinterpret_cast<uint16_t *>(smc + L_::bAIl);
    uint16_t *ATh = reinterpret_cast<uint16_t *>(smc + L_::bATh), *ATl = reinterpret_cast<uint16_t *>(smc + L_::bATl);
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
    float rq_row, rk_row;  // q^ = q rq_row, k^ = k rk_row (q^ and k^ are reloaded after phase 2)
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
        // one branch on the gate contract for the whole row
        auto activate = [&](auto mode_tag) {
            constexpr int MODE = decltype(mode_tag)::value;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const float ga[4] = {gv[t].x, gv[t].y, gv[t].z, gv[t].w}, ba[4] = {dbv[t].x, dbv[t].y, dbv[t].z, dbv[t].w};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) G2[t][jj] = gate_act(MODE, ga[jj], ba[jj], a, p.lower_bound, unit);
            }
        };
        if (p.gate_mode == kGatePre) activate(std::integral_constant<int, kGatePre>{});
        else if (p.gate_mode == kGateSoftplus) activate(std::integral_constant<int, kGateSoftplus>{});
        else activate(std::integral_constant<int, kGateLowerBound>{});
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float qa[4] = {qv[t].x, qv[t].y, qv[t].z, qv[t].w}, ka[4] = {kv[t].x, kv[t].y, kv[t].z, kv[t].w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                qh[t][jj] = qa[jj];
                kh[t][jj] = ka[jj];
                ssq += qa[jj] * qa[jj];
                ssk += ka[jj] * ka[jj];
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
        rq_row = rq;
        rk_row = rk;
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
    // the column tables, every thread taking column threadIdx.x mod K (K <= 64 NB, so every
    // column is covered; duplicates write the same values): no lane-divergent loop here,
    // whose exit block is where spill code must not land (see codecheck.py)
    static_assert(K <= 64 * NB, "one column per thread");
    {
        const int d = (int)threadIdx.x % K;
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
    float *KCS = reinterpret_cast<float *>(smc + L_::bKCS);
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
            *reinterpret_cast<float4 *>(AKK + i * LDM + 16 * s + 4 * cg) =
                make_float4(b_i * mv[0], b_i * mv[1], b_i * mv[2], b_i * mv[3]);  // Akk0 while A is formed
        }
    }
    __syncthreads();
    {
        // A = (I + Akk0)^-1: diagonal blocks by forward substitution (lane l < 16 of wave w
        // holds column l of block w), then the off-diagonal blocks by distance
        const float *Akk = AKK;
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
        // A and A^T as split planes for phases 2 and 3
        constexpr int LBC = L_::LBC;
        for (int e = threadIdx.x; e < C * C; e += blockDim.x) {
            const int r2 = e / C, c2 = e % C;
            const float x = AI[r2 * LDM + c2];
            split_store1(AIh, AIl, r2 * LBC + c2, x);
            split_store1(ATh, ATl, c2 * LBC + r2, x);
        }
    }
    __syncthreads();


    // ---- phase 2: state-side products over 32-column blocks of V ----
    // X = b k^ E of this lane's row, split, in the permuted contraction sets of the key
    // index (step m: columns 32m + 4cg + jj, then 32m + 16 + 4cg + jj)
    uint4 Xh[NT / 2], Xl[NT / 2];
#pragma unroll
    for (int m = 0; m < NT / 2; ++m) {
        float x[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) x[4 * hh + jj] = b_i * kh[2 * m + hh][jj] * fast_exp2(G2[2 * m + hh][jj]);
        split8(x, Xh[m], Xl[m]);
    }
    // T layout accumulators: rows d = 16t + 4cg + jj, column i = 16w + lr
    f32x4 dQt[NT], dWt[NT], dKt[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) dQt[t] = dWt[t] = dKt[t] = zero4();
    f32x4 dAq[NB], dA1[NB];
#pragma unroll
    for (int s = 0; s < NB; ++s) dAq[s] = dA1[s] = zero4();
    float dbv_acc = 0.f;  // db from the v term, row i = 16w + lr (this lane's share of v)
    {
        uint16_t *VVp = reinterpret_cast<uint16_t *>(smc + L_::bVV);
        uint16_t *VNh = reinterpret_cast<uint16_t *>(smc + L_::bVNh), *VNl = reinterpret_cast<uint16_t *>(smc + L_::bVNl);
        uint16_t *SPTh = reinterpret_cast<uint16_t *>(smc + L_::bSPTh), *SPTl = reinterpret_cast<uint16_t *>(smc + L_::bSPTl);
        uint16_t *YTh = reinterpret_cast<uint16_t *>(smc + L_::bYTh), *YTl = reinterpret_cast<uint16_t *>(smc + L_::bYTl);
        uint16_t *SPh = reinterpret_cast<uint16_t *>(smc + L_::bSPh), *SPl = reinterpret_cast<uint16_t *>(smc + L_::bSPl);
        uint16_t *DSh = reinterpret_cast<uint16_t *>(smc + L_::bDSh), *DSl = reinterpret_cast<uint16_t *>(smc + L_::bDSl);
        uint16_t *DOp = reinterpret_cast<uint16_t *>(smc + L_::bDO);
        uint16_t *DUh = reinterpret_cast<uint16_t *>(smc + L_::bDUh), *DUl = reinterpret_cast<uint16_t *>(smc + L_::bDUl);
        uint16_t *DUTh = reinterpret_cast<uint16_t *>(smc + L_::bDUTh), *DUTl = reinterpret_cast<uint16_t *>(smc + L_::bDUTl);
        constexpr int LB32 = L_::LB32, LBC = L_::LBC, LBK = L_::LBK;
        const float *hs = bp.states + slot * (size_t)K * V;
        const float *dh = P.dh + slot * (size_t)K * V;
        const float *du = P.dU + slot * (size_t)C * V;
        constexpr int NTHR = 64 * NB, NSD = K * 8 / NTHR, NCV = C * 8 / NTHR, NC8 = C * 4 / NTHR;
        static_assert(K * 8 % NTHR == 0 && C * 8 % NTHR == 0 && C * 4 % NTHR == 0, "staging split");
        const int njm = (16 * w + 16 + 31) / 32;  // 32-blocks of j <= 16w + 15
        const int jm0 = (16 * w) / 32;           // first 32-block of j >= 16w
        // the four lanes of a quad hold four consecutive columns (c - qd .. c - qd + 3) of
        // the same four rows in every fragment-order unit they load (frag_rows_col)
        const int qd = lane_id() & 3;
        for (int v0 = 0; v0 < V; v0 += 32) {
            // S_prev and v first (staged now); dS, dU, dO are loaded after Y
            float4 sp4[NSD];
            uint4 vv8[NC8];
            const size_t fslice = (size_t)(v0 / 32) * (K * 8);  // float4s of one slice of a [K][V] block
#pragma unroll
            for (int q = 0; q < NSD; ++q)
                sp4[q] = reinterpret_cast<const float4 *>(hs)[fslice + threadIdx.x + q * NTHR];
#pragma unroll
            for (int q = 0; q < NC8; ++q) {
                const int e = threadIdx.x + q * NTHR, r2 = e >> 2, c8 = 8 * (e & 3);
                const int rr = r2 < ci.L ? r2 : ci.L - 1;  // in bounds; zeroed below
                vv8[q] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.v) +
                                                          ((ci.tok0 + rr) * p.HV + hv) * (int64_t)V + v0 + c8);
                if (r2 >= ci.L) vv8[q] = make_uint4(0u, 0u, 0u, 0u);
            }
            // (a) S_prev [d][v] and S_prev^T [v][d] (each float4: rows d0..d0+3 of column c), v [i][v]
#pragma unroll
            for (int q = 0; q < NSD; ++q) {
                int d0, c;
                frag_rows_col<K, false>(threadIdx.x + q * NTHR, d0, c);
                split_store4(SPTh, SPTl, c * LBK + d0, sp4[q].x, sp4[q].y, sp4[q].z, sp4[q].w);
                const float4 tq = quad_transpose(sp4[q]);  // row d0 + qd, columns c - qd ..
                split_store4(SPh, SPl, (d0 + qd) * LB32 + c - qd, tq.x, tq.y, tq.z, tq.w);
            }
#pragma unroll
            for (int q = 0; q < NC8; ++q) {
                const int e = threadIdx.x + q * NTHR, r2 = e >> 2, c8 = 8 * (e & 3);
                *reinterpret_cast<uint4 *>(VVp + r2 * LB32 + c8) = vv8[q];
            }
            __syncthreads();
            // Y = b v - X S_prev (lane: rows 16w + 4cg + jj, column 16vt + lr) -> Y^T [v][i]
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) {
                f32x4 acc = zero4();
                const int vr = (16 * vt + lr) * LBK + 4 * cg;
#pragma unroll
                for (int m = 0; m < NT / 2; ++m) {
                    const uint2 h0 = *reinterpret_cast<const uint2 *>(SPTh + vr + 32 * m);
                    const uint2 h1 = *reinterpret_cast<const uint2 *>(SPTh + vr + 32 * m + 16);
                    const uint2 l0 = *reinterpret_cast<const uint2 *>(SPTl + vr + 32 * m);
                    const uint2 l1 = *reinterpret_cast<const uint2 *>(SPTl + vr + 32 * m + 16);
                    acc = mma32_ss(acc, Xh[m], Xl[m], make_uint4(h0.x, h0.y, h1.x, h1.y), make_uint4(l0.x, l0.y, l1.x, l1.y));
                }
                float y[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int r2 = 16 * w + 4 * cg + jj;
                    y[jj] = betas[r2] * bf2f(VVp[r2 * LB32 + 16 * vt + lr]) - acc[jj];
                }
                split_store4(YTh, YTl, (16 * vt + lr) * LBC + 16 * w + 4 * cg, y[0], y[1], y[2], y[3]);
            }
            __syncthreads();
            // dS, dU, dO: in flight while V_new is formed
            float4 ds4[NSD], du4[NCV];
            uint4 do8[NC8];
#pragma unroll
            for (int q = 0; q < NSD; ++q) ds4[q] = reinterpret_cast<const float4 *>(dh)[fslice + threadIdx.x + q * NTHR];
#pragma unroll
            for (int q = 0; q < NCV; ++q)
                du4[q] = reinterpret_cast<const float4 *>(du)[(size_t)(v0 / 32) * (C * 8) + threadIdx.x + q * NTHR];
#pragma unroll
            for (int q = 0; q < NC8; ++q) {
                const int e = threadIdx.x + q * NTHR, r2 = e >> 2, c8 = 8 * (e & 3);
                const int rr = r2 < ci.L ? r2 : ci.L - 1;
                do8[q] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(bp.dout) +
                                                          ((ci.tok0 + rr) * p.HV + hv) * (int64_t)V + v0 + c8);
                if (r2 >= ci.L) do8[q] = make_uint4(0u, 0u, 0u, 0u);
            }
            // V_new^T = Y^T A^T (lane: rows v = 16vt + 4cg + jj, column i = 16w + lr) -> V_new [i][v]
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) {
                f32x4 acc = zero4();
                for (int jm = 0; jm < njm; ++jm) {
                    const int ya = (16 * vt + lr) * LBC + 32 * jm + 8 * cg, aa = (16 * w + lr) * LBC + 32 * jm + 8 * cg;
                    acc = mma32_ss(acc, *reinterpret_cast<const uint4 *>(YTh + ya), *reinterpret_cast<const uint4 *>(YTl + ya),
                                   *reinterpret_cast<const uint4 *>(AIh + aa), *reinterpret_cast<const uint4 *>(AIl + aa));
                }
                split_store4(VNh, VNl, (16 * w + lr) * LB32 + 16 * vt + 4 * cg, acc[0], acc[1], acc[2], acc[3]);
            }
            __syncthreads();  // S_prev^T, Y^T no longer read; V_new complete
            // (b) dS [d][v], dO, dU [i][v], dU^T [v][i]; rowsum(S_prev o dS) (S_prev as hi + lo)
#pragma unroll
            for (int q = 0; q < NSD; ++q) {
                int d0, c;
                frag_rows_col<K, true>(threadIdx.x + q * NTHR, d0, c);
                const float4 tq = quad_transpose(ds4[q]);  // row d0 + qd, columns c - qd ..
                split_store4(DSh, DSl, (d0 + qd) * LB32 + c - qd, tq.x, tq.y, tq.z, tq.w);
            }
#pragma unroll
            for (int q = 0; q < NCV; ++q) {
                int r0, c;
                frag_rows_col<C, true>(threadIdx.x + q * NTHR, r0, c);
                split_store4(DUTh, DUTl, c * LBC + r0, du4[q].x, du4[q].y, du4[q].z, du4[q].w);
                const float4 tq = quad_transpose(du4[q]);
                split_store4(DUh, DUl, (r0 + qd) * LB32 + c - qd, tq.x, tq.y, tq.z, tq.w);
            }
#pragma unroll
            for (int q = 0; q < NC8; ++q) {
                const int e = threadIdx.x + q * NTHR, r2 = e >> 2, c8 = 8 * (e & 3);
                *reinterpret_cast<uint4 *>(DOp + r2 * LB32 + c8) = do8[q];
            }
            __syncthreads();
            // rowsum(S_prev o dS) of this block into DD (both as hi + lo), TPR threads per row
            {
                constexpr int TPR = NTHR / K >= 8 ? 8 : (NTHR / K >= 4 ? 4 : (NTHR / K >= 2 ? 2 : 1));
                constexpr int CPT = 32 / TPR;
                const int dr = (int)threadIdx.x / TPR, d = dr < K ? dr : K - 1, c0 = CPT * ((int)threadIdx.x % TPR);
                auto lo16 = [](uint32_t x) { return __uint_as_float(x << 16); };
                auto hi16 = [](uint32_t x) { return __uint_as_float(x & 0xffff0000u); };
                float sd = 0.f;
#pragma unroll
                for (int c = 0; c < CPT; c += 4) {
                    const int a = d * LB32 + c0 + c;
                    const uint2 sh = *reinterpret_cast<const uint2 *>(SPh + a), sl = *reinterpret_cast<const uint2 *>(SPl + a);
                    const uint2 gh = *reinterpret_cast<const uint2 *>(DSh + a), gl = *reinterpret_cast<const uint2 *>(DSl + a);
                    sd += (lo16(sh.x) + lo16(sl.x)) * (lo16(gh.x) + lo16(gl.x)) + (hi16(sh.x) + hi16(sl.x)) * (hi16(gh.x) + hi16(gl.x)) +
                          (lo16(sh.y) + lo16(sl.y)) * (lo16(gh.y) + lo16(gl.y)) + (hi16(sh.y) + hi16(sl.y)) * (hi16(gh.y) + hi16(gl.y));
                }
#pragma unroll
                for (int m = 1; m < TPR; m <<= 1) sd += __shfl_xor(sd, m, 64);
                if ((int)threadIdx.x % TPR == 0 && dr < K) DD[d] += sd;
            }
            // this wave's rows i = 16w + lr as the second operand (contraction over v)
            const int ri = (16 * w + lr) * LB32 + 8 * cg;
            const uint4 bO = *reinterpret_cast<const uint4 *>(DOp + ri);
            const uint4 bUh = *reinterpret_cast<const uint4 *>(DUh + ri), bUl = *reinterpret_cast<const uint4 *>(DUl + ri);
            const uint4 bNh = *reinterpret_cast<const uint4 *>(VNh + ri), bNl = *reinterpret_cast<const uint4 *>(VNl + ri);
            // dQg^T, dW^T, dKg^T tiles (T layout)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int rd = (16 * t + lr) * LB32 + 8 * cg;
                const uint4 sh = *reinterpret_cast<const uint4 *>(SPh + rd), sl = *reinterpret_cast<const uint4 *>(SPl + rd);
                const uint4 gh = *reinterpret_cast<const uint4 *>(DSh + rd), gl = *reinterpret_cast<const uint4 *>(DSl + rd);
                dQt[t] = mma32_se(dQt[t], sh, sl, bO);
                dWt[t] = mma32_ss(dWt[t], sh, sl, bUh, bUl);
                dKt[t] = mma32_ss(dKt[t], gh, gl, bNh, bNl);
                __builtin_amdgcn_sched_barrier(0);  // bounds the operands in flight
            }
            // dAqk = dO V_new^T and dU v^T (tiles s <= w; lane: rows 16w + 4cg + jj, column 16s + lr)
#pragma unroll
            for (int s = 0; s < NB; ++s) {
                if (s <= w) {
                    const int rj = (16 * s + lr) * LB32 + 8 * cg;
                    dAq[s] = mma32_es(dAq[s], bO, *reinterpret_cast<const uint4 *>(VNh + rj),
                                      *reinterpret_cast<const uint4 *>(VNl + rj));
                    dA1[s] = mma32_se(dA1[s], bUh, bUl, *reinterpret_cast<const uint4 *>(VVp + rj));
                }
            }
            // (A^T dU)^T (lane: rows v = 16vt + 4cg + jj, column i = 16w + lr): dv, db's v term
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) {
                f32x4 acc = zero4();
                for (int jm = jm0; jm < C / 32; ++jm) {
                    const int ua = (16 * vt + lr) * LBC + 32 * jm + 8 * cg, aa = (16 * w + lr) * LBC + 32 * jm + 8 * cg;
                    acc = mma32_ss(acc, *reinterpret_cast<const uint4 *>(DUTh + ua), *reinterpret_cast<const uint4 *>(DUTl + ua),
                                   *reinterpret_cast<const uint4 *>(ATh + aa), *reinterpret_cast<const uint4 *>(ATl + aa));
                }
                const uint2 vq = *reinterpret_cast<const uint2 *>(VVp + (16 * w + lr) * LB32 + 16 * vt + 4 * cg);
                dbv_acc += __uint_as_float(vq.x << 16) * acc[0] + __uint_as_float(vq.x & 0xffff0000u) * acc[1] +
                           __uint_as_float(vq.y << 16) * acc[2] + __uint_as_float(vq.y & 0xffff0000u) * acc[3];
                if (valid)
                    *reinterpret_cast<float4 *>(bp.dv + ((ci.tok0 + i) * p.HV + hv) * (int64_t)V + v0 + 16 * vt + 4 * cg) =
                        make_float4(b_i * acc[0], b_i * acc[1], b_i * acc[2], b_i * acc[3]);
            }
            __syncthreads();  // the next block's staging overwrites these buffers
        }
    }
    // the T layout results as the fp32 form keeps them: dQg, dW (sign), dKg [t][jj]
    float dQg[NT][4], dW[NT][4], dKg[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            dQg[t][jj] = dQt[t][jj];
            dW[t][jj] = -dWt[t][jj];
            dKg[t][jj] = dKt[t][jj];
        }
    // dA1 = dU (b v)^T: the column factor b_j
#pragma unroll
    for (int s = 0; s < NB; ++s) {
        const float bj = betas[16 * s + lr];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) dA1[s][jj] *= bj;
    }
    {
        const float s = sum_col_groups(dbv_acc);
        if (cg == 0) DBETA[i] += s;
    }
    // X = b k^ E for the WY chain, with k^ reloaded (the same values as in phase 0; q^ and k^
    // are not kept live through phases 2 and 3)
    float X[NT][4];
    {
        const int64_t qrow = (tok * p.H + hq) * (int64_t)K;
        float4 kv[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) kv[t] = load4_t<T>(p.k, qrow + 16 * t + 4 * cg);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float ka[4] = {kv[t].x, kv[t].y, kv[t].z, kv[t].w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) X[t][jj] = b_i * (ka[jj] * rk_row) * fast_exp2(G2[t][jj]);
        }
    }

    // ---- phase 3: the WY chain: dX = A^T dW, dA = dU (b v)^T + dW X^T, dAkk0, dM ----
    float dX[NT][4];
    f32x4 dMt[NB];
    {
        float *DWS = reinterpret_cast<float *>(smc + L_::bDWS), *XXS = reinterpret_cast<float *>(smc + L_::bXXS);
        float *DA = reinterpret_cast<float *>(smc + L_::bDA);
        constexpr int LBC = L_::LBC;
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
                float a[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] = DWS[(32 * jm + 8 * cg + e) * LDK + 16 * t + lr];
                const int aa = (16 * w + lr) * LBC + 32 * jm + 8 * cg;
                acc = mma32_fs(acc, a, *reinterpret_cast<const uint4 *>(ATh + aa), *reinterpret_cast<const uint4 *>(ATl + aa));
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
                float a[8];
                load8(DA + (16 * w + lr) * LDM + 32 * jm + 8 * cg, a);
                const int aa = (16 * lb + lr) * LBC + 32 * jm + 8 * cg;
                T1[lb] = mma32_fs(T1[lb], a, *reinterpret_cast<const uint4 *>(AIh + aa), *reinterpret_cast<const uint4 *>(AIl + aa));
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
                    float bb[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) bb[e] = DA[(32 * im + 8 * cg + e) * LDM + 16 * lb + lr];
                    const int aa = (16 * w + lr) * LBC + 32 * im + 8 * cg;
                    acc = mma32_sf(acc, *reinterpret_cast<const uint4 *>(ATh + aa), *reinterpret_cast<const uint4 *>(ATl + aa), bb);
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


    // q^ and k^ again (the same values as in phase 0)
    {
        const int64_t qrow = (tok * p.H + hq) * (int64_t)K;
        float4 qv[NT], kv[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            qv[t] = load4_t<T>(p.q, qrow + 16 * t + 4 * cg);
            kv[t] = load4_t<T>(p.k, qrow + 16 * t + 4 * cg);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float qa[4] = {qv[t].x, qv[t].y, qv[t].z, qv[t].w}, ka[4] = {kv[t].x, kv[t].y, kv[t].z, kv[t].w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                qh[t][jj] = qa[jj] * rq_row;
                kh[t][jj] = ka[jj] * rk_row;
            }
        }
    }
    // ---- phase 4: per-element terms, the pairwise terms of Aqk and M, dgamma, suffix sum ----
    constexpr int LBC = L_::LBC;
    uint16_t *KCTh = reinterpret_cast<uint16_t *>(smc + L_::bKCTh), *KCTl = reinterpret_cast<uint16_t *>(smc + L_::bKCTl);
    uint16_t *QRTh = reinterpret_cast<uint16_t *>(smc + L_::bQRTh), *QRTl = reinterpret_cast<uint16_t *>(smc + L_::bQRTl);
    uint16_t *KRTh = reinterpret_cast<uint16_t *>(smc + L_::bKRTh), *KRTl = reinterpret_cast<uint16_t *>(smc + L_::bKRTl);
    uint16_t *D1h = reinterpret_cast<uint16_t *>(smc + L_::bD1h), *D1l = reinterpret_cast<uint16_t *>(smc + L_::bD1l);
    uint16_t *D2h = reinterpret_cast<uint16_t *>(smc + L_::bD2h), *D2l = reinterpret_cast<uint16_t *>(smc + L_::bD2l);
    uint16_t *D1Th = reinterpret_cast<uint16_t *>(smc + L_::bD1Th), *D1Tl = reinterpret_cast<uint16_t *>(smc + L_::bD1Tl);
    uint16_t *D2Th = reinterpret_cast<uint16_t *>(smc + L_::bD2Th), *D2Tl = reinterpret_cast<uint16_t *>(smc + L_::bD2Tl);
    // D1 = dAqk (lower, with the diagonal), D2 = dM (strictly lower), [i][j] and [j][i]
#pragma unroll
    for (int s = 0; s < NB; ++s) {
        float d1[4], d2[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int r2 = 16 * w + 4 * cg + jj, c2 = 16 * s + lr;
            d1[jj] = (s <= w && c2 <= r2) ? dAq[s][jj] : 0.f;
            d2[jj] = (s <= w) ? dMt[s][jj] : 0.f;
            split_store1(D1h, D1l, r2 * LBC + c2, d1[jj]);
            split_store1(D2h, D2l, r2 * LBC + c2, d2[jj]);
        }
        split_store4(D1Th, D1Tl, (16 * s + lr) * LBC + 16 * w + 4 * cg, d1[0], d1[1], d1[2], d1[3]);
        split_store4(D2Th, D2Tl, (16 * s + lr) * LBC + 16 * w + 4 * cg, d2[0], d2[1], d2[2], d2[3]);
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
    // pairwise terms, one key half at a time: Qr = q^ 2^(G - GF), Kr = k^ 2^(G - GF),
    // Kc = k^ 2^(GE - G) of every block as split planes [d][i]
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        __syncthreads();  // D1, D2 written; the previous half's operands no longer read
#pragma unroll
        for (int tl = 0; tl < NTH; ++tl) {
            const int t = NTH * hh + tl, d0 = 16 * t + 4 * cg;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float rf = fast_exp2(G2[t][jj] - GF[w * K + d0 + jj]);
                const float kc = kh[t][jj] * fast_exp2(GE[w * K + d0 + jj] - G2[t][jj]);
                const int o = (16 * tl + 4 * cg + jj) * LBC + i;
                split_store1(QRTh, QRTl, o, qh[t][jj] * rf);
                split_store1(KRTh, KRTl, o, kh[t][jj] * rf);
                split_store1(KCTh, KCTl, o, kc);
            }
        }
        __syncthreads();
#pragma unroll
        for (int tl = 0; tl < NTH; ++tl) {
            const int t = NTH * hh + tl;
            const int rd = (16 * tl + lr) * LBC + 4 * cg;  // A operand rows d (local to the half)
            // row role (rows i of block w): R1 = sum_j dAqk[i][j] k^_jd e^(G_i - G_j), R2 with dM;
            // lane: rows d = 16t + 4cg + jj, column i = 16w + lr
            f32x4 r1 = zero4(), r2 = zero4();
            for (int s = 0; s <= w; ++s) {
                if (s == w && wide) continue;
                const uint2 ah = *reinterpret_cast<const uint2 *>(KCTh + rd + 16 * s);
                const uint2 al = *reinterpret_cast<const uint2 *>(KCTl + rd + 16 * s);
                const int rb = (16 * w + lr) * LBC + 16 * s + 4 * cg;
                const f32x4 t1 = mma16_ss(zero4(), ah, al, *reinterpret_cast<const uint2 *>(D1h + rb),
                                          *reinterpret_cast<const uint2 *>(D1l + rb));
                const f32x4 t2 = mma16_ss(zero4(), ah, al, *reinterpret_cast<const uint2 *>(D2h + rb),
                                          *reinterpret_cast<const uint2 *>(D2l + rb));
                const int dd = 16 * t + 4 * cg;
                float4 f;
                if (s == w) {
                    const float4 fa = *reinterpret_cast<const float4 *>(SA + w * K + dd);
                    const float4 fb = *reinterpret_cast<const float4 *>(SB + w * K + dd);
                    f = make_float4(fa.x * fb.x, fa.y * fb.y, fa.z * fb.z, fa.w * fb.w);
                } else {
                    f = *reinterpret_cast<const float4 *>(SIG + pair_of(w, s) * K + dd);
                }
                r1[0] += f.x * t1[0], r1[1] += f.y * t1[1], r1[2] += f.z * t1[2], r1[3] += f.w * t1[3];
                r2[0] += f.x * t2[0], r2[1] += f.y * t2[1], r2[2] += f.z * t2[2], r2[3] += f.w * t2[3];
            }
            // column role (rows j of block w): C1 = sum_i dAqk[i][j] q^_id e^(G_i - G_j), C2 with dM, k^
            f32x4 c1 = zero4(), c2 = zero4();
            for (int pb = w; pb < NB; ++pb) {
                if (pb == w && wide) continue;
                const int ra = rd + 16 * pb;
                const int rb = (16 * w + lr) * LBC + 16 * pb + 4 * cg;
                const f32x4 t1 = mma16_ss(zero4(), *reinterpret_cast<const uint2 *>(QRTh + ra),
                                          *reinterpret_cast<const uint2 *>(QRTl + ra),
                                          *reinterpret_cast<const uint2 *>(D1Th + rb),
                                          *reinterpret_cast<const uint2 *>(D1Tl + rb));
                const f32x4 t2 = mma16_ss(zero4(), *reinterpret_cast<const uint2 *>(KRTh + ra),
                                          *reinterpret_cast<const uint2 *>(KRTl + ra),
                                          *reinterpret_cast<const uint2 *>(D2Th + rb),
                                          *reinterpret_cast<const uint2 *>(D2Tl + rb));
                const int dd = 16 * t + 4 * cg;
                float4 f;
                if (pb == w) {
                    const float4 fa = *reinterpret_cast<const float4 *>(SA + w * K + dd);
                    const float4 fb = *reinterpret_cast<const float4 *>(SB + w * K + dd);
                    f = make_float4(fa.x * fb.x, fa.y * fb.y, fa.z * fb.z, fa.w * fb.w);
                } else {
                    f = *reinterpret_cast<const float4 *>(SIG + pair_of(pb, w) * K + dd);
                }
                c1[0] += f.x * t1[0], c1[1] += f.y * t1[1], c1[2] += f.z * t1[2], c1[3] += f.w * t1[3];
                c2[0] += f.x * t2[0], c2[1] += f.y * t2[1], c2[2] += f.z * t2[2], c2[3] += f.w * t2[3];
            }
            // r1.. hold rows d = 16t + 4cg + jj of column i; this lane's T layout element
            // (row i, columns 16t + 4cg + jj) is exactly that: the tiles are transposed
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d = 16 * t + 4 * cg + jj;
                const float rf = fast_exp2(G2[t][jj] - GF[w * K + d]);
                const float cf = fast_exp2(GE[w * K + d] - G2[t][jj]);
                float R1 = rf * r1[jj], R2 = rf * r2[jj], C1 = cf * c1[jj], C2 = cf * c2[jj];
                if (wide) {
                    // element-wise diagonal block: exponents G_i - G_j <= 0 taken directly
#pragma unroll 1
                    for (int o = 0; o < 16; ++o) {
                        const float ko = shfl(kh[t][jj], (l & 0x30) + o), qo = shfl(qh[t][jj], (l & 0x30) + o);
                        const float go = shfl(G2[t][jj], (l & 0x30) + o);
                        if (o <= lr) {  // j = o <= i = lr: row role
                            const float f = fast_exp2(G2[t][jj] - go);
                            R1 += split_load1(D1h, D1l, (16 * w + lr) * LBC + 16 * w + o) * ko * f;
                            R2 += split_load1(D2h, D2l, (16 * w + lr) * LBC + 16 * w + o) * ko * f;
                        }
                        if (o >= lr) {  // i = o >= j = lr: column role
                            const float f = fast_exp2(go - G2[t][jj]);
                            C1 += split_load1(D1h, D1l, (16 * w + o) * LBC + 16 * w + lr) * qo * f;
                            C2 += split_load1(D2h, D2l, (16 * w + o) * LBC + 16 * w + lr) * ko * f;
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
        auto chain = [&](auto mode_tag) {
            constexpr int MODE = decltype(mode_tag)::value;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const float ga[4] = {gv[t].x, gv[t].y, gv[t].z, gv[t].w}, ba[4] = {dbv[t].x, dbv[t].y, dbv[t].z, dbv[t].w};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    float da;
                    dG[t][jj] = gate_act_grad(MODE, valid ? dG[t][jj] : 0.f, ga[jj], ba[jj], a_h, p.lower_bound, da);
                    sda += da;
                }
            }
        };
        if (p.gate_mode == kGatePre) chain(std::integral_constant<int, kGatePre>{});
        else if (p.gate_mode == kGateSoftplus) chain(std::integral_constant<int, kGateSoftplus>{});
        else chain(std::integral_constant<int, kGateLowerBound>{});
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
