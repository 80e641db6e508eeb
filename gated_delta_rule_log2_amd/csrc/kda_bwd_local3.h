// kda_bwd_local3.h -- the per-chunk gradients of the KDA backward for bf16 inputs with
// K = 128, two waves per 16-row block: the quantities, formulas and split-bf16 operand
// planes of bwd_local2_kernel (kda_bwd_local2.h; the formulas are in kda_bwd_local.h),
// with the work of each row block shared by a pair of waves.
//
// With one wave per row block the kernel holds every per-element quantity of its 16 rows
// over all K columns in registers (about 500 per lane), so a CU runs one wave per SIMD
// and every LDS and memory latency is exposed.  Here wave (w, h) owns, in the "T layout"
// (lane (lr, cg): row 16w + lr, columns 16t + 4cg .. +3 of tile t), only the four tiles
// t = 4 (u / 2) + 2h + u % 2, u < 4 -- the contraction steps m = h and m = h + 2 of
// the key index (tiles 2m, 2m + 1) -- which halves its registers and puts two waves on
// every SIMD.  How each product is shared:
//   - T layout results (dQg, dW, dKg, dX, the pairwise terms, dq^, dk^, dg): each wave its
//     own tiles;
//   - row-block tiles contracted over the key index (M, Y = b v - X S_prev): each wave
//     its own contraction steps, the two partial tiles added through LDS in a fixed order;
//   - row-block tiles contracted over rows or value columns (V_new, A^T dU, dAqk, dA,
//     T1, dAkk0): split by output tile (value tile vt = h, or column blocks s = h mod 2),
//     operands read whole from LDS;
//   - row sums (the L2 norms, db): per-wave partials, added in a fixed order.
// The (I + Akk0)^-1 solve runs on the h = 0 waves as before.
#pragma once

#include "kda_bwd_local2.h"

namespace kda {

// Streams read or written exactly once here (the chunk-start states, the state gradients,
// dU; the per-value-head dq^, dk^, dg, dv): non-temporal, so they do not displace the
// operands the workgroups share through the caches.
__device__ __forceinline__ float4 load4_once(const float *p) {
    const uint4 u = load16_once(p);
    return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
}
__device__ __forceinline__ void store4_once(float *p, float4 v) {
    store16_once(p, make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)));
}

template <int C, int K>
struct LocalLds3 {
    static constexpr int NB = C / 16, NPAIR = NB * (NB - 1) / 2, KH = K / 2;
    static constexpr int LDM = C + 4, LDK = K + 4;
    static constexpr int LB32 = 40, LBC = C + 8, LBK = K + 8;
    // tables (floats): betas [C], db per key half [2][C], row norm partials [2][C][2], ...
    static constexpr size_t kBeta = 0, kDBeta = kBeta + C, kNrm = kDBeta + 2 * C, kWide = kNrm + 4 * C;
    static constexpr size_t kGF = kWide + 4 * ((NB + 3) / 4), kGM = kGF + NB * K, kGE = kGM + NB * K;
    static constexpr size_t kGL = kGE + NB * K, kSA = kGL + K, kSB = kSA + NB * K, kSIG = kSB + NB * K;
    static constexpr size_t kTOT = kSIG + NPAIR * K, kDD = kTOT + NB * K, kDGAM = kDD + K;
    static constexpr size_t t_end = kDGAM + NB * K;
    // the regions of LocalLds2, from M on
    static constexpr size_t kMM = (t_end + 3) / 4 * 4;
    static constexpr size_t bMM = kMM * 4;
    static constexpr size_t PA = (size_t)C * LBC * 2;
    static constexpr size_t bAIh = bMM + (size_t)C * LDM * 4, bAIl = bAIh + PA, bATh = bAIl + PA, bATl = bATh + PA;
    static constexpr size_t bQ = bATl + PA;
    static constexpr size_t bAI = bQ, bAKK = bAI + (size_t)C * LDM * 4, bKCS = bAKK + (size_t)C * LDM * 4;
    static constexpr size_t q1 = 2 * (size_t)C * LDM * 4 + (size_t)C * LDK * 4;
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
    static constexpr size_t bDWS = bQ, bXXS = bDWS + (size_t)C * LDK * 4, bDA = bXXS + (size_t)C * LDK * 4;
    static constexpr size_t q3 = 2 * (size_t)C * LDK * 4 + (size_t)C * LDM * 4;
    static constexpr size_t PH = (size_t)KH * LBC * 2;
    static constexpr size_t bKCTh = bMM, bKCTl = bKCTh + PH, bQRTh = bKCTl + PH, bQRTl = bQRTh + PH;
    static constexpr size_t bKRTh = bQRTl + PH, bKRTl = bKRTh + PH;
    static constexpr size_t bD1h = bKRTl + PH, bD1l = bD1h + PA, bD2h = bD1l + PA, bD2l = bD2h + PA;
    static constexpr size_t bD1Th = bD2l + PA, bD1Tl = bD1Th + PA, bD2Th = bD1Tl + PA, bD2Tl = bD2Th + PA;
    static constexpr size_t end4 = bD2Tl + PA;
    // exchanges of partial tiles: M (phase 1) in the A region before A is formed, Y (phase 2)
    // past the dU^T planes, which are written only after Y is consumed
    static constexpr size_t bXM = bAI, bXY = bU + ua;
    static_assert((size_t)NB * NB * 1024 <= (size_t)C * LDM * 4, "M exchange fits the A region");
    static_assert((size_t)2 * NB * 1024 <= ub - ua, "Y exchange fits past the dU^T planes");
    static constexpr size_t qmax = q1 > q2 ? (q1 > q3 ? q1 : q3) : (q2 > q3 ? q2 : q3);
    static constexpr size_t bytes = (bQ + qmax > end4) ? bQ + qmax : end4;
    static_assert(bytes <= 160 * 1024, "LDS budget");
    static_assert(bMM % 16 == 0 && PA % 16 == 0 && P32C % 16 == 0 && P32K % 16 == 0 && PT_K % 16 == 0 &&
                      PT_C % 16 == 0 && PH % 16 == 0 && bQ % 16 == 0 && bXY % 16 == 0,
                  "16-byte aligned planes");
};

template <int C, int NKK>
__global__ void __launch_bounds__(C / 16 * 128) bwd_local3_kernel(BwdChunkParams P) {
    using T = uint16_t;
    constexpr int MP = kMmaSplit;
    constexpr int K = 32 * NKK, NB = C / 16, NT = K / 16;
    static_assert(NT == 8, "two waves per row block, four tiles each, two per key half");
    constexpr int NTO = NT / 2, NMO = NT / 4, NBO = NB / 2;  // own tiles, own m-steps, own s blocks
    using L_ = LocalLds3<C, K>;
    constexpr int LDM = L_::LDM, LDK = L_::LDK;
    const Params &p = P.f;
    const BwdParams &bp = P.b;
    extern __shared__ __align__(16) float sm[];
    unsigned char *smc = reinterpret_cast<unsigned char *>(sm);
    float *betas = sm + L_::kBeta, *DB = sm + L_::kDBeta, *NRM = sm + L_::kNrm;
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
    const int wid = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int w = wid % NB, h = wid / NB;  // row block, key half of the tiles
    const int l = lane_id(), lr = l & 15, cg = l >> 4;
    const int i = 16 * w + lr;  // this lane's chunk row
    const bool valid = i < ci.L;
    const int il = valid ? i : ci.L - 1;
    const int64_t tok = ci.tok0 + il;
    auto tof = [&](int u) { return 4 * (u >> 1) + 2 * h + (u & 1); };  // own tile u -> tile index

    constexpr int NTHR = 128 * NB;
    static_assert(2 * C <= NTHR && K <= NTHR, "one thread per init entry");
    if ((int)threadIdx.x < 2 * C) DB[threadIdx.x] = 0.f;
    if ((int)threadIdx.x < K) DD[threadIdx.x] = 0.f;
    if ((int)threadIdx.x < NB) wideflag[threadIdx.x] = 0;

    // ---- phase 0: q^, k^, the log2 cumulative gate G2 (own tiles), beta ----
    float qh[NTO][4], kh[NTO][4], G2[NTO][4];
    float rq_row, rk_row;
    {
        float ssq = 0.f, ssk = 0.f;
        const int64_t qrow = (tok * p.H + hq) * (int64_t)K, grow = (tok * p.HV + hv) * (int64_t)K;
        const float a = p.A_log ? expf(p.A_log[hv]) : 1.f;
        const float unit = valid ? kLog2e : 0.f;
        float4 qv[NTO], kv[NTO], gv[NTO], dbv[NTO];
#pragma unroll
        for (int u = 0; u < NTO; ++u) {
            const int c0 = 16 * tof(u) + 4 * cg;
            qv[u] = load4_t<T>(p.q, qrow + c0);
            kv[u] = load4_t<T>(p.k, qrow + c0);
        }
        if (p.g_bf16) {
#pragma unroll
            for (int u = 0; u < NTO; ++u) gv[u] = load4_t<uint16_t>(p.g, grow + 16 * tof(u) + 4 * cg);
        } else {
#pragma unroll
            for (int u = 0; u < NTO; ++u) gv[u] = load4_t<float>(p.g, grow + 16 * tof(u) + 4 * cg);
        }
        if (p.dt_bias && p.gate_mode != kGatePre) {
#pragma unroll
            for (int u = 0; u < NTO; ++u)
                dbv[u] = *reinterpret_cast<const float4 *>(p.dt_bias + (int64_t)hv * K + 16 * tof(u) + 4 * cg);
        } else {
#pragma unroll
            for (int u = 0; u < NTO; ++u) dbv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        auto activate = [&](auto mode_tag) {
            constexpr int MODE = decltype(mode_tag)::value;
#pragma unroll
            for (int u = 0; u < NTO; ++u) {
                const float ga[4] = {gv[u].x, gv[u].y, gv[u].z, gv[u].w}, ba[4] = {dbv[u].x, dbv[u].y, dbv[u].z, dbv[u].w};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) G2[u][jj] = gate_act(MODE, ga[jj], ba[jj], a, p.lower_bound, unit);
            }
        };
        if (p.gate_mode == kGatePre) activate(std::integral_constant<int, kGatePre>{});
        else if (p.gate_mode == kGateSoftplus) activate(std::integral_constant<int, kGateSoftplus>{});
        else activate(std::integral_constant<int, kGateLowerBound>{});
#pragma unroll
        for (int u = 0; u < NTO; ++u) {
            const float qa[4] = {qv[u].x, qv[u].y, qv[u].z, qv[u].w}, ka[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                qh[u][jj] = qa[jj];
                kh[u][jj] = ka[jj];
                ssq += qa[jj] * qa[jj];
                ssk += ka[jj] * ka[jj];
            }
        }
        // partial row norms over this wave's columns, added to the partner's after the barrier
        ssq = sum_col_groups(ssq);
        ssk = sum_col_groups(ssk);
        if (cg == 0) *reinterpret_cast<float2 *>(NRM + 2 * (h * C + i)) = make_float2(ssq, ssk);
#pragma unroll
        for (int u = 0; u < NTO; ++u)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) G2[u][jj] = row_scan16(G2[u][jj]);
        if (lr == 15) {
#pragma unroll
            for (int u = 0; u < NTO; ++u)
                *reinterpret_cast<float4 *>(TOT + w * K + 16 * tof(u) + 4 * cg) = make_float4(G2[u][0], G2[u][1], G2[u][2], G2[u][3]);
        }
        if (h == 0 && cg == 0) betas[i] = valid ? beta_act(p.beta_mode, load_any(p.beta, tok * p.HV + hv, p.beta_bf16)) : 0.f;
    }
    __syncthreads();
    {
        float rq = p.scale, rk = 1.f;
        if (p.qk_l2norm) {
            const float2 n0 = *reinterpret_cast<const float2 *>(NRM + 2 * i);
            const float2 n1 = *reinterpret_cast<const float2 *>(NRM + 2 * (C + i));
            rq *= rsqrtf(n0.x + n1.x + 1e-6f);
            rk = rsqrtf(n0.y + n1.y + 1e-6f);
        }
        if (!valid) rq = rk = 0.f;
        rq_row = rq;
        rk_row = rk;
#pragma unroll
        for (int u = 0; u < NTO; ++u)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                qh[u][jj] *= rq;
                kh[u][jj] *= rk;
                float pre = 0.f;
                for (int bb = 0; bb < w; ++bb) pre += TOT[bb * K + 16 * tof(u) + 4 * cg + jj];
                G2[u][jj] += pre;
            }
        int e_loc = ci.L - 1 - 16 * w;
        e_loc = e_loc > 15 ? 15 : (e_loc < 0 ? 0 : e_loc);
        const int m_loc = e_loc < 8 ? e_loc : 8;
        const bool last_here = 16 * w + e_loc == ci.L - 1;
#pragma unroll
        for (int u = 0; u < NTO; ++u) {
            const float4 gv = make_float4(G2[u][0], G2[u][1], G2[u][2], G2[u][3]);
            const int d0 = 16 * tof(u) + 4 * cg;
            if (lr == 0) *reinterpret_cast<float4 *>(GF + w * K + d0) = gv;
            if (lr == m_loc) *reinterpret_cast<float4 *>(GM + w * K + d0) = gv;
            if (lr == e_loc) {
                *reinterpret_cast<float4 *>(GE + w * K + d0) = gv;
                if (last_here) *reinterpret_cast<float4 *>(GL + d0) = gv;
            }
        }
    }
    __syncthreads();
    // the column tables, every thread taking column threadIdx.x mod K (duplicates write the
    // same values; no lane-divergent loop)
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
    // KC = k^ 2^(GE - G2), own tiles -> LDS (every column of every row is written by one wave)
    float *KCS = reinterpret_cast<float *>(smc + L_::bKCS);
#pragma unroll
    for (int u = 0; u < NTO; ++u) {
        const int d0 = 16 * tof(u) + 4 * cg;
        float kc[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) kc[jj] = kh[u][jj] * fast_exp2(GE[w * K + d0 + jj] - G2[u][jj]);
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
        float KR[NTO][4];
#pragma unroll
        for (int u = 0; u < NTO; ++u)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) KR[u][jj] = kh[u][jj] * fast_exp2(G2[u][jj] - GF[w * K + 16 * tof(u) + 4 * cg + jj]);
        // this wave's contraction steps m = 2 mu + h (tiles 2m, 2m + 1 = own tiles 2mu, 2mu + 1)
#pragma unroll
        for (int s = 0; s < NB; ++s) {
            if (s < w) {
                const float *sg = SIG + pair_of(w, s) * K;
#pragma unroll
                for (int mu = 0; mu < NMO; ++mu) {
                    const int m = 2 * mu + h;
                    float a[8], bk[8];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int d0 = 32 * m + 16 * hh + 4 * cg;
                        const float4 kc = *reinterpret_cast<const float4 *>(KCS + (16 * s + lr) * LDK + d0);
                        const float4 sgv = *reinterpret_cast<const float4 *>(sg + d0);
                        a[4 * hh + 0] = kc.x * sgv.x, a[4 * hh + 1] = kc.y * sgv.y;
                        a[4 * hh + 2] = kc.z * sgv.z, a[4 * hh + 3] = kc.w * sgv.w;
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) bk[4 * hh + jj] = KR[2 * mu + hh][jj];
                    }
                    accM[s] = mmap32<MP>(accM[s], a, bk);
                }
            }
        }
        if (!wide) {
#pragma unroll
            for (int mu = 0; mu < NMO; ++mu) {
                float a[8], bk[8];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int d0 = 16 * tof(2 * mu + hh) + 4 * cg;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        a[4 * hh + jj] = KCS[i * LDK + d0 + jj] * SB[w * K + d0 + jj];
                        bk[4 * hh + jj] = KR[2 * mu + hh][jj] * SA[w * K + d0 + jj];
                    }
                }
                accM[w] = mmap32<MP>(accM[w], a, bk);
            }
        } else {
            // element-wise diagonal block over this wave's columns
            for (int jr = 0; jr < 16; ++jr) {
                float sk = 0.f;
#pragma unroll
                for (int u = 0; u < NTO; ++u)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const float kj = shfl(kh[u][jj], (l & 0x30) + jr);
                        const float gj = shfl(G2[u][jj], (l & 0x30) + jr);
                        sk += lr > jr ? kh[u][jj] * kj * fast_exp2(G2[u][jj] - gj) : 0.f;
                    }
                sk = sum_col_groups(sk);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    if (4 * cg + jj == jr) accM[w][jj] = sk;
            }
        }
        // the partner's partial tiles through LDS ([w][s][lane], in the A region), then the
        // h = 0 wave writes M and Akk0
        f32x4 *XM = reinterpret_cast<f32x4 *>(smc + L_::bXM) + (size_t)w * NB * 64 + l;
        if (h == 1) {
#pragma unroll
            for (int s = 0; s < NB; ++s) XM[s * 64] = accM[s];
        }
        __syncthreads();
        if (h == 0) {
#pragma unroll
            for (int s = 0; s < NB; ++s) {
                const f32x4 o = XM[s * 64];
                float mv[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    mv[jj] = (s < w || (s == w && 4 * cg + jj < lr)) ? accM[s][jj] + o[jj] : 0.f;
                *reinterpret_cast<float4 *>(MM + i * LDM + 16 * s + 4 * cg) = make_float4(mv[0], mv[1], mv[2], mv[3]);
                *reinterpret_cast<float4 *>(AKK + i * LDM + 16 * s + 4 * cg) =
                    make_float4(b_i * mv[0], b_i * mv[1], b_i * mv[2], b_i * mv[3]);
            }
        }
    }
    __syncthreads();
    {
        // A = (I + Akk0)^-1 on the h = 0 waves: diagonal blocks by forward substitution, then
        // the off-diagonal blocks by distance
        const float *Akk = AKK;
        if (h == 0) {
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
#pragma unroll
            for (int s = 0; s < NB; ++s) {
                if (s > w) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int f = l + 64 * e;
                        AI[(16 * w + (f >> 4)) * LDM + 16 * s + (f & 15)] = 0.f;
                    }
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int dist = 1; dist < NB; ++dist) {
            if (h == 0 && w >= dist) {
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
        // A and A^T as split planes: one 4 x 4 block per thread of the first C^2 / 16
        // threads (whole waves, so the branch is uniform per wave), its four rows written
        // to both planes with 8-byte stores
        constexpr int LBC = L_::LBC;
        static_assert(C * C / 16 <= NTHR && C * C / 16 % 64 == 0, "whole waves, one block each");
        if (wid * 64 < C * C / 16) {
            const int bt = (int)threadIdx.x, r0 = 4 * (bt / (C / 4)), c0 = 4 * (bt % (C / 4));
            float4 a[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) a[rr] = *reinterpret_cast<const float4 *>(AI + (r0 + rr) * LDM + c0);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) split_store4(AIh, AIl, (r0 + rr) * LBC + c0, a[rr].x, a[rr].y, a[rr].z, a[rr].w);
            split_store4(ATh, ATl, (c0 + 0) * LBC + r0, a[0].x, a[1].x, a[2].x, a[3].x);
            split_store4(ATh, ATl, (c0 + 1) * LBC + r0, a[0].y, a[1].y, a[2].y, a[3].y);
            split_store4(ATh, ATl, (c0 + 2) * LBC + r0, a[0].z, a[1].z, a[2].z, a[3].z);
            split_store4(ATh, ATl, (c0 + 3) * LBC + r0, a[0].w, a[1].w, a[2].w, a[3].w);
        }
    }
    __syncthreads();

    // ---- phase 2: state-side products over 32-column blocks of V ----
    uint4 Xh[NMO], Xl[NMO];  // X = b k^ E, this wave's contraction steps, split
#pragma unroll
    for (int mu = 0; mu < NMO; ++mu) {
        float x[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) x[4 * hh + jj] = b_i * kh[2 * mu + hh][jj] * fast_exp2(G2[2 * mu + hh][jj]);
        split8(x, Xh[mu], Xl[mu]);
    }
    f32x4 dQt[NTO], dWt[NTO], dKt[NTO];
#pragma unroll
    for (int u = 0; u < NTO; ++u) dQt[u] = dWt[u] = dKt[u] = zero4();
    f32x4 dAq[NBO], dA1[NBO];  // column blocks s = 2 sl + h
#pragma unroll
    for (int sl = 0; sl < NBO; ++sl) dAq[sl] = dA1[sl] = zero4();
    float dbv_acc = 0.f;
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
        f32x4 *XY = reinterpret_cast<f32x4 *>(smc + L_::bXY) + (size_t)w * 2 * 64 + l;  // [w][vt][lane]
        constexpr int LB32 = L_::LB32, LBC = L_::LBC, LBK = L_::LBK;
        const float *hs = bp.states + slot * (size_t)K * V;
        const float *dh = P.dh + slot * (size_t)K * V;
        const float *du = P.dU + slot * (size_t)C * V;
        constexpr int NSD = K * 8 / NTHR, NCV = C * 8 / NTHR;
        static_assert(K * 8 % NTHR == 0 && C * 8 % NTHR == 0 && NSD >= 1 && NCV >= 1, "staging split");
        // v and dO: C rows of 4 units of 8 bf16; threads past C * 4 repeat a unit (same data)
        const int e8 = (int)threadIdx.x % (C * 4), r8 = e8 >> 2, c8 = 8 * (e8 & 3);
        const int rr8 = r8 < ci.L ? r8 : ci.L - 1;
        const int njm = (16 * w + 16 + 31) / 32;
        const int jm0 = (16 * w) / 32;
        // the four lanes of a quad hold four consecutive columns (c - qd .. c - qd + 3) of
        // the same four rows in every fragment-order unit they load (frag_rows_col)
        const int qd = lane_id() & 3;
        for (int v0 = 0; v0 < V; v0 += 32) {
            const size_t fslice = (size_t)(v0 / 32) * (K * 8);
            float4 sp4[NSD];
#pragma unroll
            for (int q = 0; q < NSD; ++q) sp4[q] = load4_once(hs + 4 * (fslice + threadIdx.x + q * NTHR));
            uint4 vv8 = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.v) +
                                                         ((ci.tok0 + rr8) * p.HV + hv) * (int64_t)V + v0 + c8);
            if (r8 >= ci.L) vv8 = make_uint4(0u, 0u, 0u, 0u);
            // (a) S_prev [d][v] and S_prev^T [v][d], v [i][v]
#pragma unroll
            for (int q = 0; q < NSD; ++q) {
                int d0, c;
                frag_rows_col<K, false>(threadIdx.x + q * NTHR, d0, c);
                split_store4(SPTh, SPTl, c * LBK + d0, sp4[q].x, sp4[q].y, sp4[q].z, sp4[q].w);
                const float4 tq = quad_transpose(sp4[q]);  // row d0 + qd, columns c - qd ..
                split_store4(SPh, SPl, (d0 + qd) * LB32 + c - qd, tq.x, tq.y, tq.z, tq.w);
            }
            *reinterpret_cast<uint4 *>(VVp + r8 * LB32 + c8) = vv8;
            __syncthreads();
            // Y = b v - X S_prev: partial tiles over this wave's contraction steps; the
            // partner's partial of the value tile vt = h arrives through LDS
            f32x4 accY[2];
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) {
                f32x4 acc = zero4();
                const int vr = (16 * vt + lr) * LBK + 4 * cg;
#pragma unroll
                for (int mu = 0; mu < NMO; ++mu) {
                    const int m = 2 * mu + h;
                    const uint2 h0 = *reinterpret_cast<const uint2 *>(SPTh + vr + 32 * m);
                    const uint2 h1 = *reinterpret_cast<const uint2 *>(SPTh + vr + 32 * m + 16);
                    const uint2 l0 = *reinterpret_cast<const uint2 *>(SPTl + vr + 32 * m);
                    const uint2 l1 = *reinterpret_cast<const uint2 *>(SPTl + vr + 32 * m + 16);
                    acc = mma32_ss(acc, Xh[mu], Xl[mu], make_uint4(h0.x, h0.y, h1.x, h1.y), make_uint4(l0.x, l0.y, l1.x, l1.y));
                }
                accY[vt] = acc;
            }
            XY[(1 - h) * 64] = accY[1 - h];
            // dS, dU, dO: in flight while Y and V_new are formed
            float4 ds4[NSD], du4[NCV];
#pragma unroll
            for (int q = 0; q < NSD; ++q) ds4[q] = load4_once(dh + 4 * (fslice + threadIdx.x + q * NTHR));
#pragma unroll
            for (int q = 0; q < NCV; ++q)
                du4[q] = load4_once(du + 4 * ((size_t)(v0 / 32) * (C * 8) + threadIdx.x + q * NTHR));
            uint4 do8 = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(bp.dout) +
                                                         ((ci.tok0 + rr8) * p.HV + hv) * (int64_t)V + v0 + c8);
            if (r8 >= ci.L) do8 = make_uint4(0u, 0u, 0u, 0u);
            __syncthreads();
            {
                const int vt = h;
                const f32x4 o = XY[h * 64];
                float y[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int r2 = 16 * w + 4 * cg + jj;
                    // h = 0 adds its own partial first, h = 1 its partner's: the same order
                    const float yx = h == 0 ? accY[vt][jj] + o[jj] : o[jj] + accY[vt][jj];
                    y[jj] = betas[r2] * bf2f(VVp[r2 * LB32 + 16 * vt + lr]) - yx;
                }
                split_store4(YTh, YTl, (16 * vt + lr) * LBC + 16 * w + 4 * cg, y[0], y[1], y[2], y[3]);
            }
            __syncthreads();
            // V_new^T = Y^T A^T, value tile vt = h
            {
                const int vt = h;
                f32x4 acc = zero4();
                for (int jm = 0; jm < njm; ++jm) {
                    const int ya = (16 * vt + lr) * LBC + 32 * jm + 8 * cg, aa = (16 * w + lr) * LBC + 32 * jm + 8 * cg;
                    acc = mma32_ss(acc, *reinterpret_cast<const uint4 *>(YTh + ya), *reinterpret_cast<const uint4 *>(YTl + ya),
                                   *reinterpret_cast<const uint4 *>(AIh + aa), *reinterpret_cast<const uint4 *>(AIl + aa));
                }
                split_store4(VNh, VNl, (16 * w + lr) * LB32 + 16 * vt + 4 * cg, acc[0], acc[1], acc[2], acc[3]);
            }
            __syncthreads();  // S_prev^T, Y^T no longer read; V_new complete
            // (b) dS [d][v], dO, dU [i][v], dU^T [v][i]
#pragma unroll
            for (int q = 0; q < NSD; ++q) {
                int d0, c;
                frag_rows_col<K, true>(threadIdx.x + q * NTHR, d0, c);
                const float4 tq = quad_transpose(ds4[q]);
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
            *reinterpret_cast<uint4 *>(DOp + r8 * LB32 + c8) = do8;
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
            // dQg^T, dW^T, dKg^T, own tiles
#pragma unroll
            for (int u = 0; u < NTO; ++u) {
                const int rd = (16 * tof(u) + lr) * LB32 + 8 * cg;
                const uint4 sh = *reinterpret_cast<const uint4 *>(SPh + rd), sl = *reinterpret_cast<const uint4 *>(SPl + rd);
                const uint4 gh = *reinterpret_cast<const uint4 *>(DSh + rd), gl = *reinterpret_cast<const uint4 *>(DSl + rd);
                dQt[u] = mma32_se(dQt[u], sh, sl, bO);
                dWt[u] = mma32_ss(dWt[u], sh, sl, bUh, bUl);
                dKt[u] = mma32_ss(dKt[u], gh, gl, bNh, bNl);
            }
            // dAqk = dO V_new^T and dU v^T, column blocks s = 2 sl + h <= w
#pragma unroll
            for (int sl = 0; sl < NBO; ++sl) {
                const int s = 2 * sl + h;
                if (s <= w) {
                    const int rj = (16 * s + lr) * LB32 + 8 * cg;
                    dAq[sl] = mma32_es(dAq[sl], bO, *reinterpret_cast<const uint4 *>(VNh + rj),
                                       *reinterpret_cast<const uint4 *>(VNl + rj));
                    dA1[sl] = mma32_se(dA1[sl], bUh, bUl, *reinterpret_cast<const uint4 *>(VVp + rj));
                }
            }
            // (A^T dU)^T, value tile vt = h: dv, db's v term
            {
                const int vt = h;
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
                    store4_once(bp.dv + ((ci.tok0 + i) * p.HV + hv) * (int64_t)V + v0 + 16 * vt + 4 * cg,
                                make_float4(b_i * acc[0], b_i * acc[1], b_i * acc[2], b_i * acc[3]));
            }
            __syncthreads();  // the next block's staging overwrites these buffers
        }
    }
    float dQg[NTO][4], dW[NTO][4], dKg[NTO][4];
#pragma unroll
    for (int u = 0; u < NTO; ++u)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            dQg[u][jj] = dQt[u][jj];
            dW[u][jj] = -dWt[u][jj];
            dKg[u][jj] = dKt[u][jj];
        }
#pragma unroll
    for (int sl = 0; sl < NBO; ++sl) {
        const float bj = betas[16 * (2 * sl + h) + lr];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) dA1[sl][jj] *= bj;
    }
    {
        const float s = sum_col_groups(dbv_acc);
        if (cg == 0) DB[h * C + i] += s;
    }
    float X[NTO][4];
    {
        const int64_t qrow = (tok * p.H + hq) * (int64_t)K;
        float4 kv[NTO];
#pragma unroll
        for (int u = 0; u < NTO; ++u) kv[u] = load4_t<T>(p.k, qrow + 16 * tof(u) + 4 * cg);
#pragma unroll
        for (int u = 0; u < NTO; ++u) {
            const float ka[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) X[u][jj] = b_i * (ka[jj] * rk_row) * fast_exp2(G2[u][jj]);
        }
    }

    // ---- phase 3: the WY chain: dX = A^T dW, dA = dU (b v)^T + dW X^T, dAkk0, dM ----
    float dX[NTO][4];
    f32x4 dMt[NBO];  // column blocks lb = 2 sl + h
    {
        float *DWS = reinterpret_cast<float *>(smc + L_::bDWS), *XXS = reinterpret_cast<float *>(smc + L_::bXXS);
        float *DA = reinterpret_cast<float *>(smc + L_::bDA);
        constexpr int LBC = L_::LBC;
#pragma unroll
        for (int u = 0; u < NTO; ++u) {
            const int d0 = 16 * tof(u) + 4 * cg;
            *reinterpret_cast<float4 *>(DWS + i * LDK + d0) = make_float4(dW[u][0], dW[u][1], dW[u][2], dW[u][3]);
            *reinterpret_cast<float4 *>(XXS + i * LDK + d0) = make_float4(X[u][0], X[u][1], X[u][2], X[u][3]);
        }
        __syncthreads();
        // dX^T, own tiles: sum over rows j >= 16w of dW[j][d] A[j][i]
        const int jm0 = (16 * w) / 32;
#pragma unroll
        for (int u = 0; u < NTO; ++u) {
            const int t = tof(u);
            f32x4 acc = zero4();
            for (int jm = jm0; jm < C / 32; ++jm) {
                float a[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] = DWS[(32 * jm + 8 * cg + e) * LDK + 16 * t + lr];
                const int aa = (16 * w + lr) * LBC + 32 * jm + 8 * cg;
                acc = mma32_fs(acc, a, *reinterpret_cast<const uint4 *>(ATh + aa), *reinterpret_cast<const uint4 *>(ATl + aa));
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) dX[u][jj] = acc[jj];
        }
        // dA2 = dW X^T over every key column (both operands from LDS), column blocks
        // s = 2 sl + h; dA = mask(dA1 + dA2) strictly lower -> LDS
#pragma unroll
        for (int sl = 0; sl < NBO; ++sl) {
            const int s = 2 * sl + h;
            f32x4 dA = zero4();
            if (s <= w) {
                f32x4 acc = dA1[sl];
#pragma unroll
                for (int m = 0; m < NT / 2; ++m) {
                    float a[8], bb[8];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int d0 = 32 * m + 16 * hh + 4 * cg;
                        const float4 xv = *reinterpret_cast<const float4 *>(XXS + (16 * s + lr) * LDK + d0);
                        const float4 wv = *reinterpret_cast<const float4 *>(DWS + i * LDK + d0);
                        bb[4 * hh + 0] = xv.x, bb[4 * hh + 1] = xv.y, bb[4 * hh + 2] = xv.z, bb[4 * hh + 3] = xv.w;
                        a[4 * hh + 0] = wv.x, a[4 * hh + 1] = wv.y, a[4 * hh + 2] = wv.z, a[4 * hh + 3] = wv.w;
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
        // T1 = dA A^T on this row block, column blocks lb = 2 sl + h; both waves of the block
        // read all of its rows of dA, so the results are written after a barrier
        f32x4 T1[NBO];
        const int njm = (16 * w + 16 + 31) / 32;
#pragma unroll
        for (int sl = 0; sl < NBO; ++sl) {
            const int lb = 2 * sl + h;
            T1[sl] = zero4();
            for (int jm = 0; jm < njm; ++jm) {
                float a[8];
                load8(DA + (16 * w + lr) * LDM + 32 * jm + 8 * cg, a);
                const int aa = (16 * lb + lr) * LBC + 32 * jm + 8 * cg;
                T1[sl] = mma32_fs(T1[sl], a, *reinterpret_cast<const uint4 *>(AIh + aa), *reinterpret_cast<const uint4 *>(AIl + aa));
            }
        }
        __syncthreads();
#pragma unroll
        for (int sl = 0; sl < NBO; ++sl)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) DA[(16 * w + 4 * cg + jj) * LDM + 16 * (2 * sl + h) + lr] = T1[sl][jj];
        __syncthreads();
        // dAkk0 = -A^T T1 (rows 16w.., column blocks lb = 2 sl + h <= w), strictly lower;
        // dM = b dAkk0; db from rowsum(dAkk0 o M)
        const int im0 = (16 * w) / 32;
        float dbm[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sl = 0; sl < NBO; ++sl) {
            const int lb = 2 * sl + h;
            dMt[sl] = zero4();
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
                    dMt[sl][jj] = betas[r2] * dak;
                }
            }
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float s = row_sum16_all(dbm[jj]);
            if (lr == 0) DB[h * C + 16 * w + 4 * cg + jj] += s;
        }
    }
    __syncthreads();  // region Q is rewritten below

    // q^ and k^ again (the same values as in phase 0)
    {
        const int64_t qrow = (tok * p.H + hq) * (int64_t)K;
        float4 qv[NTO], kv[NTO];
#pragma unroll
        for (int u = 0; u < NTO; ++u) {
            qv[u] = load4_t<T>(p.q, qrow + 16 * tof(u) + 4 * cg);
            kv[u] = load4_t<T>(p.k, qrow + 16 * tof(u) + 4 * cg);
        }
#pragma unroll
        for (int u = 0; u < NTO; ++u) {
            const float qa[4] = {qv[u].x, qv[u].y, qv[u].z, qv[u].w}, ka[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                qh[u][jj] = qa[jj] * rq_row;
                kh[u][jj] = ka[jj] * rk_row;
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
    // D1 = dAqk (lower, with the diagonal), D2 = dM (strictly lower), [i][j] and [j][i]:
    // column blocks s = 2 sl + h of this row block
    // (the [i][j] planes after a quad transpose: lane qd then holds row 16w + 4cg + qd,
    // columns 16s + lr - qd .. +3)
    const int qd = lane_id() & 3;
#pragma unroll
    for (int sl = 0; sl < NBO; ++sl) {
        const int s = 2 * sl + h;
        float d1[4], d2[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int r2 = 16 * w + 4 * cg + jj, c2 = 16 * s + lr;
            d1[jj] = (s <= w && c2 <= r2) ? dAq[sl][jj] : 0.f;
            d2[jj] = (s <= w) ? dMt[sl][jj] : 0.f;
        }
        const int ot = (16 * w + 4 * cg + qd) * LBC + 16 * s + lr - qd;
        const float4 t1 = quad_transpose(make_float4(d1[0], d1[1], d1[2], d1[3]));
        const float4 t2 = quad_transpose(make_float4(d2[0], d2[1], d2[2], d2[3]));
        split_store4(D1h, D1l, ot, t1.x, t1.y, t1.z, t1.w);
        split_store4(D2h, D2l, ot, t2.x, t2.y, t2.z, t2.w);
        split_store4(D1Th, D1Tl, (16 * s + lr) * LBC + 16 * w + 4 * cg, d1[0], d1[1], d1[2], d1[3]);
        split_store4(D2Th, D2Tl, (16 * s + lr) * LBC + 16 * w + 4 * cg, d2[0], d2[1], d2[2], d2[3]);
    }
    float dqh[NTO][4], dkh[NTO][4], dG[NTO][4];
    {
        float gam[NTO][4], db3 = 0.f;
#pragma unroll
        for (int u = 0; u < NTO; ++u)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d = 16 * tof(u) + 4 * cg + jj;
                const float E = fast_exp2(G2[u][jj]), F = fast_exp2(GL[d] - G2[u][jj]);
                dqh[u][jj] = dQg[u][jj] * E;
                dkh[u][jj] = dKg[u][jj] * F + b_i * dX[u][jj] * E;
                dG[u][jj] = dQg[u][jj] * qh[u][jj] * E - dKg[u][jj] * kh[u][jj] * F + b_i * dX[u][jj] * kh[u][jj] * E;
                gam[u][jj] = row_sum16_all(dKg[u][jj] * kh[u][jj] * F);
                db3 += dX[u][jj] * kh[u][jj] * E;
            }
        if (lr == 0) {
#pragma unroll
            for (int u = 0; u < NTO; ++u)
                *reinterpret_cast<float4 *>(DGAM + w * K + 16 * tof(u) + 4 * cg) = make_float4(gam[u][0], gam[u][1], gam[u][2], gam[u][3]);
        }
        db3 = sum_col_groups(db3);
        if (cg == 0) DB[h * C + i] += db3;
    }
    // pairwise terms, one key half at a time (this wave's two tiles of it)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        __syncthreads();  // D1, D2 written; the previous half's operands no longer read
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
            const int u = 2 * hh + uu, t = tof(u), tl = t - 4 * hh, d0 = 16 * t + 4 * cg;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float rf = fast_exp2(G2[u][jj] - GF[w * K + d0 + jj]);
                const float kc = kh[u][jj] * fast_exp2(GE[w * K + d0 + jj] - G2[u][jj]);
                const int o = (16 * tl + 4 * cg + jj) * LBC + i;
                split_store1(QRTh, QRTl, o, qh[u][jj] * rf);
                split_store1(KRTh, KRTl, o, kh[u][jj] * rf);
                split_store1(KCTh, KCTl, o, kc);
            }
        }
        __syncthreads();
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
            const int u = 2 * hh + uu, t = tof(u), tl = t - 4 * hh;
            const int rd = (16 * tl + lr) * LBC + 4 * cg;  // A operand rows d (local to the half)
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
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d = 16 * t + 4 * cg + jj;
                const float rf = fast_exp2(G2[u][jj] - GF[w * K + d]);
                const float cf = fast_exp2(GE[w * K + d] - G2[u][jj]);
                float R1 = rf * r1[jj], R2 = rf * r2[jj], C1 = cf * c1[jj], C2 = cf * c2[jj];
                if (wide) {
#pragma unroll 1
                    for (int o = 0; o < 16; ++o) {
                        const float ko = shfl(kh[u][jj], (l & 0x30) + o), qo = shfl(qh[u][jj], (l & 0x30) + o);
                        const float go = shfl(G2[u][jj], (l & 0x30) + o);
                        if (o <= lr) {
                            const float f = fast_exp2(G2[u][jj] - go);
                            R1 += split_load1(D1h, D1l, (16 * w + lr) * LBC + 16 * w + o) * ko * f;
                            R2 += split_load1(D2h, D2l, (16 * w + lr) * LBC + 16 * w + o) * ko * f;
                        }
                        if (o >= lr) {
                            const float f = fast_exp2(go - G2[u][jj]);
                            C1 += split_load1(D1h, D1l, (16 * w + o) * LBC + 16 * w + lr) * qo * f;
                            C2 += split_load1(D2h, D2l, (16 * w + o) * LBC + 16 * w + lr) * ko * f;
                        }
                    }
                }
                dqh[u][jj] += R1;
                dkh[u][jj] += R2 + C1 + C2;
                dG[u][jj] += qh[u][jj] * R1 + kh[u][jj] * R2 - kh[u][jj] * (C1 + C2);
            }
        }
    }
    __syncthreads();  // DGAM complete
    {
        const int d = (int)threadIdx.x % K;  // duplicates write the same value
        float s = DD[d] * fast_exp2(GL[d]);
        for (int bb = 0; bb < NB; ++bb) s += DGAM[bb * K + d];
        TOT[d] = s;  // dgamma
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NTO; ++u)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            if (i == ci.L - 1) dG[u][jj] += TOT[16 * tof(u) + 4 * cg + jj];
            if (!valid) dG[u][jj] = 0.f;
            dG[u][jj] = row_suffix16(dG[u][jj]);
        }
    __syncthreads();  // TOT read
    if (lr == 0) {
#pragma unroll
        for (int u = 0; u < NTO; ++u)
            *reinterpret_cast<float4 *>(TOT + w * K + 16 * tof(u) + 4 * cg) = make_float4(dG[u][0], dG[u][1], dG[u][2], dG[u][3]);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NTO; ++u)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            float suf = 0.f;
            for (int bb = w + 1; bb < NB; ++bb) suf += TOT[bb * K + 16 * tof(u) + 4 * cg + jj];
            dG[u][jj] += suf;
        }
    // the gate's chain rule, this chunk's sums for dt_bias and A_log, dbeta
    const size_t o = (size_t)tok * p.HV + hv;
    const float a_h = p.A_log ? expf(p.A_log[hv]) : 1.f;
    float sda = 0.f;
    {
        const int64_t grow = (int64_t)o * K;
        float4 gv[NTO], dbv[NTO];
        if (p.g_bf16) {
#pragma unroll
            for (int u = 0; u < NTO; ++u) gv[u] = load4_t<uint16_t>(p.g, grow + 16 * tof(u) + 4 * cg);
        } else {
#pragma unroll
            for (int u = 0; u < NTO; ++u) gv[u] = load4_t<float>(p.g, grow + 16 * tof(u) + 4 * cg);
        }
        if (p.dt_bias && p.gate_mode != kGatePre) {
#pragma unroll
            for (int u = 0; u < NTO; ++u)
                dbv[u] = *reinterpret_cast<const float4 *>(p.dt_bias + (int64_t)hv * K + 16 * tof(u) + 4 * cg);
        } else {
#pragma unroll
            for (int u = 0; u < NTO; ++u) dbv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        auto chain = [&](auto mode_tag) {
            constexpr int MODE = decltype(mode_tag)::value;
#pragma unroll
            for (int u = 0; u < NTO; ++u) {
                const float ga[4] = {gv[u].x, gv[u].y, gv[u].z, gv[u].w}, ba[4] = {dbv[u].x, dbv[u].y, dbv[u].z, dbv[u].w};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    float da;
                    dG[u][jj] = gate_act_grad(MODE, valid ? dG[u][jj] : 0.f, ga[jj], ba[jj], a_h, p.lower_bound, da);
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
        for (int u = 0; u < NTO; ++u) {
            const int d0 = 16 * tof(u) + 4 * cg;
            store4_once(bp.p_dq + o * K + d0, make_float4(dqh[u][0], dqh[u][1], dqh[u][2], dqh[u][3]));
            store4_once(bp.p_dk + o * K + d0, make_float4(dkh[u][0], dkh[u][1], dkh[u][2], dkh[u][3]));
            store4_once(bp.dg + o * K + d0, make_float4(dG[u][0], dG[u][1], dG[u][2], dG[u][3]));
        }
        // (every DB term was added before the barriers above)
        if (h == 0 && cg == 0) {
            float dbv = DB[i] + DB[C + i];
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
        for (int u = 0; u < NTO; ++u)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float cs = row_sum16_all(dG[u][jj]);
                if (lr == 0) TOT[w * K + 16 * tof(u) + 4 * cg + jj] = cs;
            }
        sda = sum_col_groups(row_sum16_all(sda));
        if (l == 0) DGAM[2 * w + h] = sda;
        __syncthreads();
        if ((int)threadIdx.x <= K) {
            const int d = (int)threadIdx.x;
            float acc = 0.f;
            if (d < K) {
                for (int bb = 0; bb < NB; ++bb) acc += TOT[bb * K + d];
            } else {
                for (int e = 0; e < 2 * NB; ++e) acc += DGAM[e];
            }
            P.cparam[slot * (K + 1) + d] = acc;
        }
    }
}

}  // namespace kda
