// kda_intra_bf16.h -- intra-chunk stage of the KDA forward for bf16 q/k/v: one
// workgroup per (chunk, value head), one wave per 16-row sub-chunk, every matrix
// operand formed once as packed bf16 and fed to the matrix cores directly.
//
// It produces the same per-chunk intermediates, in the same fragment-major layouts,
// as the generic kernel in kda_intra.h ("Reading Notes: Implementation Notes for KDA
// in FLA", forward steps 1-3):
//   Aqk[i][j]  = sum_d q^_id k^_jd 2^(G_id - G_jd)          (j <= i)
//   Akk0[i][j] = b_i sum_d k^_id k^_jd 2^(G_id - G_jd)      (j <  i)
//   A = (I + Akk0)^-1,  W = A Diag(b) (2^G k^),  U = A Diag(b) v
//   Qg = 2^G q^,  KgT = (2^(G_last - G) k^)^T,  d = 2^G_last
//
// Differences from the generic kernel, all aimed at vector-ALU work per element:
//   - the cumulative gate is kept block-local (a 16-row scan); every quantity that
//     needs the chunk-level prefix is a per-column scalar from one column pass, so no
//     element ever adds the earlier blocks' totals;
//   - each element takes two exp2 of non-positive block-local differences,
//     Rf = 2^(G - G_first) and Cf = 2^(G_last_row - G), and every other factor is a
//     per-column scalar ("flash-linear-attention KDA 内核工程实践…", §3.1 midpoint
//     offset for the diagonal blocks, §3.2 pairwise offsets for the off-diagonal
//     blocks; the midpoint scalars 2^(G_first - G_mid) and 2^(G_mid - G_last_row)
//     are bounded by 2^60 per column, otherwise the block takes the element-wise
//     form of §4);
//   - transposes (X^T, v^T, KgT) run on the matrix cores as products with a 0/1
//     selection matrix, which is exact, instead of 2-byte LDS scatters;
//   - beta is folded into the columns of (I + Akk0)^-1 rather than into X and v.
#pragma once

#include "kda_intra.h"

namespace kda {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Two fp32 -> packed bf16 pair (round to nearest even, one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint4 pack8(const float (&x)[8]) {
    return make_uint4(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7]));
}
__device__ __forceinline__ void unpack8(uint4 u, float (&o)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(w[i] << 16);
        o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// B operand that selects contraction index off + (l & 15): with it, a 16x16x32
// product returns, in lane (lr, cg), rows 4cg..4cg+3 of column off + lr of the A
// operand's 16x32 block, i.e. a transpose into the accumulator layout.
__device__ __forceinline__ uint4 select_frag(int off) {
    const int l = lane_id(), lr = l & 15, cg = l >> 4;
    const int k = off + lr;
    const bool mine = (k >> 3) == cg;
    const int t = k & 7;
    const uint32_t one = (t & 1) ? 0x3F800000u : 0x00003F80u;
    return make_uint4(mine && (t >> 1) == 0 ? one : 0u, mine && (t >> 1) == 1 ? one : 0u,
                      mine && (t >> 1) == 2 ? one : 0u, mine && (t >> 1) == 3 ? one : 0u);
}

// [rows][C] bf16 tiles in LDS with the 16-byte column chunks permuted per row, so
// that 16 lanes reading one chunk of 16 consecutive rows, or writing 8-byte halves of
// one chunk, touch distinct banks.
template <int C>
__device__ __forceinline__ int swz(int row, int col) {
    constexpr int CPR = C / 8;
    return row * C + ((((col >> 3) ^ ((row ^ (row >> 3)) & (CPR - 1))) << 3) | (col & 7));
}

template <int C, int K>
struct IntraBf16Lds {
    static constexpr int NB = C / 16, NPAIR = NB * (NB - 1) / 2, LDA = C + 4;
    // betas [C] f32, wide-block flags [NB] i32
    static constexpr size_t kBeta = 0;
    static constexpr size_t kWide = 4 * C;
    // region A: gate column values CV [3][NB][K] and column scalars SC [4][NB][K] (f32);
    //           then Akk [C][LDA] f32; then X^T [K][C] bf16
    static constexpr size_t kA = ((C + NB) * 4 + 15) / 16 * 16;
    static constexpr size_t cv_bytes = 3 * NB * K * 4, sc_bytes = 4 * NB * K * 4;
    static constexpr size_t akk_bytes = (size_t)C * LDA * 4, tr_k_bytes = (size_t)K * C * 2;
    static constexpr size_t a_bytes = (cv_bytes + sc_bytes > akk_bytes ? cv_bytes + sc_bytes : akk_bytes) > tr_k_bytes
                                          ? (cv_bytes + sc_bytes > akk_bytes ? cv_bytes + sc_bytes : akk_bytes)
                                          : tr_k_bytes;
    // region B: pair sources [NB-1][NKK][64] uint4, pair scalars [NPAIR][K] f32,
    //           KgT staging [K][C] bf16; then Ainv [C][LDA] f32 and v^T [V][C] bf16
    static constexpr size_t kB = kA + a_bytes;
    static constexpr size_t ops_bytes = (size_t)(NB - 1) * 16 * K * 2, sig_bytes = (size_t)NPAIR * K * 4;
    static constexpr size_t kSig = kB + ops_bytes, kKst = kSig + sig_bytes;
    static constexpr size_t kVt = kB + akk_bytes;
    static __host__ __device__ size_t bytes(int V) {
        const size_t p1 = ops_bytes + sig_bytes + tr_k_bytes, p2 = akk_bytes + (size_t)V * C * 2;
        return kB + (p1 > p2 ? p1 : p2);
    }
};

#ifdef KDA_INTRA_WAVES_PER_EU
#define KDA_INTRA_OCC __attribute__((amdgpu_waves_per_eu(KDA_INTRA_WAVES_PER_EU)))
#else
#define KDA_INTRA_OCC
#endif

// Zero gate bias read in place of a missing dt_bias, so the bias loads need no branch
// (a branch around them makes the compiler wait for them before the q/k loads issue).
static __device__ float kda_zero_bias[256];

// Key widths up to 128 store W, Qg, Aqk and KgT as permuted row fragments (the
// layout of the register-resident recurrence); wider keys keep plain row fragments.
template <int K>
__host__ __device__ constexpr bool permuted_layout() { return K <= 128; }

// Gate and value inputs are read exactly once.  When the per-chunk intermediates this
// kernel writes are about the size of the memory-side cache, reading those inputs with
// the non-temporal hint keeps them from displacing the intermediates the recurrence
// reads back next (gva_bf16: recurrence -8 us, this kernel +1.5 us); far larger
// batches gain nothing and pay the slower hinted loads, so they take plain loads.
constexpr size_t kOnceLoadMaxIntermediates = size_t(384) << 20;
template <bool NT>
__device__ __forceinline__ uint4 load16_input(const void *ptr) {
    if constexpr (NT) return load16_once(ptr);
    else return *reinterpret_cast<const uint4 *>(ptr);
}

// GB, BB: gate input, beta stored as bf16 (else fp32); NT: non-temporal gate/value loads
template <int C, int NKK, bool GB, bool BB, bool NT>
__global__ void __launch_bounds__(C / 16 * 64) KDA_INTRA_OCC intra_bf16_kernel(Params p) {
    constexpr int NB = C / 16, K = 32 * NKK;
    constexpr bool PERM = permuted_layout<K>();
    using L_ = IntraBf16Lds<C, K>;
    constexpr int LDA = L_::LDA;
    extern __shared__ __align__(16) unsigned char lds[];
    const int V = p.V;
    float *betas = reinterpret_cast<float *>(lds + L_::kBeta);
    int *wideflag = reinterpret_cast<int *>(lds + L_::kWide);
    float *CV0 = reinterpret_cast<float *>(lds + L_::kA);  // [NB][K] G at the block's first row
    float *CV8 = CV0 + NB * K;                             // [NB][K] G at row 8 (the midpoint)
    float *CV15 = CV8 + NB * K;                            // [NB][K] G at the block's last row
    float *Ssa = CV15 + NB * K;                            // [NB][K] 2^(G_first - G_mid)
    float *Ssb = Ssa + NB * K;                             // [NB][K] 2^(G_mid - G_lastrow)
    float *Scn = Ssb + NB * K;                             // [NB][K] 2^(chunk G at the first row)
    float *Sck = Scn + NB * K;                             // [NB][K] 2^(G_chunklast - G_lastrow)
    float *Akk = reinterpret_cast<float *>(lds + L_::kA);
    uint16_t *XT = reinterpret_cast<uint16_t *>(lds + L_::kA);
    uint4 *OPS = reinterpret_cast<uint4 *>(lds + L_::kB);
    float *SIG = reinterpret_cast<float *>(lds + L_::kSig);
    uint16_t *KST = reinterpret_cast<uint16_t *>(lds + L_::kKst);
    float *Ainv = reinterpret_cast<float *>(lds + L_::kB);
    uint16_t *VT = reinterpret_cast<uint16_t *>(lds + L_::kVt);
    auto pair_of = [](int wb, int sb) { return wb * (wb - 1) / 2 + sb; };

    // Workgroup b runs on XCD b % 8.  The value heads of one qk head (which read the same
    // q and k rows) are given indices 8 apart, so they run on one XCD at about the same
    // time and the second one finds q and k in that XCD's L2.  Chunks are taken
    // last-to-first, so the first chunks the recurrence reads are the most recently
    // written ones (still in the memory-side cache).
    int qi, j;  // (chunk, qk head) item and the value head within its group
    {
        const int b = blockIdx.x, tile = 8 * p.group;
        const int nq = p.total_chunks * p.H, full = nq / 8;
        if (b < full * tile) {
            qi = 8 * (b / tile) + (b % 8);
            j = (b % tile) / 8;
        } else {
            const int rb = b - full * tile;
            qi = 8 * full + rb / p.group;
            j = rb % p.group;
        }
    }
    const int gc = p.total_chunks - 1 - qi / p.H;
    const int h = qi % p.H;
    const int hv = h * p.group + j;
    const ChunkInfo ci = chunk_info(p, gc);
    const int w = threadIdx.x >> 6;
    const int l = lane_id(), lr = l & 15, cg = l >> 4;
    const int r = 16 * w + lr;
    const bool valid = r < ci.L;
    const int rl = valid ? r : ci.L - 1;  // rows past the end load the last valid row, then weigh 0
    const size_t slot = (size_t)gc * p.HV + hv;
    uint16_t *Wg = static_cast<uint16_t *>(p.w_W) + slot * C * K;
    uint16_t *UTg = static_cast<uint16_t *>(p.w_U) + slot * (size_t)V * C;
    uint16_t *KgTg = static_cast<uint16_t *>(p.w_KgT) + slot * K * C;
    uint16_t *Qgg = static_cast<uint16_t *>(p.w_Qg) + slot * C * K;
    uint16_t *Aqkg = static_cast<uint16_t *>(p.w_Aqk) + slot * C * C;
    float *dg = p.w_d + slot * K;

    // ---- loads: gate and beta first (the gate math and scan start as soon as they land,
    //      while q and k are still in flight), then q, k (packed bf16) ----
    const int64_t qkrow = ((ci.tok0 + rl) * p.H + h) * (int64_t)K + 8 * cg;
    const int64_t grow = ((ci.tok0 + rl) * p.HV + hv) * (int64_t)K + 8 * cg;
    // raw gate words (bf16: one 16-byte unit per 8 values; fp32: two) and raw beta bits,
    // widened only after the q/k loads are issued, so no wait sits between the loads
    uint4 graw[NKK][GB ? 1 : 2];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if constexpr (GB) {
            graw[kk][0] = load16_input<NT>(static_cast<const uint16_t *>(p.g) + grow + 32 * kk);
        } else {
            graw[kk][0] = load16_input<NT>(static_cast<const float *>(p.g) + grow + 32 * kk);
            graw[kk][1] = load16_input<NT>(static_cast<const float *>(p.g) + grow + 32 * kk + 4);
        }
    }
    // dt_bias for this lane's 8-column groups (read by both activated-gate forms)
    static_assert(K <= 256, "zero bias size");
    const float *dtb_row = p.dt_bias ? p.dt_bias + (int64_t)hv * K : kda_zero_bias;
    float4 dtbv[NKK][2];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        dtbv[kk][0] = *reinterpret_cast<const float4 *>(dtb_row + 32 * kk + 8 * cg);
        dtbv[kk][1] = *reinterpret_cast<const float4 *>(dtb_row + 32 * kk + 8 * cg + 4);
    }
    const int64_t bidx = (ci.tok0 + rl) * p.HV + hv;
    uint32_t bbits;
    if constexpr (BB) bbits = static_cast<const uint16_t *>(p.beta)[bidx];
    else bbits = __float_as_uint(static_cast<const float *>(p.beta)[bidx]);
    uint4 qv[NKK], kv[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        qv[kk] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.q) + qkrow + 32 * kk);
        kv[kk] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.k) + qkrow + 32 * kk);
    }
    const float braw = __uint_as_float(BB ? bbits << 16 : bbits);
    float G[NKK][8];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if constexpr (GB) {
            unpack8(graw[kk][0], G[kk]);
        } else {
            const uint4 a = graw[kk][0], b = graw[kk][1];
            G[kk][0] = __uint_as_float(a.x), G[kk][1] = __uint_as_float(a.y), G[kk][2] = __uint_as_float(a.z);
            G[kk][3] = __uint_as_float(a.w), G[kk][4] = __uint_as_float(b.x), G[kk][5] = __uint_as_float(b.y);
            G[kk][6] = __uint_as_float(b.z), G[kk][7] = __uint_as_float(b.w);
        }
    }

    // ---- step 1: activated gate in log2 units (rows past the end contribute 0), 16-row
    //      inclusive scan; one loop per gate form so the element loop has no branch ----
    {
        const float a = p.A_log ? expf(p.A_log[hv]) : 1.f;
        const float unit = valid ? kLog2e : 0.f;
        auto act = [&](auto mode_tag) {
            constexpr int M = decltype(mode_tag)::value;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const float dtb[8] = {dtbv[kk][0].x, dtbv[kk][0].y, dtbv[kk][0].z, dtbv[kk][0].w,
                                      dtbv[kk][1].x, dtbv[kk][1].y, dtbv[kk][1].z, dtbv[kk][1].w};
#pragma unroll
                for (int i = 0; i < 8; ++i) G[kk][i] = gate_act(M, G[kk][i], dtb[i], a, p.lower_bound, unit);
            }
        };
        if (p.gate_mode == kGateLowerBound) act(std::integral_constant<int, kGateLowerBound>{});
        else if (p.gate_mode == kGateSoftplus) act(std::integral_constant<int, kGateSoftplus>{});
        else act(std::integral_constant<int, kGatePre>{});
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int i = 0; i < 8; ++i) G[kk][i] = row_scan16(G[kk][i]);

    // ---- step 2: block column values -> LDS; beta; norms ----
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        const int d0 = 32 * kk + 8 * cg;
        if (lr == 0) store8(CV0 + w * K + d0, G[kk]);
        if (lr == 8) store8(CV8 + w * K + d0, G[kk]);
        if (lr == 15) store8(CV15 + w * K + d0, G[kk]);
    }
    const float b_r = valid ? beta_act(p.beta_mode, braw) : 0.f;
    if (cg == 0) betas[r] = b_r;
    if (threadIdx.x < NB) wideflag[threadIdx.x] = 0;
    float rq = p.scale, rk = 1.f;
    if (p.qk_l2norm) {
        float ssq = 0.f, ssk = 0.f;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            ssq = dot2_bf16(qv[kk].x, qv[kk].x, ssq);
            ssq = dot2_bf16(qv[kk].y, qv[kk].y, ssq);
            ssq = dot2_bf16(qv[kk].z, qv[kk].z, ssq);
            ssq = dot2_bf16(qv[kk].w, qv[kk].w, ssq);
            ssk = dot2_bf16(kv[kk].x, kv[kk].x, ssk);
            ssk = dot2_bf16(kv[kk].y, kv[kk].y, ssk);
            ssk = dot2_bf16(kv[kk].z, kv[kk].z, ssk);
            ssk = dot2_bf16(kv[kk].w, kv[kk].w, ssk);
        }
        ssq = sum_col_groups(ssq);
        ssk = sum_col_groups(ssk);
        rq *= rsqrtf(ssq + 1e-6f);
        rk = rsqrtf(ssk + 1e-6f);
    }
    if (!valid) rq = rk = 0.f;
    __syncthreads();

    // ---- step 3: column pass -> per-column scalars ----
    for (int d = threadIdx.x; d < K; d += blockDim.x) {
        float P = 0.f, gn[NB], gm[NB], ge[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float v0 = CV0[b * K + d], v8 = CV8[b * K + d], v15 = CV15[b * K + d];
            gn[b] = P + v0;
            gm[b] = P + v8;
            P += v15;
            ge[b] = P;
            if (fabsf(v0 - v8) > kDiagSpanLimit || fabsf(v8 - v15) > kDiagSpanLimit) wideflag[b] = 1;
            Ssa[b * K + d] = fast_exp2(v0 - v8);
            Ssb[b * K + d] = fast_exp2(v8 - v15);
            Scn[b * K + d] = fast_exp2(gn[b]);
        }
        dg[d] = fast_exp2(P);
#pragma unroll
        for (int b = 0; b < NB; ++b) Sck[b * K + d] = fast_exp2(P - ge[b]);
#pragma unroll
        for (int wb = 1; wb < NB; ++wb)
#pragma unroll
            for (int sb = 0; sb < wb; ++sb) SIG[pair_of(wb, sb) * K + d] = fast_exp2(gn[wb] - ge[sb]);
    }
    __syncthreads();
    const bool wide = wideflag[w] != 0;

    // ---- step 4: own-block operands ----
    //   QR = q^ Rf, KR = k^ Rf, KC = k^ Cf  (Rf = 2^(G - G_first), Cf = 2^(G_lastrow - G))
    //   diagonal: (KC sb) . (QR sa) = q^_i k^_j 2^(G_i - G_j) with both factors split at the midpoint
    //   Qg = QR cn, X = KR cn, KgT = KC ck
    f32x4 accQd = zero4(), accKd = zero4();
    if (wide) {
        // element-wise diagonal block: 2^(G_i - G_j) with j <= i taken directly (<= 1)
        for (int jr = 0; jr < 16; ++jr) {
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                float qf[8], kf[8];
                unpack8(qv[kk], qf);
                unpack8(kv[kk], kf);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float kn = kf[i] * rk;
                    const float kj = shfl(kn, (l & 0x30) + jr);
                    const float gj = shfl(G[kk][i], (l & 0x30) + jr);
                    const float f = lr >= jr ? fast_exp2(G[kk][i] - gj) : 0.f;
                    sq += qf[i] * rq * kj * f;
                    sk += kn * kj * f;
                }
            }
            sq = sum_col_groups(sq);
            sk = sum_col_groups(sk);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                if (4 * cg + jj == jr) {
                    accQd[jj] = sq;
                    accKd[jj] = sk;
                }
        }
    }
    const uint4 sel0 = select_frag(0), sel1 = select_frag(16);
    uint4 QRp[NKK], KRp[NKK], Xp[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        const int d0 = 32 * kk + 8 * cg;
        float g0[8], g15[8], sa[8], sb[8], cn[8], ck[8], qf[8], kf[8];
        load8(CV0 + w * K + d0, g0);
        load8(CV15 + w * K + d0, g15);
        load8(Ssa + w * K + d0, sa);
        load8(Ssb + w * K + d0, sb);
        load8(Scn + w * K + d0, cn);
        load8(Sck + w * K + d0, ck);
        unpack8(qv[kk], qf);
        unpack8(kv[kk], kf);
        float qr[8], kr[8], kc[8], a1[8], a2[8], b1[8], qg[8], x[8], kt[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float rf = fast_exp2(G[kk][i] - g0[i]);
            const float cf = fast_exp2(g15[i] - G[kk][i]);
            qr[i] = qf[i] * rq * rf;
            kr[i] = kf[i] * rk * rf;
            kc[i] = kf[i] * rk * cf;
            a1[i] = qr[i] * sa[i];
            a2[i] = kr[i] * sa[i];
            b1[i] = kc[i] * sb[i];
            qg[i] = qr[i] * cn[i];
            x[i] = kr[i] * cn[i];
            kt[i] = kc[i] * ck[i];
        }
        QRp[kk] = pack8(qr);
        KRp[kk] = pack8(kr);
        Xp[kk] = pack8(x);
        if (!wide) {
            const uint4 b1p = pack8(b1);
            accQd = mma32_bf16(accQd, b1p, pack8(a1));
            accKd = mma32_bf16(accKd, b1p, pack8(a2));
        }
        if constexpr (PERM) {
            *reinterpret_cast<uint2 *>(Qgg + pfrag_off(r, d0, K)) = make_uint2(pack2(qg[0], qg[1]), pack2(qg[2], qg[3]));
            *reinterpret_cast<uint2 *>(Qgg + pfrag_off(r, d0 + 4, K)) =
                make_uint2(pack2(qg[4], qg[5]), pack2(qg[6], qg[7]));
        } else {
            *reinterpret_cast<uint4 *>(Qgg + frag_off(r, d0, K)) = pack8(qg);
        }
        if (w < NB - 1) OPS[(w * NKK + kk) * 64 + l] = pack8(kc);
        // KgT: transpose the 16x32 block on the matrix cores, stage [d][m] in LDS
        const uint4 ktp = pack8(kt);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const f32x4 t = mma32_bf16(zero4(), ktp, hh ? sel1 : sel0);
            *reinterpret_cast<uint2 *>(KST + swz<C>(32 * kk + 16 * hh + lr, 16 * w + 4 * cg)) =
                make_uint2(pack2(t[0], t[1]), pack2(t[2], t[3]));
        }
    }
    __syncthreads();  // pair sources and KgT staging complete; column values no longer read

    // ---- step 5: off-diagonal blocks (pairwise offsets), masks, stores ----
    f32x4 accQ[NB], accK[NB];
#pragma unroll
    for (int s = 0; s < NB; ++s) accQ[s] = accK[s] = zero4();
#pragma unroll
    for (int s = 0; s < NB - 1; ++s) {
        if (s < w) {
            const float *sg = SIG + pair_of(w, s) * K;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                float src[8], sc8[8];
                unpack8(OPS[(s * NKK + kk) * 64 + l], src);
                load8(sg + 32 * kk + 8 * cg, sc8);
#pragma unroll
                for (int i = 0; i < 8; ++i) src[i] *= sc8[i];
                const uint4 ap = pack8(src);
                accQ[s] = mma32_bf16(accQ[s], ap, QRp[kk]);
                accK[s] = mma32_bf16(accK[s], ap, KRp[kk]);
            }
        }
    }
    // KgT staging -> global (each 16-byte unit u sits at element 8u of the fragment-major layout).
    // K C / 8 units over NB waves of 64 lanes: NKK rounds, unit u = threadIdx.x + round * 64 NB,
    // i.e. fragment tile w + round * NB, lane l (unrolled, so the addressing folds to constants)
    static_assert(K * C / 8 == NKK * NB * 64, "KgT units per round");
#pragma unroll
    for (int it = 0; it < NKK; ++it) {
        const int tile = w + it * NB;
        const int u = tile * 64 + l;
        const int d = 16 * (tile / (C / 32)) + lr;
        if constexpr (PERM) {
            // lane group g of a unit holds columns 4g..4g+3 and 16+4g..16+4g+3 of its 32-column block
            const int m0 = 32 * (tile % (C / 32)) + 4 * cg;
            const uint2 a = *reinterpret_cast<const uint2 *>(KST + swz<C>(d, m0));
            const uint2 b = *reinterpret_cast<const uint2 *>(KST + swz<C>(d, m0 + 16));
            *reinterpret_cast<uint4 *>(KgTg + (size_t)u * 8) = make_uint4(a.x, a.y, b.x, b.y);
        } else {
            const int m0 = 32 * (tile % (C / 32)) + 8 * cg;
            *reinterpret_cast<uint4 *>(KgTg + (size_t)u * 8) = *reinterpret_cast<const uint4 *>(KST + swz<C>(d, m0));
        }
    }
    uint2 aqp[NB];
#pragma unroll
    for (int s = 0; s < NB; ++s) {
        float aq[4], ak[4];
        const f32x4 vq = (s == w) ? accQd : accQ[s], vk = (s == w) ? accKd : accK[s];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int jl = 4 * cg + jj;
            aq[jj] = (s < w || (s == w && jl <= lr)) ? vq[jj] : 0.f;
            ak[jj] = (s < w || (s == w && jl < lr)) ? b_r * vk[jj] : 0.f;
        }
        aqp[s] = make_uint2(pack2(aq[0], aq[1]), pack2(aq[2], aq[3]));
        store4(Akk + r * LDA + 16 * s + 4 * cg, ak[0], ak[1], ak[2], ak[3]);
    }
    if constexpr (PERM) {
        // columns 16s + 4cg.. of blocks 2m and 2m + 1 are adjacent 8-byte halves of one
        // 16-byte unit: one full store per block pair.  Pairs right of the diagonal block
        // (32m > 16w + 15) are zero and never read by the register-resident recurrence,
        // which loads only the units at or left of it; they are not written.
#pragma unroll
        for (int m = 0; m < NB / 2; ++m)
            if (32 * m <= 16 * w + 15)
                *reinterpret_cast<uint4 *>(Aqkg + pfrag_off(r, 32 * m + 4 * cg, C)) =
                    make_uint4(aqp[2 * m].x, aqp[2 * m].y, aqp[2 * m + 1].x, aqp[2 * m + 1].y);
    } else {
#pragma unroll
        for (int s = 0; s < NB; ++s) *reinterpret_cast<uint2 *>(Aqkg + frag_off(r, 16 * s + 4 * cg, C)) = aqp[s];
    }
    // v rows for U: the first four 32-column slices are loaded now, so their latency
    // overlaps the solve
    const int nvk = V / 32;
    const uint16_t *vrow = static_cast<const uint16_t *>(p.v) + ((ci.tok0 + rl) * p.HV + hv) * (int64_t)V + 8 * cg;
    uint4 vpre[4];
#pragma unroll
    for (int vk = 0; vk < 4; ++vk)
        if (vk < nvk) vpre[vk] = load16_input<NT>(vrow + 32 * vk);
    __syncthreads();  // Akk complete

    // ---- step 6: A = (I + Akk0)^-1, fp32 ----
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

    // ---- step 7: X^T and v^T into LDS (matrix-core transposes); A Diag(b) rows ----
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const f32x4 t = mma32_bf16(zero4(), Xp[kk], hh ? sel1 : sel0);
            *reinterpret_cast<uint2 *>(XT + swz<C>(32 * kk + 16 * hh + lr, 16 * w + 4 * cg)) =
                make_uint2(pack2(t[0], t[1]), pack2(t[2], t[3]));
        }
    }
#pragma unroll
    for (int vk = 0; vk < 8; ++vk) {
        if (vk < nvk) {
            const uint4 vv = vk < 4 ? vpre[vk & 3] : load16_input<NT>(vrow + 32 * vk);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const f32x4 t = mma32_bf16(zero4(), vv, hh ? sel1 : sel0);
                *reinterpret_cast<uint2 *>(VT + swz<C>(32 * vk + 16 * hh + lr, 16 * w + 4 * cg)) =
                    make_uint2(pack2(t[0], t[1]), pack2(t[2], t[3]));
            }
        }
    }
    // rows of A Diag(b) as bf16 operands: row block w for W, row block NB-1-w for U, so
    // every wave does the same number of products (block b needs (b+2)/2 32-column spans)
    const int bw = w, bu = NB - 1 - w;
    const int nmw = (16 * bw + 16 + 31) / 32, nmu = (16 * bu + 16 + 31) / 32;
    auto a_rows = [&](int b, int nm, uint4 (&am)[2]) {
#pragma unroll
        for (int ms = 0; ms < 2; ++ms) {
            if (ms < nm) {
                float a8[8], b8[8];
                load8(Ainv + (16 * b + lr) * LDA + 32 * ms + 8 * cg, a8);
                load8(betas + 32 * ms + 8 * cg, b8);
#pragma unroll
                for (int i = 0; i < 8; ++i) a8[i] *= b8[i];
                am[ms] = pack8(a8);
            } else {
                am[ms] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };
    uint4 amw[2], amu[2];
    a_rows(bw, nmw, amw);
    a_rows(bu, nmu, amu);
    __syncthreads();

    // ---- step 8: W = A Diag(b) X (lane: row m = 16bw+lr, columns 16dt+4cg..),
    //      U = A Diag(b) v (lane: rows m = 16bu+4cg.., column 16vt+lr) ----
    // (loops unrolled so each wave's LDS operand reads are in flight together rather than
    // one read-multiply-store round trip per tile)
    const int rw = 16 * bw + lr;
#pragma unroll
    for (int dp = 0; dp < K / 32; ++dp) {
        uint2 wq[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int dt = 2 * dp + hh;
            f32x4 acc = zero4();
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
                if (ms < nmw)
                    acc = mma32_bf16(acc, *reinterpret_cast<const uint4 *>(XT + swz<C>(16 * dt + lr, 32 * ms + 8 * cg)),
                                     amw[ms]);
            wq[hh] = make_uint2(pack2(acc[0], acc[1]), pack2(acc[2], acc[3]));
        }
        if constexpr (PERM) {  // the two 16-column tiles fill one 16-byte unit
            *reinterpret_cast<uint4 *>(Wg + pfrag_off(rw, 32 * dp + 4 * cg, K)) = make_uint4(wq[0].x, wq[0].y, wq[1].x, wq[1].y);
        } else {
            *reinterpret_cast<uint2 *>(Wg + frag_off(rw, 32 * dp + 4 * cg, K)) = wq[0];
            *reinterpret_cast<uint2 *>(Wg + frag_off(rw, 32 * dp + 16 + 4 * cg, K)) = wq[1];
        }
    }
    for (int vt0 = 0; vt0 < V / 16; vt0 += 2) {  // V is a multiple of 32
        uint4 vb[2][2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
                vb[hh][ms] = ms < nmu ? *reinterpret_cast<const uint4 *>(VT + swz<C>(16 * (vt0 + hh) + lr, 32 * ms + 8 * cg))
                                      : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            f32x4 acc = zero4();
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
                if (ms < nmu) acc = mma32_bf16(acc, amu[ms], vb[hh][ms]);
            *reinterpret_cast<uint2 *>(UTg + quad_off(16 * bu + 4 * cg, 16 * (vt0 + hh) + lr, C)) =
                make_uint2(pack2(acc[0], acc[1]), pack2(acc[2], acc[3]));
        }
    }
}

template <int C, int NKK>
hipError_t launch_intra_bf16_t(const Params &p, hipStream_t s) {
    const size_t lds = IntraBf16Lds<C, 32 * NKK>::bytes(p.V);
    // bytes of intermediates per (chunk, value head): W, U, KgT, Qg, Aqk (bf16) and d (fp32)
    const size_t slot_bytes = 2 * ((size_t)3 * C * (32 * NKK) + (size_t)C * p.V + (size_t)C * C) + 4 * (32 * NKK);
    const bool nt = (size_t)p.total_chunks * p.HV * slot_bytes <= kOnceLoadMaxIntermediates;
    auto pick = [&](auto nt_tag) {
        constexpr bool T = decltype(nt_tag)::value;
        return p.g_bf16 ? (p.beta_bf16 ? intra_bf16_kernel<C, NKK, true, true, T> : intra_bf16_kernel<C, NKK, true, false, T>)
                        : (p.beta_bf16 ? intra_bf16_kernel<C, NKK, false, true, T> : intra_bf16_kernel<C, NKK, false, false, T>);
    };
    auto kern = nt ? pick(std::true_type{}) : pick(std::false_type{});
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)p.total_chunks * (unsigned)p.HV), dim3(64 * (C / 16)), lds, s, p);
    return hipGetLastError();
}

template <int C>
hipError_t launch_intra_bf16_c(const Params &p, hipStream_t s) {
    switch (p.K / 32) {
    case 1: return launch_intra_bf16_t<C, 1>(p, s);
    case 2: return launch_intra_bf16_t<C, 2>(p, s);
    case 3: return launch_intra_bf16_t<C, 3>(p, s);
    case 4: return launch_intra_bf16_t<C, 4>(p, s);
    case 5: return launch_intra_bf16_t<C, 5>(p, s);
    case 6: return launch_intra_bf16_t<C, 6>(p, s);
    case 7: return launch_intra_bf16_t<C, 7>(p, s);
    case 8: return launch_intra_bf16_t<C, 8>(p, s);
    }
    return hipErrorInvalidValue;
}

template <int C>
size_t intra_bf16_lds(int K, int V) {
    switch (K / 32) {
    case 1: return IntraBf16Lds<C, 32>::bytes(V);
    case 2: return IntraBf16Lds<C, 64>::bytes(V);
    case 3: return IntraBf16Lds<C, 96>::bytes(V);
    case 4: return IntraBf16Lds<C, 128>::bytes(V);
    case 5: return IntraBf16Lds<C, 160>::bytes(V);
    case 6: return IntraBf16Lds<C, 192>::bytes(V);
    case 7: return IntraBf16Lds<C, 224>::bytes(V);
    case 8: return IntraBf16Lds<C, 256>::bytes(V);
    }
    return 0;
}

}  // namespace kda
