// kda_intra.hip -- intra-chunk stage of the KDA forward, one workgroup per
// (chunk, value head), one wave per 16-row sub-chunk.
//
// Per chunk, with G the base-2 chunk-local cumulative gate, q^ = scale*q/|q|,
// k^ = k/|k| and beta b ("Reading Notes: Implementation Notes for KDA in FLA",
// forward steps 1-3):
//   Aqk[i][j]  = sum_d q^_id k^_jd 2^(G_id - G_jd)          (j <= i)
//   Akk0[i][j] = b_i sum_d k^_id k^_jd 2^(G_id - G_jd)      (j <  i)
//   A = (I + Akk0)^-1,  W = A (b * 2^G * k^),  U = A (b * v)
//   Qg = 2^G * q^,  KgT = (2^(G_last - G) * k^)^T,  d = 2^G_last
// which the recurrence kernel consumes.
//
// Exponent handling ("flash-linear-attention KDA 内核工程实践…", §3.1 and §3.2):
//   - sub-chunk pairs (p > s) factor 2^(G_i - G_j) as 2^(G_i - G_n) * 2^(G_n - G_j)
//     with n the first row of sub-chunk p; every exponent is <= 0.  Here the
//     second factor is split once more, 2^(G_n - G_e) * 2^(G_e - G_j) with e the
//     last row of sub-chunk s, so each row's two exp2 factors are computed once
//     and only a per-column scalar depends on the pair.
//   - diagonal sub-chunks subtract the cumulative gate at the sub-chunk midpoint
//     (row min(8, rows left - 1)), so both operand exponents stay small.  The
//     kernel checks that |G - G_mid| <= 60 over the sub-chunk (always true for
//     the bounded gate with lower_bound >= -5, where it is at most 8*5*log2(e));
//     otherwise that block falls back to element-wise exp2 of non-positive
//     differences, the token-parallel form of §4.
//   - the diagonal 16x16 blocks of I + Akk0 are inverted by forward substitution
//     in fp32 and merged into the full inverse block by block (§3.1, §4), here on
//     fp32 matrix cores.
#include "kda_gate.h"

namespace kda {

constexpr float kDiagSpanLimit = 60.f;

template <int C, typename T>
struct IntraLds {
    // byte offsets into dynamic LDS
    static constexpr int NB = C / 16;
    static __host__ __device__ int ldk(int K) { return K + 8; }           // KCs row stride (elements)
    static __host__ __device__ int ldc() { return C + 8; }                 // XT / VT row stride (elements)
    static constexpr int LDA = C + 4;                                      // Akk / Ainv row stride (floats)
    static __host__ __device__ size_t tot(int) { return 0; }
    static __host__ __device__ size_t ge(int K) { return tot(K) + sizeof(float) * NB * K; }
    static __host__ __device__ size_t glast(int K) { return ge(K) + sizeof(float) * NB * K; }
    static __host__ __device__ size_t beta(int K) { return glast(K) + sizeof(float) * K; }
    static __host__ __device__ size_t ainv(int K) { return beta(K) + sizeof(float) * C; }
    static __host__ __device__ size_t region(int K) { return ainv(K) + sizeof(float) * C * LDA; }
    // region, phase 1: KCs [C][K+8] then Akk [C][LDA]
    static __host__ __device__ size_t kcs(int K) { return region(K); }
    static __host__ __device__ size_t akk(int K) {
        return (kcs(K) + sizeof(T) * C * ldk(K) + 15) / 16 * 16;
    }
    // region, phase 2: XT [K][C+8] then VT [V][C+8]
    static __host__ __device__ size_t xt(int K) { return region(K); }
    static __host__ __device__ size_t vt(int K) { return xt(K) + sizeof(T) * K * ldc(); }
    static __host__ __device__ size_t bytes(int K, int V) {
        const size_t p1 = akk(K) + sizeof(float) * C * LDA;
        const size_t p2 = vt(K) + sizeof(T) * V * ldc();
        return p1 > p2 ? p1 : p2;
    }
};

// 16x16x16 fp32 product on matrix cores: acc += X(16x16) * Y(16x16), X row-major
// in LDS with stride ldx, Y row-major in LDS with stride ldy.  Lane group cg
// supplies contraction indices 4*cg + q (q < 4).
__device__ __forceinline__ f32x4 mma16_f32_lds(f32x4 acc, const float *X, int ldx, const float *Y, int ldy) {
    const int l = lane_id(), r = l & 15, cg = l >> 4;
    const float4 a = *reinterpret_cast<const float4 *>(X + r * ldx + 4 * cg);
    const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], Y[(4 * cg + q) * ldy + r], acc, 0, 0, 0);
    return acc;
}

template <int C, typename T, int NKK>
__global__ void __launch_bounds__(C / 16 * 64) intra_kernel(Params p) {
    constexpr int NB = C / 16;
    constexpr bool F32 = sizeof(T) == 4;
    using L_ = IntraLds<C, T>;
    extern __shared__ __align__(16) unsigned char lds[];
    const int K = p.K, V = p.V;
    const int nkk = K / 32, nvk = V / 32;
    float *tot = reinterpret_cast<float *>(lds + L_::tot(K));
    float *GeS = reinterpret_cast<float *>(lds + L_::ge(K));
    float *GlastS = reinterpret_cast<float *>(lds + L_::glast(K));
    float *betaS = reinterpret_cast<float *>(lds + L_::beta(K));
    float *Ainv = reinterpret_cast<float *>(lds + L_::ainv(K));
    T *KCs = reinterpret_cast<T *>(lds + L_::kcs(K));
    float *Akk = reinterpret_cast<float *>(lds + L_::akk(K));
    T *XT = reinterpret_cast<T *>(lds + L_::xt(K));
    T *VTs = reinterpret_cast<T *>(lds + L_::vt(K));
    const int LDK = L_::ldk(K), LDC = L_::ldc();
    constexpr int LDA = L_::LDA;

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
    T *Ug = static_cast<T *>(p.w_U) + slot * C * V;
    T *KgTg = static_cast<T *>(p.w_KgT) + slot * K * C;
    T *Qgg = static_cast<T *>(p.w_Qg) + slot * C * K;
    T *Aqkg = static_cast<T *>(p.w_Aqk) + slot * C * C;
    float *dg = p.w_d + slot * K;

    // ---- step 1: gate activation + base-2 chunk-local cumsum (row fragment) ----
    float G[NKK][8], scratch[NKK][8];
    gate_cumsum_block<NKK>(p, ci, hv, w, nkk, G, tot, scratch);

    // reference rows of this sub-chunk (clamped for sub-chunks past the end)
    int e_loc = ci.L - 1 - 16 * w;
    e_loc = e_loc > 15 ? 15 : (e_loc < 0 ? 0 : e_loc);
    const int mid_loc = e_loc < 8 ? e_loc : 8;
    const int base = l & 0x30;

    // ---- step 2: q^, k^, beta ----
    float qh[NKK][8], kh[NKK][8];
    const int64_t qrow = ((ci.tok0 + r) * p.H + h) * (int64_t)K;
    float ssq = 0.f, ssk = 0.f;
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
    const float b_r = valid ? beta_act(p.beta_mode, load_any(p.beta, (ci.tok0 + r) * p.HV + hv, p.beta_bf16)) : 0.f;
    if (cg == 0) betaS[r] = b_r;

    // ---- step 3: per-element exp2 factors and operands ----
    //   QR = q^ 2^(G - G_n), KR = k^ 2^(G - G_n), KC = k^ 2^(G_e - G)
    float QR[NKK][8], KR[NKK][8], KC[NKK][8], En[NKK][8], Ge[NKK][8];
    bool wide = false;  // some |G - G_mid| beyond the limit: diagonal needs the fallback
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if (kk < nkk) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float g = G[kk][i];
                const float gn = shfl(g, base);
                const float ge = shfl(g, base + e_loc);
                const float gm = shfl(g, base + mid_loc);
                wide |= fabsf(g - gm) > kDiagSpanLimit;
                const float qn = qh[kk][i] * rq, kn = kh[kk][i] * rk;
                qh[kk][i] = qn;
                kh[kk][i] = kn;
                const float rf = exp2f(g - gn);
                QR[kk][i] = qn * rf;
                KR[kk][i] = kn * rf;
                KC[kk][i] = kn * exp2f(ge - g);
                En[kk][i] = exp2f(gn);
                Ge[kk][i] = ge;
                scratch[kk][i] = gm;  // G at the midpoint row
            }
            // KC rows -> LDS (row-major), Qg rows -> global
            float kc8[8], qg8[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                kc8[i] = KC[kk][i];
                qg8[i] = QR[kk][i] * En[kk][i];
            }
            store8(KCs + r * LDK + 32 * kk + 8 * cg, kc8);
            store8(Qgg + (size_t)r * K + 32 * kk + 8 * cg, qg8);
            if (lr == 0) {
#pragma unroll
                for (int i = 0; i < 8; ++i) GeS[w * K + 32 * kk + 8 * cg + i] = Ge[kk][i];
            }
            if (16 * w + e_loc == ci.L - 1 && lr == 0) {
#pragma unroll
                for (int i = 0; i < 8; ++i) GlastS[32 * kk + 8 * cg + i] = Ge[kk][i];
            }
        }
    }
    const bool diag_fallback = __any(wide);
    __syncthreads();

    // ---- step 4: KgT = (k^ 2^(G_last - G))^T and d = 2^G_last -> global ----
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if (kk < nkk) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int d = 32 * kk + 8 * cg + i;
                const float kg = KC[kk][i] * exp2f(GlastS[d] - Ge[kk][i]);
                KgTg[(size_t)d * C + r] = Store<T>::to(kg);
            }
        }
    }
    for (int d = threadIdx.x; d < K; d += blockDim.x) dg[d] = exp2f(GlastS[d]);

    // ---- step 5: Aqk, Akk0 for row block w (16x16 tiles against blocks s <= w) ----
    f32x4 accQ[NB], accK[NB];
#pragma unroll
    for (int s = 0; s < NB; ++s) accQ[s] = accK[s] = zero4();
#pragma unroll
    for (int s = 0; s < NB; ++s) {
        if (s < w) {
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                if (kk < nkk) {
                    float aq[8], ak[8], bk[8];
                    load8(KCs + (16 * s + lr) * LDK + 32 * kk + 8 * cg, bk);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int d = 32 * kk + 8 * cg + i;
                        // 2^(G_n(w) - G_e(s)) <= 1, the pair's decay between the sub-chunks
                        const float sig = exp2f(shfl(G[kk][i], base) - GeS[s * K + d]);
                        aq[i] = QR[kk][i] * sig;
                        ak[i] = KR[kk][i] * sig;
                    }
                    accQ[s] = mma32<F32>(accQ[s], aq, bk);
                    accK[s] = mma32<F32>(accK[s], ak, bk);
                }
            }
        }
    }
    if (!diag_fallback) {
        // midpoint split: (q^ 2^(G_i - G_mid)) . (k^ 2^(G_mid - G_j))
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            if (kk < nkk) {
                float aq[8], ak[8], bk[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float gn = shfl(G[kk][i], base), gm = scratch[kk][i];
                    const float sa = exp2f(gn - gm), sb = exp2f(gm - Ge[kk][i]);
                    aq[i] = QR[kk][i] * sa;
                    ak[i] = KR[kk][i] * sa;
                    bk[i] = KC[kk][i] * sb;
                }
                accQ[w] = mma32<F32>(accQ[w], aq, bk);
                accK[w] = mma32<F32>(accK[w], ak, bk);
            }
        }
    }
    // mask, beta, store: Aqk -> global, Akk0 -> LDS (fp32)
#pragma unroll
    for (int s = 0; s < NB; ++s) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int row = 4 * cg + jj;            // row inside block w
            const int i = 16 * w + row, j = 16 * s + lr;
            float aq = accQ[s][jj], ak = accK[s][jj];
            if (s > w || (s == w && lr > row)) aq = 0.f;
            if (s > w || (s == w && lr >= row)) ak = 0.f;
            ak *= shfl(b_r, row);
            if (!(s == w && diag_fallback)) {
                Aqkg[(size_t)i * C + j] = Store<T>::to(aq);
                Akk[i * LDA + j] = ak;
            }
        }
    }
    if (diag_fallback) {
        // element-wise diagonal block: every factor is 2^(G_i - G_j) with j <= i (<= 1)
        for (int jr = 0; jr < 16; ++jr) {
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                if (kk < nkk) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float kj = shfl(kh[kk][i], base + jr);
                        const float gj = shfl(G[kk][i], base + jr);
                        const float f = lr >= jr ? exp2f(G[kk][i] - gj) : 0.f;
                        sq += qh[kk][i] * kj * f;
                        sk += kh[kk][i] * kj * f;
                    }
                }
            }
            sq = sum_col_groups(sq);
            sk = sum_col_groups(sk);
            if (cg == 0) {
                Aqkg[(size_t)r * C + 16 * w + jr] = Store<T>::to(lr >= jr ? sq : 0.f);
                Akk[r * LDA + 16 * w + jr] = lr > jr ? b_r * sk : 0.f;
            }
        }
    }
    __syncthreads();

    // ---- step 6: A = (I + Akk0)^-1, fp32 ----
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
    // zero the strictly upper blocks of row block w
    for (int s = w + 1; s < NB; ++s)
        for (int e = l; e < 256; e += 64) Ainv[(16 * w + (e >> 4)) * LDA + 16 * s + (e & 15)] = 0.f;
    __syncthreads();
    // off-diagonal blocks by distance: A_ws = -D_w * sum_{m=s}^{w-1} L_wm A_ms
#pragma unroll
    for (int dist = 1; dist < NB; ++dist) {
        if (w >= dist) {
            const int s = w - dist;
            f32x4 t = zero4();
            for (int m = s; m < w; ++m)
                t = mma16_f32_lds(t, Akk + (16 * w) * LDA + 16 * m, LDA, Ainv + (16 * m) * LDA + 16 * s, LDA);
            // D_w * t: t is already in the B-operand layout (lane's own acc rows 4cg+q)
            const float4 a = *reinterpret_cast<const float4 *>(Ainv + (16 * w + lr) * LDA + 16 * w + 4 * cg);
            const float av[4] = {a.x, a.y, a.z, a.w};
            f32x4 u = zero4();
#pragma unroll
            for (int q = 0; q < 4; ++q) u = __builtin_amdgcn_mfma_f32_16x16x4f32(av[q], t[q], u, 0, 0, 0);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) Ainv[(16 * w + 4 * cg + jj) * LDA + 16 * s + lr] = -u[jj];
        }
        __syncthreads();
    }

    // ---- step 7: W = A (b 2^G k^), U = A (b v) ----
    // XT[d][m] = b_m k^_md 2^(G_md) (= b KR 2^G_n), VT[n][m] = b_m v_mn  (LDS, transposed)
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if (kk < nkk) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                XT[(32 * kk + 8 * cg + i) * LDC + r] = Store<T>::to(b_r * KR[kk][i] * En[kk][i]);
        }
    }
    const int64_t vrow = ((ci.tok0 + r) * p.HV + hv) * (int64_t)V;
#pragma unroll
    for (int vk = 0; vk < NKK; ++vk) {
        if (vk < nvk) {
            float x[8];
            if (valid) load8(static_cast<const T *>(p.v) + vrow + 32 * vk + 8 * cg, x);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                VTs[(32 * vk + 8 * cg + i) * LDC + r] = Store<T>::to(valid ? b_r * x[i] : 0.f);
        }
    }
    __syncthreads();
    {
        const int nms = (16 * w + 16 + 31) / 32;
        float am[2][8];
#pragma unroll
        for (int ms = 0; ms < 2; ++ms)
            if (ms < nms) load8(Ainv + (16 * w + lr) * LDA + 32 * ms + 8 * cg, am[ms]);
        for (int ct = 0; ct < K / 16; ++ct) {
            f32x4 acc = zero4();
#pragma unroll
            for (int ms = 0; ms < 2; ++ms) {
                if (ms < nms) {
                    float bx[8];
                    load8(XT + (16 * ct + lr) * LDC + 32 * ms + 8 * cg, bx);
                    acc = mma32<F32>(acc, am[ms], bx);
                }
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                Wg[(size_t)(16 * w + 4 * cg + jj) * K + 16 * ct + lr] = Store<T>::to(acc[jj]);
        }
        for (int ct = 0; ct < V / 16; ++ct) {
            f32x4 acc = zero4();
#pragma unroll
            for (int ms = 0; ms < 2; ++ms) {
                if (ms < nms) {
                    float bx[8];
                    load8(VTs + (16 * ct + lr) * LDC + 32 * ms + 8 * cg, bx);
                    acc = mma32<F32>(acc, am[ms], bx);
                }
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                Ug[(size_t)(16 * w + 4 * cg + jj) * V + 16 * ct + lr] = Store<T>::to(acc[jj]);
        }
    }
}

template <int C, typename T, int NKK>
static hipError_t launch_intra_t(const Params &p, hipStream_t s) {
    const size_t lds = IntraLds<C, T>::bytes(p.K, p.V);
    auto kern = intra_kernel<C, T, NKK>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)p.total_chunks * (unsigned)p.HV), dim3(64 * (C / 16)), lds, s, p);
    return hipGetLastError();
}

template <int C, typename T>
static hipError_t launch_intra_c(const Params &p, hipStream_t s) {
    const int dmax = p.K > p.V ? p.K : p.V;
    return dmax <= 128 ? launch_intra_t<C, T, 4>(p, s) : launch_intra_t<C, T, 8>(p, s);
}

size_t intra_lds_bytes(int C, int K, int V, bool bf16) {
    if (C == 64) return bf16 ? IntraLds<64, uint16_t>::bytes(K, V) : IntraLds<64, float>::bytes(K, V);
    return bf16 ? IntraLds<32, uint16_t>::bytes(K, V) : IntraLds<32, float>::bytes(K, V);
}

hipError_t launch_intra(const Params &p, hipStream_t s) {
    if (p.total_chunks == 0) return hipSuccess;
    if (p.C == 64) return p.qkv_bf16 ? launch_intra_c<64, uint16_t>(p, s) : launch_intra_c<64, float>(p, s);
    return p.qkv_bf16 ? launch_intra_c<32, uint16_t>(p, s) : launch_intra_c<32, float>(p, s);
}

}  // namespace kda
