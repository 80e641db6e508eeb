// kda_recur.hip -- inter-chunk state recurrence and chunk output of the KDA forward.
//
// "Reading Notes: Implementation Notes for KDA in FLA", forward steps 4 and 5,
// with the state stored [K][V] (key rows) and its decay read as Diag(2^G_last):
//   V_new = U - W S
//   O     = Qg S + Aqk V_new            (S before this chunk's update)
//   S    <- Diag(d) S + KgT V_new,       d = 2^G_last
//
// One workgroup (4 waves) per (sequence, value head, 16-column slice of V).  The
// fp32 state slice S[:, v0:v0+16] stays in the waves' accumulator registers for
// the whole sequence; each chunk step passes S (as an MFMA operand) and V_new
// between waves through LDS.  Wave w owns output rows 16w..16w+15 of a chunk and
// the state row tiles t = w, w+4, ... (16 key rows each).
#include "kda_gate.h"

namespace kda {

template <typename T> struct Frag;
template <> struct Frag<uint16_t> {
    uint4 u;
    __device__ __forceinline__ void load(const uint16_t *p) { u = *reinterpret_cast<const uint4 *>(p); }
};
template <> struct Frag<float> {
    float f[8];
    __device__ __forceinline__ void load(const float *p) { load8(p, f); }
};
__device__ __forceinline__ f32x4 mma(f32x4 acc, const Frag<uint16_t> &a, const Frag<uint16_t> &b) {
    return mma32_bf16(acc, a.u, b.u);
}
__device__ __forceinline__ f32x4 mma(f32x4 acc, const Frag<float> &a, const Frag<float> &b) {
    return mma32<true>(acc, a.f, b.f);
}

template <int C, typename T, int NKK>
__global__ void __launch_bounds__(256) recur_kernel(Params p) {
    constexpr int NRB = C / 16;          // row blocks per chunk
    constexpr int NTW = NKK / 2;         // max state tiles per wave (K/16 tiles over 4 waves)
    extern __shared__ __align__(16) unsigned char lds[];
    const int K = p.K, V = p.V;
    const int nkk = K / 32, ntiles = K / 16;
    const int LDK = K + 8, LDC = C + 8;
    T *ST = reinterpret_cast<T *>(lds);                                   // [16][K+8]: S^T
    T *VT = reinterpret_cast<T *>(lds + sizeof(T) * 16 * LDK);           // [16][C+8]: V_new^T

    const int nvt = V / 16;
    const int vt = blockIdx.x % nvt;
    const int hv = (blockIdx.x / nvt) % p.HV;
    const int n = blockIdx.x / (nvt * p.HV);
    const int v0 = 16 * vt;
    const int w = threadIdx.x >> 6, l = lane_id(), lr = l & 15, cg = l >> 4;

    // state tiles of this wave
    f32x4 S[NTW];
    const size_t sbase = ((size_t)n * p.HV + hv) * K * V;
#pragma unroll
    for (int tt = 0; tt < NTW; ++tt) {
        const int t = w + 4 * tt;
        S[tt] = zero4();
        if (t < ntiles && p.h0) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) S[tt][jj] = p.h0[sbase + (size_t)(16 * t + 4 * cg + jj) * V + v0 + lr];
        }
    }

    const int c0 = p.chunk_off[n], c1 = p.chunk_off[n + 1];
    const int64_t sb = seq_begin(p, n);
    const int64_t se = p.cu_seqlens ? p.cu_seqlens[n + 1] : sb + p.T;
    const T *Wb = static_cast<const T *>(p.w_W);
    const T *Ub = static_cast<const T *>(p.w_U);
    const T *KgTb = static_cast<const T *>(p.w_KgT);
    const T *Qgb = static_cast<const T *>(p.w_Qg);
    const T *Aqkb = static_cast<const T *>(p.w_Aqk);
    T *o = static_cast<T *>(p.o);

    for (int gc = c0; gc < c1; ++gc) {
        const int64_t tok0 = sb + (int64_t)(gc - c0) * C;
        const int L = (int)((se - tok0) < C ? (se - tok0) : C);
        const size_t slot = (size_t)gc * p.HV + hv;

        // (1) S -> LDS as S^T (bf16 or fp32), the B operand of W S and Qg S
#pragma unroll
        for (int tt = 0; tt < NTW; ++tt) {
            const int t = w + 4 * tt;
            if (t < ntiles) store4(ST + lr * LDK + 16 * t + 4 * cg, S[tt][0], S[tt][1], S[tt][2], S[tt][3]);
        }
        __syncthreads();

        // (2) V_new = U - W S and the inter part of O, for this wave's rows
        f32x4 accO = zero4();
        if (w < NRB) {
            f32x4 accV = zero4();
            const T *Wr = Wb + (slot * C + 16 * w + lr) * K;
            const T *Qr = Qgb + (slot * C + 16 * w + lr) * K;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                if (kk < nkk) {
                    Frag<T> b, aw, aq;
                    b.load(ST + lr * LDK + 32 * kk + 8 * cg);
                    aw.load(Wr + 32 * kk + 8 * cg);
                    aq.load(Qr + 32 * kk + 8 * cg);
                    accV = mma(accV, aw, b);
                    accO = mma(accO, aq, b);
                }
            }
            float vn[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int m = 16 * w + 4 * cg + jj;
                vn[jj] = load1(Ub + (slot * C + m) * V + v0 + lr) - accV[jj];
            }
            store4(VT + lr * LDC + 16 * w + 4 * cg, vn[0], vn[1], vn[2], vn[3]);
        }
        __syncthreads();

        // (3) O += Aqk V_new -> o;  S <- Diag(d) S + KgT V_new
        if (w < NRB) {
            const T *Ar = Aqkb + (slot * C + 16 * w + lr) * C;
#pragma unroll
            for (int ms = 0; ms < C / 32; ++ms) {
                Frag<T> a, b;
                a.load(Ar + 32 * ms + 8 * cg);
                b.load(VT + lr * LDC + 32 * ms + 8 * cg);
                accO = mma(accO, a, b);
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int m = 16 * w + 4 * cg + jj;
                if (m < L) o[((tok0 + m) * p.HV + hv) * (int64_t)V + v0 + lr] = Store<T>::to(accO[jj]);
            }
        }
#pragma unroll
        for (int tt = 0; tt < NTW; ++tt) {
            const int t = w + 4 * tt;
            if (t < ntiles) {
                const float4 dd = *reinterpret_cast<const float4 *>(p.w_d + slot * K + 16 * t + 4 * cg);
                f32x4 acc = S[tt];
                acc[0] *= dd.x; acc[1] *= dd.y; acc[2] *= dd.z; acc[3] *= dd.w;
                const T *Kr = KgTb + (slot * K + 16 * t + lr) * C;
#pragma unroll
                for (int ms = 0; ms < C / 32; ++ms) {
                    Frag<T> a, b;
                    a.load(Kr + 32 * ms + 8 * cg);
                    b.load(VT + lr * LDC + 32 * ms + 8 * cg);
                    acc = mma(acc, a, b);
                }
                S[tt] = acc;
            }
        }
    }

    if (p.output_final_state) {
#pragma unroll
        for (int tt = 0; tt < NTW; ++tt) {
            const int t = w + 4 * tt;
            if (t < ntiles) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) p.ht[sbase + (size_t)(16 * t + 4 * cg + jj) * V + v0 + lr] = S[tt][jj];
            }
        }
    }
}

template <int C, typename T>
static hipError_t launch_recur_t(const Params &p, hipStream_t s) {
    const size_t lds = sizeof(T) * (16 * (p.K + 8) + 16 * (C + 8));
    const dim3 grid((unsigned)p.N * (unsigned)p.HV * (unsigned)(p.V / 16));
    if (p.K <= 128) hipLaunchKernelGGL((recur_kernel<C, T, 4>), grid, dim3(256), lds, s, p);
    else hipLaunchKernelGGL((recur_kernel<C, T, 8>), grid, dim3(256), lds, s, p);
    return hipGetLastError();
}

hipError_t launch_recurrence(const Params &p, hipStream_t s) {
    if (p.N == 0) return hipSuccess;
    if (p.C == 64) return p.qkv_bf16 ? launch_recur_t<64, uint16_t>(p, s) : launch_recur_t<64, float>(p, s);
    return p.qkv_bf16 ? launch_recur_t<32, uint16_t>(p, s) : launch_recur_t<32, float>(p, s);
}

}  // namespace kda
