// kda_recur.h -- inter-chunk state recurrence and chunk output of the KDA forward.
//
// "Reading Notes: Implementation Notes for KDA in FLA", forward steps 4 and 5,
// with the state stored [K][V] (key rows) and its decay read as Diag(2^G_last):
//   V_new = U - W S
//   O     = Qg S + Aqk V_new            (S before this chunk's update)
//   S    <- Diag(d) S + KgT V_new,       d = 2^G_last
//
// One workgroup (4 waves) per (sequence, value head, 32-column slice of V).  The
// fp32 state slice S[:, v0:v0+32] stays in the waves' accumulator registers for
// the whole sequence; each chunk step passes S (as an MFMA operand) and V_new
// between waves through LDS.  Wave w owns output rows 16w..16w+15 of a chunk and
// the state row tiles t = w, w+4, ... (16 key rows each), both for the two
// 16-column halves of the slice.  The next chunk's operands are loaded into
// registers while the current chunk computes.
//
// Placement: workgroups are dealt to the 8 XCDs round-robin by index, so the
// index is arranged to put every V slice of one (sequence, head) on the same XCD,
// where they share that XCD's L2 copy of the head's W, Qg, KgT and Aqk.
#pragma once

#include "kda_gate.h"

namespace kda {

constexpr int kBV = 32;   // V columns per workgroup
constexpr int kXCD = 8;   // XCDs per MI355X

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

// 4 contiguous elements (a column of an accumulator tile, stored transposed)
template <typename T> struct Quad;
template <> struct Quad<uint16_t> {
    uint2 u;
    __device__ __forceinline__ void load(const uint16_t *p) { u = *reinterpret_cast<const uint2 *>(p); }
    __device__ __forceinline__ float get(int j) const {
        const uint32_t w = (j < 2) ? u.x : u.y;
        return (j & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
    }
};
template <> struct Quad<float> {
    float4 f;
    __device__ __forceinline__ void load(const float *p) { f = *reinterpret_cast<const float4 *>(p); }
    __device__ __forceinline__ float get(int j) const { return j == 0 ? f.x : j == 1 ? f.y : j == 2 ? f.z : f.w; }
};

// Operands of one chunk step held by one wave (K = 32 * NKK exactly).
template <int C, typename T, int NKK>
struct StepOps {
    static constexpr int K = 32 * NKK;
    static constexpr int NTILES = K / 16;
    static constexpr int NRT = (NTILES + 3) / 4;  // state row tiles per wave (K/16 tiles over 4 waves)
    static constexpr bool ALL_ROWS = (C == 64);          // every wave owns a 16-row block of the chunk
    static constexpr bool EVEN_TILES = (NTILES % 4 == 0);  // every wave owns NRT state row tiles
    static __device__ __forceinline__ bool is_row_wave(bool rw) { return ALL_ROWS || rw; }
    static __device__ __forceinline__ bool has_tile(int t) { return EVEN_TILES || t < NTILES; }
    Frag<T> w[NKK], q[NKK];              // W and Qg rows 16w.. (row fragments)
    Frag<T> a[C / 32];                   // Aqk rows 16w..
    Frag<T> kg[NRT][C / 32];             // KgT rows of the wave's state row tiles
    Quad<T> u[2];                        // U^T: rows 16w+4cg.., column halves
    float4 d[NRT];                       // 2^G_last for the wave's state rows

    __device__ __forceinline__ void load(const Params &p, size_t slot, int w_, int lr, int cg, int v0,
                                         bool row_wave) {
        if (is_row_wave(row_wave)) {
            const T *Wr = static_cast<const T *>(p.w_W) + (slot * C + 16 * w_ + lr) * K + 8 * cg;
            const T *Qr = static_cast<const T *>(p.w_Qg) + (slot * C + 16 * w_ + lr) * K + 8 * cg;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                w[kk].load(Wr + 32 * kk);
                q[kk].load(Qr + 32 * kk);
            }
            const T *Ar = static_cast<const T *>(p.w_Aqk) + (slot * C + 16 * w_ + lr) * C + 8 * cg;
#pragma unroll
            for (int ms = 0; ms < C / 32; ++ms) a[ms].load(Ar + 32 * ms);
            const T *Ut = static_cast<const T *>(p.w_U) + slot * (size_t)p.V * C;
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) u[nt].load(Ut + (size_t)(v0 + 16 * nt + lr) * C + 16 * w_ + 4 * cg);
        }
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const int t = w_ + 4 * rt;
            if (has_tile(t)) {
                const T *Kr = static_cast<const T *>(p.w_KgT) + (slot * K + 16 * t + lr) * C + 8 * cg;
#pragma unroll
                for (int ms = 0; ms < C / 32; ++ms) kg[rt][ms].load(Kr + 32 * ms);
                d[rt] = *reinterpret_cast<const float4 *>(p.w_d + slot * K + 16 * t + 4 * cg);
            }
        }
    }
};

// One chunk step.  FULL: the chunk has all C rows, so the o stores need no row guard
// (keeping every memory instruction unconditional lets the prefetch wait counts stay
// exact across the loop).
template <int C, typename T, int NKK, bool FULL>
__device__ __forceinline__ void chunk_step(const Params &p, const StepOps<C, T, NKK> &op,
                                           f32x4 (&S)[StepOps<C, T, NKK>::NRT][2], T *ST, T *VT, int w, int lr,
                                           int cg, bool row_wave_, int64_t tok0, int L, int hv, int v0) {
    using Ops = StepOps<C, T, NKK>;
    constexpr int NRT = Ops::NRT;
    constexpr int LDK = 32 * NKK + 8, LDC = C + 8;
    const bool row_wave = Ops::is_row_wave(row_wave_);
    // (1) S -> LDS as S^T (the B operand of W S and Qg S)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        const int t = w + 4 * rt;
        if (Ops::has_tile(t)) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                store4(ST + (16 * nt + lr) * LDK + 16 * t + 4 * cg, S[rt][nt][0], S[rt][nt][1], S[rt][nt][2],
                       S[rt][nt][3]);
        }
    }
    __syncthreads();
    // (2) V_new = U - W S and the inter-chunk part of O
    f32x4 accO[2] = {zero4(), zero4()};
    if (row_wave) {
        f32x4 accV[2] = {zero4(), zero4()};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                Frag<T> b;
                b.load(ST + (16 * nt + lr) * LDK + 32 * kk + 8 * cg);
                accV[nt] = mma(accV[nt], op.w[kk], b);
                accO[nt] = mma(accO[nt], op.q[kk], b);
            }
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
            store4(VT + (16 * nt + lr) * LDC + 16 * w + 4 * cg, op.u[nt].get(0) - accV[nt][0],
                   op.u[nt].get(1) - accV[nt][1], op.u[nt].get(2) - accV[nt][2], op.u[nt].get(3) - accV[nt][3]);
    }
    __syncthreads();
    // (3) O += Aqk V_new;  S <- Diag(d) S + KgT V_new
    Frag<T> bv[2][C / 32];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int ms = 0; ms < C / 32; ++ms) bv[nt][ms].load(VT + (16 * nt + lr) * LDC + 32 * ms + 8 * cg);
    if (row_wave) {
        // Aqk is zero right of the diagonal block: rows 16w.. only need columns < 16(w+1)
        const int nms = (16 * w + 16 + 31) / 32;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
            for (int ms = 0; ms < C / 32; ++ms)
                if (ms < nms) accO[nt] = mma(accO[nt], op.a[ms], bv[nt][ms]);
        }
        T *o = static_cast<T *>(p.o);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int m = 16 * w + 4 * cg + jj;
            if (FULL || m < L) {
                T *orow = o + ((tok0 + m) * p.HV + hv) * (int64_t)p.V + v0 + lr;
                orow[0] = Store<T>::to(accO[0][jj]);
                orow[16] = Store<T>::to(accO[1][jj]);
            }
        }
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        const int t = w + 4 * rt;
        if (Ops::has_tile(t)) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                f32x4 acc = S[rt][nt];
                acc[0] *= op.d[rt].x;
                acc[1] *= op.d[rt].y;
                acc[2] *= op.d[rt].z;
                acc[3] *= op.d[rt].w;
#pragma unroll
                for (int ms = 0; ms < C / 32; ++ms) acc = mma(acc, op.kg[rt][ms], bv[nt][ms]);
                S[rt][nt] = acc;
            }
        }
    }
}

template <int C, typename T, int NKK>
__global__ void __launch_bounds__(256) recur_kernel(Params p) {
    using Ops = StepOps<C, T, NKK>;
    constexpr int NRT = Ops::NRT, K = Ops::K;
    extern __shared__ __align__(16) unsigned char lds[];
    const int V = p.V;
    T *ST = reinterpret_cast<T *>(lds);                                    // [32][K+8]: S^T
    T *VT = reinterpret_cast<T *>(lds + sizeof(T) * kBV * (K + 8));       // [32][C+8]: V_new^T

    // XCD-aware decode: workgroup b runs on XCD b % 8; unit u = (n, hv) lives on XCD u % 8
    const int nvt = V / kBV;
    const int xcd = blockIdx.x % kXCD, pos = blockIdx.x / kXCD;
    const int u = (pos / nvt) * kXCD + xcd;
    const int vt = pos % nvt;
    if (u >= p.N * p.HV) return;
    const int n = u / p.HV, hv = u % p.HV;
    const int v0 = kBV * vt;
    const int w = threadIdx.x >> 6, l = lane_id(), lr = l & 15, cg = l >> 4;
    const bool row_wave = w < C / 16;

    f32x4 S[NRT][2];
    const size_t sbase = ((size_t)n * p.HV + hv) * K * V;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        const int t = w + 4 * rt;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            S[rt][nt] = zero4();
            if (Ops::has_tile(t) && p.h0) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    S[rt][nt][jj] = p.h0[sbase + (size_t)(16 * t + 4 * cg + jj) * V + v0 + 16 * nt + lr];
            }
        }
    }

    const int c0 = p.chunk_off[n], c1 = p.chunk_off[n + 1];
    const int64_t sb = seq_begin(p, n);
    const int64_t se = p.cu_seqlens ? p.cu_seqlens[n + 1] : sb + p.T;
    auto slot_of = [&](int g) { return (size_t)g * p.HV + hv; };
    auto tok_of = [&](int g) { return sb + (int64_t)(g - c0) * C; };
    // chunks [c0, cf) are full; a partial last chunk (if any) is stepped after the loop
    const int cf = c0 + (int)((se - sb) / C);
    // Two operand sets in flight: every prefetch inside the loop is unconditional
    // (the last one re-reads the final chunk) so the wait counts stay static.
    Ops op0, op1;
    int g = c0;
    if (g < c1) op0.load(p, slot_of(g), w, lr, cg, v0, row_wave);
    for (; g + 1 < cf; g += 2) {
        op1.load(p, slot_of(g + 1), w, lr, cg, v0, row_wave);
        chunk_step<C, T, NKK, true>(p, op0, S, ST, VT, w, lr, cg, row_wave, tok_of(g), C, hv, v0);
        op0.load(p, slot_of(g + 2 < c1 ? g + 2 : c1 - 1), w, lr, cg, v0, row_wave);
        chunk_step<C, T, NKK, true>(p, op1, S, ST, VT, w, lr, cg, row_wave, tok_of(g + 1), C, hv, v0);
    }
    // at most two chunks remain (one full, and/or the partial tail)
    for (; g < c1; ++g) {
        const int64_t tok0 = tok_of(g);
        const int L = (int)((se - tok0) < C ? (se - tok0) : C);
        Ops opx;
        opx.load(p, slot_of(g), w, lr, cg, v0, row_wave);
        chunk_step<C, T, NKK, false>(p, opx, S, ST, VT, w, lr, cg, row_wave, tok0, L, hv, v0);
    }

    if (p.output_final_state) {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const int t = w + 4 * rt;
            if (Ops::has_tile(t)) {
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        p.ht[sbase + (size_t)(16 * t + 4 * cg + jj) * V + v0 + 16 * nt + lr] = S[rt][nt][jj];
            }
        }
    }
}

// Exact-K dispatch (K = 32 * NKK) for one (chunk size, storage type).
template <int C, typename T>
hipError_t launch_recur_ct(const Params &p, hipStream_t s) {
    const size_t lds = sizeof(T) * (kBV * (p.K + 8) + kBV * (C + 8));
    const int units = p.N * p.HV;
    const int per_xcd = (units + kXCD - 1) / kXCD;
    const dim3 grid((unsigned)(per_xcd * kXCD * (p.V / kBV)));
    switch (p.K / 32) {
    case 1: hipLaunchKernelGGL((recur_kernel<C, T, 1>), grid, dim3(256), lds, s, p); break;
    case 2: hipLaunchKernelGGL((recur_kernel<C, T, 2>), grid, dim3(256), lds, s, p); break;
    case 3: hipLaunchKernelGGL((recur_kernel<C, T, 3>), grid, dim3(256), lds, s, p); break;
    case 4: hipLaunchKernelGGL((recur_kernel<C, T, 4>), grid, dim3(256), lds, s, p); break;
    case 5: hipLaunchKernelGGL((recur_kernel<C, T, 5>), grid, dim3(256), lds, s, p); break;
    case 6: hipLaunchKernelGGL((recur_kernel<C, T, 6>), grid, dim3(256), lds, s, p); break;
    case 7: hipLaunchKernelGGL((recur_kernel<C, T, 7>), grid, dim3(256), lds, s, p); break;
    case 8: hipLaunchKernelGGL((recur_kernel<C, T, 8>), grid, dim3(256), lds, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kda
