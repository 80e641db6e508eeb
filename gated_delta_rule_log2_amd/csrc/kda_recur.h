// kda_recur.h -- inter-chunk state recurrence and chunk output of the KDA forward.
//
// "Reading Notes: Implementation Notes for KDA in FLA", forward steps 4 and 5,
// with the state stored [K][V] (key rows) and its decay read as Diag(2^G_last):
//   V_new = U - W S
//   O     = Qg S + Aqk V_new            (S before this chunk's update)
//   S    <- Diag(d) S + KgT V_new,       d = 2^G_last
//
// One workgroup (8 waves) per (sequence, value head, 32-column slice of V).  The
// fp32 state slice S[:, v0:v0+32] stays in the state waves' accumulator registers
// for the whole sequence; each chunk step passes S (as an MFMA operand) and V_new
// between waves through LDS.  The next chunk's operands are loaded into registers
// while the current chunk computes.
//
// Placement: workgroups are dealt to the 8 XCDs round-robin by index, so the
// index is arranged to put every V slice of one (sequence, head) on the same XCD,
// where they share that XCD's L2 copy of the head's W, Qg, KgT and Aqk.
#pragma once

#include "kda_gate.h"

namespace kda {

constexpr int kBV = 32;   // V columns per workgroup
constexpr int kXCD = 8;   // XCDs per MI355X
#ifndef KDA_RECUR_STAGES
#define KDA_RECUR_STAGES 2
#endif
constexpr int kStages = KDA_RECUR_STAGES;  // operand sets in flight per wave

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

// Per-chunk operands.  The workgroup has 8 waves: waves 0-3 carry the state path
// (W S, V_new, KgT V_new: the sequential critical path) and waves 4-7 the output
// path (Qg S, Aqk V_new, o).  A state wave and an output wave share each SIMD, so
// the output work fills the stalls of the state chain, and no operand is loaded
// twice.  Wave w (of either role) owns rows 16w..16w+15 of the chunk; state wave w
// also owns the state row tiles t = w, w+4, ... (16 key rows each).
template <int C, typename T, int NKK>
struct Geo {
    static constexpr int K = 32 * NKK;
    static constexpr int NTILES = K / 16;
    static constexpr int NRT = (NTILES + 3) / 4;
    static constexpr bool ALL_ROWS = (C == 64);            // every wave owns a 16-row block of the chunk
    static constexpr bool EVEN_TILES = (NTILES % 4 == 0);  // every state wave owns NRT row tiles
    static __device__ __forceinline__ bool is_row_wave(bool rw) { return ALL_ROWS || rw; }
    static __device__ __forceinline__ bool has_tile(int t) { return EVEN_TILES || t < NTILES; }
};

template <int C, typename T, int NKK>
struct StateOps {
    using G = Geo<C, T, NKK>;
    static constexpr int K = G::K, NRT = G::NRT;
    Frag<T> w[NKK];          // W rows 16w.. (row fragments)
    Quad<T> u[2];            // U^T: rows 16w+4cg.. for the two column halves
    Frag<T> kg[NRT][C / 32]; // KgT rows of the wave's state row tiles
    float4 d[NRT];           // 2^G_last for the wave's state rows
    __device__ __forceinline__ void load(const Params &p, size_t slot, int w_, int lr, int cg, int v0, bool rw) {
        if (G::is_row_wave(rw)) {
            const int l = lr + 16 * cg;
            const T *Wr = static_cast<const T *>(p.w_W) + slot * C * K + (size_t)(w_ * NKK * 64 + l) * 8;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) w[kk].load(Wr + kk * 512);
            const T *Ut = static_cast<const T *>(p.w_U) + slot * (size_t)p.V * C;
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                u[nt].load(Ut + (size_t)((((v0 >> 4) + nt) * (C / 16) + w_) * 64 + l) * 4);
        }
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const int t = w_ + 4 * rt;
            if (G::has_tile(t)) {
                const T *Kr = static_cast<const T *>(p.w_KgT) + slot * K * C +
                              (size_t)(t * (C / 32) * 64 + lr + 16 * cg) * 8;
#pragma unroll
                for (int ms = 0; ms < C / 32; ++ms) kg[rt][ms].load(Kr + ms * 512);
                d[rt] = *reinterpret_cast<const float4 *>(p.w_d + slot * K + 16 * t + 4 * cg);
            }
        }
    }
};

template <int C, typename T, int NKK>
struct OutOps {
    using G = Geo<C, T, NKK>;
    static constexpr int K = G::K;
    Frag<T> q[NKK];          // Qg rows 16w..
    Frag<T> a[C / 32];       // Aqk rows 16w..
    __device__ __forceinline__ void load(const Params &p, size_t slot, int w_, int lr, int cg, int, bool rw) {
        if (G::is_row_wave(rw)) {
            const int l = lr + 16 * cg;
            const T *Qr = static_cast<const T *>(p.w_Qg) + slot * C * K + (size_t)(w_ * NKK * 64 + l) * 8;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) q[kk].load(Qr + kk * 512);
            const T *Ar = static_cast<const T *>(p.w_Aqk) + slot * C * C + (size_t)(w_ * (C / 32) * 64 + l) * 8;
#pragma unroll
            for (int ms = 0; ms < C / 32; ++ms) a[ms].load(Ar + ms * 512);
        }
    }
};

// Everything a chunk step needs besides its operands.
template <int C, typename T, int NKK>
struct StepCtx {
    T *ST, *VT, *OS;
    int w, lr, cg, hv, v0;
    bool row_wave;
};

// Writes the chunk output tile held in LDS (rows [0, L), kBV columns) to o with
// 16-byte stores, by the 256 output-role threads (ot = their index).
template <int C, typename T>
__device__ __forceinline__ void store_out_tile(const Params &p, const T *OS, int ot, int hv, int v0, int64_t tok0,
                                               int L) {
    constexpr int LDO = kBV + 8;
    constexpr int EPT = 16 / (int)sizeof(T);  // elements per 16-byte store
    constexpr int TPR = kBV / EPT;            // threads per row
#pragma unroll
    for (int e = ot; e < C * TPR; e += 256) {
        const int m = e / TPR, c0 = (e % TPR) * EPT;
        if (m < L) {
            T *dst = static_cast<T *>(p.o) + ((tok0 + m) * p.HV + hv) * (int64_t)p.V + v0 + c0;
            *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(OS + m * LDO + c0);
        }
    }
}

// State path of one chunk step (S kept in registers across steps):
//   S -> LDS (S^T); barrier; V_new = U - W S -> LDS (V_new^T); barrier;
//   S <- Diag(d) S + KgT V_new.
template <int C, typename T, int NKK>
__device__ __forceinline__ void state_step(const StateOps<C, T, NKK> &op, f32x4 (&S)[Geo<C, T, NKK>::NRT][2],
                                           const StepCtx<C, T, NKK> &x) {
    using G = Geo<C, T, NKK>;
    constexpr int NRT = G::NRT, LDK = 32 * NKK + 8, LDC = C + 8;
    const bool row_wave = G::is_row_wave(x.row_wave);
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        const int t = x.w + 4 * rt;
        if (G::has_tile(t)) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                store4(x.ST + (16 * nt + x.lr) * LDK + 16 * t + 4 * x.cg, S[rt][nt][0], S[rt][nt][1], S[rt][nt][2],
                       S[rt][nt][3]);
        }
    }
    __syncthreads();
    if (row_wave) {
        f32x4 accV[2] = {zero4(), zero4()};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                Frag<T> b;
                b.load(x.ST + (16 * nt + x.lr) * LDK + 32 * kk + 8 * x.cg);
                accV[nt] = mma(accV[nt], op.w[kk], b);
            }
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
            store4(x.VT + (16 * nt + x.lr) * LDC + 16 * x.w + 4 * x.cg, op.u[nt].get(0) - accV[nt][0],
                   op.u[nt].get(1) - accV[nt][1], op.u[nt].get(2) - accV[nt][2], op.u[nt].get(3) - accV[nt][3]);
    }
    __syncthreads();
    Frag<T> bv[2][C / 32];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int ms = 0; ms < C / 32; ++ms) bv[nt][ms].load(x.VT + (16 * nt + x.lr) * LDC + 32 * ms + 8 * x.cg);
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        const int t = x.w + 4 * rt;
        if (G::has_tile(t)) {
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

// Output path of one chunk step: barrier; the previous chunk's output tile (LDS)
// -> o (STORE_PREV); O = Qg S (S^T from LDS); barrier; O += Aqk V_new -> LDS tile.
template <int C, typename T, int NKK, bool STORE_PREV>
__device__ __forceinline__ void out_step(const Params &p, const OutOps<C, T, NKK> &op, const StepCtx<C, T, NKK> &x,
                                         int ot, int64_t prev_tok0) {
    using G = Geo<C, T, NKK>;
    constexpr int LDK = 32 * NKK + 8, LDC = C + 8, LDO = kBV + 8;
    const bool row_wave = G::is_row_wave(x.row_wave);
    __syncthreads();
    if constexpr (STORE_PREV) store_out_tile<C, T>(p, x.OS, ot, x.hv, x.v0, prev_tok0, C);
    f32x4 accO[2] = {zero4(), zero4()};
    if (row_wave) {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                Frag<T> b;
                b.load(x.ST + (16 * nt + x.lr) * LDK + 32 * kk + 8 * x.cg);
                accO[nt] = mma(accO[nt], op.q[kk], b);
            }
        }
    }
    __syncthreads();
    if (row_wave) {
        // Aqk is zero right of the diagonal block: rows 16w.. only need columns < 16(w+1)
        const int nms = (16 * x.w + 16 + 31) / 32;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
            for (int ms = 0; ms < C / 32; ++ms)
                if (ms < nms) {
                    Frag<T> b;
                    b.load(x.VT + (16 * nt + x.lr) * LDC + 32 * ms + 8 * x.cg);
                    accO[nt] = mma(accO[nt], op.a[ms], b);
                }
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                x.OS[(16 * x.w + 4 * x.cg + jj) * LDO + 16 * nt + x.lr] = Store<T>::to(accO[nt][jj]);
    }
}

// Runs one role's chunk loop with an NST-deep ring of operand sets: while chunk g
// computes, the operands of chunks g+1 .. g+NST-1 are in flight.  The loop is
// unrolled NST times so every ring slot is a static register set, and every
// in-loop load is unconditional (prefetches past the end re-read the final chunk),
// so the wait counts stay static.  The first chunk runs before the loop
// (step_first), the ring covers whole unrolled iterations, the rest runs after.
template <int NST, typename Ops, typename StepFirst, typename Step>
__device__ __forceinline__ void chunk_loop(const Params &p, int c0, int c1, int hv, int w, int lr, int cg, int v0,
                                           bool rw, StepFirst step_first, Step step) {
    auto slot_of = [&](int g) { return (size_t)(g < c1 ? g : c1 - 1) * p.HV + hv; };
    if (c0 >= c1) return;
    {
        Ops op;
        op.load(p, slot_of(c0), w, lr, cg, v0, rw);
        step_first(op, c0);
    }
    Ops ops[NST];
    int g = c0 + 1;
    if (c1 - g >= NST) {
#pragma unroll
        for (int k = 0; k < NST - 1; ++k) ops[k].load(p, slot_of(g + k), w, lr, cg, v0, rw);
        for (; g + NST <= c1; g += NST) {
#pragma unroll
            for (int k = 0; k < NST; ++k) {
                ops[(k + NST - 1) % NST].load(p, slot_of(g + k + NST - 1), w, lr, cg, v0, rw);
                step(ops[k], g + k);
            }
        }
    }
    for (; g < c1; ++g) {
        Ops opx;
        opx.load(p, slot_of(g), w, lr, cg, v0, rw);
        step(opx, g);
    }
}

// HS: also write the state each chunk starts from (p.hs); a separate instantiation so
// the stores add no register pressure to the plain forward.
template <int C, typename T, int NKK, bool HS>
__global__ void __launch_bounds__(512) recur_kernel(Params p) {
    using G = Geo<C, T, NKK>;
    constexpr int NRT = G::NRT, K = G::K;
    extern __shared__ __align__(16) unsigned char lds[];
    const int V = p.V;
    T *ST = reinterpret_cast<T *>(lds);  // [32][K+8]: S^T
    T *VT = ST + kBV * (K + 8);           // [32][C+8]: V_new^T
    T *OS = VT + kBV * (C + 8);           // [C][32+8]: output tile

    // XCD-aware decode: workgroup b runs on XCD b % 8; unit u = (n, hv) lives on XCD u % 8
    const int nvt = V / kBV;
    const int xcd = blockIdx.x % kXCD, pos = blockIdx.x / kXCD;
    const int u = (pos / nvt) * kXCD + xcd;
    const int vt = pos % nvt;
    if (u >= p.N * p.HV) return;
    const int n = p.cu_seqlens ? p.seq_order[u / p.HV] : u / p.HV, hv = u % p.HV;  // longest first
    const int v0 = kBV * vt;
    const int wid = threadIdx.x >> 6, l = lane_id(), lr = l & 15, cg = l >> 4;
    const bool state_role = wid < 4;
    const int w = wid & 3;
    const bool row_wave = w < C / 16;
    const StepCtx<C, T, NKK> x{ST, VT, OS, w, lr, cg, hv, v0, row_wave};

    const int c0 = seq_chunk_begin(p, n), c1 = seq_chunk_begin(p, n + 1);
    const int64_t sb = seq_begin(p, n);
    const int64_t se = p.cu_seqlens ? p.cu_seqlens[n + 1] : sb + p.T;
    auto tok_of = [&](int g) { return sb + (int64_t)(g - c0) * C; };

    if (state_role) {
        f32x4 S[NRT][2];
        const size_t sbase = ((size_t)n * p.HV + hv) * K * V;
        // offset of state element (key row, value column) in a [K][V] or [V][K] state
        auto sidx = [&](int row, int c) { return p.state_vk ? (size_t)c * K + row : (size_t)row * V + c; };
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const int t = w + 4 * rt;
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                S[rt][nt] = zero4();
                if (G::has_tile(t) && p.h0) {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        S[rt][nt][jj] = p.h0[sbase + sidx(16 * t + 4 * cg + jj, v0 + 16 * nt + lr)];
                }
            }
        }
        // intermediate-state output: a per-chunk uniform base plus this lane's offset (rows
        // 4cg.., column v0 + lr), fixed for the kernel
        const uint32_t hs_lane = p.state_vk ? (uint32_t)(v0 + lr) * K + 4 * cg : (uint32_t)(4 * cg) * V + v0 + lr;
        auto step = [&](const StateOps<C, T, NKK> &op, int g) {
            if constexpr (HS) {  // the state chunk g starts from
                float *hb = p.hs + ((size_t)g * p.HV + hv) * K * V;
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt) {
                    const int t = w + 4 * rt;
                    if (G::has_tile(t)) {
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt) {
                            if (p.state_vk) {
                                *reinterpret_cast<float4 *>(hb + (size_t)(16 * nt) * K + 16 * t + hs_lane) =
                                    make_float4(S[rt][nt][0], S[rt][nt][1], S[rt][nt][2], S[rt][nt][3]);
                            } else {
#pragma unroll
                                for (int jj = 0; jj < 4; ++jj)
                                    (hb + (size_t)(16 * t + jj) * V + 16 * nt)[hs_lane] = S[rt][nt][jj];
                            }
                        }
                    }
                }
            }
            state_step<C, T, NKK>(op, S, x);
        };
        chunk_loop<kStages, StateOps<C, T, NKK>>(p, c0, c1, hv, w, lr, cg, v0, row_wave, step, step);
        if (p.output_final_state) {
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                const int t = w + 4 * rt;
                if (G::has_tile(t)) {
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            p.ht[sbase + sidx(16 * t + 4 * cg + jj, v0 + 16 * nt + lr)] = S[rt][nt][jj];
                }
            }
        }
    } else {
        const int ot = threadIdx.x - 256;
        auto step_first = [&](const OutOps<C, T, NKK> &op, int) { out_step<C, T, NKK, false>(p, op, x, ot, 0); };
        auto step = [&](const OutOps<C, T, NKK> &op, int g) { out_step<C, T, NKK, true>(p, op, x, ot, tok_of(g - 1)); };
        chunk_loop<kStages, OutOps<C, T, NKK>>(p, c0, c1, hv, w, lr, cg, v0, row_wave, step_first, step);
    }
    // the last chunk's output tile
    __syncthreads();
    if (!state_role && c0 < c1) {
        const int64_t tl = tok_of(c1 - 1);
        store_out_tile<C, T>(p, OS, (int)threadIdx.x - 256, hv, v0, tl, (int)((se - tl) < C ? (se - tl) : C));
    }
}

template <int C, typename T>
hipError_t launch_recur_ct(const Params &p, hipStream_t s) {
    const size_t lds = sizeof(T) * (kBV * (p.K + 8) + kBV * (C + 8) + C * (kBV + 8));
    const int units = p.N * p.HV;
    const int per_xcd = (units + kXCD - 1) / kXCD;
    const dim3 grid((unsigned)(per_xcd * kXCD * (p.V / kBV)));
    const bool hs = p.hs != nullptr;
#define KDA_RECUR_CASE(n)                                                                   \
    case n:                                                                                 \
        if (hs) hipLaunchKernelGGL((recur_kernel<C, T, n, true>), grid, dim3(512), lds, s, p);  \
        else hipLaunchKernelGGL((recur_kernel<C, T, n, false>), grid, dim3(512), lds, s, p);    \
        break;
    switch (p.K / 32) {
        KDA_RECUR_CASE(1)
        KDA_RECUR_CASE(2)
        KDA_RECUR_CASE(3)
        KDA_RECUR_CASE(4)
        KDA_RECUR_CASE(5)
        KDA_RECUR_CASE(6)
        KDA_RECUR_CASE(7)
        KDA_RECUR_CASE(8)
    default: return hipErrorInvalidValue;
    }
#undef KDA_RECUR_CASE
    return hipGetLastError();
}

}  // namespace kda
