// kda_recur_reg.h -- inter-chunk state recurrence and chunk output of the KDA
// forward for bf16 intermediates and key width <= 128, with the state chain kept
// in registers and no cross-wave exchange on it.
//
// "Reading Notes: Implementation Notes for KDA in FLA", forward steps 4 and 5, with
// the state stored [K][V] and its decay read as Diag(2^G_last):
//   V_new = U - W S,   O = Qg S + Aqk V_new (S before the update),
//   S <- Diag(d) S + KgT V_new,   d = 2^G_last
//
// One workgroup of 4 + C/16 waves per (sequence, value head, 32-column slice of V):
//   waves 0, 1  state waves: wave j owns columns 16j..16j+15 of the slice and all K
//               rows of S (fp32 accumulators).  W, KgT, Qg and Aqk are stored as
//               permuted row fragments (see pfrag_off), so S and V_new in accumulator
//               layout are, converted to bf16 in place, the contraction operands of
//               the next products: the whole chain W S -> V_new -> KgT V_new -> S runs
//               inside one wave.  Each step reads all of its ring operands first, so
//               the LDS latency is paid once per step rather than once per product.
//   C/16 output waves, one step behind: output wave o forms O = Qg S + Aqk V_new for
//               chunk rows 16o..16o+15 and both column halves, from the S and V_new
//               the state waves hand over through LDS, with its rows of Qg and Aqk
//               prefetched a step ahead into its own registers; O is staged in LDS
//               and written as 16-byte row segments.
//   2 loaders   stream each step's W, KgT, U slice and d into a 3-slot LDS ring with
//               direct global->LDS loads, two steps ahead of the state waves.
// Waves are dealt to the 4 SIMDs round-robin by index; the roles are numbered so the
// two state waves share their SIMDs only with the loaders (their matrix-core chain is
// the critical path) and the output waves take the other two SIMDs.
// One barrier per step orders the ring, the hand-over buffers and the waves.
//
// Placement: workgroups are dealt to the 8 XCDs round-robin by index; the index is
// arranged so every V slice of one (sequence, head) runs on the same XCD and shares
// that XCD's L2 copy of the head's operands.
#pragma once

#include "kda_intra_bf16.h"
#include "kda_recur.h"

namespace kda {

template <int C, int K>
struct RegRecur {
    static constexpr int NKK = K / 32, NMT = C / 16, NMS = C / 32, NT = K / 16;
    static constexpr int NS = 3;            // ring slots
    static constexpr int NMO = 1;           // row tiles per output wave
    static constexpr int NWAVES = 4 + NMT;  // 2 state, NMT output, 2 loader waves
    // one ring slot (bytes): W [NMT][NKK] and KgT [NT][NMS] fragment units of 1 KB, U for
    // the slice's two 16-column tiles ([2][NMT] quad units of 512 B), d [K] fp32
    static constexpr int NLW = C * K * 2 / 1024, NLU = C * 32 * 2 / 1024;
    static constexpr size_t kW = 0, kKgT = kW + (size_t)NLW * 1024, kU = kKgT + (size_t)NLW * 1024;
    static constexpr size_t kD = kU + (size_t)NLU * 1024, kSlot = kD + (size_t)K * 4;
    // hand-over buffers [2][2 state waves]: S as [NKK] operand units, V_new as [NMS] units
    static constexpr size_t kExWave = (size_t)(NKK + NMS) * 1024;
    static constexpr size_t kEx = NS * kSlot, kOs = kEx + 4 * kExWave;
    static constexpr int LDO = kBV + 8;  // output tile row stride (bf16)
    static constexpr size_t kBytes = kOs + (size_t)C * LDO * 2;
    // 1 KB ring units per step, dealt to the two loader waves alternately; loader 1 also
    // loads d (16 bytes on each of the first K/4 lanes)
    static constexpr int NUNITS = 2 * NLW + NLU;
    static constexpr int nload(int i) { return (NUNITS - i + 1) / 2 + (i == 1 ? 1 : 0); }
    static_assert(nload(0) <= 31 && nload(1) <= 31, "loader wait count");
    static_assert(K / 4 <= 64, "d in one load");
};

// s_waitcnt immediate that waits until at most n vector-memory operations of this wave
// are outstanding (expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

__device__ __forceinline__ void lds_dma16(const void *g, void *l) {
    __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}

// Loader wave I: its share of step k's ring loads (slot k % NS).
template <int C, int K, int I>
__device__ __forceinline__ void ring_issue(const Params &p, unsigned char *ring, size_t sl, int k, int v0, int l) {
    using R = RegRecur<C, K>;
    unsigned char *dst = ring + (size_t)(k % R::NS) * R::kSlot;
    const unsigned char *gW = reinterpret_cast<const unsigned char *>(p.w_W) + sl * C * K * 2;
    const unsigned char *gK = reinterpret_cast<const unsigned char *>(p.w_KgT) + sl * K * C * 2;
    const unsigned char *gU =
        reinterpret_cast<const unsigned char *>(p.w_U) + (sl * (size_t)p.V * C + quad_off(0, v0, C)) * 2;
    const unsigned char *gD = reinterpret_cast<const unsigned char *>(p.w_d + sl * K);
#pragma unroll
    for (int u = I; u < R::NUNITS; u += 2) {
        const unsigned char *src;
        size_t off;
        if (u < R::NLW) src = gW + u * 1024, off = R::kW + u * 1024;
        else if (u < 2 * R::NLW) src = gK + (u - R::NLW) * 1024, off = R::kKgT + (u - R::NLW) * 1024;
        else src = gU + (u - 2 * R::NLW) * 1024, off = R::kU + (u - 2 * R::NLW) * 1024;
        lds_dma16(src + l * 16, dst + off);
    }
    if constexpr (I == 1) {
        if (l < K / 4) lds_dma16(gD + l * 16, dst + R::kD);
    }
}

template <int C, int NKK>
__global__ void __launch_bounds__(64 * (4 + C / 16)) __attribute__((amdgpu_waves_per_eu(2, 2)))
recur_reg_kernel(Params p) {
    constexpr int K = 32 * NKK;
    using R = RegRecur<C, K>;
    constexpr int NMT = R::NMT, NMS = R::NMS, NT = R::NT, NS = R::NS, NMO = R::NMO;
    extern __shared__ __align__(16) unsigned char lds[];
    const int V = p.V;

    // XCD-aware decode: workgroup b runs on XCD b % 8; unit u = (n, hv) lives on XCD u % 8
    const int nvt = V / kBV;
    const int xcd = blockIdx.x % kXCD, pos = blockIdx.x / kXCD;
    const int u = (pos / nvt) * kXCD + xcd;
    if (u >= p.N * p.HV) return;
    const int n = u / p.HV, hv = u % p.HV;
    const int v0 = kBV * (pos % nvt);
    const int wid = threadIdx.x >> 6, l = lane_id(), lr = l & 15, cg = l >> 4;
    // roles: waves 0, 1 state; 4, 5 loaders; 2, 3 and (C = 64) 6, 7 output
    const bool is_state = wid < 2, is_loader = wid == 4 || wid == 5;
    const int out_idx = wid < 4 ? wid - 2 : wid - 4;

    const int c0 = seq_chunk_begin(p, n), c1 = seq_chunk_begin(p, n + 1);
    const int nsteps = c1 - c0;
    const int64_t sb = seq_begin(p, n);
    const int64_t se = p.cu_seqlens ? p.cu_seqlens[n + 1] : sb + p.T;
    auto slot_of = [&](int k) { return (size_t)(c0 + k) * p.HV + hv; };
    unsigned char *ring = lds;
    auto ex_s = [&](int e, int j) { return reinterpret_cast<uint4 *>(lds + R::kEx + (size_t)(2 * e + j) * R::kExWave); };
    auto ex_v = [&](int e, int j) { return ex_s(e, j) + NKK * 64; };
    uint16_t *OS = reinterpret_cast<uint16_t *>(lds + R::kOs);

    if (is_state) {
        // ------------------------------------------------------------ state wave j
        const int j = wid;
        const int col = v0 + 16 * j + lr;
        const size_t sbase = ((size_t)n * p.HV + hv) * K * V;
        f32x4 S[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            S[t] = zero4();
            if (p.h0) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) S[t][jj] = p.h0[sbase + (size_t)(16 * t + 4 * cg + jj) * V + col];
            }
        }
        for (int k = 0; k <= nsteps; ++k) {
            __syncthreads();
            if (k == nsteps) break;
            const unsigned char *sl = ring + (size_t)(k % NS) * R::kSlot;
            const uint4 *Wr = reinterpret_cast<const uint4 *>(sl + R::kW);
            const uint4 *Kr = reinterpret_cast<const uint4 *>(sl + R::kKgT);
            const uint2 *Ur = reinterpret_cast<const uint2 *>(sl + R::kU);
            const float4 *Dr = reinterpret_cast<const float4 *>(sl + R::kD);
            // every ring operand of the step first
            uint4 wf[NMT][NKK], kf[NT][NMS];
            uint2 uq[NMT];
            float4 dd[NT];
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) wf[mt][kk] = Wr[(mt * NKK + kk) * 64 + l];
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) uq[mt] = Ur[(j * NMT + mt) * 64 + l];
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int ms = 0; ms < NMS; ++ms) kf[t][ms] = Kr[(t * NMS + ms) * 64 + l];
#pragma unroll
            for (int t = 0; t < NT; ++t) dd[t] = Dr[4 * t + cg];
            __builtin_amdgcn_sched_barrier(0);
            uint4 *xs = ex_s(k & 1, j), *xv = ex_v(k & 1, j);
            // S in bf16 as the contraction operand (permuted order), handed to the output waves
            uint4 Sb[NKK];
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
                Sb[kk] = make_uint4(pack2(S[2 * kk][0], S[2 * kk][1]), pack2(S[2 * kk][2], S[2 * kk][3]),
                                    pack2(S[2 * kk + 1][0], S[2 * kk + 1][1]),
                                    pack2(S[2 * kk + 1][2], S[2 * kk + 1][3]));
            // V_new = U - W S  (accumulator layout: rows 16mt+4cg+jj, column lr)
            f32x4 Pw[NMT];
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) Pw[mt] = zero4();
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int mt = 0; mt < NMT; ++mt) Pw[mt] = mma32_bf16(Pw[mt], wf[mt][kk], Sb[kk]);
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) xs[kk * 64 + l] = Sb[kk];
            f32x4 Vn[NMT];
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) {
                Vn[mt][0] = __uint_as_float(uq[mt].x << 16) - Pw[mt][0];
                Vn[mt][1] = __uint_as_float(uq[mt].x & 0xffff0000u) - Pw[mt][1];
                Vn[mt][2] = __uint_as_float(uq[mt].y << 16) - Pw[mt][2];
                Vn[mt][3] = __uint_as_float(uq[mt].y & 0xffff0000u) - Pw[mt][3];
            }
            uint4 Vb[NMS];
#pragma unroll
            for (int ms = 0; ms < NMS; ++ms)
                Vb[ms] = make_uint4(pack2(Vn[2 * ms][0], Vn[2 * ms][1]), pack2(Vn[2 * ms][2], Vn[2 * ms][3]),
                                    pack2(Vn[2 * ms + 1][0], Vn[2 * ms + 1][1]),
                                    pack2(Vn[2 * ms + 1][2], Vn[2 * ms + 1][3]));
            // S <- Diag(d) S + KgT V_new
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                S[t][0] *= dd[t].x;
                S[t][1] *= dd[t].y;
                S[t][2] *= dd[t].z;
                S[t][3] *= dd[t].w;
            }
#pragma unroll
            for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
                for (int t = 0; t < NT; ++t) S[t] = mma32_bf16(S[t], kf[t][ms], Vb[ms]);
#pragma unroll
            for (int ms = 0; ms < NMS; ++ms) xv[ms * 64 + l] = Vb[ms];
        }
        if (p.output_final_state) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) p.ht[sbase + (size_t)(16 * t + 4 * cg + jj) * V + col] = S[t][jj];
        }
    } else if (!is_loader) {
        // ------------------------------------------------------------ output wave o
        const int o = out_idx;
        const int mt0 = o * NMO;
        // this wave's rows of Qg [NMO][NKK] and of the non-zero Aqk blocks [NMO][NMS]
        struct QA {
            uint4 q[NMO][NKK];
            uint4 a[NMO][NMS];
        };
        auto load_qa = [&](QA &x, int k) {
            const size_t sl = slot_of(k);
            const uint4 *Qr = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.w_Qg) + sl * C * K);
            const uint4 *Ar = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.w_Aqk) + sl * C * C);
#pragma unroll
            for (int mo = 0; mo < NMO; ++mo) {
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) x.q[mo][kk] = Qr[((mt0 + mo) * NKK + kk) * 64 + l];
#pragma unroll
                for (int ms = 0; ms < NMS; ++ms)
                    if (32 * ms <= 16 * (mt0 + mo) + 15) x.a[mo][ms] = Ar[((mt0 + mo) * NMS + ms) * 64 + l];
            }
        };
        auto out_step = [&](const QA &x, int k) {
            // output rows of step k from hand-over buffer k & 1
            uint4 Sb[2][NKK], Vb[2][NMS];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint4 *xs = ex_s(k & 1, j), *xv = ex_v(k & 1, j);
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) Sb[j][kk] = xs[kk * 64 + l];
#pragma unroll
                for (int ms = 0; ms < NMS; ++ms) Vb[j][ms] = xv[ms * 64 + l];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int mo = 0; mo < NMO; ++mo) {
                    const int mt = mt0 + mo;
                    f32x4 acc = zero4();
#pragma unroll
                    for (int kk = 0; kk < NKK; ++kk) acc = mma32_bf16(acc, Sb[j][kk], x.q[mo][kk]);
#pragma unroll
                    for (int ms = 0; ms < NMS; ++ms)
                        if (32 * ms <= 16 * mt + 15) acc = mma32_bf16(acc, Vb[j][ms], x.a[mo][ms]);
                    // lane: row 16mt+lr, columns 16j+4cg..+3
                    *reinterpret_cast<uint2 *>(OS + (16 * mt + lr) * R::LDO + 16 * j + 4 * cg) =
                        make_uint2(pack2(acc[0], acc[1]), pack2(acc[2], acc[3]));
                }
            }
            const int64_t tok0 = sb + (int64_t)k * C;
            const int L = (int)((se - tok0) < C ? (se - tok0) : C);
#pragma unroll
            for (int it = 0; it < NMO; ++it) {
                const int m = 16 * mt0 + 16 * it + (l >> 2), c8 = 8 * (l & 3);
                if (m < L)
                    *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p.o) + ((tok0 + m) * p.HV + hv) * (int64_t)V +
                                               v0 + c8) = *reinterpret_cast<const uint4 *>(OS + m * R::LDO + c8);
            }
        };
        QA qa[2];
        // iteration k: prefetch step k's operands, barrier, output of step k - 1
        int k = 0;
        for (; k + 1 <= nsteps; k += 2) {
            load_qa(qa[0], k);
            __syncthreads();
            if (k >= 1) out_step(qa[1], k - 1);
            if (k + 1 < nsteps) load_qa(qa[1], k + 1);
            __syncthreads();
            out_step(qa[0], k);
        }
        if (k <= nsteps) {  // k == nsteps: the last barrier and the final output
            __syncthreads();
            if (k >= 1) out_step(qa[1], k - 1);
        }
    } else {
        // ------------------------------------------------------------ loader wave i
        const int i = wid - 4;
        auto issue = [&](int k) {
            if (i == 0) ring_issue<C, K, 0>(p, ring, slot_of(k), k, v0, l);
            else ring_issue<C, K, 1>(p, ring, slot_of(k), k, v0, l);
        };
        auto wait_one_step = [&]() {
            if (i == 0) wait_vmcnt<R::nload(0)>();
            else wait_vmcnt<R::nload(1)>();
        };
        if (nsteps > 0) issue(0);
        if (nsteps > 1) {
            issue(1);
            wait_one_step();
        } else {
            wait_vmcnt<0>();
        }
        for (int k = 0; k <= nsteps; ++k) {
            __builtin_amdgcn_s_barrier();
            if (k + 2 < nsteps) {
                issue(k + 2);
                wait_one_step();  // step k + 1 has landed
            } else {
                wait_vmcnt<0>();
            }
        }
    }
}

template <int C>
hipError_t launch_recur_reg(const Params &p, hipStream_t s) {
    const int units = p.N * p.HV;
    const int per_xcd = (units + kXCD - 1) / kXCD;
    const dim3 grid((unsigned)(per_xcd * kXCD * (p.V / kBV)));
    hipError_t e = hipSuccess;
    auto go = [&](auto kern, size_t lds) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds);
        if (e != hipSuccess) return;
        hipLaunchKernelGGL(kern, grid, dim3(64 * (4 + C / 16)), lds, s, p);
        e = hipGetLastError();
    };
    switch (p.K / 32) {
    case 1: go(recur_reg_kernel<C, 1>, RegRecur<C, 32>::kBytes); break;
    case 2: go(recur_reg_kernel<C, 2>, RegRecur<C, 64>::kBytes); break;
    case 3: go(recur_reg_kernel<C, 3>, RegRecur<C, 96>::kBytes); break;
    case 4: go(recur_reg_kernel<C, 4>, RegRecur<C, 128>::kBytes); break;
    default: return hipErrorInvalidValue;
    }
    return e;
}

}  // namespace kda
