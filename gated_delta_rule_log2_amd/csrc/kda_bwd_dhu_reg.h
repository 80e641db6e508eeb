// kda_bwd_dhu_reg.h -- the reverse chunk recurrence of the KDA backward for bf16
// intermediates and K <= 128, with the state gradient kept in registers ("Reading Notes:
// Implementation Notes for KDA in FLA", backward step 4):
//   dU  = Aqk^T dO + Kg dS                  the gradient of V_new = U - W S_prev
//   dS <- Diag(d) dS + Qg^T dO - W^T dU      the gradient of S_prev
// per (sequence, value head, 32-column slice of V), chunks last to first.
//
// Every product of the chain contracts over a different index than the forward's
// product with the same matrix (Kg over the key index, W, Qg and Aqk over the chunk
// row), so the forward's operand fragments do not serve: bwd_prep_kernel first writes,
// per (chunk, value head), the fragments of the transposed matrices (Kg, W^T, Qg^T,
// Aqk^T, permuted row fragments as the forward uses) and dO in accumulator-tile order.
//
// bwd_dhu_reg_kernel then mirrors the forward's register-resident recurrence, with
// 4 + C/16 waves per workgroup:
//   waves 0, 1  state waves: wave j owns columns 16j..16j+15 of the slice and all K rows
//               of dS (fp32 accumulators).  dS and dU in accumulator layout are, converted
//               to bf16 in place, the contraction operands of the next products, so
//               dS -> Kg dS -> dU -> W^T dU -> dS runs inside one wave.  Each step's Kg,
//               W^T and decay are read from the LDS ring during the step before.
//   C/16 P-waves, one step ahead: the terms that do not depend on the chain,
//               P1 = Aqk^T dO and P2 = Qg^T dO, for both 16-column halves, handed to the
//               state waves through LDS (bf16, double-buffered by step parity); their
//               operands are loaded from global memory two steps ahead.
//   2 loaders   stream each step's Kg, W^T (fragments) and decay into a 4-slot ring with
//               direct global->LDS loads: after barrier b they fill the slot of step b + 3
//               (the one step b - 1 used) and wait for what they issued a step earlier.
// Roles are numbered as in the forward so the state waves share their SIMDs only with
// the loaders.  One barrier per step.  Workgroups are placed XCD-aware as in the forward.
#pragma once

#include "kda_bwd_dhu.h"
#include "kda_recur_reg.h"

namespace kda {

// ---------------------------------------------------------------- operand preparation

// Element counts (bf16) of the prepared operands of one (chunk, value head) slot.
template <int C, int K>
struct DhuPack {
    static constexpr size_t ring = 2 * (size_t)C * K;         // Kg [C][K], then W^T [K][C]
    static constexpr size_t pterm = (size_t)C * C + (size_t)K * C;  // Aqk^T [C][C], then Qg^T [K][C]
};

// Transposes one permuted-fragment bf16 matrix X [R][NC] into the permuted fragments of
// X^T [NC][R] through LDS (buf: R rows of NC + 8), in two steps so that a workgroup can
// request all of its matrices before staging the first: `load` brings this thread's units
// into registers, `stage_store` writes them through LDS as X^T.  CAUSAL: X is lower
// triangular and its units right of the 16-row block's diagonal are zeros that were not
// written.
template <int R, int NC, bool CAUSAL>
struct PfragT {
    static constexpr int NU = R * NC / 8, NPT = (NU + 255) / 256, LD = NC + 8;
    static_assert(NU % 64 == 0, "whole waves");
    __device__ static void load(const uint16_t *src, uint4 (&x)[NPT]) {
#pragma unroll
        for (int k = 0; k < NPT; ++k) {
            const int u = (int)threadIdx.x + 256 * k;
            x[k] = make_uint4(0u, 0u, 0u, 0u);
            if (u < NU) {
                int row, col[8];
                unit_coords<true>(u, NC, row, col);
                if (!(CAUSAL && col[0] - col[0] % 32 > (row | 15))) x[k] = *reinterpret_cast<const uint4 *>(src + (size_t)u * 8);
            }
        }
    }
    __device__ static void stage_store(const uint4 (&x)[NPT], uint16_t *buf, uint16_t *dst) {
#pragma unroll
        for (int k = 0; k < NPT; ++k) {
            const int u = (int)threadIdx.x + 256 * k;
            if (u < NU) {
                int row, col[8];
                unit_coords<true>(u, NC, row, col);
                *reinterpret_cast<uint2 *>(buf + row * LD + col[0]) = make_uint2(x[k].x, x[k].y);
                *reinterpret_cast<uint2 *>(buf + row * LD + col[4]) = make_uint2(x[k].z, x[k].w);
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < NPT; ++k) {
            const int u = (int)threadIdx.x + 256 * k;
            if (u < NU) {
                int orow, ocol[8];
                unit_coords<true>(u, R, orow, ocol);  // X^T has NC rows and R columns
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = (uint32_t)buf[ocol[2 * e] * LD + orow] | ((uint32_t)buf[ocol[2 * e + 1] * LD + orow] << 16);
                *reinterpret_cast<uint4 *>(dst + (size_t)u * 8) = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
        __syncthreads();
    }
};

// One workgroup of 256 threads per (chunk, value head) slot.
template <int C, int NKK>
__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdChunkParams P) {
    constexpr int K = 32 * NKK;
    constexpr int RMAX = C > K ? C : K;
    __shared__ __align__(16) uint16_t buf[RMAX * (RMAX + 8)];
    const Params &p = P.f;
    const size_t slot = blockIdx.x;
    const int gc = (int)(slot / p.HV), hv = (int)(slot % p.HV);
    using PK = DhuPack<C, K>;
    const uint16_t *Aqk = static_cast<const uint16_t *>(p.w_Aqk) + slot * C * C;
    const uint16_t *Qg = static_cast<const uint16_t *>(p.w_Qg) + slot * C * K;
    const uint16_t *W = static_cast<const uint16_t *>(p.w_W) + slot * C * K;
    const uint16_t *KgT = static_cast<const uint16_t *>(p.w_KgT) + slot * K * C;
    uint16_t *ring = P.rpack + slot * PK::ring, *pterm = P.ppack + slot * PK::pterm;
    // all four matrices requested before the first is staged
    using TK = PfragT<K, C, false>;
    using TW = PfragT<C, K, false>;
    using TA = PfragT<C, C, true>;
    uint4 xk[TK::NPT], xw[TW::NPT], xa[TA::NPT], xq[TW::NPT];
    TK::load(KgT, xk);
    TW::load(W, xw);
    TA::load(Aqk, xa);
    TW::load(Qg, xq);
    TK::stage_store(xk, buf, ring);                      // Kg     [C][K]
    TW::stage_store(xw, buf, ring + (size_t)C * K);      // W^T    [K][C]
    TA::stage_store(xa, buf, pterm);                     // Aqk^T  [C][C]
    TW::stage_store(xq, buf, pterm + (size_t)C * C);     // Qg^T   [K][C]
    // dO of the chunk in accumulator-tile order (see quad_off), rows past the end zero
    const ChunkInfo ci = chunk_info(p, gc);
    const int V = p.V;
    uint16_t *dq = P.doq + slot * (size_t)V * C;
    const uint16_t *dout = static_cast<const uint16_t *>(P.b.dout);
    for (int e = threadIdx.x; e < V * C / 4; e += blockDim.x) {
        // quad e: tile (vt, mt), lane (v & 15) + 16 ((m & 15) >> 2), rows m..m+3 of column v
        const int unit = e >> 6, lane = e & 63;
        const int vt = unit / (C / 16), mt = unit % (C / 16);
        const int v = 16 * vt + (lane & 15), m0 = 16 * mt + 4 * (lane >> 4);
        uint16_t x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            x[r] = (m0 + r < ci.L) ? dout[((ci.tok0 + m0 + r) * p.HV + hv) * (int64_t)V + v] : (uint16_t)0;
        *reinterpret_cast<uint2 *>(dq + (size_t)e * 4) =
            make_uint2((uint32_t)x[0] | ((uint32_t)x[1] << 16), (uint32_t)x[2] | ((uint32_t)x[3] << 16));
    }
}

// ---------------------------------------------------------------- the recurrence

template <int C, int K>
struct DhuReg {
    static constexpr int NKK = K / 32, NMT = C / 16, NMS = C / 32, NT = K / 16;
    static constexpr int NS = 4;                     // ring slots
    static constexpr int NU = C * K * 2 / 1024;      // 1 KB fragment units of Kg (and of W^T)
    static constexpr size_t kA = 0, kWT = (size_t)NU * 1024, kD = 2 * (size_t)NU * 1024;
    static constexpr size_t kSlot = kD + (size_t)K * 4;
    static __device__ size_t slot_off(int m) { return (size_t)(m % NS) * kSlot; }
    // hand-over of P1 (tiles 2 mt + vt) and P2 (tiles 2 NMT + 2 t + vt): 64 lanes x 4 bf16
    static constexpr int NPT = 2 * (NMT + NT);
    static constexpr int NTAU = NPT / NMT;           // tiles per P-wave
    static constexpr size_t kP = NS * kSlot, kPBuf = (size_t)NPT * 512;
    static constexpr size_t kBytes = kP + 2 * kPBuf;
    // ring loads per step of loader i: its units (alternate), loader 1 also the decay
    static constexpr int nload(int i) { return (2 * NU - i + 1) / 2 + (i == 1 ? 1 : 0); }
    static_assert(NPT % NMT == 0 && NMT % 2 == 0, "P tiles dealt evenly, one column half per P-wave");
    static_assert(nload(0) <= 63 && nload(1) <= 63, "loader wait count");
    static_assert(K / 4 <= 64, "decay in one load");
    static_assert(kBytes <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ f32x4 unpack_bf16x4(uint2 x) {
    return f32x4{__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u), __uint_as_float(x.y << 16),
                 __uint_as_float(x.y & 0xffff0000u)};
}

template <int C, int NKK>
__global__ void __launch_bounds__(64 * (4 + C / 16)) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dhu_reg_kernel(BwdChunkParams P) {
    constexpr int K = 32 * NKK;
    using R = DhuReg<C, K>;
    using PK = DhuPack<C, K>;
    constexpr int NMT = R::NMT, NMS = R::NMS, NT = R::NT, NTAU = R::NTAU;
    extern __shared__ __align__(16) unsigned char lds[];
    const Params &p = P.f;
    const BwdParams &b = P.b;
    const int V = p.V;

    const int nvt = V / kBV;
    const int xcd = blockIdx.x % kXCD, pos = blockIdx.x / kXCD;
    const int u = (pos / nvt) * kXCD + xcd;
    if (u >= p.N * p.HV) return;
    const int n = p.cu_seqlens ? p.seq_order[u / p.HV] : u / p.HV, hv = u % p.HV;
    const int v0 = kBV * (pos % nvt);
    const int wid = threadIdx.x >> 6, l = lane_id(), lr = l & 15, cg = l >> 4;
    const bool is_state = wid < 2, is_loader = wid == 4 || wid == 5;
    const int pidx = wid < 4 ? wid - 2 : wid - 4;

    const int c0 = seq_chunk_begin(p, n), nsteps = seq_chunk_begin(p, n + 1) - c0;
    // step m handles chunk c0 + nsteps - 1 - m
    auto slot_of = [&](int m) { return (size_t)(c0 + nsteps - 1 - m) * p.HV + hv; };
    auto pbuf = [&](int m) { return reinterpret_cast<uint2 *>(lds + R::kP + (size_t)(m & 1) * R::kPBuf); };

    if (is_state) {
        // ------------------------------------------------------------ state wave j
        const int j = wid;
        const int col = v0 + 16 * j + lr;
        f32x4 dS[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            dS[t] = zero4();
            if (b.dht) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    dS[t][jj] = b.dht[(((size_t)n * p.HV + hv) * K + 16 * t + 4 * cg + jj) * V + col];
            }
        }
        struct Ops {
            uint4 a[NMT][NKK], wt[NT][NMS];
            float4 d[NT];
        };
        auto read_a = [&](Ops &o, int m) {
            const uint4 *Ar = reinterpret_cast<const uint4 *>(lds + R::slot_off(m) + R::kA);
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) o.a[mt][kk] = Ar[(mt * NKK + kk) * 64 + l];
        };
        auto read_d = [&](Ops &o, int m) {
            const float4 *Dr = reinterpret_cast<const float4 *>(lds + R::slot_off(m) + R::kD);
#pragma unroll
            for (int t = 0; t < NT; ++t) o.d[t] = Dr[4 * t + cg];
        };
        auto read_w = [&](Ops &o, int m) {
            const uint4 *Wr = reinterpret_cast<const uint4 *>(lds + R::slot_off(m) + R::kWT);
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int ms = 0; ms < NMS; ++ms) o.wt[t][ms] = Wr[(t * NMS + ms) * 64 + l];
        };
        Ops o;
        __syncthreads();  // ring steps 0 and 1 have landed
        if (nsteps > 0) {
            read_a(o, 0);
            read_d(o, 0);
            read_w(o, 0);
        }
        __syncthreads();  // P(0) handed over
        auto step = [&](int m, auto next_tag) {
            constexpr bool has_next = decltype(next_tag)::value;
            const size_t sl = slot_of(m);
            const uint2 *PB = pbuf(m);
            uint2 p1[NMT];
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) p1[mt] = PB[(2 * mt + j) * 64 + l];
            // the gradient of the state after this chunk, for the per-chunk gradients, in
            // fragment order: float4 ((v0 / 32 * 2 + j) * NT + t) * 64 + lane of the chunk's
            // K x V block holds rows 16t + 4cg .. +3 of column v0 + 16 j + lr
            float4 *gdh = reinterpret_cast<float4 *>(P.dh + sl * K * (size_t)V) + ((size_t)(v0 / kBV) * 2 + j) * NT * 64 + l;
#pragma unroll
            for (int t = 0; t < NT; ++t)  // read back by a later kernel: non-temporal
                store16_once(gdh + t * 64, make_uint4(__float_as_uint(dS[t][0]), __float_as_uint(dS[t][1]),
                                                      __float_as_uint(dS[t][2]), __float_as_uint(dS[t][3])));
            uint4 Sb[NKK];
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
                Sb[kk] = make_uint4(pack2(dS[2 * kk][0], dS[2 * kk][1]), pack2(dS[2 * kk][2], dS[2 * kk][3]),
                                    pack2(dS[2 * kk + 1][0], dS[2 * kk + 1][1]),
                                    pack2(dS[2 * kk + 1][2], dS[2 * kk + 1][3]));
            // dU = P1 + Kg dS  (accumulator layout: rows 16mt + 4cg + jj, column lr)
            f32x4 dU[NMT];
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) dU[mt] = unpack_bf16x4(p1[mt]);
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int mt = 0; mt < NMT; ++mt) dU[mt] = mma32_bf16(dU[mt], o.a[mt][kk], Sb[kk]);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (has_next) read_a(o, m + 1);
            uint2 p2[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) p2[t] = PB[(2 * NMT + 2 * t + j) * 64 + l];
            // -dU in bf16 as the operand of the update
            uint4 Ub[NMS];
#pragma unroll
            for (int ms = 0; ms < NMS; ++ms)
                Ub[ms] = make_uint4(pack2(-dU[2 * ms][0], -dU[2 * ms][1]), pack2(-dU[2 * ms][2], -dU[2 * ms][3]),
                                    pack2(-dU[2 * ms + 1][0], -dU[2 * ms + 1][1]),
                                    pack2(-dU[2 * ms + 1][2], -dU[2 * ms + 1][3]));
            // dU in the same fragment order over the chunk's C x V block (NMT row tiles)
            float4 *gdu = reinterpret_cast<float4 *>(P.dU + sl * C * (size_t)V) + ((size_t)(v0 / kBV) * 2 + j) * NMT * 64 + l;
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt)
                store16_once(gdu + mt * 64, make_uint4(__float_as_uint(dU[mt][0]), __float_as_uint(dU[mt][1]),
                                                       __float_as_uint(dU[mt][2]), __float_as_uint(dU[mt][3])));
            // dS <- Diag(d) dS + P2 - W^T dU
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const f32x4 p2v = unpack_bf16x4(p2[t]);
                dS[t][0] = o.d[t].x * dS[t][0] + p2v[0];
                dS[t][1] = o.d[t].y * dS[t][1] + p2v[1];
                dS[t][2] = o.d[t].z * dS[t][2] + p2v[2];
                dS[t][3] = o.d[t].w * dS[t][3] + p2v[3];
            }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (has_next) read_d(o, m + 1);
#pragma unroll
            for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
                for (int t = 0; t < NT; ++t) dS[t] = mma32_bf16(dS[t], o.wt[t][ms], Ub[ms]);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (has_next) read_w(o, m + 1);
            // Barrier m + 1.  Nothing of this wave needs to complete first: the P buffer it
            // read is rewritten only after barrier m + 2, and the ring reads of step m + 1
            // now in flight touch a slot the loaders refill only after barrier m + 3.
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        for (int m = 0; m + 1 < nsteps; ++m) step(m, std::true_type{});
        if (nsteps > 0) step(nsteps - 1, std::false_type{});
        if (b.dh0) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    b.dh0[(((size_t)n * p.HV + hv) * K + 16 * t + 4 * cg + jj) * V + col] = dS[t][jj];
        }
    } else if (!is_loader) {
        // ------------------------------------------------------------ P-wave o
        // tiles tau = o + NMT q: P1 tile (mt, vt) = (tau / 2, tau % 2) for tau < 2 NMT, else
        // P2 tile (t, vt) = ((tau - 2 NMT) / 2, tau % 2); vt = o % 2 throughout
        const int o = pidx;
        const int vt = o & 1;
        struct PO {
            uint4 a[NTAU][NMS];
            uint4 bo[NMS];
        };
        auto nonzero = [&](int tau, int ms) {  // Aqk^T unit (mt, ms) holds rows j, columns i >= j
            return tau >= 2 * NMT || 32 * ms + 31 >= 16 * (tau >> 1);
        };
        auto load = [&](PO &x, int m) {
            const size_t sl = slot_of(m);
            const uint4 *At = reinterpret_cast<const uint4 *>(P.ppack + sl * PK::pterm);
            const uint4 *Qt = reinterpret_cast<const uint4 *>(P.ppack + sl * PK::pterm + (size_t)C * C);
#pragma unroll
            for (int q = 0; q < NTAU; ++q) {
                const int tau = o + NMT * q;
#pragma unroll
                for (int ms = 0; ms < NMS; ++ms) {
                    if (tau < 2 * NMT) {
                        if (nonzero(tau, ms)) x.a[q][ms] = At[((tau >> 1) * NMS + ms) * 64 + l];
                    } else {
                        x.a[q][ms] = Qt[(((tau - 2 * NMT) >> 1) * NMS + ms) * 64 + l];
                    }
                }
            }
            const uint2 *Dq = reinterpret_cast<const uint2 *>(P.doq + sl * (size_t)V * C);
#pragma unroll
            for (int ms = 0; ms < NMS; ++ms) {
                const int vtile = (v0 >> 4) + vt;
                const uint2 lo = Dq[(vtile * NMT + 2 * ms) * 64 + l], hi = Dq[(vtile * NMT + 2 * ms + 1) * 64 + l];
                x.bo[ms] = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
        };
        auto compute = [&](const PO &x, int m) {
            uint2 *PB = pbuf(m);
#pragma unroll
            for (int q = 0; q < NTAU; ++q) {
                const int tau = o + NMT * q;
                f32x4 acc = zero4();
#pragma unroll
                for (int ms = 0; ms < NMS; ++ms)
                    if (nonzero(tau, ms)) acc = mma32_bf16(acc, x.a[q][ms], x.bo[ms]);
                PB[tau * 64 + l] = make_uint2(pack2(acc[0], acc[1]), pack2(acc[2], acc[3]));
            }
        };
        PO buf[3];
        if (nsteps > 0) load(buf[0], 0);
        if (nsteps > 1) load(buf[1], 1);
        if (nsteps > 2) load(buf[2], 2);
        if (nsteps > 0) compute(buf[0], 0);
        __syncthreads();  // ring prologue
        __syncthreads();  // P(0) handed over
        // iteration m (after barrier m): P(m + 1) from the buffer loaded two iterations
        // earlier, then step m + 3's operands into the buffer step m used
        auto iter = [&](int m, PO &cb, PO &lb) {
            if (m + 1 < nsteps) compute(cb, m + 1);
            if (m + 3 < nsteps) load(lb, m + 3);
            __syncthreads();  // barrier m + 1
        };
        for (int m = 0; m < nsteps; m += 3) {
            iter(m, buf[1], buf[0]);
            if (m + 1 >= nsteps) break;
            iter(m + 1, buf[2], buf[1]);
            if (m + 2 >= nsteps) break;
            iter(m + 2, buf[0], buf[2]);
        }
    } else {
        // ------------------------------------------------------------ loader wave i
        const int i = wid - 4;
        auto issue = [&](int m) {
            if (m >= nsteps) return;
            const size_t sl = slot_of(m);
            unsigned char *dst = lds + R::slot_off(m);
            const unsigned char *src = reinterpret_cast<const unsigned char *>(P.rpack + sl * PK::ring);
#pragma unroll
            for (int uu = 0; uu < 2 * R::NU; uu += 2) {
                const int un = uu + i;
                if (un < 2 * R::NU) lds_dma16(src + un * 1024 + l * 16, dst + un * 1024);
            }
            if (i == 1 && l < K / 4) lds_dma16(reinterpret_cast<const unsigned char *>(p.w_d + sl * K) + l * 16, dst + R::kD);
        };
        auto wait_all_but = [&](int mr) {
            if (mr < nsteps) {
                if (i == 0) wait_vmcnt<R::nload(0)>();
                else wait_vmcnt<R::nload(1)>();
            } else {
                wait_vmcnt<0>();
            }
        };
        for (int m = 0; m < 3; ++m) issue(m);
        wait_all_but(2);
        __builtin_amdgcn_s_barrier();  // steps 0 and 1 landed
        for (int bb = 0; bb <= nsteps; ++bb) {
            __builtin_amdgcn_s_barrier();  // barrier bb: step bb - 1's slot is free
            issue(bb + 3);
            wait_all_but(bb + 3);
        }
    }
}

template <int C, int NKK>
hipError_t launch_bwd_prep_t(const BwdChunkParams &p, hipStream_t s) {
    const unsigned slots = (unsigned)p.f.total_chunks * (unsigned)p.f.HV;
    if (slots > 0) hipLaunchKernelGGL((bwd_prep_kernel<C, NKK>), dim3(slots), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int C, int NKK>
hipError_t launch_bwd_dhu_reg_t(const BwdChunkParams &p, hipStream_t s) {
    constexpr int K = 32 * NKK;
    if (!p.prep_done) {
        const hipError_t e = launch_bwd_prep_t<C, NKK>(p, s);
        if (e != hipSuccess) return e;
    }
    const int units = p.f.N * p.f.HV;
    if (units == 0) return hipSuccess;
    const int per_xcd = (units + kXCD - 1) / kXCD;
    const dim3 grid((unsigned)(per_xcd * kXCD * (p.f.V / kBV)));
    auto kern = bwd_dhu_reg_kernel<C, NKK>;
    const size_t lds = DhuReg<C, K>::kBytes;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(64 * (4 + C / 16)), lds, s, p);
    return hipGetLastError();
}

}  // namespace kda
