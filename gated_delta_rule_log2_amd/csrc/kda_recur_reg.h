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
//               inside one wave.  Each operand is read from the ring one phase ahead of
//               its use (the next step's W and U during the current update, KgT while
//               W S runs), so LDS latency stays off the chain.
//   C/16 output waves, one step behind: output wave o forms O = Qg S + Aqk V_new for
//               chunk rows 16o..16o+15 and both column halves, from the S and V_new
//               the state waves hand over through LDS, with its rows of Qg and Aqk
//               prefetched two steps ahead into its own registers.  The state waves'
//               columns are interleaved in groups of 4, so each output lane holds 8
//               consecutive columns of one row and writes them with one 16-byte store.
//   2 loaders   stream each step's W and U slice (3-slot ring) and KgT and d (4-slot
//               ring) into LDS with direct global->LDS loads: after barrier k they
//               fill the slots of step k + 3 and wait for what they issued a step
//               earlier before barrier k + 1, so step k + 1 has landed a full step
//               before the state waves read it during step k.
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
    static constexpr int NSW = 3, NSK = 4;  // ring slots for W/U and for KgT/d
    static constexpr int NWAVES = 4 + NMT;  // 2 state, NMT output, 2 loader waves
    // ring slots (bytes): W [NMT][NKK] fragment units of 1 KB then U for the slice's two
    // 16-column tiles ([2][NMT] quad units of 512 B); KgT [NT][NMS] units of 1 KB then d [K]
    static constexpr int NLW = C * K * 2 / 1024, NLU = C * 32 * 2 / 1024;
    static constexpr size_t kW = 0, kU = (size_t)NLW * 1024, kWSlot = kU + (size_t)NLU * 1024;
    static constexpr size_t kKgT = 0, kD = (size_t)NLW * 1024, kKSlot = kD + (size_t)K * 4;
    static constexpr size_t kRingK = NSW * kWSlot;
    static __device__ size_t wslot(int k) { return (size_t)(k % NSW) * kWSlot; }
    static __device__ size_t kslot(int k) { return kRingK + (size_t)(k % NSK) * kKSlot; }
    // hand-over buffers [2][2 state waves]: S as [NKK] operand units, V_new as [NMS] units
    static constexpr size_t kExWave = (size_t)(NKK + NMS) * 1024;
    static constexpr size_t kEx = kRingK + NSK * kKSlot;
    static constexpr size_t kBytes = kEx + 4 * kExWave;
    // 1 KB ring units per step, dealt to the two loader waves alternately: the W and U
    // part (NLW + NLU units) and the KgT part (NLW units; loader 1 also loads d, 16 bytes
    // on each of the first K/4 lanes).  Loads each loader issues per part:
    static constexpr int nload_w(int i) { return (NLW + NLU - i + 1) / 2; }
    static constexpr int nload_k(int i) { return (NLW - i + 1) / 2 + (i == 1 ? 1 : 0); }
    static_assert(2 * (nload_w(0) + nload_k(0)) <= 63 && 2 * (nload_w(1) + nload_k(1)) <= 63, "loader wait count");
    static_assert(K / 4 <= 64, "d in one load");
    static_assert(kBytes <= 160 * 1024, "LDS budget");
};

// s_waitcnt immediate that waits until at most n vector-memory operations of this wave
// are outstanding (expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// s_waitcnt immediate that waits until at most n LDS/scalar-memory operations of this
// wave are outstanding (vmcnt and expcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
    static_assert(N >= 0 && N <= 15, "lgkmcnt range");
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (N << 8) | (3 << 14));
}

__device__ __forceinline__ void lds_dma16(const void *g, void *l) {
    __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}

// Loader wave I: its share of step k's W and U (W/U slot k % NSW).
template <int C, int K, int I>
__device__ __forceinline__ void ring_issue_w(const Params &p, unsigned char *ring, size_t sl, int k, int v0, int l) {
    using R = RegRecur<C, K>;
    unsigned char *dst = ring + R::wslot(k);
    const unsigned char *gW = reinterpret_cast<const unsigned char *>(p.w_W) + sl * C * K * 2;
    const unsigned char *gU =
        reinterpret_cast<const unsigned char *>(p.w_U) + (sl * (size_t)p.V * C + quad_off(0, v0, C)) * 2;
#pragma unroll
    for (int u = I; u < R::NLW + R::NLU; u += 2) {
        if (u < R::NLW) lds_dma16(gW + u * 1024 + l * 16, dst + R::kW + u * 1024);
        else lds_dma16(gU + (u - R::NLW) * 1024 + l * 16, dst + R::kU + (u - R::NLW) * 1024);
    }
}

// Loader wave I: its share of step k's KgT and d (KgT/d slot k % NSK).
template <int C, int K, int I>
__device__ __forceinline__ void ring_issue_k(const Params &p, unsigned char *ring, size_t sl, int k, int l) {
    using R = RegRecur<C, K>;
    unsigned char *dst = ring + R::kslot(k);
    const unsigned char *gK = reinterpret_cast<const unsigned char *>(p.w_KgT) + sl * K * C * 2;
    const unsigned char *gD = reinterpret_cast<const unsigned char *>(p.w_d + sl * K);
#pragma unroll
    for (int u = I; u < R::NLW; u += 2) lds_dma16(gK + u * 1024 + l * 16, dst + R::kKgT + u * 1024);
    if constexpr (I == 1) {
        if (l < K / 4) lds_dma16(gD + l * 16, dst + R::kD);
    }
}

// HS: also write the state each chunk starts from (p.hs); a separate instantiation so
// the stores add no register pressure to the plain forward.  With p.hs_frag the states
// are written in this kernel's own fragment order, one 16-byte store per lane and tile:
// within the K x V state of a (chunk, value head), the float4 at index
// ((vs * 2 + j) * NT + t) * 64 + lane holds rows 16t + 4cg .. +3 of column
// 32 vs + 8 (lr / 4) + 4 j + lr % 4 (vs: 32-column slice, j: state wave, lane = 16 cg + lr)
// -- the backward's per-chunk kernel reads that order back.  With p.skip_output (the
// backward's recompute, which needs the states and not o) the output waves only keep
// the barrier count.
template <int C, int NKK, bool HS>
__global__ void __launch_bounds__(64 * (4 + C / 16)) __attribute__((amdgpu_waves_per_eu(2, 2)))
recur_reg_kernel(Params p) {
    constexpr int K = 32 * NKK;
    using R = RegRecur<C, K>;
    constexpr int NMT = R::NMT, NMS = R::NMS, NT = R::NT;
    extern __shared__ __align__(16) unsigned char lds[];
    const int V = p.V;

    // XCD-aware decode: workgroup b runs on XCD b % 8; unit u = (n, hv) lives on XCD u % 8
    const int nvt = V / kBV;
    const int xcd = blockIdx.x % kXCD, pos = blockIdx.x / kXCD;
    const int u = (pos / nvt) * kXCD + xcd;
    if (u >= p.N * p.HV) return;
    const int n = p.cu_seqlens ? p.seq_order[u / p.HV] : u / p.HV, hv = u % p.HV;  // longest first
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

    if (is_state) {
        // ------------------------------------------------------------ state wave j
        const int j = wid;
        // lane lr holds slice column cc = 8 (lr / 4) + 4 j + lr % 4, so that an output lane
        // ends up with 8 consecutive columns of one row (see the output wave)
        const int cc = 8 * (lr >> 2) + 4 * j + (lr & 3);
        const int col = v0 + cc;
        const size_t sbase = ((size_t)n * p.HV + hv) * K * V;
        // offset of state element (key row, this lane's column) in a [K][V] or [V][K] state
        auto sidx = [&](int row) { return p.state_vk ? (size_t)col * K + row : (size_t)row * V + col; };
        f32x4 S[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            S[t] = zero4();
            if (p.h0) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) S[t][jj] = p.h0[sbase + sidx(16 * t + 4 * cg + jj)];
            }
        }
        // the state chunk c0 + k starts from, into the intermediate-state output: a per-step
        // uniform base plus this lane's offset (rows 4cg.., its column), fixed for the kernel
        const uint32_t hs_lane = p.state_vk ? (uint32_t)col * K + 4 * cg : (uint32_t)(4 * cg) * V + col;
        auto put_states = [&](int k) {
            float *hb = p.hs + ((size_t)(c0 + k) * p.HV + hv) * K * V;
            if (p.hs_frag) {
                float4 *fb = reinterpret_cast<float4 *>(hb) + ((size_t)(v0 / kBV) * 2 + j) * NT * 64 + l;
#pragma unroll
                for (int t = 0; t < NT; ++t)  // read back by a later kernel: non-temporal
                    store16_once(fb + t * 64, make_uint4(__float_as_uint(S[t][0]), __float_as_uint(S[t][1]),
                                                         __float_as_uint(S[t][2]), __float_as_uint(S[t][3])));
            } else if (p.state_vk) {
#pragma unroll
                for (int t = 0; t < NT; ++t)  // rows 16t + 4cg .. +3 are contiguous in [V][K]
                    *reinterpret_cast<float4 *>(hb + hs_lane + 16 * t) = make_float4(S[t][0], S[t][1], S[t][2], S[t][3]);
            } else {
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) (hb + (size_t)(16 * t + jj) * V)[hs_lane] = S[t][jj];
            }
        };
        // one step's ring operands in registers
        struct Ops {
            uint4 w[NMT][NKK], kg[NT][NMS];
            uint2 u[NMT];
            float4 d[NT];
        };
        auto read_w = [&](Ops &o, int k) {  // W and U of step k
            const unsigned char *sl = ring + R::wslot(k);
            const uint4 *Wr = reinterpret_cast<const uint4 *>(sl + R::kW);
            const uint2 *Ur = reinterpret_cast<const uint2 *>(sl + R::kU);
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) o.w[mt][kk] = Wr[(mt * NKK + kk) * 64 + l];
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) o.u[mt] = Ur[((cc >> 4) * NMT + mt) * 64 + (cc & 15) + 16 * cg];
        };
        auto read_d = [&](Ops &o, int k) {  // decay of step k
            const float4 *Dr = reinterpret_cast<const float4 *>(ring + R::kslot(k) + R::kD);
#pragma unroll
            for (int t = 0; t < NT; ++t) o.d[t] = Dr[4 * t + cg];
        };
        auto read_k = [&](Ops &o, int k) {  // KgT of step k
            const uint4 *Kr = reinterpret_cast<const uint4 *>(ring + R::kslot(k) + R::kKgT);
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int ms = 0; ms < NMS; ++ms) o.kg[t][ms] = Kr[(t * NMS + ms) * 64 + l];
        };
        // Each operand is re-read in place once its last use in the current step has been
        // issued: the decay, W and U of step k + 1 after V_new, KgT of step k + 1 after the
        // update (all landed before barrier k).  The step ends with a barrier that waits only
        // for this wave's hand-over writes (and so for the W/U reads issued before them: LDS
        // operations of one wave complete in order); the KgT reads issued after them stay in
        // flight across it, and the loaders refill that KgT slot only after the next barrier.
        Ops o;
        __syncthreads();  // step 0 and step 1 have landed
        if (nsteps > 0) {
            read_d(o, 0);  // same order as inside the loop, so the LDS waits line up
            read_w(o, 0);
            read_k(o, 0);
        }
        // step 0's W/U slot is the one the loaders refill first (with step 3): the reads
        // above complete before the barrier that lets them start
        wait_lgkmcnt<0>();
        __syncthreads();
        auto step = [&](int k, auto next_tag) {
            constexpr bool has_next = decltype(next_tag)::value;
            uint4 *xs = ex_s(k & 1, j), *xv = ex_v(k & 1, j);
            if constexpr (HS) put_states(k);
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
                for (int mt = 0; mt < NMT; ++mt) Pw[mt] = mma32_bf16(Pw[mt], o.w[mt][kk], Sb[kk]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) xs[kk * 64 + l] = Sb[kk];
            f32x4 Vn[NMT];
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) {
                Vn[mt][0] = __uint_as_float(o.u[mt].x << 16) - Pw[mt][0];
                Vn[mt][1] = __uint_as_float(o.u[mt].x & 0xffff0000u) - Pw[mt][1];
                Vn[mt][2] = __uint_as_float(o.u[mt].y << 16) - Pw[mt][2];
                Vn[mt][3] = __uint_as_float(o.u[mt].y & 0xffff0000u) - Pw[mt][3];
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
                S[t][0] *= o.d[t].x;
                S[t][1] *= o.d[t].y;
                S[t][2] *= o.d[t].z;
                S[t][3] *= o.d[t].w;
            }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (has_next) {
                read_d(o, k + 1);
                read_w(o, k + 1);
            }
#pragma unroll
            for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
                for (int t = 0; t < NT; ++t) S[t] = mma32_bf16(S[t], o.kg[t][ms], Vb[ms]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ms = 0; ms < NMS; ++ms) xv[ms * 64 + l] = Vb[ms];
            if constexpr (has_next) {
                read_k(o, k + 1);
                __builtin_amdgcn_sched_barrier(0);
                asm volatile("" ::: "memory");
                wait_lgkmcnt<(NT * NMS < 15 ? NT * NMS : 15)>();  // hand-over writes done
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            } else {
                __syncthreads();
            }
        };
        for (int k = 0; k + 1 < nsteps; ++k) step(k, std::true_type{});
        if (nsteps > 0) step(nsteps - 1, std::false_type{});
        if (p.output_final_state) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) p.ht[sbase + sidx(16 * t + 4 * cg + jj)] = S[t][jj];
        }
    } else if (!is_loader) {
        // ------------------------------------------------------------ output wave o
        if constexpr (HS) {
            if (p.skip_output) {
                // the backward's recompute needs the states, not the output: these waves
                // only take part in the barriers (the prologue's and one per step, as below)
                __syncthreads();
                for (int m = 0; m <= nsteps; ++m) __syncthreads();
                return;
            }
        }
        const int o = out_idx;
        const int mt0 = o;
        // this wave's rows of Qg [NKK] and of the non-zero Aqk blocks [NMS]
        struct QA {
            uint4 q[NKK];
            uint4 a[NMS];
        };
        auto load_qa = [&](QA &x, int k) {
            const size_t sl = slot_of(k);
            const uint4 *Qr = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.w_Qg) + sl * C * K);
            const uint4 *Ar = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.w_Aqk) + sl * C * C);
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) x.q[kk] = Qr[(mt0 * NKK + kk) * 64 + l];
#pragma unroll
            for (int ms = 0; ms < NMS; ++ms)
                if (32 * ms <= 16 * mt0 + 15) x.a[ms] = Ar[(mt0 * NMS + ms) * 64 + l];
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
            f32x4 acc[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                acc[j] = zero4();
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) acc[j] = mma32_bf16(acc[j], Sb[j][kk], x.q[kk]);
#pragma unroll
                for (int ms = 0; ms < NMS; ++ms)
                    if (32 * ms <= 16 * mt0 + 15) acc[j] = mma32_bf16(acc[j], Vb[j][ms], x.a[ms]);
            }
            // lane: row 16 mt0 + lr; element jj of tile j is column 4 cg + jj of state wave j,
            // i.e. slice column 8 cg + 4 j + jj: eight consecutive columns, one 16-byte store
            const int64_t tok0 = sb + (int64_t)k * C;
            const int m = 16 * mt0 + lr;
            if (tok0 + m < se)
                store16_once(static_cast<uint16_t *>(p.o) + ((tok0 + m) * p.HV + hv) * (int64_t)V + v0 + 8 * cg,
                             make_uint4(pack2(acc[0][0], acc[0][1]), pack2(acc[0][2], acc[0][3]),
                                        pack2(acc[1][0], acc[1][1]), pack2(acc[1][2], acc[1][3])));
        };
        // Barrier m, then the output of step m - 1 and the loads of step m + 2 into the
        // buffer that output just released: three steps of Qg/Aqk in flight, so the loads'
        // latency (and that of the output stores queued ahead of them) is covered.
        QA qa[3];
        if (nsteps > 0) load_qa(qa[0], 0);
        if (nsteps > 1) load_qa(qa[1], 1);
        __syncthreads();  // the state waves' ring prologue (no hand-over yet)
        auto iter = [&](int m, QA &buf) {
            __syncthreads();
            if (m >= 1) out_step(buf, m - 1);
            if (m + 2 < nsteps) load_qa(buf, m + 2);
        };
        for (int m = 0; m <= nsteps; m += 3) {
            iter(m, qa[2]);
            if (m + 1 > nsteps) break;
            iter(m + 1, qa[0]);
            if (m + 2 > nsteps) break;
            iter(m + 2, qa[1]);
        }
    } else {
        // ------------------------------------------------------------ loader wave i
        // Iteration k (after barrier k) issues W/U and KgT/d of step k + 3, then waits until
        // only those are outstanding, so what iteration k - 1 issued (step k + 2) has landed
        // before barrier k + 1, one step before the state waves start reading it.  The
        // prologue issues steps 0..2 and waits for all but step 2; barrier 0 comes after the
        // state waves have read step 0's operands, since step 3 refills step 0's W/U slot.
        const int i = wid - 4;
        auto issue_w = [&](int k) {
            if (k >= nsteps) return;
            if (i == 0) ring_issue_w<C, K, 0>(p, ring, slot_of(k), k, v0, l);
            else ring_issue_w<C, K, 1>(p, ring, slot_of(k), k, v0, l);
        };
        auto issue_k = [&](int k) {
            if (k >= nsteps) return;
            if (i == 0) ring_issue_k<C, K, 0>(p, ring, slot_of(k), k, l);
            else ring_issue_k<C, K, 1>(p, ring, slot_of(k), k, l);
        };
        // wait until at most the ring loads of step kr (if issued) are outstanding
        auto wait_all_but = [&](int kr) {
            if (kr < nsteps) {
                if (i == 0) wait_vmcnt<R::nload_w(0) + R::nload_k(0)>();
                else wait_vmcnt<R::nload_w(1) + R::nload_k(1)>();
            } else {
                wait_vmcnt<0>();
            }
        };
        for (int k = 0; k < 3; ++k) {
            issue_w(k);
            issue_k(k);
        }
        wait_all_but(2);
        __builtin_amdgcn_s_barrier();  // steps 0 and 1 landed; the state waves now read step 0
        for (int k = 0; k <= nsteps; ++k) {
            __builtin_amdgcn_s_barrier();  // k = 0: step 0's operands are in registers
            issue_w(k + 3);
            issue_k(k + 3);
            wait_all_but(k + 3);
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
    const bool hs = p.hs != nullptr;
    switch (p.K / 32) {
    case 1: go(hs ? recur_reg_kernel<C, 1, true> : recur_reg_kernel<C, 1, false>, RegRecur<C, 32>::kBytes); break;
    case 2: go(hs ? recur_reg_kernel<C, 2, true> : recur_reg_kernel<C, 2, false>, RegRecur<C, 64>::kBytes); break;
    case 3: go(hs ? recur_reg_kernel<C, 3, true> : recur_reg_kernel<C, 3, false>, RegRecur<C, 96>::kBytes); break;
    case 4: go(hs ? recur_reg_kernel<C, 4, true> : recur_reg_kernel<C, 4, false>, RegRecur<C, 128>::kBytes); break;
    default: return hipErrorInvalidValue;
    }
    return e;
}

}  // namespace kda
