// kda_bwd_dhu.h -- the reverse chunk recurrence of the KDA backward ("Reading Notes:
// Implementation Notes for KDA in FLA", backward step 4), for K <= 128.
//
// Per (sequence, value head, 32-column slice of V), chunks last to first, with dS the
// gradient of the state after the chunk (dht for the sequence's last chunk, else 0):
//   dU  = Aqk^T dO + Kg dS                  (C x 32)   the gradient of V_new = U - W S_prev
//   dS <- Diag(d) dS + Qg^T dO - W^T dU      (K x 32)   the gradient of S_prev
// with Aqk, Kg = (KgT)^T, Qg, W and d = 2^G_last the forward's per-chunk intermediates
// (backward steps 1-2 recompute them with the forward's own kernels).  dU and the dS
// each chunk is entered with go to the workspace for the per-chunk gradient kernel; the
// final dS is the initial-state gradient dh0.
//
// One workgroup of 4 waves.  Each step stages the chunk's four intermediates from their
// fragment-major layouts into LDS as fp32, transposed where a product needs it, then
// forms the two products on the matrix cores (bf16 operands with fp32 accumulation
// for bf16 intermediates, fp32 otherwise); dS stays in registers (fp32) between steps.
#pragma once

#include "kda_backward.h"
#include "kda_intra.h"

namespace kda {

// 4 x 4 transpose inside each quad of lanes (lanes 4a .. 4a + 3): lane 4a + q returns, as
// its element i, element q of lane 4a + i.  Two exchange rounds (partner lane q ^ 1, then
// q ^ 2), each moving the two elements whose index bit differs from the lane's bit.  The
// recurrences hand over four consecutive rows of one column per lane, and the four lanes
// of a quad hold four consecutive columns; after the transpose each lane holds four
// consecutive columns of one row, so a [row][column] plane takes one 8-byte store per lane
// and plane instead of four 2-byte ones.
__device__ __forceinline__ float4 quad_transpose(float4 x) {
    const int q = lane_id() & 3;
    const bool q0 = (q & 1) != 0, q1 = (q & 2) != 0;
    auto xor1 = [](float v) {  // quad_perm [1, 0, 3, 2]
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xf, 0xf, false));
    };
    auto xor2 = [](float v) {  // quad_perm [2, 3, 0, 1]
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xf, 0xf, false));
    };
    const float r0 = xor1(q0 ? x.x : x.y), r1 = xor1(q0 ? x.z : x.w);
    const float t0 = q0 ? r0 : x.x, t1 = q0 ? x.y : r0, t2 = q0 ? r1 : x.z, t3 = q0 ? x.w : r1;
    const float v0 = xor2(q1 ? t0 : t2), v1 = xor2(q1 ? t1 : t3);
    return make_float4(q1 ? v0 : t0, q1 ? v1 : t1, q1 ? t2 : v0, q1 ? t3 : v1);
}


template <int C, int K>
struct DhuLds {
    static constexpr int VS = 32, LDC = C + 4, LDK = K + 4;
    static constexpr size_t kX1 = 0;                                 // [C][LDC]  Aqk[j][i] at [i][j]
    static constexpr size_t kKG = kX1 + (size_t)C * LDC;              // [C][LDK]  Kg[i][d]
    static constexpr size_t kQGT = kKG + (size_t)C * LDK;             // [K][LDC]  Qg[i][d] at [d][i]
    static constexpr size_t kWT = kQGT + (size_t)K * LDC;             // [K][LDC]  W[i][d] at [d][i]
    static constexpr size_t kDOT = kWT + (size_t)K * LDC;             // [VS][LDC] dO[i][v] at [v][i]
    static constexpr size_t kDUT = kDOT + (size_t)VS * LDC;           // [VS][LDC] dU[i][v] at [v][i]
    static constexpr size_t kDST = kDUT + (size_t)VS * LDC;           // [VS][LDK] dS[d][v] at [v][d]
    static constexpr size_t kDD = kDST + (size_t)VS * LDK;            // [K] chunk decay
    static constexpr size_t floats = kDD + K;
    static constexpr size_t bytes = floats * 4;
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

// Element (row, e-th of the 8) of unit u of a [R][NC] fragment-major matrix: the unit's
// row and the columns its 8 elements hold (permuted row fragments for bf16, plain row
// fragments for fp32; see frag_off / pfrag_off).
template <bool PERM>
__device__ __forceinline__ void unit_coords(int u, int NC, int &row, int (&col)[8]) {
    const int rbcb = u >> 6, lane = u & 63;
    const int rb = rbcb / (NC >> 5), cb = rbcb % (NC >> 5);
    const int g = lane >> 4;
    row = 16 * rb + (lane & 15);
#pragma unroll
    for (int e = 0; e < 8; ++e)
        col[e] = 32 * cb + (PERM ? (e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4)) : 8 * g + e);
}

// Loads unit u (8 elements) of a fragment-major matrix stored as T.
template <typename T>
__device__ __forceinline__ void unit_load(const T *base, int u, float (&x)[8]) {
    load8(base + (size_t)u * 8, x);
}

// Stages a fragment-major [R][NC] matrix into LDS: element (row, col) to
// dst[col * ld + row] (transposed) or dst[row * ld + col].  CAUSAL: a lower-triangular
// square matrix whose 32-column units right of the 16-row block's diagonal are zero and
// may not have been written (the bf16 forward skips them), so they are staged as zeros.
template <typename T, bool PERM, bool TRANS, bool CAUSAL = false>
__device__ __forceinline__ void stage_frag(const T *src, int R, int NC, float *dst, int ld) {
    const int nu = R * NC / 8;
    for (int u = threadIdx.x; u < nu; u += blockDim.x) {
        float x[8];
        int row, col[8];
        unit_coords<PERM>(u, NC, row, col);
        if (CAUSAL && col[0] - col[0] % 32 > (row | 15)) {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = 0.f;
        } else {
            unit_load<T>(src, u, x);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (TRANS) dst[col[e] * ld + row] = x[e];
            else dst[row * ld + col[e]] = x[e];
        }
    }
}

template <int C, typename T, int NKK>
__global__ void __launch_bounds__(256) bwd_dhu_kernel(BwdChunkParams P) {
    constexpr bool F32 = sizeof(T) == 4;
    constexpr bool PERM = !F32;  // bf16 intermediates with K <= 128 are permuted row fragments
    constexpr int K = 32 * NKK, NB = C / 16;
    using L_ = DhuLds<C, K>;
    constexpr int VS = L_::VS, LDC = L_::LDC, LDK = L_::LDK;
    constexpr int NDU = (2 * NB + 3) / 4;  // dU tiles per wave
    constexpr int NDS = NKK;               // dS tiles per wave ((K/16) * 2 over 4 waves)
    const Params &p = P.f;
    const BwdParams &b = P.b;
    extern __shared__ __align__(16) float sm[];
    float *X1 = sm + L_::kX1, *KG = sm + L_::kKG, *QGT = sm + L_::kQGT, *WT = sm + L_::kWT;
    float *DOT = sm + L_::kDOT, *DUT = sm + L_::kDUT, *DST = sm + L_::kDST, *DD = sm + L_::kDD;

    const int V = p.V, nvs = V / VS;
    const int unit = blockIdx.x / nvs;
    if (unit >= p.N * p.HV) return;
    const int n = unit / p.HV, hv = unit % p.HV;
    const int v0 = VS * (blockIdx.x % nvs);
    const int tid = threadIdx.x, w = tid >> 6, l = lane_id(), lr = l & 15, cg = l >> 4;
    const int c0 = seq_chunk_begin(p, n), nsteps = seq_chunk_begin(p, n + 1) - c0;

    // dS tiles of this wave: tile ts = w + 4e covers rows 16 (ts >> 1).., columns 16 (ts & 1)..;
    // lane: rows 16db + 4cg + jj, column 16vb + lr
    f32x4 dS[NDS];
#pragma unroll
    for (int e = 0; e < NDS; ++e) {
        const int ts = w + 4 * e, db = ts >> 1, vb = ts & 1;
        dS[e] = zero4();
        if (b.dht) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                dS[e][jj] = b.dht[(((size_t)n * p.HV + hv) * K + 16 * db + 4 * cg + jj) * V + v0 + 16 * vb + lr];
        }
        *reinterpret_cast<float4 *>(DST + (16 * vb + lr) * LDK + 16 * db + 4 * cg) =
            make_float4(dS[e][0], dS[e][1], dS[e][2], dS[e][3]);
    }

    for (int k = nsteps - 1; k >= 0; --k) {
        const int gc = c0 + k;
        const ChunkInfo ci = chunk_info(p, gc);
        const size_t slot = (size_t)gc * p.HV + hv;
        // ---- stage the chunk's intermediates and dO slice (rows past the end as zeros) ----
        stage_frag<T, PERM, true, true>(static_cast<const T *>(p.w_Aqk) + slot * C * C, C, C, X1, LDC);
        stage_frag<T, PERM, true>(static_cast<const T *>(p.w_KgT) + slot * K * C, K, C, KG, LDK);
        stage_frag<T, PERM, true>(static_cast<const T *>(p.w_Qg) + slot * C * K, C, K, QGT, LDC);
        stage_frag<T, PERM, true>(static_cast<const T *>(p.w_W) + slot * C * K, C, K, WT, LDC);
        for (int e = tid; e < K; e += blockDim.x) DD[e] = p.w_d[slot * K + e];
        for (int e = tid; e < C * VS / 8; e += blockDim.x) {
            const int i = e / (VS / 8), v8 = 8 * (e % (VS / 8));
            float x[8];
            if (i < ci.L) {
                if (b.qkv_bf16) load8(static_cast<const uint16_t *>(b.dout) + ((ci.tok0 + i) * p.HV + hv) * (int64_t)V + v0 + v8, x);
                else load8(static_cast<const float *>(b.dout) + ((ci.tok0 + i) * p.HV + hv) * (int64_t)V + v0 + v8, x);
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) x[q] = 0.f;
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) DOT[(v8 + q) * LDC + i] = x[q];
        }
        __syncthreads();

        // ---- dU = Aqk^T dO + Kg dS (lane: rows 16ib + 4cg + jj, column 16vb + lr) ----
#pragma unroll
        for (int e = 0; e < NDU; ++e) {
            const int tu = w + 4 * e;
            if (tu < 2 * NB) {
                const int ib = tu >> 1, vb = tu & 1;
                f32x4 acc = zero4();
#pragma unroll
                for (int jm = 0; jm < C / 32; ++jm) {
                    float a[8], bb[8];
                    load8(X1 + (16 * ib + lr) * LDC + 32 * jm + 8 * cg, a);
                    load8(DOT + (16 * vb + lr) * LDC + 32 * jm + 8 * cg, bb);
                    acc = mma32<F32>(acc, a, bb);
                }
#pragma unroll
                for (int dm = 0; dm < K / 32; ++dm) {
                    float a[8], bb[8];
                    load8(KG + (16 * ib + lr) * LDK + 32 * dm + 8 * cg, a);
                    load8(DST + (16 * vb + lr) * LDK + 32 * dm + 8 * cg, bb);
                    acc = mma32<F32>(acc, a, bb);
                }
                *reinterpret_cast<float4 *>(DUT + (16 * vb + lr) * LDC + 16 * ib + 4 * cg) =
                    make_float4(acc[0], acc[1], acc[2], acc[3]);
                float *gdu = P.dU + (slot * C + 16 * ib + 4 * cg) * (size_t)V + v0 + 16 * vb + lr;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) gdu[(size_t)jj * V] = acc[jj];
            }
        }
        // the state gradient this chunk is entered with (after the chunk's update)
#pragma unroll
        for (int e = 0; e < NDS; ++e) {
            const int ts = w + 4 * e, db = ts >> 1, vb = ts & 1;
            float *gdh = P.dh + (slot * K + 16 * db + 4 * cg) * (size_t)V + v0 + 16 * vb + lr;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) gdh[(size_t)jj * V] = dS[e][jj];
        }
        __syncthreads();  // dU^T complete

        // ---- dS <- Diag(d) dS + Qg^T dO - W^T dU (lane: rows 16db + 4cg + jj, column 16vb + lr) ----
#pragma unroll
        for (int e = 0; e < NDS; ++e) {
            const int ts = w + 4 * e, db = ts >> 1, vb = ts & 1;
            f32x4 acc, accw = zero4();
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) acc[jj] = DD[16 * db + 4 * cg + jj] * dS[e][jj];
#pragma unroll
            for (int im = 0; im < C / 32; ++im) {
                float a[8], bb[8], a2[8], b2[8];
                load8(QGT + (16 * db + lr) * LDC + 32 * im + 8 * cg, a);
                load8(DOT + (16 * vb + lr) * LDC + 32 * im + 8 * cg, bb);
                load8(WT + (16 * db + lr) * LDC + 32 * im + 8 * cg, a2);
                load8(DUT + (16 * vb + lr) * LDC + 32 * im + 8 * cg, b2);
                acc = mma32<F32>(acc, a, bb);
                accw = mma32<F32>(accw, a2, b2);
            }
            dS[e] = acc - accw;
        }
        __syncthreads();  // every read of this step's staging is done
#pragma unroll
        for (int e = 0; e < NDS; ++e) {
            const int ts = w + 4 * e, db = ts >> 1, vb = ts & 1;
            *reinterpret_cast<float4 *>(DST + (16 * vb + lr) * LDK + 16 * db + 4 * cg) =
                make_float4(dS[e][0], dS[e][1], dS[e][2], dS[e][3]);
        }
    }
    if (b.dh0) {
#pragma unroll
        for (int e = 0; e < NDS; ++e) {
            const int ts = w + 4 * e, db = ts >> 1, vb = ts & 1;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                b.dh0[(((size_t)n * p.HV + hv) * K + 16 * db + 4 * cg + jj) * V + v0 + 16 * vb + lr] = dS[e][jj];
        }
    }
}

}  // namespace kda
