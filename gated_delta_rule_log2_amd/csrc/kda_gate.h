// kda_gate.h -- chunk geometry and the fused gate activation + base-2 chunk-local
// cumulative sum, evaluated by one wave on a 16-row block of a chunk.
//
// Method ("flash-linear-attention KDA 内核工程实践…", §2: the pre-gated and in-kernel
// gate contracts; "Reading Notes: Implementation Notes for KDA in FLA", forward
// step 1: the chunk-local cumulative log decay; "FlashKDA gate偏置加載路徑完整解析",
// §二 第2段 / §三: bias, then exp(A_log), then the scaled sigmoid, with log2(e)
// folded in so that the later decay factors are exp2 of differences).
#pragma once

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

struct ChunkInfo {
    int64_t tok0;  // first token of the chunk on the flattened [B*T] token axis
    int L;         // valid rows (1..C)
    int seq;       // sequence index
};

__device__ __forceinline__ int64_t seq_begin(const Params &p, int n) {
    return p.cu_seqlens ? p.cu_seqlens[n] : (int64_t)n * p.T;
}

// Global chunk gc -> its sequence, first token and length.  Chunks start at every
// sequence start and then every C tokens, so a chunk never straddles sequences.
__device__ __forceinline__ ChunkInfo chunk_info(const Params &p, int gc) {
    const int n = p.chunk_seq[gc];
    const int c = gc - p.chunk_off[n];
    const int64_t s0 = seq_begin(p, n);
    const int64_t s1 = p.cu_seqlens ? p.cu_seqlens[n + 1] : s0 + p.T;
    const int64_t tok0 = s0 + (int64_t)c * p.C;
    const int64_t rem = s1 - tok0;
    return ChunkInfo{tok0, (int)(rem < p.C ? rem : p.C), n};
}

// Activated gate in natural-log units for one element.  a = exp(A_log[hv]) (or 1
// when A_log is absent with a lower bound), dtb = dt_bias[hv*K + d] (or 0).
__device__ __forceinline__ float gate_natural(int mode, float graw, float dtb, float a, float lb) {
    if (mode == kGatePre) return graw;
    const float x = graw + dtb;
    if (mode == kGateSoftplus) {
        // softplus(x) = log(1 + e^x); above 20 it equals x to within e^-20 relative
        const float sp = x > 20.f ? x : log1pf(expf(x));
        return -a * sp;
    }
    const float z = a * x;
    return lb * (1.f / (1.f + expf(-z)));  // lb * sigmoid(z); 0 once e^-z overflows
}

__device__ __forceinline__ float beta_act(int mode, float b) {
    if (mode == kBetaGiven) return b;
    const float s = 1.f / (1.f + expf(-b));
    return mode == kBetaTwoSigmoid ? 2.f * s : s;
}

__device__ __forceinline__ float load_any(const void *p, int64_t idx, int is_bf16) {
    return is_bf16 ? bf2f(static_cast<const uint16_t *>(p)[idx]) : static_cast<const float *>(p)[idx];
}

// 8 contiguous gate inputs of one row (fp32 or bf16 storage, chosen at run time).
__device__ __forceinline__ void load8_any(const void *base, int64_t idx, int is_bf16, float (&o)[8]) {
    if (is_bf16) load8(static_cast<const uint16_t *>(base) + idx, o);
    else load8(static_cast<const float *>(base) + idx, o);
}

// One wave computes, for the 16-row block `blk` of a chunk, the activated gate
// and its inclusive cumulative sum in log2 units, in row-fragment layout:
//   G[kk][i] = log2(e) * sum_{r' <= r} g'[r'][32*kk + 8*(l>>4) + i],  r = 16*blk + (l & 15)
// Rows at or past the chunk's length contribute g' = 0, so they repeat the last
// valid row's value.  Sums of earlier blocks arrive through `tot` ([nblk][K] fp32
// in LDS), which the caller must clear-free: every block writes its own totals
// before the __syncthreads() this function executes, and reads earlier ones after.
// If `gact` is non-null the natural-log activated gate is stored there too.
// All waves of the block must call this (it contains one __syncthreads()).
template <int NKK>
__device__ __forceinline__ void gate_cumsum_block(const Params &p, const ChunkInfo &ci, int hv, int blk,
                                                  int nkk, float (&G)[NKK][8], float *tot,
                                                  float (&gact)[NKK][8]) {
    const int l = lane_id();
    const int r = 16 * blk + (l & 15);
    const int cg = l >> 4;
    const bool valid = r < ci.L;
    const int K = p.K;
    const float a = (p.gate_mode == kGatePre) ? 1.f : (p.A_log ? expf(p.A_log[hv]) : 1.f);
    const float lb = p.lower_bound_log2 / kLog2e;
    const int64_t row = ((ci.tok0 + r) * p.HV + hv) * (int64_t)K;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if (kk < nkk) {
            const int d0 = 32 * kk + 8 * cg;
            float x[8];
            if (valid) load8_any(p.g, row + d0, p.g_bf16, x);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float dtb = (p.dt_bias && p.gate_mode != kGatePre) ? p.dt_bias[(int64_t)hv * K + d0 + i] : 0.f;
                const float gn = valid ? gate_natural(p.gate_mode, x[i], dtb, a, lb) : 0.f;
                gact[kk][i] = gn;
                G[kk][i] = row_scan16(gn * kLog2e);
            }
        }
    }
    // block totals (row 15 of this block) -> LDS
    if ((l & 15) == 15) {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
            if (kk < nkk) {
#pragma unroll
                for (int i = 0; i < 8; ++i) tot[blk * K + 32 * kk + 8 * cg + i] = G[kk][i];
            }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
        if (kk < nkk) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float pre = 0.f;
                for (int b = 0; b < blk; ++b) pre += tot[b * K + 32 * kk + 8 * cg + i];
                G[kk][i] += pre;
            }
        }
}

}  // namespace kda
