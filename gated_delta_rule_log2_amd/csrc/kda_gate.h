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

// Chunks start at every sequence start and then every C tokens, so a chunk never
// straddles sequences.  Without cu_seqlens every sequence has ceil(T / C) chunks and
// the chunk tables are plain arithmetic; with it they come from the plan kernel.
__device__ __forceinline__ int chunks_per_seq(const Params &p) { return (p.T + p.C - 1) / p.C; }
__device__ __forceinline__ int seq_chunk_begin(const Params &p, int n) {
    return p.cu_seqlens ? p.chunk_off[n] : n * chunks_per_seq(p);
}

// Global chunk gc -> its sequence, first token and length.
__device__ __forceinline__ ChunkInfo chunk_info(const Params &p, int gc) {
    int n, c;
    if (p.cu_seqlens) {
        n = p.chunk_seq[gc];
        c = gc - p.chunk_off[n];
    } else {
        const int nc = chunks_per_seq(p);
        n = gc / nc;
        c = gc - n * nc;
    }
    const int64_t s0 = seq_begin(p, n);
    const int64_t s1 = p.cu_seqlens ? p.cu_seqlens[n + 1] : s0 + p.T;
    const int64_t tok0 = s0 + (int64_t)c * p.C;
    const int64_t rem = s1 - tok0;
    return ChunkInfo{tok0, (int)(rem < p.C ? rem : p.C), n};
}

// Activated gate g' of one element times `unit`: 1 gives natural-log units, log2(e)
// the log2 units every chunk kernel scans (so each later decay factor is an exp2).
// a = exp(A_log[hv]) (1 when A_log is absent with a lower bound), dtb = dt_bias[hv*K + d]
// (0 when absent), lb = the natural-log lower bound.  Every kernel that activates the
// gate calls this one function: the gate entry, both intra kernels, the token-by-token
// kernel.
//   pre-gated:  g' = g
//   softplus:   g' = -a * softplus(g + dtb);  above 20 softplus(x) = x to e^-20 relative
//   bounded:    g' = lb * sigmoid(a (g + dtb)), the sigmoid taken as 1 / (1 + 2^(-a log2(e) x)),
//               which is 0 once the power overflows and never leaves [lb, 0]
__device__ __forceinline__ float gate_act(int mode, float graw, float dtb, float a, float lb, float unit) {
    if (mode == kGatePre) return graw * unit;
    const float x = graw + dtb;
    if (mode == kGateSoftplus) {
        const float sp = x > 20.f ? x : log1pf(expf(x));
        return -(a * unit) * sp;
    }
    return (lb * unit) * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-(a * kLog2e) * x));
}

// Chain rule of gate_act in natural-log units: from gp = dL/dg' returns dL/dg and sets
// da to the element's term of dL/dA_log (a = exp(A_log[hv]); 0 when pre-gated).
//   softplus:  dg'/dg = -a sigmoid(x),          dg'/dA_log = g' = -a softplus(x)
//   bounded:   dg'/dg = lb a s (1 - s), s = sigmoid(a x),   dg'/dA_log = lb a x s (1 - s)
__device__ __forceinline__ float gate_act_grad(int mode, float gp, float graw, float dtb, float a, float lb, float &da) {
    da = 0.f;
    if (mode == kGatePre) return gp;
    const float x = graw + dtb;
    if (mode == kGateSoftplus) {
        const float sp = x > 20.f ? x : log1pf(expf(x));
        da = gp * (-a * sp);
        return gp * (-a) / (1.f + expf(-x));
    }
    // s as gate_act evaluates it: 1 / (1 + 2^(-a log2(e) x)), 0 once the power overflows
    const float s = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-(a * kLog2e) * x));
    const float ds = lb * s * (1.f - s) * a;
    da = gp * ds * x;
    return gp * ds;
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
// and its inclusive cumulative sum inside the block, in log2 units, in row-fragment
// layout:  G[kk][i] = log2(e) * sum_{16*blk <= r' <= r} g'[r'][32*kk + 8*(l>>4) + i]
// with r = 16*blk + (l & 15).  Rows at or past the chunk's length contribute
// g' = 0, so they repeat the last valid row's value.  gact receives g' itself.
template <int NKK>
__device__ __forceinline__ void gate_scan_block(const Params &p, const ChunkInfo &ci, int hv, int blk, int nkk,
                                                float (&G)[NKK][8], float (&gact)[NKK][8]) {
    const int l = lane_id();
    const int r = 16 * blk + (l & 15);
    const int cg = l >> 4;
    const bool valid = r < ci.L;
    const int K = p.K;
    const int64_t row = ((ci.tok0 + r) * p.HV + hv) * (int64_t)K;
    // raw gate rows (one dtype branch for the whole block)
    if (valid) {
        if (p.g_bf16) {
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
                if (kk < nkk) load8(static_cast<const uint16_t *>(p.g) + row + 32 * kk + 8 * cg, G[kk]);
        } else {
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
                if (kk < nkk) load8(static_cast<const float *>(p.g) + row + 32 * kk + 8 * cg, G[kk]);
        }
    } else {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
            for (int i = 0; i < 8; ++i) G[kk][i] = 0.f;
    }
    const float a = p.A_log ? expf(p.A_log[hv]) : 1.f;
    const float lb = p.lower_bound;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if (kk < nkk) {
            float dtb[8];
            if (p.dt_bias && p.gate_mode != kGatePre) load8(p.dt_bias + (int64_t)hv * K + 32 * kk + 8 * cg, dtb);
            else {
#pragma unroll
                for (int i = 0; i < 8; ++i) dtb[i] = 0.f;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float x = G[kk][i];
                gact[kk][i] = valid ? gate_act(p.gate_mode, x, dtb[i], a, lb, 1.f) : 0.f;
                G[kk][i] = row_scan16(valid ? gate_act(p.gate_mode, x, dtb[i], a, lb, kLog2e) : 0.f);
            }
        }
    }
}

// Adds the totals of the earlier blocks (from `tot`, [nblk][K] fp32) to a block scan.
template <int NKK>
__device__ __forceinline__ void gate_add_prefix(const float *tot, int K, int blk, int nkk, float (&G)[NKK][8]) {
    const int cg = lane_id() >> 4;
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

// Full chunk-local cumsum for the block: block scan, block totals through `tot`
// (LDS [nblk][K] fp32), one __syncthreads() (every wave of the workgroup must
// call this), then the earlier blocks' totals added.
template <int NKK>
__device__ __forceinline__ void gate_cumsum_block(const Params &p, const ChunkInfo &ci, int hv, int blk,
                                                  int nkk, float (&G)[NKK][8], float *tot,
                                                  float (&gact)[NKK][8]) {
    const int l = lane_id();
    const int cg = l >> 4;
    const int K = p.K;
    gate_scan_block<NKK>(p, ci, hv, blk, nkk, G, gact);
    if ((l & 15) == 15) {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
            if (kk < nkk) {
#pragma unroll
                for (int i = 0; i < 8; ++i) tot[blk * K + 32 * kk + 8 * cg + i] = G[kk][i];
            }
    }
    __syncthreads();
    gate_add_prefix<NKK>(tot, K, blk, nkk, G);
}

}  // namespace kda
