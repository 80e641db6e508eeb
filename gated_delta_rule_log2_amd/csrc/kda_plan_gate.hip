// kda_plan_gate.hip -- chunk plan and the standalone gate + chunk-local cumsum kernel.
//
// Plan: sequences are the batch rows, or the packed segments given by cu_seqlens
// ("flash-linear-attention KDA 内核工程实践…", §2.2: varlen flattens the batch to 1
// and passes the segment offsets).  Chunks restart at every sequence start, so
// sequence n owns ceil(len_n / C) consecutive global chunks.
#include "kda_gate.h"

namespace kda {

constexpr int kMaxRankedSeqs = 4096;

// One workgroup of 256 threads: exclusive scan of per-sequence chunk counts into
// chunk_off[0..N], the inverse map chunk_seq[gc] = n by binary search, and the
// recurrence's issue order seq_order.  Only packed (cu_seqlens) batches need it;
// fixed-length batches compute the tables inline and keep the batch order.
__global__ void __launch_bounds__(256) plan_kernel(Params p) {
    __shared__ int warp_tot[4];
    __shared__ int carry_s;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int base = 0; base < p.N; base += 256) {
        const int n = base + tid;
        int cnt = 0;
        if (n < p.N) {
            const int64_t len = p.cu_seqlens ? (p.cu_seqlens[n + 1] - p.cu_seqlens[n]) : (int64_t)p.T;
            cnt = (int)((len + p.C - 1) / p.C);
        }
        // inclusive wave scan
        int x = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        if (lane == 63) warp_tot[w] = x;
        __syncthreads();
        int pre = carry_s;
        for (int i = 0; i < w; ++i) pre += warp_tot[i];
        if (n < p.N) p.chunk_off[n] = pre + x - cnt;
        __syncthreads();
        if (tid == 255) carry_s = pre + x;
        __syncthreads();
    }
    if (tid == 0) p.chunk_off[p.N] = carry_s;
    __syncthreads();
    const int total = carry_s;
    for (int gc = tid; gc < total; gc += 256) {
        int lo = 0, hi = p.N - 1;  // last n with chunk_off[n] <= gc (empty sequences skipped)
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.chunk_off[mid] <= gc) lo = mid;
            else hi = mid - 1;
        }
        p.chunk_seq[gc] = lo;
    }
    // Issue order of the recurrence: sequences by decreasing length (ties by index), so
    // the longest chains start first and the short ones fill in behind them.  The rank
    // of n is the number of sequences that go before it; O(N^2 / 256), so above
    // kMaxRankedSeqs sequences the order stays the packing order.
    for (int n = tid; n < p.N; n += 256) {
        int rank = n;
        if (p.N <= kMaxRankedSeqs) {
            const int64_t ln = p.cu_seqlens[n + 1] - p.cu_seqlens[n];
            rank = 0;
            for (int m = 0; m < p.N; ++m) {
                const int64_t lm = p.cu_seqlens[m + 1] - p.cu_seqlens[m];
                rank += (lm > ln || (lm == ln && m < n)) ? 1 : 0;
            }
        }
        p.seq_order[rank] = n;
    }
}

// Gate-only entry: one workgroup per (global chunk, value head); C/16 waves, one
// 16-row block each.  Writes the natural-log activated gate (optional) and the
// base-2 chunk-local cumsum, for valid rows only.
template <int NKK>
__global__ void __launch_bounds__(256) gate_cumsum_kernel(Params p) {
    extern __shared__ float tot[];  // [C/16][K]
    const int hv = blockIdx.x % p.HV;
    const int gc = blockIdx.x / p.HV;
    const ChunkInfo ci = chunk_info(p, gc);
    const int blk = threadIdx.x >> 6;
    const int nkk = p.K / 32;
    float G[NKK][8], ga[NKK][8];
    gate_cumsum_block<NKK>(p, ci, hv, blk, nkk, G, tot, ga);
    const int l = lane_id();
    const int r = 16 * blk + (l & 15);
    if (r >= ci.L) return;
    const int64_t row = ((ci.tok0 + r) * p.HV + hv) * (int64_t)p.K;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
        if (kk < nkk) {
            const int d0 = 32 * kk + 8 * (l >> 4);
            store8(p.g_cum + row + d0, G[kk]);
            if (p.g_act) store8(p.g_act + row + d0, ga[kk]);
        }
}

hipError_t launch_plan(const Params &p, hipStream_t s) {
    if (!p.cu_seqlens) return hipSuccess;  // fixed-length batches need no tables
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_gate_cumsum(const Params &p, hipStream_t s) {
    if (p.total_chunks == 0) return hipSuccess;
    const dim3 grid((unsigned)p.total_chunks * (unsigned)p.HV);
    const dim3 block(64 * (p.C / 16));
    const size_t lds = sizeof(float) * (p.C / 16) * p.K;
    if (p.K <= 128) hipLaunchKernelGGL(gate_cumsum_kernel<4>, grid, block, lds, s, p);
    else hipLaunchKernelGGL(gate_cumsum_kernel<8>, grid, block, lds, s, p);
    return hipGetLastError();
}

}  // namespace kda
