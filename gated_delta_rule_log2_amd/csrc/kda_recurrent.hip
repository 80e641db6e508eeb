// kda_recurrent.hip -- token-by-token KDA forward (the fused recurrent entry for
// autoregressive decoding: "flash-linear-attention KDA 内核工程实践…", §1, the
// second public entry next to chunk_kda).
//
// Per token t of a sequence, with the state S stored [K][V] (key rows):
//   S <- Diag(alpha_t) S,   alpha_t = exp(g'_t)  (the activated gate of chunk_kda)
//   u  = S^T k^_t,   S <- S + beta_t k^_t (v_t - u)^T,   o_t = S^T q^_t
// i.e. S_t = (I - beta_t k^_t k^_t^T) Diag(alpha_t) S_{t-1} + beta_t k^_t v_t^T, the
// recurrence the chunk form reorganises ("Reading Notes: Implementation Notes for KDA
// in FLA", forward; q^, k^ optionally L2-normalised, q^ scaled).
//
// One workgroup of 256 threads per (sequence, value head, 32-column slice of V); the
// slice of S stays in registers for the whole sequence: thread (row group rg, column
// c) holds rows rg*K/8 .. rg*K/8 + K/8 - 1 of column c.  Each token's q, k, gate
// (one channel per thread), v slice and beta are loaded one token ahead into
// registers, staged in LDS, and the two column reductions (u and o) go through LDS:
// three barriers per token.
#include "kda_gate.h"

namespace kda {

namespace {

constexpr int kRecCols = 32;      // V columns per workgroup
constexpr int kRecThreads = 256;  // 8 row groups x 32 columns

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += shfl_xor(x, m);
    return x;
}

template <int NKK>
__global__ void __launch_bounds__(kRecThreads) fused_recurrent_kernel(Params p) {
    constexpr int K = 32 * NKK, RPT = K / 8;  // state rows per thread
    __shared__ float qs[K], ks[K], als[K];
    __shared__ float vsl[kRecCols];
    __shared__ float red[2][8][kRecCols + 1];
    __shared__ float nrm[2][4];
    __shared__ float bsh;

    const int V = p.V, nvt = V / kRecCols;
    const int unit = blockIdx.x / nvt, v0 = kRecCols * (int)(blockIdx.x % nvt);
    const int n = unit / p.HV, hv = unit % p.HV, h = hv / p.group;
    const int tid = threadIdx.x, c = tid & (kRecCols - 1), rg = tid >> 5, wid = tid >> 6;
    const int d0 = rg * RPT;
    const int64_t s0 = seq_begin(p, n);
    const int64_t s1 = p.cu_seqlens ? p.cu_seqlens[n + 1] : s0 + p.T;

    float S[RPT];
    // element (key row d, value column v0 + c) of this unit's state, [K][V] or [V][K]
    const size_t sbase = ((size_t)n * p.HV + hv) * K * V;
    auto sidx = [&](int d) { return sbase + (p.state_vk ? (size_t)(v0 + c) * K + d : (size_t)d * V + v0 + c); };
#pragma unroll
    for (int i = 0; i < RPT; ++i) S[i] = p.h0 ? p.h0[sidx(d0 + i)] : 0.f;

    const float a = p.A_log ? expf(p.A_log[hv]) : 1.f;
    const float lb = p.lower_bound;  // natural-log lower bound
    const float dtb = (p.dt_bias && tid < K) ? p.dt_bias[(int64_t)hv * K + tid] : 0.f;

    // raw inputs of one token: channel tid of q, k and the gate; column tid of the v slice;
    // beta on thread 0
    float qr = 0.f, kr = 0.f, gr = 0.f, vr = 0.f, br = 0.f;
    auto load_token = [&](int64_t t) {
        if (tid < K) {
            qr = load_any(p.q, (t * p.H + h) * K + tid, p.qkv_bf16);
            kr = load_any(p.k, (t * p.H + h) * K + tid, p.qkv_bf16);
            gr = load_any(p.g, (t * p.HV + hv) * K + tid, p.g_bf16);
        }
        if (tid < kRecCols) vr = load_any(p.v, (t * p.HV + hv) * (int64_t)V + v0 + tid, p.qkv_bf16);
        if (tid == 0) br = load_any(p.beta, t * p.HV + hv, p.beta_bf16);
    };
    if (s0 < s1) load_token(s0);

    for (int64_t t = s0; t < s1; ++t) {
        // stage token t: decay factor per channel, squared norms per wave
        float q2 = 0.f, k2 = 0.f;
        if (tid < K) {
            qs[tid] = qr;
            ks[tid] = kr;
            als[tid] = __builtin_amdgcn_exp2f(gate_act(p.gate_mode, gr, dtb, a, lb, kLog2e));
            q2 = qr * qr;
            k2 = kr * kr;
        }
        if (tid < kRecCols) vsl[tid] = vr;
        if (tid == 0) bsh = beta_act(p.beta_mode, br);
        if (p.qk_l2norm) {
            q2 = wave_sum(q2);
            k2 = wave_sum(k2);
            if ((tid & 63) == 0) {
                nrm[0][wid] = q2;
                nrm[1][wid] = k2;
            }
        }
        if (t + 1 < s1) load_token(t + 1);
        __syncthreads();

        float rq = p.scale, rk = 1.f;
        if (p.qk_l2norm) {
            rq *= rsqrtf(nrm[0][0] + nrm[0][1] + nrm[0][2] + nrm[0][3] + 1e-6f);
            rk = rsqrtf(nrm[1][0] + nrm[1][1] + nrm[1][2] + nrm[1][3] + 1e-6f);
        }
        // S <- Diag(alpha) S;  u = S^T k^ (this thread's rows)
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            S[i] *= als[d0 + i];
            part += (ks[d0 + i] * rk) * S[i];
        }
        red[0][rg][c] = part;
        __syncthreads();

        float uc = 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) uc += red[0][r][c];
        const float vnew = bsh * (vsl[c] - uc);
        // S <- S + beta k^ (v - u)^T;  o = S^T q^ (this thread's rows)
        float part2 = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            S[i] += (ks[d0 + i] * rk) * vnew;
            part2 += (qs[d0 + i] * rq) * S[i];
        }
        red[1][rg][c] = part2;
        __syncthreads();

        if (rg == 0) {
            float oc = 0.f;
#pragma unroll
            for (int r = 0; r < 8; ++r) oc += red[1][r][c];
            const int64_t oi = (t * p.HV + hv) * (int64_t)V + v0 + c;
            if (p.qkv_bf16) static_cast<uint16_t *>(p.o)[oi] = f2bf(oc);
            else static_cast<float *>(p.o)[oi] = oc;
        }
    }
    if (p.output_final_state) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) p.ht[sidx(d0 + i)] = S[i];
    }
}

}  // namespace

hipError_t launch_fused_recurrent(const Params &p, hipStream_t s) {
    const int64_t units = (int64_t)p.N * p.HV;
    if (units == 0) return hipSuccess;
    const dim3 grid((unsigned)(units * (p.V / kRecCols)));
    switch (p.K / 32) {
    case 1: hipLaunchKernelGGL(fused_recurrent_kernel<1>, grid, dim3(kRecThreads), 0, s, p); break;
    case 2: hipLaunchKernelGGL(fused_recurrent_kernel<2>, grid, dim3(kRecThreads), 0, s, p); break;
    case 3: hipLaunchKernelGGL(fused_recurrent_kernel<3>, grid, dim3(kRecThreads), 0, s, p); break;
    case 4: hipLaunchKernelGGL(fused_recurrent_kernel<4>, grid, dim3(kRecThreads), 0, s, p); break;
    case 5: hipLaunchKernelGGL(fused_recurrent_kernel<5>, grid, dim3(kRecThreads), 0, s, p); break;
    case 6: hipLaunchKernelGGL(fused_recurrent_kernel<6>, grid, dim3(kRecThreads), 0, s, p); break;
    case 7: hipLaunchKernelGGL(fused_recurrent_kernel<7>, grid, dim3(kRecThreads), 0, s, p); break;
    case 8: hipLaunchKernelGGL(fused_recurrent_kernel<8>, grid, dim3(kRecThreads), 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kda
