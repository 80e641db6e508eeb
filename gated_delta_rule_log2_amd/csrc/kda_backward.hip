// kda_backward.hip -- gradients of the KDA forward ("Reading Notes: Implementation
// Notes for KDA in FLA", backward section): dq, dk, dv, dg, dbeta, dA_log, dt_bias and
// initial-state gradients of L = <do, o> + <dht, final_state>.
//
// A first, token-level form.  The forward runs first and keeps the state each chunk
// starts from (the same kernels as the forward entry, with intermediate states), and a
// parallel pre-pass forms every token's q^, k^, exp(g') and b.  Then one workgroup per
// (sequence, value head, 16-column slice of V) walks its chunks last to first: half of
// it recomputes the next chunk's token states from that chunk's start state while the
// other half takes the reverse token steps of the current chunk (per token, with
// P = Diag(alpha) S_prev, u = P^T k^, w = v - u, S = P + b k^ w^T):
//   dS += q^ do^T;   dq^ = S do;   c = dS^T k^;   e = b c;   dv = e;   db = w . c;
//   dk^ = b dS w - P e;   dP = dS - k^ e^T;   dg' = rowsum(dP o P);   dS <- Diag(alpha) dP
// The sums over V (dq^, dk^, dg', db) are written per slice and added by the finishing
// kernels in a fixed order, which then apply the chain rules of the L2 norm and scale,
// the gate activation and the beta transform (sums over a GVA group for q and k, over
// tokens for dA_log and dt_bias).  Everything is fp32.
#include <hip/hip_runtime.h>

#include "kda_backward.h"

namespace kda {

namespace {

constexpr int kBwdThreads = 256;  // the per-token and per-head kernels
constexpr int kRoleThreads = 512;  // per role of the sequential kernel: kRowGroups row groups x kSlice columns
constexpr int kSeqThreads = 2 * kRoleThreads;
constexpr int kSlice = 16;
constexpr int kRowGroups = kRoleThreads / kSlice;

__device__ __forceinline__ float ldf(const void *p, int64_t i, bool bf) {
    if (bf) return __uint_as_float((uint32_t)static_cast<const uint16_t *>(p)[i] << 16);
    return static_cast<const float *>(p)[i];
}

__device__ __forceinline__ float sigm(float x) { return 1.f / (1.f + expf(-x)); }

__device__ __forceinline__ float softplus_f(float x) { return x > 0.f ? x + log1pf(expf(-x)) : log1pf(expf(x)); }

// natural-log activated gate (the forward's three contracts); ea = exp(A_log[hv]) (1
// without A_log) and bias = dt_bias[hv][d] (0 without) are the per-head constants
__device__ __forceinline__ float gate_nat(const BwdParams &p, float ea, float bias, float graw) {
    if (p.gate_mode == kGatePre) return graw;
    const float x = graw + bias;
    if (p.gate_mode == kGateSoftplus) return -ea * softplus_f(x);
    return p.lower_bound * sigm(ea * x);
}

__device__ __forceinline__ float beta_val(const BwdParams &p, float b) {
    if (p.beta_mode == kBetaSigmoid) return sigm(b);
    if (p.beta_mode == kBetaTwoSigmoid) return 2.f * sigm(b);
    return b;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// sum over the 16 lanes of a DPP row, in every lane: quad_perm [1,0,3,2] and [2,3,0,1]
// add the quad, row_ror 4 and 8 the other quads (every lane of a row stays in its row)
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x124>(x);
    x += dpp<0x128>(x);
    return x;
}

// sum over the 32 lanes of a half wave (the 32 columns of one row group)
__device__ __forceinline__ float half_sum(float x) {
    x = row_sum16(x);
    return x + __shfl_xor(x, 16, 64);
}

__device__ __forceinline__ float wave_sum(float x) {
    x = half_sum(x);
    return x + __shfl_xor(x, 32, 64);
}

// Per (token, value head): q^ = scale q r_q, k^ = k r_k (r = (|x|^2 + 1e-6)^-1/2 with the
// L2 norm, else 1), alpha = exp(g'), b, into the workspace, so the sequential kernel
// reads them without reductions of its own.  Block of 256 threads, thread d < K.
__global__ void __launch_bounds__(kBwdThreads) bwd_token_prep_kernel(BwdParams p) {
    __shared__ float ws[4][2];
    const int64_t t = blockIdx.x / p.HV;
    const int hv = blockIdx.x % p.HV, h = hv / (p.HV / p.H), d = threadIdx.x;
    float qv = 0.f, kv = 0.f, gp = 0.f;
    if (d < p.K) {
        qv = ldf(p.q, (t * p.H + h) * p.K + d, p.qkv_bf16);
        kv = ldf(p.k, (t * p.H + h) * p.K + d, p.qkv_bf16);
        const float ea = p.A_log ? expf(p.A_log[hv]) : 1.f;
        const float bias = p.dt_bias ? p.dt_bias[(int64_t)hv * p.K + d] : 0.f;
        gp = gate_nat(p, ea, bias, ldf(p.g, (t * p.HV + hv) * p.K + d, p.g_bf16));
    }
    float rq = 1.f, rk = 1.f;
    if (p.qk_l2norm) {
        const float sq = wave_sum(qv * qv), sk = wave_sum(kv * kv);
        if ((d & 63) == 0) ws[d >> 6][0] = sq, ws[d >> 6][1] = sk;
        __syncthreads();
        float tq = 0.f, tk = 0.f;
        for (int i = 0; i < kBwdThreads / 64; ++i) tq += ws[i][0], tk += ws[i][1];
        rq = 1.f / sqrtf(tq + 1e-6f);
        rk = 1.f / sqrtf(tk + 1e-6f);
    }
    const size_t o = ((size_t)t * p.HV + hv) * p.K + d;
    if (d < p.K) {
        p.t_q[o] = qv * rq * p.scale;
        p.t_k[o] = kv * rk;
        p.t_a[o] = expf(gp);
    }
    if (d == 0) p.t_b[t * p.HV + hv] = beta_val(p, ldf(p.beta, t * p.HV + hv, p.beta_bf16));
}

// Two roles of 512 threads each, run side by side: role 1 recomputes the token states
// of chunk c - 1 (from its chunk-start state, into scratch buffer (c - 1) & 1) while
// role 0 takes the reverse steps of chunk c (from buffer c & 1).  Phase ph handles
// recompute chunk ph - 1 and reverse chunk ph; both roles run max(lengths) steps with
// one workgroup barrier per step, outside any role-dependent branch, and one barrier
// between phases, so the barrier counts of the two roles always match.
template <int NR>
__global__ void __launch_bounds__(kSeqThreads) bwd_seq_kernel(BwdParams p) {
    const int ns = p.V / kSlice;
    const int slice = blockIdx.x % ns;
    const int hv = (blockIdx.x / ns) % p.HV;
    const int n = blockIdx.x / (ns * p.HV);
    const int tid = threadIdx.x;
    const int role = tid / kRoleThreads;  // 0: reverse steps, 1: recompute (wave-uniform)
    const int lt = tid % kRoleThreads, j = lt & (kSlice - 1), rg = lt / kSlice;
    const int col = slice * kSlice + j;
    const int K = p.K, V = p.V, C = p.C;
    // rows of this thread: rg + kRowGroups i
    int64_t t_begin, t_end, first_chunk = 0;
    if (p.cu_seqlens) {
        t_begin = p.cu_seqlens[n];
        t_end = p.cu_seqlens[n + 1];
        for (int m = 0; m < n; ++m) first_chunk += (p.cu_seqlens[m + 1] - p.cu_seqlens[m] + C - 1) / C;
    } else {
        t_begin = (int64_t)n * p.T;
        t_end = t_begin + p.T;
        first_chunk = (int64_t)n * ((p.T + C - 1) / C);
    }
    const int64_t len = t_end - t_begin;
    const int nchunks = (int)((len + C - 1) / C);
    auto chunk_len = [&](int c) -> int {
        if (c < 0 || c >= nchunks) return 0;
        const int64_t t0 = t_begin + (int64_t)c * C;
        return (int)((t0 + C < t_end ? t0 + C : t_end) - t0);
    };
    // two scratch buffers: S after each token of a chunk, and each token's w
    auto sc = [&](int buf) { return p.scr_state + ((size_t)blockIdx.x * 2 + buf) * C * K * kSlice; };
    auto sw = [&](int buf) { return p.scr_w + ((size_t)blockIdx.x * 2 + buf) * C * kSlice; };

    // per-wave column sums: [role][parity][wave of the role][column]
    __shared__ float red[2][2][kRoleThreads / 64][kSlice];
    // one token's per-row operands (rows rg + kRowGroups i) and this thread's column input
    struct Rows {
        float q[NR], k[NR], a[NR];
        float b;
        uint32_t col;  // raw bits of the column input (widened at its use, so the load can stay in flight)
    };
    auto colval = [&](uint32_t raw) { return __uint_as_float(p.qkv_bf16 ? raw << 16 : raw); };
    auto load_rows = [&](int64_t t, const void *colsrc, Rows &x) {
        const size_t base = ((size_t)t * p.HV + hv) * K;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int r = rg + kRowGroups * i;
            x.q[i] = p.t_q[base + r];
            x.k[i] = p.t_k[base + r];
            x.a[i] = p.t_a[base + r];
        }
        x.b = p.t_b[t * p.HV + hv];
        const int64_t ci = (t * p.HV + hv) * V + col;
        if (p.qkv_bf16) x.col = static_cast<const uint16_t *>(colsrc)[ci];
        else x.col = __float_as_uint(static_cast<const float *>(colsrc)[ci]);
    };
    auto load_start = [&](int c, float (&dst)[NR]) {  // state chunk c starts from
        const float *hc = p.states + ((size_t)(first_chunk + c) * p.HV + hv) * K * V;
#pragma unroll
        for (int i = 0; i < NR; ++i) dst[i] = hc[(size_t)(rg + kRowGroups * i) * V + col];
    };

    // role 0 (reverse) state
    float dS[NR], S0[NR], St[NR], Sp[NR], Spn[NR], w = 0.f, wn = 0.f, part = 0.f, doj = 0.f;
    // role 1 (recompute) state
    float S[NR];
    Rows cur, nxt;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        dS[i] = (role == 0 && p.dht) ? p.dht[(((int64_t)n * p.HV + hv) * K + rg + kRowGroups * i) * V + col] : 0.f;
        S0[i] = St[i] = Sp[i] = Spn[i] = S[i] = 0.f;
    }
    int parity = 0;
    for (int ph = nchunks; ph >= 0; --ph) {
        const int cr = ph - 1, cv = ph;  // chunk recomputed, chunk reversed
        const int lr = chunk_len(cr), lv = chunk_len(cv);
        const int nst = lr > lv ? lr : lv;
        const int64_t t0r = t_begin + (int64_t)cr * C, t0v = t_begin + (int64_t)cv * C;
        float *scr = sc(cr & 1), *swr = sw(cr & 1);
        const float *scv = sc(cv & 1), *swv = sw(cv & 1);
        if (role == 1 && lr > 0) {
            load_start(cr, S);
            load_rows(t0r, p.v, cur);
        }
        if (role == 0 && lv > 0) {
            load_start(cv, S0);
            const int tl = lv - 1;
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                St[i] = scv[((size_t)tl * K + rg + kRowGroups * i) * kSlice + j];
                Sp[i] = tl > 0 ? scv[((size_t)(tl - 1) * K + rg + kRowGroups * i) * kSlice + j] : S0[i];
            }
            w = swv[tl * kSlice + j];
            load_rows(t0v + tl, p.dout, cur);
        }
        for (int st = 0; st < nst; ++st) {
            // ---- before the step's barrier
            if (role == 1 && st < lr) {
                if (st + 1 < lr) load_rows(t0r + st + 1, p.v, nxt);
                part = 0.f;
#pragma unroll
                for (int i = 0; i < NR; ++i) {
                    S[i] *= cur.a[i];
                    part += S[i] * cur.k[i];
                }
                part += __shfl_xor(part, 16, 64);  // the wave's four row groups
                part += __shfl_xor(part, 32, 64);
                if ((lt & 63) < kSlice) red[1][parity][lt >> 6][j] = part;
            }
            if (role == 0 && st < lv) {
                const int tl = lv - 1 - st;
                const int64_t t = t0v + tl;
                if (tl > 0) {
                    load_rows(t - 1, p.dout, nxt);
#pragma unroll
                    for (int i = 0; i < NR; ++i)
                        Spn[i] = tl - 1 > 0 ? scv[((size_t)(tl - 2) * K + rg + kRowGroups * i) * kSlice + j] : S0[i];
                    wn = swv[(tl - 1) * kSlice + j];
                }
                doj = colval(cur.col);
                const size_t pbase = ((size_t)slice * p.Ttot + t) * p.HV + hv;
                part = 0.f;
#pragma unroll
                for (int i = 0; i < NR; ++i) {
                    dS[i] += cur.q[i] * doj;
                    part += dS[i] * cur.k[i];
                }
                part += __shfl_xor(part, 16, 64);
                part += __shfl_xor(part, 32, 64);
                if ((lt & 63) < kSlice) red[0][parity][lt >> 6][j] = part;
#pragma unroll
                for (int i = 0; i < NR; ++i) {  // dq^ rows, summed over the slice's columns
                    const float x = row_sum16(St[i] * doj);
                    if (j == 0) p.p_dq[pbase * K + rg + kRowGroups * i] = x;
                }
            }
            __syncthreads();
            // ---- after it
            if (role == 1 && st < lr) {
                float u = 0.f;
                for (int g = 0; g < kRoleThreads / 64; ++g) u += red[1][parity][g][j];
                const float wv = colval(cur.col) - u;
#pragma unroll
                for (int i = 0; i < NR; ++i) {
                    S[i] += cur.b * cur.k[i] * wv;
                    scr[((size_t)st * K + rg + kRowGroups * i) * kSlice + j] = S[i];
                }
                if (rg == 0) swr[st * kSlice + j] = wv;
                if (st + 1 < lr) cur = nxt;
            }
            if (role == 0 && st < lv) {
                const int tl = lv - 1 - st;
                const int64_t t = t0v + tl;
                const size_t pbase = ((size_t)slice * p.Ttot + t) * p.HV + hv;
                float cj = 0.f;
                for (int g = 0; g < kRoleThreads / 64; ++g) cj += red[0][parity][g][j];
                const float b = cur.b;
                const float e = b * cj;
                if (rg == 0) p.dv[(t * p.HV + hv) * V + col] = e;
                const float db = row_sum16(w * cj);
                if (lt == 0) p.p_db[pbase] = db;
#pragma unroll
                for (int i = 0; i < NR; ++i) {
                    const float P = cur.a[i] * Sp[i];
                    const float dk = row_sum16(b * dS[i] * w - P * e);
                    const float dP = dS[i] - cur.k[i] * e;
                    const float dgp = row_sum16(dP * P);
                    if (j == 0) {
                        p.p_dk[pbase * K + rg + kRowGroups * i] = dk;
                        p.p_dg[pbase * K + rg + kRowGroups * i] = dgp;
                    }
                    dS[i] = cur.a[i] * dP;
                }
                if (tl > 0) {
                    cur = nxt;
#pragma unroll
                    for (int i = 0; i < NR; ++i) St[i] = Sp[i], Sp[i] = Spn[i];
                    w = wn;
                }
            }
            parity ^= 1;  // the next write to this parity's buffers is a barrier away from its reads
        }
        __syncthreads();  // scratch written in this phase is read in the next; read buffers are refilled after it
    }
    if (role == 0 && p.dh0) {
#pragma unroll
        for (int i = 0; i < NR; ++i)
            p.dh0[(((int64_t)n * p.HV + hv) * K + rg + kRowGroups * i) * V + col] = dS[i];
    }
}

// dq, dk per (token, qk head): the value heads of the group and the partial sums
// summed in order, then the scale and L2-norm chain rule.  One wave per (token, qk head)
// row, four rows per block; lane l holds elements 4l .. 4l + 3 of the row (K <= 256).
__device__ __forceinline__ float4 ld4(const void *p, int64_t i, bool bf) {
    if (bf) {
        const uint2 u = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + i);
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                           __uint_as_float(u.y & 0xffff0000u));
    }
    return *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i);
}

// One row (token, qk head) per LANES lanes: a half wave when K <= 128 (every lane holds 4
// elements), a whole wave for wider keys.
template <int LANES>
__global__ void __launch_bounds__(kBwdThreads) bwd_qk_kernel(BwdParams p) {
    const int64_t row = (int64_t)blockIdx.x * (kBwdThreads / LANES) + (threadIdx.x / LANES);
    const bool valid = row < p.Ttot * p.H;  // rows past the end still join the reductions
    const int64_t t = valid ? row / p.H : 0;
    const int h = valid ? (int)(row % p.H) : 0, l = threadIdx.x & (LANES - 1);
    const int group = p.HV / p.H, ns = p.nslices, K = p.K;
    const bool on = valid && 4 * l < K;
    auto rsum = [](float x) { return LANES == 32 ? half_sum(x) : wave_sum(x); };
    float4 gq = make_float4(0.f, 0.f, 0.f, 0.f), gk = gq, qv = gq, kv = gq;
    if (on) {
        for (int sl = 0; sl < ns; ++sl)
            for (int jv = 0; jv < group; ++jv) {
                const size_t r = (((size_t)sl * p.Ttot + t) * p.HV + h * group + jv) * K + 4 * l;
                const float4 a = *reinterpret_cast<const float4 *>(p.p_dq + r);
                const float4 b = *reinterpret_cast<const float4 *>(p.p_dk + r);
                gq.x += a.x, gq.y += a.y, gq.z += a.z, gq.w += a.w;
                gk.x += b.x, gk.y += b.y, gk.z += b.z, gk.w += b.w;
            }
        qv = ld4(p.q, row * K + 4 * l, p.qkv_bf16);
        kv = ld4(p.k, row * K + 4 * l, p.qkv_bf16);
    }
    float4 dq = make_float4(gq.x * p.scale, gq.y * p.scale, gq.z * p.scale, gq.w * p.scale), dk = gk;
    if (p.qk_l2norm) {
        const float sq = rsum(qv.x * qv.x + qv.y * qv.y + qv.z * qv.z + qv.w * qv.w);
        const float sk = rsum(kv.x * kv.x + kv.y * kv.y + kv.z * kv.z + kv.w * kv.w);
        const float qd = rsum(qv.x * gq.x + qv.y * gq.y + qv.z * gq.z + qv.w * gq.w);
        const float kd = rsum(kv.x * gk.x + kv.y * gk.y + kv.z * gk.z + kv.w * gk.w);
        const float rq = 1.f / sqrtf(sq + 1e-6f), rk = 1.f / sqrtf(sk + 1e-6f);
        // x^ = x r, r = (|x|^2 + eps)^-1/2:  dx = r dx^ - r^3 x (x . dx^)
        const float cq = rq * rq * rq * qd, ck = rk * rk * rk * kd;
        dq = make_float4(p.scale * (rq * gq.x - cq * qv.x), p.scale * (rq * gq.y - cq * qv.y),
                         p.scale * (rq * gq.z - cq * qv.z), p.scale * (rq * gq.w - cq * qv.w));
        dk = make_float4(rk * gk.x - ck * kv.x, rk * gk.y - ck * kv.y, rk * gk.z - ck * kv.z, rk * gk.w - ck * kv.w);
    }
    if (on) {
        *reinterpret_cast<float4 *>(p.dq + row * K + 4 * l) = dq;
        *reinterpret_cast<float4 *>(p.dk + row * K + 4 * l) = dk;
    }
}

// dg and the per-element dA_log terms per (token, value head), and dbeta.
__global__ void __launch_bounds__(kBwdThreads) bwd_gate_kernel(BwdParams p) {
    const int64_t t = blockIdx.x / p.HV;
    const int hv = blockIdx.x % p.HV, d = threadIdx.x;
    const int ns = p.nslices;
    if (d < p.K) {
        float gp = 0.f;  // dL/dg' (natural-log activated gate)
        for (int sl = 0; sl < ns; ++sl) gp += p.p_dg[(((size_t)sl * p.Ttot + t) * p.HV + hv) * p.K + d];
        const size_t idx = (t * p.HV + hv) * p.K + d;
        float dg = gp, da = 0.f;
        if (p.gate_mode != kGatePre) {
            const float x = ldf(p.g, idx, p.g_bf16) + (p.dt_bias ? p.dt_bias[(int64_t)hv * p.K + d] : 0.f);
            if (p.gate_mode == kGateSoftplus) {
                const float ea = expf(p.A_log[hv]);
                dg = gp * (-ea) * sigm(x);
                da = gp * (-ea * softplus_f(x));
            } else {
                const float a = p.A_log ? expf(p.A_log[hv]) : 1.f;
                const float sg = sigm(a * x);
                const float ds = p.lower_bound * sg * (1.f - sg);
                dg = gp * ds * a;
                da = gp * ds * a * x;
            }
        }
        p.dg[idx] = dg;
        p.scr_da[idx] = da;
    }
    if (d == 0) {
        float db = 0.f;
        for (int sl = 0; sl < ns; ++sl) db += p.p_db[((size_t)sl * p.Ttot + t) * p.HV + hv];
        const float braw = ldf(p.beta, t * p.HV + hv, p.beta_bf16);
        if (p.beta_mode == kBetaSigmoid) db *= sigm(braw) * (1.f - sigm(braw));
        else if (p.beta_mode == kBetaTwoSigmoid) db *= 2.f * sigm(braw) * (1.f - sigm(braw));
        p.dbeta[t * p.HV + hv] = db;
    }
}

// dt_bias and A_log gradients: sums over tokens (and channels for A_log).  First per
// (value head, token segment), then the segments in order, so the result does not
// depend on scheduling.
constexpr int kParamSegs = 64;

__global__ void __launch_bounds__(kBwdThreads) bwd_param_partial_kernel(BwdParams p) {
    __shared__ float ws[4];
    const int hv = blockIdx.x / kParamSegs, seg = blockIdx.x % kParamSegs, d = threadIdx.x;
    const int64_t per = (p.Ttot + kParamSegs - 1) / kParamSegs;
    const int64_t ta = seg * per, tb = ta + per < p.Ttot ? ta + per : p.Ttot;
    float sdg = 0.f, sda = 0.f;
    if (d < p.K)
        for (int64_t t = ta; t < tb; ++t) {
            const size_t idx = (t * p.HV + hv) * p.K + d;
            sdg += p.dg[idx];
            sda += p.scr_da[idx];
        }
    float *part = p.scr_param + (size_t)(hv * kParamSegs + seg) * (p.K + 1);
    if (d < p.K) part[d] = sdg;
    const float r = wave_sum(sda);
    if ((d & 63) == 0) ws[d >> 6] = r;
    __syncthreads();
    if (d == 0) part[p.K] = ws[0] + ws[1] + ws[2] + ws[3];
}

__global__ void __launch_bounds__(kBwdThreads) bwd_param_kernel(BwdParams p) {
    const int hv = blockIdx.x, d = threadIdx.x;
    const float *part = p.scr_param + (size_t)hv * kParamSegs * (p.K + 1);
    if (d < p.K && p.ddt_bias) {
        float acc = 0.f;
        for (int seg = 0; seg < kParamSegs; ++seg) acc += part[(size_t)seg * (p.K + 1) + d];
        p.ddt_bias[(int64_t)hv * p.K + d] = acc;
    }
    if (d == 0 && p.dA_log) {
        float acc = 0.f;
        for (int seg = 0; seg < kParamSegs; ++seg) acc += part[(size_t)seg * (p.K + 1) + p.K];
        p.dA_log[hv] = acc;
    }
}

}  // namespace

size_t bwd_param_scratch_floats(int HV, int K) { return (size_t)HV * kParamSegs * (K + 1); }

int bwd_slices(int V) { return V / kSlice; }

size_t bwd_seq_state_floats(int N, int HV, int K, int V, int C) {  // two buffers per workgroup
    return (size_t)N * HV * (V / kSlice) * 2 * C * (size_t)K * kSlice;
}

size_t bwd_seq_scratch_floats(int N, int HV, int K, int V, int C) {
    return bwd_seq_state_floats(N, HV, K, V, C) + (size_t)N * HV * (V / kSlice) * 2 * C * kSlice;
}

hipError_t launch_backward(const BwdParams &p, hipStream_t s) {
    const int ns = p.V / kSlice;
    const unsigned units = (unsigned)p.N * (unsigned)p.HV * (unsigned)ns;
    if (p.Ttot > 0) {
        hipLaunchKernelGGL(bwd_token_prep_kernel, dim3((unsigned)(p.Ttot * p.HV)), dim3(kBwdThreads), 0, s, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (units > 0) {
        switch (p.K / 32) {
        case 1: hipLaunchKernelGGL(bwd_seq_kernel<1>, dim3(units), dim3(kSeqThreads), 0, s, p); break;
        case 2: hipLaunchKernelGGL(bwd_seq_kernel<2>, dim3(units), dim3(kSeqThreads), 0, s, p); break;
        case 3: hipLaunchKernelGGL(bwd_seq_kernel<3>, dim3(units), dim3(kSeqThreads), 0, s, p); break;
        case 4: hipLaunchKernelGGL(bwd_seq_kernel<4>, dim3(units), dim3(kSeqThreads), 0, s, p); break;
        case 5: hipLaunchKernelGGL(bwd_seq_kernel<5>, dim3(units), dim3(kSeqThreads), 0, s, p); break;
        case 6: hipLaunchKernelGGL(bwd_seq_kernel<6>, dim3(units), dim3(kSeqThreads), 0, s, p); break;
        case 7: hipLaunchKernelGGL(bwd_seq_kernel<7>, dim3(units), dim3(kSeqThreads), 0, s, p); break;
        case 8: hipLaunchKernelGGL(bwd_seq_kernel<8>, dim3(units), dim3(kSeqThreads), 0, s, p); break;
        default: return hipErrorInvalidValue;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_bwd_finish(p, s);
}

// The finishing kernels shared by both backward forms: per-element partial sums
// (p.nslices of them) -> dq, dk (GVA sum, scale and L2-norm chain rule), dg, dbeta
// (activation chain rules), then the dt_bias and A_log token sums.
hipError_t launch_bwd_finish(const BwdParams &p, hipStream_t s) {
    if (p.Ttot > 0) {
        if (p.K <= 128)
            hipLaunchKernelGGL(bwd_qk_kernel<32>, dim3((unsigned)((p.Ttot * p.H + 7) / 8)), dim3(kBwdThreads), 0, s, p);
        else
            hipLaunchKernelGGL(bwd_qk_kernel<64>, dim3((unsigned)((p.Ttot * p.H + 3) / 4)), dim3(kBwdThreads), 0, s, p);
        hipLaunchKernelGGL(bwd_gate_kernel, dim3((unsigned)(p.Ttot * p.HV)), dim3(kBwdThreads), 0, s, p);
    }
    if (p.gate_mode != kGatePre) {
        hipLaunchKernelGGL(bwd_param_partial_kernel, dim3((unsigned)p.HV * kParamSegs), dim3(kBwdThreads), 0, s, p);
        hipLaunchKernelGGL(bwd_param_kernel, dim3((unsigned)p.HV), dim3(kBwdThreads), 0, s, p);
    }
    return hipGetLastError();
}

// dt_bias and A_log gradients of the chunked form: the per-chunk sums of every chunk of
// the value head.  One block of 1024 threads per value head: 8 stripes of 128 columns,
// stripe j adding chunks j, j + 8, ... in order, then the 8 stripe sums in order, so the
// result does not depend on scheduling.
constexpr int kParamStripes = 8;

__global__ void __launch_bounds__(1024) bwd_chunk_param_kernel(BwdChunkParams P) {
    __shared__ float part[kParamStripes][257 + 1];
    const int hv = blockIdx.x, K = P.b.K, HV = P.b.HV, nc = P.f.total_chunks;
    const int stripe = threadIdx.x >> 7, c0 = threadIdx.x & 127;
    for (int d = c0; d <= K; d += 128) {
        float acc = 0.f;
        for (int c = stripe; c < nc; c += kParamStripes) acc += P.cparam[((size_t)c * HV + hv) * (K + 1) + d];
        part[stripe][d] = acc;
    }
    __syncthreads();
    for (int d = threadIdx.x; d <= K; d += blockDim.x) {
        float acc = 0.f;
        for (int j = 0; j < kParamStripes; ++j) acc += part[j][d];
        if (d < K) {
            if (P.b.ddt_bias) P.b.ddt_bias[(int64_t)hv * K + d] = acc;
        } else if (P.b.dA_log) {
            P.b.dA_log[hv] = acc;
        }
    }
}

// The chunked form's finishing kernels: dq and dk from the per-value-head partial sums
// (dg and dbeta are final from the per-chunk kernel), then dt_bias and A_log.
hipError_t launch_bwd_finish_chunked(const BwdChunkParams &P, hipStream_t s) {
    const BwdParams &p = P.b;
    if (p.Ttot > 0)
        if (p.K <= 128)
            hipLaunchKernelGGL(bwd_qk_kernel<32>, dim3((unsigned)((p.Ttot * p.H + 7) / 8)), dim3(kBwdThreads), 0, s, p);
        else
            hipLaunchKernelGGL(bwd_qk_kernel<64>, dim3((unsigned)((p.Ttot * p.H + 3) / 4)), dim3(kBwdThreads), 0, s, p);
    if (p.gate_mode != kGatePre && (p.ddt_bias || p.dA_log))
        hipLaunchKernelGGL(bwd_chunk_param_kernel, dim3((unsigned)p.HV), dim3(1024), 0, s, P);
    return hipGetLastError();
}

}  // namespace kda
