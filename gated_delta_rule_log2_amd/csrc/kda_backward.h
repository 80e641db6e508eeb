// kda_backward.h -- launch parameters of the backward kernels (kda_backward.hip).
// Not part of the public ABI.
#pragma once

#include "kda_internal.h"

namespace kda {

struct BwdParams {
    int32_t N, T, H, HV, K, V, C;   // T: tokens per batch row (fixed-length batches)
    int64_t Ttot;                   // tokens in all
    int32_t gate_mode, beta_mode, qk_l2norm;
    int32_t qkv_bf16, g_bf16, beta_bf16;
    float scale;
    float lower_bound;              // natural-log units
    // inputs
    const void *q, *k, *v, *g, *beta, *dout;
    const float *A_log, *dt_bias, *dht;
    const int64_t *cu_seqlens;      // device offsets or nullptr
    const float *states;            // [total chunks, HV, K, V] state each chunk starts from
    // outputs (fp32); dA_log, ddt_bias, dh0 may be nullptr
    float *dq, *dk, *dv, *dg, *dbeta, *dA_log, *ddt_bias, *dh0;
    // workspace
    float *p_dq, *p_dk, *p_dg;      // [slices, Ttot, HV, K] per-slice sums over V
    float *p_db;                    // [slices, Ttot, HV]
    float *scr_state, *scr_w;       // per workgroup: [C, K, slice] token states, [C, slice] w
    float *scr_da;                  // [Ttot, HV, K] dA_log terms
    float *t_q, *t_k, *t_a;         // [Ttot, HV, K] q^, k^ (of the head's qk head), exp(g')
    float *t_b;                     // [Ttot, HV] beta after its transform
    float *scr_param;               // [HV, 64, K + 1] per-segment dt_bias / A_log sums
    int32_t nslices;                // partial sums per element in p_dq, p_dk, p_dg, p_db (summed in order)
};

// The chunked backward's kernels see the forward's parameters (chunk plan, the per-chunk
// intermediates W, Qg, KgT, Aqk, d in the forward workspace) beside the backward's.
struct BwdChunkParams {
    Params f;
    BwdParams b;
    float *dU;                      // [total chunks * HV][C][V] gradient of U - W S (dV_new)
    float *dh;                      // [total chunks * HV][K][V] gradient of the state after each chunk
    // bf16 intermediates: the reverse recurrence's operands, per (chunk, value head) slot
    uint16_t *rpack;                // Kg [C][K], W^T [K][C] (permuted row fragments)
    uint16_t *ppack;                // Aqk^T [C][C], Qg^T [K][C] (permuted row fragments)
    uint16_t *doq;                  // dO [V][C] in accumulator-tile order
    float *cparam;                  // [total chunks * HV][K + 1] per-chunk dt_bias sums, then the A_log sum
    int32_t prep_done;              // bf16: rpack, ppack and doq were written by launch_bwd_prep
                                    // beforehand (else launch_bwd_dhu writes them first)
};

// The chunked backward covers K <= 128 (the token-level form above that).
bool bwd_chunk_fits(int K);
hipError_t launch_bwd_dhu(const BwdChunkParams &p, hipStream_t s);
hipError_t launch_bwd_prep(const BwdChunkParams &p, hipStream_t s);  // bf16 only; else nothing
hipError_t launch_bwd_local(const BwdChunkParams &p, hipStream_t s);
hipError_t launch_bwd_finish(const BwdParams &p, hipStream_t s);
hipError_t launch_bwd_finish_chunked(const BwdChunkParams &p, hipStream_t s);

int bwd_slices(int V);
size_t bwd_seq_state_floats(int N, int HV, int K, int V, int C);
size_t bwd_seq_scratch_floats(int N, int HV, int K, int V, int C);
size_t bwd_param_scratch_floats(int HV, int K);
hipError_t launch_backward(const BwdParams &p, hipStream_t s);

}  // namespace kda
