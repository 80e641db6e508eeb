// kda_internal.h -- launch parameters shared by the C-ABI host code and the
// HIP kernel launchers.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

enum GateMode : int32_t { kGatePre = 0, kGateSoftplus = 1, kGateLowerBound = 2 };
enum BetaMode : int32_t { kBetaGiven = 0, kBetaSigmoid = 1, kBetaTwoSigmoid = 2 };

struct Params {
    // sizes
    int32_t B, T, H, HV, K, V, C;  // C = chunk size
    int32_t N;                     // sequences
    int32_t total_chunks;          // chunks over all sequences (each sequence starts a chunk)
    int32_t group;                 // HV / H
    // modes
    int32_t gate_mode, beta_mode, qk_l2norm;
    int32_t qkv_bf16, g_bf16, beta_bf16;
    float scale;
    float lower_bound;             // natural-log lower bound of the bounded gate (0 without one)
    int32_t output_final_state;
    int32_t state_vk;              // state tensors stored [V][K] (else [K][V]) per (sequence, head)
    // inputs
    const void *q, *k, *v, *g, *beta;
    const float *A_log, *dt_bias, *h0;
    const int64_t *cu_seqlens;     // device offsets or nullptr (then sequence n = batch row n)
    // outputs
    void *o;
    float *ht;
    float *hs;                     // [total_chunks, HV, K, V] state each chunk starts from, or nullptr
    int32_t hs_frag;               // hs in the register-resident recurrence's fragment order
                                   // (backward hand-over; see recur_reg_kernel), else [K][V] / [V][K]
    int32_t skip_output;           // with hs: o is not needed (the backward's recompute), the
                                   // register-resident recurrence leaves it unwritten
    float *g_act, *g_cum;          // gate-only entry point
    // workspace
    int32_t *chunk_off;            // [N + 1] first global chunk of each sequence
    int32_t *chunk_seq;            // [total_chunks] sequence of each global chunk
    int32_t *seq_order;            // [N] sequences longest first (packed batches; the
                                   // recurrence issues its workgroups in this order)
    void *w_W, *w_U, *w_KgT, *w_Qg, *w_Aqk;  // per (chunk, value head) intermediates
    float *w_d;                               // [total_chunks * HV * K] 2^(chunk gate total)
};

// Byte layout of the workspace; offsets are 256-byte aligned.
struct WorkspaceLayout {
    size_t off_chunk_off, off_chunk_seq, off_seq_order, off_W, off_U, off_KgT, off_Qg, off_Aqk, off_d;
    size_t plan_bytes, total_bytes;
};

WorkspaceLayout workspace_layout(int32_t N, int32_t total_chunks, int32_t HV, int32_t K, int32_t V,
                                 int32_t C, size_t elem_bytes);
void bind_workspace(Params &p, void *workspace, const WorkspaceLayout &L);

// Launchers (return hipSuccess or the launch error).
hipError_t launch_plan(const Params &p, hipStream_t s);
hipError_t launch_gate_cumsum(const Params &p, hipStream_t s);
hipError_t launch_intra(const Params &p, hipStream_t s);
hipError_t launch_recurrence(const Params &p, hipStream_t s);
hipError_t launch_fused_recurrent(const Params &p, hipStream_t s);

}  // namespace kda

#include "../../include/kda.h"

namespace kda {
// The forward of kda_chunk_fwd / _states / _profiled: descriptor, pointer and workspace
// checks, then plan -> intra -> recurrence on `stream` (kda_abi.cpp).
kda_status chunk_fwd_run(const kda_fwd_desc *d, const void *q, const void *k, const void *v, const void *g,
                         const void *beta, const float *A_log, const float *dt_bias, const float *initial_state,
                         const int64_t *cu_seqlens, void *o, float *final_state, bool want_states, float *states,
                         void *workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t *ev,
                         bool states_frag = false, bool skip_output = false);
}  // namespace kda
