// kda_abi.cpp -- the C ABI declared in include/kda.h: argument checks, the
// workspace layout and the launch sequence (plan -> intra -> recurrence).
//
// The checks follow the contract of chunk_kda described in "flash-linear-attention
// KDA 内核工程实践…", §2.1 (chunk size, K limit, GVA divisibility, A_log
// requirement, safe-gate lower-bound interval, allow_neg_eigval needing the beta
// sigmoid, fp32 initial state), and the host-side validation of
// "FlashKDA gate偏置加載路徑完整解析", §二 第2段 / §四 (fp32 A_log and dt_bias,
// contiguous tensors, an error instead of a silent failure).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/kda.h"
#include "kda_backward.h"
#include "kda_internal.h"

namespace kda {
size_t intra_lds_bytes(int C, int K, int V, bool bf16);

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

WorkspaceLayout workspace_layout(int32_t N, int32_t total_chunks, int32_t HV, int32_t K, int32_t V,
                                 int32_t C, size_t eb) {
    WorkspaceLayout L{};
    size_t off = 0;
    L.off_chunk_off = off;
    off = align256(off + sizeof(int32_t) * ((size_t)N + 1));
    L.off_chunk_seq = off;
    off = align256(off + sizeof(int32_t) * (size_t)(total_chunks > 0 ? total_chunks : 1));
    L.off_seq_order = off;
    off = align256(off + sizeof(int32_t) * ((size_t)N + 1));
    L.plan_bytes = off;
    const size_t slots = (size_t)total_chunks * (size_t)HV;
    L.off_W = off;
    off = align256(off + eb * slots * C * K);
    L.off_U = off;
    off = align256(off + eb * slots * C * V);
    L.off_KgT = off;
    off = align256(off + eb * slots * K * C);
    L.off_Qg = off;
    off = align256(off + eb * slots * C * K);
    L.off_Aqk = off;
    off = align256(off + eb * slots * C * C);
    L.off_d = off;
    off = align256(off + sizeof(float) * slots * K);
    L.total_bytes = off;
    return L;
}

void bind_workspace(Params &p, void *ws, const WorkspaceLayout &L) {
    unsigned char *b = static_cast<unsigned char *>(ws);
    p.chunk_off = reinterpret_cast<int32_t *>(b + L.off_chunk_off);
    p.chunk_seq = reinterpret_cast<int32_t *>(b + L.off_chunk_seq);
    p.seq_order = reinterpret_cast<int32_t *>(b + L.off_seq_order);
    p.w_W = b + L.off_W;
    p.w_U = b + L.off_U;
    p.w_KgT = b + L.off_KgT;
    p.w_Qg = b + L.off_Qg;
    p.w_Aqk = b + L.off_Aqk;
    p.w_d = reinterpret_cast<float *>(b + L.off_d);
}

// Descriptor checks shared by every entry point.  On success fills the sizes of p.
static kda_status check_desc(const kda_fwd_desc *d, Params &p) {
    if (!d) return KDA_ERR_NULL_POINTER;
    if (d->B < 1 || d->T < 0 || d->H < 1 || d->HV < 1 || d->K < 1 || d->V < 1 || d->num_seqs < 0)
        return KDA_ERR_SHAPE;
    if ((int64_t)d->B * d->T > (int64_t)INT32_MAX / 2) return KDA_ERR_SHAPE;
    if (d->chunk_size != 32 && d->chunk_size != 64) return KDA_ERR_CHUNK_SIZE;
    if (d->K > 256) return KDA_ERR_HEAD_DIM;
    if (d->K % 32 != 0 || d->V % 32 != 0 || d->V > 256) return KDA_ERR_UNSUPPORTED;
    if (intra_lds_bytes(d->chunk_size, d->K, d->V, d->qkv_dtype == KDA_DTYPE_BF16) > 160u * 1024u)
        return KDA_ERR_UNSUPPORTED;  // fp32 inputs with K = V = 256 exceed one CU's LDS
    if (d->HV % d->H != 0) return KDA_ERR_GVA;
    const uint32_t f = d->flags;
    if (f & ~0xffu) return KDA_ERR_UNSUPPORTED;
    const bool has_lb = f & KDA_HAS_LOWER_BOUND;
    const float lb = d->lower_bound;
    if ((f & KDA_SAFE_GATE) && (!has_lb || !(lb >= -5.f && lb < 0.f))) return KDA_ERR_LOWER_BOUND;
    if (has_lb && !(lb < 0.f)) return KDA_ERR_LOWER_BOUND;
    if ((f & KDA_ALLOW_NEG_EIGVAL) && !(f & KDA_BETA_SIGMOID)) return KDA_ERR_NEG_EIGVAL;
    // sequences
    int64_t total_chunks = 0;
    if (d->cu_seqlens_host) {
        if (d->B != 1 || d->num_seqs < 1) return KDA_ERR_VARLEN;
        const int64_t *cu = d->cu_seqlens_host;
        if (cu[0] != 0 || cu[d->num_seqs] != d->T) return KDA_ERR_VARLEN;
        for (int n = 0; n < d->num_seqs; ++n) {
            if (cu[n + 1] < cu[n]) return KDA_ERR_VARLEN;
            total_chunks += (cu[n + 1] - cu[n] + d->chunk_size - 1) / d->chunk_size;
        }
    } else {
        if (d->num_seqs != d->B) return KDA_ERR_SHAPE;
        total_chunks = (int64_t)d->B * ((d->T + d->chunk_size - 1) / d->chunk_size);
    }
    if (total_chunks * d->HV > (int64_t)INT32_MAX) return KDA_ERR_SHAPE;
    auto dtype_ok = [](int32_t t) { return t == KDA_DTYPE_FP32 || t == KDA_DTYPE_BF16; };
    if (!dtype_ok(d->qkv_dtype) || !dtype_ok(d->g_dtype) || !dtype_ok(d->beta_dtype)) return KDA_ERR_DTYPE;

    std::memset(&p, 0, sizeof(p));
    p.B = d->B; p.T = d->T; p.H = d->H; p.HV = d->HV; p.K = d->K; p.V = d->V;
    p.C = d->chunk_size;
    p.N = d->cu_seqlens_host ? d->num_seqs : d->B;
    p.total_chunks = (int32_t)total_chunks;
    p.group = d->HV / d->H;
    p.gate_mode = !(f & KDA_GATE_IN_KERNEL) ? kGatePre : (has_lb ? kGateLowerBound : kGateSoftplus);
    p.beta_mode = !(f & KDA_BETA_SIGMOID) ? kBetaGiven : ((f & KDA_ALLOW_NEG_EIGVAL) ? kBetaTwoSigmoid : kBetaSigmoid);
    p.qk_l2norm = (f & KDA_QK_L2NORM) ? 1 : 0;
    p.qkv_bf16 = d->qkv_dtype == KDA_DTYPE_BF16;
    p.g_bf16 = d->g_dtype == KDA_DTYPE_BF16;
    p.beta_bf16 = d->beta_dtype == KDA_DTYPE_BF16;
    p.scale = d->scale;
    p.lower_bound = has_lb ? lb : 0.f;
    p.output_final_state = (f & KDA_OUTPUT_FINAL_STATE) ? 1 : 0;
    p.state_vk = (f & KDA_TRANSPOSE_STATE) ? 1 : 0;
    return KDA_OK;
}

static kda_status to_status(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

}  // namespace kda

using namespace kda;

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char *kda_status_string(kda_status s) {
    switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "invalid or inconsistent sizes";
    case KDA_ERR_CHUNK_SIZE: return "chunk_size must be 32 or 64";
    case KDA_ERR_HEAD_DIM: return "K must be <= 256";
    case KDA_ERR_UNSUPPORTED: return "unsupported configuration (K and V must be multiples of 32, V <= 256)";
    case KDA_ERR_GVA: return "HV must be a multiple of H";
    case KDA_ERR_MISSING_A_LOG: return "A_log is required for the in-kernel gate without a lower bound";
    case KDA_ERR_LOWER_BOUND: return "safe_gate needs -5 <= lower_bound < 0, and a lower bound must be < 0";
    case KDA_ERR_NEG_EIGVAL: return "allow_neg_eigval requires use_beta_sigmoid_in_kernel";
    case KDA_ERR_VARLEN: return "cu_seqlens needs B == 1 and offsets 0 = cu[0] <= ... <= cu[N] = T";
    case KDA_ERR_DTYPE: return "dtype must be fp32 or bf16";
    case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

kda_status kda_chunk_fwd_workspace_size(const kda_fwd_desc *d, size_t *bytes) {
    Params p;
    kda_status st = check_desc(d, p);
    if (st != KDA_OK) return st;
    if (!bytes) return KDA_ERR_NULL_POINTER;
    *bytes = workspace_layout(p.N, p.total_chunks, p.HV, p.K, p.V, p.C, p.qkv_bf16 ? 2 : 4).total_bytes;
    return KDA_OK;
}

kda_status kda_gate_chunk_cumsum_workspace_size(const kda_fwd_desc *d, size_t *bytes) {
    Params p;
    kda_status st = check_desc(d, p);
    if (st != KDA_OK) return st;
    if (!bytes) return KDA_ERR_NULL_POINTER;
    *bytes = workspace_layout(p.N, p.total_chunks, 0, p.K, p.V, p.C, 4).plan_bytes;
    return KDA_OK;
}

static const char *const kStageNames[] = {"plan", "intra", "recurrence"};
static const int kNumStages = 3;

int kda_chunk_fwd_stage_count(void) { return kNumStages; }

const char *kda_chunk_fwd_stage_name(int i) { return (i >= 0 && i < kNumStages) ? kStageNames[i] : nullptr; }

}  // extern "C"

// The forward's pointer checks (inputs, outputs, A_log, cu_seqlens against the descriptor).
static kda_status fwd_pointer_checks(const kda_fwd_desc *d, const void *q, const void *k, const void *v, const void *g,
                                     const void *beta, const float *A_log, const int64_t *cu_seqlens, const void *o,
                                     const float *final_state) {
    const bool tokens = (int64_t)d->B * d->T > 0;
    if (tokens && (!q || !k || !v || !g || !beta || !o)) return KDA_ERR_NULL_POINTER;
    if ((d->flags & KDA_OUTPUT_FINAL_STATE) && !final_state) return KDA_ERR_NULL_POINTER;
    if ((d->flags & KDA_GATE_IN_KERNEL) && !(d->flags & KDA_HAS_LOWER_BOUND) && !A_log)
        return KDA_ERR_MISSING_A_LOG;
    if ((cu_seqlens == nullptr) != (d->cu_seqlens_host == nullptr)) return KDA_ERR_VARLEN;
    return KDA_OK;
}

// The whole forward: checks, then plan -> intra -> recurrence on `stream`.  `states`
// (the state each chunk starts from) is written when want_states, in the recurrence's
// fragment order when states_frag (only where the register-resident recurrence runs);
// `ev` as for kda_chunk_fwd_profiled.
kda_status kda::chunk_fwd_run(const kda_fwd_desc *d, const void *q, const void *k, const void *v, const void *g,
                            const void *beta, const float *A_log, const float *dt_bias, const float *initial_state,
                            const int64_t *cu_seqlens, void *o, float *final_state, bool want_states,
                            float *states, void *workspace, size_t workspace_bytes, hipStream_t stream,
                            hipEvent_t *ev, bool states_frag, bool skip_output) {
    Params p;
    kda_status st = check_desc(d, p);
    if (st != KDA_OK) return st;
    if (want_states && p.total_chunks > 0 && !states) return KDA_ERR_NULL_POINTER;
    st = fwd_pointer_checks(d, q, k, v, g, beta, A_log, cu_seqlens, o, final_state);
    if (st != KDA_OK) return st;
    const WorkspaceLayout L = workspace_layout(p.N, p.total_chunks, p.HV, p.K, p.V, p.C, p.qkv_bf16 ? 2 : 4);
    if (!workspace || workspace_bytes < L.total_bytes) return KDA_ERR_WORKSPACE;

    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
    p.A_log = A_log; p.dt_bias = dt_bias; p.h0 = initial_state;
    p.cu_seqlens = cu_seqlens;
    p.o = o; p.ht = final_state;
    p.hs = want_states ? states : nullptr;
    p.hs_frag = want_states && states_frag ? 1 : 0;
    p.skip_output = want_states && skip_output ? 1 : 0;
    bind_workspace(p, workspace, L);

    hipError_t (*const stages[kNumStages])(const Params &, hipStream_t) = {launch_plan, launch_intra,
                                                                            launch_recurrence};
    hipError_t e = hipSuccess;
    for (int i = 0; i < kNumStages && e == hipSuccess; ++i) {
        if (ev) e = hipEventRecord(ev[i], stream);
        if (e == hipSuccess) e = stages[i](p, stream);
    }
    if (ev && e == hipSuccess) e = hipEventRecord(ev[kNumStages], stream);
    return to_status(e);
}

extern "C" {

kda_status kda_chunk_fwd_profiled(const kda_fwd_desc *d, const void *q, const void *k, const void *v,
                                  const void *g, const void *beta, const float *A_log, const float *dt_bias,
                                  const float *initial_state, const int64_t *cu_seqlens, void *o,
                                  float *final_state, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream, hipEvent_t *ev) {
    return chunk_fwd_run(d, q, k, v, g, beta, A_log, dt_bias, initial_state, cu_seqlens, o, final_state, false,
                     nullptr, workspace, workspace_bytes, stream, ev);
}

kda_status kda_chunk_fwd(const kda_fwd_desc *d, const void *q, const void *k, const void *v,
                         const void *g, const void *beta, const float *A_log, const float *dt_bias,
                         const float *initial_state, const int64_t *cu_seqlens, void *o,
                         float *final_state, void *workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    return chunk_fwd_run(d, q, k, v, g, beta, A_log, dt_bias, initial_state, cu_seqlens, o, final_state, false,
                     nullptr, workspace, workspace_bytes, stream, nullptr);
}

kda_status kda_chunk_fwd_states(const kda_fwd_desc *d, const void *q, const void *k, const void *v,
                                const void *g, const void *beta, const float *A_log, const float *dt_bias,
                                const float *initial_state, const int64_t *cu_seqlens, void *o,
                                float *final_state, float *states, void *workspace, size_t workspace_bytes,
                                hipStream_t stream) {
    return chunk_fwd_run(d, q, k, v, g, beta, A_log, dt_bias, initial_state, cu_seqlens, o, final_state, true,
                     states, workspace, workspace_bytes, stream, nullptr);
}

kda_status kda_fused_recurrent_fwd(const kda_fwd_desc *d, const void *q, const void *k, const void *v,
                                   const void *g, const void *beta, const float *A_log, const float *dt_bias,
                                   const float *initial_state, const int64_t *cu_seqlens, void *o,
                                   float *final_state, hipStream_t stream) {
    Params p;
    kda_status st = check_desc(d, p);
    if (st != KDA_OK) return st;
    const bool tokens = (int64_t)d->B * d->T > 0;
    if (tokens && (!q || !k || !v || !g || !beta || !o)) return KDA_ERR_NULL_POINTER;
    if ((d->flags & KDA_OUTPUT_FINAL_STATE) && !final_state) return KDA_ERR_NULL_POINTER;
    if ((d->flags & KDA_GATE_IN_KERNEL) && !(d->flags & KDA_HAS_LOWER_BOUND) && !A_log)
        return KDA_ERR_MISSING_A_LOG;
    if ((cu_seqlens == nullptr) != (d->cu_seqlens_host == nullptr)) return KDA_ERR_VARLEN;
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
    p.A_log = A_log; p.dt_bias = dt_bias; p.h0 = initial_state;
    p.cu_seqlens = cu_seqlens;
    p.o = o; p.ht = final_state;
    return to_status(launch_fused_recurrent(p, stream));
}

kda_status kda_gate_chunk_cumsum(const kda_fwd_desc *d, const void *g, const float *A_log,
                                 const float *dt_bias, const int64_t *cu_seqlens, float *g_act,
                                 float *g_cum_log2, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
    Params p;
    kda_status st = check_desc(d, p);
    if (st != KDA_OK) return st;
    const bool tokens = (int64_t)d->B * d->T > 0;
    if (tokens && (!g || !g_cum_log2)) return KDA_ERR_NULL_POINTER;
    if ((d->flags & KDA_GATE_IN_KERNEL) && !(d->flags & KDA_HAS_LOWER_BOUND) && !A_log)
        return KDA_ERR_MISSING_A_LOG;
    if ((cu_seqlens == nullptr) != (d->cu_seqlens_host == nullptr)) return KDA_ERR_VARLEN;
    const WorkspaceLayout L = workspace_layout(p.N, p.total_chunks, 0, p.K, p.V, p.C, 4);
    if (!workspace || workspace_bytes < L.plan_bytes) return KDA_ERR_WORKSPACE;
    p.g = g; p.A_log = A_log; p.dt_bias = dt_bias; p.cu_seqlens = cu_seqlens;
    p.g_act = g_act; p.g_cum = g_cum_log2;
    bind_workspace(p, workspace, L);
    hipError_t e = launch_plan(p, stream);
    if (e == hipSuccess) e = launch_gate_cumsum(p, stream);
    return to_status(e);
}

}  // extern "C"

// ---------------------------------------------------------------- backward
namespace {

// A second stream per device, created on first use, for work that overlaps the caller's
// stream inside one call: the bf16 backward's operand preparation (which needs only the
// forward's intermediates) beside the latency-bound recurrence, which occupies half the
// CUs.  `ev` receives chunk_fwd_run's stage events, `done` marks the side work; `mu` is
// held from the first event record to the caller stream's wait, so concurrent calls on
// one device cannot interleave their records and waits.  Default stream priority.
constexpr int kMaxDevices = 64;
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t ev[kNumStages + 1] = {};
    hipEvent_t done = nullptr;
    std::mutex mu;
};
SideStream g_side[kMaxDevices];
std::mutex g_side_init;

hipError_t side_stream(SideStream **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    SideStream &ss = g_side[dev];
    std::lock_guard<std::mutex> lk(g_side_init);
    if (!ss.s) {
        hipStream_t st = nullptr;
        hipEvent_t ev[kNumStages + 2] = {};
        e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
        for (int i = 0; i < kNumStages + 2 && e == hipSuccess; ++i) e = hipEventCreateWithFlags(&ev[i], hipEventDisableTiming);
        if (e != hipSuccess) {  // nothing half-made is kept
            for (hipEvent_t x : ev)
                if (x) hipEventDestroy(x);
            if (st) hipStreamDestroy(st);
            return e;
        }
        for (int i = 0; i <= kNumStages; ++i) ss.ev[i] = ev[i];
        ss.done = ev[kNumStages + 1];
        ss.s = st;
    }
    *out = &ss;
    return hipSuccess;
}

// The side stream runs the operand preparation once the caller's stream has passed the
// forward's intra stage (ss.ev[2], recorded by chunk_fwd_run before the recurrence); the
// caller's stream then waits for it.
hipError_t prep_beside_recurrence(SideStream &ss, const BwdChunkParams &P, hipStream_t stream) {
    hipError_t e = hipStreamWaitEvent(ss.s, ss.ev[2], 0);
    if (e == hipSuccess) e = launch_bwd_prep(P, ss.s);
    if (e == hipSuccess) e = hipEventRecord(ss.done, ss.s);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, ss.done, 0);
    return e;
}

struct BwdLayout {
    size_t off_states, off_o, off_pdq, off_pdk, off_pdg, off_pdb, off_sstate, off_sw, off_da, off_tq, off_tk,
        off_ta, off_tb, off_param, off_du, off_dh, off_cparam, off_rpack, off_ppack, off_doq, total;
    int nslices;
};

// After the forward's own workspace: the chunk-start states, the forward output (not
// returned), the per-value-head partial sums of dq and dk, and the scratch of the form
// in use.  The chunked form keeps dU, the per-chunk state gradients, the per-chunk
// dt_bias / A_log sums and (bf16) the reverse recurrence's operands; the token-level form
// one partial sum per 16-column slice of V of dq, dk, dg, dbeta plus its per-token
// operands and token-state scratch.
BwdLayout bwd_layout(const Params &p, size_t fwd_bytes, bool chunked) {
    BwdLayout L{};
    const size_t Ttot = (size_t)p.B * p.T, f = sizeof(float);
    const size_t ns = chunked ? 1 : (size_t)bwd_slices(p.V);
    const size_t slots = (size_t)p.total_chunks * p.HV;
    L.nslices = (int)ns;
    size_t off = align256(fwd_bytes);
    L.off_states = off;
    off = align256(off + f * slots * p.K * p.V);
    L.off_o = off;
    off = align256(off + (p.qkv_bf16 ? 2 : 4) * Ttot * p.HV * p.V);
    L.off_pdq = off;
    off = align256(off + f * ns * Ttot * p.HV * p.K);
    L.off_pdk = off;
    off = align256(off + f * ns * Ttot * p.HV * p.K);
    if (chunked) {
        // dg and dbeta are final from the per-chunk kernel; dt_bias and A_log come from
        // per-chunk sums
        L.off_du = off;
        off = align256(off + f * slots * p.C * p.V);
        L.off_dh = off;
        off = align256(off + f * slots * p.K * p.V);
        L.off_cparam = off;
        off = align256(off + f * slots * (p.K + 1));
        if (p.qkv_bf16) {  // the reverse recurrence's transposed operands and dO (bf16)
            L.off_rpack = off;
            off = align256(off + 2 * slots * 2 * p.C * p.K);
            L.off_ppack = off;
            off = align256(off + 2 * slots * ((size_t)p.C * p.C + (size_t)p.K * p.C));
            L.off_doq = off;
            off = align256(off + 2 * slots * p.V * p.C);
        }
    } else {
        L.off_pdg = off;
        off = align256(off + f * ns * Ttot * p.HV * p.K);
        L.off_pdb = off;
        off = align256(off + f * ns * Ttot * p.HV);
        L.off_da = off;
        off = align256(off + f * Ttot * p.HV * p.K);
        L.off_param = off;
        off = align256(off + f * bwd_param_scratch_floats(p.HV, p.K));
        const size_t scr = bwd_seq_scratch_floats(p.N, p.HV, p.K, p.V, p.C);
        L.off_sstate = off;
        off = align256(off + f * scr);
        L.off_sw = L.off_sstate + f * bwd_seq_state_floats(p.N, p.HV, p.K, p.V, p.C);
        L.off_tq = off;
        off = align256(off + f * Ttot * p.HV * p.K);
        L.off_tk = off;
        off = align256(off + f * Ttot * p.HV * p.K);
        L.off_ta = off;
        off = align256(off + f * Ttot * p.HV * p.K);
        L.off_tb = off;
        off = align256(off + f * Ttot * p.HV);
    }
    L.total = off;
    return L;
}

kda_status bwd_check(const kda_fwd_desc *d, Params &p) {
    kda_status st = check_desc(d, p);
    if (st != KDA_OK) return st;
    if (d->flags & KDA_TRANSPOSE_STATE) return KDA_ERR_UNSUPPORTED;  // [K][V] states only
    return KDA_OK;
}

kda_status bwd_workspace(const kda_fwd_desc *d, size_t *bytes, bool tokenwise) {
    Params p;
    kda_status st = bwd_check(d, p);
    if (st != KDA_OK) return st;
    if (!bytes) return KDA_ERR_NULL_POINTER;
    const size_t fwd = workspace_layout(p.N, p.total_chunks, p.HV, p.K, p.V, p.C, p.qkv_bf16 ? 2 : 4).total_bytes;
    *bytes = bwd_layout(p, fwd, !tokenwise && bwd_chunk_fits(p.K)).total;
    return KDA_OK;
}

kda_status bwd_run(const kda_fwd_desc *d, const void *q, const void *k, const void *v, const void *g,
                   const void *beta, const float *A_log, const float *dt_bias, const float *initial_state,
                   const int64_t *cu_seqlens, const void *dout, const float *dht, float *dq, float *dk, float *dv,
                   float *dg, float *dbeta, float *dA_log, float *ddt_bias, float *dh0, void *workspace,
                   size_t workspace_bytes, hipStream_t stream, bool tokenwise, bool saved) {
    Params p;
    kda_status st = bwd_check(d, p);
    if (st != KDA_OK) return st;
    const bool tokens = (int64_t)d->B * d->T > 0;
    if (tokens && (!q || !k || !v || !g || !beta || !dout || !dq || !dk || !dv || !dg || !dbeta))
        return KDA_ERR_NULL_POINTER;
    if ((d->flags & KDA_GATE_IN_KERNEL) && !(d->flags & KDA_HAS_LOWER_BOUND) && !A_log)
        return KDA_ERR_MISSING_A_LOG;
    if ((cu_seqlens == nullptr) != (d->cu_seqlens_host == nullptr)) return KDA_ERR_VARLEN;
    const bool chunked = !tokenwise && bwd_chunk_fits(p.K);
    const WorkspaceLayout FL = workspace_layout(p.N, p.total_chunks, p.HV, p.K, p.V, p.C, p.qkv_bf16 ? 2 : 4);
    const BwdLayout L = bwd_layout(p, FL.total_bytes, chunked);
    if (!workspace || workspace_bytes < L.total) return KDA_ERR_WORKSPACE;
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    float *states = reinterpret_cast<float *>(ws + L.off_states);

    // backward steps 1-2: the forward with the state each chunk starts from (its output o
    // is not needed); its per-chunk intermediates stay in the workspace.  `saved`: a
    // kda_chunk_fwd_save call left them there already.
    // bf16 chunked form: the operand preparation runs on the side stream beside the
    // forward's recurrence.
    const bool beside = chunked && p.qkv_bf16 && !saved && p.total_chunks > 0;
    SideStream *ss = nullptr;
    std::unique_lock<std::mutex> side_lock;
    if (beside) {
        const hipError_t e = side_stream(&ss);
        if (e != hipSuccess) return to_status(e);
        side_lock = std::unique_lock<std::mutex>(ss->mu);
    }
    if (!saved) {
        kda_fwd_desc fd = *d;
        fd.flags &= ~(uint32_t)KDA_OUTPUT_FINAL_STATE;
        st = chunk_fwd_run(&fd, q, k, v, g, beta, A_log, dt_bias, initial_state, cu_seqlens, ws + L.off_o, nullptr,
                           true, states, workspace, FL.total_bytes, stream, beside ? ss->ev : nullptr,
                           chunked && p.qkv_bf16, true);
        if (st != KDA_OK) return st;
    }

    BwdParams b{};
    b.N = p.N; b.T = p.T; b.H = p.H; b.HV = p.HV; b.K = p.K; b.V = p.V; b.C = p.C;
    b.Ttot = (int64_t)p.B * p.T;
    b.gate_mode = p.gate_mode; b.beta_mode = p.beta_mode; b.qk_l2norm = p.qk_l2norm;
    b.qkv_bf16 = p.qkv_bf16; b.g_bf16 = p.g_bf16; b.beta_bf16 = p.beta_bf16;
    b.scale = d->scale;
    b.lower_bound = (d->flags & KDA_HAS_LOWER_BOUND) ? d->lower_bound : 0.f;
    b.q = q; b.k = k; b.v = v; b.g = g; b.beta = beta; b.dout = dout;
    b.A_log = A_log; b.dt_bias = dt_bias; b.dht = dht; b.cu_seqlens = cu_seqlens; b.states = states;
    b.dq = dq; b.dk = dk; b.dv = dv; b.dg = dg; b.dbeta = dbeta;
    b.dA_log = A_log ? dA_log : nullptr;
    b.ddt_bias = dt_bias ? ddt_bias : nullptr;
    b.dh0 = dh0;
    b.nslices = L.nslices;
    b.p_dq = reinterpret_cast<float *>(ws + L.off_pdq);
    b.p_dk = reinterpret_cast<float *>(ws + L.off_pdk);
    if (!chunked) {
        b.p_dg = reinterpret_cast<float *>(ws + L.off_pdg);
        b.p_db = reinterpret_cast<float *>(ws + L.off_pdb);
        b.scr_da = reinterpret_cast<float *>(ws + L.off_da);
        b.scr_param = reinterpret_cast<float *>(ws + L.off_param);
        b.scr_state = reinterpret_cast<float *>(ws + L.off_sstate);
        b.scr_w = reinterpret_cast<float *>(ws + L.off_sw);
        b.t_q = reinterpret_cast<float *>(ws + L.off_tq);
        b.t_k = reinterpret_cast<float *>(ws + L.off_tk);
        b.t_a = reinterpret_cast<float *>(ws + L.off_ta);
        b.t_b = reinterpret_cast<float *>(ws + L.off_tb);
        return to_status(launch_backward(b, stream));
    }
    // backward steps 3-7: the reverse chunk recurrence, the per-chunk gradients, then the
    // chain rules of the input transforms
    BwdChunkParams P{};
    P.f = p;
    P.f.q = q; P.f.k = k; P.f.v = v; P.f.g = g; P.f.beta = beta;
    P.f.A_log = A_log; P.f.dt_bias = dt_bias; P.f.h0 = initial_state; P.f.cu_seqlens = cu_seqlens;
    bind_workspace(P.f, workspace, FL);
    P.b = b;
    P.dU = reinterpret_cast<float *>(ws + L.off_du);
    P.dh = reinterpret_cast<float *>(ws + L.off_dh);
    P.cparam = reinterpret_cast<float *>(ws + L.off_cparam);
    if (p.qkv_bf16) {
        P.rpack = reinterpret_cast<uint16_t *>(ws + L.off_rpack);
        P.ppack = reinterpret_cast<uint16_t *>(ws + L.off_ppack);
        P.doq = reinterpret_cast<uint16_t *>(ws + L.off_doq);
    }
    if (beside) {
        const hipError_t e0 = prep_beside_recurrence(*ss, P, stream);
        side_lock.unlock();
        if (e0 != hipSuccess) return to_status(e0);
        P.prep_done = 1;
    }
    hipError_t e = launch_bwd_dhu(P, stream);
    if (e == hipSuccess) e = launch_bwd_local(P, stream);
    if (e == hipSuccess) e = launch_bwd_finish_chunked(P, stream);
    return to_status(e);
}

}  // namespace

extern "C" {

kda_status kda_chunk_bwd_workspace_size(const kda_fwd_desc *d, size_t *bytes) { return bwd_workspace(d, bytes, false); }

kda_status kda_chunk_fwd_save(const kda_fwd_desc *d, const void *q, const void *k, const void *v, const void *g,
                              const void *beta, const float *A_log, const float *dt_bias, const float *initial_state,
                              const int64_t *cu_seqlens, void *o, float *final_state, void *workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    Params p;
    kda_status st = bwd_check(d, p);
    if (st != KDA_OK) return st;
    const bool chunked = bwd_chunk_fits(p.K);
    const WorkspaceLayout FL = workspace_layout(p.N, p.total_chunks, p.HV, p.K, p.V, p.C, p.qkv_bf16 ? 2 : 4);
    const BwdLayout L = bwd_layout(p, FL.total_bytes, chunked);
    if (!workspace || workspace_bytes < L.total) return KDA_ERR_WORKSPACE;
    // the states and intermediates exactly as kda_chunk_bwd's recompute leaves them, and o
    float *states = reinterpret_cast<float *>(static_cast<unsigned char *>(workspace) + L.off_states);
    return chunk_fwd_run(d, q, k, v, g, beta, A_log, dt_bias, initial_state, cu_seqlens, o, final_state, true, states,
                         workspace, FL.total_bytes, stream, nullptr, chunked && p.qkv_bf16, false);
}

kda_status kda_chunk_bwd_saved(const kda_fwd_desc *d, const void *q, const void *k, const void *v, const void *g,
                               const void *beta, const float *A_log, const float *dt_bias,
                               const float *initial_state, const int64_t *cu_seqlens, const void *dout,
                               const float *dht, float *dq, float *dk, float *dv, float *dg, float *dbeta,
                               float *dA_log, float *ddt_bias, float *dh0, void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    return bwd_run(d, q, k, v, g, beta, A_log, dt_bias, initial_state, cu_seqlens, dout, dht, dq, dk, dv, dg, dbeta,
                   dA_log, ddt_bias, dh0, workspace, workspace_bytes, stream, false, true);
}

kda_status kda_chunk_bwd(const kda_fwd_desc *d, const void *q, const void *k, const void *v, const void *g,
                         const void *beta, const float *A_log, const float *dt_bias, const float *initial_state,
                         const int64_t *cu_seqlens, const void *dout, const float *dht, float *dq, float *dk,
                         float *dv, float *dg, float *dbeta, float *dA_log, float *ddt_bias, float *dh0,
                         void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return bwd_run(d, q, k, v, g, beta, A_log, dt_bias, initial_state, cu_seqlens, dout, dht, dq, dk, dv, dg, dbeta,
                   dA_log, ddt_bias, dh0, workspace, workspace_bytes, stream, false, false);
}

kda_status kda_chunk_bwd_tokenwise_workspace_size(const kda_fwd_desc *d, size_t *bytes) {
    return bwd_workspace(d, bytes, true);
}

kda_status kda_chunk_bwd_tokenwise(const kda_fwd_desc *d, const void *q, const void *k, const void *v, const void *g,
                                   const void *beta, const float *A_log, const float *dt_bias,
                                   const float *initial_state, const int64_t *cu_seqlens, const void *dout,
                                   const float *dht, float *dq, float *dk, float *dv, float *dg, float *dbeta,
                                   float *dA_log, float *ddt_bias, float *dh0, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
    return bwd_run(d, q, k, v, g, beta, A_log, dt_bias, initial_state, cu_seqlens, dout, dht, dq, dk, dv, dg, dbeta,
                   dA_log, ddt_bias, dh0, workspace, workspace_bytes, stream, true, false);
}

}  // extern "C"
