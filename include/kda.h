/*
 * kda.h -- C ABI of the MI355X (gfx950) chunk-parallel Kimi Delta Attention
 * (KDA) forward pass.
 *
 * Sources (web pages; cited by title and section):
 *   [ENG]   "flash-linear-attention KDA 内核工程实践：门控模式、safe_gate 数值稳定性
 *            与 chunk intra/inter 双路径解析" (dpshk.com news 4765615)
 *   [NOTES] "Reading Notes: Implementation Notes for KDA in FLA"
 *            (mzeromiko.github.io, kimi_linear / kda-fla)
 *   [FKDA]  "FlashKDA gate偏置加載路徑完整解析如何讀取A_log與dt_bias"
 *            (m.czchanglian.com news 37351)
 *
 * The method.  For each sequence and value head hv (qk head h = hv / (HV/H)),
 * with per-key-channel log decays g'_t (natural log), betas b_t and keys,
 * values and queries k_t, v_t, q_t (q already multiplied by `scale`):
 *     S_t = (I - b_t k_t k_t^T) Diag(exp g'_t) S_{t-1} + b_t k_t v_t^T
 *     o_t = S_t^T q_t
 * computed chunk-parallel as in [NOTES] "forward" steps 1-5: a base-2
 * chunk-local cumulative gate, the intra-chunk matrices Aqk and
 * (I + Akk0)^-1 from 16-token sub-chunks, the WY factors W and U, the
 * inter-chunk state recurrence and the chunk output.
 *
 * Conventions for every entry point
 *   - Every tensor pointer is DEVICE memory owned by the caller, row-major
 *     and contiguous, unless it is documented as host memory.  The library
 *     keeps no pointer after it returns and never allocates device memory.
 *   - Work is enqueued on `stream` and runs asynchronously; nothing is
 *     synchronised on the host.  Inputs must stay valid until the stream has
 *     executed the work.
 *   - All argument checks run on the host before anything is enqueued:
 *     descriptor checks first (in the order of kda_status below), then the
 *     pointer checks, then the workspace size.  On any error nothing is written.
 *   - KDA_ERR_HIP is returned when a kernel launch fails; the stream's work up
 *     to that point may then be incomplete.
 *   - Calls that share a workspace on different streams race.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 4

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL_POINTER = 1,   /* a required pointer (descriptor, tensor, host cu_seqlens) is NULL */
    KDA_ERR_SHAPE = 2,          /* a size is negative or zero where it must be positive, or too large */
    KDA_ERR_CHUNK_SIZE = 3,     /* chunk_size not 32 or 64 ([ENG] §2.1) */
    KDA_ERR_HEAD_DIM = 4,       /* K > 256 ([ENG] §2.1) */
    KDA_ERR_UNSUPPORTED = 5,    /* build limit: K or V not a multiple of 32, V > 256, fp32 q/k/v with
                                   K = V = 256 (over one CU's 160 KB of LDS), or an unknown flag bit */
    KDA_ERR_GVA = 6,            /* HV is not a multiple of H ([ENG] §2.1) */
    KDA_ERR_MISSING_A_LOG = 7,  /* in-kernel gate without lower bound needs A_log ([ENG] §2.1) */
    KDA_ERR_LOWER_BOUND = 8,    /* safe gate needs -5 <= lower_bound < 0; any bound must be < 0 ([ENG] §2.1) */
    KDA_ERR_NEG_EIGVAL = 9,     /* allow_neg_eigval needs the in-kernel beta sigmoid ([ENG] §2.1) */
    KDA_ERR_VARLEN = 10,        /* cu_seqlens with B != 1, or host offsets not 0..T non-decreasing */
    KDA_ERR_DTYPE = 11,         /* a dtype code is not KDA_DTYPE_FP32 or KDA_DTYPE_BF16 */
    KDA_ERR_WORKSPACE = 12,     /* workspace NULL or smaller than the queried size */
    KDA_ERR_HIP = 13            /* a HIP runtime call or kernel launch failed */
} kda_status;

typedef enum kda_dtype {
    KDA_DTYPE_FP32 = 0,
    KDA_DTYPE_BF16 = 1
} kda_dtype;

/* Flags of kda_fwd_desc.flags (the keyword switches of chunk_kda, [ENG] §2, §2.2). */
enum {
    KDA_GATE_IN_KERNEL = 1u << 0,     /* g is the raw gate input; activation is fused ([ENG] §2 contract 2) */
    KDA_SAFE_GATE = 1u << 1,          /* caller promises g' in [lower_bound, 0), lower_bound in [-5, 0) ([ENG] §3) */
    KDA_HAS_LOWER_BOUND = 1u << 2,    /* the gate is lower_bound * sigmoid(...) ([ENG] §2) */
    KDA_QK_L2NORM = 1u << 3,          /* q, k are L2-normalised per (token, head) in the kernel */
    KDA_BETA_SIGMOID = 1u << 4,       /* beta holds logits; b = sigmoid(beta) */
    KDA_ALLOW_NEG_EIGVAL = 1u << 5,   /* with BETA_SIGMOID: b = 2 * sigmoid(beta), in [0, 2) */
    KDA_OUTPUT_FINAL_STATE = 1u << 6, /* write final_state */
    KDA_TRANSPOSE_STATE = 1u << 7     /* every state tensor stored [V][K] per (sequence, value head)
                                         instead of [K][V] ("state_v_first", [ENG] §2.2) */
};

/*
 * Problem descriptor (host memory, read during the call only).
 *   B, T         batch and tokens per batch row.  With cu_seqlens B must be 1 and
 *                the T tokens hold num_seqs packed sequences.
 *   H, HV        qk heads and value heads (GVA: HV % H == 0).
 *   K, V         key and value head dims.
 *   chunk_size   32 or 64.
 *   num_seqs     number of sequences: B without cu_seqlens, len(cu_seqlens) - 1 with.
 *   cu_seqlens_host  host copy of the int64 offsets [num_seqs + 1] (required with
 *                cu_seqlens; it sizes the launch, and must equal the device copy).
 *   qkv_dtype    dtype of q, k, v and o.  g_dtype, beta_dtype: dtypes of g and beta.
 *   scale        multiplies q (after the L2 normalisation when that is on).
 *   lower_bound  natural-log lower bound of the gate (used with KDA_HAS_LOWER_BOUND).
 *   flags        KDA_* flags above.
 */
typedef struct kda_fwd_desc {
    int32_t B, T, H, HV, K, V;
    int32_t chunk_size;
    int32_t num_seqs;
    const int64_t *cu_seqlens_host;
    int32_t qkv_dtype, g_dtype, beta_dtype; /* kda_dtype codes */
    float scale;
    float lower_bound;
    uint32_t flags;
} kda_fwd_desc;

/* ABI version of the loaded library (KDA_ABI_VERSION it was built with). */
int kda_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char *kda_status_string(kda_status s);

/*
 * Bytes of device workspace kda_chunk_fwd needs for this descriptor.  The caller
 * allocates the workspace and passes it in, as FlashKDA's Python layer allocates the
 * workspace its kernels use ("FlashKDA gate偏置加載路徑完整解析…", §二 第1段); the
 * library itself never allocates.  Runs the same descriptor checks as kda_chunk_fwd
 * (no device pointers involved) and writes *bytes only on KDA_OK.  Host only; no HIP
 * call.
 */
kda_status kda_chunk_fwd_workspace_size(const kda_fwd_desc *d, size_t *bytes);

/*
 * chunk_kda forward ([NOTES] "forward", steps 1-5; contract checks of [ENG] §2.1).
 *
 *   q, k        [B, T, H, K]   qkv_dtype
 *   v           [B, T, HV, V]  qkv_dtype
 *   g           [B, T, HV, K]  g_dtype: raw gate input with KDA_GATE_IN_KERNEL, else the
 *               natural-log decay g' itself (pre-gated, must be <= 0)
 *   beta        [B, T, HV]     beta_dtype: logits with KDA_BETA_SIGMOID, else b itself
 *   A_log       [HV] fp32 or NULL (required for the in-kernel softplus gate;
 *               optional with a lower bound, NULL meaning exp(A_log) = 1)
 *   dt_bias     [HV * K] fp32 or NULL (0), added to g before the activation
 *   initial_state [num_seqs, HV, K, V] fp32 or NULL (zeros); state rows are keys
 *               ([num_seqs, HV, V, K] with KDA_TRANSPOSE_STATE, as final_state)
 *   cu_seqlens  [num_seqs + 1] int64 device copy of the packed offsets, or NULL
 *   o           [B, T, HV, V]  qkv_dtype, fully overwritten
 *   final_state [num_seqs, HV, K, V] fp32, written iff KDA_OUTPUT_FINAL_STATE
 *               (then it must not be NULL); may alias initial_state
 *   workspace   device scratch of at least kda_chunk_fwd_workspace_size bytes,
 *               256-byte aligned; its contents on entry do not matter
 *
 * In-kernel gate ([ENG] §2; order of [FKDA] §三), natural log, x = g + dt_bias:
 *   lower bound:  g' = lower_bound * sigmoid(exp(A_log[hv]) * x)
 *   otherwise:    g' = -exp(A_log[hv]) * softplus(x)
 */
kda_status kda_chunk_fwd(const kda_fwd_desc *d,
                         const void *q, const void *k, const void *v, const void *g,
                         const void *beta, const float *A_log, const float *dt_bias,
                         const float *initial_state, const int64_t *cu_seqlens,
                         void *o, float *final_state,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_chunk_fwd that also returns the intermediate states: the state each chunk
 * starts from, for every sequence and value head (the inference-only
 * "return_intermediate_states" of [ENG] §2.2, the h of [NOTES] forward step 4,
 * S_[t-1] before the chunk's update), for serving engines that keep per-chunk
 * states.
 *   states      [total_chunks, HV, K, V] fp32 ([.., V, K] with KDA_TRANSPOSE_STATE),
 *               fully overwritten.  Chunks start at every sequence start and then
 *               every chunk_size tokens; sequence n's chunks follow those of
 *               sequences 0..n-1, so total_chunks = sum over sequences of
 *               ceil(length / chunk_size) (B * ceil(T / chunk_size) without
 *               cu_seqlens).  A sequence's first entry is its initial state (or
 *               zeros); a sequence of length 0 has none.
 * Everything else (arguments, workspace, checks, errors) is that of kda_chunk_fwd,
 * plus KDA_ERR_NULL_POINTER when states is NULL and there are chunks.  o and
 * final_state are bit for bit those of kda_chunk_fwd.
 */
kda_status kda_chunk_fwd_states(const kda_fwd_desc *d,
                                const void *q, const void *k, const void *v, const void *g,
                                const void *beta, const float *A_log, const float *dt_bias,
                                const float *initial_state, const int64_t *cu_seqlens,
                                void *o, float *final_state, float *states,
                                void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fused_recurrent_kda forward: the token-by-token form of the same operator, the
 * public entry for autoregressive decoding ("flash-linear-attention KDA 内核工程实践…",
 * §1).  Per token, with the state stored [K][V]:
 *   S <- Diag(exp(g')) S;  u = S^T k^;  S <- S + beta k^ (v - u)^T;  o = S^T q^
 * ("Reading Notes: Implementation Notes for KDA in FLA", forward), g' the activated
 * gate of kda_chunk_fwd, q^ = scale * q (L2-normalised first with
 * KDA_QK_L2NORM), k^ = k (likewise normalised).
 *
 * Arguments, layouts, flags and error codes are those of kda_chunk_fwd; there is no
 * workspace.  The descriptor passes the same checks (so chunk_size must still be 32
 * or 64 although the token recurrence does not use it, and KDA_SAFE_GATE still
 * validates the lower bound).  Each (sequence, value head) keeps its state on chip
 * for the whole sequence, so the cost grows with T token by token: meant for
 * decoding steps and short prompts, not for long prefill (use kda_chunk_fwd there).
 */
kda_status kda_fused_recurrent_fwd(const kda_fwd_desc *d,
                                   const void *q, const void *k, const void *v, const void *g,
                                   const void *beta, const float *A_log, const float *dt_bias,
                                   const float *initial_state, const int64_t *cu_seqlens,
                                   void *o, float *final_state, hipStream_t stream);

/*
 * chunk_kda backward: the gradients of L = <do, o> + <dht, final_state> with respect
 * to every input of kda_chunk_fwd ("Reading Notes: Implementation Notes for KDA in
 * FLA", backward; the same operator, descriptor and input contract as kda_chunk_fwd),
 * in the chunked form of that section's steps 1-7: the forward is recomputed with the
 * state each chunk starts from (steps 1-2), a reverse recurrence over chunks carries the
 * state gradient and gives dU = dL/dV_new per chunk (step 4), and one pass per (chunk,
 * value head) forms dAqk (step 3), the WY chain (step 5), the intra-chunk terms with the
 * gate offsets of the forward (step 6) and the suffix sum that turns cumulative-gate
 * gradients into gate gradients (step 7).  For K > 128 the token-level form of
 * kda_chunk_bwd_tokenwise runs instead.  KDA_TRANSPOSE_STATE is refused
 * (KDA_ERR_UNSUPPORTED).
 *   dout     [B*T, HV, V]  dtype qkv_dtype (the dtype of o); required when B*T > 0
 *   dht      [N, HV, K, V] fp32 gradient of final_state, or NULL (zero)
 * Outputs, all fp32, fully overwritten, same layouts as the inputs:
 *   dq, dk   [B*T, H, K]   (summed over the value heads of each GVA group)
 *   dv       [B*T, HV, V];  dg [B*T, HV, K] (w.r.t. the g given, natural-log units,
 *            through the activation when KDA_GATE_IN_KERNEL);  dbeta [B*T, HV]
 *            (w.r.t. the beta given, through the sigmoid when KDA_BETA_SIGMOID)
 *   dA_log   [HV]     written when both A_log and dA_log are non-NULL
 *   ddt_bias [HV, K]  written when both dt_bias and ddt_bias are non-NULL
 *   dh0      [N, HV, K, V] gradient of the initial state, written when non-NULL
 *            (also without initial_state: the gradient at a zero initial state)
 * Workspace: kda_chunk_bwd_workspace_size bytes, device memory owned by the caller,
 * not retained (the forward's workspace, the chunk-start states, dU and the per-chunk
 * state gradients: 1.61 GB at B = 1, T = 8192, HV = 32, K = V = 128, bf16).  Errors: those of
 * kda_chunk_fwd, KDA_ERR_NULL_POINTER for a missing dout or required output when
 * B*T > 0.  Asynchronous on `stream`.  Results do not depend on scheduling (no atomics).
 * With bf16 inputs and K <= 128 part of the work (the reverse recurrence's operand
 * preparation) runs on a second stream of the library on the same device, created on the
 * first call there, forked from and joined back into `stream` with events (so the call
 * stays ordered on `stream`).
 */
kda_status kda_chunk_bwd_workspace_size(const kda_fwd_desc *d, size_t *bytes);
kda_status kda_chunk_bwd(const kda_fwd_desc *d,
                         const void *q, const void *k, const void *v, const void *g,
                         const void *beta, const float *A_log, const float *dt_bias,
                         const float *initial_state, const int64_t *cu_seqlens,
                         const void *dout, const float *dht,
                         float *dq, float *dk, float *dv, float *dg, float *dbeta,
                         float *dA_log, float *ddt_bias, float *dh0,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The forward and backward with recomputation switched off (the disable_recompute
 * switch of chunk_kda and of its backward, "flash-linear-attention KDA 内核工程实践…"
 * §2.2 parameter list; "Reading Notes: Implementation Notes for KDA in FLA", backward
 * signature): the forward keeps more of its intermediates in memory so that the backward
 * need not rebuild them, trading memory for the time of backward steps 1-2.
 *
 * kda_chunk_fwd_save computes o and final_state exactly as kda_chunk_fwd does and, in
 * `workspace`, leaves what kda_chunk_bwd's recompute would put there: the per-chunk
 * intermediates (W, U, Kg, Qg, Aqk, the chunk decay) and the state each chunk starts
 * from.  Arguments as kda_chunk_fwd, but the workspace must hold
 * kda_chunk_bwd_workspace_size bytes (1.61 GB at B = 1, T = 8192, HV = 32, K = V = 128,
 * bf16) and KDA_TRANSPOSE_STATE is refused (KDA_ERR_UNSUPPORTED), as for the backward.
 *
 * kda_chunk_bwd_saved returns the same gradients as kda_chunk_bwd, bit for bit, from a
 * workspace that the last kda_chunk_fwd_save call on it filled for the same descriptor
 * and the same q, k, v, g, beta, A_log, dt_bias, initial_state and cu_seqlens; it skips
 * backward steps 1-2.  Arguments and errors as kda_chunk_bwd.  The library cannot check
 * that the workspace matches: with another workspace the gradients are undefined (no
 * fault: every access stays inside the workspace size that is checked).  Between the
 * calls the caller keeps the workspace (it is owned by the caller and not retained); the
 * backward only reads the saved part and uses the rest as scratch, so one
 * kda_chunk_fwd_save serves any number of kda_chunk_bwd_saved calls (other dout, dht)
 * issued one after another on one stream.  Both asynchronous on `stream`.
 */
kda_status kda_chunk_fwd_save(const kda_fwd_desc *d,
                              const void *q, const void *k, const void *v, const void *g,
                              const void *beta, const float *A_log, const float *dt_bias,
                              const float *initial_state, const int64_t *cu_seqlens,
                              void *o, float *final_state,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);
kda_status kda_chunk_bwd_saved(const kda_fwd_desc *d,
                               const void *q, const void *k, const void *v, const void *g,
                               const void *beta, const float *A_log, const float *dt_bias,
                               const float *initial_state, const int64_t *cu_seqlens,
                               const void *dout, const float *dht,
                               float *dq, float *dk, float *dv, float *dg, float *dbeta,
                               float *dA_log, float *ddt_bias, float *dh0,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The same gradients as kda_chunk_bwd by the token-level form: after the forward with
 * chunk-start states, one workgroup per (sequence, value head, 16-column slice of V)
 * takes the token recurrence's reverse steps from the last token to the first.  Every
 * configuration kda_chunk_fwd accepts except KDA_TRANSPOSE_STATE; slower than the
 * chunked form, and kept as an independent cross-check of it.  Arguments and errors as
 * kda_chunk_bwd; its own workspace size.
 */
kda_status kda_chunk_bwd_tokenwise_workspace_size(const kda_fwd_desc *d, size_t *bytes);
kda_status kda_chunk_bwd_tokenwise(const kda_fwd_desc *d,
                                   const void *q, const void *k, const void *v, const void *g,
                                   const void *beta, const float *A_log, const float *dt_bias,
                                   const float *initial_state, const int64_t *cu_seqlens,
                                   const void *dout, const float *dht,
                                   float *dq, float *dk, float *dv, float *dg, float *dbeta,
                                   float *dA_log, float *ddt_bias, float *dh0,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * For callers that cannot allocate device memory -- code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc: kda_chunk_fwd with its
 * workspace taken from a fixed device array inside the library, so the call itself
 * allocates nothing (no hipMalloc, no hipFree, no allocating library routine).
 *
 * Arguments, layouts, flags, checks and results are those of kda_chunk_fwd, without
 * the workspace arguments; o and final_state are bit for bit those of kda_chunk_fwd.
 *   - The array holds KDA_NOALLOC_SCRATCH_BYTES; a descriptor whose
 *     kda_chunk_fwd_workspace_size exceeds it returns KDA_ERR_WORKSPACE before
 *     anything is enqueued (for K = V = 128, chunk 64: up to 904 (chunk, value head)
 *     pairs per call, e.g. 1 792 tokens at 32 value heads).
 *   - Every GPU the library runs on holds its own copy of the array from module load
 *     until the process ends.  The first call on a device looks up its device address
 *     once (hipGetSymbolAddress, with that device current); KDA_ERR_HIP if that fails.
 *   - `stream` must belong to the current device.
 *   - Every call on one GPU shares that GPU's array, which keeps the last call's
 *     contents (no call reads contents it did not write itself).  Calls on one stream
 *     are ordered and safe; calls that overlap on one GPU (different streams, or
 *     threads without ordering) race.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kda_status kda_chunk_fwd_noalloc(const kda_fwd_desc *d,
                                 const void *q, const void *k, const void *v, const void *g,
                                 const void *beta, const float *A_log, const float *dt_bias,
                                 const float *initial_state, const int64_t *cu_seqlens,
                                 void *o, float *final_state, hipStream_t stream);

/*
 * Stage introspection for profiling.  kda_chunk_fwd enqueues
 * kda_chunk_fwd_stage_count() kernels in order; kda_chunk_fwd_stage_name(i)
 * names stage i (NULL when i is out of range).
 */
int kda_chunk_fwd_stage_count(void);
const char *kda_chunk_fwd_stage_name(int i);

/*
 * kda_chunk_fwd that also records caller-created HIP events on `stream`:
 * stage_events[i] right before stage i and stage_events[count] after the last
 * stage (count = kda_chunk_fwd_stage_count()), so hipEventElapsedTime gives each
 * stage's device time.  stage_events must hold count + 1 valid events; NULL makes
 * this identical to kda_chunk_fwd.  Same checks and errors as kda_chunk_fwd, plus
 * KDA_ERR_HIP if an event record fails.
 */
kda_status kda_chunk_fwd_profiled(const kda_fwd_desc *d,
                                  const void *q, const void *k, const void *v, const void *g,
                                  const void *beta, const float *A_log, const float *dt_bias,
                                  const float *initial_state, const int64_t *cu_seqlens,
                                  void *o, float *final_state,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream,
                                  hipEvent_t *stage_events);

/*
 * Bytes of device workspace kda_gate_chunk_cumsum needs (the chunk plan only).
 * Host only; same descriptor checks as kda_chunk_fwd_workspace_size.
 */
kda_status kda_gate_chunk_cumsum_workspace_size(const kda_fwd_desc *d, size_t *bytes);

/*
 * Gate activation fused with the chunk-local cumulative sum ([ENG] §2, the fused
 * "activation + in-chunk cumsum" kernel; [NOTES] forward step 1), exported on
 * its own for inspection.  The activation is the one device function the bf16 and
 * fp32 intra kernels of kda_chunk_fwd also call (gate_act in kda_gate.h); the
 * cumulative sum here runs over whole chunks, while inside kda_chunk_fwd the bf16
 * kernel scans 16-row sub-chunks and adds the earlier sub-chunks' totals per column.
 *
 *   g           [B, T, HV, K]  g_dtype (raw with KDA_GATE_IN_KERNEL, else pre-gated)
 *   A_log, dt_bias, cu_seqlens  as for kda_chunk_fwd
 *   g_act       [B, T, HV, K] fp32 or NULL: the activated gate g' (natural log)
 *   g_cum_log2  [B, T, HV, K] fp32: log2(e) * inclusive sum of g' from the start of
 *               the row's chunk; chunks restart at every sequence start
 *   workspace   at least kda_gate_chunk_cumsum_workspace_size bytes
 */
kda_status kda_gate_chunk_cumsum(const kda_fwd_desc *d, const void *g, const float *A_log,
                                 const float *dt_bias, const int64_t *cu_seqlens,
                                 float *g_act, float *g_cum_log2,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
