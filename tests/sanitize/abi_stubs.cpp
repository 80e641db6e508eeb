// Stand-ins for the GPU side of libkda.so, so that the host code of kda_abi.cpp (its
// argument checks, workspace layout and launch sequencing) can be built with the host
// compiler under AddressSanitizer and UndefinedBehaviorSanitizer.  No launcher is ever
// reached with real device pointers: each stand-in records that it was called and
// returns success.
#include <hip/hip_runtime_api.h>

#include "../../gated_delta_rule_log2_amd/csrc/kda_backward.h"
#include "../../gated_delta_rule_log2_amd/csrc/kda_internal.h"

int g_stub_launches = 0;

namespace kda {
// LDS bytes of the intra kernels: only the fp32 K = V = 256 case is over a CU's 160 KB.
size_t intra_lds_bytes(int C, int K, int V, bool bf16) { return (!bf16 && K == 256 && V == 256) ? (200u << 10) : (48u << 10); }
hipError_t launch_plan(const Params &, hipStream_t) { ++g_stub_launches; return hipSuccess; }
hipError_t launch_gate_cumsum(const Params &, hipStream_t) { ++g_stub_launches; return hipSuccess; }
hipError_t launch_intra(const Params &, hipStream_t) { ++g_stub_launches; return hipSuccess; }
hipError_t launch_recurrence(const Params &, hipStream_t) { ++g_stub_launches; return hipSuccess; }
hipError_t launch_fused_recurrent(const Params &, hipStream_t) { ++g_stub_launches; return hipSuccess; }
hipError_t launch_backward(const BwdParams &, hipStream_t) { ++g_stub_launches; return hipSuccess; }
hipError_t launch_bwd_dhu(const BwdChunkParams &, hipStream_t) { ++g_stub_launches; return hipSuccess; }
hipError_t launch_bwd_prep(const BwdChunkParams &, hipStream_t) { ++g_stub_launches; return hipSuccess; }
hipError_t launch_bwd_local(const BwdChunkParams &, hipStream_t) { ++g_stub_launches; return hipSuccess; }
hipError_t launch_bwd_finish(const BwdParams &, hipStream_t) { ++g_stub_launches; return hipSuccess; }
hipError_t launch_bwd_finish_chunked(const BwdChunkParams &, hipStream_t) { ++g_stub_launches; return hipSuccess; }
bool bwd_chunk_fits(int K) { return K <= 128; }
}  // namespace kda

namespace kda {
// Scratch sizes of the backward (any consistent sizes serve: no memory is touched).
int bwd_slices(int V) { return V / 16 > 0 ? V / 16 : 1; }
size_t bwd_seq_state_floats(int N, int HV, int K, int V, int C) { return (size_t)N * HV * V * C * K / 8; }
size_t bwd_seq_scratch_floats(int N, int HV, int K, int V, int C) { return 2 * bwd_seq_state_floats(N, HV, K, V, C); }
size_t bwd_param_scratch_floats(int HV, int K) { return (size_t)HV * 64 * (K + 1); }
}  // namespace kda
