// Chunked backward kernels for bf16 q/k/v (bf16 intermediates: bf16 matrix-core
// operands with fp32 accumulation), chunk 32 and 64, K = 32..128.
#include "kda_bwd_chunk.h"

namespace kda {
hipError_t launch_bwd_dhu_bf16(const BwdChunkParams &p, hipStream_t s) { return launch_bwd_dhu_c<uint16_t>(p, s); }
hipError_t launch_bwd_local_bf16(const BwdChunkParams &p, hipStream_t s) { return launch_bwd_local_c<uint16_t>(p, s); }
}  // namespace kda
