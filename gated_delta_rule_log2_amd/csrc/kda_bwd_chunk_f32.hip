// Chunked backward kernels for fp32 q/k/v (fp32 intermediates and matrix cores),
// chunk 32 and 64, K = 32..128.
#include "kda_bwd_chunk.h"

namespace kda {
hipError_t launch_bwd_dhu_f32(const BwdChunkParams &p, hipStream_t s) { return launch_bwd_dhu_c<float>(p, s); }
hipError_t launch_bwd_local_f32(const BwdChunkParams &p, hipStream_t s) { return launch_bwd_local_c<float>(p, s); }
bool bwd_chunk_fits(int K) { return K <= 128; }
hipError_t launch_bwd_dhu_bf16(const BwdChunkParams &p, hipStream_t s);
hipError_t launch_bwd_local_bf16(const BwdChunkParams &p, hipStream_t s);
hipError_t launch_bwd_prep_bf16(const BwdChunkParams &p, hipStream_t s);
hipError_t launch_bwd_prep(const BwdChunkParams &p, hipStream_t s) {
    return p.f.qkv_bf16 ? launch_bwd_prep_bf16(p, s) : hipSuccess;
}
hipError_t launch_bwd_dhu(const BwdChunkParams &p, hipStream_t s) {
    return p.f.qkv_bf16 ? launch_bwd_dhu_bf16(p, s) : launch_bwd_dhu_f32(p, s);
}
hipError_t launch_bwd_local(const BwdChunkParams &p, hipStream_t s) {
    return p.f.qkv_bf16 ? launch_bwd_local_bf16(p, s) : launch_bwd_local_f32(p, s);
}
}  // namespace kda
