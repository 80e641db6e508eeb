// kda_dispatch.hip -- picks the kernel instantiation for a chunk size and storage type.
#include "kda_internal.h"

namespace kda {
hipError_t launch_intra_c64_bf16(const Params &, hipStream_t);
hipError_t launch_intra_c64_f32(const Params &, hipStream_t);
hipError_t launch_intra_c32_bf16(const Params &, hipStream_t);
hipError_t launch_intra_c32_f32(const Params &, hipStream_t);
hipError_t launch_recur_c64_bf16(const Params &, hipStream_t);
hipError_t launch_recur_c64_f32(const Params &, hipStream_t);
hipError_t launch_recur_c32_bf16(const Params &, hipStream_t);
hipError_t launch_recur_c32_f32(const Params &, hipStream_t);
size_t intra_lds_c64_bf16(int, int);
size_t intra_lds_c64_f32(int, int);
size_t intra_lds_c32_bf16(int, int);
size_t intra_lds_c32_f32(int, int);

size_t intra_lds_bytes(int C, int K, int V, bool bf16) {
    if (C == 64) return bf16 ? intra_lds_c64_bf16(K, V) : intra_lds_c64_f32(K, V);
    return bf16 ? intra_lds_c32_bf16(K, V) : intra_lds_c32_f32(K, V);
}

hipError_t launch_intra(const Params &p, hipStream_t s) {
    if (p.total_chunks == 0) return hipSuccess;
    if (p.C == 64) return p.qkv_bf16 ? launch_intra_c64_bf16(p, s) : launch_intra_c64_f32(p, s);
    return p.qkv_bf16 ? launch_intra_c32_bf16(p, s) : launch_intra_c32_f32(p, s);
}

hipError_t launch_recurrence(const Params &p, hipStream_t s) {
    if (p.N == 0) return hipSuccess;
    if (p.C == 64) return p.qkv_bf16 ? launch_recur_c64_bf16(p, s) : launch_recur_c64_f32(p, s);
    return p.qkv_bf16 ? launch_recur_c32_bf16(p, s) : launch_recur_c32_f32(p, s);
}
}  // namespace kda
