// Intra-chunk kernels for chunk size 32, bf16 storage (one translation unit per
// combination so the exact-K instantiations compile in parallel).
#include "kda_intra_bf16.h"

namespace kda {
hipError_t launch_intra_c32_bf16(const Params &p, hipStream_t s) { return launch_intra_bf16_c<32>(p, s); }
size_t intra_lds_c32_bf16(int K, int V) { return intra_bf16_lds<32>(K, V); }
}  // namespace kda
