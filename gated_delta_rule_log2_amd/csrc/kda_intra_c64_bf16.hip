// Intra-chunk kernels for chunk size 64, bf16 storage (one translation unit per
// combination so the exact-K instantiations compile in parallel).
#include "kda_intra_bf16.h"

namespace kda {
hipError_t launch_intra_c64_bf16(const Params &p, hipStream_t s) { return launch_intra_bf16_c<64>(p, s); }
size_t intra_lds_c64_bf16(int K, int V) { return intra_bf16_lds<64>(K, V); }
}  // namespace kda
