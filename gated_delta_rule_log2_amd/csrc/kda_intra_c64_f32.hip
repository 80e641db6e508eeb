// Intra-chunk kernels for chunk size 64, f32 storage (one translation unit per
// combination so the exact-K instantiations compile in parallel).
#include "kda_intra.h"

namespace kda {
hipError_t launch_intra_c64_f32(const Params &p, hipStream_t s) { return launch_intra_ct<64, float>(p, s); }
size_t intra_lds_c64_f32(int K, int V) { return IntraLds<64, float>::bytes(K, V); }
}  // namespace kda
