// Intra-chunk kernels for chunk size 32, f32 storage (one translation unit per
// combination so the exact-K instantiations compile in parallel).
#include "kda_intra.h"

namespace kda {
hipError_t launch_intra_c32_f32(const Params &p, hipStream_t s) { return launch_intra_ct<32, float>(p, s); }
size_t intra_lds_c32_f32(int K, int V) { return IntraLds<32, float>::bytes(K, V); }
}  // namespace kda
