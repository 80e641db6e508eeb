// Recurrence kernels for chunk size 64, f32 storage (one translation unit per
// combination so the exact-K instantiations compile in parallel).
#include "kda_recur.h"

namespace kda {
hipError_t launch_recur_c64_f32(const Params &p, hipStream_t s) { return launch_recur_ct<64, float>(p, s); }
}  // namespace kda
