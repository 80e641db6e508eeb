// Recurrence kernels for chunk size 64, bf16 intermediates: the register-resident
// chain for key widths up to 128 (the intra kernel writes permuted fragments there),
// the LDS-exchange kernel above that.
#include "kda_recur_reg.h"

namespace kda {
hipError_t launch_recur_c64_bf16(const Params &p, hipStream_t s) {
    if (p.K <= 128) return launch_recur_reg<64>(p, s);
    return launch_recur_ct<64, uint16_t>(p, s);
}
}  // namespace kda
