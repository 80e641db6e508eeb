// Chunked backward kernels for bf16 q/k/v (bf16 intermediates: bf16 matrix-core
// operands with fp32 accumulation), chunk 32 and 64, K = 32..128.
#include "kda_bwd_chunk.h"
#include "kda_bwd_dhu_reg.h"
#include "kda_bwd_local3.h"

namespace kda {
// the reverse recurrence with the state gradient in registers (bf16 intermediates)
hipError_t launch_bwd_dhu_bf16(const BwdChunkParams &p, hipStream_t s) {
    const int nkk = p.f.K / 32;
    if (p.f.C == 64) {
        switch (nkk) {
        case 1: return launch_bwd_dhu_reg_t<64, 1>(p, s);
        case 2: return launch_bwd_dhu_reg_t<64, 2>(p, s);
        case 3: return launch_bwd_dhu_reg_t<64, 3>(p, s);
        case 4: return launch_bwd_dhu_reg_t<64, 4>(p, s);
        }
    } else {
        switch (nkk) {
        case 1: return launch_bwd_dhu_reg_t<32, 1>(p, s);
        case 2: return launch_bwd_dhu_reg_t<32, 2>(p, s);
        case 3: return launch_bwd_dhu_reg_t<32, 3>(p, s);
        case 4: return launch_bwd_dhu_reg_t<32, 4>(p, s);
        }
    }
    return hipErrorInvalidValue;
}
// the reverse recurrence's operand preparation alone (then not repeated by launch_bwd_dhu)
hipError_t launch_bwd_prep_bf16(const BwdChunkParams &p, hipStream_t s) {
    const int nkk = p.f.K / 32;
    if (p.f.C == 64) {
        switch (nkk) {
        case 1: return launch_bwd_prep_t<64, 1>(p, s);
        case 2: return launch_bwd_prep_t<64, 2>(p, s);
        case 3: return launch_bwd_prep_t<64, 3>(p, s);
        case 4: return launch_bwd_prep_t<64, 4>(p, s);
        }
    } else {
        switch (nkk) {
        case 1: return launch_bwd_prep_t<32, 1>(p, s);
        case 2: return launch_bwd_prep_t<32, 2>(p, s);
        case 3: return launch_bwd_prep_t<32, 3>(p, s);
        case 4: return launch_bwd_prep_t<32, 4>(p, s);
        }
    }
    return hipErrorInvalidValue;
}
// the per-chunk gradients with every operand split into bf16 planes once (kda_bwd_local2.h)
template <int C, int NKK>
hipError_t launch_local2_t(const BwdChunkParams &p, hipStream_t s) {
    const unsigned items = (unsigned)p.f.total_chunks * (unsigned)p.f.HV;
    if (items == 0) return hipSuccess;
    return set_lds_and_launch<uint16_t>(bwd_local2_kernel<C, NKK>, LocalLds2<C, 32 * NKK>::bytes, dim3(items),
                                        dim3(64 * (C / 16)), s, p);
}
// K = 128: two waves per 16-row block (kda_bwd_local3.h)
template <int C>
hipError_t launch_local3_t(const BwdChunkParams &p, hipStream_t s) {
    const unsigned items = (unsigned)p.f.total_chunks * (unsigned)p.f.HV;
    if (items == 0) return hipSuccess;
    return set_lds_and_launch<uint16_t>(bwd_local3_kernel<C, 4>, LocalLds3<C, 128>::bytes, dim3(items),
                                        dim3(128 * (C / 16)), s, p);
}
hipError_t launch_bwd_local_bf16(const BwdChunkParams &p, hipStream_t s) {
    const int nkk = p.f.K / 32;
    if (p.f.C == 64) {
        switch (nkk) {
        case 1: return launch_local2_t<64, 1>(p, s);
        case 2: return launch_local2_t<64, 2>(p, s);
        case 3: return launch_local2_t<64, 3>(p, s);
        case 4: return launch_local3_t<64>(p, s);
        }
    } else {
        switch (nkk) {
        case 1: return launch_local2_t<32, 1>(p, s);
        case 2: return launch_local2_t<32, 2>(p, s);
        case 3: return launch_local2_t<32, 3>(p, s);
        case 4: return launch_local3_t<32>(p, s);
        }
    }
    return hipErrorInvalidValue;
}
}  // namespace kda
