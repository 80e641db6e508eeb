// kda_bwd_chunk.h -- launchers of the chunked backward's two kernels (the reverse chunk
// recurrence and the per-chunk gradients), instantiated per storage type.
#pragma once

#include "kda_bwd_local.h"

namespace kda {

template <typename K_, typename F>
hipError_t set_lds_and_launch(F kern, size_t lds, dim3 grid, dim3 block, hipStream_t s, const BwdChunkParams &p) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, block, lds, s, p);
    return hipGetLastError();
}

template <int C, typename T, int NKK>
hipError_t launch_dhu_t(const BwdChunkParams &p, hipStream_t s) {
    const unsigned units = (unsigned)p.f.N * (unsigned)p.f.HV * (unsigned)(p.f.V / 32);
    if (units == 0) return hipSuccess;
    return set_lds_and_launch<T>(bwd_dhu_kernel<C, T, NKK>, DhuLds<C, 32 * NKK>::bytes, dim3(units), dim3(256), s, p);
}

template <int C, typename T, int NKK>
hipError_t launch_local_t(const BwdChunkParams &p, hipStream_t s) {
    const unsigned items = (unsigned)p.f.total_chunks * (unsigned)p.f.HV;
    if (items == 0) return hipSuccess;
    return set_lds_and_launch<T>(bwd_local_kernel<C, T, NKK>, LocalLds<C, 32 * NKK>::bytes, dim3(items),
                                 dim3(64 * (C / 16)), s, p);
}

template <typename T>
hipError_t launch_bwd_dhu_c(const BwdChunkParams &p, hipStream_t s) {
    const int nkk = p.f.K / 32;
    if (p.f.C == 64) {
        switch (nkk) {
        case 1: return launch_dhu_t<64, T, 1>(p, s);
        case 2: return launch_dhu_t<64, T, 2>(p, s);
        case 3: return launch_dhu_t<64, T, 3>(p, s);
        case 4: return launch_dhu_t<64, T, 4>(p, s);
        }
    } else {
        switch (nkk) {
        case 1: return launch_dhu_t<32, T, 1>(p, s);
        case 2: return launch_dhu_t<32, T, 2>(p, s);
        case 3: return launch_dhu_t<32, T, 3>(p, s);
        case 4: return launch_dhu_t<32, T, 4>(p, s);
        }
    }
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_bwd_local_c(const BwdChunkParams &p, hipStream_t s) {
    const int nkk = p.f.K / 32;
    if (p.f.C == 64) {
        switch (nkk) {
        case 1: return launch_local_t<64, T, 1>(p, s);
        case 2: return launch_local_t<64, T, 2>(p, s);
        case 3: return launch_local_t<64, T, 3>(p, s);
        case 4: return launch_local_t<64, T, 4>(p, s);
        }
    } else {
        switch (nkk) {
        case 1: return launch_local_t<32, T, 1>(p, s);
        case 2: return launch_local_t<32, T, 2>(p, s);
        case 3: return launch_local_t<32, T, 3>(p, s);
        case 4: return launch_local_t<32, T, 4>(p, s);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
