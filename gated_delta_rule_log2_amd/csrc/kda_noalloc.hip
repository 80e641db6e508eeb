// kda_noalloc.hip -- kda_chunk_fwd_noalloc: the forward of kda_chunk_fwd with its
// workspace taken from a fixed device array of the library instead of a caller buffer,
// for callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The array `scratch` below is a file-scope device variable: every GPU the library
// runs on holds its own copy, at its own address, from module load until the process
// ends.  Its name is only a host-side stand-in for that memory, so host code never
// passes it anywhere: on the first call on a device (with that device current) the
// device address is looked up once with hipGetSymbolAddress and kept per device, and
// that address is what the kernels receive as their workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

constexpr size_t kScratchBytes = KDA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first call there.
kda_status scratch_address(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KDA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return KDA_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return KDA_OK;
}

}  // namespace

extern "C" kda_status kda_chunk_fwd_noalloc(const kda_fwd_desc *d, const void *q, const void *k, const void *v,
                                            const void *g, const void *beta, const float *A_log,
                                            const float *dt_bias, const float *initial_state,
                                            const int64_t *cu_seqlens, void *o, float *final_state,
                                            hipStream_t stream) {
    // size first (host only): a problem whose workspace exceeds the array is refused
    // before any device work
    size_t need = 0;
    kda_status st = kda_chunk_fwd_workspace_size(d, &need);
    if (st != KDA_OK) return st;
    if (need > kScratchBytes) return KDA_ERR_WORKSPACE;
    void *ws = nullptr;
    st = scratch_address(&ws);
    if (st != KDA_OK) return st;
    // The forward never reads workspace contents it has not written in the same call,
    // so nothing is cleared between calls.
    return kda::chunk_fwd_run(d, q, k, v, g, beta, A_log, dt_bias, initial_state, cu_seqlens, o, final_state,
                              false, nullptr, ws, kScratchBytes, stream, nullptr);
}
