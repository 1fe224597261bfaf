// Allocation-free entry point of the segmented chunk prefill.
//
// kda_chunk_fwd_segmented takes its scratch space (the segment maps and the
// segments' incoming states) as a caller-owned workspace.  Callers that cannot
// allocate device memory (code under HIP graph capture, serving loops that
// forbid hipMalloc) use kda_chunk_fwd_segmented_noalloc instead: the scratch
// space is the fixed-size device array below, one copy per GPU, held from the
// library's load until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a handle for the runtime): its
// device address is looked up once per device with hipGetSymbolAddress and
// cached, and that address is what the kernels receive.
#include <hip/hip_runtime.h>

#include <atomic>

#include "kda_launch.h"
#include "libkda.h"

static constexpr unsigned long long kScratchBytes = 64ull << 20;   // KDA_NOALLOC_SCRATCH_BYTES

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

static_assert(kScratchBytes == KDA_NOALLOC_SCRATCH_BYTES, "header and array agree on the scratch size");

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device, looked up on the first
// call on that device (with it current) and cached.
void *scratch_address(const char **err)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        *err = "hipGetDevice failed";
        return nullptr;
    }
    if (dev >= kMaxDevices) {
        *err = "device index beyond the library's per-device table";
        return nullptr;
    }
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
        *err = hipGetErrorString(e);
        return nullptr;
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);
    return p;
}

}  // namespace

extern "C" kda_status_t kda_chunk_fwd_segmented_noalloc(const void *q, const void *k, const void *v,
                                                        const float *log_alpha, const float *beta,
                                                        const float *S0, void *out, float *S_final, int B,
                                                        int T, int H, int dk, int dv, int C, int nseg,
                                                        void *stream)
{
    const kda::StaticScratch s{kScratchBytes, scratch_address};
    return (kda_status_t)kda::chunk_segmented_static(q, k, v, log_alpha, beta, S0, out, S_final, B, T, H, dk, dv,
                                                     C, nseg, s, stream);
}
