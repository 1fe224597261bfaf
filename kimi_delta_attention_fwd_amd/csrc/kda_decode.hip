// Instantiates the decode kernels, one token and T tokens per launch (bf16
// and fp32 inputs, dk in {16, 32, 64, 128}), and the streaming copy used as
// the bandwidth reference.
#include "kda_decode.h"

namespace kda {

hipError_t launch_decode(const DecodeArgs &a, bool f32)
{
    switch (a.dk) {
    case 16: return f32 ? launch_decode_t<float, 16>(a) : launch_decode_t<bf16, 16>(a);
    case 32: return f32 ? launch_decode_t<float, 32>(a) : launch_decode_t<bf16, 32>(a);
    case 64: return f32 ? launch_decode_t<float, 64>(a) : launch_decode_t<bf16, 64>(a);
    case 128: return f32 ? launch_decode_t<float, 128>(a) : launch_decode_t<bf16, 128>(a);
    default: return hipErrorInvalidConfiguration;
    }
}

// Bandwidth reference: n16 16-byte elements copied with nontemporal loads and
// stores (the decode kernels' access pattern for the state), one element per
// thread over as many 256-thread workgroups as that takes; that shape streams
// faster than loops with several elements per thread.  The grid-stride loop
// only matters past 2^31 - 1 workgroups.
__global__ void __launch_bounds__(256) stream_copy_kernel(const f32x4 *__restrict__ src, f32x4 *__restrict__ dst,
                                                          long n16)
{
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n16; i += (long)gridDim.x * 256)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

hipError_t launch_stream_copy(const void *src, void *dst, long n16, hipStream_t stream)
{
    if (n16 <= 0) return hipSuccess;
    const long need = (n16 + 255) / 256, cap = 0x7fffffffL;
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)(need < cap ? need : cap)), dim3(256), 0, stream,
                       (const f32x4 *)src, (f32x4 *)dst, n16);
    return hipGetLastError();
}

hipError_t launch_decode_multi(const DecodeArgs &a, int T, bool f32)
{
    switch (a.dk) {
    case 16: return f32 ? launch_decode_multi_t<float, 16>(a, T) : launch_decode_multi_t<bf16, 16>(a, T);
    case 32: return f32 ? launch_decode_multi_t<float, 32>(a, T) : launch_decode_multi_t<bf16, 32>(a, T);
    case 64: return f32 ? launch_decode_multi_t<float, 64>(a, T) : launch_decode_multi_t<bf16, 64>(a, T);
    case 128: return f32 ? launch_decode_multi_t<float, 128>(a, T) : launch_decode_multi_t<bf16, 128>(a, T);
    default: return hipErrorInvalidConfiguration;
    }
}

}  // namespace kda
