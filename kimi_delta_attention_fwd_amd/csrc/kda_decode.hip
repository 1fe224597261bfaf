// Instantiates the decode kernels, one token and T tokens per launch (bf16
// and fp32 inputs, dk in {16, 32, 64, 128}).
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
