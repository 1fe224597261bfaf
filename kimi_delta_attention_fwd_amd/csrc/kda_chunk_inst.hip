// Instantiates the chunk prefill kernels for one (input type, dk) pair.
// Compiled several times with -DKDA_INST_F32=0|1 -DKDA_INST_DK=16|32|64|128
// so the kernel variants build in parallel.
#include "kda_chunk.h"

#if !defined(KDA_INST_F32) || !defined(KDA_INST_DK)
#error "compile with -DKDA_INST_F32=0|1 and -DKDA_INST_DK=16|32|64|128"
#endif

#define KDA_JOIN4(a, b, c, d) a##b##c##d
#define KDA_NAME(tag, dk) KDA_JOIN4(launch_chunk_, tag, _, dk)

namespace kda {

#if KDA_INST_F32
hipError_t KDA_NAME(f32, KDA_INST_DK)(const ChunkArgs &a) { return launch_chunk_dk<float, KDA_INST_DK>(a); }
#else
hipError_t KDA_NAME(bf16, KDA_INST_DK)(const ChunkArgs &a) { return launch_chunk_dk<bf16, KDA_INST_DK>(a); }
#endif

#if KDA_INST_F32 == 0 && KDA_INST_DK == 16
// The fit table is compile-time data of the kernel configurations; it lives
// in exactly one translation unit.
bool chunk_fits(bool f32, int dk, int BV, int C)
{
    switch (dk) {
    case 16: return f32 ? chunk_fits_dk<float, 16>(BV, C) : chunk_fits_dk<bf16, 16>(BV, C);
    case 32: return f32 ? chunk_fits_dk<float, 32>(BV, C) : chunk_fits_dk<bf16, 32>(BV, C);
    case 64: return f32 ? chunk_fits_dk<float, 64>(BV, C) : chunk_fits_dk<bf16, 64>(BV, C);
    case 128: return f32 ? chunk_fits_dk<float, 128>(BV, C) : chunk_fits_dk<bf16, 128>(BV, C);
    default: return false;
    }
}
#endif

}  // namespace kda
