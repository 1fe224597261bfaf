// Internal launcher interface between the C ABI (kda_api.cpp, host only) and
// the kernel translation units.  Not part of the public API.
#pragma once

#include <hip/hip_runtime_api.h>

namespace kda {

struct ChunkArgs {
    const void *q, *k, *v;
    const float *log_alpha, *beta, *S0;
    void *out;
    float *S_final;
    const int *cu_seqlens;   // device; NULL for the dense [B, T, H, d] layout
    int nseq, T, H, dk, dv, C, BV;   // T: tokens per sequence, or T_total with cu_seqlens
    // segment-parallel schedule (nsegs > 1): caller-owned workspace,
    // seg_map [nseq*H][nsegs-1][dv+dk][dk] (mout: [nseq*H][nsegs][dv+dk][dk], slot 0
    // unused) and seg_start [nseq*H][nsegs][dv][dk] fp32
    int nsegs;
    float *seg_map, *seg_start;
    // lead > 0: segment 0 is about lead / 10 times as long as each later one and
    // runs its whole pass in the map launch (nsegs >= 2); 0: equal segments
    int lead;
    // variant: gate 0 per channel, 1 scalar per token and head, 2 none;
    // add 1 = additive write; prep 1 = raw q, k and gate pre-activations
    int gate, add, prep;
    // mout (lead > 0): the schedule without a second pass; mws holds the
    // virtual rows' outputs [tokens, H, dk] in the input type
    void *mws;
    int mout;
    int cus;   // compute units of the device (launch sizing)
    hipStream_t stream;
};

struct DecodeArgs {
    const void *q, *k, *v;
    const float *log_alpha, *beta;
    float *S;
    void *out;
    int N, H, dk, dv;
    int gate, add, prep;   // as in ChunkArgs
    hipStream_t stream;
};

// Chunk prefill launchers, one per (input type, dk); BV in {16, 32, 64},
// C in {16, 32, 64}.  Defined in kda_chunk_inst.hip.
hipError_t launch_chunk_bf16_16(const ChunkArgs &);
hipError_t launch_chunk_bf16_32(const ChunkArgs &);
hipError_t launch_chunk_bf16_64(const ChunkArgs &);
hipError_t launch_chunk_bf16_128(const ChunkArgs &);
hipError_t launch_chunk_f32_16(const ChunkArgs &);
hipError_t launch_chunk_f32_32(const ChunkArgs &);
hipError_t launch_chunk_f32_64(const ChunkArgs &);
hipError_t launch_chunk_f32_128(const ChunkArgs &);

// Whether the (input type, dk, BV, C) kernel fits the 160 KiB of LDS of a
// gfx950 workgroup (and is therefore instantiated).  Defined next to the
// launchers; pure host code, no HIP call.
bool chunk_fits(bool f32, int dk, int BV, int C);

// Decode launchers: one token, and T tokens per sequence (q, k, v, out,
// log_alpha, beta laid out [N, T, H, d]).  Defined in kda_decode.hip.
hipError_t launch_decode(const DecodeArgs &, bool f32);
hipError_t launch_decode_multi(const DecodeArgs &, int T, bool f32);
hipError_t launch_stream_copy(const void *src, void *dst, long n16, hipStream_t stream);

// A fixed-size device array that stands in for the caller's workspace of the
// segmented schedule (kda_noalloc.hip).  `get` returns its address on the
// current device (looked up once per device), or NULL with a message in *err.
struct StaticScratch {
    unsigned long long bytes;
    void *(*get)(const char **err);
};

// kda_chunk_fwd_segmented with the workspace taken from `scratch` instead of
// the caller: every argument check runs first (a workspace larger than
// scratch.bytes is rejected there), then scratch.get(), then the launches.
// Defined in kda_api.cpp.
int chunk_segmented_static(const void *q, const void *k, const void *v, const float *log_alpha,
                           const float *beta, const float *S0, void *out, float *S_final, int B, int T, int H,
                           int dk, int dv, int C, int nseg, const StaticScratch &scratch, void *stream);

}  // namespace kda
