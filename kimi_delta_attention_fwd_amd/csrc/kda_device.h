// Device-side helpers shared by the libkda kernels (gfx950 / CDNA4 only):
// bf16 <-> fp32 conversion, 16x16 MFMA tile products, DPP lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float tof(bf16 x) { return (float)x; }
__device__ __forceinline__ float tof(float x) { return x; }

template <typename T> __device__ __forceinline__ T fromf(float x);
template <> __device__ __forceinline__ float fromf<float>(float x) { return x; }
// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
template <> __device__ __forceinline__ bf16 fromf<bf16>(float x) { return (bf16)x; }

// ---------------------------------------------------------------------------
// 16x16 MFMA tiles.  For every variant used here the output tile is held in
// the same "accumulator layout": lane l owns D[4*(l>>4) + i][l & 15], i=0..3.
// Operands: lane l supplies A[l & 15][k0 + KPL*(l>>4) + 0..KPL-1] and
// B[k0 + KPL*(l>>4) + 0..KPL-1][l & 15].
// ---------------------------------------------------------------------------
template <typename OpT, int KS> struct Mma;

template <> struct Mma<bf16, 32> {   // v_mfma_f32_16x16x32_bf16
    static constexpr int KPL = 8;
    typedef bf16x8 frag;
    static __device__ __forceinline__ f32x4 run(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mma<bf16, 16> {   // v_mfma_f32_16x16x16_bf16
    static constexpr int KPL = 4;
    typedef bf16x4 frag;
    static __device__ __forceinline__ f32x4 run(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                         __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
    }
};

template <> struct Mma<float, 4> {   // v_mfma_f32_16x16x4_f32
    static constexpr int KPL = 1;
    typedef float frag;
    static __device__ __forceinline__ f32x4 run(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// Contraction step used for a contraction of length KL.
template <typename OpT, int KL> struct KStep {
    static constexpr int value = sizeof(OpT) == 4 ? 4 : (KL % 32 == 0 ? 32 : 16);
};

// The MFMA operand fragments of one 16-row panel (16 x KL), loaded once from
// LDS and reused for several tiles.  Lane l holds row (l & 15) and, for each
// contraction step s, KPL consecutive k starting at s*KS + KPL*(l >> 4).
// KS_ selects the MFMA shape; products that accumulate into the same tile
// must use the same shape (back-to-back dependent MFMAs of different shapes
// need wait states the compiler does not insert).
template <typename OpT, int KL, int KS_ = KStep<OpT, KL>::value>
struct Panel {
    static constexpr int KS = KS_;
    static_assert(KL % KS == 0, "contraction length is a multiple of the MFMA step");
    static constexpr int NS = KL / KS;
    typedef Mma<OpT, KS> M;
    typename M::frag f[NS];

    // rows of a row-major array; steps starting at k >= kmax are not loaded
    __device__ __forceinline__ void load(const OpT *rows, int pitch, int lane, int kmax = KL) {
        const OpT *p = rows + (lane & 15) * pitch + (lane >> 4) * M::KPL;
#pragma unroll
        for (int s = 0; s < NS; ++s)
            if (s * KS < kmax) f[s] = *(const typename M::frag *)(p + s * KS);
    }
    // rows row0.. of an array stored with swz_index() below
    __device__ __forceinline__ void load_swz(const OpT *base, int row0, int pitch, int mask, int lane) {
        const int row = row0 + (lane & 15);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int col = s * KS + (lane >> 4) * M::KPL;
            f[s] = *(const typename M::frag *)(base + swz_index(row, col, pitch, mask));
        }
    }
    // element (row, col) of a 16-byte-chunk XOR-swizzled array: chunk col/V is
    // stored at chunk (col/V) ^ ((row >> 2) & mask), V = 16 bytes of OpT.  The
    // swizzle spreads the transposed writes of four consecutive rows over
    // different banks.
    static __device__ __forceinline__ int swz_index(int row, int col, int pitch, int mask) {
        constexpr int V = 16 / (int)sizeof(OpT);
        return row * pitch + (((col / V) ^ ((row >> 2) & mask)) * V) + (col % V);
    }
};

// acc += A B^T over one 16x16 tile from two preloaded panels (A rows, B rows);
// contraction steps starting at k >= kmax are skipped.
template <typename OpT, int KLA, int KLB, int KS>
__device__ __forceinline__ f32x4 mma(f32x4 acc, const Panel<OpT, KLA, KS> &a, const Panel<OpT, KLB, KS> &b,
                                     int kmax = KLA) {
    static_assert(KLA == KLB, "operand panels of one product share the contraction length");
    typedef Panel<OpT, KLA, KS> P;
#pragma unroll
    for (int s = 0; s < P::NS; ++s)
        if (s * P::KS < kmax) acc = P::M::run(a.f[s], b.f[s], acc);
    return acc;
}

// fp32 16x16xKL product with general strides (used for the small triangular
// inverse, where one operand is read column-wise): acc[m][n] += sum_k
// A[m*ars + k*acs] * B[k*brs + n*bcs].
template <int KL>
__device__ __forceinline__ f32x4 mma_f32_strided(f32x4 acc, const float *A, int ars, int acs,
                                                 const float *B, int brs, int bcs, int lane) {
    const int r = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < KL; k0 += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[r * ars + (k0 + kq) * acs],
                                                   B[(k0 + kq) * brs + r * bcs], acc, 0, 0, 0);
    return acc;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// Sum over aligned groups of G lanes (G in {1, 2, 4, 8}) with DPP; every lane
// of the group receives the group's sum.
// ---------------------------------------------------------------------------
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (G >= 2)   // quad_perm [1,0,3,2]: lane ^ 1
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
    if constexpr (G >= 4)   // quad_perm [2,3,0,1]: lane ^ 2
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));
    if constexpr (G >= 8)   // row_half_mirror: lane i <-> 7 - i inside each group of 8
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, true));
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
    return x;
}

// Lane i of each 16-lane row receives x of lane i - D (row_shr) or i + D
// (row_shl) of the same row; lanes with no such source receive `fill`.
template <int D>
__device__ __forceinline__ float row_shr(float x, float fill) {
    static_assert(D >= 1 && D <= 15, "row shift");
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill), __builtin_bit_cast(int, x),
                                                                 0x110 + D, 0xF, 0xF, false));
}
template <int D>
__device__ __forceinline__ float row_shl(float x, float fill) {
    static_assert(D >= 1 && D <= 15, "row shift");
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill), __builtin_bit_cast(int, x),
                                                                 0x100 + D, 0xF, 0xF, false));
}

// log(alpha) = -softplus(g) = -(max(g, 0) + log(1 + e^{-|g|})), through the
// hardware base-2 exponential and logarithm (for e^{-|g|} below ~6e-8 the
// sum rounds to 1 and log(alpha) to -max(g, 0), an error below 6e-8).
__device__ __forceinline__ float neg_softplus(float g)
{
    const float t = __builtin_amdgcn_exp2f(-fabsf(g) * 1.4426950408889634f);
    return -(fmaxf(g, 0.f) + __builtin_amdgcn_logf(1.f + t) * 0.6931471805599453f);
}

}  // namespace kda
