// Fused chunkwise KDA prefill kernel for gfx950.
//
// One workgroup owns one (sequence, head, block of BV value rows) and walks the
// sequence's chunks of C tokens in order.  Per chunk, with G_r the cumulative
// log-decay of token r inside the chunk (per key channel) and S the state that
// enters the chunk:
//
//   A_rj = beta_r sum_c k_rc k_jc e^{G_rc - G_jc}   (j <  r)   KK^T system
//   P_rj =        sum_c q_rc k_jc e^{G_rc - G_jc}   (j <= r)   causal QK^T
//   R    = Diag(beta) (V - Kbar S^T),   Kbar = K e^{G}         provisional errors
//   (I + A) E = R                                              corrected errors
//   O    = Qbar S^T + P E,              Qbar = Q e^{G}
//   S^T <- Diag(e^{G_last}) S^T + Ktil^T E,  Ktil = K e^{G_last - G}
//
// This is the chunk mode of the "KDA derivation summary" page (sect. 6: the
// recurrence regrouped into matrix products plus a lower-triangular solve that
// corrects each token's provisional error), on the chunk skeleton of the
// "Linear/sparse attention tutorial" page (sect. 6.2: intra-chunk causal part,
// inter-chunk state hand-off, cumulative decay folded into the state and the
// intra-chunk mask).  The equations follow from the recurrence by unrolling it
// over one chunk.
//
// Work split (wave specialisation).  The state-independent work of a chunk
// (decay-scaled operands, the diagonal A tiles and the inverses of the
// diagonal blocks of I + A) runs on four "operand" waves one chunk ahead of
// the state-dependent chain (R, the solve, O, the state update), which runs
// on BV/16 "state" waves, one per 16 value rows.  The state update needs only
// the chunk's own E and double-buffered operands, so it closes the state
// waves' first segment; their second segment forms the next chunk's P tiles
// and off-diagonal A tiles (with a single state wave: the off-diagonal P
// tiles only, the operand waves keep the rest).  Value rows of the state
// evolve independently, so each state wave runs its whole chain alone: its
// 16 x DK slice of the fp32 state stays in MFMA accumulator registers across
// the whole sequence, and every accumulator tile feeds the next product
// directly as an operand (a tile held as lane l <-> D[4(l>>4)+i][l&15] is both
// the B operand over its rows and the A operand of its transpose).  The two
// groups meet at two workgroup barriers per chunk; everything the state waves
// read is double-buffered in LDS.
//
// Decay factoring.  e^{G_r - G_j} is not formed pairwise.  Rows are split
// into 16-token blocks and every key channel c gets a reference rho_I[c] per
// block I: 0 (the chunk start) when the channel decays by at most 80 nats over
// the whole chunk, else G just before block I.  With B_I the channel's decay
// inside block I (a sum of log-decays, <= 0), the operand waves store, per
// token r of block I,
//   Kr = k e^{G_r - rho_I},  Qr = q e^{G_r - rho_I}        (<= |k|, |q|)
//   Kc = k e^{-G_r} (chunk-start channels, <= |k| e^{80}),
//        k e^{rho_{I+1} - G_r} (block-referenced ones, <= |k|)
// and per channel e^{rho_I} and a column scale s_IJ per tile pair: 1 for
// chunk-start channels, else e^{B_{J+1} + .. + B_{I-1}} (J < I, <= 1) and
// e^{-B_I} (J = I).  Then
//   A/P tile (I, J) = [Kr|Qr]_I (Kc_J s_IJ)^T,  Kbar S^T = Kr (S Diag(e^{rho_I}))^T,
// and Ktil = k e^{G_last - G_r} <= |k|.  When every channel of a chunk takes
// the chunk-start reference all scales are 1 and the consumers skip them.  A
// channel whose decay inside block I exceeds 80 nats cannot take e^{-B_I}: it
// gets s_II = 0 and its pairs of that diagonal tile are formed apart, as
// products of per-token decays split by halves (hard_block_fn), so any decay,
// down to a complete clear (alpha = 0), is exact.  The factors come from
// alpha = e^{log_alpha} by prefix and suffix products over each lane's tokens,
// times one exponential per channel of sums of the other lanes' log-decays,
// taken inside the block for block-referenced channels: exponents are sums of
// log-decays, never differences of cumulative ones, so a deep decay early in
// a chunk costs no precision later.

// (I + A) E = R is solved by block forward substitution over the 16-row
// blocks, E_b = D_b (R_b - sum_{J<b} A_bJ E_J) with D_b the inverse of the
// b-th diagonal block of I + A.  In the bf16 kernels the fp32 A, D_b and the
// fp32 right-hand side enter the bf16 MFMA as hi + lo bf16 pairs.
//
// MFMA: bf16 operands with fp32 accumulation (16x16x32, or 16x16x16 for
// 16-long contractions) in the bf16 entry points, fp32 16x16x4 in the fp32
// ones.  Each accumulator chain uses one MFMA shape.
#pragma once

#include "kda_device.h"
#include "kda_launch.h"

#include <type_traits>

namespace kda {

template <typename T> struct V4T { typedef T type __attribute__((ext_vector_type(4))); };

// ---------------------------------------------------------------------------
// acc += A B over N 16-wide contraction tiles.  For tile t the lane supplies
// a[t][e] = A[lane & 15][16t + 4(lane>>4) + e] and
// b[t][e] = B[16t + 4(lane>>4) + e][lane & 15], e = 0..3; the result is in
// accumulator layout.  KS selects the MFMA: 32 pairs tiles (2s, 2s+1) into one
// 16x16x32 bf16 product (both operands permuted the same way along k), 16 uses
// 16x16x16 bf16, 4 uses four 16x16x4 fp32 products per tile.
// ---------------------------------------------------------------------------
template <int KS, typename OpT, int N>
__device__ __forceinline__ f32x4 mma_tiles(f32x4 acc, const typename V4T<OpT>::type (&a)[N],
                                           const typename V4T<OpT>::type (&b)[N])
{
    if constexpr (KS == 32) {
        static_assert(N % 2 == 0 && sizeof(OpT) == 2, "paired bf16 tiles");
#pragma unroll
        for (int s = 0; s < N / 2; ++s) {
            const bf16x8 a8 = __builtin_shufflevector(a[2 * s], a[2 * s + 1], 0, 1, 2, 3, 4, 5, 6, 7);
            const bf16x8 b8 = __builtin_shufflevector(b[2 * s], b[2 * s + 1], 0, 1, 2, 3, 4, 5, 6, 7);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, acc, 0, 0, 0);
        }
    } else if constexpr (KS == 16) {
        static_assert(sizeof(OpT) == 2, "bf16 tiles");
#pragma unroll
        for (int t = 0; t < N; ++t)
            acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a[t]),
                                                            __builtin_bit_cast(i16x4, b[t]), acc, 0, 0, 0);
    } else {
        static_assert(KS == 4 && sizeof(OpT) == 4, "fp32 tiles");
#pragma unroll
        for (int t = 0; t < N; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t][i], b[t][i], acc, 0, 0, 0);
    }
    return acc;
}

template <typename OpT>
__device__ __forceinline__ typename V4T<OpT>::type to_op(f32x4 x)
{
    typename V4T<OpT>::type r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = fromf<OpT>(x[i]);
    return r;
}

template <typename OpT>
__device__ __forceinline__ f32x4 to_f32(typename V4T<OpT>::type x)
{
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = tof(x[i]);
    return r;
}

// acc += A B for an fp32 A tile fragment and an operand-type B fragment.  In
// the bf16 kernels A enters as hi + lo bf16 parts (about 16 significant bits).
template <typename OpT>
__device__ __forceinline__ f32x4 mma_fp32a(f32x4 acc, f32x4 a, typename V4T<OpT>::type b)
{
    typedef typename V4T<OpT>::type V4;
    if constexpr (sizeof(OpT) == 4) {
        const V4 aa[1] = {a}, bb[1] = {b};
        return mma_tiles<4, OpT, 1>(acc, aa, bb);
    } else {
        const V4 hi = to_op<OpT>(a);
        const V4 lo = to_op<OpT>(a - to_f32<OpT>(hi));
        const V4 a2[2] = {hi, lo}, b2[2] = {b, b};
        return mma_tiles<16, OpT, 2>(acc, a2, b2);
    }
}

// A X for fp32 A and fp32 X fragments; bf16 kernels use hi/lo parts of both
// (the lo x lo term is dropped).
template <typename OpT>
__device__ __forceinline__ f32x4 mma_fp32ab(f32x4 a, f32x4 x)
{
    typedef typename V4T<OpT>::type V4;
    if constexpr (sizeof(OpT) == 4) {
        const V4 aa[1] = {a}, xx[1] = {x};
        return mma_tiles<4, OpT, 1>(zero4(), aa, xx);
    } else {
        const V4 ah = to_op<OpT>(a), al = to_op<OpT>(a - to_f32<OpT>(ah));
        const V4 xh = to_op<OpT>(x), xl = to_op<OpT>(x - to_f32<OpT>(xh));
        const V4 a3[3] = {ah, ah, al}, x3[3] = {xh, xl, xh};
        return mma_tiles<16, OpT, 3>(zero4(), a3, x3);
    }
}

template <typename T>
__device__ __forceinline__ void store4(T *p, f32x4 v) { *(typename V4T<T>::type *)p = to_op<T>(v); }

// Raw buffer access (gfx9 descriptor word 3 = 0x00020000).  The descriptor is
// built from a wave-uniform base and a byte bound; reads at or past the bound
// return zeros and writes there are dropped, which is how tokens past the end
// of a sequence become identity tokens and how their outputs are skipped.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
template <typename T>
__device__ __forceinline__ T buf_load(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    if constexpr (sizeof(T) == 16) return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    else if constexpr (sizeof(T) == 8) return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
    else if constexpr (sizeof(T) == 4) return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
    else return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
}
// A store of more than 8 bytes reads its data registers after it issues, and
// a vector ALU write to them must wait one cycle.  The compiler inserts that
// wait only when the scalar offset is the constant 0, so 16-byte stores fold
// the offset into the per-lane one (with an SGPR offset a following write has
// been seen to replace the stored data).
template <typename T>
__device__ __forceinline__ void buf_store(T v, __amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    if constexpr (sizeof(T) == 16) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff + soff, 0, 0);
    else __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, voff, soff, 0);
}

// Writes v[0..RS) to row `row`, columns col0 .. col0+RS-1, of an array stored
// with Panel::swz_index (16-byte chunks XOR-swizzled by row), in 16-byte or
// smaller pieces.
template <typename OpT, int RS>
__device__ __forceinline__ void store_row_swz(OpT *base, int row, int col0, int pitch, int mask, const OpT (&v)[RS]) {
    constexpr int V = 16 / (int)sizeof(OpT);
    constexpr int W = RS < V ? RS : V;
    typedef OpT Vec __attribute__((ext_vector_type(W)));
#pragma unroll
    for (int i0 = 0; i0 < RS; i0 += W) {
        Vec x;
#pragma unroll
        for (int i = 0; i < W; ++i) x[i] = v[i0 + i];
        *(Vec *)(base + Panel<OpT, 16>::swz_index(row, col0 + i0, pitch, mask)) = x;
    }
}

// e^x via the hardware base-2 exponential; arguments here stay below 89, and
// results under the fp32 normal range may flush to zero, which only drops
// contributions that are that small.
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }


// Tiles of the lower block triangle (I >= J) of a chunk: the NB diagonal tiles
// first, then the off-diagonal ones row by row.
__host__ __device__ constexpr int tile_index(int NB, int I, int J)
{
    return I == J ? I : NB + I * (I - 1) / 2 + J;
}

// True when every operand wave flagged its channels as referenced to the chunk
// start (flags are 1.0 or 0.0 in LDS); wave-uniform.
template <int NF>
__device__ __forceinline__ bool all_flags(const float *fl)
{
    float m = 1.f;
#pragma unroll
    for (int i = 0; i < NF; ++i) m *= fl[i];
    return __builtin_amdgcn_readfirstlane((int)m) != 0;
}

template <typename In, int DK, int BV, int C, bool PAIRED = true>
struct ChunkCfg {
    typedef In OpT;                                  // MFMA operand type
    static constexpr bool F32 = sizeof(In) == 4;
    static constexpr int NB = C / 16;                // 16-token blocks per chunk
    static constexpr int NBV = BV / 16;              // 16-row value blocks = state waves
    static constexpr int NDK = DK / 16;
    static constexpr int NXW = 4;                    // operand waves
    static constexpr int NW = NBV + NXW;
    static constexpr int NT = 64 * NW;
    static constexpr int KD = F32 ? 4 : (DK % 32 == 0 ? 32 : 16);   // MFMA step of d_k contractions
    static constexpr int KC = F32 ? 4 : (C % 32 == 0 ? 32 : 16);    // MFMA step of token contractions
    static constexpr int PADE = 16 / (int)sizeof(In);
    // Paired operand order.  A 16x16x32 product takes, in lane (n, g), the
    // contraction indices 32s + 4g + e and 32s + 16 + 4g + e (e = 0..3) of two
    // 16-wide tiles.  Stored at pair_pos() of their index, these eight sit side
    // by side and the lane loads them with one 16-byte LDS read instead of two
    // 8-byte ones.  PAIRK: the d_k axis of Kr, Qr and Kd, whose rows are then
    // 16-byte aligned and 4 banks apart.
    static constexpr bool PAIRK = PAIRED && KD == 32;
    static constexpr int PK = DK + (PAIRK ? 8 : 4);  // rows of [token, d_k] operands
    // position of index c in the paired order (4-aligned groups of four stay together)
    static __device__ __forceinline__ int pair_pos(int c) {
        return (c & ~31) | ((c & 12) << 1) | ((c & 16) >> 2) | (c & 3);
    }
    static constexpr int PC = C + PADE;              // rows of Ktil^T (16-byte aligned, chunk-swizzled)
    static constexpr int SWZ = C * (int)sizeof(In) / 16 - 1;
    static constexpr int PT = 20;                    // rows of an A (fp32) or P tile
    static constexpr int NPAIR = NB * (NB + 1) / 2;
    static constexpr int NOFF = NB * (NB - 1) / 2;
    // operand-wave element mapping: wave x owns channels [x CPW, (x+1) CPW);
    // a lane owns RS consecutive tokens of 4 channels
    static constexpr int CPW = DK / NXW;
    static constexpr int NCG = CPW / 4;
    static constexpr int RS = (C * NCG > 64) ? C * NCG / 64 : 1;
    static constexpr int NSEG = C / RS;
    static constexpr int NACT = NCG * NSEG;
    // scales block: e^{rho_I} [NB][DK], e^{G_last} [DK], beta [C], per-wave
    // "all channels referenced to the chunk start" flags [NXW], per-wave masks
    // of the blocks with a channel too deep to factor (bit I: block I) [NXW]
    static constexpr int SC_GL = NB * DK, SC_BETA = NB * DK + DK, SC_FLAG = SC_BETA + C;
    static constexpr int SC_HARD = SC_FLAG + NXW;
    // input preparation (raw q, k): per-wave partial squared norms of k and q
    // [C][NXW] (a token's four partials in one 16-byte LDS read), then per
    // token beta / |k|^2, |k| and 1 / |q|
    static constexpr int SC_PK = SC_HARD + NXW, SC_PQ = SC_PK + NXW * C, SC_BH = SC_PQ + NXW * C;
    static constexpr int SC_KN = SC_BH + C, SC_QI = SC_KN + C, SC_END = SC_QI + C;
    static constexpr float FAST_NATS = 80.f;

    static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
    static constexpr size_t SZ_R = al(size_t(C) * PK * sizeof(In));     // Kr, Qr, Kd
    static constexpr size_t SZ_KT = al(size_t(DK) * PC * sizeof(In));   // Ktil^T
    static constexpr size_t SZ_SC = al(size_t(SC_END) * sizeof(float));
    static constexpr size_t SZ_W = al(size_t(NPAIR) * DK * sizeof(float));   // column scales per tile pair
    static constexpr size_t SZ_A = al(size_t(NPAIR) * 16 * PT * sizeof(float));
    static constexpr size_t SZ_P = al(size_t(NPAIR) * 16 * PT * sizeof(In));
    // double-buffered: written by the operand waves for chunk t+1 while the
    // state waves read chunk t
    static constexpr size_t O_KR = 0;
    static constexpr size_t O_QR = O_KR + 2 * SZ_R;
    static constexpr size_t O_KT = O_QR + 2 * SZ_R;
    static constexpr size_t O_SC = O_KT + 2 * SZ_KT;
    // single: Kd and w are private to the operand waves; A and P are written
    // after the state waves' last read of the previous chunk's
    static constexpr size_t O_KD = O_SC + 2 * SZ_SC;
    static constexpr size_t O_W = O_KD + SZ_R;
    static constexpr size_t O_A = O_W + SZ_W;
    static constexpr size_t O_P = O_A + SZ_A;
    static constexpr size_t LDS = O_P + SZ_P;
    static constexpr bool fits = LDS <= 160 * 1024;

    static_assert(C % 16 == 0 && C <= 64, "chunk length");
    static_assert(DK % 16 == 0 && DK <= 128 && BV % 16 == 0 && BV <= 64, "tile sizes");
    static_assert(16 % RS == 0, "a lane's tokens stay inside one 16-token block");
    static_assert(NACT <= 64, "one operand wave covers its channels");
    static_assert((NSEG & (NSEG - 1)) == 0, "segment scan over a power of two");
    static_assert(NSEG >= NB, "a segment of lanes per block scale vector");
};

// D = (I + L)^{-1} for the strictly lower 16 x 16 diagonal tile L of A, stored
// over that tile (At, row pitch PT) so that lane (n, g) writes row n, columns
// 4g..4g+3.  bf16 kernels: (I - L)(I + L^2)(I + L^4)(I + L^8) (L^16 = 0), from
// L and L^T in accumulator layout (lt0[i] = L[4g + i][n], lt1[i] = L[n][4g + i]);
// one fp32 MFMA product of two accumulator tiles gives acc(X^T Y).  (The powers
// of L can grow like binomial coefficients before they cancel, about 1e-4
// relative at worst: fine for the bf16 kernels.)
__device__ __forceinline__ void diag_inverse_bf16(float *At, int PT, int n, int g, f32x4 lt0, f32x4 lt1,
                                                  bool keep_l = false)
{
    auto mm = [](f32x4 x, f32x4 y) {   // acc(X^T Y)
        const f32x4 a[1] = {x}, b[1] = {y};
        return mma_tiles<4, float, 1>(zero4(), a, b);
    };
    const f32x4 L1 = lt0, U1 = lt1;
    const f32x4 U2 = mm(L1, U1), L2 = mm(U1, L1);
    const f32x4 L4 = mm(U2, L2);
    f32x4 id;
#pragma unroll
    for (int i = 0; i < 4; ++i) id[i] = (4 * g + i == n) ? 1.f : 0.f;
    const f32x4 X = id - U1;                          // (I - L)^T
    const f32x4 M1t = X + mm(L2, X);                  // ((I - L)(I + L^2))^T
    const f32x4 M2t = M1t + mm(L4, M1t);              // ... (I + L^4)
    const f32x4 W = mm(L4, M2t);                      // (L^4)^T M2t: L^8 as two L^4 factors
    const f32x4 Dt = M2t + mm(L4, W);                 // ... (I + L^8)
    // stored pre-split for the bf16 solve: hi then lo bf16 parts in the lane's 16 bytes
    const bf16x4 hi = to_op<bf16>(Dt), lo = to_op<bf16>(Dt - to_f32<bf16>(hi));
    const f32x2 h2 = __builtin_bit_cast(f32x2, hi), l2 = __builtin_bit_cast(f32x2, lo);
    // keep_l (wave-uniform): store L itself (lt1, what the tile already holds)
    // instead, with no branch, so the products above share one basic block with
    // the code before them
    f32x4 st = f32x4{h2[0], h2[1], l2[0], l2[1]};
#pragma unroll
    for (int i = 0; i < 4; ++i) st[i] = keep_l ? lt1[i] : st[i];
    *(f32x4 *)(At + n * PT + 4 * g) = st;
}

// fp32 kernels: column n of D by forward substitution over the rows of the
// stored tile L (lanes of the other 16-lane rows repeat the work and store
// nothing).
__device__ __forceinline__ void diag_inverse_f32(float *At, int PT, int n, int lane)
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float *Lr = At + i * PT;
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int kk = 0; kk + 1 < i; kk += 2) {
            s0 += Lr[kk] * x[kk];
            s1 += Lr[kk + 1] * x[kk + 1];
        }
        if (i & 1) s0 += Lr[i - 1] * x[i - 1];
        x[i] = ((i == n) ? 1.f : 0.f) - (s0 + s1);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if (lane < 16) {
#pragma unroll
        for (int i = 0; i < 16; ++i) At[i * PT + n] = x[i];
    }
}

// beta / |k|^2 of token r from the operand waves' partial squared norms in a
// scales block (0 for a zero key: identity tokens past the end of a sequence)
template <typename K>
__device__ __forceinline__ float beta_hat(const float *scc, int r)
{
    float sk = 0.f;
#pragma unroll
    for (int w = 0; w < K::NXW; ++w) sk += scc[K::SC_PK + r * K::NXW + w];
    return sk > 0.f ? scc[K::SC_BETA + r] * __builtin_amdgcn_rcpf(sk) : 0.f;
}

// Hard-block correction of diagonal tile I of chunk ch, for the key
// channels whose decay inside the block is too deep to factor through one
// reference (their column scale s_II is 0, so the A and P tiles above left
// them out).  Their pairwise decays e^{G_r - G_j} = prod_{s=j+1..r} alpha_s
// (r >= j in the block) are split by halves: for h = 8, 4, 2, 1 and tokens
// r, j of one aligned 2h-token group, r in its upper and j in its lower
// half, the product is (prod from the upper half's first token to r) x
// (prod from j + 1 to the lower half's last token), and both factors are
// <= 1.  Each level is one MFMA product of the two scaled operands, masked
// to its pairs; the diagonal of P (r = j, no decay) adds q_r . k_r.  Every
// pair r > j is in exactly one level.  The products come from the chunk's
// raw inputs, reloaded (they were just read, so they come from L2): lane
// (n, g) takes token 16 I + n and channels 16 t + 4 g + e.  The corrected
// A tile is inverted like the others.  Run by one wave per block.
// Kept out of line (it runs only in chunks with such blocks): the chunk loop's
// code and schedule stay those of the common case.  LDS arrays arrive as
// generic pointers.
template <typename In, int DK, int C>
__device__ __noinline__ void hard_block_fn(const In *__restrict__ k, const In *__restrict__ q,
                                           const float *__restrict__ log_alpha, const float *__restrict__ beta,
                                           long hrow, long t0, long len, int H, int gate, int add, int prep, bool map,
                                           const float *sW, float *sA, In *sP, const float *scc, int I)
{
    typedef ChunkCfg<In, DK, 16, C> K;   // the scales block does not depend on the value-block width
    typedef typename V4T<In>::type V4;
    constexpr int NDK = K::NDK, PT = K::PT;
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
    const int HDK = H * DK;
        const unsigned nv = (unsigned)((len - t0 < C) ? len - t0 : C);
    const int r = 16 * I + n;
    const int rowb = HDK * (int)sizeof(In);
    const int voff = r * rowb + 4 * g * (int)sizeof(In);
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(k + (hrow + t0 * H) * DK, nv * rowb);
    const __amdgpu_buffer_rsrc_t rq = buf_rsrc(q + (hrow + t0 * H) * DK, map ? 0u : nv * rowb);
    const In *gp = (const In *)log_alpha;
    const __amdgpu_buffer_rsrc_t rg =
        prep ? (gate == 1 ? buf_rsrc(gp + hrow + t0 * H, nv * H * (int)sizeof(In))
                          : buf_rsrc(gp + (hrow + t0 * H) * DK, gate == 0 ? nv * rowb : 0u))
             : (gate == 1 ? buf_rsrc(log_alpha + hrow + t0 * H, nv * H * 4)
                          : buf_rsrc(gate == 0 ? log_alpha + (hrow + t0 * H) * DK : beta,
                                     gate == 0 ? nv * HDK * 4 : 0u));
    constexpr int TPS = K::KD == 32 ? 2 : 1;   // 16-channel tiles per MFMA step
    f32x4 accA[4], accP[4], accD = zero4();
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        accA[b] = zero4();
        accP[b] = zero4();
    }
    // one MFMA step of channels at a time (a rolled loop keeps the live
    // registers few; this path is rare)
#pragma unroll 1
    for (int s = 0; s < NDK / TPS; ++s) {
        V4 kk[TPS], qq[TPS], km[TPS];
        f32x4 al[TPS];
#pragma unroll
        for (int u = 0; u < TPS; ++u) {
            const int c = 16 * (s * TPS + u);       // this tile's first channel
            kk[u] = buf_load<V4>(rk, voff + c * (int)sizeof(In), 0);
            qq[u] = map ? V4{} : buf_load<V4>(rq, voff + c * (int)sizeof(In), 0);
            if (prep) {   // g in the input type; log_alpha = -softplus(g), 0 past the end
                if (gate == 1) {
                    const float x = tof(buf_load<In>(rg, r * H * (int)sizeof(In), 0));
                    al[u] = f32x4{x, x, x, x};
                } else {
                    al[u] = to_f32<In>(buf_load<V4>(rg, voff + c * (int)sizeof(In), 0));
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) al[u][e] = (gate == 2 || r >= (int)nv) ? 0.f : neg_softplus(al[u][e]);
            } else if (gate == 1) {
                const float x = buf_load<float>(rg, r * H * 4, 0);
                al[u] = f32x4{x, x, x, x};
            } else {
                al[u] = buf_load<f32x4>(rg, r * HDK * 4 + (c + 4 * g) * 4, 0);
            }
            // alpha, and k masked to the hard channels (s_II == 0) for the column side
            const f32x4 sd = *(const f32x4 *)(sW + I * DK + c + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                al[u][e] = fexp(al[u][e]);
                km[u][e] = sd[e] == 0.f ? kk[u][e] : fromf<In>(0.f);
            }
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int h = 1 << b, pos = n & (h - 1);
            const bool up = (n >> b) & 1;
            V4 ya[TPS], xk[TPS], xq[TPS];
#pragma unroll
            for (int u = 0; u < TPS; ++u) {
                f32x4 vk, vq, vy;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // inclusive prefix products (x) and suffix products (y) of
                    // alpha inside aligned h-token groups
                    float x = al[u][e], y = al[u][e];
                    if (h > 1) {
                        const float a = row_shr<1>(x, 1.f), c = row_shl<1>(y, 1.f);
                        if (pos >= 1) x *= a;
                        if (pos + 1 < h) y *= c;
                    }
                    if (h > 2) {
                        const float a = row_shr<2>(x, 1.f), c = row_shl<2>(y, 1.f);
                        if (pos >= 2) x *= a;
                        if (pos + 2 < h) y *= c;
                    }
                    if (h > 4) {
                        const float a = row_shr<4>(x, 1.f), c = row_shl<4>(y, 1.f);
                        if (pos >= 4) x *= a;
                        if (pos + 4 < h) y *= c;
                    }
                    float suf = 1.f;   // exclusive: from the next token to the group's end
                    if (h > 1) {
                        const float c = row_shl<1>(y, 1.f);
                        if (pos < h - 1) suf = c;
                    }
                    vk[e] = up ? tof(kk[u][e]) * x : 0.f;
                    vq[e] = up ? tof(qq[u][e]) * x : 0.f;
                    vy[e] = up ? 0.f : tof(km[u][e]) * suf;
                }
                xk[u] = to_op<In>(vk);
                xq[u] = to_op<In>(vq);
                ya[u] = to_op<In>(vy);
            }
            if (!add) accA[b] = mma_tiles<K::KD, In, TPS>(accA[b], ya, xk);
            if (!map) accP[b] = mma_tiles<K::KD, In, TPS>(accP[b], ya, xq);
        }
        if (!map) accD = mma_tiles<K::KD, In, TPS>(accD, km, qq);   // P's diagonal: q_r . k_r
    }
    // pair (r = n, j = 4g + i) belongs to level b when r and j share their
    // aligned 2h-token group (the operands keep only r upper, j lower)
    f32x4 dA = zero4(), dP = zero4();
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool same = ((n ^ (4 * g + i)) >> (b + 1)) == 0;
            dA[i] += same ? accA[b][i] : 0.f;
            dP[i] += same ? accP[b][i] : 0.f;
        }
#pragma unroll
    for (int i = 0; i < 4; ++i) dP[i] += (4 * g + i == n) ? accD[i] : 0.f;
        if (!map) {
        In *pt = sP + I * 16 * PT + n * PT + 4 * g;
        store4(pt, to_f32<In>(*(const V4 *)pt) + dP);
    }
    if (!add) {
        const float bb = prep ? beta_hat<K>(scc, r) : scc[K::SC_BETA + r];
        float *at = sA + I * 16 * PT + n * PT + 4 * g;
        const f32x4 lt1 = *(const f32x4 *)at + dA * bb;   // L[n][4g + i]
        *(f32x4 *)at = lt1;
        if constexpr (K::F32) {
            diag_inverse_f32(sA + I * 16 * PT, PT, n, lane);
        } else {
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            f32x4 lt0;                                    // L[4g + i][n]
#pragma unroll
            for (int i = 0; i < 4; ++i) lt0[i] = sA[I * 16 * PT + (4 * g + i) * PT + n];
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            diag_inverse_bf16(sA + I * 16 * PT, PT, n, g, lt0, lt1);
        }
    }
}

// Segment bounds of the chunk schedule, shared by the chunk kernel and the
// output epilogue: chunks [c0, c1) of a sequence of n chunks for segment seg
// of nsegs (lead > 0: segments 1 .. nsegs - 1 take L = ceil(10 n / (10
// (nsegs - 1) + lead)) each from the end, segment 0 the rest; else equal).
__device__ __forceinline__ void seg_bounds(long n, int nsegs, int lead, int seg, long &c0, long &c1)
{
    if (lead > 0) {
        const long L = (10 * n + 10 * (nsegs - 1) + lead - 1) / (10 * (nsegs - 1) + lead);
        const long l0 = max(0L, n - (nsegs - 1) * L);
        c0 = seg == 0 ? 0 : min(l0 + (seg - 1) * L, n);
        c1 = seg == 0 ? l0 : min(c0 + L, n);
    } else {
        const long L = (n + nsegs - 1) / nsegs;
        c0 = min((long)seg * L, n);
        c1 = min(c0 + L, n);
    }
}

// Packed sequences split on the device (the one-pass schedule with two
// segments and lead = -(16 cus + nvA)): the makespan target, in chunk steps,
// is the longer of the second-longest sequence and the balanced share
// nvA H sum(n) / cus; a sequence longer than the target by more than an
// eighth runs its first `target` chunks as segment 0 and the rest as its
// mapped segment 1 (whose workgroups start as shorter sequences free their
// compute units); every other sequence is segment 0 whole.  One workgroup
// writes plan[i], the chunks of segment 0 of sequence i, for the launches
// that follow (offsets clamped to [0, T] as the kernels clamp them; any value
// there is safe: the kernels clamp each segment to their own sequence).
// (A template only so that every translation unit may hold its copy.)
template <int UNUSED = 0>
__global__ void __launch_bounds__(256) seg_plan_kernel(const int *__restrict__ cu_seqlens, int N, int T, int C,
                                                       int H, int code, int *__restrict__ plan)
{
    __shared__ long s_sum[256], s_m1[256], s_m2[256];
    const int tid = threadIdx.x;
    auto chunks = [&](int i) {
        const long a0 = min(max((long)cu_seqlens[i], 0L), (long)T);
        const long a1 = min(max((long)cu_seqlens[i + 1], a0), (long)T);
        return (a1 - a0 + C - 1) / C;
    };
    long sum = 0, m1 = 0, m2 = 0;   // this thread's sum and two largest
    for (int i = tid; i < N; i += 256) {
        const long n = chunks(i);
        sum += n;
        if (n > m1) {
            m2 = m1;
            m1 = n;
        } else if (n > m2) {
            m2 = n;
        }
    }
    s_sum[tid] = sum;
    s_m1[tid] = m1;
    s_m2[tid] = m2;
    __syncthreads();
    for (int d = 128; d > 0; d >>= 1) {
        if (tid < d) {
            const long a1 = s_m1[tid], a2 = s_m2[tid], b1 = s_m1[tid + d], b2 = s_m2[tid + d];
            s_sum[tid] += s_sum[tid + d];
            s_m1[tid] = max(a1, b1);
            s_m2[tid] = a1 >= b1 ? max(a2, b1) : max(a1, b2);
        }
        __syncthreads();
    }
    const int cus = (-code) >> 4, nvA = (-code) & 15;
    const long share = ((long)nvA * H * s_sum[0] + cus - 1) / cus;
    const long tgt = max(s_m2[0], share);
    for (int i = tid; i < N; i += 256) {
        const long n = chunks(i);
        plan[i] = (int)(n > tgt + tgt / 8 ? tgt : n);
    }
}

// Variants (uniform arguments, read only when VAR): gate 0 = per-channel log_alpha [.., H, DK],
// 1 = one log_alpha per token and head [.., H] shared by all key channels,
// 2 = no decay (log_alpha not read); add = 1 replaces the delta write by the
// additive one (e = beta v: no prediction, A = 0, E = R = beta V).
// prep = 1: q and k arrive raw and are L2-normalised here, and the gate
// argument holds g (input type) with log_alpha = -softplus(g).  With unit
// keys k^ = k / |k| the recurrence is the same as the one on the raw keys
// with beta^ = beta / |k|^2 and v' = |k| v (the error scales by 1 / |k|, the
// write e k^T does not change), and o = S q / |q|; so the chunk algorithm runs
// on the raw operands with those per-token factors.
//
// MAP = false: the prefill itself.  With nsegs > 1 each workgroup runs one of
// nsegs consecutive segments of its sequence's chunks, from the incoming state
// seg_start[(head, seg)]; only the last segment writes S_final.  With equal
// segments (lead = 0) that is every segment, segment 0's incoming state being
// S0; with a lead segment (lead > 0) segments 1 .. nsegs - 1.
// MAP = true: the affine map of each segment but the last (lead > 0: but the
// first and the last).  The state is augmented with DK "virtual" rows that
// start at the identity and see v = 0; the dv real rows start at zero.  After
// the segment the real rows hold N and the virtual rows M of
// S_end = S_start M + N, written to seg_map[(head, seg)]; no output is written
// and q is not read.  With a lead segment the launch's first workgroups run
// segment 0 as a plain pass instead (a runtime flag, folded away when MAP is
// false): from S0, writing its outputs and seg_start[(head, 1)].
// MAP = true with mout_arg (the schedule without a second pass, lead != 0):
// every segment after the first is mapped, at slot seg of nsegs per head, and
// its maps also read q and write outputs from the zero incoming state: the real
// rows' into out, the virtual rows' (their readouts S q) into mws [tokens, H,
// DK].  lead < 0 (-(16 cus + value blocks per head)): packed sequences in two
// segments, split on the device (seg_plan_kernel; the plan follows m in mws).  (hard_block_fn's `map` argument
// means "no outputs, q not read" and receives noout.)
template <typename In, int DK, int BV, int C, bool MAP, int VAR>
__global__ void __launch_bounds__((ChunkCfg<In, DK, BV, C>::NT), 1)
chunk_fwd_kernel(const In *__restrict__ q, const In *__restrict__ k, const In *__restrict__ v,
                 const float *__restrict__ log_alpha, const float *__restrict__ beta,
                 const float *S0, In *__restrict__ out, float *S_final,
                 const int *__restrict__ cu_seqlens, int T, int H, int dv, int xcd_map,
                 int nsegs, float *seg_start, float *seg_map, int gate_arg, int add_arg, int prep_arg,
                 int lead, In *__restrict__ mws, int mout_arg)
{
    // VAR = 0: the plain recurrence, the variant arguments folded away; 1: any
    // variant, read from the arguments; 2: raw inputs with the per-channel gate
    // and the delta write (the usual projection outputs), folded in
    const int gate = VAR == 1 ? gate_arg : 0, add = VAR == 1 ? add_arg : 0;
    const int prep = VAR == 2 ? 1 : (VAR == 1 ? prep_arg : 0);
    // every kernel takes the paired operand layouts (the raw-input one too:
    // 1.0% faster there on the current kernel, with the paired Ktil^T)
    typedef ChunkCfg<In, DK, BV, C> K;
    typedef typename V4T<In>::type V4;
    // Chunk indices and lengths are 32-bit (cheaper scalar arithmetic, and
    // fewer scalar registers for the kernel to spill into vector lanes); the
    // raw-input kernel timed faster with 64-bit ones
    typedef typename std::conditional<VAR == 2, long, int>::type CI;
    constexpr int NB = K::NB, NDK = K::NDK, PK = K::PK, PC = K::PC, PT = K::PT, RS = K::RS;

    __shared__ __attribute__((aligned(16))) unsigned char smem[K::LDS];
    In *const sKd = (In *)(smem + K::O_KD);
    float *const sW = (float *)(smem + K::O_W);
    float *const sA = (float *)(smem + K::O_A);
    In *const sP = (In *)(smem + K::O_P);
    auto bufKr = [&](CI ch) { return (In *)(smem + K::O_KR + (ch & 1) * K::SZ_R); };
    auto bufQr = [&](CI ch) { return (In *)(smem + K::O_QR + (ch & 1) * K::SZ_R); };
    auto bufKt = [&](CI ch) { return (In *)(smem + K::O_KT + (ch & 1) * K::SZ_KT); };
    auto bufSc = [&](CI ch) { return (float *)(smem + K::O_SC + (ch & 1) * K::SZ_SC); };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar) index
    const int n = lane & 15, g = lane >> 4;
    // Work units are (head, segment) pairs, each split into value blocks of BV
    // state rows.  Segments (nsegs > 1): the map launch (MAP) takes every
    // segment but the last and the later launch every segment from its
    // incoming state.  With a lead segment (lead > 0) segment 0 needs no map:
    // its units in the map launch run the whole pass from S0 (outputs
    // included, its final state being segment 1's incoming one), in the first
    // nA workgroups, beside the maps of segments 1 .. nsegs - 2; the later
    // launch then takes segments 1 .. nsegs - 1.
    const int nvA = dv / BV, nvB = (dv + DK) / BV;   // value blocks of a plain / augmented unit
    // Workgroups are dealt to the 8 XCDs round-robin; with the remap (a flag
    // per region) all value blocks of one unit sit on one XCD, so their shared
    // q / k / log_alpha reads hit the same L2.
    auto place = [&](int b, int nvb, bool xcd, int &unit, int &vb_) {
        if (xcd) {
            const int x = b & 7, slot = b >> 3;
            unit = (slot / nvb) * 8 + x;
            vb_ = slot % nvb;
        } else {
            unit = b / nvb;
            vb_ = b % nvb;
        }
    };
    int head, seg, vb;
    bool lead_full = false;                          // the lead segment's whole pass in the map launch
    // mout: the map launch of the schedule without a second pass maps every
    // segment after the first and writes their outputs from a zero incoming
    // state (real rows, into out) and those of the virtual rows (into mws)
    const bool mout = MAP && mout_arg != 0 && lead != 0;
    const int nmap = mout ? nsegs - 1 : nsegs - 2;   // mapped segments per sequence beside the lead one
    int nheads_grid = 0;   // (sequence, head) pairs of the launch, for the device-side split
    if (MAP && lead != 0) {
        nheads_grid = (int)(gridDim.x / (nvA + nmap * nvB));
        const int nA = nheads_grid * nvA;
        int unit;
        if ((int)blockIdx.x < nA) {
            place(blockIdx.x, nvA, xcd_map & 1, unit, vb);
            head = unit;
            seg = 0;
            lead_full = true;
        } else {
            place(blockIdx.x - nA, nvB, xcd_map & 2, unit, vb);
            head = unit / nmap;
            seg = 1 + unit % nmap;
        }
    } else {
        const int nsu = (MAP || lead > 0) ? nsegs - 1 : nsegs;   // segments per sequence in this grid
        int unit;
        place(blockIdx.x, MAP ? nvB : nvA, xcd_map & 1, unit, vb);
        head = unit / nsu;
        seg = unit % nsu + ((!MAP && lead > 0) ? 1 : 0);
    }
    const bool map = MAP && !lead_full;              // augmented state
    const bool noout = map && !mout;                 // ... and no outputs (q not read)
    const int seq = head / H, h = head % H;
    long tok0;
    CI len;   // tokens of this unit (at most T)
    if (cu_seqlens) {   // T is the stream length here; offsets clamped to [0, T] keep every access inside it
        const long a0 = min(max((long)cu_seqlens[seq], 0L), (long)T);
        const long a1 = min(max((long)cu_seqlens[seq + 1], a0), (long)T);
        tok0 = a0;
        len = (CI)(a1 - a0);
    } else {
        tok0 = (long)seq * T;
        len = T;
    }
    if (nsegs > 1) {
        // segment seg: chunks [c0, c1) of the sequence's n.  Uniform: ceil(n /
        // nsegs) each.  Lead: segments 1 .. nsegs - 1 take L = ceil(10 n /
        // (10 (nsegs - 1) + lead)) each from the end, segment 0 the rest (about
        // lead / 10 L; none when the sequence is short).
        long c0, c1;
        if (lead < 0) {   // two segments, split on the device
            const long l0 = ((const int *)(mws + (long)T * H * DK))[seq];   // the plan, after m
            c0 = seg == 0 ? 0 : l0;
            c1 = seg == 0 ? l0 : (len + C - 1) / C;
        } else {
            seg_bounds((len + C - 1) / C, nsegs, lead, seg, c0, c1);
        }
        tok0 += c0 * C;
        len = (CI)max(0L, min((long)len - c0 * C, (c1 - c0) * C));
    }
    const CI nch = (len + C - 1) / C;
    const int HDK = H * DK, HDV = H * dv;
    const long hrow = tok0 * H + h;                 // token rows are H*d elements apart

    // Ktil^T in the paired order along the tokens (its contraction with E in
    // the state update); not in the map pass, where it timed slower
    constexpr bool PAIRT = !K::F32 && K::KC == 32 && !MAP;
    // The off-diagonal A tiles enter the bf16 solve as one bf16 part.  The
    // raw-input kernel rounds them when it stores them (half the LDS bytes;
    // 1.4% faster there, 1% slower on varlen in the plain kernel, which
    // rounds them in the solve instead: the same bits either way).
    constexpr bool ABF = !K::F32 && VAR == 2;
    // The operand waves form the diagonal P tiles along with the diagonal A
    // tiles (always with a single state wave; with more, in the plain kernel
    // and the variants' map pass).  The raw-input kernel and the variants'
    // single pass leave them to the state waves, with their off-diagonal
    // pairs: 1.4% and 2.7% faster there, and the variant kernel then fits its
    // registers without a spill.
    constexpr bool DPOP = K::NBV == 1 || VAR == 0 || (VAR == 1 && MAP);
    // LDS column of channel c of a [token, d_k] operand
    auto kcol = [&](int c) { return K::PAIRK ? K::pair_pos(c) : c; };
    // Fragments of one row of a [token, d_k] operand: x[t] = channels
    // 16 t + 4 g .. 16 t + 4 g + 3
    auto load_krow = [&](V4 (&x)[NDK], const In *row) __attribute__((always_inline)) {
        if constexpr (K::PAIRK) {
            typedef In V8 __attribute__((ext_vector_type(8)));
#pragma unroll
            for (int s2 = 0; s2 < NDK / 2; ++s2) {
                const V8 w = *(const V8 *)(row + 32 * s2 + 8 * g);
                x[2 * s2] = __builtin_shufflevector(w, w, 0, 1, 2, 3);
                x[2 * s2 + 1] = __builtin_shufflevector(w, w, 4, 5, 6, 7);
            }
        } else {
#pragma unroll
            for (int t = 0; t < NDK; ++t) x[t] = *(const V4 *)(row + 16 * t + 4 * g);
        }
    };

    // One lower-triangle tile pair (I, J) of chunk ch: the A tile (beta-scaled,
    // strictly lower on the diagonal) and / or the P tile (lower incl. the
    // diagonal).  Tiles are computed transposed, d[i] = X[16I + n][16J + 4g + i],
    // so each lane stores four consecutive columns of one row.
    auto tile_job = [&](CI ch, int p, bool doA, bool doP, f32x4 *lt = nullptr) __attribute__((always_inline)) {
        // (I, J) of tile p without a loop: off-diagonal tile o = p - NB has row
        // block I = the o-th entry of 1, 2, 2, 3, 3, 3 (four bits each)
        int I = p, J = p;
        if (p >= NB) {
            const int o = p - NB;
            I = (int)((0x333221u >> (4 * o)) & 15u);
            J = o - I * (I - 1) / 2;
        }
        const float *scc = bufSc(ch);
        const float *fl = scc + K::SC_FLAG;
        const bool allfast = all_flags<K::NXW>(fl);
        V4 cf[NDK];
        load_krow(cf, sKd + (16 * J + n) * PK);
        if (!allfast) {   // the pair's column scale: Kc_J s_IJ = k e^{rho_I - G}
            const float *wr = sW + p * DK + 4 * g;
#pragma unroll
            for (int t = 0; t < NDK; ++t) {
                const f32x4 w4 = *(const f32x4 *)(wr + 16 * t);
                cf[t] = to_op<In>(to_f32<In>(cf[t]) * w4);
            }
        }
        if (doA) {
            const In *Kr = bufKr(ch);
            V4 rk[NDK];
            load_krow(rk, Kr + (16 * I + n) * PK);
            const f32x4 da = mma_tiles<K::KD, In, NDK>(zero4(), cf, rk);
            const float b = prep ? beta_hat<K>(scc, 16 * I + n) : scc[K::SC_BETA + 16 * I + n];
            f32x4 va;
#pragma unroll
            for (int i = 0; i < 4; ++i) va[i] = (I > J || 4 * g + i < n) ? da[i] * b : 0.f;
            if (ABF && I > J) {
                *(V4 *)(sA + p * 16 * PT + n * PT + 4 * g) = to_op<In>(va);
            } else {
                *(f32x4 *)(sA + p * 16 * PT + n * PT + 4 * g) = va;
            }
            if (lt) {
                // diagonal tile: also L itself in accumulator layout,
                // lt[0][i] = L[4g + i][n] (and lt[1] = L^T, the tile just stored)
                const f32x4 dl = mma_tiles<K::KD, In, NDK>(zero4(), rk, cf);
                f32x4 b4 = *(const f32x4 *)(scc + K::SC_BETA + 16 * I + 4 * g);
                if (prep) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) b4[i] = beta_hat<K>(scc, 16 * I + 4 * g + i);
                }
                f32x4 vl;
#pragma unroll
                for (int i = 0; i < 4; ++i) vl[i] = (n < 4 * g + i) ? dl[i] * b4[i] : 0.f;
                lt[0] = vl;
                lt[1] = va;
            }
        }
        if (doP) {
            const In *Qr = bufQr(ch);
            V4 rq[NDK];
            load_krow(rq, Qr + (16 * I + n) * PK);
            const f32x4 dp = mma_tiles<K::KD, In, NDK>(zero4(), cf, rq);
            f32x4 vp;
#pragma unroll
            for (int i = 0; i < 4; ++i) vp[i] = (I > J || 4 * g + i <= n) ? dp[i] : 0.f;
            store4(sP + p * 16 * PT + n * PT + 4 * g, vp);
        }
    };

    // Blocks of chunk ch with a key channel too deep to factor (bit I: block I),
    // from the operand waves' masks; workgroup-uniform after the first barrier.
    auto hard_mask = [&](CI ch) __attribute__((always_inline)) {
        static_assert(K::NXW == 4 && K::SC_HARD % 4 == 0, "the four masks are one 16-byte LDS read");
        const f32x4 m4 = *(const f32x4 *)(bufSc(ch) + K::SC_HARD);
        int m = 0;
#pragma unroll
        for (int w = 0; w < K::NXW; ++w) m |= __builtin_bit_cast(int, m4[w]);
        return __builtin_amdgcn_readfirstlane(m);
    };

    auto inv_bf16 = [&](int p, f32x4 lt0, f32x4 lt1, bool keep_l) __attribute__((always_inline)) {
        diag_inverse_bf16(sA + p * 16 * PT, PT, n, g, lt0, lt1, keep_l);
    };
    auto inv_f32 = [&](int p) __attribute__((always_inline)) { diag_inverse_f32(sA + p * 16 * PT, PT, n, lane); };
    auto hard_block = [&](CI ch, int I) {
        hard_block_fn<In, DK, C>(k, q, log_alpha, beta, hrow, (long)ch * C, (long)len, H, gate, add, prep, noout, sW, sA, sP,
                                 bufSc(ch), I);
    };

    if (wave >= K::NBV) {
        // =============== operand waves: chunk t+1 while the state waves run chunk t
        const int xw = wave - K::NBV;
        const int cg = lane % K::NCG, seg = lane / K::NCG;
        const bool act = lane < K::NACT;
        const int c0 = xw * K::CPW + 4 * cg;        // this lane's channels c0 .. c0+3
        const int r0 = seg * RS;                    // and tokens r0 .. r0+RS-1 (inactive lanes: >= C)
        typedef typename V4T<In>::type In4;

        // Global loads, a chunk ahead, through buffer descriptors bounded to the
        // chunk's valid tokens (tokens past the end read as zeros: identity
        // tokens).  Each input of the next chunk is requested as soon as this
        // chunk's copy is no longer needed: log_alpha once it has become decay
        // factors (early in stage A), q after the forward pass, k and beta at
        // the end of stage A.  Token i of this lane sits at the lane's fixed
        // offset plus i token rows (the scalar offset).
        In4 kr[RS], qr[RS], grp[RS];
        f32x4 gr[RS];   // log_alpha; with prep first the raw bits of g, converted in stage A
        float betar = 0.f;
        const int rowb_in = HDK * (int)sizeof(In), rowb_f = HDK * 4;
        const int voff_in = r0 * rowb_in + c0 * (int)sizeof(In), voff_f = r0 * rowb_f + c0 * 4;
        auto chunk_valid = [&](long t0) { const CI r = len - (CI)t0; return (unsigned)(r < C ? r : C); };
        auto prefetch_g = [&](long t0) __attribute__((always_inline)) {
            if (prep) {        // g in the input type, its bits kept in gr until stage A
                const In *gp = (const In *)log_alpha;
                if (gate == 1) {
                    const __amdgpu_buffer_rsrc_t rg = buf_rsrc(gp + hrow + t0 * H, chunk_valid(t0) * H * (int)sizeof(In));
#pragma unroll
                    for (int i = 0; i < RS; ++i) {
                        const In x = buf_load<In>(rg, r0 * H * (int)sizeof(In), i * H * (int)sizeof(In));
                        gr[i][0] = tof(x);
                    }
                } else if (gate == 0) {
                    const __amdgpu_buffer_rsrc_t rg = buf_rsrc(gp + (hrow + t0 * H) * DK, chunk_valid(t0) * rowb_in);
#pragma unroll
                    for (int i = 0; i < RS; ++i) {
                        if constexpr (sizeof(In) == 2) {   // 4 bf16 in the first two dwords
                            grp[i] = buf_load<In4>(rg, voff_in, i * rowb_in);
                        } else {
                            gr[i] = buf_load<f32x4>(rg, voff_in, i * rowb_in);
                        }
                    }
                }
                return;
            }
            if (gate == 1) {   // one value per token, broadcast to the lane's 4 channels
                const __amdgpu_buffer_rsrc_t rg = buf_rsrc(log_alpha + hrow + t0 * H, chunk_valid(t0) * H * 4);
#pragma unroll
                for (int i = 0; i < RS; ++i) {
                    const float x = buf_load<float>(rg, r0 * H * 4, i * H * 4);
                    gr[i] = f32x4{x, x, x, x};
                }
            } else {           // gate 2: an empty descriptor, every load reads 0
                const __amdgpu_buffer_rsrc_t rg = buf_rsrc(gate == 0 ? log_alpha + (hrow + t0 * H) * DK : beta,
                                                          gate == 0 ? chunk_valid(t0) * rowb_f : 0u);
#pragma unroll
                for (int i = 0; i < RS; ++i) gr[i] = buf_load<f32x4>(rg, voff_f, i * rowb_f);
            }
        };
        auto prefetch_q = [&](long t0) __attribute__((always_inline)) {
            if (noout) return;
            const __amdgpu_buffer_rsrc_t rq = buf_rsrc(q + (hrow + t0 * H) * DK, chunk_valid(t0) * rowb_in);
#pragma unroll
            for (int i = 0; i < RS; ++i) qr[i] = buf_load<In4>(rq, voff_in, i * rowb_in);
        };
        auto prefetch_k = [&](long t0) __attribute__((always_inline)) {
            const unsigned nv = chunk_valid(t0);
            if (xw == 0) betar = buf_load<float>(buf_rsrc(beta + hrow + t0 * H, nv * H * 4), lane * H * 4, 0);
            const __amdgpu_buffer_rsrc_t rk = buf_rsrc(k + (hrow + t0 * H) * DK, nv * rowb_in);
#pragma unroll
            for (int i = 0; i < RS; ++i) kr[i] = buf_load<In4>(rk, voff_in, i * rowb_in);
        };

        // The plain kernel scans a chunk's log-decays ahead, at the end of the
        // previous chunk's stage A (its loads are in by then), so the scan's
        // lane shuffles are off the start of the stage.
        constexpr bool PSCAN = VAR == 0;
        float nx_inc[4], nx_gl[4];
        auto scan_g = [&](float (&inc)[4], float (&glast)[4]) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < RS; ++i) acc += gr[i][j];
                inc[j] = acc;
            }
            // inclusive scan of the segment sums over the lanes of one channel group
#pragma unroll
            for (int d = 1; d < K::NSEG; d <<= 1)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float y = __shfl_up(inc[j], d * K::NCG, 64);
                    if (seg >= d) inc[j] += y;
                }
#pragma unroll
            for (int j = 0; j < 4; ++j) glast[j] = __shfl(inc[j], (K::NSEG - 1) * K::NCG + cg, 64);   // G_last
        };

        // ---- stage A: cumulative decay, references, scaled operands
        auto stage_a = [&](CI ch) __attribute__((always_inline)) {
            const long t0 = (long)ch * C;
            const int nval = (int)(len - ch * C < C ? len - ch * C : C);
            if (prep) {   // log_alpha = -softplus(g); no gate: 0
#pragma unroll
                for (int i = 0; i < RS; ++i) {
                    f32x4 gv = gr[i];
                    if (gate == 1) {
                        gv = f32x4{gr[i][0], gr[i][0], gr[i][0], gr[i][0]};
                    } else if constexpr (sizeof(In) == 2) {   // unpack the 4 bf16 of channels c0 .. c0+3
                        gv = f32x4{tof(grp[i][0]), tof(grp[i][1]), tof(grp[i][2]), tof(grp[i][3])};
                    }
                    // rows past the end are identity tokens: log_alpha = 0 there, not -softplus(0)
#pragma unroll
                    for (int j = 0; j < 4; ++j) gr[i][j] = (gate == 2 || r0 + i >= nval) ? 0.f : neg_softplus(gv[j]);
                }
            }
            float tot[4], inc[4], exc[4], glast[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < RS; ++i) acc += gr[i][j];
                tot[j] = acc;
            }
            if constexpr (PSCAN) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    inc[j] = nx_inc[j];
                    glast[j] = nx_gl[j];
                }
            } else {
                scan_g(inc, glast);
            }
            bool fastc[4], lane_fast = true;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                exc[j] = inc[j] - tot[j];                                       // G before my first token
                fastc[j] = glast[j] >= -K::FAST_NATS;
                lane_fast = lane_fast && fastc[j];
            }
            const bool wave_fast = __all(lane_fast);
            // Exponents at the start of the forward (prefix) pass, of the backward
            // (suffix) pass for Ktil, and (block-referenced channels) of the
            // backward pass for the column operand; block sums of log_alpha.
            float pst[4], sst[4], bst[4], Bt[NB][4];
            if (wave_fast) {   // every channel of the wave takes the chunk-start reference
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pst[j] = exc[j];
                    sst[j] = glast[j] - inc[j];
                    bst[j] = 0.f;
#pragma unroll
                    for (int I = 0; I < NB; ++I) Bt[I][j] = 0.f;
                }
            } else {
                // Block-local scans of the lane sums: every exponent below is a sum
                // of log-decays, never a difference of cumulative ones, so a deep
                // decay earlier in the chunk costs no precision later.
                constexpr int LPB = 16 / RS;            // lanes of one channel group per 16-token block
                const int sib = seg % LPB, myI = r0 / 16;
                float incb[4], sufb[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    incb[j] = tot[j];
                    sufb[j] = tot[j];
                }
#pragma unroll
                for (int d = 1; d < LPB; d <<= 1)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float y = __shfl_up(incb[j], d * K::NCG, 64);
                        const float z = __shfl_down(sufb[j], d * K::NCG, 64);
                        if (sib >= d) incb[j] += y;
                        if (sib + d < LPB) sufb[j] += z;
                    }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float y = __shfl_up(incb[j], K::NCG, 64);
                    const float z = __shfl_down(sufb[j], K::NCG, 64);
                    const float excb = sib > 0 ? y : 0.f;          // my block's decay before my tokens
                    const float sufx = sib < LPB - 1 ? z : 0.f;    // ... and after them
                    float aft = 0.f;                               // the later blocks' decay
#pragma unroll
                    for (int I = 0; I < NB; ++I) {
                        Bt[I][j] = __shfl(incb[j], ((I + 1) * LPB - 1) * K::NCG + cg, 64);
                        if (I > myI) aft += Bt[I][j];
                    }
                    pst[j] = fastc[j] ? exc[j] : excb;
                    sst[j] = fastc[j] ? glast[j] - inc[j] : sufx + aft;
                    bst[j] = sufx;
                }
            }
            // per-channel scales, one 4-channel vector store per lane: e^{G_last}
            // by the first segment's lanes, e^{rho_I} by segment I, the column
            // scale s_p of tile pair p by segment p mod NSEG.  For a block-
            // referenced channel (rho_I = G before block I, B_I = block I's decay)
            //   s_IJ = e^{B_{J+1} + .. + B_{I-1}} (J < I, <= 1),  s_II = e^{-B_I};
            // a channel whose decay inside block I is too deep for e^{-B_I}
            // (B_I < -80) gets s_II = 0 and its pairs of that diagonal tile are
            // formed apart (the hard-block correction).  Chunk-start channels
            // take 1 everywhere.  The scales are stored also when all are 1: other
            // waves may take block references, and then the tiles read them for
            // every channel.
            float *sc = bufSc(ch);
            int hard = 0;   // blocks with a channel too deep to factor (bit I)
            if (!wave_fast) {   // (all factors 1: stored at the end of the stage)
#pragma unroll
                for (int I = 0; I < NB; ++I) {
                    if (seg == I) {
                        f32x4 e;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            float rho = 0.f;
#pragma unroll
                            for (int m = 0; m < I; ++m) rho += Bt[m][j];
                            e[j] = fastc[j] ? 1.f : fexp(rho);
                        }
                        *(f32x4 *)(sc + I * DK + c0) = e;
                    }
#pragma unroll
                    for (int J = 0; J <= I; ++J) {
                        const int p = tile_index(NB, I, J);
                        if (seg == p % K::NSEG) {
                            f32x4 w;
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                float x = 0.f;
#pragma unroll
                                for (int m = J + 1; m < I; ++m) x += Bt[m][j];
                                const float sd = Bt[I][j] >= -K::FAST_NATS ? fexp(-Bt[I][j]) : 0.f;
                                w[j] = fastc[j] ? 1.f : (J < I ? fexp(x) : sd);
                            }
                            *(f32x4 *)(sW + p * DK + c0) = w;
                        }
                    }
                    bool deep = false;
#pragma unroll
                    for (int j = 0; j < 4; ++j) deep = deep || (!fastc[j] && Bt[I][j] < -K::FAST_NATS);
                    if (__ballot(act && deep) != 0) hard |= 1 << I;
                }
            }
            float al[RS][4];
#pragma unroll
            for (int i = 0; i < RS; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) al[i][j] = fexp(gr[i][j]);   // alpha of each token
            // gr is free: request the next chunk's log_alpha now (the empty asm
            // keeps the loads from being hoisted above the uses of gr)
            __asm__ volatile("" ::: "memory");
            if (ch + 1 < nch) prefetch_g(t0 + C);
            In *Kr = bufKr(ch), *Qr = bufQr(ch), *Kt = bufKt(ch);
            // forward over my tokens: e^{G - rho} by prefix products -> Kr, Qr
            {
                float pp[4];
                float sk[RS], sq[RS];   // prep: squared norms over this wave's channels
#pragma unroll
                for (int j = 0; j < 4; ++j) pp[j] = fexp(pst[j]);
#pragma unroll
                for (int i = 0; i < RS; ++i) {
                    f32x4 vkr, vqr;
                    sk[i] = 0.f;
                    sq[i] = 0.f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        pp[j] *= al[i][j];
                        const float kf = tof(kr[i][j]);
                        vkr[j] = kf * pp[j];                       // k e^{G - ref}
                        if (!noout) vqr[j] = tof(qr[i][j]) * pp[j];   // q e^{G - ref}
                        if (prep) {
                            sk[i] += kf * kf;
                            if (!noout) sq[i] += tof(qr[i][j]) * tof(qr[i][j]);
                        }
                    }
                    if (act) {
                        const int r = r0 + i;
                        store4(Kr + r * PK + kcol(c0), vkr);
                        if (!noout) store4(Qr + r * PK + kcol(c0), vqr);
                    }
                }
                if (prep) {   // per token over the channel group's lanes, stored by its first lane
#pragma unroll
                    for (int i = 0; i < RS; ++i) {
                        sk[i] = group_sum<K::NCG>(sk[i]);
                        sq[i] = group_sum<K::NCG>(sq[i]);
                    }
                    if (act && cg == 0) {
#pragma unroll
                        for (int i = 0; i < RS; ++i) {
                            sc[K::SC_PK + (r0 + i) * K::NXW + xw] = sk[i];
                            sc[K::SC_PQ + (r0 + i) * K::NXW + xw] = sq[i];
                        }
                    }
                }
            }
            // q is free: request the next chunk's q
            __asm__ volatile("" ::: "memory");
            if (ch + 1 < nch) prefetch_q(t0 + C);
            // backward: e^{G_last - G} by suffix products -> Ktil, and the column
            // operand Kc: Ktil e^{-G_last} = k e^{-G} for channels referenced to the
            // chunk start, k e^{rho_{I+1} - G} (the block's own suffix products,
            // <= |k|) for block-referenced ones
            {
                float sf[4], gli[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    sf[j] = fexp(sst[j]);
                    gli[j] = fexp(-glast[j]);   // used for chunk-start channels only (G_last >= -80)
                }
                In kt[4][RS];
                if (wave_fast) {   // a uniform branch: the common case keeps its short loop
#pragma unroll
                    for (int i = RS - 1; i >= 0; --i) {
                        f32x4 vkd;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float ktf = tof(kr[i][j]) * sf[j];   // k e^{G_last - G}
                            kt[j][i] = fromf<In>(ktf);
                            vkd[j] = ktf * gli[j];                     // k e^{-G}
                            sf[j] *= al[i][j];
                        }
                        if (act) store4(sKd + (r0 + i) * PK + kcol(c0), vkd);
                    }
                } else {
                    float sb[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) sb[j] = fexp(bst[j]);
#pragma unroll
                    for (int i = RS - 1; i >= 0; --i) {
                        f32x4 vkd;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float kf = tof(kr[i][j]);
                            const float ktf = kf * sf[j];
                            kt[j][i] = fromf<In>(ktf);
                            vkd[j] = fastc[j] ? ktf * gli[j] : kf * sb[j];
                            sf[j] *= al[i][j];
                            sb[j] *= al[i][j];
                        }
                        if (act) store4(sKd + (r0 + i) * PK + kcol(c0), vkd);
                    }
                }
                if (act) {
                    if constexpr (PAIRT) {   // tokens in the paired order: pieces of up to four
                        constexpr int W = RS < 4 ? RS : 4;
#pragma unroll
                        for (int j = 0; j < 4; ++j)
#pragma unroll
                            for (int i0 = 0; i0 < RS; i0 += W) {
                                In *dst = Kt + Panel<In, 16>::swz_index(c0 + j, K::pair_pos(r0 + i0), PC, K::SWZ);
                                if constexpr (W == 1) {
                                    *dst = kt[j][i0];
                                } else {
                                    typedef In VW __attribute__((ext_vector_type(W)));
                                    VW x;
#pragma unroll
                                    for (int i = 0; i < W; ++i) x[i] = kt[j][i0 + i];
                                    *(VW *)dst = x;
                                }
                            }
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) store_row_swz<In, RS>(Kt, c0 + j, r0, PC, K::SWZ, kt[j]);
                    }
                }
            }
            if (seg == 0) *(f32x4 *)(sc + K::SC_GL + c0) = f32x4{fexp(glast[0]), fexp(glast[1]), fexp(glast[2]), fexp(glast[3])};
            if (wave_fast) {   // a uniform branch: no exponentials when every factor is 1
                const f32x4 one{1.f, 1.f, 1.f, 1.f};
                if (seg < NB) *(f32x4 *)(sc + seg * DK + c0) = one;
#pragma unroll
                for (int p = 0; p < K::NPAIR; p += K::NSEG)
                    if (p + seg < K::NPAIR) *(f32x4 *)(sW + (p + seg) * DK + c0) = one;
            }
            if (lane == 0) {
                sc[K::SC_FLAG + xw] = wave_fast ? 1.f : 0.f;
                sc[K::SC_HARD + xw] = __builtin_bit_cast(float, hard);
            }
            if (xw == 0 && lane < C) sc[K::SC_BETA + lane] = (lane < nval) ? betar : 0.f;
            if (PSCAN && ch + 1 < nch) scan_g(nx_inc, nx_gl);
        };

        // ---- stage B: the diagonal A tiles and their block inverses, with the
        //      diagonal P tiles (DPOP; a single state wave also leaves the
        //      off-diagonal A tiles here)
        auto stage_b = [&](CI ch, int hard) __attribute__((always_inline)) {
            if (prep && xw == 0 && lane < C) {
                // per-token factors for the state waves' next chunk: beta / |k|^2,
                // |k| and 1 / |q| (zero vectors give 0)
                float *sc = bufSc(ch);
                float sk = 0.f, sq = 0.f;
#pragma unroll
                for (int w = 0; w < K::NXW; ++w) {
                    sk += sc[K::SC_PK + lane * K::NXW + w];
                    sq += sc[K::SC_PQ + lane * K::NXW + w];
                }
                sc[K::SC_BH + lane] = sk > 0.f ? sc[K::SC_BETA + lane] * __builtin_amdgcn_rcpf(sk) : 0.f;
                sc[K::SC_KN + lane] = __builtin_sqrtf(sk);
                sc[K::SC_QI + lane] = sq > 0.f ? __builtin_amdgcn_rsqf(sq) : 0.f;
            }
            if (add) {   // no A: only the diagonal P tiles
                if (DPOP && !noout) {
                    for (int p = xw; p < NB; p += K::NXW) tile_job(ch, p, false, true);
                }
                return;
            }
            // a diagonal tile of a hard block keeps L here: the hard-block
            // correction completes it and inverts it after the next barrier
            auto job = [&](int p) __attribute__((always_inline)) {
                if (p < NB && !K::F32) {
                    f32x4 lt[2];
                    tile_job(ch, p, true, DPOP && !noout, lt);
                    inv_bf16(p, lt[0], lt[1], (hard >> p) & 1);
                } else if (p < NB) {
                    tile_job(ch, p, true, DPOP && !noout);
                    if (!((hard >> p) & 1)) inv_f32(p);
                } else {
                    tile_job(ch, p, true, false);
                }
            };
            constexpr int NJB = K::NBV == 1 ? K::NPAIR : NB;
            if constexpr (NJB <= K::NXW) {   // at most one job per wave: straight-line code
                if (xw < NJB) job(xw);
            } else {
                for (int p = xw; p < NJB; p += K::NXW) job(p);
            }
        };

        // Same barrier sequence as the state waves: two per step, steps -1 .. nch - 1
        // (step -1 prepares chunk 0; one copy of each stage keeps the code small),
        // and one more after the tiles of a chunk with hard blocks (the state
        // waves' hard-block correction).
        if (nch > 0) {
            prefetch_g(0);
            prefetch_q(0);
            prefetch_k(0);
            if (PSCAN) scan_g(nx_inc, nx_gl);
        }
        // Stage A sets the pace of the first segment, where each operand wave
        // shares its SIMD with a state wave that has time to spare: the operand
        // waves issue first there (wave priority, this workgroup only).  In the
        // raw-input kernel, whose operand waves carry the input preparation,
        // they keep the priority through stage B as well (0.7% faster there,
        // 2% slower in the others).
        for (CI ch = -1; ch < nch; ++ch) {
            __builtin_amdgcn_s_setprio(3);
            if (ch + 1 < nch) {
                stage_a(ch + 1);
                if (ch + 2 < nch) prefetch_k((ch + 2) * C);
            }
            if constexpr (VAR != 2) __builtin_amdgcn_s_setprio(0);
            __syncthreads();
            const int hard = ch + 1 < nch ? hard_mask(ch + 1) : 0;
            if (ch + 1 < nch) stage_b(ch + 1, hard);
            if (hard) __syncthreads();
            __syncthreads();
        }
    } else {
        // =============== state waves: value rows 16 cb .. 16 cb + 15 of the block
        const int cb = wave;
        __builtin_assume(cb >= 0 && cb < K::NBV);
        const int row = vb * BV + 16 * cb + n;     // this lane's state row (of the augmented state in MAP mode)
        const bool vreal = !map || vb * BV < dv;   // real value rows (virtual ones see v = 0)
        // bf16: lane (n, g) loads row 16 (2 u + g/2) + n, columns 8 (g&1) .. +7;
        // fp32: row 16 u + n, columns 4g .. 4g+3 (u = load index)
        const int rowb_v = HDV * (int)sizeof(In);
        const int voff_v = (K::F32 ? n : (16 * (g >> 1) + n)) * rowb_v + (K::F32 ? 4 * g : 8 * (g & 1)) * (int)sizeof(In);
        const long vcol = hrow * dv + vb * BV + 16 * cb;
        // outputs: out (real rows), or mws [tokens, H, DK] for the virtual rows of a map with outputs
        In *const obase = vreal ? out + vcol : mws + hrow * DK + (vb * BV - dv) + 16 * cb;
        const int opitch = vreal ? HDV : HDK;
        const int rowb_o = opitch * (int)sizeof(In);
        const int voff_o = n * rowb_o + 4 * g * (int)sizeof(In);   // output row 16 I + n, columns 4g .. 4g+3

        // State, transposed, in accumulator layout: Sacc[ct][i] = S[16 cb + n][16 ct + 4g + i].
        // Where it comes from and goes to: S0 / S_final for a whole sequence;
        // the segment's incoming state / S_final (last segment only) for a
        // segment; zero or the identity / the segment's map in MAP mode; S0 /
        // segment 1's incoming state for the lead segment in the map launch.
        f32x4 Sacc[NDK];
        const float *s0row = nullptr;
        float *sfrow = nullptr;
        if (map) {
            sfrow = seg_map + (((long)head * (mout ? nsegs : nsegs - 1) + seg) * (dv + DK) + row) * DK;
        } else if (MAP) {
            if (S0) s0row = S0 + ((long)head * dv + row) * DK;
            sfrow = seg_start + (((long)head * nsegs + 1) * dv + row) * DK;
        } else if (nsegs > 1) {
            s0row = seg_start + (((long)head * nsegs + seg) * dv + row) * DK;
            if (seg == nsegs - 1 && S_final) sfrow = S_final + ((long)head * dv + row) * DK;
        } else {
            if (S0) s0row = S0 + ((long)head * dv + row) * DK;
            if (S_final) sfrow = S_final + ((long)head * dv + row) * DK;
        }
#pragma unroll
        for (int ct = 0; ct < NDK; ++ct) {
            if (map) {
#pragma unroll
                for (int i = 0; i < 4; ++i) Sacc[ct][i] = (row - dv == 16 * ct + 4 * g + i) ? 1.f : 0.f;
            } else {
                Sacc[ct] = s0row ? *(const f32x4 *)(s0row + 16 * ct + 4 * g) : zero4();
            }
        }

        // V of the chunk, prefetched a chunk ahead; an MFMA against an identity
        // fragment moves it into accumulator layout.
        constexpr int NVL = K::F32 ? NB : (NB + 1) / 2;
        typedef In VL __attribute__((ext_vector_type(K::F32 ? 4 : 8)));
        VL vr[NVL];
        auto prefetch_v = [&](long t0) __attribute__((always_inline)) {
            const CI rv_ = len - (CI)t0;
            const unsigned nv = vreal ? (unsigned)(rv_ < C ? rv_ : C) : 0u;
            const __amdgpu_buffer_rsrc_t rv = buf_rsrc(v + (vreal ? vcol + t0 * HDV : 0), nv * rowb_v);
#pragma unroll
            for (int u = 0; u < NVL; ++u) vr[u] = buf_load<VL>(rv, voff_v, (K::F32 ? 16 : 32) * u * rowb_v);
        };
        // identity fragments: k-slot s of the lane's operand -> column n
        VL ident[K::F32 ? 1 : 2];
#pragma unroll
        for (int e = 0; e < (K::F32 ? 4 : 8); ++e) {
            if constexpr (K::F32) {
                ident[0][e] = (4 * g + e == n) ? 1.f : 0.f;
            } else {
                ident[0][e] = fromf<In>((8 * g + e == n) ? 1.f : 0.f);
                ident[1][e] = fromf<In>((8 * g + e - 16 == n) ? 1.f : 0.f);
            }
        }
        // Tiles the state waves form for a chunk, in their second segment: with
        // two or more state waves the off-diagonal pairs (A and P, and then the
        // diagonal P tiles when the operand waves leave them), else the
        // off-diagonal P tiles (MAP mode: no P tiles).  Jobs are dealt in snake
        // order so the heavier pairs spread evenly over the waves.
        // When the operand waves keep the diagonal tiles (and there is no map),
        // each off-diagonal pair is dealt as two jobs, its A tile and its P tile,
        // so that the waves' shares differ by at most one tile.
        constexpr bool SPLITJ = K::NBV >= 2 && DPOP && !MAP;
        const bool split = SPLITJ && !add;
        constexpr int NJOB_MAP = K::NBV >= 2 ? K::NOFF : 0, NJOB_FULL = (K::NBV >= 2 && !DPOP) ? K::NPAIR : K::NOFF;
        const int njob = split ? 2 * K::NOFF : (noout ? NJOB_MAP : NJOB_FULL);
        constexpr int NJOB_MAX = SPLITJ ? 2 * K::NOFF : NJOB_FULL;   // NJOB_MAP <= NJOB_FULL
        constexpr int NROUND = (NJOB_MAX + K::NBV - 1) / K::NBV;
        auto y_tiles = [&](CI ch) __attribute__((always_inline)) {
#pragma unroll
            for (int r = 0; r < NROUND; ++r) {
                const int s = r * K::NBV + ((r & 1) ? K::NBV - 1 - cb : cb);
                if (s < njob) {
                    if (split) {
                        tile_job(ch, NB + (s >> 1), (s & 1) == 0, (s & 1) != 0);
                    } else {
                        const int p = s < K::NOFF ? NB + s : s - K::NOFF;
                        tile_job(ch, p, K::NBV >= 2 && p >= NB && !add, !noout);
                    }
                }
            }
        };
        // Chunks with hard blocks take one more barrier after their tiles; then
        // the state waves correct those blocks' diagonal tiles.
        auto hard_phase = [&](CI ch, int hm) __attribute__((always_inline)) {
            if (hm) {
                __syncthreads();
                for (int I = cb; I < NB; I += K::NBV)
                    if ((hm >> I) & 1) hard_block(ch, I);
            }
        };
        if (nch > 0) prefetch_v(0);

        V4 Eb[NB];   // corrected errors of the chunk, operand type: E[16b + 4g + i][n]
        for (CI ch = -1; ch < nch; ++ch) {   // step -1: only the tiles of chunk 0
            if (ch >= 0) {
                const long t0 = (long)ch * C;
                const int nval = (int)(len - ch * C < C ? len - ch * C : C);
                const In *Kr = bufKr(ch), *Qr = bufQr(ch);
                const float *sc = bufSc(ch);
                const float *fl = sc + K::SC_FLAG;
                const bool allfast = all_flags<K::NXW>(fl);
                // ---- R = beta (V - Kbar S^T) and (Qbar S^T)^T, per 16-token block I
                // VFOLD: V enters accumulator layout first and R accumulates onto it
                // with the state negated (R = V - Kbar S^T with no subtraction; O1
                // then holds -(Qbar S^T)^T).  Only where the V product and the row
                // products share one MFMA shape; the plain kernel only (0.6% faster
                // there, 2% slower with raw inputs).
                constexpr bool VFOLD = (K::F32 || K::KD == 32) && VAR == 0;
                f32x4 R[NB], O1[NB];
                V4 ss[NDK];
                if constexpr (VFOLD) {
#pragma unroll
                    for (int I = 0; I < NB; ++I) {
                        f32x4 vt;                                       // V[16I + 4g + i][n]
                        if constexpr (K::F32) {
                            const V4 va[1] = {vr[I]}, vi[1] = {ident[0]};
                            vt = mma_tiles<4, In, 1>(zero4(), va, vi);
                        } else {
                            vt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr[I / 2], ident[I & 1], zero4(), 0, 0, 0);
                        }
                        if (prep) vt = vt * *(const f32x4 *)(sc + K::SC_KN + 16 * I + 4 * g);   // |k| v
                        R[I] = vt;
                    }
                }
                auto rows = [&](int I) __attribute__((always_inline)) {
                    V4 ak[NDK], bq[NDK];
                    if (!add) load_krow(ak, Kr + (16 * I + n) * PK);
                    if (!noout) load_krow(bq, Qr + (16 * I + n) * PK);
                    if constexpr (VFOLD) {
                        if (!add) R[I] = mma_tiles<K::KD, In, NDK>(R[I], ak, ss);    // V - Kbar S^T
                    } else {
                        R[I] = add ? zero4() : mma_tiles<K::KD, In, NDK>(zero4(), ak, ss);    // [16I + 4g + i][n]
                    }
                    if (!noout) O1[I] = mma_tiles<K::KD, In, NDK>(zero4(), ss, bq);   // [v = 4g + i][16I + n]
                };
                if (allfast) {
#pragma unroll
                    for (int ct = 0; ct < NDK; ++ct) ss[ct] = to_op<In>(VFOLD ? -Sacc[ct] : Sacc[ct]);
#pragma unroll
                    for (int I = 0; I < NB; ++I) rows(I);
                } else {
#pragma unroll
                    for (int I = 0; I < NB; ++I) {
#pragma unroll
                        for (int ct = 0; ct < NDK; ++ct) {
                            const f32x4 er = *(const f32x4 *)(sc + I * DK + 16 * ct + 4 * g);
                            ss[ct] = to_op<In>(Sacc[ct] * (VFOLD ? -er : er));   // S Diag(e^{rho_I}), transposed
                        }
                        rows(I);
                    }
                }
#pragma unroll
                for (int I = 0; I < NB; ++I) {
                    const f32x4 b4 = *(const f32x4 *)(sc + (prep ? K::SC_BH : K::SC_BETA) + 16 * I + 4 * g);
                    if constexpr (VFOLD) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) R[I][i] *= b4[i];
                        continue;
                    }
                    f32x4 vt;                                           // V[16I + 4g + i][n]
                    if constexpr (K::F32) {
                        const V4 va[1] = {vr[I]}, vi[1] = {ident[0]};
                        vt = mma_tiles<4, In, 1>(zero4(), va, vi);
                    } else {
                        vt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr[I / 2], ident[I & 1], zero4(), 0, 0, 0);
                    }
                    if (prep) vt = vt * *(const f32x4 *)(sc + K::SC_KN + 16 * I + 4 * g);   // |k| v
#pragma unroll
                    for (int i = 0; i < 4; ++i) R[I][i] = b4[i] * (vt[i] - R[I][i]);
                }
                if (ch + 1 < nch) prefetch_v(t0 + C);

                // ---- (I + A) E = R, block forward substitution (additive write: E = R)
                if (add) {
#pragma unroll
                    for (int b = 0; b < NB; ++b) Eb[b] = to_op<In>(R[b]);
                } else {
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        f32x4 y = zero4();
#pragma unroll
                        for (int J = 0; J < b; ++J) {
                            const float *at = sA + tile_index(NB, b, J) * 16 * PT + n * PT + 4 * g;
                            if constexpr (K::F32) {
                                y = mma_fp32a<In>(y, *(const f32x4 *)at, Eb[J]);
                            } else {   // bf16 A (no lo part)
                                const V4 aa[1] = {ABF ? *(const V4 *)at : to_op<In>(*(const f32x4 *)at)}, bb[1] = {Eb[J]};
                                y = mma_tiles<16, In, 1>(y, aa, bb);
                            }
                        }
                        const f32x4 d = *(const f32x4 *)(sA + b * 16 * PT + n * PT + 4 * g);
                        f32x4 e;
                        if constexpr (K::F32) {
                            e = mma_fp32ab<In>(d, R[b] - y);
                        } else {   // D stored pre-split: hi then lo bf16 parts in the tile's 16 bytes
                            const V4 dh = __builtin_bit_cast(V4, f32x2{d[0], d[1]}), dl = __builtin_bit_cast(V4, f32x2{d[2], d[3]});
                            const f32x4 x = R[b] - y;
                            const V4 xh = to_op<In>(x), xl = to_op<In>(x - to_f32<In>(xh));
                            const V4 a3[3] = {dh, dh, dl}, x3[3] = {xh, xl, xh};
                            e = mma_tiles<16, In, 3>(zero4(), a3, x3);
                        }
                        Eb[b] = to_op<In>(e);
                    }
                }

                // ---- O^T = (Qbar S^T)^T + E^T P^T, written as O rows (rows past the end dropped)
                const __amdgpu_buffer_rsrc_t ro = buf_rsrc(obase + t0 * opitch, (unsigned)nval * rowb_o);
#pragma unroll
                for (int I = 0; I < (noout ? 0 : NB); ++I) {
                    V4 pb[NB];
#pragma unroll
                    for (int J = 0; J < NB; ++J)
                        pb[J] = (J <= I) ? *(const V4 *)(sP + tile_index(NB, I, J) * 16 * PT + n * PT + 4 * g) : V4{};
                    f32x4 po = zero4();
                    if constexpr (!MAP && K::KC == 32) {   // pairs of tiles past the diagonal are zero: skipped
#pragma unroll
                        for (int s2 = 0; s2 < NB / 2; ++s2)
                            if (2 * s2 <= I) {
                                const V4 e2[2] = {Eb[2 * s2], Eb[2 * s2 + 1]}, p2[2] = {pb[2 * s2], pb[2 * s2 + 1]};
                                po = mma_tiles<32, In, 2>(po, e2, p2);
                            }
                    } else {
                        po = mma_tiles<K::KC, In, NB>(zero4(), Eb, pb);
                    }
                    f32x4 o = VFOLD ? po - O1[I] : O1[I] + po;   // O[16I + n][16cb + 4g + i]
                    if (prep) o = o * sc[K::SC_QI + 16 * I + n];                   // / |q|
                    buf_store(to_op<In>(o), ro, voff_o, 16 * I * rowb_o);
                }
                // ---- S^T <- Diag(e^{G_last}) S^T + Ktil^T E (Ktil and the scales of this chunk are
                //      double-buffered, so this needs no barrier)
                const In *Kt = bufKt(ch);
#pragma unroll
                for (int ct = 0; ct < NDK; ++ct) {
                    const f32x4 gl = *(const f32x4 *)(sc + K::SC_GL + 16 * ct + 4 * g);
                    V4 ka[NB];
                    if constexpr (PAIRT) {   // tokens 16 b + 4 g .. + 3 of blocks 2 s2, 2 s2 + 1 in one read
                        typedef In V8 __attribute__((ext_vector_type(8)));
#pragma unroll
                        for (int s2 = 0; s2 < NB / 2; ++s2) {
                            const V8 w = *(const V8 *)(Kt + Panel<In, 16>::swz_index(16 * ct + n, 32 * s2 + 8 * g, PC, K::SWZ));
                            ka[2 * s2] = __builtin_shufflevector(w, w, 0, 1, 2, 3);
                            ka[2 * s2 + 1] = __builtin_shufflevector(w, w, 4, 5, 6, 7);
                        }
                    } else {
#pragma unroll
                        for (int b = 0; b < NB; ++b)
                            ka[b] = *(const V4 *)(Kt + Panel<In, 16>::swz_index(16 * ct + n, 16 * b + 4 * g, PC, K::SWZ));
                    }
                    Sacc[ct] = mma_tiles<K::KC, In, NB>(Sacc[ct] * gl, ka, Eb);
                }
            }
            __syncthreads();

            // ---- the next chunk's tiles (the hard-block mask is read first, so
            //      its latency hides behind them)
            const int hm = ch + 1 < nch ? hard_mask(ch + 1) : 0;
            if (ch + 1 < nch) y_tiles(ch + 1);
            if (ch + 1 < nch) hard_phase(ch + 1, hm);
            __syncthreads();
        }
        if (sfrow) {
#pragma unroll
            for (int ct = 0; ct < NDK; ++ct) *(f32x4 *)(sfrow + 16 * ct + 4 * g) = Sacc[ct];
        }
    }
}

// Incoming states of the segments of every (sequence, head): slot 0 holds S0
// (zero when absent), slot p + 1 = slot p M_p + N_p, row by row, with (M_p,
// N_p) the map of segment p from the MAP pass.  fp32 throughout, the products
// as fp32 MFMAs: one workgroup per 16 state rows s of a head, and per step
// D = M_p^T s^T + N_p^T, so that wave w's accumulator tiles (key-channel
// tiles w, w + 4, ...) hold the new rows in exactly the layout the next
// step's products read them in.  The rows go through LDS once per step (every
// wave needs all of them); M_p is staged in LDS with coalesced 16-byte loads,
// and the next map's loads are issued before this step's products.
//
// mout (the schedule without a second pass): every segment p >= 1 has a map,
// at slot p of nsegs per head, and the last one carries the state on to
// S_final (skipped when S_final is NULL).
//
// Device-side split of packed sequences (plan non-NULL): a sequence the plan
// left whole has an identity map; its final state is its incoming slot 1, copied.
template <int DK>
__global__ void __launch_bounds__(256) seg_compose_kernel(const float *S0, const float *seg_map,
                                                          float *seg_start, int dv, int nsegs, int p0,
                                                          int mout, float *S_final, const int *cu_seqlens,
                                                          int T, int C, int H, const int *plan)
{
    constexpr int NCT = DK / 16;                 // key-channel tiles
    constexpr int TPW = (NCT + 3) / 4;           // tiles per wave, at most
    constexpr int PM = DK + 4;                   // LDS row pitch (floats)
    constexpr int NLD = DK * DK / (4 * 256);     // 16-byte loads of a map per thread (DK >= 32)
    constexpr int NLDX = NLD > 0 ? NLD : 1;
    __shared__ __attribute__((aligned(16))) float sM[DK * PM];
    __shared__ __attribute__((aligned(16))) float sS[16 * PM];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, g = lane >> 4;
    const int nrb = dv / 16;
    const int head = blockIdx.x / nrb, rb = blockIdx.x % nrb;
    const int mstride = mout ? nsegs : nsegs - 1;
    // the incoming rows 16 rb .. 16 rb + 15 of slot p0
    for (int e = 4 * tid; e < 16 * DK; e += 4 * 256) {
        const int r = e / DK, c = e % DK;
        const long row = (long)head * dv + 16 * rb + r;
        f32x4 x = zero4();
        if (p0 > 0) x = *(const f32x4 *)(seg_start + (((long)head * nsegs + p0) * dv + 16 * rb + r) * DK + c);
        else if (S0) x = *(const f32x4 *)(S0 + row * DK + c);
        *(f32x4 *)(sS + r * PM + c) = x;
    }
    // map loads: element 4 (tid + 256 j) of M, row-major [DK][DK]
    f32x4 ml[NLDX];
    f32x4 nl[TPW];   // and this wave's tiles of N_p's rows 16 rb ..
    auto load_map = [&](int p) __attribute__((always_inline)) {
        const float *Np = seg_map + ((long)head * mstride + p) * (dv + DK) * DK + (long)(16 * rb) * DK;
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int ct = wave + 4 * u;
            if (ct < NCT) nl[u] = *(const f32x4 *)(Np + (long)n * DK + 16 * ct + 4 * g);
        }
        const float *M = seg_map + ((long)head * mstride + p) * (dv + DK) * DK + (long)dv * DK;
        if constexpr (NLD > 0) {
#pragma unroll
            for (int j = 0; j < NLD; ++j) ml[j] = *(const f32x4 *)(M + 4 * (tid + 256 * j));
        } else {
            if (4 * tid < DK * DK) ml[0] = *(const f32x4 *)(M + 4 * tid);
        }
    };
    auto store_map = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NLDX; ++j) {
            const int e = 4 * (tid + 256 * j);
            if (e < DK * DK) *(f32x4 *)(sM + (e / DK) * PM + e % DK) = ml[j];
        }
    };
    bool whole = false;   // a packed sequence the device-side split left whole
    if (plan) {
        const int seq = head / H;
        const long a0 = min(max((long)cu_seqlens[seq], 0L), (long)T);
        const long a1 = min(max((long)cu_seqlens[seq + 1], a0), (long)T);
        whole = plan[seq] >= (a1 - a0 + C - 1) / C;
    }
    const bool more = !whole && (p0 + 1 < nsegs || (mout && S_final));
    if (more) load_map(p0);
    for (int p = p0;; ++p) {
        __syncthreads();   // the rows of slot p are in sS
        // slot p out
        for (int e = 4 * tid; e < 16 * DK; e += 4 * 256) {
            const int r = e / DK, c = e % DK;
            *(f32x4 *)(seg_start + (((long)head * nsegs + p) * dv + 16 * rb + r) * DK + c) = *(const f32x4 *)(sS + r * PM + c);
        }
        const bool last = p + 1 >= nsegs;
        if (whole) {   // the incoming slot is the final state
            if (mout && S_final) {
                for (int e = 4 * tid; e < 16 * DK; e += 4 * 256) {
                    const int r = e / DK, c = e % DK;
                    *(f32x4 *)(S_final + ((long)head * dv + 16 * rb + r) * DK + c) = *(const f32x4 *)(sS + r * PM + c);
                }
            }
            break;
        }
        if (last && !(mout && S_final)) break;
        store_map();        // M_p (the threads' own loads)
        f32x4 ncur[TPW];
#pragma unroll
        for (int u = 0; u < TPW; ++u) ncur[u] = nl[u];
        const bool next = !last && (p + 2 < nsegs || (mout && S_final));
        if (next) load_map(p + 1);   // in flight across this step
        __syncthreads();
        f32x4 acc[TPW];
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int ct = wave + 4 * u;
            if (ct >= NCT) break;
            // D^T tile: lane (n, g) accumulates s_new[n][16 ct + 4 g + i]
            acc[u] = ncur[u];
#pragma unroll
            for (int t = 0; t < NCT; ++t) {
                const f32x4 b = *(const f32x4 *)(sS + n * PM + 16 * t + 4 * g);   // s[n][16 t + 4 g + i]
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(sM[(16 * t + 4 * g + i) * PM + 16 * ct + n], b[i],
                                                                  acc[u], 0, 0, 0);
            }
        }
        __syncthreads();   // every wave is done reading sS and sM
        if (last) {   // mout: the final state
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int ct = wave + 4 * u;
                if (ct >= NCT) break;
                *(f32x4 *)(S_final + ((long)head * dv + 16 * rb + n) * DK + 16 * ct + 4 * g) = acc[u];
            }
            break;
        }
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int ct = wave + 4 * u;
            if (ct >= NCT) break;
            *(f32x4 *)(sS + n * PM + 16 * ct + 4 * g) = acc[u];
        }
    }
}

// Output epilogue of the schedule without a second pass.  A segment p >= 1
// was run from a zero incoming state, with DK virtual rows that start at the
// identity; since every output is linear in the incoming state, the true
// output of token t is o_t = o0_t + S_p m_t, where o0_t (in out) is the real
// rows' output from zero and m_t (in mws, [tokens, H, DK]) the virtual rows'.
// This adds S_p m_t, with S_p the composed incoming state of segment p, as
// MFMA products D[v][t] = sum_c S_p[v][c] m_t[c] (bf16 inputs: S_p rounded
// to bf16, as the chunk kernel rounds the state for its row products).  It
// streams m and out once (HBM-bound).  A workgroup stages S_p in LDS in the
// operand type; each wave takes blocks of 16 tokens with every value tile,
// NBK blocks per step with all their loads issued before the first product.
// Workgroups: W per (sequence, head, segment); a segment's blocks are dealt
// round-robin to its 4 W waves.
template <typename In, int DK>
__global__ void __launch_bounds__(256) seg_out_kernel(const In *__restrict__ mws, const float *__restrict__ seg_start,
                                                      In *__restrict__ out, const int *__restrict__ cu_seqlens,
                                                      int T, int H, int dv, int C, int nsegs, int lead, int W)
{
    constexpr bool F32 = sizeof(In) == 4;
    // k-chunk per lane and MFMA: 8 contiguous channels (bf16, 16x16x32), else
    // 4 (bf16 16x16x16 at DK = 16, fp32 16x16x4 over the chunk's 4 elements)
    constexpr bool K8 = !F32 && DK % 32 == 0;
    constexpr int KW = K8 ? 8 : 4;               // channels per lane per step
    constexpr int NKS = DK / (4 * KW);           // k steps
    constexpr int PS = DK + 16 / (int)sizeof(In);   // LDS row pitch (elements)
    constexpr int NBK = 2;
    typedef In VK __attribute__((ext_vector_type(KW)));
    typedef typename V4T<In>::type V4;
    __shared__ __attribute__((aligned(16))) In sS[128 * PS];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 15, g = lane >> 4;
    const int w = blockIdx.x % W, hs = blockIdx.x / W;
    const int head = hs / (nsegs - 1), seg = 1 + hs % (nsegs - 1);
    const int seq = head / H, h = head % H;
    long tok0, len;
    if (cu_seqlens) {
        const long a0 = min(max((long)cu_seqlens[seq], 0L), (long)T);
        const long a1 = min(max((long)cu_seqlens[seq + 1], a0), (long)T);
        tok0 = a0;
        len = a1 - a0;
    } else {
        tok0 = (long)seq * T;
        len = T;
    }
    long c0, c1;
    if (lead < 0) {   // two segments, split on the device
        c0 = ((const int *)(mws + (long)T * H * DK))[seq];   // the plan, after m
        c1 = (len + C - 1) / C;
    } else {
        seg_bounds((len + C - 1) / C, nsegs, lead, seg, c0, c1);
    }
    const long s0 = tok0 + c0 * C, s1 = tok0 + min(c1 * C, len);
    if (s1 <= s0) return;
    const int ndv = dv / 16;
    // S_p [dv][DK] fp32 -> LDS in the operand type
    const float *sp = seg_start + ((long)head * nsegs + seg) * dv * DK;
    for (int e = 4 * (int)threadIdx.x; e < dv * DK; e += 4 * 256) {
        const f32x4 x = *(const f32x4 *)(sp + e);
        const int r = e / DK, c = e % DK;
#pragma unroll
        for (int i = 0; i < 4; ++i) sS[r * PS + c + i] = fromf<In>(x[i]);
    }
    __syncthreads();
    const int HDK = H * DK, HDV = H * dv;
    const int es = (int)sizeof(In);
    const long stride = 16L * 4 * W;
    // bf16 with two or more value tiles: the tiles go in pairs whose A rows are
    // interleaved (tile 2P row r is S_p row 32 P + 8 (r >> 2) + (r & 3), tile
    // 2P + 1 the same plus 4), so that lane (n, g) holds 8 consecutive outputs
    // 32 P + 8 g .. + 7 of token n: 16-byte loads and stores of out
    const bool pairo = !F32 && ndv >= 2;
    auto arow = [&](int u, int r) { return pairo ? 32 * (u >> 1) + 8 * (r >> 2) + 4 * (u & 1) + (r & 3) : 16 * u + r; };
    typedef In V8 __attribute__((ext_vector_type(8)));
    for (long b0 = s0 + 16L * (4 * w + wave); b0 < s1; b0 += NBK * stride) {
        VK bm[NBK][NKS];
        V4 ov[NBK][8];
        __amdgpu_buffer_rsrc_t ro[NBK];
#pragma unroll
        for (int j = 0; j < NBK; ++j) {
            const long bj = b0 + j * stride;
            const unsigned nval = bj < s1 ? (unsigned)min(16L, s1 - bj) : 0u;   // 0: an empty descriptor
            const long bb = bj < s1 ? bj : s0;
            const __amdgpu_buffer_rsrc_t rm = buf_rsrc(mws + (bb * H + h) * DK, nval * HDK * (unsigned)es);
#pragma unroll
            for (int s = 0; s < NKS; ++s) bm[j][s] = buf_load<VK>(rm, (n * HDK + KW * (4 * s + g)) * es, 0);
            ro[j] = buf_rsrc(out + (bb * H + h) * dv, nval * HDV * (unsigned)es);
            if constexpr (!F32) {
                if (pairo) {
#pragma unroll
                    for (int P = 0; P < 4; ++P)
                        if (2 * P < ndv) {
                            const V8 x = buf_load<V8>(ro[j], (n * HDV + 32 * P + 8 * g) * es, 0);
                            ov[j][2 * P] = __builtin_shufflevector(x, x, 0, 1, 2, 3);
                            ov[j][2 * P + 1] = __builtin_shufflevector(x, x, 4, 5, 6, 7);
                        }
                    continue;
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (u < ndv) ov[j][u] = buf_load<V4>(ro[j], (n * HDV + 16 * u + 4 * g) * es, 0);
        }
#pragma unroll
        for (int j = 0; j < NBK; ++j) {
            f32x4 res[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (u >= ndv) break;
                f32x4 acc = to_f32<In>(ov[j][u]);   // out[b0 + j stride + n][arow(u, 4 g + i)]
                const In *ar = sS + arow(u, n) * PS;
#pragma unroll
                for (int s = 0; s < NKS; ++s) {
                    const VK a = *(const VK *)(ar + KW * (4 * s + g));
                    if constexpr (K8) {
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bm[j][s], acc, 0, 0, 0);
                    } else if constexpr (!F32) {
                        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                                        __builtin_bit_cast(i16x4, bm[j][s]), acc, 0, 0, 0);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], bm[j][s][e], acc, 0, 0, 0);
                    }
                }
                res[u] = acc;
            }
            if constexpr (!F32) {
                if (pairo) {
#pragma unroll
                    for (int P = 0; P < 4; ++P)
                        if (2 * P < ndv) {
                            const V4 lo = to_op<In>(res[2 * P]), hi = to_op<In>(res[2 * P + 1]);
                            buf_store(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), ro[j],
                                      (n * HDV + 32 * P + 8 * g) * es, 0);
                        }
                    continue;
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (u < ndv) buf_store(to_op<In>(res[u]), ro[j], (n * HDV + 16 * u + 4 * g) * es, 0);
        }
    }
}

// One launch of the chunk kernel over `grid` workgroups (xcd_map: the per-region
// XCD remap flags, each set only where its region's unit count is a multiple of 8).
template <typename In, int DK, int BV, int C, bool MAP, int VAR>
hipError_t launch_chunk_grid_v(const ChunkArgs &a, long grid, int xcd_map)
{
    typedef ChunkCfg<In, DK, BV, C> K;
    if (grid == 0) return hipSuccess;
    // the kernel divides by the segment count: never pass less than 1
    hipLaunchKernelGGL((chunk_fwd_kernel<In, DK, BV, C, MAP, VAR>), dim3((unsigned)grid), dim3(K::NT), 0,
                       a.stream, (const In *)a.q, (const In *)a.k, (const In *)a.v, a.log_alpha, a.beta, a.S0,
                       (In *)a.out, a.S_final, a.cu_seqlens, a.T, a.H, a.dv, xcd_map, a.nsegs < 1 ? 1 : a.nsegs,
                       a.seg_start, a.seg_map, a.gate, a.add, a.prep, a.nsegs > 1 ? a.lead : 0, (In *)a.mws,
                       a.mout);
    return hipGetLastError();
}

// The same, with the kernel specialised for the plain recurrence or not.
template <typename In, int DK, int BV, int C, bool MAP>
hipError_t launch_chunk_grid(const ChunkArgs &a, long grid, int xcd_map)
{
    if (a.prep != 0 && a.gate == 0 && a.add == 0) return launch_chunk_grid_v<In, DK, BV, C, MAP, 2>(a, grid, xcd_map);
    if (a.gate != 0 || a.add != 0 || a.prep != 0) return launch_chunk_grid_v<In, DK, BV, C, MAP, 1>(a, grid, xcd_map);
    return launch_chunk_grid_v<In, DK, BV, C, MAP, 0>(a, grid, xcd_map);
}

// The whole prefill: one pass, or (nsegs > 1) the map launch (the maps of every
// segment but the last; with a lead segment, segment 0's whole pass beside the
// maps of segments 1 .. nsegs - 2), the composition of the maps, and the pass
// over every segment that still needs one.
template <typename In, int DK, int BV, int C>
hipError_t launch_chunk_t(const ChunkArgs &a)
{
    typedef ChunkCfg<In, DK, BV, C> K;
    if constexpr (!K::fits) {
        return hipErrorInvalidConfiguration;
    } else {
        const long nheads = (long)a.nseq * a.H, nvA = a.dv / BV;
        if (a.nsegs <= 1) return launch_chunk_grid<In, DK, BV, C, false>(a, nheads * nvA, nheads % 8 == 0);
        if constexpr (DK % BV != 0) {
            return hipErrorInvalidConfiguration;   // the virtual rows fill whole value blocks
        } else {
            const long nvB = (a.dv + DK) / BV;
            const bool lead = a.lead != 0;   // (negative: the device-side split of packed sequences)
            hipError_t e;
            if (lead && a.mout) {
                // no second pass: the map launch (segment 0's pass, and every later
                // segment's map with its outputs from a zero state), the
                // composition (through S_final), then the output epilogue
                const long unitsB = nheads * (a.nsegs - 1);
                const int *plan = a.lead < 0 ? (const int *)((const In *)a.mws + (long)a.T * a.H * DK) : nullptr;
                if (plan) {   // packed sequences: the device-side split, once
                    hipLaunchKernelGGL(seg_plan_kernel<0>, dim3(1), dim3(256), 0, a.stream, a.cu_seqlens, a.nseq, a.T, C,
                                       a.H, a.lead, (int *)plan);
                    e = hipGetLastError();
                    if (e != hipSuccess) return e;
                }
                e = launch_chunk_grid<In, DK, BV, C, true>(a, nheads * nvA + unitsB * nvB,
                                                            (nheads % 8 == 0 ? 1 : 0) | (unitsB % 8 == 0 ? 2 : 0));
                if (e != hipSuccess) return e;
                const long ncomp = (long)a.nseq * a.H * (a.dv / 16);
                hipLaunchKernelGGL((seg_compose_kernel<DK>), dim3((unsigned)ncomp), dim3(256), 0, a.stream, a.S0,
                                   (const float *)a.seg_map, a.seg_start, a.dv, a.nsegs, 1, 1, a.S_final,
                                   a.cu_seqlens, a.T, C, a.H, plan);
                e = hipGetLastError();
                if (e != hipSuccess) return e;
                const long units = nheads * (a.nsegs - 1);
                // about one resident round of workgroups (two per compute unit);
                // with the device-side split only the split sequences have work,
                // and the others' workgroups exit at once
                long W = units >= 2L * a.cus ? 1 : (2L * a.cus) / units;
                if (a.lead < 0 && W < 16) W = 16;
                hipLaunchKernelGGL((seg_out_kernel<In, DK>), dim3((unsigned)(units * W)), dim3(256), 0, a.stream,
                                   (const In *)a.mws, (const float *)a.seg_start, (In *)a.out, a.cu_seqlens, a.T,
                                   a.H, a.dv, C, a.nsegs, a.lead, (int)W);
                return hipGetLastError();
            }
            if (lead) {
                const long unitsB = nheads * (a.nsegs - 2);
                e = launch_chunk_grid<In, DK, BV, C, true>(a, nheads * nvA + unitsB * nvB,
                                                            (nheads % 8 == 0 ? 1 : 0) | (unitsB % 8 == 0 ? 2 : 0));
            } else {
                const long units = nheads * (a.nsegs - 1);
                e = launch_chunk_grid<In, DK, BV, C, true>(a, units * nvB, units % 8 == 0);
            }
            if (e != hipSuccess) return e;
            const long ncomp = (long)a.nseq * a.H * (a.dv / 16);
            if (ncomp > 0) {
                hipLaunchKernelGGL((seg_compose_kernel<DK>), dim3((unsigned)ncomp), dim3(256), 0, a.stream, a.S0,
                                   (const float *)a.seg_map, a.seg_start, a.dv, a.nsegs, lead ? 1 : 0, 0, nullptr,
                                   nullptr, 0, C, a.H, nullptr);
                e = hipGetLastError();
                if (e != hipSuccess) return e;
            }
            const long units = nheads * (lead ? a.nsegs - 1 : a.nsegs);
            return launch_chunk_grid<In, DK, BV, C, false>(a, units * nvA, units % 8 == 0);
        }
    }
}

template <typename In, int DK>
hipError_t launch_chunk_dk(const ChunkArgs &a)
{
#define KDA_CASE(BV_, C_) \
    if (a.BV == BV_ && a.C == C_) return launch_chunk_t<In, DK, BV_, C_>(a);
    KDA_CASE(16, 16) KDA_CASE(16, 32) KDA_CASE(16, 64)
    KDA_CASE(32, 16) KDA_CASE(32, 32) KDA_CASE(32, 64)
    KDA_CASE(64, 16) KDA_CASE(64, 32) KDA_CASE(64, 64)
#undef KDA_CASE
    return hipErrorInvalidConfiguration;
}

template <typename In, int DK>
constexpr bool chunk_fits_dk(int BV, int C)
{
#define KDA_CASE(BV_, C_) \
    if (BV == BV_ && C == C_) return ChunkCfg<In, DK, BV_, C_>::fits;
    KDA_CASE(16, 16) KDA_CASE(16, 32) KDA_CASE(16, 64)
    KDA_CASE(32, 16) KDA_CASE(32, 32) KDA_CASE(32, 64)
    KDA_CASE(64, 16) KDA_CASE(64, 32) KDA_CASE(64, 64)
#undef KDA_CASE
    return false;
}

}  // namespace kda
