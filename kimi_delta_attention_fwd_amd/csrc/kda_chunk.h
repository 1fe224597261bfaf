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
// Decay factoring.  e^{G_r - G_j} is never formed pairwise.  Rows are split
// into 16-token blocks and every key channel c gets a reference rho_I[c] per
// block I: 0 (the chunk start) when the channel decays by at most 80 nats over
// the whole chunk, else G just before block I.  The operand waves store, per
// token r of block I,
//   Kr = k e^{G_r - rho_I},  Qr = q e^{G_r - rho_I}   (both <= |k|, |q|)
//   Kd = k e^{rho_I - G_r}                             (<= |k| e^{80})
// and per channel e^{rho_I} and w_IJ = e^{rho_I - rho_J} (J < I, <= 1).  Then
//   A/P tile (I, J) = [Kr|Qr]_I (Kd_J w_IJ)^T,  Kbar S^T = Kr (S Diag(e^{rho_I}))^T,
// and Ktil = k e^{G_last - G_r} <= |k|.  When every channel of a chunk takes
// the chunk-start reference, e^{rho_I} = w_IJ = 1 and both consumers skip the
// scaling.  Every factor stays in range as long as no key channel decays by
// more than 80 nats inside one 16-token block (the precondition in the public
// header).  The factors come from alpha = e^{log_alpha} by running prefix and
// suffix products inside each lane's tokens, times one exponential per
// channel of the partial sums across lanes (all exponents <= 0).
//
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

template <typename In, int DK, int BV, int C>
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
    static constexpr int PK = DK + 4;                // rows of [token, d_k] operands
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
    // "all channels referenced to the chunk start" flags [NXW]
    static constexpr int SC_GL = NB * DK, SC_BETA = NB * DK + DK, SC_FLAG = SC_BETA + C;
    // input preparation (raw q, k): per-wave partial squared norms of k and q
    // [C][NXW] (a token's four partials in one 16-byte LDS read), then per
    // token beta / |k|^2, |k| and 1 / |q|
    static constexpr int SC_PK = SC_FLAG + NXW, SC_PQ = SC_PK + NXW * C, SC_BH = SC_PQ + NXW * C;
    static constexpr int SC_KN = SC_BH + C, SC_QI = SC_KN + C, SC_END = SC_QI + C;
    static constexpr float FAST_NATS = 80.f;

    static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
    static constexpr size_t SZ_R = al(size_t(C) * PK * sizeof(In));     // Kr, Qr, Kd
    static constexpr size_t SZ_KT = al(size_t(DK) * PC * sizeof(In));   // Ktil^T
    static constexpr size_t SZ_SC = al(size_t(SC_END) * sizeof(float));
    static constexpr size_t SZ_W = al(size_t(NOFF > 0 ? NOFF : 1) * DK * sizeof(float));
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
    static_assert(NSEG >= NB && NSEG >= NOFF, "a segment of lanes per scale and w vector");
};

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
template <typename In, int DK, int BV, int C, bool MAP, int VAR>
__global__ void __launch_bounds__((ChunkCfg<In, DK, BV, C>::NT), 1)
chunk_fwd_kernel(const In *__restrict__ q, const In *__restrict__ k, const In *__restrict__ v,
                 const float *__restrict__ log_alpha, const float *__restrict__ beta,
                 const float *S0, In *__restrict__ out, float *S_final,
                 const int *__restrict__ cu_seqlens, int T, int H, int dv, int xcd_map,
                 int nsegs, float *seg_start, float *seg_map, int gate_arg, int add_arg, int prep_arg,
                 int lead)
{
    // VAR = 0: the plain recurrence, the variant arguments folded away; 1: any
    // variant, read from the arguments; 2: raw inputs with the per-channel gate
    // and the delta write (the usual projection outputs), folded in
    const int gate = VAR == 1 ? gate_arg : 0, add = VAR == 1 ? add_arg : 0;
    const int prep = VAR == 2 ? 1 : (VAR == 1 ? prep_arg : 0);
    typedef ChunkCfg<In, DK, BV, C> K;
    typedef typename V4T<In>::type V4;
    constexpr int NB = K::NB, NDK = K::NDK, PK = K::PK, PC = K::PC, PT = K::PT, RS = K::RS;

    __shared__ __attribute__((aligned(16))) unsigned char smem[K::LDS];
    In *const sKd = (In *)(smem + K::O_KD);
    float *const sW = (float *)(smem + K::O_W);
    float *const sA = (float *)(smem + K::O_A);
    In *const sP = (In *)(smem + K::O_P);
    auto bufKr = [&](long ch) { return (In *)(smem + K::O_KR + (ch & 1) * K::SZ_R); };
    auto bufQr = [&](long ch) { return (In *)(smem + K::O_QR + (ch & 1) * K::SZ_R); };
    auto bufKt = [&](long ch) { return (In *)(smem + K::O_KT + (ch & 1) * K::SZ_KT); };
    auto bufSc = [&](long ch) { return (float *)(smem + K::O_SC + (ch & 1) * K::SZ_SC); };

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
    if (MAP && lead > 0) {
        const int nA = (int)(gridDim.x / (nvA + (nsegs - 2) * nvB)) * nvA;
        int unit;
        if ((int)blockIdx.x < nA) {
            place(blockIdx.x, nvA, xcd_map & 1, unit, vb);
            head = unit;
            seg = 0;
            lead_full = true;
        } else {
            place(blockIdx.x - nA, nvB, xcd_map & 2, unit, vb);
            head = unit / (nsegs - 2);
            seg = 1 + unit % (nsegs - 2);
        }
    } else {
        const int nsu = (MAP || lead > 0) ? nsegs - 1 : nsegs;   // segments per sequence in this grid
        int unit;
        place(blockIdx.x, MAP ? nvB : nvA, xcd_map & 1, unit, vb);
        head = unit / nsu;
        seg = unit % nsu + ((!MAP && lead > 0) ? 1 : 0);
    }
    const bool map = MAP && !lead_full;              // augmented state, no outputs
    const int seq = head / H, h = head % H;
    long tok0, len;
    if (cu_seqlens) {   // T is the stream length here; offsets clamped to [0, T] keep every access inside it
        const long a0 = min(max((long)cu_seqlens[seq], 0L), (long)T);
        const long a1 = min(max((long)cu_seqlens[seq + 1], a0), (long)T);
        tok0 = a0;
        len = a1 - a0;
    } else {
        tok0 = (long)seq * T;
        len = T;
    }
    if (nsegs > 1) {
        // segment seg: chunks [c0, c1) of the sequence's n.  Uniform: ceil(n /
        // nsegs) each.  Lead: segments 1 .. nsegs - 1 take L = ceil(10 n /
        // (10 (nsegs - 1) + lead)) each from the end, segment 0 the rest (about
        // lead / 10 L; none when the sequence is short).
        const long n = (len + C - 1) / C;
        long c0, c1;
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
        tok0 += c0 * C;
        len = max(0L, min(len - c0 * C, (c1 - c0) * C));
    }
    const long nch = (len + C - 1) / C;
    const int HDK = H * DK, HDV = H * dv;
    const long hrow = tok0 * H + h;                 // token rows are H*d elements apart

    // One lower-triangle tile pair (I, J) of chunk ch: the A tile (beta-scaled,
    // strictly lower on the diagonal) and / or the P tile (lower incl. the
    // diagonal).  Tiles are computed transposed, d[i] = X[16I + n][16J + 4g + i],
    // so each lane stores four consecutive columns of one row.
    // beta / |k|^2 of token r from the operand waves' partial squared norms
    // (0 for a zero key: identity tokens past the end of a sequence)
    auto beta_hat = [&](const float *scc, int r) __attribute__((always_inline)) {
        float sk = 0.f;
#pragma unroll
        for (int w = 0; w < K::NXW; ++w) sk += scc[K::SC_PK + r * K::NXW + w];
        return sk > 0.f ? scc[K::SC_BETA + r] * __builtin_amdgcn_rcpf(sk) : 0.f;
    };
    auto tile_job = [&](long ch, int p, bool doA, bool doP, f32x4 *lt = nullptr) __attribute__((always_inline)) {
        int I = p, J = p;
        if (p >= NB) {
            const int o = p - NB;
            I = 1;
            while ((I + 1) * I / 2 <= o) ++I;
            J = o - I * (I - 1) / 2;
        }
        const float *scc = bufSc(ch);
        const float *fl = scc + K::SC_FLAG;
        const bool allfast = all_flags<K::NXW>(fl);
        V4 cf[NDK];
#pragma unroll
        for (int t = 0; t < NDK; ++t) cf[t] = *(const V4 *)(sKd + (16 * J + n) * PK + 16 * t + 4 * g);
        if (I > J && !allfast) {   // Kd_J w_IJ = k e^{rho_I - G} <= |k|
            const float *wr = sW + (I * (I - 1) / 2 + J) * DK + 4 * g;
#pragma unroll
            for (int t = 0; t < NDK; ++t) {
                const f32x4 w4 = *(const f32x4 *)(wr + 16 * t);
                cf[t] = to_op<In>(to_f32<In>(cf[t]) * w4);
            }
        }
        if (doA) {
            const In *Kr = bufKr(ch);
            V4 rk[NDK];
#pragma unroll
            for (int t = 0; t < NDK; ++t) rk[t] = *(const V4 *)(Kr + (16 * I + n) * PK + 16 * t + 4 * g);
            const f32x4 da = mma_tiles<K::KD, In, NDK>(zero4(), cf, rk);
            const float b = prep ? beta_hat(scc, 16 * I + n) : scc[K::SC_BETA + 16 * I + n];
            f32x4 va;
#pragma unroll
            for (int i = 0; i < 4; ++i) va[i] = (I > J || 4 * g + i < n) ? da[i] * b : 0.f;
            *(f32x4 *)(sA + p * 16 * PT + n * PT + 4 * g) = va;
            if (lt) {
                // diagonal tile: also L itself in accumulator layout,
                // lt[0][i] = L[4g + i][n] (and lt[1] = L^T, the tile just stored)
                const f32x4 dl = mma_tiles<K::KD, In, NDK>(zero4(), rk, cf);
                f32x4 b4 = *(const f32x4 *)(scc + K::SC_BETA + 16 * I + 4 * g);
                if (prep) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) b4[i] = beta_hat(scc, 16 * I + 4 * g + i);
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
#pragma unroll
            for (int t = 0; t < NDK; ++t) rq[t] = *(const V4 *)(Qr + (16 * I + n) * PK + 16 * t + 4 * g);
            const f32x4 dp = mma_tiles<K::KD, In, NDK>(zero4(), cf, rq);
            f32x4 vp;
#pragma unroll
            for (int i = 0; i < 4; ++i) vp[i] = (I > J || 4 * g + i <= n) ? dp[i] : 0.f;
            store4(sP + p * 16 * PT + n * PT + 4 * g, vp);
        }
    };

    if (wave >= K::NBV) {
        // =============== operand waves: chunk t+1 while the state waves run chunk t
        const int xw = wave - K::NBV;
        const int cg = lane % K::NCG, seg = lane / K::NCG;
        const bool act = lane < K::NACT;
        const int c0 = xw * K::CPW + 4 * cg;        // this lane's channels c0 .. c0+3
        const int r0 = seg * RS;                    // and tokens r0 .. r0+RS-1 (inactive lanes: >= C)
        const int blk_src = ((r0 / 16) * (16 / RS)) * K::NCG + cg;   // lane holding rho of my block
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
        auto chunk_valid = [&](long t0) { return (unsigned)((len - t0 < C) ? len - t0 : C); };
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
            if (map) return;
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

        // ---- stage A: cumulative decay, references, scaled operands
        auto stage_a = [&](long ch) __attribute__((always_inline)) {
            const long t0 = ch * C;
            const int nval = (int)((len - t0 < C) ? len - t0 : C);
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
            float tot[4], inc[4], exc[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < RS; ++i) acc += gr[i][j];
                tot[j] = acc;
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
            float rhoI[NB][4], ref[4], glast[4];
            bool fastc[4], lane_fast = true;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                exc[j] = inc[j] - tot[j];                                       // G before my first token
                glast[j] = __shfl(inc[j], (K::NSEG - 1) * K::NCG + cg, 64);      // G_last
                fastc[j] = glast[j] >= -K::FAST_NATS;
                lane_fast = lane_fast && fastc[j];
            }
            const bool wave_fast = __all(lane_fast);
            if (wave_fast) {   // every channel of the wave takes the chunk-start reference
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    ref[j] = 0.f;
#pragma unroll
                    for (int I = 0; I < NB; ++I) rhoI[I][j] = 0.f;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float rb = __shfl(exc[j], blk_src, 64);               // G before my block
                    ref[j] = fastc[j] ? 0.f : rb;
#pragma unroll
                    for (int I = 0; I < NB; ++I) {
                        const float r = __shfl(exc[j], (I * (16 / RS)) * K::NCG + cg, 64);
                        rhoI[I][j] = fastc[j] ? 0.f : r;
                    }
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
            float *sc = bufSc(ch);
            // forward over my tokens: e^{G - ref} by prefix products -> Kr, Qr
            // (and Kd = k / e^{G - ref} where some channel keeps a block reference)
            {
                float pp[4];
                float sk[RS], sq[RS];   // prep: squared norms over this wave's channels
#pragma unroll
                for (int j = 0; j < 4; ++j) pp[j] = fexp(exc[j] - ref[j]);
#pragma unroll
                for (int i = 0; i < RS; ++i) {
                    f32x4 vkr, vqr, vkd;
                    sk[i] = 0.f;
                    sq[i] = 0.f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        pp[j] *= al[i][j];
                        const float kf = tof(kr[i][j]);
                        vkr[j] = kf * pp[j];                       // k e^{G - ref}
                        if (!map) vqr[j] = tof(qr[i][j]) * pp[j];   // q e^{G - ref}
                        if (prep) {
                            sk[i] += kf * kf;
                            if (!map) sq[i] += tof(qr[i][j]) * tof(qr[i][j]);
                        }
                    }
                    if (act) {
                        const int r = r0 + i;
                        store4(Kr + r * PK + c0, vkr);
                        if (!map) store4(Qr + r * PK + c0, vqr);
                        if (!lane_fast) {
#pragma unroll
                            for (int j = 0; j < 4; ++j) vkd[j] = tof(kr[i][j]) * __builtin_amdgcn_rcpf(pp[j]);   // k e^{ref - G}
                            store4(sKd + r * PK + c0, vkd);
                        }
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
            // backward: e^{G_last - G} by suffix products -> Ktil, and Kd = Ktil e^{-G_last}
            // where every channel of the lane takes the chunk-start reference
            {
                float sf[4], gli[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    sf[j] = fexp(glast[j] - inc[j]);
                    gli[j] = fexp(-glast[j]);
                }
                In kt[4][RS];
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
                    if (act && lane_fast) store4(sKd + (r0 + i) * PK + c0, vkd);
                }
                if (act) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) store_row_swz<In, RS>(Kt, c0 + j, r0, PC, K::SWZ, kt[j]);
                }
            }
            // per-channel scales, one 4-channel vector store per lane: e^{G_last}
            // by the first segment's lanes, e^{rho_I} by segment I, w_IJ by
            // segment I(I-1)/2 + J.  w is stored also when all factors are 1:
            // other waves may take block references, and then the tiles read w
            // for every channel.
            if (seg == 0) *(f32x4 *)(sc + K::SC_GL + c0) = f32x4{fexp(glast[0]), fexp(glast[1]), fexp(glast[2]), fexp(glast[3])};
            if (wave_fast) {   // a uniform branch: no exponentials when every factor is 1
                const f32x4 one{1.f, 1.f, 1.f, 1.f};
                if (seg < NB) *(f32x4 *)(sc + seg * DK + c0) = one;
                if (seg < K::NOFF) *(f32x4 *)(sW + seg * DK + c0) = one;
            } else {
#pragma unroll
                for (int I = 0; I < NB; ++I) {
                    if (seg == I) {
                        f32x4 e;
#pragma unroll
                        for (int j = 0; j < 4; ++j) e[j] = fexp(rhoI[I][j]);
                        *(f32x4 *)(sc + I * DK + c0) = e;
                    }
#pragma unroll
                    for (int J = 0; J < I; ++J) {
                        if (seg == I * (I - 1) / 2 + J) {
                            f32x4 w;
#pragma unroll
                            for (int j = 0; j < 4; ++j) w[j] = fexp(rhoI[I][j] - rhoI[J][j]);
                            *(f32x4 *)(sW + (I * (I - 1) / 2 + J) * DK + c0) = w;
                        }
                    }
                }
            }
            if (lane == 0) sc[K::SC_FLAG + xw] = wave_fast ? 1.f : 0.f;
            if (xw == 0 && lane < C) sc[K::SC_BETA + lane] = (lane < nval) ? betar : 0.f;
        };

        // ---- stage B: the diagonal A tiles and their block inverses (with P
        //      when there is a single state wave, which then also leaves the
        //      off-diagonal A tiles here)
        auto stage_b = [&](long ch) __attribute__((always_inline)) {
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
            if (add) {   // no A: only the diagonal P tiles of a single state wave
                if (K::NBV == 1 && !map) {
                    for (int p = xw; p < NB; p += K::NXW) tile_job(ch, p, false, true);
                }
                return;
            }
            for (int p = xw; p < (K::NBV == 1 ? K::NPAIR : NB); p += K::NXW) {
                if (p < NB && !K::F32) {
                    // D_p = (I + L)^{-1} for the strictly lower diagonal tile L, as
                    // (I - L)(I + L^2)(I + L^4)(I + L^8) (L^16 = 0).  With two
                    // tiles in accumulator layout, one fp32 MFMA product gives
                    // acc(X^T Y); D_p^T is built that way from acc(L), acc(L^T)
                    // and stored so that lane (n, g) writes row n, columns 4g..4g+3.
                    // (The powers of L can grow like binomial coefficients before
                    // they cancel, about 1e-4 relative at worst: fine for the bf16
                    // kernels, the fp32 ones use the substitution below.)
                    f32x4 lt[2];
                    tile_job(ch, p, true, K::NBV == 1 && !map, lt);
                    auto mm = [](f32x4 x, f32x4 y) {   // acc(X^T Y)
                        const f32x4 a[1] = {x}, b[1] = {y};
                        return mma_tiles<4, float, 1>(zero4(), a, b);
                    };
                    const f32x4 L1 = lt[0], U1 = lt[1];
                    const f32x4 U2 = mm(L1, U1), L2 = mm(U1, L1);
                    const f32x4 U3 = mm(L1, U2), L4 = mm(U2, L2), U4 = mm(L2, U2);
                    const f32x4 L8 = mm(U4, L4);
                    f32x4 id;
#pragma unroll
                    for (int i = 0; i < 4; ++i) id[i] = (4 * g + i == n) ? 1.f : 0.f;
                    const f32x4 M1t = id - U1 + U2 - U3;              // ((I - L)(I + L^2))^T
                    const f32x4 M2t = M1t + mm(L4, M1t);              // ... (I + L^4)
                    const f32x4 Dt = M2t + mm(L8, M2t);               // ... (I + L^8)
                    *(f32x4 *)(sA + p * 16 * PT + n * PT + 4 * g) = Dt;
                } else if (p < NB) {
                    // fp32 kernels: column n of D_p by forward substitution over the
                    // rows of the stored tile (lanes of the other 16-lane rows repeat
                    // the work and store nothing)
                    tile_job(ch, p, true, K::NBV == 1 && !map);
                    float *At = sA + p * 16 * PT;
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
                } else {
                    tile_job(ch, p, true, false);
                }
            }
        };

        // Same barrier sequence as the state waves: two per chunk plus two.
        if (nch > 0) {
            prefetch_g(0);
            prefetch_q(0);
            prefetch_k(0);
            stage_a(0);
            if (nch > 1) prefetch_k(C);
        }
        __syncthreads();
        if (nch > 0) stage_b(0);
        __syncthreads();
        // Stage A sets the pace of the first segment, where each operand wave
        // shares its SIMD with a state wave that has time to spare: the operand
        // waves issue first there (wave priority, this workgroup only).
        for (long ch = 0; ch < nch; ++ch) {
            __builtin_amdgcn_s_setprio(3);
            if (ch + 1 < nch) {
                stage_a(ch + 1);
                if (ch + 2 < nch) prefetch_k((ch + 2) * C);
            }
            __builtin_amdgcn_s_setprio(0);
            __syncthreads();
            if (ch + 1 < nch) stage_b(ch + 1);
            __syncthreads();
        }
    } else {
        // =============== state waves: value rows 16 cb .. 16 cb + 15 of the block
        const int cb = wave;
        const int row = vb * BV + 16 * cb + n;     // this lane's state row (of the augmented state in MAP mode)
        const bool vreal = !map || vb * BV < dv;   // real value rows (virtual ones see v = 0)
        // bf16: lane (n, g) loads row 16 (2 u + g/2) + n, columns 8 (g&1) .. +7;
        // fp32: row 16 u + n, columns 4g .. 4g+3 (u = load index)
        const int rowb_v = HDV * (int)sizeof(In);
        const int voff_v = (K::F32 ? n : (16 * (g >> 1) + n)) * rowb_v + (K::F32 ? 4 * g : 8 * (g & 1)) * (int)sizeof(In);
        const int voff_o = n * rowb_v + 4 * g * (int)sizeof(In);   // output row 16 I + n, columns 4g .. 4g+3
        const long vcol = hrow * dv + vb * BV + 16 * cb;

        // State, transposed, in accumulator layout: Sacc[ct][i] = S[16 cb + n][16 ct + 4g + i].
        // Where it comes from and goes to: S0 / S_final for a whole sequence;
        // the segment's incoming state / S_final (last segment only) for a
        // segment; zero or the identity / the segment's map in MAP mode; S0 /
        // segment 1's incoming state for the lead segment in the map launch.
        f32x4 Sacc[NDK];
        const float *s0row = nullptr;
        float *sfrow = nullptr;
        if (map) {
            sfrow = seg_map + (((long)head * (nsegs - 1) + seg) * (dv + DK) + row) * DK;
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
            const unsigned nv = vreal ? (unsigned)((len - t0 < C) ? len - t0 : C) : 0u;
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
        // two or more state waves the off-diagonal pairs (A and P) and then the
        // diagonal P tiles, else the off-diagonal P tiles (MAP mode: no P tiles).
        // Jobs are dealt in snake order so the heavier pairs spread evenly over
        // the waves.
        constexpr int NJOB_MAP = K::NBV >= 2 ? K::NOFF : 0, NJOB_FULL = K::NBV >= 2 ? K::NPAIR : K::NOFF;
        const int njob = map ? NJOB_MAP : NJOB_FULL;
        constexpr int NROUND = (NJOB_FULL + K::NBV - 1) / K::NBV;   // NJOB_MAP <= NJOB_FULL
        auto y_tiles = [&](long ch) __attribute__((always_inline)) {
#pragma unroll
            for (int r = 0; r < NROUND; ++r) {
                const int s = r * K::NBV + ((r & 1) ? K::NBV - 1 - cb : cb);
                if (s < njob) {
                    const int p = s < K::NOFF ? NB + s : s - K::NOFF;
                    tile_job(ch, p, K::NBV >= 2 && p >= NB && !add, !map);
                }
            }
        };
        if (nch > 0) prefetch_v(0);
        __syncthreads();
        if (nch > 0) y_tiles(0);
        __syncthreads();

        V4 Eb[NB];   // corrected errors of the chunk, operand type: E[16b + 4g + i][n]
        for (long ch = 0; ch < nch; ++ch) {
            const long t0 = ch * C;
            const int nval = (int)((len - t0 < C) ? len - t0 : C);
            const In *Kr = bufKr(ch), *Qr = bufQr(ch);
            const float *sc = bufSc(ch);
            const float *fl = sc + K::SC_FLAG;
            const bool allfast = all_flags<K::NXW>(fl);
            // ---- R = beta (V - Kbar S^T) and (Qbar S^T)^T, per 16-token block I
            f32x4 R[NB], O1[NB];
            V4 ss[NDK];
            auto rows = [&](int I) __attribute__((always_inline)) {
                V4 ak[NDK], bq[NDK];
#pragma unroll
                for (int ct = 0; ct < NDK; ++ct) {
                    if (!add) ak[ct] = *(const V4 *)(Kr + (16 * I + n) * PK + 16 * ct + 4 * g);
                    if (!map) bq[ct] = *(const V4 *)(Qr + (16 * I + n) * PK + 16 * ct + 4 * g);
                }
                R[I] = add ? zero4() : mma_tiles<K::KD, In, NDK>(zero4(), ak, ss);    // [16I + 4g + i][n]
                if (!map) O1[I] = mma_tiles<K::KD, In, NDK>(zero4(), ss, bq);   // [v = 4g + i][16I + n]
            };
            if (allfast) {
#pragma unroll
                for (int ct = 0; ct < NDK; ++ct) ss[ct] = to_op<In>(Sacc[ct]);
#pragma unroll
                for (int I = 0; I < NB; ++I) rows(I);
            } else {
#pragma unroll
                for (int I = 0; I < NB; ++I) {
#pragma unroll
                    for (int ct = 0; ct < NDK; ++ct) {
                        const f32x4 er = *(const f32x4 *)(sc + I * DK + 16 * ct + 4 * g);
                        ss[ct] = to_op<In>(Sacc[ct] * er);        // S Diag(e^{rho_I}), transposed
                    }
                    rows(I);
                }
            }
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                const f32x4 b4 = *(const f32x4 *)(sc + (prep ? K::SC_BH : K::SC_BETA) + 16 * I + 4 * g);
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
                        const f32x4 a = *(const f32x4 *)(sA + tile_index(NB, b, J) * 16 * PT + n * PT + 4 * g);
                        y = mma_fp32a<In>(y, a, Eb[J]);
                    }
                    const f32x4 d = *(const f32x4 *)(sA + b * 16 * PT + n * PT + 4 * g);
                    const f32x4 e = mma_fp32ab<In>(d, R[b] - y);
                    Eb[b] = to_op<In>(e);
                }
            }

            // ---- O^T = (Qbar S^T)^T + E^T P^T, written as O rows (rows past the end dropped)
            const __amdgpu_buffer_rsrc_t ro = buf_rsrc(out + vcol + t0 * HDV, (unsigned)nval * rowb_v);
#pragma unroll
            for (int I = 0; I < (map ? 0 : NB); ++I) {
                V4 pb[NB];
#pragma unroll
                for (int J = 0; J < NB; ++J)
                    pb[J] = (J <= I) ? *(const V4 *)(sP + tile_index(NB, I, J) * 16 * PT + n * PT + 4 * g) : V4{};
                f32x4 o = O1[I] + mma_tiles<K::KC, In, NB>(zero4(), Eb, pb);   // O[16I + n][16cb + 4g + i]
                if (prep) o = o * sc[K::SC_QI + 16 * I + n];                   // / |q|
                buf_store(to_op<In>(o), ro, voff_o, 16 * I * rowb_v);
            }
            // ---- S^T <- Diag(e^{G_last}) S^T + Ktil^T E (Ktil and the scales of this chunk are
            //      double-buffered, so this needs no barrier)
            const In *Kt = bufKt(ch);
#pragma unroll
            for (int ct = 0; ct < NDK; ++ct) {
                const f32x4 gl = *(const f32x4 *)(sc + K::SC_GL + 16 * ct + 4 * g);
                V4 ka[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    ka[b] = *(const V4 *)(Kt + Panel<In, 16>::swz_index(16 * ct + n, 16 * b + 4 * g, PC, K::SWZ));
                Sacc[ct] = mma_tiles<K::KC, In, NB>(Sacc[ct] * gl, ka, Eb);
            }
            __syncthreads();

            // ---- the next chunk's tiles
            if (ch + 1 < nch) y_tiles(ch + 1);
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
// N_p) the map of segment p from the MAP pass.  One workgroup per 16 state rows
// of a head; thread (r, cg) keeps columns cg DK/16 .. of row r.  Each step
// stages M_p in LDS (coalesced 16-byte loads, in two halves of DK/2 rows for
// DK = 128 to stay within the LDS budget) next to the current rows.  fp32
// throughout.
template <int DK>
__global__ void __launch_bounds__(256) seg_compose_kernel(const float *S0, const float *seg_map,
                                                          float *seg_start, int dv, int nsegs, int p0)
{
    constexpr int CPT = DK / 16;                  // columns per thread
    constexpr int MR = DK > 64 ? DK / 2 : DK;     // rows of M staged at a time
    __shared__ __attribute__((aligned(16))) float srow[16][DK + 4];
    __shared__ __attribute__((aligned(16))) float sm[MR][DK];
    const int nrb = dv / 16;
    const int head = blockIdx.x / nrb, rb = blockIdx.x % nrb;
    const int tid = threadIdx.x, r = tid >> 4, c0 = (tid & 15) * CPT;
    const int row = rb * 16 + r;
    float acc[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j)
        acc[j] = p0 > 0 ? seg_start[(((long)head * nsegs + p0) * dv + row) * DK + c0 + j]
                        : (S0 ? S0[((long)head * dv + row) * DK + c0 + j] : 0.f);
    for (int p = p0;; ++p) {
        float *dst = seg_start + (((long)head * nsegs + p) * dv + row) * DK + c0;
#pragma unroll
        for (int j = 0; j < CPT; ++j) dst[j] = acc[j];
        if (p + 1 >= nsegs) break;
        __syncthreads();   // the previous step's reads of srow are done
#pragma unroll
        for (int j = 0; j < CPT; ++j) srow[r][c0 + j] = acc[j];
        const float *mp = seg_map + ((long)head * (nsegs - 1) + p) * (dv + DK) * DK;
#pragma unroll
        for (int j = 0; j < CPT; ++j) acc[j] = mp[(long)row * DK + c0 + j];   // N_p
        const float *M = mp + (long)dv * DK;
        for (int h0 = 0; h0 < DK; h0 += MR) {
            if (h0 > 0) __syncthreads();   // everyone is done with the previous half of M
            for (int e = tid * 4; e < MR * DK; e += 256 * 4)
                *(f32x4 *)(&sm[0][0] + e) = *(const f32x4 *)(M + (long)h0 * DK + e);
            __syncthreads();
#pragma unroll 8
            for (int i = 0; i < MR; ++i) {
                const float si = srow[r][h0 + i];
#pragma unroll
                for (int j = 0; j < CPT; ++j) acc[j] = fmaf(si, sm[i][c0 + j], acc[j]);
            }
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
                       a.seg_start, a.seg_map, a.gate, a.add, a.prep, a.nsegs > 1 ? a.lead : 0);
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
            const bool lead = a.lead > 0;
            hipError_t e;
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
                                   (const float *)a.seg_map, a.seg_start, a.dv, a.nsegs, lead ? 1 : 0);
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
