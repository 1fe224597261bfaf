// Fused chunkwise KDA prefill kernel for gfx950.
//
// One workgroup owns one (sequence, head, value block of BV state rows) and
// walks that sequence's chunks of C tokens in order, keeping its BV x DK slice
// of the fp32 state in registers the whole time.  Per chunk (cumulative decay
// G_r = sum_{s<=r} log_alpha_s, per key channel, restarted at the chunk start;
// S = incoming state):
//
//   A_rj = beta_r sum_c k_rc k_jc e^{G_rc - G_jc}   (j <  r)   KK^T system
//   P_rj =        sum_c q_rc k_jc e^{G_rc - G_jc}   (j <= r)   causal QK^T
//   R    = Diag(beta) (V - Kbar S^T),  Kbar = K e^{G}         provisional errors
//   E    = (I + A)^{-1} R                                     corrected errors
//   O    = Qbar S^T + P E,             Qbar = Q e^{G}
//   S^T <- Diag(e^{G_last}) S^T + Ktil^T E,  Ktil = K e^{G_last - G}
//
// This is the chunk mode of the "KDA derivation summary" page (sect. 6: the
// recurrence regrouped into matrix products plus a lower-triangular solve that
// corrects each token's provisional error), on the chunk skeleton of the
// "Linear/sparse attention tutorial" page (sect. 6.2: intra-chunk causal part,
// inter-chunk state hand-off, cumulative decay folded into the state and the
// intra-chunk mask).  The equations above follow from the recurrence by
// unrolling it over one chunk.
//
// Decay factoring.  e^{G_r - G_j} is never formed pairwise; A and P are MFMA
// products of pre-scaled operands.  Each chunk takes one of two exact paths,
// chosen per chunk (uniformly for the workgroup):
//  * fast path, when no key channel decays by more than 80 nats over the
//    chunk: rows k e^{G}, q e^{G}, columns k e^{-G}.  All factors lie in
//    [e^-80, e^80], far inside the fp32 / bf16 range.
//  * sub-block path otherwise: rows are split into 16-row blocks b with start
//    reference rho_b = G_{16b-1} and end reference sigma_b = G_{16b+15};
//    rows k e^{G - rho_b} (<= |k|), diagonal-block columns k e^{rho_b - G}
//    (bounded by the block's own decay), and for row block I > b the columns
//    k e^{rho_I - G} (<= |k|).  Only the diagonal blocks carry factors above
//    one: this path needs every channel to decay by less than 80 nats inside
//    each 16-token block (the precondition in the public header).
// Every exponent is a sum of same-sign partial sums (no cancellation).
//
// (I + A) E = R is solved in fp32 by block forward substitution over the
// 16-row blocks: the inverses of the 16x16 diagonal blocks come from forward
// substitution in registers (one lane per column, the A entries broadcast
// inside each 16-lane row with DPP); the off-diagonal updates and the
// diagonal-block products run on fp32 MFMA, one wave per 16 value columns.
//
// Matrix products run on MFMA 16x16 tiles: bf16 operands with fp32
// accumulation in the bf16 entry points, fp32 operands in the fp32 ones.
#pragma once

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

template <typename In, int DK, int BV, int C, int NW = 4>
struct ChunkCfg {
    typedef In OpT;                                  // MFMA operand type
    static constexpr int NWAVE = NW;
    static constexpr int NT = 64 * NW;               // threads
    static constexpr int NB = C / 16;                // 16-row blocks per chunk
    static constexpr int NBV = BV / 16;
    static constexpr int NDK = DK / 16;
    static constexpr int PADE = 16 / (int)sizeof(OpT);
    static constexpr int PK = DK + PADE;             // pitch of [*, DK] operands
    static constexpr int PC = C + PADE;              // pitch of [*, C] operands
    static constexpr int PA = C + 4;                 // pitch of the fp32 A matrix (16-byte rows)
    static constexpr int SWZ = C * (int)sizeof(OpT) / 16 - 1;   // chunk XOR mask of the swizzled Ktil^T
    static constexpr int VE = 16 / (int)sizeof(In);  // elements per 16-byte vector of v / out
    static constexpr int PV = BV + VE;               // pitch of the staged V tile
    // pitch of the staged output tile (padded when it still fits the R^T slot)
    static constexpr int PO = (C * (BV + VE) <= BV * (C + PADE)) ? BV + VE : BV;
    static constexpr int NPAIR = NB * (NB + 1) / 2;  // (I, J <= I) column-operand tiles
    // element-wise phase: each thread owns RS rows x 4 channels
    static constexpr int NCG = DK / 4;
    static constexpr int RS = (C * NCG > NT) ? (C * NCG / NT) : 1;
    static constexpr int NSEG = C / RS;
    static constexpr int NACT = NCG * NSEG;
    static constexpr int SEG_PER_BLK = 16 / RS;
    // fast path: every segment's decay below 80 / NSEG nats bounds the chunk's by 80
    static constexpr float SEG_LIMIT = 80.f / NSEG;
    static constexpr int NVCH = C * BV / VE;         // 16-byte vectors in a V / O tile
    static constexpr int VCH_PER_T = (NVCH + NT - 1) / NT;
    static constexpr int NOT = NB * NBV;             // output tiles (C x BV)
    static constexpr int OT_PER_W = (NOT + NW - 1) / NW;
    static constexpr int NST = NDK * NBV;            // state tiles (DK x BV, transposed state)
    static constexpr int ST_PER_W = (NST + NW - 1) / NW;

    static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
    static constexpr size_t SZ_KR = al(size_t(C) * PK * sizeof(OpT));
    static constexpr size_t SZ_KCOL = al(size_t(NPAIR) * 16 * PK * sizeof(OpT));
    static constexpr size_t SZ_GA = 2 * SZ_KR + SZ_KCOL;            // sub-block path: Kr, Qr, Kcol
    static constexpr size_t SZ_KTT = al(size_t(DK) * PC * sizeof(OpT));
    static constexpr size_t SZ_GB = 3 * SZ_KR + SZ_KTT;             // Kbar, Qbar, Khat, Ktil^T
    static constexpr size_t SZ_G = SZ_GA > SZ_GB ? SZ_GA : SZ_GB;
    static constexpr size_t SZ_S = al(size_t(BV) * PK * sizeof(OpT));
    static constexpr size_t SZ_CC = al(size_t(C) * PC * sizeof(OpT));
    static constexpr int PX = 20;                    // pitch of a wave's 16x16 fp32 substitution scratch
    static constexpr size_t SZ_X = al(size_t(NW) * 16 * PX * sizeof(float));
    static constexpr size_t SZ_V = al(size_t(C) * PV * sizeof(In));
    static constexpr size_t SZ_SEG = al(size_t(NSEG) * DK * sizeof(float));
    static constexpr size_t SZ_BETA = al(size_t(C) * sizeof(float));
    static constexpr size_t SZ_GL = al(size_t(DK) * sizeof(float));
    static constexpr size_t SZ_FLAG = 16;
    static constexpr size_t SZ_A = al(size_t(C) * PA * sizeof(float));
    static constexpr size_t SZ_VT = al(size_t(BV) * PC * sizeof(OpT));
    // segment sums live in the E^T slot when they fit (they are dead by the time E^T is written)
    static constexpr bool SEG_IN_ET = SZ_SEG <= SZ_VT;

    static constexpr size_t O_KR = 0, O_QR = SZ_KR, O_KCOL = 2 * SZ_KR;
    static constexpr size_t O_KBAR = 0, O_QBAR = SZ_KR, O_KHAT = 2 * SZ_KR, O_KTT = 3 * SZ_KR;
    static constexpr size_t O_S = SZ_G;
    static constexpr size_t O_X = O_S + SZ_S;
    static constexpr size_t O_P = O_X + SZ_X;
    static constexpr size_t O_V = O_P + SZ_CC;
    static constexpr size_t O_SEGX = O_V + SZ_V;                         // segment sums, when not in E^T
    static constexpr size_t O_BETA = O_SEGX + (SEG_IN_ET ? 0 : SZ_SEG);
    static constexpr size_t O_GL = O_BETA + SZ_BETA;
    static constexpr size_t O_FLAG = O_GL + SZ_GL;
    static constexpr size_t O_A = O_FLAG + SZ_FLAG;
    static constexpr size_t O_RT = O_A + SZ_A, O_ET = O_RT + SZ_VT, O_O = O_RT;
    static constexpr size_t O_SEG = SEG_IN_ET ? O_ET : O_SEGX;
    static constexpr size_t LDS = O_ET + SZ_VT;
    static constexpr bool fits = LDS <= 160 * 1024;

    static_assert(C % 16 == 0 && C <= 64, "chunk length");
    static_assert(DK % 16 == 0 && BV % 16 == 0, "tile sizes");
    static_assert(16 % RS == 0, "a thread's rows stay inside one 16-row block");
    static_assert(size_t(C) * BV * sizeof(In) <= SZ_VT, "O staging fits the R^T slot");
    static_assert(NW >= 2, "A and P are formed by separate halves of the waves");
    static_assert(NW % NBV == 0, "each wave keeps one value column block");
};

template <typename T>
__device__ __forceinline__ void store4(T *p, f32x4 v);
template <>
__device__ __forceinline__ void store4<float>(float *p, f32x4 v) { *(f32x4 *)p = v; }
template <>
__device__ __forceinline__ void store4<bf16>(bf16 *p, f32x4 v) {
    bf16x4 b = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
    *(bf16x4 *)p = b;
}

__device__ __forceinline__ constexpr int pair_index(int I, int J) { return I * (I + 1) / 2 + J; }

// Writes v[0..RS) to row `row`, columns col0 .. col0+RS-1, of an array in the
// chunk-swizzled layout of Panel::swz_index, in 16-byte (or smaller) pieces.
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

// value of `v` in lane K of this lane's 16-lane row (DPP row_newbcast)
template <int K>
__device__ __forceinline__ float row_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + K, 0xF, 0xF, false));
}

// Column j (= lane & 15) of the inverse of the unit lower-triangular 16x16
// block I + L, where lane j holds column j of L in acol[0..15] (acol[i] =
// L[i][j]).  Forward substitution x <- x - L[:, k] x_k, the L entries read
// from lane k of the row.  Every lane of the wave must take part.
__device__ __forceinline__ void inv_unit_lower16(const float (&acol)[16], float (&x)[16], int j)
{
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
#define KDA_STEP(KK)                                                                                   \
    {                                                                                                  \
        _Pragma("unroll") for (int i = KK + 1; i < 16; ++i) x[i] -= row_bcast<KK>(acol[i]) * x[KK]; \
    }
    KDA_STEP(0) KDA_STEP(1) KDA_STEP(2) KDA_STEP(3) KDA_STEP(4) KDA_STEP(5) KDA_STEP(6) KDA_STEP(7)
    KDA_STEP(8) KDA_STEP(9) KDA_STEP(10) KDA_STEP(11) KDA_STEP(12) KDA_STEP(13) KDA_STEP(14)
#undef KDA_STEP
}

template <typename In, int DK, int BV, int C, int NW>
__global__ void __launch_bounds__(64 * NW, 1)
chunk_fwd_kernel(const In *__restrict__ q, const In *__restrict__ k, const In *__restrict__ v,
                 const float *__restrict__ log_alpha, const float *__restrict__ beta,
                 const float *S0, In *__restrict__ out, float *S_final,
                 const int *__restrict__ cu_seqlens, int T, int H, int dv, int xcd_map)
{
    typedef ChunkCfg<In, DK, BV, C, NW> K;
    typedef typename K::OpT OpT;
    typedef In In4 __attribute__((ext_vector_type(4)));
    constexpr int NB = K::NB, NBV = K::NBV, RS = K::RS, PK = K::PK, PC = K::PC, PA = K::PA;
    constexpr int PV = K::PV, VE = K::VE, PO = K::PO;
    // one bf16 MFMA shape for the whole kernel (16x16x32 unless a contraction is only 16 long)
    constexpr int KSB = sizeof(OpT) == 4 ? 4 : ((DK % 32 == 0 && C % 32 == 0) ? 32 : 16);
    typedef Panel<OpT, DK, KSB> PanelK;
    typedef Panel<OpT, C, KSB> PanelC;

    __shared__ __attribute__((aligned(16))) unsigned char smem[K::LDS];
    OpT *sKr = (OpT *)(smem + K::O_KR);
    OpT *sQr = (OpT *)(smem + K::O_QR);
    OpT *sKcol = (OpT *)(smem + K::O_KCOL);
    OpT *sKbar = (OpT *)(smem + K::O_KBAR);
    OpT *sQbar = (OpT *)(smem + K::O_QBAR);
    OpT *sKhat = (OpT *)(smem + K::O_KHAT);
    OpT *sKtT = (OpT *)(smem + K::O_KTT);
    OpT *sS = (OpT *)(smem + K::O_S);
    float *sX = (float *)(smem + K::O_X);
    OpT *sP = (OpT *)(smem + K::O_P);
    In *sV = (In *)(smem + K::O_V);
    float *sSeg = (float *)(smem + K::O_SEG);
    float *sBeta = (float *)(smem + K::O_BETA);
    float *sGL = (float *)(smem + K::O_GL);
    int *sFlag = (int *)(smem + K::O_FLAG);
    float *sA = (float *)(smem + K::O_A);
    OpT *sRT = (OpT *)(smem + K::O_RT);
    OpT *sET = (OpT *)(smem + K::O_ET);
    In *sO = (In *)(smem + K::O_O);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar) index
    const int nvb = dv / BV;
    int head, vb;
    if (xcd_map) {
        // Workgroups are dealt to the 8 XCDs round-robin; keep all value blocks
        // of one head on one XCD so their shared q / k / log_alpha reads hit
        // the same L2.
        const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
        head = (slot / nvb) * 8 + x;
        vb = slot % nvb;
    } else {
        head = blockIdx.x / nvb;
        vb = blockIdx.x % nvb;
    }
    const int seq = head / H, h = head % H;
    long tok0, len;
    if (cu_seqlens) {
        tok0 = cu_seqlens[seq];
        len = (long)cu_seqlens[seq + 1] - tok0;
    } else {
        tok0 = (long)seq * T;
        len = T;
    }

    // element-wise mapping: thread owns rows r0 .. r0+RS-1, channels c0 .. c0+3
    const int cg = tid % K::NCG, seg = tid / K::NCG;
    const bool ew = tid < K::NACT;
    const int c0 = 4 * cg, r0 = seg * RS, blk = r0 / 16;

    // The upper (J > I) 16x16 tiles of P are zero and never rewritten.
    for (int idx = tid; idx < C * C; idx += K::NT) {
        const int r = idx / C, j = idx % C;
        if (j / 16 > r / 16) sP[r * PC + j] = fromf<OpT>(0.f);
    }
    if (tid < 2) sFlag[tid] = 0;

    // Incoming state, held transposed (DK x BV) in accumulator layout: wave owns
    // tiles st = wave + NW s; lane holds S[16 sb + (lane & 15)][16 ct + 4 (lane >> 4) + i].
    f32x4 Sreg[K::ST_PER_W];
#pragma unroll
    for (int s = 0; s < K::ST_PER_W; ++s) {
        const int st = wave + NW * s;
        Sreg[s] = zero4();
        if (st < K::NST) {
            const int ct = st / NBV, sb = st % NBV;
            const int irow = 16 * sb + (lane & 15), c = 16 * ct + 4 * (lane >> 4);
            if (S0) Sreg[s] = *(const f32x4 *)(S0 + ((long)head * dv + vb * BV + irow) * DK + c);
            store4(sS + irow * PK + c, Sreg[s]);
        }
    }

    // -------- global loads of one chunk into registers (prefetched a chunk ahead).
    // Rows past the end of the sequence load the last valid row (always in
    // bounds, no branch around the loads) and are zeroed where they are used.
    In4 kr[RS], qr[RS];
    f32x4 gr[RS];
    float betar = 0.f;
    f32x4 vr[K::VCH_PER_T];
    // Per-head base pointers; a token row is H*DK (H*dv) elements further on.
    const int HDK = H * DK, HDV = H * dv;
    const long hrow = tok0 * H + h;
    const In *kb = k + hrow * DK + c0, *qb = q + hrow * DK + c0;
    const float *gb = log_alpha + hrow * DK + c0;
    const In *vbp = v + hrow * dv + vb * BV;
    In *ob = out + hrow * dv + vb * BV;
    const float *bb = beta + hrow;
    auto prefetch = [&](long t0) {
        const int last = (int)((len - t0 < C) ? len - t0 : C) - 1;
        // V and beta first: the waits the compiler places around these loads then
        // cover only older memory operations, not the q / k / log_alpha loads below.
        const long tv = t0 * HDV;
#pragma unroll
        for (int u = 0; u < K::VCH_PER_T; ++u) {
            const int idx = tid + u * K::NT;
            if (K::NVCH % K::NT == 0 || idx < K::NVCH) {
                const int r = min(idx / (BV / VE), last), cc = idx % (BV / VE);
                vr[u] = *(const f32x4 *)(vbp + tv + r * HDV + cc * VE);
            }
        }
        betar = bb[(t0 + min(tid, last)) * H];   // every lane loads (no branch); lanes >= C ignore it
        const long tk = t0 * HDK;
        if (ew) {
#pragma unroll
            for (int i = 0; i < RS; ++i) {
                const int ro = min(r0 + i, last) * HDK;
                kr[i] = *(const In4 *)(kb + tk + ro);
                qr[i] = *(const In4 *)(qb + tk + ro);
                gr[i] = *(const f32x4 *)(gb + tk + ro);
            }
        }
    };
    // Output rows of a chunk staged in sO go to HBM one chunk later, after the
    // next prefetch has been issued, so the stores drain while the loads wait.
    auto store_out = [&](long t0, int nv) {
        const long tv = t0 * HDV;
#pragma unroll
        for (int u = 0; u < K::VCH_PER_T; ++u) {
            const int idx = tid + u * K::NT;
            if (idx < K::NVCH) {
                const int r = idx / (BV / VE), cc = idx % (BV / VE);
                if (r < nv) *(f32x4 *)(ob + tv + r * HDV + cc * VE) = *(const f32x4 *)(sO + r * PO + cc * VE);
            }
        }
    };

    const long nch = (len + C - 1) / C;
    if (nch > 0) prefetch(0);
    __syncthreads();

    f32x4 Oacc[K::OT_PER_W];
    for (long ch = 0; ch < nch; ++ch) {
        const long t0 = ch * C;
        const int nval = (int)((len - t0 < C) ? len - t0 : C);

        // ---- (1) per-thread inclusive scan of log_alpha over its rows; stage beta and V;
        //      flag the chunk for the sub-block path if any segment decays too fast
        float L[RS][4];
        if (ew) {
#pragma unroll
            for (int i = 0; i < RS; ++i)
                if (r0 + i >= nval) {   // identity tokens past the end: k = q = 0, log_alpha = 0
                    gr[i] = zero4();
                    kr[i] = In4{};
                    qr[i] = In4{};
                }
            bool steep = false;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < RS; ++i) {
                    acc += gr[i][j];
                    L[i][j] = acc;
                }
                sSeg[seg * DK + c0 + j] = acc;
                steep |= !(fabsf(acc) <= K::SEG_LIMIT);
            }
            if (steep) sFlag[ch & 1] = 1;
        }
        if (tid < C) sBeta[tid] = (tid < nval) ? betar : 0.f;
#pragma unroll
        for (int u = 0; u < K::VCH_PER_T; ++u) {
            const int idx = tid + u * K::NT;
            if (idx < K::NVCH) {
                const int r = idx / (BV / VE), cc = idx % (BV / VE);
                *(f32x4 *)(sV + r * PV + cc * VE) = (r < nval) ? vr[u] : zero4();
            }
        }
        __syncthreads();
        const bool fast = __builtin_amdgcn_readfirstlane(sFlag[ch & 1]) == 0;

        // ---- (2) decay factors and the pre-scaled operands of A and P
        if (ew) {
            if (fast) {
                float pre[4] = {0.f, 0.f, 0.f, 0.f}, tot[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < K::NSEG; ++s)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float t = sSeg[s * DK + c0 + j];
                        tot[j] += t;
                        if (s < seg) pre[j] += t;
                    }
                float eGL[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) eGL[j] = __expf(tot[j]);
                if (seg == 0) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) sGL[c0 + j] = eGL[j];
                }
                OpT kt[4][RS];
#pragma unroll
                for (int i = 0; i < RS; ++i) {
                    const int r = r0 + i;
                    f32x4 vKb, vQb, vKh;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float g = pre[j] + L[i][j];          // G_r (chunk-relative)
                        const float e = __expf(g), ie = __expf(-g);
                        const float kf = tof(kr[i][j]);
                        vKb[j] = kf * e;                           // k e^{G}
                        vQb[j] = tof(qr[i][j]) * e;                // q e^{G}
                        vKh[j] = kf * ie;                          // k e^{-G}
                        kt[j][i] = fromf<OpT>(vKh[j] * eGL[j]);    // k e^{G_last - G}
                    }
                    store4(sKbar + r * PK + c0, vKb);
                    store4(sQbar + r * PK + c0, vQb);
                    store4(sKhat + r * PK + c0, vKh);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) store_row_swz<OpT, RS>(sKtT, c0 + j, r0, PC, K::SWZ, kt[j]);
            } else {
                float BT[NB][4];                // per-block total log-decay
                float pre[4], post[4];          // in-block sums before / after this segment
#pragma unroll
                for (int j = 0; j < 4; ++j) {
#pragma unroll
                    for (int I = 0; I < NB; ++I) BT[I][j] = 0.f;
                    pre[j] = 0.f;
                    post[j] = 0.f;
                }
#pragma unroll
                for (int s = 0; s < K::NSEG; ++s) {
                    const int I = s / K::SEG_PER_BLK;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float t = sSeg[s * DK + c0 + j];
                        BT[I][j] += t;
                        if (I == blk && s < seg) pre[j] += t;
                        if (I == blk && s > seg) post[j] += t;
                    }
                }
                float invTb[4], dI[NB][4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float total = 0.f;
#pragma unroll
                    for (int I = 0; I < NB; ++I) total += BT[I][j];
                    if (seg == 0) sGL[c0 + j] = __expf(total);
                    invTb[j] = __expf(-BT[blk][j]);     // e^{rho_b - sigma_b}
                    float between = 0.f;               // block totals strictly between blk and I
#pragma unroll
                    for (int I = 0; I < NB; ++I) {
                        dI[I][j] = 0.f;
                        if (I > blk) {
                            dI[I][j] = __expf(between);     // e^{rho_I - sigma_b}
                            between += BT[I][j];
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < RS; ++i) {
                    const int r = r0 + i;
                    f32x4 vKr, vQr, vKd, vKc[NB];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float suf = L[RS - 1][j] - L[i][j];      // sum over rows i+1 .. RS-1
                        const float x = __expf(pre[j] + L[i][j]);     // e^{G_r - rho_b}
                        const float y = __expf(post[j] + suf);        // e^{sigma_b - G_r}
                        const float kf = tof(kr[i][j]);
                        vKr[j] = kf * x;
                        vQr[j] = tof(qr[i][j]) * x;
                        vKd[j] = kf * y * invTb[j];                   // k e^{rho_b - G_r}
#pragma unroll
                        for (int I = 0; I < NB; ++I) vKc[I][j] = kf * y * dI[I][j];   // k e^{rho_I - G_r}
                    }
                    store4(sKr + r * PK + c0, vKr);
                    store4(sQr + r * PK + c0, vQr);
                    store4(sKcol + (pair_index(blk, blk) * 16 + (r - 16 * blk)) * PK + c0, vKd);
#pragma unroll
                    for (int I = 0; I < NB; ++I)
                        if (I > blk) store4(sKcol + (pair_index(I, blk) * 16 + (r - 16 * blk)) * PK + c0, vKc[I]);
                }
            }
        }
        if (tid == 0) sFlag[(ch + 1) & 1] = 0;   // slot of the next chunk (last read a chunk ago)
        if (ch + 1 < nch) prefetch(t0 + C);
        if (ch > 0) store_out(t0 - C, C);   // the previous chunk was a full one
        __syncthreads();

        // ---- (3) A (fp32, beta-scaled, strictly lower) and P (inclusive lower) on MFMA.
        //      Tiles are computed transposed (column block J of A / P against row block I),
        //      so each lane ends up with 4 consecutive columns of one row: vector stores,
        //      one beta per lane.  Half the waves make A, half P; each takes whole column
        //      blocks (0 and 3, or 1 and 2, when there are four).
        {
            constexpr int HW = NW / 2;
            const bool isA = wave < HW;
            const int hw = isA ? wave : wave - HW;
            const int n = lane & 15, g = lane >> 4;
#pragma unroll
            for (int J = 0; J < NB; ++J) {
                const int owner = (HW >= NB) ? J : (NB == 4) ? ((J < 2 ? J : 3 - J) % HW) : (J % HW);
                if (owner != hw) continue;
                PanelK cp;
                if (fast) cp.load(sKhat + 16 * J * PK, PK, lane);
#pragma unroll
                for (int I = J; I < NB; ++I) {
                    if (!fast) cp.load(sKcol + pair_index(I, J) * 16 * PK, PK, lane);
                    PanelK rp;
                    rp.load(fast ? ((isA ? sKbar : sQbar) + 16 * I * PK) : ((isA ? sKr : sQr) + 16 * I * PK), PK, lane);
                    const f32x4 acc = mma(zero4(), cp, rp);   // acc[i] = X[16I + n][16J + 4g + i]
                    const int r = 16 * I + n, j0 = 16 * J + 4 * g;
                    f32x4 val;
                    if (isA) {
                        const float b = sBeta[r];
#pragma unroll
                        for (int i = 0; i < 4; ++i) val[i] = (J < I || 4 * g + i < n) ? acc[i] * b : 0.f;
                        *(f32x4 *)(sA + r * PA + j0) = val;
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) val[i] = (J < I || 4 * g + i <= n) ? acc[i] : 0.f;
                        store4(sP + r * PC + j0, val);
                    }
                }
            }
        }
        __syncthreads();

        // ---- (4) sub-block path only: turn Kr / Qr / Kd into Kbar, Qbar, Ktil^T
        if (!fast) {
            OpT kt[4][RS];
            if (ew) {
                float before[4] = {0.f, 0.f, 0.f, 0.f}, after[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < K::NSEG; ++s) {
                    const int I = s / K::SEG_PER_BLK;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float t = sSeg[s * DK + c0 + j];
                        if (I < blk) before[j] += t;
                        else after[j] += t;
                    }
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    before[j] = __expf(before[j]);   // e^{rho_b}
                    after[j] = __expf(after[j]);     // e^{G_last - rho_b}
                }
#pragma unroll
                for (int i = 0; i < RS; ++i) {
                    const int r = r0 + i;
                    OpT *pk = sKr + r * PK + c0, *pq = sQr + r * PK + c0;
                    const OpT *pd = sKcol + (pair_index(blk, blk) * 16 + (r - 16 * blk)) * PK + c0;
                    f32x4 vk, vq;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        vk[j] = tof(pk[j]) * before[j];                   // k e^{G}
                        vq[j] = tof(pq[j]) * before[j];                   // q e^{G}
                        kt[j][i] = fromf<OpT>(tof(pd[j]) * after[j]);     // k e^{G_last - G}
                    }
                    store4(pk, vk);   // Kbar over Kr, Qbar over Qr (same slots)
                    store4(pq, vq);
                }
            }
            __syncthreads();   // Kd reads done before Ktil^T overwrites the Kcol region
            if (ew) {
#pragma unroll
                for (int j = 0; j < 4; ++j) store_row_swz<OpT, RS>(sKtT, c0 + j, r0, PC, K::SWZ, kt[j]);
            }
            __syncthreads();
        }

        // ---- (5) wave 0: inverses D_b' of the diagonal 16x16 blocks of I + A, in place in
        //      sA (forward substitution in registers, DPP broadcasts); the other waves
        //      meanwhile form R = beta (V - Kbar S^T), stored transposed.
        if (wave == 0) {
            const int b = min(lane >> 4, NB - 1), j = lane & 15;
            float *Ab = sA + 16 * b * PA + 16 * b;
            float acol[16], x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) acol[i] = Ab[i * PA + j];
            inv_unit_lower16(acol, x, j);
            if ((lane >> 4) < NB) {
#pragma unroll
                for (int i = 0; i < 16; ++i) Ab[i * PA + j] = x[i];
            }
        } else {
            const int n = lane & 15, g = lane >> 4;
            for (int t = wave - 1; t < K::NOT; t += NW - 1) {
                const int rb = t / NBV, cb2 = t % NBV;
                PanelK kp, sp;
                kp.load(sKbar + 16 * rb * PK, PK, lane);
                sp.load(sS + 16 * cb2 * PK, PK, lane);
                const f32x4 ak = mma(zero4(), kp, sp);   // (Kbar S^T)[16rb + 4g + i][16cb2 + n]
                f32x4 rv;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * rb + 4 * g + i;
                    rv[i] = sBeta[r] * (tof(sV[r * PV + 16 * cb2 + n]) - ak[i]);
                }
                store4(sRT + (16 * cb2 + n) * PC + 16 * rb + 4 * g, rv);
            }
        }
        __syncthreads();

        // Each wave owns one value column block cb of the C x BV outputs (all its
        // row blocks rb) and the matching state column block, so the operand panels
        // of cb are loaded once per phase.
        const int cb = wave % NBV;

        // ---- (6) E = (I + A)^{-1} R by block forward substitution,
        //      E_b = D_b' (R_b - sum_{J<b} A_bJ E_J).  Value columns are independent, so
        //      wave w solves column block w on its own (fp32 MFMA, wave-local LDS round
        //      trips, no workgroup barrier) and writes E^T for the updates below.
        if (wave < NBV) {
            float *xs = sX + wave * 16 * K::PX;
            const int n = lane & 15, g = lane >> 4, kq = lane >> 4;
            const OpT *et = sET + (16 * cb + n) * PC;          // row v = 16 cb + n of E^T
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                f32x4 y = zero4();                               // sum_{J<b} A_bJ E_J
#pragma unroll
                for (int J = 0; J < b; ++J)
#pragma unroll
                    for (int k0 = 0; k0 < 16; k0 += 4)
                        y = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(16 * b + n) * PA + 16 * J + k0 + kq],
                                                                 tof(et[16 * J + k0 + kq]), y, 0, 0, 0);
                typedef OpT Op4 __attribute__((ext_vector_type(4)));
                const Op4 rr = *(const Op4 *)(sRT + (16 * cb + n) * PC + 16 * b + 4 * g);
                f32x4 xv;
#pragma unroll
                for (int i = 0; i < 4; ++i) xv[i] = tof(rr[i]) - y[i];   // X[16b + 4g + i][n]
                *(f32x4 *)(xs + n * K::PX + 4 * g) = xv;                  // X^T, row n
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                f32x4 e = zero4();
#pragma unroll
                for (int k0 = 0; k0 < 16; k0 += 4)
                    e = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(16 * b + n) * PA + 16 * b + k0 + kq],
                                                             xs[n * K::PX + k0 + kq], e, 0, 0, 0);
                store4(sET + (16 * cb + n) * PC + 16 * b + 4 * g, e);    // E^T[16cb + n][16b + 4g + i]
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            }
        }
        __syncthreads();

        // ---- (7) O^T = S Qbar^T + E^T P^T;  S^T <- Diag(e^{G_last}) S^T + Ktil^T E
        {
            PanelC ep;
            ep.load(sET + 16 * cb * PC, PC, lane);
            PanelK sp;
            sp.load(sS + 16 * cb * PK, PK, lane);
#pragma unroll
            for (int s = 0; s < K::OT_PER_W; ++s) {
                const int ot = wave + NW * s;
                if (ot < K::NOT) {
                    const int rb = ot / NBV;
                    PanelK qp;
                    qp.load(sQbar + 16 * rb * PK, PK, lane);
                    PanelC pp;
                    pp.load(sP + 16 * rb * PC, PC, lane, 16 * (rb + 1));
                    Oacc[s] = mma(zero4(), sp, qp);               // O^T[16cb + 4g + i][16rb + n]
                    Oacc[s] = mma(Oacc[s], ep, pp, 16 * (rb + 1));
                }
            }
#pragma unroll
            for (int s = 0; s < K::ST_PER_W; ++s) {
                const int st = wave + NW * s;
                if (st < K::NST) {
                    const int ct = st / NBV;
                    PanelC kp;
                    kp.load_swz(sKtT, 16 * ct, PC, K::SWZ, lane);
                    const f32x4 acc = mma(zero4(), kp, ep);
#pragma unroll
                    for (int i = 0; i < 4; ++i) Sreg[s][i] = Sreg[s][i] * sGL[16 * ct + 4 * (lane >> 4) + i] + acc[i];
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < K::OT_PER_W; ++s) {
            const int ot = wave + NW * s;
            if (ot < K::NOT) {
                const int rb = ot / NBV;
                store4(sO + (16 * rb + (lane & 15)) * PO + 16 * cb + 4 * (lane >> 4), Oacc[s]);
            }
        }
#pragma unroll
        for (int s = 0; s < K::ST_PER_W; ++s) {
            const int st = wave + NW * s;
            if (st < K::NST) {
                const int ct = st / NBV;
                store4(sS + (16 * cb + (lane & 15)) * PK + 16 * ct + 4 * (lane >> 4), Sreg[s]);
            }
        }
        __syncthreads();
    }
    if (nch > 0) store_out((nch - 1) * C, (int)(len - (nch - 1) * C));

    if (S_final) {
#pragma unroll
        for (int s = 0; s < K::ST_PER_W; ++s) {
            const int st = wave + NW * s;
            if (st < K::NST) {
                const int ct = st / NBV, sb = st % NBV;
                const int irow = 16 * sb + (lane & 15), c = 16 * ct + 4 * (lane >> 4);
                *(f32x4 *)(S_final + ((long)head * dv + vb * BV + irow) * DK + c) = Sreg[s];
            }
        }
    }
}

// Waves per workgroup of the chunk kernel.
constexpr int kChunkWaves = 4;

template <typename In, int DK, int BV, int C>
hipError_t launch_chunk_t(const ChunkArgs &a)
{
    typedef ChunkCfg<In, DK, BV, C, kChunkWaves> K;
    if constexpr (!K::fits) {
        return hipErrorInvalidConfiguration;
    } else {
        const int nheads = a.nseq * a.H;
        const int nvb = a.dv / BV;
        const int grid = nheads * nvb;
        if (grid == 0) return hipSuccess;
        const int xcd_map = (nheads % 8 == 0) ? 1 : 0;
        hipLaunchKernelGGL((chunk_fwd_kernel<In, DK, BV, C, kChunkWaves>), dim3(grid), dim3(K::NT), 0, a.stream,
                           (const In *)a.q, (const In *)a.k, (const In *)a.v, a.log_alpha, a.beta, a.S0,
                           (In *)a.out, a.S_final, a.cu_seqlens, a.T, a.H, a.dv, xcd_map);
        return hipGetLastError();
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
    if (BV == BV_ && C == C_) return ChunkCfg<In, DK, BV_, C_, kChunkWaves>::fits;
    KDA_CASE(16, 16) KDA_CASE(16, 32) KDA_CASE(16, 64)
    KDA_CASE(32, 16) KDA_CASE(32, 32) KDA_CASE(32, 64)
    KDA_CASE(64, 16) KDA_CASE(64, 32) KDA_CASE(64, 64)
#undef KDA_CASE
    return false;
}

}  // namespace kda
