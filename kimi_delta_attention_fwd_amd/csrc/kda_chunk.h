// Fused chunkwise KDA prefill kernel for gfx950.
//
// One workgroup (4 waves) owns one (sequence, head, value block of BV state
// rows) and walks that sequence's chunks of C tokens in order, keeping its
// BV x DK slice of the fp32 state in registers the whole time.  Per chunk
// (cumulative decay G_r = sum_{s<=r} log_alpha_s, per key channel, restarted
// at the chunk start; S = incoming state):
//
//   A_rj = beta_r sum_c k_rc k_jc e^{G_rc - G_jc}   (j <  r)   KK^T system
//   P_rj =        sum_c q_rc k_jc e^{G_rc - G_jc}   (j <= r)   causal QK^T
//   T    = (I + A)^{-1}
//   R    = Diag(beta) (V - Kbar S^T),  Kbar = K e^{G}         provisional errors
//   E    = T R                                                corrected errors
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
// Decay factoring.  e^{G_r - G_j} is never formed pairwise.  Rows are split
// into 16-row blocks b with start reference rho_b = G_{16b-1} (rho_0 = 0) and
// end reference sigma_b = G_{16b+15}:
//   row operand  Kr = k e^{G - rho_b}   (<= |k|)
//   diag columns Kd = k e^{rho_b - G}   (>= |k|, bounded by the block's decay)
//   off-diagonal columns for row block I > b:  k e^{rho_I - G}  (<= |k|)
// so A and P are plain MFMA products of pre-scaled operands; every exponent
// is built from sums of same-sign partial sums (no cancellation).  The only
// factors above one are inside 16-row diagonal blocks, which is where the
// "< 80 nats per 16 tokens" precondition of the public header comes from.
//
// T = (I + A)^{-1} is built in fp32: the four 16x16 diagonal blocks by
// forward substitution (one wave, one lane per column), then the off-diagonal
// blocks by block doubling (16 -> 32 -> 64) with fp32 MFMA.
//
// Matrix products run on MFMA 16x16 tiles: bf16 operands with fp32
// accumulation in the bf16 entry points, fp32 operands in the fp32 ones.
#pragma once

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

template <typename In, int DK, int BV, int C>
struct ChunkCfg {
    typedef In OpT;                                  // MFMA operand type
    static constexpr int NT = 256;                   // threads (4 waves)
    static constexpr int NB = C / 16;                // 16-row blocks per chunk
    static constexpr int NBV = BV / 16;
    static constexpr int NDK = DK / 16;
    static constexpr int PADE = 16 / (int)sizeof(OpT);
    static constexpr int PK = DK + PADE;             // pitch of [*, DK] operands
    static constexpr int PC = C + PADE;              // pitch of [*, C] operands
    static constexpr int PA = C + 1;                 // pitch of the fp32 A / T work matrix
    static constexpr int VE = 16 / (int)sizeof(In);  // elements per 16-byte vector of v / out
    static constexpr int PV = BV + VE;               // pitch of the staged V tile
    static constexpr int NPAIR = NB * (NB + 1) / 2;  // (I, J <= I) column-operand tiles
    // element-wise phase: each thread owns RS rows x 4 channels
    static constexpr int NCG = DK / 4;
    static constexpr int RS = (C * NCG > NT) ? (C * NCG / NT) : 1;
    static constexpr int NSEG = C / RS;
    static constexpr int NACT = NCG * NSEG;
    static constexpr int SEG_PER_BLK = 16 / RS;
    static constexpr int NVCH = C * BV / VE;         // 16-byte vectors in a V / O tile
    static constexpr int VCH_PER_T = (NVCH + NT - 1) / NT;
    static constexpr int NOT = NB * NBV;             // output tiles (C x BV)
    static constexpr int OT_PER_W = (NOT + 3) / 4;
    static constexpr int NST = NDK * NBV;            // state tiles (DK x BV, transposed state)
    static constexpr int ST_PER_W = (NST + 3) / 4;

    static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
    static constexpr size_t SZ_KR = al(size_t(C) * PK * sizeof(OpT));
    static constexpr size_t SZ_KCOL = al(size_t(NPAIR) * 16 * PK * sizeof(OpT));
    static constexpr size_t SZ_GA = 2 * SZ_KR + SZ_KCOL;            // Kr, Qr, Kcol
    static constexpr size_t SZ_KTT = al(size_t(DK) * PC * sizeof(OpT));
    static constexpr size_t SZ_GB = 2 * SZ_KR + SZ_KTT;             // Kbar, Qbar, Ktil^T
    static constexpr size_t SZ_G = SZ_GA > SZ_GB ? SZ_GA : SZ_GB;
    static constexpr size_t SZ_S = al(size_t(BV) * PK * sizeof(OpT));
    static constexpr size_t SZ_CC = al(size_t(C) * PC * sizeof(OpT));
    static constexpr size_t SZ_V = al(size_t(C) * PV * sizeof(In));
    static constexpr size_t SZ_SEG = al(size_t(NSEG) * DK * sizeof(float));
    static constexpr size_t SZ_BETA = al(size_t(C) * sizeof(float));
    static constexpr size_t SZ_GL = al(size_t(DK) * sizeof(float));
    static constexpr size_t SZ_A = al(size_t(C) * PA * sizeof(float));
    static constexpr size_t SZ_VT = al(size_t(BV) * PC * sizeof(OpT));
    static constexpr size_t SZ_U = SZ_A > 2 * SZ_VT ? SZ_A : 2 * SZ_VT;

    static constexpr size_t O_KR = 0, O_QR = SZ_KR, O_KCOL = 2 * SZ_KR;
    static constexpr size_t O_KBAR = 0, O_QBAR = SZ_KR, O_KTT = 2 * SZ_KR;
    static constexpr size_t O_S = SZ_G;
    static constexpr size_t O_T = O_S + SZ_S;
    static constexpr size_t O_P = O_T + SZ_CC;
    static constexpr size_t O_V = O_P + SZ_CC;
    static constexpr size_t O_SEG = O_V + SZ_V;
    static constexpr size_t O_BETA = O_SEG + SZ_SEG;
    static constexpr size_t O_GL = O_BETA + SZ_BETA;
    static constexpr size_t O_U = O_GL + SZ_GL;
    static constexpr size_t O_A = O_U, O_RT = O_U, O_ET = O_U + SZ_VT, O_O = O_U;
    static constexpr size_t LDS = O_U + SZ_U;
    static constexpr bool fits = LDS <= 160 * 1024;

    static_assert(C % 16 == 0 && C <= 64, "chunk length");
    static_assert(DK % 16 == 0 && BV % 16 == 0, "tile sizes");
    static_assert(16 % RS == 0, "a thread's rows stay inside one 16-row block");
    static_assert(size_t(C) * BV * sizeof(In) <= SZ_VT, "O staging fits the R^T slot");
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

template <typename In, int DK, int BV, int C>
__global__ void __launch_bounds__(256, 1)
chunk_fwd_kernel(const In *__restrict__ q, const In *__restrict__ k, const In *__restrict__ v,
                 const float *__restrict__ log_alpha, const float *__restrict__ beta,
                 const float *S0, In *__restrict__ out, float *S_final,
                 const int *__restrict__ cu_seqlens, int T, int H, int dv, int xcd_map)
{
    typedef ChunkCfg<In, DK, BV, C> K;
    typedef typename K::OpT OpT;
    typedef In In4 __attribute__((ext_vector_type(4)));
    typedef OpT Op4 __attribute__((ext_vector_type(4)));
    constexpr int NB = K::NB, NBV = K::NBV, RS = K::RS, PK = K::PK, PC = K::PC, PA = K::PA;
    constexpr int PV = K::PV, VE = K::VE;

    __shared__ __attribute__((aligned(16))) unsigned char smem[K::LDS];
    OpT *sKr = (OpT *)(smem + K::O_KR);
    OpT *sQr = (OpT *)(smem + K::O_QR);
    OpT *sKcol = (OpT *)(smem + K::O_KCOL);
    OpT *sKbar = (OpT *)(smem + K::O_KBAR);
    OpT *sQbar = (OpT *)(smem + K::O_QBAR);
    OpT *sKtT = (OpT *)(smem + K::O_KTT);
    OpT *sS = (OpT *)(smem + K::O_S);
    OpT *sT = (OpT *)(smem + K::O_T);
    OpT *sP = (OpT *)(smem + K::O_P);
    In *sV = (In *)(smem + K::O_V);
    float *sSeg = (float *)(smem + K::O_SEG);
    float *sBeta = (float *)(smem + K::O_BETA);
    float *sGL = (float *)(smem + K::O_GL);
    float *sA = (float *)(smem + K::O_A);
    OpT *sRT = (OpT *)(smem + K::O_RT);
    OpT *sET = (OpT *)(smem + K::O_ET);
    In *sO = (In *)(smem + K::O_O);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

    // The upper (J > I) 16x16 tiles of T and P are zero and never rewritten.
    for (int idx = tid; idx < C * C; idx += K::NT) {
        const int r = idx / C, j = idx % C;
        if (j / 16 > r / 16) {
            sT[r * PC + j] = fromf<OpT>(0.f);
            sP[r * PC + j] = fromf<OpT>(0.f);
        }
    }

    // Incoming state, held transposed (DK x BV) in accumulator layout: wave owns
    // tiles st = wave + 4 s; lane holds S[16 sb + (lane & 15)][16 ct + 4 (lane >> 4) + i].
    f32x4 Sreg[K::ST_PER_W];
#pragma unroll
    for (int s = 0; s < K::ST_PER_W; ++s) {
        const int st = wave + 4 * s;
        Sreg[s] = zero4();
        if (st < K::NST) {
            const int ct = st / NBV, sb = st % NBV;
            const int irow = 16 * sb + (lane & 15), c = 16 * ct + 4 * (lane >> 4);
            if (S0) Sreg[s] = *(const f32x4 *)(S0 + ((long)head * dv + vb * BV + irow) * DK + c);
            store4(sS + irow * PK + c, Sreg[s]);
        }
    }

    // -------- global loads of one chunk into registers (prefetched a chunk ahead)
    In4 kr[RS], qr[RS];
    f32x4 gr[RS];
    float betar = 0.f;
    f32x4 vr[K::VCH_PER_T];
    auto prefetch = [&](long t0) {
        const long nval = (len - t0 < C) ? len - t0 : C;
        if (ew) {
#pragma unroll
            for (int i = 0; i < RS; ++i) {
                const int r = r0 + i;
                if (r < nval) {
                    const long row = ((tok0 + t0 + r) * H + h) * DK + c0;
                    kr[i] = *(const In4 *)(k + row);
                    qr[i] = *(const In4 *)(q + row);
                    gr[i] = *(const f32x4 *)(log_alpha + row);
                } else {
                    kr[i] = In4{} ;
                    qr[i] = In4{};
                    gr[i] = zero4();
                }
            }
        }
        if (tid < C) betar = (tid < nval) ? beta[(tok0 + t0 + tid) * H + h] : 0.f;
#pragma unroll
        for (int u = 0; u < K::VCH_PER_T; ++u) {
            const int idx = tid + u * K::NT;
            vr[u] = zero4();
            if (idx < K::NVCH) {
                const int r = idx / (BV / VE), cc = idx % (BV / VE);
                if (r < nval)
                    vr[u] = *(const f32x4 *)(v + ((tok0 + t0 + r) * H + h) * dv + vb * BV + cc * VE);
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

        // ---- (1) per-thread inclusive scan of log_alpha over its rows; stage beta and V
        float L[RS][4];
        if (ew) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < RS; ++i) {
                    acc += gr[i][j];
                    L[i][j] = acc;
                }
                sSeg[seg * DK + c0 + j] = acc;
            }
        }
        if (tid < C) sBeta[tid] = betar;
#pragma unroll
        for (int u = 0; u < K::VCH_PER_T; ++u) {
            const int idx = tid + u * K::NT;
            if (idx < K::NVCH) {
                const int r = idx / (BV / VE), cc = idx % (BV / VE);
                *(f32x4 *)(sV + r * PV + cc * VE) = vr[u];
            }
        }
        __syncthreads();

        // ---- (2) decay factors and the pre-scaled operands of A and P
        Op4 kbar[RS], qbar[RS], ktil[RS];   // inter-chunk operands, packed until written to LDS
        if (ew) {
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
            float invTb[4], eR[4], eL[4], eGL[4], dI[NB][4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float before = 0.f, after = 0.f, total = 0.f;
#pragma unroll
                for (int I = 0; I < NB; ++I) {
                    total += BT[I][j];
                    if (I < blk) before += BT[I][j];
                    if (I > blk) after += BT[I][j];
                }
                invTb[j] = __expf(-BT[blk][j]);     // e^{rho_b - sigma_b}
                eR[j] = __expf(before);            // e^{rho_b}
                eL[j] = __expf(after);             // e^{G_last - sigma_b}
                eGL[j] = __expf(total);            // e^{G_last}
                float between = 0.f;               // sum of block totals strictly between blk and I
#pragma unroll
                for (int I = 0; I < NB; ++I) {
                    dI[I][j] = 0.f;
                    if (I > blk) {
                        dI[I][j] = __expf(between);     // e^{rho_I - sigma_b}
                        between += BT[I][j];
                    }
                }
            }
            if (seg == 0) {
#pragma unroll
                for (int j = 0; j < 4; ++j) sGL[c0 + j] = eGL[j];
            }
            // suffix sums inside the segment: sum of log_alpha over rows i+1..RS-1
            float suf[RS][4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float acc = 0.f;
#pragma unroll
                for (int i = RS - 1; i >= 0; --i) {
                    suf[i][j] = acc;
                    acc += gr[i][j];
                }
            }
#pragma unroll
            for (int i = 0; i < RS; ++i) {
                const int r = r0 + i;
                f32x4 vKr, vQr, vKd, vKc[NB];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float x = __expf(pre[j] + L[i][j]);      // e^{G_r - rho_b}
                    const float y = __expf(post[j] + suf[i][j]);   // e^{sigma_b - G_r}
                    const float kf = tof(kr[i][j]), qf = tof(qr[i][j]);
                    vKr[j] = kf * x;
                    vQr[j] = qf * x;
                    vKd[j] = kf * y * invTb[j];                    // k e^{rho_b - G_r}
#pragma unroll
                    for (int I = 0; I < NB; ++I) vKc[I][j] = kf * y * dI[I][j];   // k e^{rho_I - G_r}
                    kbar[i][j] = fromf<OpT>(vKr[j] * eR[j]);
                    qbar[i][j] = fromf<OpT>(vQr[j] * eR[j]);
                    ktil[i][j] = fromf<OpT>(kf * y * eL[j]);
                }
                store4(sKr + r * PK + c0, vKr);
                store4(sQr + r * PK + c0, vQr);
                store4(sKcol + (pair_index(blk, blk) * 16 + (r - 16 * blk)) * PK + c0, vKd);
#pragma unroll
                for (int I = 0; I < NB; ++I)
                    if (I > blk) store4(sKcol + (pair_index(I, blk) * 16 + (r - 16 * blk)) * PK + c0, vKc[I]);
            }
        }
        if (ch + 1 < nch) prefetch(t0 + C);
        __syncthreads();

        // ---- (3) A (fp32, beta-scaled, strictly lower) and P (inclusive lower) on MFMA
        for (int t = wave; t < 2 * K::NPAIR; t += 4) {
            const bool isA = t < K::NPAIR;
            const int p = isA ? t : t - K::NPAIR;
            int I = 0;
            while ((I + 1) * (I + 2) / 2 <= p) ++I;
            const int J = p - I * (I + 1) / 2;
            const OpT *rowop = (isA ? sKr : sQr) + 16 * I * PK;
            const f32x4 acc = mma_tile<OpT, DK>(zero4(), rowop, PK, sKcol + p * 16 * PK, PK, lane);
            const int n = lane & 15;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * (lane >> 4) + i;
                const int r = 16 * I + m, jj = 16 * J + n;
                if (isA) sA[r * PA + jj] = (J < I || n < m) ? acc[i] * sBeta[r] : 0.f;
                else sP[r * PC + jj] = fromf<OpT>((J < I || n <= m) ? acc[i] : 0.f);
            }
        }
        __syncthreads();

        // ---- (4) T = (I + A)^{-1}; meanwhile the inter-chunk operands replace Kr/Qr/Kcol
        if (ew) {
#pragma unroll
            for (int i = 0; i < RS; ++i) {
                *(Op4 *)(sKbar + (r0 + i) * PK + c0) = kbar[i];
                *(Op4 *)(sQbar + (r0 + i) * PK + c0) = qbar[i];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < RS; ++i) sKtT[(c0 + j) * PC + r0 + i] = ktil[i][j];
        }
        if (wave == 0 && lane < 16 * NB) {
            // diagonal 16x16 blocks: column j of (I + A_bb)^{-1} by forward substitution
            const int b = lane >> 4, j = lane & 15;
            float *Ab = sA + 16 * b * PA + 16 * b;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int kk = 0; kk < 15; ++kk)
#pragma unroll
                for (int i = kk + 1; i < 16; ++i) x[i] -= Ab[i * PA + kk] * x[kk];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                Ab[i * PA + j] = x[i];
                sT[(16 * b + i) * PC + 16 * b + j] = fromf<OpT>(x[i]);
            }
        }
        __syncthreads();
        if constexpr (NB >= 2) {
            // 16 -> 32: T_ij = -D_i' A_ij D_j' for (i, j) = (1, 0) and (3, 2)
            constexpr int NP1 = (NB == 4) ? 2 : 1;
            const int pi = 2 * wave + 1, pj = 2 * wave;
            const int row0 = 4 * (lane >> 4), col = lane & 15;
            if (wave < NP1) {
                const f32x4 M = mma_f32_strided<16>(zero4(), sA + 16 * pi * PA + 16 * pj, PA, 1,
                                                    sA + 16 * pj * PA + 16 * pj, PA, 1, lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) sA[(16 * pj + row0 + i) * PA + 16 * pi + col] = M[i];
            }
            __syncthreads();
            if (wave < NP1) {
                const f32x4 X = mma_f32_strided<16>(zero4(), sA + 16 * pi * PA + 16 * pi, PA, 1,
                                                    sA + 16 * pj * PA + 16 * pi, PA, 1, lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sA[(16 * pi + row0 + i) * PA + 16 * pj + col] = -X[i];
                    sT[(16 * pi + row0 + i) * PC + 16 * pj + col] = fromf<OpT>(-X[i]);
                    sA[(16 * pj + row0 + i) * PA + 16 * pi + col] = 0.f;
                }
            }
            __syncthreads();
        }
        if constexpr (NB == 4) {
            // 32 -> 64: T_LL = -T1 (A_LL T0), T0 / T1 the 32x32 diagonal inverses
            const int mt = wave >> 1, nt = wave & 1;
            const int row0 = 4 * (lane >> 4), col = lane & 15;
            const f32x4 M = mma_f32_strided<32>(zero4(), sA + (32 + 16 * mt) * PA, PA, 1,
                                                sA + 16 * nt, PA, 1, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) sA[(16 * mt + row0 + i) * PA + 32 + 16 * nt + col] = M[i];
            __syncthreads();
            const f32x4 X = mma_f32_strided<32>(zero4(), sA + (32 + 16 * mt) * PA + 32, PA, 1,
                                                sA + 32 + 16 * nt, PA, 1, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sT[(32 + 16 * mt + row0 + i) * PC + 16 * nt + col] = fromf<OpT>(-X[i]);
            __syncthreads();
        }

        // ---- (5) Kbar S^T -> R = beta (V - Kbar S^T) (stored transposed); Qbar S^T kept
#pragma unroll
        for (int s = 0; s < K::OT_PER_W; ++s) {
            const int ot = wave + 4 * s;
            if (ot < K::NOT) {
                const int rb = ot / NBV, cb = ot % NBV, n = lane & 15;
                const f32x4 ak = mma_tile<OpT, DK>(zero4(), sKbar + 16 * rb * PK, PK, sS + 16 * cb * PK, PK, lane);
                Oacc[s] = mma_tile<OpT, DK>(zero4(), sQbar + 16 * rb * PK, PK, sS + 16 * cb * PK, PK, lane);
                f32x4 rv;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * rb + 4 * (lane >> 4) + i;
                    rv[i] = sBeta[r] * (tof(sV[r * PV + 16 * cb + n]) - ak[i]);
                }
                store4(sRT + (16 * cb + n) * PC + 16 * rb + 4 * (lane >> 4), rv);
            }
        }
        __syncthreads();

        // ---- (6) E = T R (stored transposed)
#pragma unroll
        for (int s = 0; s < K::OT_PER_W; ++s) {
            const int ot = wave + 4 * s;
            if (ot < K::NOT) {
                const int rb = ot / NBV, cb = ot % NBV, n = lane & 15;
                const f32x4 e = mma_tile<OpT, C>(zero4(), sT + 16 * rb * PC, PC, sRT + 16 * cb * PC, PC, lane,
                                                 16 * (rb + 1));
                store4(sET + (16 * cb + n) * PC + 16 * rb + 4 * (lane >> 4), e);
            }
        }
        __syncthreads();

        // ---- (7) O = Qbar S^T + P E;  S^T <- Diag(e^{G_last}) S^T + Ktil^T E
#pragma unroll
        for (int s = 0; s < K::OT_PER_W; ++s) {
            const int ot = wave + 4 * s;
            if (ot < K::NOT) {
                const int rb = ot / NBV, cb = ot % NBV;
                Oacc[s] = mma_tile<OpT, C>(Oacc[s], sP + 16 * rb * PC, PC, sET + 16 * cb * PC, PC, lane,
                                           16 * (rb + 1));
            }
        }
#pragma unroll
        for (int s = 0; s < K::ST_PER_W; ++s) {
            const int st = wave + 4 * s;
            if (st < K::NST) {
                const int ct = st / NBV, sb = st % NBV;
                const f32x4 acc = mma_tile<OpT, C>(zero4(), sKtT + 16 * ct * PC, PC, sET + 16 * sb * PC, PC, lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) Sreg[s][i] = Sreg[s][i] * sGL[16 * ct + 4 * (lane >> 4) + i] + acc[i];
            }
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < K::OT_PER_W; ++s) {
            const int ot = wave + 4 * s;
            if (ot < K::NOT) {
                const int rb = ot / NBV, cb = ot % NBV, n = lane & 15;
#pragma unroll
                for (int i = 0; i < 4; ++i) sO[(16 * rb + 4 * (lane >> 4) + i) * BV + 16 * cb + n] = fromf<In>(Oacc[s][i]);
            }
        }
#pragma unroll
        for (int s = 0; s < K::ST_PER_W; ++s) {
            const int st = wave + 4 * s;
            if (st < K::NST) {
                const int ct = st / NBV, sb = st % NBV;
                store4(sS + (16 * sb + (lane & 15)) * PK + 16 * ct + 4 * (lane >> 4), Sreg[s]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < K::VCH_PER_T; ++u) {
            const int idx = tid + u * K::NT;
            if (idx < K::NVCH) {
                const int r = idx / (BV / VE), cc = idx % (BV / VE);
                if (r < nval)
                    *(f32x4 *)(out + ((tok0 + t0 + r) * H + h) * dv + vb * BV + cc * VE) =
                        *(const f32x4 *)(sO + r * BV + cc * VE);
            }
        }
    }

    if (S_final) {
#pragma unroll
        for (int s = 0; s < K::ST_PER_W; ++s) {
            const int st = wave + 4 * s;
            if (st < K::NST) {
                const int ct = st / NBV, sb = st % NBV;
                const int irow = 16 * sb + (lane & 15), c = 16 * ct + 4 * (lane >> 4);
                *(f32x4 *)(S_final + ((long)head * dv + vb * BV + irow) * DK + c) = Sreg[s];
            }
        }
    }
}

template <typename In, int DK, int BV, int C>
hipError_t launch_chunk_t(const ChunkArgs &a)
{
    typedef ChunkCfg<In, DK, BV, C> K;
    if constexpr (!K::fits) {
        return hipErrorInvalidConfiguration;
    } else {
        const int nheads = a.nseq * a.H;
        const int nvb = a.dv / BV;
        const int grid = nheads * nvb;
        if (grid == 0) return hipSuccess;
        const int xcd_map = (nheads % 8 == 0) ? 1 : 0;
        hipLaunchKernelGGL((chunk_fwd_kernel<In, DK, BV, C>), dim3(grid), dim3(K::NT), 0, a.stream,
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
    if (BV == BV_ && C == C_) return ChunkCfg<In, DK, BV_, C_>::fits;
    KDA_CASE(16, 16) KDA_CASE(16, 32) KDA_CASE(16, 64)
    KDA_CASE(32, 16) KDA_CASE(32, 32) KDA_CASE(32, 64)
    KDA_CASE(64, 16) KDA_CASE(64, 32) KDA_CASE(64, 64)
#undef KDA_CASE
    return false;
}

}  // namespace kda
