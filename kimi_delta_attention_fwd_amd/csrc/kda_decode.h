// KDA decode step for gfx950: one token per (sequence, head), state in place.
//
// Per state row i (a value channel; the row's DK entries are key channels):
//   s~   = s (.) alpha                 decay, alpha = exp(log_alpha)
//   p    = <s~, k>                     prediction of v_i
//   e    = beta (v_i - p)              error
//   s'   = s~ + e k                    write
//   o_i  = <s', q>                     readout
// ("KDA derivation summary" page, sect. 3 and 5; the fused recurrent mode of
// sect. 6; a step only reads and writes the fixed-size state, "Linear/sparse
// attention tutorial" page, sect. 8.1.)
//
// The state dominates the traffic (64 KiB per head at d = 128 against < 1 KiB
// of token data), so the kernel is a streaming kernel: each row is read once
// and written once with 16-byte nontemporal accesses (the state is not reused
// within a step, so it should not displace cached data), and the two row
// reductions use DPP within groups of DK/16 lanes.  The single step gives a
// workgroup of 256 lanes RPP = 256 / (DK/16) rows of one head, so a head
// spans ceil(dv / RPP) workgroups (4 at d = 128), each lane holds one row
// slice (four 16-byte loads in flight), and the head's token data is read by
// each of them from cache: many small workgroups stream faster than a few
// that keep several rows per lane in flight.  The multi-token kernel splits
// heads the same way and stages its tokens in LDS.
#pragma once

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// log decays of 4 key channels starting at element c of the token's
// log_alpha row: per channel (gate 0), one value per token and head at index
// tok (gate 1), or none (gate 2: alpha = 1).  With prep the argument holds
// the pre-activations g in the input type and log(alpha) = -softplus(g).
template <typename In>
__device__ __forceinline__ f32x4 decay_logs(const float *log_alpha, long c, long tok, int gate, int prep)
{
    typedef In In4 __attribute__((ext_vector_type(4)));
    if (prep) {
        const In *gp = (const In *)log_alpha;
        if (gate == 0) {
            const In4 gv = *(const In4 *)(gp + c);
            return f32x4{neg_softplus(tof(gv[0])), neg_softplus(tof(gv[1])), neg_softplus(tof(gv[2])),
                         neg_softplus(tof(gv[3]))};
        }
        if (gate == 1) {
            const float x = neg_softplus(tof(gp[tok]));
            return f32x4{x, x, x, x};
        }
        return zero4();
    }
    if (gate == 0) return *(const f32x4 *)(log_alpha + c);
    if (gate == 1) {
        const float x = log_alpha[tok];
        return f32x4{x, x, x, x};
    }
    return zero4();
}

// prep: scales the lane's 16 channels of a token's k (or q) to unit L2 norm
// over the row's LPR lanes (a zero vector stays zero).
template <int LPR>
__device__ __forceinline__ void normalise16(f32x4 (&x)[4])
{
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) ss += x[u][j] * x[u][j];
    ss = group_sum<LPR>(ss);
    const float r = ss > 0.f ? __builtin_amdgcn_rsqf(ss) : 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = x[u] * r;
}

// Variants (uniform arguments, read only when VAR): gate as in decay_logs;
// add = 1 is the additive write e = beta v (no prediction).
template <typename In, int DK, bool VAR>
__global__ void __launch_bounds__(256)
decode_step_kernel(const In *__restrict__ q, const In *__restrict__ k, const In *__restrict__ v,
                   const float *__restrict__ log_alpha, const float *__restrict__ beta,
                   float *__restrict__ S, In *__restrict__ out, int dv, int gate_arg, int add_arg,
                   int prep_arg)
{
    const int gate = VAR ? gate_arg : 0, add = VAR ? add_arg : 0, prep = VAR ? prep_arg : 0;
    typedef In In4 __attribute__((ext_vector_type(4)));
    constexpr int LPR = DK / 16;          // lanes per state row, 16 floats (4 x float4) each
    constexpr int RPP = 256 / LPR;        // rows per workgroup
    const int nsplit = (dv + RPP - 1) / RPP;
    // Consecutive workgroups go to different XCDs, so each of a head's nsplit
    // workgroups fetches the head's token data (about 1.3 KiB) into its own
    // L2: 2.6% more HBM reads at d = 128.  Grouping a head's workgroups on one
    // XCD saves them but ran 0.8% slower.
    const long head = blockIdx.x / nsplit;
    const int tid = threadIdx.x, sub = tid % LPR;
    const int row = (blockIdx.x % nsplit) * RPP + tid / LPR;

    // this lane's channels: float4 index f_u = sub + LPR u, channels 4 f_u .. 4 f_u + 3
    f32x4 a[4], kk[4], qq[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const long c = head * DK + 4 * (sub + LPR * u);
        const f32x4 la = decay_logs<In>(log_alpha, c, head, gate, prep);
        const In4 kv = *(const In4 *)(k + c);
        const In4 qv = *(const In4 *)(q + c);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[u][j] = __expf(la[j]);
            kk[u][j] = tof(kv[j]);
            qq[u][j] = tof(qv[j]);
        }
    }
    if (prep) {
        normalise16<LPR>(kk);
        normalise16<LPR>(qq);
    }
    const float b = beta[head];

    // the lane groups of rows past dv (dv < RPP) have nothing to do; a whole
    // group of LPR lanes shares the row, so the reductions below stay inside
    // groups that all take the same branch
    if (row < dv) {
        f32x4 s[4];
        const float *src = S + (head * dv + row) * DK + 4 * sub;
#pragma unroll
        for (int u = 0; u < 4; ++u) s[u] = __builtin_nontemporal_load((const f32x4 *)(src + 4 * LPR * u));
        const float vi = tof(v[head * dv + row]);
        float pred = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s[u][j] *= a[u][j];
                pred += s[u][j] * kk[u][j];
            }
        pred = add ? 0.f : group_sum<LPR>(pred);
        const float e = b * (vi - pred);
        float o = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s[u][j] += e * kk[u][j];
                o += s[u][j] * qq[u][j];
            }
        o = group_sum<LPR>(o);
        float *dst = S + (head * dv + row) * DK + 4 * sub;
#pragma unroll
        for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(s[u], (f32x4 *)(dst + 4 * LPR * u));
        if (sub == 0) out[head * dv + row] = fromf<In>(o);
    }
}

// T tokens per (sequence, head) in one launch: the rows are read once, carried
// in registers through the tokens in order, and written once.  This is the
// fused recurrent mode itself (the "KDA derivation summary" page, sect. 6: a
// program per sequence, value head and value block looping the update over
// the tokens).  Token t of sequence n sits at row (n T + t) H + h of the
// [N, T, H, d] inputs.  Per token the arithmetic is the decode step's, in the
// same order, so T tokens match T calls of kda_recurrent_step bit for bit.
//
// Workgroups split a head's rows as in the single step.  The token loop would
// wait on every token's loads, so the workgroup first stages a tile of up to
// TT tokens in LDS (k, q, the decay factors alpha, beta, and v of its own
// rows), with one set of loads in flight for the whole tile, and then runs
// the tile's tokens from LDS.  Each alpha is computed once per workgroup.
template <typename In, int DK, bool VAR>
__global__ void __launch_bounds__(256)
decode_multi_kernel(const In *__restrict__ q, const In *__restrict__ k, const In *__restrict__ v,
                    const float *__restrict__ log_alpha, const float *__restrict__ beta,
                    float *__restrict__ S, In *__restrict__ out, int T, int H, int dv, int xcd_map,
                    int gate_arg, int add_arg, int prep_arg)
{
    const int gate = VAR ? gate_arg : 0, add = VAR ? add_arg : 0, prep = VAR ? prep_arg : 0;
    typedef In In4 __attribute__((ext_vector_type(4)));
    constexpr int LPR = DK / 16;
    constexpr int RPP = 256 / LPR;        // rows per workgroup, as in the single step
    constexpr int TT = 16;                // tokens staged per tile
    constexpr int C4 = DK / 4;            // 4-channel groups per token
    __shared__ __attribute__((aligned(16))) float s_a[TT][DK], s_k[TT][DK], s_q[TT][DK], s_v[TT][RPP], s_b[TT];
    const int nsplit = (dv + RPP - 1) / RPP;
    long head;
    int part;
    if (xcd_map) {
        // workgroups are dealt to the 8 XCDs round-robin: the nsplit
        // workgroups of a head share an XCD, so its tokens come from HBM once
        // (the head count is a multiple of 8 here)
        const long slot = blockIdx.x >> 3;
        head = (slot / nsplit) * 8 + (blockIdx.x & 7);
        part = (int)(slot % nsplit);
    } else {
        head = blockIdx.x / nsplit;
        part = blockIdx.x % nsplit;
    }
    const long n = head / H, h = head % H;
    const int tid = threadIdx.x, sub = tid % LPR, rloc = tid / LPR;
    const int row = part * RPP + rloc;
    const bool active = row < dv;         // whole groups of LPR lanes share a row

    f32x4 s[4];
    if (active) {
        const float *src = S + (head * dv + row) * DK + 4 * sub;
#pragma unroll
        for (int u = 0; u < 4; ++u) s[u] = __builtin_nontemporal_load((const f32x4 *)(src + 4 * LPR * u));
    }
    for (int t0 = 0; t0 < T; t0 += TT) {
        const int nt = T - t0 < TT ? T - t0 : TT;
        __syncthreads();   // the previous tile's reads are done
        for (int i = tid; i < nt * C4; i += 256) {
            const int tl = i / C4, c = 4 * (i % C4);
            const long tok = (n * T + t0 + tl) * H + h;
            const f32x4 la = decay_logs<In>(log_alpha, tok * DK + c, tok, gate, prep);
            const In4 kv = *(const In4 *)(k + tok * DK + c);
            const In4 qv = *(const In4 *)(q + tok * DK + c);
            f32x4 av, kf, qf;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                av[j] = __expf(la[j]);
                kf[j] = tof(kv[j]);
                qf[j] = tof(qv[j]);
            }
            *(f32x4 *)&s_a[tl][c] = av;
            *(f32x4 *)&s_k[tl][c] = kf;
            *(f32x4 *)&s_q[tl][c] = qf;
        }
        for (int i = tid; i < nt * RPP; i += 256) {
            const int tl = i / RPP, r = i % RPP;
            const long tok = (n * T + t0 + tl) * H + h;
            if (part * RPP + r < dv) s_v[tl][r] = tof(v[tok * dv + part * RPP + r]);
        }
        if (tid < nt) s_b[tid] = beta[(n * T + t0 + tid) * H + h];
        __syncthreads();
        for (int tl = 0; tl < nt; ++tl) {
            f32x4 a[4], kk[4], qq[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = 4 * (sub + LPR * u);
                a[u] = *(const f32x4 *)&s_a[tl][c];
                kk[u] = *(const f32x4 *)&s_k[tl][c];
                qq[u] = *(const f32x4 *)&s_q[tl][c];
            }
            if (prep) {
                normalise16<LPR>(kk);
                normalise16<LPR>(qq);
            }
            const float b = s_b[tl];
            if (active) {
                const long tok = (n * T + t0 + tl) * H + h;
                const float vi = s_v[tl][rloc];
                float pred = 0.f;
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        s[u][j] *= a[u][j];
                        pred += s[u][j] * kk[u][j];
                    }
                pred = add ? 0.f : group_sum<LPR>(pred);
                const float e = b * (vi - pred);
                float o = 0.f;
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        s[u][j] += e * kk[u][j];
                        o += s[u][j] * qq[u][j];
                    }
                o = group_sum<LPR>(o);
                if (sub == 0) out[tok * dv + row] = fromf<In>(o);
            }
        }
    }
    if (active) {
        float *dst = S + (head * dv + row) * DK + 4 * sub;
#pragma unroll
        for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(s[u], (f32x4 *)(dst + 4 * LPR * u));
    }
}

template <typename In, int DK>
hipError_t launch_decode_multi_t(const DecodeArgs &a, int T)
{
    constexpr int RPP = 256 / (DK / 16);
    const long nheads = (long)a.N * a.H, nsplit = (a.dv + RPP - 1) / RPP;
    const long grid = nheads * nsplit;   // workgroups: RPP rows of one head each
    if (grid == 0) return hipSuccess;
    const int xcd = (nsplit > 1 && nheads % 8 == 0) ? 1 : 0;
    if (a.gate != 0 || a.add != 0 || a.prep != 0)
        hipLaunchKernelGGL((decode_multi_kernel<In, DK, true>), dim3((unsigned)grid), dim3(256), 0, a.stream,
                           (const In *)a.q, (const In *)a.k, (const In *)a.v, a.log_alpha, a.beta, a.S,
                           (In *)a.out, T, a.H, a.dv, xcd, a.gate, a.add, a.prep);
    else
        hipLaunchKernelGGL((decode_multi_kernel<In, DK, false>), dim3((unsigned)grid), dim3(256), 0, a.stream,
                           (const In *)a.q, (const In *)a.k, (const In *)a.v, a.log_alpha, a.beta, a.S,
                           (In *)a.out, T, a.H, a.dv, xcd, 0, 0, 0);
    return hipGetLastError();
}

template <typename In, int DK>
hipError_t launch_decode_t(const DecodeArgs &a)
{
    constexpr int RPP = 256 / (DK / 16);
    const long grid = (long)a.N * a.H * ((a.dv + RPP - 1) / RPP);   // workgroups: RPP rows of one head each
    if (grid == 0) return hipSuccess;
    if (a.gate != 0 || a.add != 0 || a.prep != 0)
        hipLaunchKernelGGL((decode_step_kernel<In, DK, true>), dim3((unsigned)grid), dim3(256), 0, a.stream,
                           (const In *)a.q, (const In *)a.k, (const In *)a.v, a.log_alpha, a.beta, a.S,
                           (In *)a.out, a.dv, a.gate, a.add, a.prep);
    else
        hipLaunchKernelGGL((decode_step_kernel<In, DK, false>), dim3((unsigned)grid), dim3(256), 0, a.stream,
                           (const In *)a.q, (const In *)a.k, (const In *)a.v, a.log_alpha, a.beta, a.S,
                           (In *)a.out, a.dv, 0, 0, 0);
    return hipGetLastError();
}

}  // namespace kda
