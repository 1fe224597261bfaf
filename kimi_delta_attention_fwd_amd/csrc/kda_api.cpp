// libkda C ABI: argument validation and dispatch to the HIP kernels.
//
// Every check below runs before the first HIP call, so a rejected call has no
// side effect and needs no GPU.  The operation, layouts and error codes are
// documented in include/libkda.h.
#include "libkda.h"

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "kda_launch.h"

namespace {

thread_local char g_err[512] = "";

kda_status_t fail(kda_status_t st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

kda_status_t ok()
{
    g_err[0] = '\0';
    return KDA_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

bool supported_c(int c) { return c == 16 || c == 32 || c == 64; }

// Byte ranges [p, p + n) overlap (empty ranges never do).
bool overlap(const void *a, uint64_t na, const void *b, uint64_t nb)
{
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

struct Buf {
    const void *p;
    uint64_t bytes;
    const char *name;
};

// out and the state output must not overlap any input (S0 excluded from `ins`); the
// state output may alias S0 only as the identical pointer.
kda_status_t check_aliasing(const Buf &out, const Buf *ins, int nin, const Buf &sfin, const Buf &s0)
{
    for (int i = 0; i < nin; ++i) {
        if (overlap(out.p, out.bytes, ins[i].p, ins[i].bytes))
            return fail(KDA_ERR_ALIASING, "%s overlaps input %s", out.name, ins[i].name);
        if (overlap(sfin.p, sfin.bytes, ins[i].p, ins[i].bytes))
            return fail(KDA_ERR_ALIASING, "%s overlaps input %s", sfin.name, ins[i].name);
    }
    if (overlap(out.p, out.bytes, sfin.p, sfin.bytes))
        return fail(KDA_ERR_ALIASING, "%s overlaps %s", out.name, sfin.name);
    if (overlap(out.p, out.bytes, s0.p, s0.bytes))
        return fail(KDA_ERR_ALIASING, "%s overlaps %s", out.name, s0.name);
    if (sfin.p != s0.p && overlap(sfin.p, sfin.bytes, s0.p, s0.bytes))
        return fail(KDA_ERR_ALIASING, "%s partially overlaps %s (only identical pointers may alias)",
                    sfin.name, s0.name);
    return KDA_OK;
}

// Value-block width of the chunk kernel: the widest block (at most maxbv) that
// fits the LDS.  A workgroup walks all chunks of its sequence (or segment)
// whatever its width, so a narrower block never shortens the serial chain: it
// only repeats the operand waves' work in more workgroups and leaves more tile
// jobs to each state wave (one state wave at BV = 16).  Measured on one MI355X:
// B1 H16 T65536 d128 single pass 4.44 ms at BV = 64 against 5.23 ms at 16, and
// B2 H4 T1024 d64 63 against 67 us.  KDA_CHUNK_BV overrides the choice (tests
// and tuning).
int choose_bv(bool f32, int dk, int dv, int C, int maxbv = 64)
{
    if (const char *env = std::getenv("KDA_CHUNK_BV")) {
        const int bv = std::atoi(env);
        if ((bv == 16 || bv == 32 || bv == 64) && bv <= dv && bv <= maxbv && kda::chunk_fits(f32, dk, bv, C))
            return bv;
    }
    for (int bv : {64, 32, 16})
        if (bv <= dv && bv <= maxbv && kda::chunk_fits(f32, dk, bv, C)) return bv;
    return 0;
}

constexpr int kMaxSegments = 1024;

// Chunk length the kernels run for a requested C: C itself, or the largest
// shorter one whose kernel fits the LDS (fp32 operands at dk = 128: 64-token
// chunks would need about 280 KB, 173 KB even single-buffered, so those
// requests run as 32-token chunks).  The chunk length is a schedule choice:
// both give the recurrence's result, up to rounding.
int run_chunk_len(bool f32, int dk, int C)
{
    for (int c = C; c >= 16; c /= 2)
        if (kda::chunk_fits(f32, dk, 16, c)) return c;
    return 0;
}

// Variant selector of the *_ex entry points: bits 0-1 the gate (0 per
// channel, 1 one value per token and head, 2 none), bit 2 the additive write,
// bit 3 raw inputs (q, k normalised in the kernel, gate pre-activations).
bool valid_variant(int variant) { return (variant & ~15) == 0 && (variant & 3) != 3; }

// Bit 4 of the chunk entry points' variant: the segmented schedule without a
// second pass (KDA_SCHED_MAP_OUTPUTS).
constexpr int kSchedMapOut = 16;

// Bytes and alignment of the gate argument: fp32 log_alpha, or with raw
// inputs g in the input type (es bytes per element).
uint64_t gate_bytes(int variant, uint64_t ntok_heads, int dk, uint64_t es)
{
    const uint64_t e = (variant & 8) ? es : 4;
    switch (variant & 3) {
    case 0: return ntok_heads * (uint64_t)dk * e;
    case 1: return ntok_heads * e;
    default: return 0;
    }
}

uintptr_t gate_align(int variant, uint64_t es)
{
    if ((variant & 3) == 0) return 16;
    return (variant & 8) ? es : 4;
}

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

// Workspace of the segment-parallel schedule: the segment maps, then the
// segments' incoming states (fp32).
uint64_t seg_map_bytes(uint64_t nheads, int dk, int dv, int nseg)
{
    return align256(nheads * (uint64_t)(nseg - 1) * (uint64_t)(dv + dk) * (uint64_t)dk * 4u);
}

uint64_t seg_workspace_bytes(uint64_t nheads, int dk, int dv, int nseg)
{
    if (nseg <= 1) return 0;
    return seg_map_bytes(nheads, dk, dv, nseg) + nheads * (uint64_t)nseg * (uint64_t)dv * (uint64_t)dk * 4u;
}

// Workspace of the schedule without a second pass: a map for every segment
// (slot 0 unused), the incoming states, then the virtual rows' outputs
// [ntok, H, dk] in the input type (es bytes).
uint64_t mout_map_bytes(uint64_t nheads, int dk, int dv, int nseg)
{
    return align256(nheads * (uint64_t)nseg * (uint64_t)(dv + dk) * (uint64_t)dk * 4u);
}

uint64_t mout_start_bytes(uint64_t nheads, int dk, int dv, int nseg)
{
    return align256(nheads * (uint64_t)nseg * (uint64_t)dv * (uint64_t)dk * 4u);
}

uint64_t mout_workspace_bytes(uint64_t nheads, uint64_t ntok_heads, int dk, int dv, int nseg, uint64_t es)
{
    if (nseg <= 1) return 0;
    return mout_map_bytes(nheads, dk, dv, nseg) + mout_start_bytes(nheads, dk, dv, nseg) + ntok_heads * dk * es;
}

// Compute units of the current device, queried once per device (256, the
// MI355X count, when the query fails).
int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int m = 0;
    if (hipDeviceGetAttribute(&m, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || m <= 0) m = 256;
    if (dev < 64) cache[dev].store(m, std::memory_order_relaxed);
    return m;
}

// Rounds of workgroups in the map launch: g workgroups, one per CU, the first
// nA of them (segment 0's whole pass) holding their CUs for the whole launch.
// Workgroups are dealt to the 8 XCDs round-robin and, within one, to its 4
// shader engines round-robin (cus / 32 CUs each), so a later round fits only
// where the engine holding the most lead workgroups has CUs left for its
// share.  (Measured: 496 workgroups with 16 lead ones take three rounds, 480
// with 32 take two.)
long map_launch_rounds(long g, long nA, int cus)
{
    if (g <= cus) return 1;
    const long per_se = cus / 32 > 0 ? cus / 32 : 1;
    const long free_se = per_se - (nA + 31) / 32;
    if (free_se <= 0) return 1L << 30;
    return 1 + (g - cus + 32 * free_se - 1) / (32 * free_se);
}

// Lead segment of the segmented schedule (tenths of a later segment's length).
// The map launch holds segment 0's whole pass (nheads * dv / bv workgroups)
// beside the maps of segments 1 .. nseg - 2 ((dv + dk) / bv each); a map chunk
// costs about 0.85 of a full one, so segment 0 gets 0.85 chunks per chunk of a
// map times the launch's rounds of workgroups.  KDA_SEG_LEAD overrides it
// (0: equal segments, segment 0 mapped like the others).
int seg_lead(long nheads, int dk, int dv, int bv, int nseg, int cus)
{
    if (nseg < 2) return 0;
    if (const char *env = std::getenv("KDA_SEG_LEAD")) {
        const int v = std::atoi(env);
        if (v >= 0 && v <= 1000) return v;
    }
    const long nA = nheads * (dv / bv);
    const long rounds = map_launch_rounds(nheads * (long)(nseg - 2) * ((dv + dk) / bv) + nA, nA, cus);
    return rounds > 100 ? 1000 : (int)(8.5 * (double)rounds + 0.5);
}

// Lead segment of the schedule without a second pass: the map launch holds
// segment 0's pass beside the maps of segments 1 .. nseg - 1, whose chunks
// (with their outputs) cost about what a full one does, so segment 0 gets one
// chunk per map chunk and round of workgroups.
int seg_lead_mout(long nheads, int dk, int dv, int bv, int nseg, int cus)
{
    if (nseg < 2) return 0;
    if (const char *env = std::getenv("KDA_SEG_LEAD")) {
        const int v = std::atoi(env);
        if (v >= 1 && v <= 1000) return v;
    }
    const long nA = nheads * (dv / bv);
    const long rounds = map_launch_rounds(nheads * (long)(nseg - 1) * ((dv + dk) / bv) + nA, nA, cus);
    return rounds > 100 ? 1000 : (int)(10 * rounds);
}

// Segment count for a dense batch from a model of the run time in chunk steps.
// A pass of g workgroups that each walk L chunks takes ceil(g / CUs) (L + 1)
// steps (one workgroup per compute unit; the extra step is the prologue: the
// first chunk's operands, the incoming state and the final store).  With s
// segments the map launch takes max(L0 + 1, 0.85 rounds (L + 1)) (the
// lead segment's whole pass beside the maps, a map chunk being about 0.85 of a
// full one), the serial composition 0.3 (dk / 64)^1.5 steps per segment, the
// second pass ceil(g3 / CUs) (L + 1) over segments 1 .. s - 1, and the two
// extra launches about one step; rounds as in map_launch_rounds.  Fitted to
// measured runs: 1 segment for B=4 H=32 T=8192, 9 for B=1 H=16 T=65536
// (d = 128), 9 for B=2 H=4 T=1024 (d = 64).
//
// Schedule without a second pass (mout): the map launch takes max(L0 + 1,
// rounds (L + 1)) steps (its map chunks, which also form the outputs, cost
// about a full chunk), the composition as above, and the epilogue streams m
// and out once: about one step per 20 MB.  Fitted to measured runs (ms, the
// model's segment count marked *): B=1 H=16 T=65536 d=128: one-pass 8* 1.11,
// two-pass 9 1.23; B=2 H=16 T=32768 d=128: one-pass 4* 0.97, two-pass 5 1.04
// (the one shape where the schedule comparison misses: the models put the
// two within 1% and pick the two-pass one);
// B=1 H=16 T=65536 d=64: one-pass 8* 0.52, two-pass 16 0.59; B=1 H=8
// T=131072 d=128: one-pass 8* 1.24, two-pass 16 1.43; fp32 B=1 H=16 T=65536
// d=128: one-pass 8* 3.69, two-pass 9 4.07 (one segment fewer or more: slower
// in every case).
double auto_cost(bool f32, int B, int T, int H, int dk, int dv, int C, bool mout, int &best_s)
{
    best_s = 1;
    if (B <= 0 || T <= 0 || H <= 0 || !supported_d(dk) || !supported_d(dv) || !supported_c(C)) return 0.0;
    const int Cr = run_chunk_len(f32, dk, C);
    if (Cr == 0) return 0.0;
    const int cus = device_cus();
    const long nch = (T + Cr - 1) / Cr, nheads = (long)B * H;
    double best = 0.0;
    for (int s = 1; s <= 64 && s <= nch; ++s) {
        const int bv = choose_bv(f32, dk, dv, Cr, s > 1 ? dk : 64);
        if (bv == 0) continue;
        const long nvA = dv / bv, nvB = (dv + dk) / bv;
        double cost;
        if (s == 1) {
            cost = (double)((nheads * nvA + cus - 1) / cus) * (double)(nch + 1);
        } else if (mout) {
            const int lead = seg_lead_mout(nheads, dk, dv, bv, s, cus);
            const long L = (10 * nch + 10 * (s - 1) + lead - 1) / (10 * (s - 1) + lead);
            const long L0 = nch - (s - 1) * L > 0 ? nch - (s - 1) * L : 0;
            const long g1 = nheads * ((s - 1) * nvB + nvA);
            const double map = (double)map_launch_rounds(g1, nheads * nvA, cus) * (double)(L + 1);
            const double epi = (double)B * (double)T * (double)H * (double)(dk + 2 * dv) * (f32 ? 4.0 : 2.0) / 20e6;
            cost = (map > (double)(L0 + 1) ? map : (double)(L0 + 1)) + 0.3 * std::pow(dk / 64.0, 1.5) * s + epi + 1.0;
        } else {
            const int lead = seg_lead(nheads, dk, dv, bv, s, cus);
            const long L = (10 * nch + 10 * (s - 1) + lead - 1) / (10 * (s - 1) + lead);
            const long L0 = nch - (s - 1) * L > 0 ? nch - (s - 1) * L : 0;
            const long g1 = nheads * ((s - 2) * nvB + nvA), g3 = nheads * (s - 1) * nvA;
            const double map = 0.85 * (double)map_launch_rounds(g1, nheads * nvA, cus) * (double)(L + 1);
            cost = (map > (double)(L0 + 1) ? map : (double)(L0 + 1)) + 0.3 * std::pow(dk / 64.0, 1.5) * s +
                   (double)((g3 + cus - 1) / cus) * (double)(L + 1) + 1.0;
        }
        if (s == 1 || cost < best) {
            best = cost;
            best_s = s;
        }
    }
    return best;
}

int auto_segments(bool f32, int B, int T, int H, int dk, int dv, int C, bool mout = false)
{
    int s = 1;
    auto_cost(f32, B, T, H, dk, dv, C, mout, s);
    return s;
}

hipError_t dispatch_chunk(bool f32, const kda::ChunkArgs &a)
{
    switch (a.dk) {
    case 16: return f32 ? kda::launch_chunk_f32_16(a) : kda::launch_chunk_bf16_16(a);
    case 32: return f32 ? kda::launch_chunk_f32_32(a) : kda::launch_chunk_bf16_32(a);
    case 64: return f32 ? kda::launch_chunk_f32_64(a) : kda::launch_chunk_bf16_64(a);
    case 128: return f32 ? kda::launch_chunk_f32_128(a) : kda::launch_chunk_bf16_128(a);
    default: return hipErrorInvalidConfiguration;
    }
}

// Shared body of the four chunk entry points.  For the dense layout nseq = B
// and each sequence has T tokens; for the packed layout nseq = N, the stream
// holds T_total tokens and cu_seqlens (device memory) delimits the sequences.
kda_status_t chunk_common(bool f32, bool varlen, const void *q, const void *k, const void *v,
                          const float *log_alpha, const float *beta, const float *S0, void *out,
                          float *S_final, const int32_t *cu_seqlens, int nseq, int T, int T_total,
                          int H, int dk, int dv, int C, void *stream, int nseg = 1, void *workspace = nullptr,
                          uint64_t workspace_bytes = 0, int variant = 0,
                          const kda::StaticScratch *scratch = nullptr)
{
    const bool mout = (variant & kSchedMapOut) != 0;
    variant &= ~kSchedMapOut;
    if (!valid_variant(variant)) return fail(KDA_ERR_BAD_SHAPE, "invalid variant %d", variant | (mout ? kSchedMapOut : 0));
    if (mout && scratch) return fail(KDA_ERR_UNSUPPORTED, "the allocation-free entry point has no one-pass schedule");
    const int gate = variant & 3;
    // nseg = 0 with the one-pass schedule and packed sequences: two segments,
    // only the sequences much longer than the rest split, on the device
    const bool plan = varlen && mout && nseg == 0 && !scratch;
    if (plan) nseg = 2;
    if (nseg < 1 || nseg > kMaxSegments)
        return fail(KDA_ERR_BAD_SHAPE, "segment count must be in [1, %d] (got %d)", kMaxSegments, nseg);
    if (nseq < 0 || T < 0 || T_total < 0)
        return fail(KDA_ERR_BAD_SHAPE, "negative size (sequences %d, T %d, T_total %d)", nseq, T, T_total);
    if (H < 1) return fail(KDA_ERR_BAD_SHAPE, "H must be >= 1 (got %d)", H);
    if (!supported_d(dk) || !supported_d(dv))
        return fail(KDA_ERR_UNSUPPORTED, "dk and dv must be 16, 32, 64 or 128 (got %d, %d)", dk, dv);
    if (!supported_c(C)) return fail(KDA_ERR_UNSUPPORTED, "C must be 16, 32 or 64 (got %d)", C);

    const uint64_t ntok = varlen ? (uint64_t)T_total : (uint64_t)nseq * (uint64_t)T;
    const uint64_t nheads = (uint64_t)nseq * (uint64_t)H;
    // the kernels address the token rows of one chunk with 32-bit byte offsets
    // (64 rows of H * d elements of up to 4 bytes)
    if (ntok * (uint64_t)H * 128u > (uint64_t)1 << 60 || nheads * 8u > (uint64_t)INT32_MAX ||
        (uint64_t)H * 128u * 64u * 4u > (uint64_t)INT32_MAX ||
        nheads * (uint64_t)nseg * (uint64_t)(dv + dk) / 16u > (uint64_t)INT32_MAX)
        return fail(KDA_ERR_BAD_SHAPE, "problem too large");
    const uint64_t nk = ntok * H * dk, nv = ntok * H * dv, nb = ntok * H, ns = nheads * dv * dk;

    if (ntok > 0 && (!q || !k || !v || (gate != 2 && !log_alpha) || !beta || !out))
        return fail(KDA_ERR_NULL_POINTER, "q, k, v, log_alpha, beta and out are required when there are tokens");
    if (gate == 2) log_alpha = nullptr;   // not read
    if (varlen && nseq > 0 && !cu_seqlens) return fail(KDA_ERR_NULL_POINTER, "cu_seqlens is required");
    const uint64_t es = f32 ? 4 : 2;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(log_alpha, gate_align(variant, es)))
        return fail(KDA_ERR_MISALIGNED, "q, k, v, out and log_alpha must be 16-byte aligned (log_alpha: its "
                                         "element size with one gate per token)");
    if (!aligned(S0, 16) || !aligned(S_final, 16))
        return fail(KDA_ERR_MISALIGNED, "S0 and S_final must be 16-byte aligned");
    if (!aligned(beta, 4) || !aligned(cu_seqlens, 4))
        return fail(KDA_ERR_MISALIGNED, "beta and cu_seqlens must be 4-byte aligned");

    const Buf ins[] = {{q, nk * es, "q"}, {k, nk * es, "k"}, {v, nv * es, "v"},
                       {log_alpha, gate_bytes(variant, nb, dk, es), "log_alpha"}, {beta, nb * 4, "beta"},
                       {cu_seqlens, varlen ? (uint64_t)(nseq + 1) * 4 : 0, "cu_seqlens"}};
    kda_status_t st = check_aliasing(Buf{out, nv * es, "out"}, ins, 6,
                                     Buf{S_final, S_final ? ns * 4 : 0, "S_final"},
                                     Buf{S0, S0 ? ns * 4 : 0, "S0"});
    if (st != KDA_OK) return st;
    // (the device-side split also keeps its plan, one int per sequence, after m)
    const uint64_t wsb = mout ? mout_workspace_bytes(nheads, ntok * H, dk, dv, nseg, f32 ? 4 : 2) + (plan ? 4u * (uint64_t)nseq : 0u)
                              : seg_workspace_bytes(nheads, dk, dv, nseg);
    if (nseg > 1 && scratch) {
        // the library's own fixed-size array: it aliases nothing the caller owns
        if (wsb > scratch->bytes)
            return fail(KDA_ERR_UNSUPPORTED,
                        "the segmented schedule needs %llu bytes of scratch here, more than the %llu-byte "
                        "static array of the allocation-free entry point (use fewer segments or the "
                        "workspace entry point)",
                        (unsigned long long)wsb, (unsigned long long)scratch->bytes);
    } else if (nseg > 1) {
        if (!workspace) return fail(KDA_ERR_NULL_POINTER, "the segmented schedule needs a workspace");
        if (!aligned(workspace, 256)) return fail(KDA_ERR_MISALIGNED, "workspace must be 256-byte aligned");
        if (workspace_bytes < wsb)
            return fail(KDA_ERR_BAD_SHAPE, "workspace holds %llu bytes, %llu needed",
                        (unsigned long long)workspace_bytes, (unsigned long long)wsb);
        const Buf all[] = {ins[0], ins[1], ins[2], ins[3], ins[4], ins[5], Buf{out, nv * es, "out"},
                           Buf{S_final, S_final ? ns * 4 : 0, "S_final"}, Buf{S0, S0 ? ns * 4 : 0, "S0"}};
        for (const Buf &b : all)
            if (overlap(workspace, wsb, b.p, b.bytes))
                return fail(KDA_ERR_ALIASING, "workspace overlaps %s", b.name);
    }

    const int Crun = run_chunk_len(f32, dk, C);
    const int BV = Crun > 0 ? choose_bv(f32, dk, dv, Crun, nseg > 1 ? dk : 64) : 0;
    if (BV == 0)
        return fail(KDA_ERR_UNSUPPORTED, "no %s kernel fits LDS for dk=%d, dv=%d, C=%d",
                    f32 ? "fp32" : "bf16", dk, dv, C);
    if (nheads == 0 || (ntok == 0 && !S_final)) return ok();
    if (ntok == 0) nseg = 1;   // nothing to split: S0 (or zeros) is copied to S_final
    if (nseg > 1 && scratch) {   // every check has passed: now the (first) HIP call
        const char *why = "unknown";
        workspace = scratch->get(&why);
        if (!workspace) return fail(KDA_ERR_HIP, "static scratch array not available: %s", why);
    }

    kda::ChunkArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.log_alpha = log_alpha;
    a.beta = beta;
    a.S0 = S0;
    a.out = out;
    a.S_final = S_final;
    a.cu_seqlens = varlen ? cu_seqlens : nullptr;
    a.nseq = nseq;
    a.T = varlen ? T_total : T;
    a.H = H;
    a.dk = dk;
    a.dv = dv;
    a.C = Crun;
    a.BV = BV;
    a.nsegs = nseg;
    a.gate = gate;
    a.add = (variant >> 2) & 1;
    a.prep = (variant >> 3) & 1;
    a.mout = (mout && nseg > 1) ? 1 : 0;
    a.cus = device_cus();
    a.mws = nullptr;
    if (a.mout) {
        a.lead = plan ? -(16 * device_cus() + dv / BV) : seg_lead_mout((long)nheads, dk, dv, BV, nseg, device_cus());
        a.seg_map = (float *)workspace;
        a.seg_start = (float *)((char *)workspace + mout_map_bytes(nheads, dk, dv, nseg));
        a.mws = (char *)workspace + mout_map_bytes(nheads, dk, dv, nseg) + mout_start_bytes(nheads, dk, dv, nseg);
    } else {
        a.lead = nseg > 1 ? seg_lead((long)nheads, dk, dv, BV, nseg, device_cus()) : 0;
        a.seg_map = nseg > 1 ? (float *)workspace : nullptr;
        a.seg_start = nseg > 1 ? (float *)((char *)workspace + seg_map_bytes(nheads, dk, dv, nseg)) : nullptr;
    }
    a.stream = (hipStream_t)stream;
    const hipError_t e = dispatch_chunk(f32, a);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "chunk kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

// Shared body of the decode entry points: T tokens per sequence (T = 1 for
// the step entry points, whose [N, H, d] tensors are the [N, 1, H, d] case).
kda_status_t step_common(bool f32, const void *q, const void *k, const void *v, const float *log_alpha,
                         const float *beta, float *S, void *out, int N, int H, int dk, int dv, void *stream,
                         int T = 1, bool multi = false, int variant = 0)
{
    if (!valid_variant(variant)) return fail(KDA_ERR_BAD_SHAPE, "invalid variant %d", variant);
    const int gate = variant & 3;
    if (N < 0) return fail(KDA_ERR_BAD_SHAPE, "N must be >= 0 (got %d)", N);
    if (T < 0) return fail(KDA_ERR_BAD_SHAPE, "T must be >= 0 (got %d)", T);
    if (H < 1) return fail(KDA_ERR_BAD_SHAPE, "H must be >= 1 (got %d)", H);
    if (!supported_d(dk) || !supported_d(dv))
        return fail(KDA_ERR_UNSUPPORTED, "dk and dv must be 16, 32, 64 or 128 (got %d, %d)", dk, dv);
    const uint64_t nheads = (uint64_t)N * (uint64_t)H;
    const uint64_t ntok = nheads * (uint64_t)T;
    // the decode grid has up to 4 workgroups per head
    if (nheads > (uint64_t)INT32_MAX / 4 || ntok * 128u > (uint64_t)1 << 60)
        return fail(KDA_ERR_BAD_SHAPE, "problem too large");
    if (nheads == 0 || T == 0) return ok();
    if (!q || !k || !v || (gate != 2 && !log_alpha) || !beta || !S || !out)
        return fail(KDA_ERR_NULL_POINTER, "q, k, v, log_alpha, beta, S and out are required");
    if (gate == 2) log_alpha = nullptr;   // not read
    const uint64_t es = f32 ? 4 : 2;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(log_alpha, gate_align(variant, es)) || !aligned(S, 16))
        return fail(KDA_ERR_MISALIGNED, "q, k, v, out, log_alpha and S must be 16-byte aligned (log_alpha: its "
                                         "element size with one gate per token)");
    if (!aligned(beta, 4)) return fail(KDA_ERR_MISALIGNED, "beta must be 4-byte aligned");
    const Buf ins[] = {{q, ntok * dk * es, "q"}, {k, ntok * dk * es, "k"}, {v, ntok * dv * es, "v"},
                       {log_alpha, gate_bytes(variant, ntok, dk, es), "log_alpha"}, {beta, ntok * 4, "beta"}};
    const Buf sb{S, nheads * dv * dk * 4, "S"};
    kda_status_t st = check_aliasing(Buf{out, ntok * dv * es, "out"}, ins, 5, sb, sb);
    if (st != KDA_OK) return st;

    kda::DecodeArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.log_alpha = log_alpha;
    a.beta = beta;
    a.S = S;
    a.out = out;
    a.N = N;
    a.H = H;
    a.dk = dk;
    a.dv = dv;
    a.gate = gate;
    a.add = (variant >> 2) & 1;
    a.prep = (variant >> 3) & 1;
    a.stream = (hipStream_t)stream;
    const hipError_t e = (multi && T > 1) ? kda::launch_decode_multi(a, T, f32) : kda::launch_decode(a, f32);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "decode kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

int kda::chunk_segmented_static(const void *q, const void *k, const void *v, const float *log_alpha,
                                const float *beta, const float *S0, void *out, float *S_final, int B, int T,
                                int H, int dk, int dv, int C, int nseg, const StaticScratch &scratch,
                                void *stream)
{
    return chunk_common(false, false, q, k, v, log_alpha, beta, S0, out, S_final, nullptr, B, T, 0, H, dk, dv, C,
                        stream, nseg, nullptr, 0, 0, &scratch);
}

extern "C" {

kda_status_t kda_chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                           const float *beta, const float *S0, void *out, float *S_final, int B, int T,
                           int H, int dk, int dv, int C, void *stream)
{
    return chunk_common(false, false, q, k, v, log_alpha, beta, S0, out, S_final, nullptr, B, T, 0, H, dk,
                        dv, C, stream);
}

kda_status_t kda_chunk_fwd_f32(const float *q, const float *k, const float *v, const float *log_alpha,
                               const float *beta, const float *S0, float *out, float *S_final, int B,
                               int T, int H, int dk, int dv, int C, void *stream)
{
    return chunk_common(true, false, q, k, v, log_alpha, beta, S0, out, S_final, nullptr, B, T, 0, H, dk,
                        dv, C, stream);
}

kda_status_t kda_chunk_fwd_varlen(const void *q, const void *k, const void *v, const float *log_alpha,
                                  const float *beta, const float *S0, void *out, float *S_final,
                                  const int32_t *cu_seqlens, int N, int T_total, int H, int dk, int dv,
                                  int C, void *stream)
{
    return chunk_common(false, true, q, k, v, log_alpha, beta, S0, out, S_final, cu_seqlens, N, 0, T_total,
                        H, dk, dv, C, stream);
}

kda_status_t kda_chunk_fwd_varlen_f32(const float *q, const float *k, const float *v,
                                      const float *log_alpha, const float *beta, const float *S0,
                                      float *out, float *S_final, const int32_t *cu_seqlens, int N,
                                      int T_total, int H, int dk, int dv, int C, void *stream)
{
    return chunk_common(true, true, q, k, v, log_alpha, beta, S0, out, S_final, cu_seqlens, N, 0, T_total,
                        H, dk, dv, C, stream);
}

kda_status_t kda_chunk_fwd_segmented(const void *q, const void *k, const void *v, const float *log_alpha,
                                     const float *beta, const float *S0, void *out, float *S_final, int B,
                                     int T, int H, int dk, int dv, int C, int nseg, void *workspace,
                                     size_t workspace_bytes, void *stream)
{
    return chunk_common(false, false, q, k, v, log_alpha, beta, S0, out, S_final, nullptr, B, T, 0, H, dk,
                        dv, C, stream, nseg, workspace, workspace_bytes);
}

kda_status_t kda_chunk_fwd_segmented_f32(const float *q, const float *k, const float *v,
                                         const float *log_alpha, const float *beta, const float *S0,
                                         float *out, float *S_final, int B, int T, int H, int dk, int dv,
                                         int C, int nseg, void *workspace, size_t workspace_bytes,
                                         void *stream)
{
    return chunk_common(true, false, q, k, v, log_alpha, beta, S0, out, S_final, nullptr, B, T, 0, H, dk,
                        dv, C, stream, nseg, workspace, workspace_bytes);
}

kda_status_t kda_chunk_fwd_varlen_segmented(const void *q, const void *k, const void *v,
                                            const float *log_alpha, const float *beta, const float *S0,
                                            void *out, float *S_final, const int32_t *cu_seqlens, int N,
                                            int T_total, int H, int dk, int dv, int C, int nseg,
                                            void *workspace, size_t workspace_bytes, void *stream)
{
    return chunk_common(false, true, q, k, v, log_alpha, beta, S0, out, S_final, cu_seqlens, N, 0, T_total,
                        H, dk, dv, C, stream, nseg, workspace, workspace_bytes);
}

kda_status_t kda_chunk_fwd_varlen_segmented_f32(const float *q, const float *k, const float *v,
                                                const float *log_alpha, const float *beta, const float *S0,
                                                float *out, float *S_final, const int32_t *cu_seqlens, int N,
                                                int T_total, int H, int dk, int dv, int C, int nseg,
                                                void *workspace, size_t workspace_bytes, void *stream)
{
    return chunk_common(true, true, q, k, v, log_alpha, beta, S0, out, S_final, cu_seqlens, N, 0, T_total,
                        H, dk, dv, C, stream, nseg, workspace, workspace_bytes);
}

kda_status_t kda_chunk_fwd_ex(const void *q, const void *k, const void *v, const float *log_alpha,
                              const float *beta, const float *S0, void *out, float *S_final, int B, int T, int H,
                              int dk, int dv, int C, int variant, int nseg, void *workspace,
                              size_t workspace_bytes, void *stream)
{
    return chunk_common(false, false, q, k, v, log_alpha, beta, S0, out, S_final, nullptr, B, T, 0, H, dk,
                        dv, C, stream, nseg, workspace, workspace_bytes, variant);
}

kda_status_t kda_chunk_fwd_ex_f32(const float *q, const float *k, const float *v, const float *log_alpha,
                                  const float *beta, const float *S0, float *out, float *S_final, int B, int T,
                                  int H, int dk, int dv, int C, int variant, int nseg, void *workspace,
                                  size_t workspace_bytes, void *stream)
{
    return chunk_common(true, false, q, k, v, log_alpha, beta, S0, out, S_final, nullptr, B, T, 0, H, dk,
                        dv, C, stream, nseg, workspace, workspace_bytes, variant);
}

kda_status_t kda_chunk_fwd_varlen_ex(const void *q, const void *k, const void *v, const float *log_alpha,
                                     const float *beta, const float *S0, void *out, float *S_final,
                                     const int32_t *cu_seqlens, int N, int T_total, int H, int dk, int dv, int C,
                                     int variant, int nseg, void *workspace, size_t workspace_bytes,
                                     void *stream)
{
    return chunk_common(false, true, q, k, v, log_alpha, beta, S0, out, S_final, cu_seqlens, N, 0, T_total,
                        H, dk, dv, C, stream, nseg, workspace, workspace_bytes, variant);
}

kda_status_t kda_chunk_fwd_varlen_ex_f32(const float *q, const float *k, const float *v,
                                         const float *log_alpha, const float *beta, const float *S0,
                                         float *out, float *S_final, const int32_t *cu_seqlens, int N,
                                         int T_total, int H, int dk, int dv, int C, int variant, int nseg,
                                         void *workspace, size_t workspace_bytes, void *stream)
{
    return chunk_common(true, true, q, k, v, log_alpha, beta, S0, out, S_final, cu_seqlens, N, 0, T_total,
                        H, dk, dv, C, stream, nseg, workspace, workspace_bytes, variant);
}

kda_status_t kda_recurrent_fwd_ex(const void *q, const void *k, const void *v, const float *log_alpha,
                                  const float *beta, float *S, void *out, int N, int T, int H, int dk, int dv,
                                  int variant, void *stream)
{
    return step_common(false, q, k, v, log_alpha, beta, S, out, N, H, dk, dv, stream, T, true, variant);
}

kda_status_t kda_recurrent_fwd_ex_f32(const float *q, const float *k, const float *v, const float *log_alpha,
                                      const float *beta, float *S, float *out, int N, int T, int H, int dk,
                                      int dv, int variant, void *stream)
{
    return step_common(true, q, k, v, log_alpha, beta, S, out, N, H, dk, dv, stream, T, true, variant);
}

size_t kda_chunk_segmented_workspace_bytes(int nseq, int H, int dk, int dv, int nseg)
{
    if (nseq <= 0 || H <= 0 || !supported_d(dk) || !supported_d(dv) || nseg < 1 || nseg > kMaxSegments) return 0;
    return (size_t)seg_workspace_bytes((uint64_t)nseq * (uint64_t)H, dk, dv, nseg);
}

int kda_chunk_auto_segments(int B, int T, int H, int dk, int dv, int C, int fp32_inputs)
{
    return auto_segments(fp32_inputs != 0, B, T, H, dk, dv, C);
}

int kda_chunk_auto_segments_ex(int B, int T, int H, int dk, int dv, int C, int fp32_inputs, int variant)
{
    return auto_segments(fp32_inputs != 0, B, T, H, dk, dv, C, (variant & kSchedMapOut) != 0);
}

int kda_chunk_auto_schedule(int B, int T, int H, int dk, int dv, int C, int fp32_inputs)
{
    int s2 = 1, s1 = 1;
    const double two = auto_cost(fp32_inputs != 0, B, T, H, dk, dv, C, false, s2);
    const double one = auto_cost(fp32_inputs != 0, B, T, H, dk, dv, C, true, s1);
    return (s1 > 1 && s2 > 1 && one < two) ? kSchedMapOut : 0;
}

size_t kda_chunk_segmented_workspace_bytes_ex(int nseq, int T_total, int H, int dk, int dv, int nseg, int variant,
                                              int fp32_inputs)
{
    const bool plan = (variant & kSchedMapOut) && nseg == 0;   // the device-side split of packed sequences
    if (plan) nseg = 2;
    if (nseq <= 0 || T_total < 0 || H <= 0 || !supported_d(dk) || !supported_d(dv) || nseg < 1 ||
        nseg > kMaxSegments || !valid_variant(variant & ~kSchedMapOut))
        return 0;
    const uint64_t nheads = (uint64_t)nseq * (uint64_t)H;
    if (variant & kSchedMapOut)
        return (size_t)(mout_workspace_bytes(nheads, (uint64_t)T_total * (uint64_t)H, dk, dv, nseg, fp32_inputs ? 4 : 2) +
                        (plan ? 4u * (uint64_t)nseq : 0u));
    return (size_t)seg_workspace_bytes(nheads, dk, dv, nseg);
}

kda_status_t kda_recurrent_step(const void *q, const void *k, const void *v, const float *log_alpha,
                                const float *beta, float *S, void *out, int N, int H, int dk, int dv,
                                void *stream)
{
    return step_common(false, q, k, v, log_alpha, beta, S, out, N, H, dk, dv, stream);
}

kda_status_t kda_recurrent_step_f32(const float *q, const float *k, const float *v, const float *log_alpha,
                                    const float *beta, float *S, float *out, int N, int H, int dk, int dv,
                                    void *stream)
{
    return step_common(true, q, k, v, log_alpha, beta, S, out, N, H, dk, dv, stream);
}

kda_status_t kda_recurrent_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                               const float *beta, float *S, void *out, int N, int T, int H, int dk, int dv,
                               void *stream)
{
    return step_common(false, q, k, v, log_alpha, beta, S, out, N, H, dk, dv, stream, T, true);
}

kda_status_t kda_recurrent_fwd_f32(const float *q, const float *k, const float *v, const float *log_alpha,
                                   const float *beta, float *S, float *out, int N, int T, int H, int dk, int dv,
                                   void *stream)
{
    return step_common(true, q, k, v, log_alpha, beta, S, out, N, H, dk, dv, stream, T, true);
}

kda_status_t kda_stream_copy(const void *src, void *dst, size_t bytes, void *stream)
{
    if (bytes == 0) return ok();
    if (!src || !dst) return fail(KDA_ERR_NULL_POINTER, "src and dst are required");
    if (bytes % 16) return fail(KDA_ERR_BAD_SHAPE, "bytes must be a multiple of 16 (got %zu)", bytes);
    if (!aligned(src, 16) || !aligned(dst, 16)) return fail(KDA_ERR_MISALIGNED, "src and dst must be 16-byte aligned");
    if (overlap(src, bytes, dst, bytes)) return fail(KDA_ERR_ALIASING, "src and dst overlap");
    const hipError_t e = kda::launch_stream_copy(src, dst, (long)(bytes / 16), (hipStream_t)stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "copy kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

kda_status_t kda_check_cu_seqlens_host(const int32_t *cu, int N, int T_total)
{
    if (N < 0 || T_total < 0) return fail(KDA_ERR_BAD_SHAPE, "negative N or T_total");
    if (!cu) return fail(KDA_ERR_NULL_POINTER, "cu_seqlens is NULL");
    if (cu[0] != 0) return fail(KDA_ERR_BAD_SHAPE, "cu_seqlens[0] = %d, expected 0", cu[0]);
    for (int n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n])
            return fail(KDA_ERR_BAD_SHAPE, "cu_seqlens decreases at %d (%d -> %d)", n, cu[n], cu[n + 1]);
    if (cu[N] != T_total)
        return fail(KDA_ERR_BAD_SHAPE, "cu_seqlens[N] = %d, expected T_total = %d", cu[N], T_total);
    return ok();
}

const char *kda_status_string(kda_status_t s)
{
    switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_NULL_POINTER: return "KDA_ERR_NULL_POINTER";
    case KDA_ERR_BAD_SHAPE: return "KDA_ERR_BAD_SHAPE";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_MISALIGNED: return "KDA_ERR_MISALIGNED";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
    case KDA_ERR_ALIASING: return "KDA_ERR_ALIASING";
    default: return "KDA_ERR_UNKNOWN";
    }
}

const char *kda_last_error(void) { return g_err; }

int kda_version(void) { return 100; }

}  // extern "C"
