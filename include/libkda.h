/*
 * libkda -- Kimi Delta Attention (KDA) forward pass on AMD Instinct MI355X
 * (gfx950), C ABI.
 *
 * THE OPERATION.  Per (sequence, head) the library runs the KDA recurrence with
 * an fp32 state S of d_v rows (value channels) by d_k columns (key channels):
 *
 *   S~_t = S_{t-1} Diag(alpha_t),  alpha_t = exp(log_alpha_t)  (per key channel)
 *   e_t  = beta_t (v_t - S~_t k_t)                              (prediction error)
 *   S_t  = S~_t + e_t k_t^T                                     (write)
 *   o_t  = S_t q_t                                              (readout)
 *
 * Sources: "KDA derivation summary" page (hn.213312.xyz article 49085909),
 * sect. 3 (predict / error / write, readout S_t|q_t>) and sect. 5 (per-column,
 * i.e. per-key-channel, decay D_t applied before the prediction); "Kimi K3
 * notes 1: KDA" page (jaimeyzzz.com), sect. 4 and the summary box of sect. 5
 * (the same update written for the transposed d_k x d_v state).  There is no
 * query scale and no normaliser; the readout uses the post-write state.
 *
 * Two schedules of this one recurrence (same page, sect. 6): the chunkwise
 * prefill (kda_chunk_fwd*) and the token-by-token decode step
 * (kda_recurrent_step*).  Both give the recurrence's result up to floating
 * point rounding.
 *
 * LAYOUTS (row-major, last index fastest; "token-major"):
 *   q, k, log_alpha : [B, T, H, dk]        v, out : [B, T, H, dv]
 *   beta            : [B, T, H]            S0, S_final, S : [B, H, dv, dk]
 * bf16 tensors are IEEE bfloat16 (the upper half of an IEEE float32);
 * log_alpha, beta and every state are fp32.  In the *_f32 entry points q, k,
 * v and out are fp32 as well.
 *
 * OWNERSHIP AND EXECUTION.  Every pointer is device memory owned by the
 * caller (the segmented entry points take their scratch space as a
 * caller-owned workspace).  The library allocates nothing and is thread-safe;
 * its only global state is a per-thread message for kda_last_error(), a
 * per-device cache of the compute-unit count, and the fixed scratch array of
 * kda_chunk_fwd_segmented_noalloc (with its per-device address).  Work is
 * enqueued asynchronously on `stream` (a hipStream_t passed as void*; NULL is
 * the default stream).  KDA_OK means "validated and
 * enqueued"; faults inside a kernel surface at the caller's next
 * synchronisation of that stream.
 *
 * ERRORS.  Status codes only; the library never aborts and throws nothing
 * across the ABI.  All argument checks run before any HIP call, so an invalid
 * call has no side effect.  kda_last_error() gives a message for the calling
 * thread's last failed call.
 *
 * SUPPORTED SHAPES.  dk, dv in {16, 32, 64, 128}; C in {16, 32, 64}.  C is the
 * chunk length of the schedule and does not change the result beyond
 * rounding; the fp32 entry points at dk = 128 run C = 64 as 32-token chunks
 * (64-token fp32 operands of 128 channels do not fit a workgroup's 160 KiB of
 * LDS).
 * B, T, H, N >= 0 (a batch with no tokens only writes S_final).  Pointers to
 * q, k, v, out, log_alpha, S0, S_final and S must be 16-byte aligned; beta
 * 4-byte aligned.
 *
 * VALUE PRECONDITIONS (documented, not checked): log_alpha finite and <= 0;
 * beta in [0, 1]; q and k L2-normalised by the caller ("Kimi K3 notes 1"
 * page, sect. 4: q, k pass a feature map and an L2 normalisation first).
 * There is no lower bound on log_alpha: a key channel may decay by any
 * amount, down to a complete clear (log_alpha = -1e4 gives alpha = 0 in
 * fp32), in every schedule; the per-channel gate exists to keep some channels
 * while clearing others ("KDA derivation summary" page, sect. 5).
 */
#ifndef LIBKDA_H
#define LIBKDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL_POINTER = 1,  /* a required pointer is NULL */
    KDA_ERR_BAD_SHAPE = 2,     /* negative size, H < 1, inconsistent sizes */
    KDA_ERR_UNSUPPORTED = 3,   /* dk, dv or C outside the supported set */
    KDA_ERR_MISALIGNED = 4,    /* pointer alignment below what the loads need */
    KDA_ERR_HIP = 5,           /* the HIP runtime refused the launch */
    KDA_ERR_ALIASING = 6       /* out overlaps an input, or S_final partially overlaps S0 */
} kda_status_t;

/*
 * Chunkwise prefill, bf16 inputs ("KDA derivation summary" page, sect. 6,
 * chunk mode; the chunk skeleton of the "Linear/sparse attention tutorial"
 * page, sect. 6.2).  Inside each chunk of C tokens the kernel forms the
 * cumulative log-decay, the strictly lower-triangular K K^T system whose
 * solution corrects each token's provisional error, the causal Q K^T block,
 * and hands the fp32 state to the next chunk.
 *
 *   q, k     bf16 [B,T,H,dk]  (L2-normalised rows)
 *   v        bf16 [B,T,H,dv]
 *   log_alpha fp32 [B,T,H,dk], natural log of the per-channel decay (<= 0)
 *   beta     fp32 [B,T,H]
 *   S0       fp32 [B,H,dv,dk] incoming state; NULL = zero state
 *   out      bf16 [B,T,H,dv]  o_t (round-to-nearest-even from fp32)
 *   S_final  fp32 [B,H,dv,dk] state after token T-1; NULL = not written.
 *            May be the same pointer as S0 (in-place continuation).
 *   C        chunk length; T need not be a multiple of C.
 * Each workgroup takes one (sequence, head) and a block of value rows, the
 * widest of 64, 32 or 16 that fits; the environment variable KDA_CHUNK_BV
 * (16, 32 or 64) overrides that schedule choice, as it does for every chunk
 * entry point.
 */
kda_status_t kda_chunk_fwd(const void *q, const void *k, const void *v,
                           const float *log_alpha, const float *beta,
                           const float *S0, void *out, float *S_final,
                           int B, int T, int H, int dk, int dv, int C,
                           void *stream);

/* Same as kda_chunk_fwd with fp32 q, k, v and out (all arithmetic in fp32). */
kda_status_t kda_chunk_fwd_f32(const float *q, const float *k, const float *v,
                               const float *log_alpha, const float *beta,
                               const float *S0, float *out, float *S_final,
                               int B, int T, int H, int dk, int dv, int C,
                               void *stream);

/*
 * Chunkwise prefill over N sequences packed along the token axis of one
 * [1, T_total, H, d] stream.  Sequence n owns tokens
 * [cu_seqlens[n], cu_seqlens[n+1]); its chunk grid starts at its first token
 * and its partial last chunk is padded with identity tokens (k = 0, beta = 0,
 * log_alpha = 0, which leave the state unchanged).  S0 / S_final are
 * [N, H, dv, dk].  cu_seqlens is DEVICE memory, int32 [N+1]; precondition
 * (not checked on the device): cu_seqlens[0] = 0, non-decreasing,
 * cu_seqlens[N] = T_total.  kda_check_cu_seqlens_host() checks a host copy.
 * The kernel clamps each sequence's [start, end) to [0, T_total] with
 * end >= start, so offsets that break the precondition give unspecified
 * outputs and states but never touch memory outside the buffers.
 */
kda_status_t kda_chunk_fwd_varlen(const void *q, const void *k, const void *v,
                                  const float *log_alpha, const float *beta,
                                  const float *S0, void *out, float *S_final,
                                  const int32_t *cu_seqlens, int N, int T_total,
                                  int H, int dk, int dv, int C, void *stream);

/* fp32 q, k, v, out variant of kda_chunk_fwd_varlen. */
kda_status_t kda_chunk_fwd_varlen_f32(const float *q, const float *k, const float *v,
                                      const float *log_alpha, const float *beta,
                                      const float *S0, float *out, float *S_final,
                                      const int32_t *cu_seqlens, int N, int T_total,
                                      int H, int dk, int dv, int C, void *stream);

/*
 * Segment-parallel chunkwise prefill, for long sequences with few (sequence,
 * head) pairs.  Same operation, layouts and results (up to rounding) as
 * kda_chunk_fwd / kda_chunk_fwd_varlen; only the schedule differs.  The chunk
 * mode of the "KDA derivation summary" page (sect. 6) hands the state from
 * chunk to chunk, and every quantity a chunk forms from it is affine in the
 * incoming state; so is a run of chunks: S_end = S_start M + N, with M
 * (dk x dk) and N (dv x dk) independent of S_start (derived from the chunk
 * equations, not stated on the pages).  The chunks of every sequence are cut
 * into nseg consecutive segments, and three passes run on `stream`:
 *   1. segment 0 runs its whole pass from S0 (writing its outputs and segment
 *      1's incoming state) while segments 1 .. nseg-2, in parallel, run from
 *      S_start = 0 with dk extra state rows that start at the identity and
 *      see v = 0: the real rows end at N, the extra rows at M;
 *   2. the later segments' incoming states are composed in order, in fp32;
 *   3. segments 1 .. nseg-1, in parallel, run from their incoming states,
 *      writing out and (last segment) S_final.
 * Segment 0 is longer than the others, so that its pass takes about as long
 * as the maps beside it; segments may be empty for short sequences.  The
 * environment variable KDA_SEG_LEAD (a length ratio in tenths; 0 = equal
 * segments, segment 0 mapped like the others) overrides the split.
 * nseg = 1 is the plain single pass (workspace may be NULL).
 *
 *   nseg       1 .. 1024; kda_chunk_auto_segments() picks one for a dense batch.
 *   workspace  device memory owned by the caller, 256-byte aligned, at least
 *              kda_chunk_segmented_workspace_bytes(...) bytes, disjoint from
 *              every other argument; its contents on entry do not matter and
 *              are undefined on exit.  Calls that share a workspace must not
 *              overlap in time.
 * Other arguments as in kda_chunk_fwd (dense) / kda_chunk_fwd_varlen.
 * S_final may be the same pointer as S0 here too.
 */
kda_status_t kda_chunk_fwd_segmented(const void *q, const void *k, const void *v,
                                     const float *log_alpha, const float *beta,
                                     const float *S0, void *out, float *S_final,
                                     int B, int T, int H, int dk, int dv, int C,
                                     int nseg, void *workspace, size_t workspace_bytes,
                                     void *stream);

/* fp32 q, k, v, out variant of kda_chunk_fwd_segmented. */
kda_status_t kda_chunk_fwd_segmented_f32(const float *q, const float *k, const float *v,
                                         const float *log_alpha, const float *beta,
                                         const float *S0, float *out, float *S_final,
                                         int B, int T, int H, int dk, int dv, int C,
                                         int nseg, void *workspace, size_t workspace_bytes,
                                         void *stream);

/*
 * kda_chunk_fwd_segmented without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, serving loops
 * and harnesses that forbid hipMalloc.  The scratch space is a fixed device
 * array inside the library of KDA_NOALLOC_SCRATCH_BYTES (64 MiB), one copy per
 * GPU, held from the library's load until the process ends; this call
 * allocates nothing (no hipMalloc, no hipFree, no allocating library call).
 *
 *   - A request whose workspace (kda_chunk_segmented_workspace_bytes) exceeds
 *     KDA_NOALLOC_SCRATCH_BYTES is rejected with KDA_ERR_UNSUPPORTED before
 *     any HIP call.  At d = 128 one segment of one (sequence, head) needs
 *     192 KiB (B=1, H=16 takes up to 22 segments).
 *   - Every call on one GPU uses that GPU's one array.  Calls that overlap in
 *     time on the same GPU (two streams, two threads) race and give undefined
 *     results; calls on one stream are ordered and safe.  Nothing needs
 *     clearing between calls: every scratch byte a call reads, the same call
 *     wrote first.
 *   - The first call on a device looks up the array's device address there
 *     (hipGetSymbolAddress, after the argument checks); a failed lookup is
 *     KDA_ERR_HIP.
 * Operation, layouts, other arguments and results (bit for bit) as in
 * kda_chunk_fwd_segmented with the same nseg.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (64ull << 20)
kda_status_t kda_chunk_fwd_segmented_noalloc(const void *q, const void *k, const void *v,
                                             const float *log_alpha, const float *beta,
                                             const float *S0, void *out, float *S_final,
                                             int B, int T, int H, int dk, int dv, int C,
                                             int nseg, void *stream);

/* Packed-sequence variants: every sequence is cut into nseg segments. */
kda_status_t kda_chunk_fwd_varlen_segmented(const void *q, const void *k, const void *v,
                                            const float *log_alpha, const float *beta,
                                            const float *S0, void *out, float *S_final,
                                            const int32_t *cu_seqlens, int N, int T_total,
                                            int H, int dk, int dv, int C, int nseg,
                                            void *workspace, size_t workspace_bytes,
                                            void *stream);
kda_status_t kda_chunk_fwd_varlen_segmented_f32(const float *q, const float *k, const float *v,
                                                const float *log_alpha, const float *beta,
                                                const float *S0, float *out, float *S_final,
                                                const int32_t *cu_seqlens, int N, int T_total,
                                                int H, int dk, int dv, int C, int nseg,
                                                void *workspace, size_t workspace_bytes,
                                                void *stream);

/*
 * VARIANTS.  The pages place KDA in a family that differs only in how the
 * state forgets and how it writes ("Kimi K3 notes 1: KDA" page, the boxed
 * summary of sect. 5: linear attention, DeltaNet, Gated DeltaNet, KDA;
 * "Linear/sparse attention tutorial" page, sect. 2.4: RetNet's scalar decay
 * and GLA's per-channel gate on an additive write).  The *_ex entry points
 * run any member with the same kernels:
 *   gate   KDA_GATE_CHANNEL  log_alpha [.., H, dk], one decay per key channel
 *                            (KDA, GLA)
 *          KDA_GATE_SCALAR   log_alpha [.., H], one decay per token and head
 *                            for all key channels (Gated DeltaNet, RetNet-like);
 *                            4-byte alignment suffices
 *          KDA_GATE_NONE     alpha = 1; log_alpha is not read and may be NULL
 *                            (DeltaNet, linear attention)
 *   write  KDA_WRITE_DELTA   e_t = beta_t (v_t - S~_t k_t)   (the delta rule)
 *          KDA_WRITE_ADD     e_t = beta_t v_t, S_t = S~_t + beta_t v_t k_t^T
 *                            (linear attention, GLA; beta = 1 gives them exactly)
 *   input  KDA_INPUT_RAW     fused input preparation: q and k arrive as they
 *                            come out of their projections and are L2-normalised
 *                            per token inside the kernels (a zero row stays
 *                            zero; "Kimi K3 notes 1: KDA" page, sect. 4), and
 *                            the gate argument holds pre-activations g in the
 *                            input type (bf16 in the bf16 entry points, fp32 in
 *                            the _f32 ones) with log_alpha = -softplus(g).  For
 *                            bf16 this halves the gate's HBM bytes and removes
 *                            the separate normalisation and softplus passes.
 * variant = gate | write | input; anything else is KDA_ERR_BAD_SHAPE.  The
 * plain entry points are variant 0 (KDA_GATE_CHANNEL | KDA_WRITE_DELTA).
 *
 * SCHEDULE (chunk *_ex entry points only; the decode ones reject it).
 *   KDA_SCHED_MAP_OUTPUTS  with nseg > 1: the segmented schedule without a
 *   second pass.  Every output is affine in the incoming state too: with the
 *   extra state rows of a map started at the identity, o_t = o0_t + S_p m_t,
 *   where o0_t is the real rows' output from S_start = 0 and m_t (dk values)
 *   the extra rows' own output (their readout S_t q_t).  So the map launch
 *   maps every segment after the first and also writes o0 into out and m into
 *   the workspace, beside segment 0's whole pass; the composition carries the
 *   incoming states on through S_final; and an epilogue adds S_p m_t to every
 *   output of segment p.  The state in the epilogue's products is rounded to
 *   bf16 in the bf16 entry points (as in the chunk kernel's own products with
 *   it), and a bf16 output is rounded twice (o0, then the sum).  The
 *   workspace also holds m, T_total * H * dk values of the input type:
 *   kda_chunk_segmented_workspace_bytes_ex() gives its size.  Same results as
 *   the two-pass schedule up to rounding.  With packed sequences, nseg = 0
 *   asks for two segments per sequence split on the device from cu_seqlens:
 *   the makespan target (in chunks) is the longer of the second-longest
 *   sequence and the balanced share (workgroups per head) H sum(chunks) /
 *   compute units, and only a sequence longer than the target by more than an
 *   eighth is split, its first `target` chunks as segment 0 and the rest as
 *   its mapped segment 1, which runs on the compute units that shorter
 *   sequences free.  (One long sequence among shorter ones then no longer
 *   sets the time alone.)  The plan is made once per call by one workgroup
 *   and kept in the workspace: that of nseg = 2 plus 4 * N bytes.
 */
enum {
    KDA_GATE_CHANNEL = 0,
    KDA_GATE_SCALAR = 1,
    KDA_GATE_NONE = 2,
    KDA_WRITE_DELTA = 0,
    KDA_WRITE_ADD = 4,
    KDA_INPUT_RAW = 8,
    KDA_SCHED_MAP_OUTPUTS = 16
};

/* Chunk prefill with a variant and an optional segment-parallel schedule
 * (nseg, workspace as in kda_chunk_fwd_segmented, or with
 * KDA_SCHED_MAP_OUTPUTS in variant the schedule without a second pass and its
 * larger workspace; nseg = 1 needs no workspace).  Dense and packed layouts,
 * bf16 and fp32 inputs. */
kda_status_t kda_chunk_fwd_ex(const void *q, const void *k, const void *v,
                              const float *log_alpha, const float *beta,
                              const float *S0, void *out, float *S_final,
                              int B, int T, int H, int dk, int dv, int C,
                              int variant, int nseg, void *workspace, size_t workspace_bytes,
                              void *stream);
kda_status_t kda_chunk_fwd_ex_f32(const float *q, const float *k, const float *v,
                                  const float *log_alpha, const float *beta,
                                  const float *S0, float *out, float *S_final,
                                  int B, int T, int H, int dk, int dv, int C,
                                  int variant, int nseg, void *workspace, size_t workspace_bytes,
                                  void *stream);
kda_status_t kda_chunk_fwd_varlen_ex(const void *q, const void *k, const void *v,
                                     const float *log_alpha, const float *beta,
                                     const float *S0, void *out, float *S_final,
                                     const int32_t *cu_seqlens, int N, int T_total,
                                     int H, int dk, int dv, int C,
                                     int variant, int nseg, void *workspace, size_t workspace_bytes,
                                     void *stream);
kda_status_t kda_chunk_fwd_varlen_ex_f32(const float *q, const float *k, const float *v,
                                         const float *log_alpha, const float *beta,
                                         const float *S0, float *out, float *S_final,
                                         const int32_t *cu_seqlens, int N, int T_total,
                                         int H, int dk, int dv, int C,
                                         int variant, int nseg, void *workspace, size_t workspace_bytes,
                                         void *stream);

/*
 * Workspace bytes of the segmented entry points for nseq sequences (B or N)
 * of H heads: 4 * nseq * H * ((nseg - 1) (dv + dk) dk + nseg dv dk), the
 * first part rounded up to 256 bytes.  0 for nseg = 1 or invalid sizes.
 */
size_t kda_chunk_segmented_workspace_bytes(int nseq, int H, int dk, int dv, int nseg);

/*
 * Workspace bytes of the *_ex chunk entry points for nseq sequences of
 * T_total tokens in all (B * T for the dense layout) and H heads, for the
 * schedule `variant` selects (fp32_inputs: 1 for the _f32 entry points).
 * Without KDA_SCHED_MAP_OUTPUTS, kda_chunk_segmented_workspace_bytes(); with
 * it: 4 * nseq * H * nseg * (dv + dk) dk rounded up to 256, plus
 * 4 * nseq * H * nseg * dv * dk rounded up to 256, plus T_total * H * dk
 * values of the input type; nseg = 0 with KDA_SCHED_MAP_OUTPUTS (packed
 * sequences split on the device) is nseg = 2 plus 4 * nseq bytes for the plan.
 * 0 for nseg = 1 or invalid arguments.
 */
size_t kda_chunk_segmented_workspace_bytes_ex(int nseq, int T_total, int H, int dk, int dv, int nseg,
                                              int variant, int fp32_inputs);

/*
 * Segment count for a dense batch (fp32_inputs: 0 for the bf16 entry points,
 * 1 for the fp32 ones), from a model of the run time: 1 when the plain pass
 * already fills the GPU, more when few (sequence, head) pairs walk many
 * chunks.  Queries the current device's compute-unit count (256 assumed if
 * that fails); never fails, returns at least 1.
 */
int kda_chunk_auto_segments(int B, int T, int H, int dk, int dv, int C, int fp32_inputs);

/*
 * kda_chunk_auto_segments for the schedule `variant` selects: with
 * KDA_SCHED_MAP_OUTPUTS the run-time model of the schedule without a second
 * pass (its map chunks costing about a full chunk, plus the epilogue's
 * streaming of m and out), else kda_chunk_auto_segments().
 */
int kda_chunk_auto_segments_ex(int B, int T, int H, int dk, int dv, int C, int fp32_inputs, int variant);

/*
 * The schedule the two run-time models above favour for a dense batch:
 * KDA_SCHED_MAP_OUTPUTS when both pick more than one segment and the one
 * without a second pass comes out cheaper, else 0 (the two-pass schedule, or
 * the single pass when kda_chunk_auto_segments() returns 1).
 */
int kda_chunk_auto_schedule(int B, int T, int H, int dk, int dv, int C, int fp32_inputs);

/*
 * One decode step ("KDA derivation summary" page, sect. 6, fused recurrent
 * mode; "Linear/sparse attention tutorial" page, sect. 8.1: a step reads and
 * writes only the fixed-size state).  Advances N sequences by one token each:
 *
 *   q, k      bf16 [N,H,dk];  v, out bf16 [N,H,dv]
 *   log_alpha fp32 [N,H,dk];  beta fp32 [N,H]
 *   S         fp32 [N,H,dv,dk], updated IN PLACE from S_{t-1} to S_t.
 *
 * Each state row is read once and written once.
 */
kda_status_t kda_recurrent_step(const void *q, const void *k, const void *v,
                                const float *log_alpha, const float *beta,
                                float *S, void *out,
                                int N, int H, int dk, int dv, void *stream);

/* fp32 q, k, v, out variant of kda_recurrent_step. */
kda_status_t kda_recurrent_step_f32(const float *q, const float *k, const float *v,
                                    const float *log_alpha, const float *beta,
                                    float *S, float *out,
                                    int N, int H, int dk, int dv, void *stream);

/*
 * T decode tokens per sequence in one launch: the fused recurrent mode of the
 * "KDA derivation summary" page (sect. 6), whose kernel gives each program a
 * sequence, a value head and a value block and loops the update over the
 * tokens.  The state is read once, advanced through the T tokens in order
 * and written once, so a launch moves 8 dv dk bytes of state per head
 * however large T is (short prompts, speculative-decoding verification).
 *
 *   q, k      bf16 [N,T,H,dk];  v, out bf16 [N,T,H,dv]
 *   log_alpha fp32 [N,T,H,dk];  beta fp32 [N,T,H]
 *   S         fp32 [N,H,dv,dk], updated IN PLACE from S_{t-1} to S_{t+T-1}.
 *
 * T = 0 is a no-op.  T = 1 gives exactly kda_recurrent_step's result, and
 * any T the same bits as T single steps.  The per-token work is serial inside
 * a workgroup: from about T = 16 on, the chunk schedule on the same tensors
 * (kda_chunk_fwd with B = N, S0 = S_final = S, C = 16 below T = 32, else 32)
 * is faster.  Measured at N = 256, H = 32, d = 128: T = 8 0.24 ms here against
 * 0.26; T = 16 0.38 against 0.27; T = 64 1.25 against 0.45.
 */
kda_status_t kda_recurrent_fwd(const void *q, const void *k, const void *v,
                               const float *log_alpha, const float *beta,
                               float *S, void *out,
                               int N, int T, int H, int dk, int dv, void *stream);

/* fp32 q, k, v, out variant of kda_recurrent_fwd. */
kda_status_t kda_recurrent_fwd_f32(const float *q, const float *k, const float *v,
                                   const float *log_alpha, const float *beta,
                                   float *S, float *out,
                                   int N, int T, int H, int dk, int dv, void *stream);

/* kda_recurrent_fwd with a variant (see VARIANTS above). */
kda_status_t kda_recurrent_fwd_ex(const void *q, const void *k, const void *v,
                                  const float *log_alpha, const float *beta,
                                  float *S, void *out,
                                  int N, int T, int H, int dk, int dv, int variant, void *stream);
kda_status_t kda_recurrent_fwd_ex_f32(const float *q, const float *k, const float *v,
                                      const float *log_alpha, const float *beta,
                                      float *S, float *out,
                                      int N, int T, int H, int dk, int dv, int variant, void *stream);

/*
 * Bandwidth reference, not part of the attention computation: copies `bytes`
 * from src to dst (device memory, 16-byte aligned, bytes a multiple of 16,
 * non-overlapping) with 16-byte nontemporal loads and stores, the access
 * pattern the decode kernels stream the state with.  Timing it gives the
 * achievable HBM bandwidth that the streaming kernels are compared against.
 * bytes = 0 is a no-op.  Errors: KDA_ERR_NULL_POINTER, KDA_ERR_BAD_SHAPE
 * (bytes not a multiple of 16), KDA_ERR_MISALIGNED, KDA_ERR_ALIASING,
 * KDA_ERR_HIP.
 */
kda_status_t kda_stream_copy(const void *src, void *dst, size_t bytes, void *stream);

/*
 * Host-side check of a cu_seqlens array held in HOST memory: N >= 0,
 * cu[0] = 0, non-decreasing, cu[N] = T_total.  Returns KDA_OK or
 * KDA_ERR_BAD_SHAPE / KDA_ERR_NULL_POINTER.
 */
kda_status_t kda_check_cu_seqlens_host(const int32_t *cu_seqlens_host, int N, int T_total);

/* Static name of a status code. */
const char *kda_status_string(kda_status_t status);

/* Message describing the calling thread's last failed call ("" if none). */
const char *kda_last_error(void);

/* Library version as major * 10000 + minor * 100 + patch. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBKDA_H */
