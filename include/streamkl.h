/*
 * streamkl.h -- C ABI of the fused attention KL-divergence primitive for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (StreamKL, arXiv 2606.20005; abstract on paperdance.org and
 * fugumt.com): for every (batch b, head h, query row i)
 *
 *     s_t,ij = scale * <Q_t[b,h,i,:], K_t[b,h,j,:]>          t = 1 teacher, 2 student
 *     P_t,ij = exp(s_t,ij) / sum_{k visible} exp(s_t,ik)
 *     KL_i   = sum_{j visible} P1_ij * log(P1_ij / P2_ij)    = KL(P1 || P2), row i
 *     LSE_t,i = log sum_{j visible} exp(s_t,ij)              (natural log)
 *
 * Key j is visible to row i iff j < NK and, when `causal` is set,
 * j <= i + NK - NQ (bottom-right aligned mask; for NQ == NK this is j <= i).
 * Neither N_Q x N_K probability matrix is ever stored: the forward streams
 * key tiles through on-chip memory keeping five running scalars per row
 * (gist.science, "Formulacion Online"), and the backward recomputes the
 * probabilities tile by tile from the saved LSE vectors (gist.science,
 * "Estrategia de Recomputacion").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates no device memory.  Its only global state belongs to
 *    streamkl_fwd_splitk_noalloc: a device scratch array per GPU and the
 *    table of their addresses, filled once per device under a lock.
 *  - Q1, Q2 are [B, H, NQ, D] and K1, K2 are [B, H, NK, D], contiguous,
 *    row-major, element type `dtype` (bf16, fp32 or fp8 e4m3).  Per-row
 *    vectors (KL,
 *    LSE1, LSE2, g) are fp32 [B, H, NQ].  Gradients are fp32 and have the
 *    shape of the tensor they belong to.
 *  - Every pointer must be 16-byte aligned.  D must be 64 or 128.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    and the call returns without waiting for it.
 *  - Argument errors are detected on the host before anything is enqueued;
 *    then nothing is written.  A failed kernel launch returns
 *    STREAMKL_ERR_HIP.  No call throws.
 *  - Calls that share no output buffer may run concurrently on different
 *    streams.
 */
#ifndef STREAMKL_H
#define STREAMKL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    STREAMKL_OK = 0,
    STREAMKL_ERR_NULL = 1,      /* a required pointer is NULL */
    STREAMKL_ERR_SHAPE = 2,     /* bad sizes: negative, D not 64/128, NK == 0 with rows,
                                   causal with NQ > NK, a per-head fp32 tensor of
                                   ceil(N / 64) * 64 rows of D reaching 2^31 bytes,
                                   B * H reaching 2^31, a kernel grid past the GPU's
                                   2^32 - 1 work-items, split count out of range */
    STREAMKL_ERR_DTYPE = 3,     /* dtype is not a streamkl_dtype */
    STREAMKL_ERR_ALIGN = 4,     /* a pointer is not 16-byte aligned */
    STREAMKL_ERR_WORKSPACE = 5, /* workspace missing or smaller than the size query */
    STREAMKL_ERR_HIP = 6        /* the HIP runtime rejected a launch */
} streamkl_status;

/*
 * STREAMKL_FP8_E4M3: the OCP 8-bit float with 4 exponent bits (bias 7), 3
 * significand bits, no infinities and NaN as S.1111.111 (torch.float8_e4m3fn).
 * Every entry point takes it.  The logits products, in the forward and in
 * both backward passes, run on the fp8 matrix instructions (exact products,
 * fp32 accumulation); the backward's gradient products take the inputs as
 * fp16 operands, which hold every e4m3 value exactly (no operand scale, so
 * the prepare step only forms sigma), against the same sigma-scaled fp16 dS
 * as for bf16.  This is the mixed-precision direction the pages leave as
 * future work (arxivlens.com paper view of StreamKL, future-work list).
 * Rounding bf16 tensors to e4m3 changes the distributions themselves far more
 * than the 2e-3 the kernels hold to; the type is for inputs that are fp8
 * already.  At most 128 queries per head take the fused single-visit
 * backward as for bf16 (the keys' one-hot transposition on the fp8
 * instruction, bf16 hi/lo dS).
 */
typedef enum { STREAMKL_BF16 = 0, STREAMKL_FP32 = 1, STREAMKL_FP8_E4M3 = 2 } streamkl_dtype;

typedef struct {
    int64_t B, H;   /* batch, heads */
    int64_t NQ;     /* query rows per head */
    int64_t NK;     /* key rows per head */
    int64_t D;      /* head dimension: 64 or 128 */
    float scale;    /* logit scale (1/sqrt(D) for plain attention; 1/(tau*sqrt(D))
                       folds a distillation temperature tau into both distributions) */
    int32_t causal; /* nonzero: bottom-right aligned causal mask */
    int32_t dtype;  /* streamkl_dtype of Q1, K1, Q2, K2 */
} streamkl_problem;

/*
 * Forward: one online pass over the key tiles (gist.science, "Formulacion
 * Online"; arXiv abstract, "single one-pass forward kernel").  Writes per row
 * KL(P1||P2), LSE1 and LSE2 -- the only state the backward needs
 * (gist.science, "Estrategia de Recomputacion", saved state).
 * Extra device memory: none.
 */
streamkl_status streamkl_fwd(const streamkl_problem *p,
                             const void *q1, const void *k1,
                             const void *q2, const void *k2,
                             float *kl, float *lse1, float *lse2,
                             void *stream);

/*
 * Bytes of device workspace streamkl_fwd_splitk needs for `num_splits`
 * chunks: 5 fp32 partial row states (m1, l1, m2, l2, acc) per split per row.
 * Returns 0 if the problem or split count is invalid.
 */
size_t streamkl_fwd_splitk_workspace_size(const streamkl_problem *p, int num_splits);

/*
 * Split-K forward for short-query, long-key shapes (gist.science,
 * "Optimizaciones de Kernel de GPU", Split-K variant): the key range is cut
 * into `num_splits` contiguous chunks processed by separate workgroups, each
 * producing a partial row state; a second kernel merges the states with
 * log-sum-exp rescaling and writes KL, LSE1, LSE2 exactly as streamkl_fwd
 * does.  1 <= num_splits <= ceil(NK / 64).  Chunks are whole 128-key tiles
 * of ceil(ceil(NK / 128) / num_splits) tiles each, so past ceil(NK / 128)
 * splits the trailing chunks are empty (correct, but idle workgroups).
 * `workspace` (device, caller-owned, >= the size query) is scratch between
 * the two kernels; its contents on return are unspecified.
 */
streamkl_status streamkl_fwd_splitk(const streamkl_problem *p,
                                    const void *q1, const void *k1,
                                    const void *q2, const void *k2,
                                    float *kl, float *lse1, float *lse2,
                                    int num_splits, void *workspace, size_t workspace_bytes,
                                    void *stream);

/*
 * For callers that cannot allocate device memory or hand the library a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  The same split-K forward as streamkl_fwd_splitk
 * (same arguments without the workspace, same results bit for bit, same
 * errors), with the partial row states in a device array the library owns:
 * STREAMKL_NOALLOC_SCRATCH_BYTES (64 MiB) on every GPU it runs on, set up by
 * the first call on that GPU (run one call outside graph capture first) and
 * held until the process ends.  A problem whose split-K workspace
 * (streamkl_fwd_splitk_workspace_size) exceeds the array is rejected with
 * STREAMKL_ERR_WORKSPACE before anything is enqueued; num_splits == 1 runs
 * streamkl_fwd and uses no scratch.  The call allocates nothing.  Every call
 * on one GPU shares that GPU's array and leaves its last contents there, so
 * calls that may overlap on one GPU (other streams, other host threads) race:
 * the caller serialises them.  A failed set-up returns STREAMKL_ERR_HIP.
 */
#define STREAMKL_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
streamkl_status streamkl_fwd_splitk_noalloc(const streamkl_problem *p,
                                            const void *q1, const void *k1,
                                            const void *q2, const void *k2,
                                            float *kl, float *lse1, float *lse2,
                                            int num_splits, void *stream);

/*
 * Bytes of device workspace streamkl_bwd needs.  It holds, per (batch, head),
 * the fp32 factor sigma by which dS is scaled before rounding, four fp32
 * powers of two by which the fp16 gradient-product operands of q1, q2, k1
 * and k2 are scaled, and (bf16 inputs) 64 fp32 partial maxima from which
 * those come: O(B * H), a few KiB at 32 heads.  With bf16 or fp8 inputs and
 * fewer than 256 query tiles of 128 rows in all (B * H * ceil(NQ / 128) < 256), the
 * query-gradient pass splits the keys into S chunks, S = min(ceil(256 /
 * tiles), 64, ceil(NK / 64)) (then as many chunks as whole 64-key tiles fill),
 * and the workspace also holds S partial dQ1, dQ2 in fp32 (S * 2 * B * H * NQ
 * * D * 4 bytes), summed in chunk order.  Returns 0 if the problem is invalid.
 */
size_t streamkl_bwd_workspace_size(const streamkl_problem *p);
/* (For bf16 problems of at most 128 queries the size query also covers the
 * fused pass's dQ partials, C * 2 * B * H * NQ * D * 4 bytes for C key chunks,
 * C = min(ceil(W / (B * H)), 64, ceil(NK / 32)) with W = 2048 for at most 32
 * queries and 512 above, when that is larger.) */

/*
 * Smallest workspace streamkl_bwd accepts: the per-(batch, head) factors
 * without the split partial dQ.  Given less than streamkl_bwd_workspace_size
 * (but at least this), the two passes run and the query-gradient pass runs
 * unsplit: dQ differs only in the fp32 summation order (and, where the fused
 * pass would have run, in rounding within the bounds), and short query
 * ranges run slower.  Returns 0 if the problem is invalid.
 */
size_t streamkl_bwd_workspace_size_min(const streamkl_problem *p);

/*
 * Backward of L = sum_{b,h,i} g[b,h,i] * KL[b,h,i] (gist.science, "Estrategia
 * de Recomputacion"): probabilities are recomputed tile by tile as
 * P_t = exp(s_t - LSE_t) from Q, K and the saved LSE vectors, and
 *     dS2 = g * (P2 - P1)                                   ("Configuracion 1")
 *     dS1 = g * P1 * ((s1 - LSE1) - (s2 - LSE2) - KL_row)   ("Configuracion 2"),
 * the log-ratio taken from logits and the saved LSEs ("Estabilidad Numerica").
 * Then dQ_t = scale * dS_t K_t and dK_t = scale * dS_t^T Q_t, with no atomics;
 * results are bitwise repeatable.  bf16 problems of at most 128 queries per
 * (batch, head) run one fused single-visit pass ("Fusion de Kernel"): the
 * queries stay resident, each key is read once, dS is formed once per pair
 * and feeds both products, dK is written directly and dQ as one partial per
 * key chunk, summed in chunk order.  Its products are bf16 with dS split
 * into a high and a low bf16 part (no operand scaling, no prepare step).
 * All other problems run two passes (one over key tiles for dK, one over
 * query tiles for dQ), as do the step-wise entry points below.
 *
 * kl, lse1, lse2 must be the outputs of streamkl_fwd / streamkl_fwd_splitk for
 * the same inputs.  Gradient outputs come in pairs: pass dq1 = dk1 = NULL to
 * skip the teacher gradients (teacher fixed) or dq2 = dk2 = NULL to skip the
 * student's; a half-NULL pair is STREAMKL_ERR_NULL.  Outputs are overwritten.
 * With bf16 (or fp8) inputs the two gradient products run on fp16 matrix
 * cores with fp32 accumulation (dS in bf16 would exceed a 2e-3 relative
 * error).  With bf16 inputs the streamed Q or K operand is scaled per
 * (batch, head, tensor) by a power of two that puts its largest entry in
 * [2^14, 2^15), so any finite bf16 input fits fp16 (entries below 2^-29 of
 * the tensor's largest lose precision, a contribution below 2^-29 of the
 * largest).  The fp16 dS operands are scaled
 * so that the largest |g| maps to [2^7, 2^8), so P1 * |log(P1/P2) - KL| must
 * stay below about 255 at every pair; it exceeds that only where the teacher
 * gives a key real mass and the student a log-probability hundreds of nats
 * lower.  `workspace` (at least streamkl_bwd_workspace_size_min bytes) is
 * overwritten.  Extra device memory beyond the caller's buffers: none.
 */
streamkl_status streamkl_bwd(const streamkl_problem *p,
                             const void *q1, const void *k1,
                             const void *q2, const void *k2,
                             const float *kl, const float *lse1, const float *lse2,
                             const float *g,
                             float *dq1, float *dk1, float *dq2, float *dk2,
                             void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * The backward in steps: streamkl_bwd is exactly streamkl_bwd_prepare, then
 * streamkl_bwd_dk, then streamkl_bwd_dq, on one stream.  The two passes only
 * read their inputs and the prepared workspace, so once the prepare step has
 * completed they may run on different streams.
 *
 * streamkl_bwd_prepare writes into `workspace`, per (batch, head): the power
 * of two sigma with max_i |g_i| * sigma in [2^7, 2^8), by which the passes
 * scale dS before rounding it to fp16 (1 for fp32 inputs), negated when some
 * g of that head is negative; and the powers of two that scale the fp16
 * operands of q1, q2, k1, k2 (1 for fp32 and fp8 inputs), from their largest
 * magnitudes.  It reads q1, k1, q2, k2 (bf16 inputs only) and g, with the
 * layouts and alignment rules of streamkl_bwd, and needs at least
 * streamkl_bwd_workspace_size_min bytes; the passes take the workspace size
 * rules of streamkl_bwd (the dQ pass splits its keys only given the full size).
 * streamkl_bwd_dk writes dK1, dK2 (one pass over key tiles, queries streamed);
 * streamkl_bwd_dq writes dQ1, dQ2 (one pass over query tiles, keys streamed).
 * NULL-pair rules, layouts and errors are those of streamkl_bwd.  The dK
 * pass only reads `workspace`; the dQ pass also writes the partial dQ area
 * when its keys are split, so two dQ passes must not share a workspace
 * concurrently.
 */
streamkl_status streamkl_bwd_prepare(const streamkl_problem *p,
                                     const void *q1, const void *k1,
                                     const void *q2, const void *k2,
                                     const float *g,
                                     void *workspace, size_t workspace_bytes, void *stream);

streamkl_status streamkl_bwd_dk(const streamkl_problem *p,
                                const void *q1, const void *k1,
                                const void *q2, const void *k2,
                                const float *kl, const float *lse1, const float *lse2,
                                const float *g, float *dk1, float *dk2,
                                const void *workspace, size_t workspace_bytes, void *stream);

streamkl_status streamkl_bwd_dq(const streamkl_problem *p,
                                const void *q1, const void *k1,
                                const void *q2, const void *k2,
                                const float *kl, const float *lse1, const float *lse2,
                                const float *g, float *dq1, float *dq2,
                                const void *workspace, size_t workspace_bytes, void *stream);

/*
 * Packed variable-length batches.  The pages list variable-length queries and
 * keys as future work (arxivlens.com paper view of StreamKL, future
 * directions).  Here each sequence is an independent problem of the kind
 * above, and a batch of them is packed without padding.
 *
 * Sequence b owns query rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key
 * rows [cu_seqlens_k[b], cu_seqlens_k[b+1]) of every head, with
 * TQ = cu_seqlens_q[B] and TK = cu_seqlens_k[B]:
 *  - Q1, Q2 are [H, TQ, D] and K1, K2 are [H, TK, D], contiguous, in `dtype`
 *    (head-major: each head's sequences follow one another);
 *  - KL, LSE1, LSE2 and g are fp32 [H, TQ];
 *  - gradients are fp32 with the shape of their tensor.
 * Within a sequence, the visible set, the scale and the causal rule are
 * those of streamkl_problem with NQ, NK the sequence's own lengths (causal
 * masks are bottom-right aligned per sequence).  Results are those of a
 * separate streamkl_fwd / streamkl_bwd call per sequence.
 *
 * cu_seqlens_q and cu_seqlens_k are HOST arrays of B + 1 int32 offsets
 * starting at 0.  They are read during the call only and never kept.
 * Errors (STREAMKL_ERR_SHAPE) are:
 *  - a nonzero first offset or a decreasing offset;
 *  - any sequence that would be rejected as a streamkl_problem: keys == 0
 *    with queries > 0, causal with more queries than keys, or per-sequence
 *    sizes past the 32-bit limits.
 * Sequences with no query rows produce nothing in the forward and zero key
 * gradients in the backward.  Consecutive sequences of equal lengths form a
 * run.  The runs share launches: each kernel runs over up to 32 runs at once
 * (longest first), so that batches of many short sequences still fill the
 * GPU.  Exceptions launch per run, after the shared launches:
 *  - bf16 runs of at most 32 queries per sequence (the forward's one-wave
 *    shapes);
 *  - in the backward, when the whole batch has fewer than 256 query tiles of
 *    128 rows, runs whose own problem would split the query-gradient pass's
 *    keys (see streamkl_bwd_workspace_size).
 * Each sequence's results are those of streamkl_fwd / streamkl_bwd on that
 * sequence alone (the same bits, except dQ where the stand-alone call would
 * split its keys, which changes only the fp32 summation order).
 */
typedef struct {
    int64_t B, H;                  /* sequences, heads */
    int64_t D;                     /* head dimension: 64 or 128 */
    const int32_t *cu_seqlens_q;   /* host, B + 1 query-row offsets */
    const int32_t *cu_seqlens_k;   /* host, B + 1 key-row offsets */
    float scale;                   /* logit scale, as in streamkl_problem */
    int32_t causal;                /* nonzero: per-sequence bottom-right causal mask */
    int32_t dtype;                 /* streamkl_dtype of Q1, K1, Q2, K2 */
} streamkl_varlen_problem;

/* Forward of every sequence (as streamkl_fwd).  Extra device memory: none. */
streamkl_status streamkl_fwd_varlen(const streamkl_varlen_problem *v,
                                    const void *q1, const void *k1,
                                    const void *q2, const void *k2,
                                    float *kl, float *lse1, float *lse2,
                                    void *stream);

/*
 * Workspace bytes for streamkl_bwd_varlen: the per-(sequence, head) factors
 * of streamkl_bwd_workspace_size (sigma, operand scales and, for bf16 inputs,
 * their partial maxima) for all B * H (sequence, head) pairs, laid out as for
 * a problem of B * H heads.  If larger, it is instead the largest full-size
 * streamkl_bwd workspace of a run launched on its own (those reuse the front
 * of the workspace one after another).  Returns 0 if `v` is invalid.
 */
size_t streamkl_bwd_varlen_workspace_size(const streamkl_varlen_problem *v);

/*
 * Backward of every sequence (as streamkl_bwd, same NULL-pair rules and
 * operand scaling).  kl, lse1 and lse2 must come from
 * streamkl_fwd_varlen on the same inputs.  `workspace` must hold at least
 * streamkl_bwd_varlen_workspace_size bytes (STREAMKL_ERR_WORKSPACE
 * otherwise) and is overwritten.
 */
streamkl_status streamkl_bwd_varlen(const streamkl_varlen_problem *v,
                                    const void *q1, const void *k1,
                                    const void *q2, const void *k2,
                                    const float *kl, const float *lse1, const float *lse2,
                                    const float *g,
                                    float *dq1, float *dk1, float *dq2, float *dk2,
                                    void *workspace, size_t workspace_bytes,
                                    void *stream);

/* Static, NUL-terminated description of a status code. */
const char *streamkl_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int streamkl_version(void);

/*
 * Measurement helper, not part of the method: the sustained rate of the bf16
 * matrix instruction the kernels use (v_mfma_f32_32x32x16_bf16), which a
 * roofline report can set beside the published peak.  Launches `workgroups`
 * workgroups of four waves; each wave runs `iters` rounds of four independent
 * 32x32x16 products on register operands (no memory traffic in the loop), so
 * the work is workgroups * 4 * iters * 4 * 32768 flop.  `sink` is a device
 * buffer of at least workgroups * 4 floats owned by the caller; it receives
 * one value per wave (to keep the products live) and carries no meaning.
 * The caller times the call on `stream` (events before and after).
 * iters must be in [1, 2^24] and workgroups in [1, 2^20]: STREAMKL_ERR_SHAPE
 * otherwise; NULL sink: STREAMKL_ERR_NULL; sink not 16-byte aligned:
 * STREAMKL_ERR_ALIGN.  Asynchronous like every other call.
 */
streamkl_status streamkl_probe_mfma_bf16(int64_t iters, int64_t workgroups, float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* STREAMKL_H */
