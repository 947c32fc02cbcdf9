/*
 * gdp.h -- C ABI of the MI355X (gfx950) chunked Gated Delta Product forward.
 *
 * Operations (names follow the Megatron-Core GDP op pages):
 *   gdp_prefill_prepare  split / GQA-expand / Householder-fold / gate a prefill
 *                        step (core.ssm.ops.gdp.prepare, gdp_prefill_prepare)
 *   gdp_recompute_w_u    per-chunk WY factors: L2 norm of k, within-chunk
 *                        cumulative decay, the strictly-lower transition
 *                        block, its unit-lower inverse, then w and u
 *                        (core.ssm.ops.gdp.wy_fast, recompute_w_u_fwd)
 *   gdp_chunk_h          inter-chunk state recurrence: state at every chunk
 *                        boundary and the corrected values (the chunk_h stage
 *                        named by core.ssm.ops.gdp.chunk_o)
 *   gdp_chunk_o          output from the boundary state plus causal in-chunk
 *                        attention summed over the Householder copies
 *                        (core.ssm.ops.gdp.chunk_o,
 *                        chunk_gated_delta_product_fwd_o)
 *   gdp_chunk_fwd        the three chunk stages in order
 *   gdp_chunk_fwd_pipelined  the same for one long sequence, in segments
 *                        whose parallel stages overlap the serial one
 *   gdp_prefill_fwd_pipelined  prepare plus the pipelined chunk forward,
 *                        with each segment's prepare overlapped too
 *   gdp_chunk_fwd_scan   the same for one long sequence or packed requests,
 *                        with each long serial state chain cut into segments
 *                        run in parallel
 *   gdp_chunk_fwd_scan_noalloc  that form with its workspace in a device
 *                        array of the library's own (callers that cannot
 *                        allocate)
 *   gdp_prefill_fwd_scan prepare fused into the WY stage of that form
 *   gdp_decode_prepare   the prepare of a decode step: query and decay
 *                        interleaved onto the Householder copies
 *                        (core.ssm.ops.gdp.prepare, gdp_decode_prepare)
 *   gdp_decode_update    the recurrence over a decode step's S*M rows, the
 *                        state read from and written back to a state pool
 *                        (the fused recurrent update the prepare page names
 *                        as the decode consumer)
 *
 * Conventions shared by every entry point
 *   * All tensor pointers are device pointers owned by the caller.  No call
 *     allocates or frees device memory or synchronises with the host; each
 *     only enqueues kernels on `stream` (a hipStream_t; NULL is the null
 *     stream) and returns.  Shapes are runtime values, so calls can be
 *     captured into a HIP graph.  Two entry points hold resources of their
 *     own: the pipelined forwards create two side streams and their events
 *     once per device, and gdp_chunk_fwd_scan_noalloc looks up its static
 *     device array once per device; make the first such call on a device
 *     outside graph capture.
 *   * Every call validates its arguments before launching anything.  A bad
 *     argument returns GDP_ERR_INVALID or GDP_ERR_UNSUPPORTED with nothing
 *     launched and nothing written; gdp_last_error() then describes it.  A
 *     failed launch returns GDP_ERR_HIP.
 *   * Results are deterministic: no atomics, every output element is owned
 *     by exactly one thread, and the order of every reduction is fixed.
 *   * Tensors are row-major and contiguous unless a stride is given.
 *   * "Expanded stream": the Householder copies folded into the sequence
 *     dimension; copy j of token t is row t*M + j.
 */
#ifndef GDP_H
#define GDP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdp_status {
    GDP_OK = 0,
    GDP_ERR_INVALID = 1,      /* inconsistent or out-of-range argument */
    GDP_ERR_UNSUPPORTED = 2,  /* valid but not built (head dims, M, chunk) */
    GDP_ERR_HIP = 3           /* a HIP launch failed */
} gdp_status;

typedef enum gdp_dtype {
    GDP_F32 = 0,
    GDP_BF16 = 1
} gdp_dtype;

/*
 * gdp_prefill_prepare -- one launch that turns the post-conv activations of a
 * prefill step into the inputs of the chunk forward
 * (core.ssm.ops.gdp.prepare: module description, gdp_prefill_prepare).
 *
 *   x     [n, T, M*H*P + M*G*N + G*N]  dtype; value (M,H,P) | key (M,G,N) |
 *         query (G,N) along the last dimension.  Element (b, t, c) is at
 *         x + b*x_n_stride + t*x_t_stride + c (strides in elements; the last
 *         dimension must be contiguous).
 *   ba    [n, T, M*H + H]              dtype; b (M,H) | a (H), strides as x.
 *   A_log, dt_bias [H]                 float32.
 *   Outputs (contiguous, caller-allocated):
 *   q     [n, T,   H, N]   dtype   q[b,t,h]      = query group h/(H/G)
 *   k     [n, T*M, H, N]   dtype   k[b,t*M+j,h]  = key copy j, group h/(H/G)
 *   v     [n, T*M, H, P]   dtype   v[b,t*M+j,h]  = value copy j, head h
 *   beta  [n, T*M, H]      float32 sigmoid(b[t, j, h])
 *   g     [n, T,   H]      float32 -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h])
 * softplus(s) is s for s > 20, else log1p(exp(s)).  Gate arithmetic is
 * float32 per operation in the order written, with exp and log1p evaluated
 * in float64 and rounded once.  The L2 norm of q and k is left to the chunk
 * forward.  Requires H % G == 0 and n, T >= 0 (T == 0 launches nothing).
 */
gdp_status gdp_prefill_prepare(
    const void *x, int64_t x_n_stride, int64_t x_t_stride,
    const void *ba, int64_t ba_n_stride, int64_t ba_t_stride,
    const float *A_log, const float *dt_bias,
    int64_t n, int64_t T, int32_t M, int32_t H, int32_t G, int32_t P, int32_t N,
    gdp_dtype dtype,
    void *q, void *k, void *v, float *beta, float *g,
    void *stream);

/*
 * gdp_decode_prepare -- the decode-step form of gdp_prefill_prepare
 * (core.ssm.ops.gdp.prepare: module description, the decode bullet, and
 * gdp_decode_prepare).  The S tokens of each request (1 plus the draft
 * length) walk the copies as one sequence of S*M rows: row t*M + j is copy j
 * of token t.  Same arguments and validation as gdp_prefill_prepare with T =
 * S; the outputs differ only in where query and g go:
 *   q     [n, S*M, H, N]   query of token t on row t*M + M - 1, zeros on the
 *                          other copies
 *   k     [n, S*M, H, N]   as prefill
 *   v     [n, S*M, H, P]   as prefill
 *   beta  [n, S*M, H]      float32, as prefill
 *   g     [n, S*M, H]      float32, g of token t on row t*M, zeros elsewhere
 */
gdp_status gdp_decode_prepare(
    const void *x, int64_t x_n_stride, int64_t x_t_stride,
    const void *ba, int64_t ba_n_stride, int64_t ba_t_stride,
    const float *A_log, const float *dt_bias,
    int64_t n, int64_t S, int32_t M, int32_t H, int32_t G, int32_t P, int32_t N,
    gdp_dtype dtype,
    void *q, void *k, void *v, float *beta, float *g,
    void *stream);

/*
 * Arguments of gdp_decode_update: one decode step of n requests, each a
 * sequence of L = S*M rows (the outputs of gdp_decode_prepare), gated delta
 * rule per row with the row's own decay and query:
 *   delta = beta (v - exp(g) S khat),  S <- exp(g) S + delta khat^T,
 *   o     = scale * S qhat             (zero on rows whose query is zero)
 * with khat, qhat L2-normalised as in the chunk forward.  Over rows from
 * gdp_decode_prepare this is the Gated Delta Product recurrence of the S
 * tokens (the decode interleave of the prepare page).
 *   q, k   [n, L, H, K]  dtype;  v [n, L, HV, V] dtype
 *   beta   [n, L, HV] float32;  g [n, L, HV] float32 natural-log decay per
 *          row, or NULL (ungated)
 *   state  [pool, HV, V, K] float32, the state S of each slot; read and
 *          written in place
 *   slots  int32 [n] device: the state slot of each request, or NULL (slot
 *          i for request i).  A slot outside [0, pool) -- e.g. -1 for a
 *          padding entry -- skips the request: no state is touched and its
 *          o rows are zero.  Slots of one call must be distinct.
 *   o      [n, L, HV, V] dtype, every row
 *   scale  <= 0 selects 1/sqrt(K).
 * Sizes: K in {64, 128}, V in {64, 128, 256}, HV % H == 0, 1 <= M <= 4,
 * S*M <= 4096, n < 2^31, HV <= 65535.
 */
typedef struct gdp_decode_args {
    int64_t n;
    int64_t S;
    int32_t H;
    int32_t HV;
    int32_t K;
    int32_t V;
    int32_t M;
    float scale;
    gdp_dtype dtype;
    int64_t pool;
    const void *q;
    const void *k;
    const void *v;
    const float *beta;
    const float *g;
    float *state;
    const int32_t *slots;
    void *o;
} gdp_decode_args;

gdp_status gdp_decode_update(const gdp_decode_args *a, void *stream);

/*
 * Arguments of the chunk stages.  Sizes:
 *   B           batch rows.  Without cu_seqlens every row is one sequence of
 *               T tokens; with cu_seqlens B must be 1 and the T tokens are
 *               packed requests (dynamic-batching prefill,
 *               core.ssm.ops.gdp.prepare, gdp_prefill_prepare).
 *   T           tokens per batch row (the packed total with cu_seqlens).
 *   H, HV       query/key heads and value/output heads; HV % H == 0 and
 *               value head hv reads key head hv / (HV/H)
 *               (core.ssm.ops.gdp.wy_fast, recompute_w_u_fwd, Parameters).
 *   K, V        key and value head dims; K in {64, 128}, V in {64, 128, 256}.
 *   M           Householder copies, 1..4.
 *   chunk_size  64 (rows of the expanded stream per chunk).
 *   scale       output scale; <= 0 selects 1/sqrt(K).
 *   cu_seqlens  device int32 [num_seqs + 1], token offsets of the requests
 *               on the unexpanded stream, or NULL.  Offsets are clamped into
 *               [0, T] on the device; a non-monotone array gives undefined
 *               results but never an out-of-bounds access.
 *   h_chunks    number of chunks h can hold (see gdp_num_state_chunks); h is
 *               written only below it.
 * Tensors (dtype unless noted; e = expanded row):
 *   q      [B, T,   H,  K]  in
 *   k      [B, T*M, H,  K]  in
 *   v      [B, T*M, HV, V]  in
 *   beta   [B, T*M, HV]     in, float32
 *   g      [B, T,   HV]     in, float32 natural-log decay per token; it acts
 *                           on copy 0 of its token.  NULL selects the
 *                           ungated rule (every decay is 0; the pages' g=None)
 *   k_rnorm[B, H, T*M]      float32 1/sqrt(sum k^2 + 1e-6) per key row (head-major);
 *                           written by gdp_recompute_w_u, read by gdp_chunk_o
 *   gcum   [B, HV, T*M]     float32 (head-major) within-chunk cumulative decay in log2
 *                           units per expanded row (the sum of g*log2(e) over
 *                           the first-copy rows of the chunk up to and
 *                           including the row); written by gdp_recompute_w_u,
 *                           read by gdp_chunk_h
 *   kdecay [B, HV, T*M]     float32 (head-major) per expanded row e of chunk c:
 *                           k_rnorm[e] * 2^(gcum[last row of c] - gcum[e]),
 *                           the factor with which the row's normalised key
 *                           enters the state at the end of its chunk;
 *                           written by gdp_recompute_w_u, read by gdp_chunk_h
 *   w      [B, T*M, HV, K]  out of gdp_recompute_w_u (effective keys)
 *   u      [B, HV, V/16, T*M, 16]  out of gdp_recompute_w_u (effective
 *                           values), in 16-column slices: element (b, e, hv,
 *                           c) at ((b*HV + hv)*(V/16) + c/16)*T*M*16 + e*16 +
 *                           c%16, so the rows of one slice are contiguous
 *   v_new  [B, HV, V/16, T*M, 16]  out of gdp_chunk_h (corrected values),
 *                           sliced like u
 *   h      [h_chunks, HV, V, K]  out of gdp_chunk_h: the V x K state S
 *                           entering each chunk (S maps a normalised key to a
 *                           value); chunk c of sequence i is at index
 *                           (chunks of sequences < i) + c
 *   o      [B, T,   HV, V]  out of gdp_chunk_o
 *   h0     [nseq, HV, V, K] in, float32, or NULL: the state S each sequence
 *                           starts from (NULL: zero).  h[first chunk] is
 *                           its storage-precision copy.  Read by gdp_chunk_h.
 *   ht     [nseq, HV, V, K] out, float32, or NULL: the state S after each
 *                           sequence's last row (h0, or zero, for an empty
 *                           sequence).  Written by gdp_chunk_h.  Passing one
 *                           call's ht as the next call's h0 continues the
 *                           recurrence exactly (chunked prefill).
 * nseq is num_seqs with cu_seqlens, else B.
 */
typedef struct gdp_chunk_args {
    int64_t B;
    int64_t T;
    int32_t H;
    int32_t HV;
    int32_t K;
    int32_t V;
    int32_t M;
    int32_t chunk_size;
    float scale;
    gdp_dtype dtype;
    const int32_t *cu_seqlens;
    int64_t num_seqs;
    int64_t h_chunks;
    const void *q;
    const void *k;
    const void *v;
    const float *beta;
    const float *g;
    float *k_rnorm;
    float *gcum;
    float *kdecay;
    void *w;
    void *u;
    void *v_new;
    void *h;
    void *o;
    const float *h0;
    float *ht;
} gdp_chunk_args;

/* w, u, k_rnorm, gcum and kdecay from k, v, beta, g. */
gdp_status gdp_recompute_w_u(const gdp_chunk_args *a, void *stream);
/* h, v_new and (if requested) ht from k, kdecay, gcum, w, u and h0.  One serial pass per sequence and
   value head over its chunks. */
gdp_status gdp_chunk_h(const gdp_chunk_args *a, void *stream);
/* o from q, k, k_rnorm, v_new, h, g. */
gdp_status gdp_chunk_o(const gdp_chunk_args *a, void *stream);
/* gdp_recompute_w_u, gdp_chunk_h, gdp_chunk_o in order on one stream.
 * With v_new and h both NULL (bf16, M >= 2) chunk_h and chunk_o run as one
 * pass (core.ssm.ops.gdp.chunk_o, module description: chunk_h's boundary
 * states combined with the causal in-chunk attention over the copies) that
 * stores neither, and h_chunks is not checked.  w, u, k_rnorm, gcum, kdecay
 * and ht are then bit-identical to the two-stage call, and o agrees with it
 * to rounding: the one pass forms each score's decay and norm factor as one
 * power of two of log2-scaled decays and norms, and runs the output product
 * V^T P^T on fp16 operands, so v_new must stay within fp16's range
 * (|v_new| < 65504), else o is not finite.  v_new and h NULL with another
 * dtype or M == 1 return GDP_ERR_UNSUPPORTED; only one of them NULL returns
 * GDP_ERR_INVALID. */
gdp_status gdp_chunk_fwd(const gdp_chunk_args *a, void *stream);

/*
 * gdp_chunk_fwd_pipelined -- the same results as gdp_chunk_fwd for one long
 * sequence (B == 1, cu_seqlens == NULL), computed in num_segments pieces of
 * whole 64-token chunks (gdp_pipeline_plan gives where each starts) so that
 * the parallel stages overlap the serial one:
 * chunk_h runs the segments in order on `stream`, handing the fp32 state
 * from one segment to the next (as h0 / ht).  The first segment's
 * gdp_recompute_w_u and the last one's gdp_chunk_o also run on `stream`;
 * the other segments' gdp_recompute_w_u (back to back, from the end of the
 * first one) and gdp_chunk_o (each after its own chunk_h) run on two
 * streams of the library's own (created once per device, default
 * priority) that join `stream` through events.  With one segment every
 * stage runs on `stream`.  On return all work is ordered before later work
 * on `stream`; nothing is synchronised with the host.  The first call on a
 * device, and a call with more segments than any before it, create the
 * streams and events it needs: make such a call outside graph capture.
 * Later calls create nothing and can be captured into a HIP graph (the
 * side streams join the capture through the events).
 *   state_workspace  float32 [2, HV, V, K], device, caller-owned: the state
 *                    handed between segments.
 *   chunk_h_events   NULL, or 2 * gdp_pipeline_segments(T, num_segments)
 *                    hipEvent_t handles (as void *), which are recorded on
 *                    `stream` right before and right after each segment's
 *                    chunk_h launch (for timing that stage).
 *   The per-row intermediates k_rnorm, gcum and kdecay are laid out per
 *   segment (segment s, starting at token t_s, holds its head-major block of
 *   H or HV rows of (its tokens * M) values at offset t_s * M * (H or HV)).
 *   Every other tensor is as for gdp_chunk_fwd, and o, w, u, v_new, h and ht
 *   are bit-identical to it.
 * Concurrent calls on one device are serialised while they enqueue.
 */
gdp_status gdp_chunk_fwd_pipelined(const gdp_chunk_args *a, int32_t num_segments, float *state_workspace,
                                   void *const *chunk_h_events, void *stream);

/*
 * Arguments of gdp_prefill_prepare that gdp_prefill_fwd_pipelined needs
 * besides the chunk arguments (whose B = n, T, M, H, V = P, K = N and dtype
 * it shares).
 */
typedef struct gdp_prepare_args {
    const void *x;
    int64_t x_n_stride;
    int64_t x_t_stride;
    const void *ba;
    int64_t ba_n_stride;
    int64_t ba_t_stride;
    const float *A_log;
    const float *dt_bias;
    int32_t G;
} gdp_prepare_args;

/*
 * gdp_prefill_fwd_pipelined -- gdp_prefill_prepare followed by
 * gdp_chunk_fwd_pipelined, with the prepare of each segment run just
 * before that segment's WY, on the same stream, so that only the first
 * segment's prepare precedes the serial stage.  Prepare writes the chunk
 * arguments' q, k, v, beta and g (which must therefore be writable, g not
 * NULL, and HV == H: prepare makes H value heads).  Results are
 * bit-identical to the two calls in sequence; the requirements and the
 * per-segment layout of k_rnorm, gcum and kdecay are those of
 * gdp_chunk_fwd_pipelined, the prepare arguments are checked as by
 * gdp_prefill_prepare.
 */
gdp_status gdp_prefill_fwd_pipelined(const gdp_prepare_args *p, const gdp_chunk_args *a, int32_t num_segments,
                                     float *state_workspace, void *const *chunk_h_events, void *stream);

/*
 * gdp_chunk_fwd_scan -- the same results as gdp_chunk_fwd, within rounding,
 * for one long sequence (B == 1, cu_seqlens == NULL) or for packed requests
 * (B == 1 with cu_seqlens: the dynamic-batching prefill of
 * core.ssm.ops.gdp.prepare), with the serial chunk_h chain of every long
 * sequence cut into segments that run in parallel.  Over one chunk the state
 * update is affine in the entering state (the chunk transition of the WY
 * representation of the product of the chunk's generalised Householder
 * factors, core.ssm.ops.gdp.wy_fast and the chunk_h stage of
 * core.ssm.ops.gdp.chunk_o), so each segment's map h -> D h + E is
 * composed first, all segments at once; a short serial pass over each
 * sequence's segments then gives the state entering each of them, and one
 * chunk_h pass runs every segment from its own entering state.  All work is
 * enqueued on `stream`, in this order: gdp_recompute_w_u; for packed
 * requests the segment plan (gdp_seg_plan_k, on the device from
 * cu_seqlens); the segment maps (gdp_seg_map_k); the scan over segments
 * (gdp_seg_scan_k); chunk_h; gdp_chunk_o; and, if ht is given, the final
 * states (a device copy, or gdp_seg_final_k for packed requests).
 *   num_segments    1..GDP_SCAN_MAX_SEGMENTS requested; segments are
 *                   seg_tok = ceil(ceil(T/64) / num_segments) * 64 tokens
 *                   long, T the sequence length or the packed total.  One
 *                   sequence is cut into ceil(T / seg_tok) of them
 *                   (gdp_scan_segments); each packed request of length L
 *                   into ceil(L / seg_tok), so requests shorter than seg_tok
 *                   stay whole and need no map.
 *   workspace       device memory of at least gdp_scan_workspace_bytes(...)
 *                   (one sequence) or gdp_scan_workspace_bytes_varlen(...)
 *                   (packed requests) bytes, 256-byte aligned,
 *                   caller-owned; its contents on entry do not matter and on
 *                   return are unspecified.
 *   stage_events    NULL, or 5 hipEvent_t handles (as void *) recorded on
 *                   `stream` right after the WY stage (and the plan), after
 *                   the segment maps, after the scan, after chunk_h and after
 *                   chunk_o (for timing each stage).
 * Every tensor of `a` is as for gdp_chunk_fwd, except h: only the states
 * entering chunks c = i*M of each sequence (those entering each 64-token
 * chunk, the ones gdp_chunk_o reads) are written; the other slots of h are
 * left untouched.  w, u, k_rnorm, gcum and kdecay are bit-identical to
 * gdp_chunk_fwd, and so are h, v_new and o over the first segment of each
 * sequence; the states entering later segments come out of the composed
 * maps, so h, v_new, o and ht there agree with gdp_chunk_fwd to rounding
 * (the composition runs on matrix-core operands with fp32 accumulation like
 * the chunk recurrence itself: bf16 in its first product and fp16 in its
 * second, so keys must stay within fp16's range, |k| < 65504).  v_new
 * and h may both be NULL as for gdp_chunk_fwd: chunk_h and chunk_o then run
 * as one pass over every segment, from its scanned state, and no state
 * leaves the chip.  Supported: dtype bf16 with
 * K, V in {64, 128} and T*M*V*2 < 2^31; other shapes return
 * GDP_ERR_UNSUPPORTED.  B > 1 without cu_seqlens returns GDP_ERR_INVALID.
 */
#define GDP_SCAN_MAX_SEGMENTS 64
gdp_status gdp_chunk_fwd_scan(const gdp_chunk_args *a, int32_t num_segments, void *workspace,
                              int64_t workspace_bytes, void *const *stage_events, void *stream);

/*
 * gdp_chunk_fwd_scan_noalloc -- gdp_chunk_fwd_scan for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels, results bit-identical
 * to gdp_chunk_fwd_scan, with the workspace taken from a device array of the
 * library's own instead of from the caller.  The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine); the caller still passes
 * every input and output in `a`.
 *   Limit: the workspace gdp_scan_workspace_bytes(T, HV, K, V,
 *   num_segments) reports (gdp_scan_workspace_bytes_varlen with
 *   cu_seqlens) must fit GDP_NOALLOC_SCRATCH_BYTES (64 MiB; the
 *   32768-token, 16-head, K = V = 128 sequence with 16 segments needs 47.5
 *   MiB); a larger call returns GDP_ERR_UNSUPPORTED, launches nothing and
 *   makes no HIP call.  Every other argument is checked, and refused, as by
 *   gdp_chunk_fwd_scan.
 *   The array: each GPU the library runs on holds one copy of
 *   GDP_NOALLOC_SCRATCH_BYTES until the process ends.  Every call on a GPU
 *   shares that GPU's copy and leaves its last contents there (nothing in it
 *   needs to start at zero): calls on one GPU that overlap in time -- on
 *   different streams, or from several threads without ordering -- race and
 *   give undefined results; calls on one stream are ordered and safe.  The
 *   first call on each device looks the array's device address up
 *   (hipGetSymbolAddress) and keeps it; make that first call outside graph
 *   capture.  Later calls can be captured.
 *   stage_events as for gdp_chunk_fwd_scan.
 */
#define GDP_NOALLOC_SCRATCH_BYTES (64LL * 1024 * 1024)
gdp_status gdp_chunk_fwd_scan_noalloc(const gdp_chunk_args *a, int32_t num_segments, void *const *stage_events,
                                      void *stream);

/*
 * gdp_prefill_fwd_scan -- gdp_prefill_prepare followed by gdp_chunk_fwd_scan
 * for one sequence or packed requests (n == B == 1, with or without
 * cu_seqlens), with the prepare done inside the WY stage: each
 * gdp_recompute_w_u block reads its key and value copies, query and gate
 * inputs straight from x and ba (the layouts of gdp_prefill_prepare), writes
 * prepare's outputs for its rows (q and g of a token by the block holding
 * the token's copy 0) and uses them, so the key and value copies are not
 * read back from HBM.  Prepare writes the chunk arguments' q, k, v, beta and
 * g (which must therefore be writable, g not NULL, and HV == H: prepare
 * makes H value heads).  v and beta may be NULL: no stage after WY reads
 * them (the values enter u inside it), so they are then not stored, which
 * saves their HBM writes; every other output is unchanged.  With v_new and
 * h NULL (the one-pass form), q and k may be NULL too, both or neither: WY
 * then neither stores the key copies and queries nor loads the queries, and
 * the segment maps and the one pass read the key and query rows from x at
 * prepare's offsets, so every other output is bit-identical to the run that
 * stores them.  q and k NULL with v_new or h given return
 * GDP_ERR_UNSUPPORTED; only one of q, k NULL returns GDP_ERR_INVALID.  Every output is
 * bit-identical to the two calls in sequence, except that with cu_seqlens
 * the prepare outputs of tokens outside every request (none when the
 * offsets run from 0 to T) are not written.  The requirements are those of
 * gdp_chunk_fwd_scan (B == n == 1) and of gdp_prefill_prepare, plus 16-byte
 * aligned rows of x and of the outputs; stage_events as for
 * gdp_chunk_fwd_scan (the first one is recorded after the WY-with-prepare
 * stage).
 */
gdp_status gdp_prefill_fwd_scan(const gdp_prepare_args *p, const gdp_chunk_args *a, int32_t num_segments,
                                void *workspace, int64_t workspace_bytes, void *const *stage_events, void *stream);

/* Segments gdp_chunk_fwd_scan runs for T tokens and num_segments requested
   (0 for T == 0), or -1 on bad arguments. */
int32_t gdp_scan_segments(int64_t T, int32_t num_segments);

/* Workspace bytes gdp_chunk_fwd_scan needs for one sequence: per value
   head, a map of K x (V + K) floats' bytes for every segment but the last
   (E in fp32, then D as a high and a low bf16 part) and a V x K fp32 state
   for every segment, plus the segment offsets; -1 on bad arguments.  The
   workspace is opaque to the caller. */
int64_t gdp_scan_workspace_bytes(int64_t T, int32_t HV, int32_t K, int32_t V, int32_t num_segments);

/* Workspace bytes gdp_chunk_fwd_scan needs for num_seqs packed requests of T
   tokens in all: a map and a state per value head for each of the
   ceil(T / seg_tok) + num_seqs slots that can hold a segment, plus the plan
   (offsets and flags per slot, first slot and count per request); -1 on bad
   arguments.  It depends on T and num_seqs only, not on the lengths. */
int64_t gdp_scan_workspace_bytes_varlen(int64_t T, int64_t num_seqs, int32_t HV, int32_t K, int32_t V,
                                        int32_t num_segments);

/* Segments gdp_chunk_fwd_pipelined actually runs for T tokens (whole
   64-token chunks, at most num_segments); 0 for T == 0, -1 on bad
   arguments. */
int32_t gdp_pipeline_segments(int64_t T, int32_t num_segments);

/* Where those segments start: writes n + 1 token offsets to starts (host
   memory, room for num_segments + 1), starts[0] = 0 and starts[n] = T, and
   returns n = gdp_pipeline_segments(T, num_segments); -1 on bad arguments
   (starts NULL included).  Segments hold equal shares of the 64-token
   chunks (boundaries rounded to whole chunks, so every boundary is a
   multiple of 64 tokens).  The per-segment blocks of k_rnorm, gcum and
   kdecay start at these offsets. */
int32_t gdp_pipeline_plan(int64_t T, int32_t num_segments, int64_t *starts);

/*
 * Number of state chunks h must hold: sum over sequences of
 * ceil(len * M / chunk_size).  With cu_seqlens_host == NULL it is
 * B * ceil(T * M / chunk_size).  cu_seqlens_host is a host copy of the
 * offsets.  Returns -1 on bad arguments.  ceil(T*M/chunk_size) + num_seqs is
 * always enough and needs no copy of the offsets.
 */
int64_t gdp_num_state_chunks(const int32_t *cu_seqlens_host, int64_t num_seqs,
                             int64_t B, int64_t T, int32_t M, int32_t chunk_size);

/* Message describing the last non-OK status of this thread ("" if none). */
const char *gdp_last_error(void);

/* Library version string. */
const char *gdp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDP_H */
