/*
 * gdn.h -- C ABI of libgdn, the Gated DeltaNet (GDN) token mixer for AMD
 * MI355X (gfx950).
 *
 * The GDN layer is the linear-attention block that HyLo places in half or
 * more of a Transformer's layers so that those layers keep a fixed-size
 * recurrent state instead of a KV cache (kwkr.cn digest of
 * HyLo-Llama-8MLA8GDN-8K-SFT, architecture section on 8 MLA + 8 Gated
 * DeltaNet layers; ftxj.github.io digest of arXiv 2604.24715, Key Ideas and
 * Method).  The pages describe its update only in words -- a gated delta rule
 * that can erase or rewrite the value stored under one key (we0.ai article on
 * Priming, comparison of Mamba-2, Gated DeltaNet and Gated KalmaNet).  The
 * library computes the standard form of that rule, per sequence b and head h:
 *
 *     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   a_t = exp(g_t)
 *     o_t = S_t q_t / sqrt(d_k)
 *
 * with the state S in R^{d_v x d_k}.  The readout uses the updated state.
 *
 * Conventions shared by every call
 *   - Every pointer is a device pointer owned by the caller.  The library
 *     allocates, frees and retains no memory.
 *   - Tensors are dense, row-major and contiguous, and every pointer must be
 *     16-byte aligned.
 *   - q, k, v are stored as qkv_dtype (GDN_F32 or GDN_BF16); g, beta, states
 *     and outputs are always fp32.
 *   - States are stored key-major: [.., d_k, d_v], element (j, i) = S[i][j].
 *   - q and k are used as given (the library does not normalise them);
 *     scale = 1/sqrt(d_k) is fixed; g is expected finite and <= 0; beta is
 *     used as given (no clamp).
 *   - Work is queued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns at once.  Arguments are validated on the host before
 *     anything is queued: a call that returns an error has queued nothing and
 *     written nothing.  Faults inside kernels surface at the caller's next
 *     synchronisation with the stream.
 *   - Supported sizes: d_k, d_v in {16, 64, 128}; chunk in {16, 32, 64}.
 *
 * A second rule (gdn_rule, the *_rule entry points) drops the erase term:
 *
 *     S_t = a_t S_{t-1} + b_t v_t k_t^T
 *
 * the uniform decay the Priming article attributes to Mamba-2, which the
 * HyLo hybrids use as the other linear block (aiexpert.news article on HyLo:
 * selected attention layers become Mamba2 or Gated DeltaNet blocks; we0.ai
 * Priming article: Mamba-2 lets the whole state fade while new information is
 * added).  Everything else -- layouts, readout, scale, chunking, workspace --
 * is shared by both rules.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 7

#if defined(__GNUC__) || defined(__clang__)
#define GDN_API __attribute__((visibility("default")))
#else
#define GDN_API
#endif

/* In C++ the enums below get int as their underlying type, so every int a C
 * caller passes is a value of the type (unknown codes are then rejected, not
 * undefined). */
#ifdef __cplusplus
#define GDN_ENUM_INT : int
#else
#define GDN_ENUM_INT
#endif

typedef enum gdn_status GDN_ENUM_INT {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,        /* a required pointer is NULL */
    GDN_ERR_SHAPE = 2,       /* a size is negative / zero where not allowed, or too large */
    GDN_ERR_UNSUPPORTED = 3, /* d_k, d_v, chunk or dtype outside the supported set */
    GDN_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
    GDN_ERR_ALIAS = 5,       /* an output overlaps an input (other than the allowed in-place state) */
    GDN_ERR_WORKSPACE = 6,   /* workspace missing or smaller than gdn_chunk_prefill_workspace_size() */
    GDN_ERR_HIP = 7,         /* the HIP runtime reported an error while queuing work */
    GDN_ERR_CAPTURE = 8      /* the stream is capturing a graph, and this call copies host
                                data that must not outlive it (packed-sequence calls) */
} gdn_status;

typedef enum gdn_dtype GDN_ENUM_INT {
    GDN_F32 = 0,  /* IEEE binary32 */
    GDN_BF16 = 1  /* bfloat16 (upper half of a binary32) */
} gdn_dtype;

typedef enum gdn_rule GDN_ENUM_INT {
    GDN_RULE_GATED_DELTA = 0, /* S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T */
    GDN_RULE_GATED_DECAY = 1  /* S_t = a_t S_{t-1} + b_t v_t k_t^T (no erase term) */
} gdn_rule;

/*
 * gdn_chunk_prefill -- run the rule over T tokens of B sequences at once.
 *
 * The sequence is processed in chunks of at most `chunk` tokens (the last chunk
 * may be partial): `chunk` is the longest chunk the kernels may use, and they
 * pick their chunk length within it (bf16 inputs with 64- or 128-wide heads
 * run the gated delta rule in 32-token chunks when 64 is allowed, which is
 * faster on gfx950; the rule without the erase term keeps 64).  Any chunk
 * length gives the same recurrence up to rounding.  Inside a chunk the
 * per-token updates are folded into dense
 * products: a cumulative log-gate, the lower-triangular system
 * (I + tril(diag(b) K K^T * decay)) solved by forward substitution, the
 * W/U products, a scan of the fp32 state from chunk to chunk, and outputs as
 * the intra-chunk term plus Q times the chunk's start state.  The result
 * equals the token-by-token rule up to rounding.  A long sequence on few heads
 * is split into pieces run side by side, each piece's affine map from its
 * start state to its end state chained afterwards; the map's part that
 * multiplies the start state is set to zero once every element is at most
 * 2^-32 while no token of the piece so far could enlarge it (log-gate <= 0
 * and b |k|^2 <= 2), which moves a piece's end state by at most 2^-25 of the
 * start state's norm, below fp32 rounding (inputs outside that range get the
 * map without this).  The final state is the
 * fixed-size hidden state a GDN layer keeps per request in place of a KV
 * cache, so a long prompt can be fed in successive calls with the state
 * carried between them (ftxj.github.io digest of arXiv 2604.24715, Key Ideas;
 * Figure 5 runs such hybrids to 2M-token contexts).
 *
 *   q, k           [B, T, H, d_k]  qkv_dtype
 *   v              [B, T, H, d_v]  qkv_dtype
 *   g, beta        [B, T, H]       fp32 (log-gate; a_t = exp(g_t))
 *   initial_state  [B, H, d_k, d_v] fp32, or NULL for a zero start state
 *   o              [B, T, H, d_v]  fp32, written
 *   final_state    [B, H, d_k, d_v] fp32, written; may be the same pointer
 *                  as initial_state (in-place chaining of calls), but may not
 *                  overlap it otherwise
 *   workspace      device scratch of at least
 *                  gdn_chunk_prefill_workspace_size(...) bytes (may be NULL
 *                  when that size is 0); its contents on entry do not matter
 *   T may be 0: then nothing is read but the start state, which is copied to
 *   final_state (zeros when initial_state is NULL).
 * Errors: GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_UNSUPPORTED, GDN_ERR_ALIGN,
 * GDN_ERR_ALIAS (o overlapping any input or final_state, final_state
 * overlapping q/k/v/g/beta, or the workspace overlapping anything),
 * GDN_ERR_WORKSPACE, GDN_ERR_HIP.
 */
GDN_API gdn_status gdn_chunk_prefill(const void *q, const void *k, const void *v,
                             const float *g, const float *beta,
                             const float *initial_state,
                             float *o, float *final_state,
                             int B, int T, int H, int d_k, int d_v, int chunk,
                             gdn_dtype qkv_dtype,
                             void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * gdn_chunk_prefill_rule -- gdn_chunk_prefill for either rule.  Identical
 * arguments, layouts, workspace and errors; an unknown `rule` returns
 * GDN_ERR_UNSUPPORTED.  gdn_chunk_prefill(...) is
 * gdn_chunk_prefill_rule(GDN_RULE_GATED_DELTA, ...).
 */
GDN_API gdn_status gdn_chunk_prefill_rule(gdn_rule rule,
                             const void *q, const void *k, const void *v,
                             const float *g, const float *beta,
                             const float *initial_state,
                             float *o, float *final_state,
                             int B, int T, int H, int d_k, int d_v, int chunk,
                             gdn_dtype qkv_dtype,
                             void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * Bytes of device scratch gdn_chunk_prefill needs for these sizes (0 if
 * none); the same size serves gdn_chunk_prefill_rule with either rule.
 * Returns 0 as well for arguments gdn_chunk_prefill would reject.  It holds
 * the maps and start states of the sequence pieces (bounded by the chip's
 * workgroup slots, not by T) and, for d_k = d_v = 128, every chunk's
 * T diag(b) (T the inverse of the chunk's unit lower-triangular system of
 * the chunked rule, kept as hi/lo bf16 operand fragments: 4 KiB per 32-token
 * chunk and head), formed once in the pieces' first pass and read in the
 * second.
 */
GDN_API size_t gdn_chunk_prefill_workspace_size(int B, int T, int H, int d_k, int d_v, int chunk,
                                        gdn_dtype qkv_dtype);

/*
 * gdn_chunk_prefill_noalloc -- gdn_chunk_prefill_rule that allocates nothing
 * and takes no workspace, for callers that cannot allocate device memory:
 * code under HIP graph capture, serving loops that must not call hipMalloc,
 * harnesses that forbid allocation.  The scratch the call needs comes from
 * one static device array of GDN_NOALLOC_SCRATCH_BYTES per GPU, which the
 * library holds from the first call on that GPU until the process ends.
 *
 * Arguments, layouts, results and errors are those of gdn_chunk_prefill_rule
 * without the workspace; GDN_ERR_WORKSPACE means that the pieces' maps and
 * start states exceed GDN_NOALLOC_SCRATCH_BYTES (no dense call does today: the
 * piece plan bounds them by the chip's workgroup slots, not by T; the largest,
 * 128-wide heads, need about 50 MiB).  The per-chunk T diag(b) fragments that
 * gdn_chunk_prefill_workspace_size also counts for 128-wide heads are not
 * kept here: this call forms them again in the second pass, with the same
 * results.
 * Every call on one GPU uses that GPU's single array: calls that may overlap
 * in time on one GPU (different streams, or threads) race on it and must be
 * ordered by the caller.  Nothing in the array needs clearing between calls
 * (each call writes every scratch byte it reads).
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

GDN_API gdn_status gdn_chunk_prefill_noalloc(gdn_rule rule,
                             const void *q, const void *k, const void *v,
                             const float *g, const float *beta,
                             const float *initial_state,
                             float *o, float *final_state,
                             int B, int T, int H, int d_k, int d_v, int chunk,
                             gdn_dtype qkv_dtype, void *stream);

/*
 * gdn_decode_step -- one token for each of N independent sequences: the rule
 * with T = 1, applied to a batch of per-sequence states in place.  The state
 * has a fixed size, so a step costs the same at any context length (we0.ai
 * article on Priming: attention layers converted into fixed-state SSM layers;
 * ftxj.github.io digest of arXiv 2604.24715, Figure 5: with the recurrent
 * layers' fixed state, time per output token stays about level from 8K to 64K).
 *
 *   q, k      [N, H, d_k]  qkv_dtype
 *   v         [N, H, d_v]  qkv_dtype
 *   g, beta   [N, H]       fp32
 *   state     [N, H, d_k, d_v] fp32, read and updated in place
 *   o         [N, H, d_v]  fp32, written
 * N may be 0 (nothing is done); N * H * 8 must stay below 2^31 (GDN_ERR_SHAPE).
 * Errors: GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_UNSUPPORTED, GDN_ERR_ALIGN,
 * GDN_ERR_ALIAS (o or state overlapping an input or each other), GDN_ERR_HIP.
 */
GDN_API gdn_status gdn_decode_step(const void *q, const void *k, const void *v,
                           const float *g, const float *beta,
                           float *state, float *o,
                           int N, int H, int d_k, int d_v,
                           gdn_dtype qkv_dtype, void *stream);

/*
 * gdn_decode_step_rule -- gdn_decode_step for either rule (same arguments and
 * errors; an unknown `rule` returns GDN_ERR_UNSUPPORTED).
 */
GDN_API gdn_status gdn_decode_step_rule(gdn_rule rule,
                           const void *q, const void *k, const void *v,
                           const float *g, const float *beta,
                           float *state, float *o,
                           int N, int H, int d_k, int d_v,
                           gdn_dtype qkv_dtype, void *stream);

/*
 * gdn_decode_step_slots -- gdn_decode_step_rule with states kept in a pool
 * (continuous batching: one fixed-size state per live request; the Priming
 * article lists continuous batching among its serving plugin's features).
 *
 *   state_pool  [pool_size, H, d_k, d_v] fp32: sequence n reads and updates
 *               state_pool[slots[n]] in place
 *   slots       [N] int32, device memory.  A slot outside [0, pool_size)
 *               marks a padding entry: o[n] is written as zeros and no state
 *               is read or written.  Valid slots must be distinct (two
 *               sequences updating one slot race).
 * Other arguments as for gdn_decode_step.  Slot values are device data and
 * are not validated on the host beyond the rule above.
 * Errors: as gdn_decode_step_rule, plus GDN_ERR_NULL for slots == NULL
 * (N > 0) and GDN_ERR_SHAPE for pool_size < 0; GDN_ERR_ALIAS also covers o
 * or state_pool overlapping slots.
 */
GDN_API gdn_status gdn_decode_step_slots(gdn_rule rule,
                           const void *q, const void *k, const void *v,
                           const float *g, const float *beta,
                           float *state_pool, const int32_t *slots, int pool_size,
                           float *o,
                           int N, int H, int d_k, int d_v,
                           gdn_dtype qkv_dtype, void *stream);

/*
 * gdn_chunk_prefill_varlen -- prefill of S packed sequences of different
 * lengths in one call, states in a pool (continuous batching: the serving
 * runs batch whole prompts of any length next to each other; HyLo's vLLM
 * runtime keeps a fixed-size state per request, ftxj.github.io digest of
 * arXiv 2604.24715, Key Ideas).
 *
 *   q, k           [T_total, H, d_k] qkv_dtype (sequence s = tokens cu_seqlens[s] ..
 *                  cu_seqlens[s+1]-1)
 *   v              [T_total, H, d_v] qkv_dtype
 *   g, beta        [T_total, H] fp32
 *   cu_seqlens     HOST array [S + 1]: 0 = cu[0] <= cu[1] <= ... <= cu[S] = T_total
 *                  (empty sequences allowed)
 *   state_pool     [pool_size, H, d_k, d_v] fp32: sequence s starts from
 *                  state_pool[slot(s)] (or zeros, see has_initial) and its final
 *                  state is written back to the same slot
 *   slots          HOST array [S], or NULL for slot(s) = s (then pool_size >= S).
 *                  Slot -1: the sequence starts from zeros and its final state is
 *                  dropped; other slots must lie in [0, pool_size) and be distinct
 *   has_initial    HOST array [S], or NULL (all start from their stored state);
 *                  0 = start from zeros (a new request)
 *   o              [T_total, H, d_v] fp32, written
 *   workspace      at least gdn_chunk_prefill_varlen_workspace_size(...) bytes
 * Supported: the sizes and types of gdn_chunk_prefill, both rules.  bf16 q/k/v
 * with d_k, d_v in {64, 128} and chunk in {32, 64} run the MFMA chunk kernels,
 * long sequences split into pieces; fp32 q/k/v and the 16-wide shapes run the
 * fp32 VALU chunk kernel, one workgroup per sequence, head and 16 value
 * columns (as the dense call does for them).  The host arrays are read during the call only: the call turns
 * them into a table that one host-to-device copy on `stream` puts into the
 * workspace.  A graph recorded from that copy would keep a pointer to host
 * memory that is gone once the call returns, so the call refuses a stream that
 * is capturing (GDN_ERR_CAPTURE, before anything is queued); capture the
 * dense calls instead, or run this one eagerly between graph launches.
 * Errors: GDN_ERR_UNSUPPORTED (rule, dtype or sizes), GDN_ERR_SHAPE (bad
 * offsets, slots out of range, pool_size < S without slots), GDN_ERR_NULL,
 * GDN_ERR_ALIGN, GDN_ERR_ALIAS (repeated slot, overlapping buffers),
 * GDN_ERR_WORKSPACE, GDN_ERR_CAPTURE, GDN_ERR_HIP.
 */
GDN_API gdn_status gdn_chunk_prefill_varlen(gdn_rule rule,
                             const void *q, const void *k, const void *v,
                             const float *g, const float *beta,
                             const int32_t *cu_seqlens, int S, int T_total,
                             float *state_pool, int pool_size,
                             const int32_t *slots, const int32_t *has_initial,
                             float *o,
                             int H, int d_k, int d_v, int chunk,
                             gdn_dtype qkv_dtype,
                             void *workspace, size_t workspace_bytes,
                             void *stream);

/* Workspace bytes gdn_chunk_prefill_varlen needs for this batch (0 when the
 * arguments would be rejected). */
GDN_API size_t gdn_chunk_prefill_varlen_workspace_size(const int32_t *cu_seqlens, int S, int H,
                                               int d_k, int d_v, int chunk, gdn_dtype qkv_dtype);

/*
 * gdn_prepare -- the input preparation that feeds the mixer, fused into one
 * pass over the raw projections.  The GDN block carries a short convolution
 * and gate/decay parameters of its own (ftxj.github.io digest of arXiv
 * 2604.24715, Method: these start from random values when an attention layer
 * is converted); the pages give no formulas, and the library computes the
 * usual GDN input path.  Per token t, head h and channel c:
 *
 *   conv   c_t = w[c,0] x_{t-3} + w[c,1] x_{t-2} + w[c,2] x_{t-1} + w[c,3] x_t
 *          (causal, depthwise, width 4; inputs before t = 0 come from
 *          conv_state_in, or are zero)
 *   q, k   y = silu(c) = c sigmoid(c), then y / sqrt(sum_c y^2 + 1e-6) over
 *          the head's d_k channels
 *   v      silu(c)
 *   g      -A_h softplus(a_t + bias_h)   (A_h = 1, bias_h = 0 when absent)
 *   beta   sigmoid(b_t)
 *
 * so that q, k, v, g, beta go straight into gdn_chunk_prefill or
 * gdn_decode_step (decode = T = 1 with the carried convolution state).
 *
 *   xq, xk          [B, T, H, d_k] x_dtype (raw projections)
 *   xv              [B, T, H, d_v] x_dtype
 *   conv_weight     [H*(2 d_k + d_v), 4] fp32: rows are the q channels
 *                   (head-major), then k, then v; column 3 weighs the current
 *                   token
 *   a_raw, b_raw    [B, T, H] fp32 gate and write-strength logits
 *   decay_rate      [H] fp32 (A_h > 0) or NULL;  gate_bias [H] fp32 or NULL
 *   conv_state_in   [B, H*(2 d_k + d_v), 3] fp32, the three raw inputs before
 *                   t = 0 (oldest first, channels ordered as conv_weight), or
 *                   NULL for zeros
 *   conv_state_out  same shape, written with the last three raw inputs of
 *                   [conv_state_in, x] (so calls chain exactly), or NULL; may
 *                   be the same pointer as conv_state_in, not overlap it
 *                   otherwise
 *   q, k            [B, T, H, d_k] x_dtype, written (rounded once to bf16 for
 *                   GDN_BF16)
 *   v               [B, T, H, d_v] x_dtype, written
 *   g, beta         [B, T, H] fp32, written
 * T may be 0: only conv_state_out is written (a copy of the start state).
 * conv_weight is required even then.
 * Errors: GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_UNSUPPORTED (d_k, d_v not in
 * {16, 64, 128}, or dtype), GDN_ERR_ALIGN, GDN_ERR_ALIAS (an output
 * overlapping an input or another output, other than conv_state_out ==
 * conv_state_in), GDN_ERR_HIP.
 */
GDN_API gdn_status gdn_prepare(const void *xq, const void *xk, const void *xv,
                               const float *conv_weight,
                               const float *a_raw, const float *b_raw,
                               const float *decay_rate, const float *gate_bias,
                               const float *conv_state_in, float *conv_state_out,
                               void *q, void *k, void *v, float *g, float *beta,
                               int B, int T, int H, int d_k, int d_v,
                               gdn_dtype x_dtype, void *stream);

/*
 * gdn_prepare_chunk_prefill -- gdn_prepare followed by gdn_chunk_prefill_rule in
 * one pass: the chunk kernels read the raw projections and logits and apply
 * the short convolution, SiLU, the q/k L2 norm and the gate activations as
 * they load each chunk, so the prepared q, k, v, g, beta never go to device
 * memory (the GDN block's own convolution and gates sit right before the
 * mixer: ftxj.github.io digest of arXiv 2604.24715, Method).  The prepared
 * q, k, v are rounded once to bf16, as gdn_prepare stores them for GDN_BF16,
 * so the call computes what the two calls compute, up to the summation order
 * of each head's squared q and k norms.
 *
 *   rule                      GDN_RULE_GATED_DELTA or GDN_RULE_GATED_DECAY
 *   xq, xk, xv, conv_weight, a_raw, b_raw, decay_rate, gate_bias
 *                             as for gdn_prepare (x_dtype must be GDN_BF16)
 *   conv_state_in             [B, H*(2 d_k + d_v), 3] fp32 or NULL (zeros); it
 *                             holds raw inputs and is read through bf16
 *   conv_state_out            same shape or NULL; may be conv_state_in itself
 *   initial_state, o, final_state, chunk, workspace
 *                             as for gdn_chunk_prefill_rule (workspace of
 *                             gdn_prepare_chunk_prefill_workspace_size bytes;
 *                             chunk 32 or 64 = the longest chunk allowed, the
 *                             kernels run 32-token chunks)
 * Supported: GDN_BF16, d_k = d_v in {64, 128}.  T may be 0 (the states are
 * copied).
 * Errors: GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_UNSUPPORTED, GDN_ERR_ALIGN,
 * GDN_ERR_ALIAS (an output overlapping an input or another output, other than
 * final_state == initial_state and conv_state_out == conv_state_in),
 * GDN_ERR_WORKSPACE, GDN_ERR_HIP.
 */
GDN_API gdn_status gdn_prepare_chunk_prefill(gdn_rule rule,
                             const void *xq, const void *xk, const void *xv,
                             const float *conv_weight,
                             const float *a_raw, const float *b_raw,
                             const float *decay_rate, const float *gate_bias,
                             const float *conv_state_in, float *conv_state_out,
                             const float *initial_state, float *o, float *final_state,
                             int B, int T, int H, int d_k, int d_v, int chunk,
                             gdn_dtype x_dtype,
                             void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes gdn_prepare_chunk_prefill needs (0 if none or when the
 * arguments would be rejected). */
GDN_API size_t gdn_prepare_chunk_prefill_workspace_size(int B, int T, int H, int d_k, int d_v, int chunk,
                                                        gdn_dtype x_dtype);

/*
 * gdn_prepare_decode_step -- one generated token for each of N sequences, from
 * the raw projections: gdn_prepare with T = 1 and the convolution window
 * updated in place, then gdn_decode_step_rule on the prepared q, k, v, g, beta,
 * in one launch (the prepared values stay on chip, in fp32: unlike gdn_prepare's
 * outputs they are not rounded to bf16 for GDN_BF16).  The per-token loop of a serving
 * engine (the pages' hybrids decode with a fixed-size state per request;
 * ftxj.github.io digest of arXiv 2604.24715, Method: the converted GDN block keeps
 * a short convolution and gate/decay parameters of its own).
 *
 *   rule            GDN_RULE_GATED_DELTA or GDN_RULE_GATED_DECAY
 *   xq, xk          [N, H, d_k] x_dtype (raw projections of this token)
 *   xv              [N, H, d_v] x_dtype
 *   conv_weight     [H*(2 d_k + d_v), 4] fp32, as for gdn_prepare
 *   a_raw, b_raw    [N, H] fp32 gate and write-strength logits
 *   decay_rate      [H] fp32 or NULL (1);  gate_bias [H] fp32 or NULL (0)
 *   conv_state      [N, H*(2 d_k + d_v), 3] fp32, the three raw inputs before
 *                   this token (oldest first), read and updated in place
 *   state           [N, H, d_k, d_v] fp32, read and updated in place
 *   o               [N, H, d_v] fp32, written
 * Supported: d_k = d_v in {64, 128}.  N may be 0 (nothing is done).  For GDN_F32
 * the result equals gdn_prepare followed by gdn_decode_step_rule up to the
 * summation order of each head's squared q and k norms; for GDN_BF16 it is that of the
 * separate steps without the bf16 rounding of the prepared q, k, v.
 * Errors: GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_UNSUPPORTED (rule, dtype, or
 * d_k, d_v unequal or not 64 or 128), GDN_ERR_ALIGN, GDN_ERR_ALIAS (conv_state, state or
 * o overlapping an input or each other), GDN_ERR_HIP.
 */
GDN_API gdn_status gdn_prepare_decode_step(gdn_rule rule,
                                           const void *xq, const void *xk, const void *xv,
                                           const float *conv_weight,
                                           const float *a_raw, const float *b_raw,
                                           const float *decay_rate, const float *gate_bias,
                                           float *conv_state, float *state, float *o,
                                           int N, int H, int d_k, int d_v,
                                           gdn_dtype x_dtype, void *stream);

/*
 * gdn_prepare_varlen -- gdn_prepare over S packed sequences of different
 * lengths, convolution states in a pool (continuous batching; a decode step
 * is the case of S sequences of one token each).  The convolution restarts at
 * every sequence: the three inputs before a sequence's first token come from
 * conv_pool[slot(s)], or are zero.
 *
 *   xq, xk         [T_total, H, d_k] x_dtype;  xv [T_total, H, d_v]
 *   a_raw, b_raw   [T_total, H] fp32
 *   cu_seqlens     HOST array [S + 1], 0 = cu[0] <= ... <= cu[S] = T_total
 *   conv_pool      [pool_size, H*(2 d_k + d_v), 3] fp32: sequence s starts
 *                  from conv_pool[slot(s)] (zeros when has_initial[s] == 0) and
 *                  its new state (the last three raw inputs of [start state,
 *                  its tokens]) is written back to the same slot
 *   slots          HOST array [S] or NULL for slot(s) = s (then pool_size >=
 *                  S); -1 = start from zeros, new state dropped; other slots
 *                  distinct and in [0, pool_size)
 *   has_initial    HOST array [S] or NULL (all start from their slot)
 *   q, k, v, g, beta   written, packed like the inputs
 *   workspace      device scratch of gdn_prepare_varlen_workspace_size(S) bytes
 * Other arguments and the computation as gdn_prepare.  The host arrays are
 * read during the call only, through one host-to-device copy into the
 * workspace; as for gdn_chunk_prefill_varlen, a stream that is capturing a
 * graph is refused with GDN_ERR_CAPTURE before anything is queued (a decode
 * loop that is captured uses gdn_prepare or gdn_prepare_decode_step).
 * Errors: as gdn_prepare, plus GDN_ERR_SHAPE (bad offsets or slots),
 * GDN_ERR_ALIAS (a repeated slot), GDN_ERR_WORKSPACE, GDN_ERR_CAPTURE.
 */
GDN_API gdn_status gdn_prepare_varlen(const void *xq, const void *xk, const void *xv,
                               const float *conv_weight,
                               const float *a_raw, const float *b_raw,
                               const float *decay_rate, const float *gate_bias,
                               const int32_t *cu_seqlens, int S, int T_total,
                               float *conv_pool, int pool_size,
                               const int32_t *slots, const int32_t *has_initial,
                               void *q, void *k, void *v, float *g, float *beta,
                               int H, int d_k, int d_v, gdn_dtype x_dtype,
                               void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes gdn_prepare_varlen needs for S sequences. */
GDN_API size_t gdn_prepare_varlen_workspace_size(int S);

/*
 * gdn_chunk_backward -- gradients of gdn_chunk_prefill_rule (training of the GDN
 * layers: the converted blocks are trained by layer-wise distillation and then
 * end to end, ftxj.github.io digest of arXiv 2604.24715, Method; kwkr.cn digest
 * of HyLo-Llama-8MLA8GDN-8K-SFT, training stages).
 *
 * For the loss L = sum_t <d_o_t, o_t> + <d_final_state, S_T> of one prefill
 * call with the same inputs, writes dL/dq, dL/dk, dL/dv, dL/dg, dL/dbeta and
 * dL/dS_0.  The forward pass is recomputed inside the call (nothing has to be
 * kept from it), in chunks of 32 tokens.
 *
 *   q, k, v, g, beta, initial_state   as for gdn_chunk_prefill (initial_state
 *                    NULL = zeros)
 *   d_o              [B, T, H, d_v] fp32
 *   d_final_state    [B, H, d_k, d_v] fp32, or NULL for zero
 *   dq, dk           [B, T, H, d_k] fp32, written
 *   dv               [B, T, H, d_v] fp32, written
 *   dg, dbeta        [B, T, H] fp32, written
 *   d_initial_state  [B, H, d_k, d_v] fp32, written, or NULL (not computed)
 *   workspace        at least gdn_chunk_backward_workspace_size(...) bytes
 * Supported: qkv_dtype GDN_BF16 or GDN_F32, d_k = d_v in {64, 128}; both
 * rules.  T may be 0 (then d_initial_state = d_final_state, or zeros).  For
 * 128-wide heads the workspace also holds 256 slots of the gradient pass's
 * larger per-chunk matrices (about 47 MB), which do not fit on chip.
 * Errors: GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_UNSUPPORTED, GDN_ERR_ALIGN,
 * GDN_ERR_ALIAS (an output overlapping an input, another output or the
 * workspace), GDN_ERR_WORKSPACE, GDN_ERR_HIP.
 */
GDN_API gdn_status gdn_chunk_backward(gdn_rule rule,
                             const void *q, const void *k, const void *v,
                             const float *g, const float *beta,
                             const float *initial_state,
                             const float *d_o, const float *d_final_state,
                             float *dq, float *dk, float *dv, float *dg, float *dbeta,
                             float *d_initial_state,
                             int B, int T, int H, int d_k, int d_v,
                             gdn_dtype qkv_dtype,
                             void *workspace, size_t workspace_bytes,
                             void *stream);

/* Workspace bytes gdn_chunk_backward needs (0 when the arguments would be
 * rejected). */
GDN_API size_t gdn_chunk_backward_workspace_size(int B, int T, int H, int d_k, int d_v,
                                                 gdn_dtype qkv_dtype);

/* Static, human-readable text for a status code (never NULL). */
GDN_API const char *gdn_status_string(gdn_status status);

/* GDN_ABI_VERSION of the built library. */
GDN_API int gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
