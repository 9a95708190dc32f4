/*
 * blt.h -- C ABI of the MI355X (gfx950) Fast-BLT local byte decoder step.
 *
 * The library runs the local byte decoder of a Byte Latent Transformer as
 * described in the pytorch.kr Fast-BLT summary ("Fast Byte Latent
 * Transformer (Fast-BLT) 연구 소개"): per layer a cross-attention read of the
 * global model's patch latents added to the residual stream, then a decoder
 * transformer layer (section on the BLT architecture, the layer equation);
 * the BLT-D block of [MASK] positions attended bidirectionally over a causal
 * clean prefix (section "BLT-D attention mask"); confidence-threshold
 * unmasking (section "block unmasking strategies"); and the greedy
 * exact-match verification shared by BLT-S and BLT-DV (section "BLT-S and
 * BLT-DV").  The parameter-load bandwidth proxy follows the wangzhan123.com
 * Fast-BLT article, section six.
 *
 * Conventions for every entry point:
 *  - "device" pointers are HIP device memory owned by the caller (e.g.
 *    PyTorch tensors); "host" pointers are ordinary host memory, read before
 *    the call returns.  The library never frees caller memory.
 *  - Calls that launch GPU work are asynchronous on the stream given to
 *    blt_create; their device outputs are valid once that stream has
 *    synchronised.  A context is not thread-safe: one context per stream.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    rejected call enqueues nothing.  Errors never abort or throw across the
 *    ABI: the return code says what failed and blt_last_error() gives text.
 *  - Matrices are row-major [out][in] (the weight of y = W x has W[o][i] at
 *    o * in + i), in the context's dtype: float32 (BLT_F32) or bfloat16
 *    (BLT_BF16).  Norm gains are in the same dtype.
 *  - Token ids are 0..255 for bytes and 256 for [MASK].
 *  - Per-sequence host arrays are indexed by the position b of the sequence
 *    in the call (0..batch-1).  Per-sequence DEVICE arrays are indexed by the
 *    sequence's state slot, so a caller can keep one buffer per slot while
 *    sequences join or leave passes: e.g. block_tok[slot*B + j].  They must
 *    hold max_batch sequences.
 */
#ifndef BLT_H
#define BLT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BLT_OK = 0,
  BLT_EINVAL = -1,     /* bad argument: NULL, out of range, inconsistent sizes */
  BLT_ECAPACITY = -2,  /* a size exceeds a capacity fixed in blt_config */
  BLT_EDTYPE = -3,     /* unsupported dtype */
  BLT_EHIP = -4,       /* a HIP runtime call failed (message in blt_last_error) */
  BLT_ENOTIMPL = -5    /* a combination of options this library does not implement */
} blt_status;

typedef enum { BLT_F32 = 0, BLT_BF16 = 1 } blt_dtype;

/* How a decode step commits masked block positions (pytorch.kr summary,
 * "block unmasking strategies"): THRESHOLD commits every masked position
 * whose confidence (largest byte probability) is > alpha, and the single most
 * confident one (lowest position on ties) when none is; ONE_STEP commits
 * every masked position in one pass (the one-step diffusion draft of BLT-DV);
 * ENTROPY (entropy-bounded, EB) ranks the masked positions by the entropy in
 * nats of their byte distribution (ties by position) and commits them in rank
 * order while the running sum of their entropies is <= alpha (the bound
 * gamma), at least the first one.  Committed positions take their greedy byte. */
typedef enum {
  BLT_UNMASK_THRESHOLD = 0,
  BLT_UNMASK_ONE_STEP = 1,
  BLT_UNMASK_ENTROPY = 2
} blt_unmask;

/* Self-attention inside the block: bidirectional (diffusion mode) or causal
 * (the same weights run autoregressively). */
typedef enum { BLT_BLOCK_BIDIR = 0, BLT_BLOCK_CAUSAL = 1 } blt_block_mask;

typedef struct {
  int32_t n_layers, d_model, n_heads, d_ffn;
  int32_t vocab;        /* must be 257: 256 bytes + [MASK] */
  int32_t d_global;     /* width of the global model's latents */
  int32_t max_batch;    /* sequence slots held by a state */
  int32_t max_ctx;      /* KV rows per sequence (prefix + one block) */
  int32_t max_latents;  /* latent (patch) slots per sequence */
  int32_t max_rows;     /* rows of one decoder pass, summed over its sequences */
  int32_t max_block;    /* largest block size B (and verify window) */
  blt_dtype dtype;
  float rope_theta;     /* RoPE base, e.g. 10000 */
  float rms_eps;        /* RMSNorm epsilon, e.g. 1e-5 */
} blt_config;

/* Per-layer decoder weights (device).  Cross-attention reads exactly one
 * latent per row, so its softmax is identically 1 and only the value and
 * output projections reach the output; the query/key projections are not
 * taken. */
typedef struct {
  const void *wv_c;    /* [d][d]  cross-attention value projection        */
  const void *wo_c;    /* [d][d]  cross-attention output projection       */
  const void *wqkv;    /* [3d][d] self-attention q (rows 0..d-1), k, v    */
  const void *wo;      /* [d][d]  self-attention output projection        */
  const void *g_attn;  /* [d]     RMSNorm gain before self-attention      */
  const void *g_ffn;   /* [d]     RMSNorm gain before the FFN             */
  const void *w1;      /* [F][d]  FFN up projection (SiLU after it)       */
  const void *w2;      /* [d][F]  FFN down projection                     */
} blt_layer_weights;

typedef struct {
  const void *embed;   /* [257][d] byte + [MASK] embedding (device)      */
  const void *w_lat;   /* [d][d_global] latent projection (device)       */
  const void *w_out;   /* [257][d] byte head (device)                    */
  const void *g_out;   /* [d] final RMSNorm gain (device)                */
  const blt_layer_weights *layers; /* host array of n_layers entries    */
} blt_weights;

/* Caller-owned decode state (device), sized by blt_state_size:
 *   kv    : keys (after RoPE) and values of cached rows, per
 *           [max_batch][n_layers] a K plane [n_heads][ctx/32][d_h/32][32][32]
 *           (tiles of 32 positions, each holding the tile's keys one
 *           32-dimension slice at a time) and a V plane
 *           [n_heads][ctx/32][d_h][32] (V transposed in tiles of 32
 *           positions), dtype, with d_h = d_model/n_heads and ctx = max_ctx
 *           rounded up to a multiple of 128;
 *   cross : per-latent cross-attention contributions W_o^c W_v^c W_lat o_m,
 *           [max_batch][max_latents][n_layers][d_model], float32.
 * Rows beyond a sequence's committed length hold scratch (the current
 * block's keys and values) and are overwritten by later calls. */
typedef struct {
  void *kv;
  void *cross;
} blt_state;

typedef struct blt_ctx blt_ctx; /* opaque, library-owned */

/* Bytes the caller must allocate for blt_state.kv and blt_state.cross. */
blt_status blt_state_size(const blt_config *cfg, size_t *kv_bytes, size_t *cross_bytes);

/* Create a context bound to `hip_stream` (a hipStream_t, 0 = null stream)
 * and to the weights, which must stay alive and unchanged while the context
 * lives.  Allocates the library's workspace on the current device; for a
 * bfloat16 context with max_rows >= 16 that includes a copy of the
 * projection weights (every layer's W_qkv, W_o, W1, W2, the byte head,
 * W_lat and the combined cross matrices, about 2 bytes per decoder
 * parameter) in the fragment order that the matrix-core GEMM of passes of
 * 16 rows or more streams, made here from the caller's weights. */
blt_status blt_create(const blt_config *cfg, const blt_weights *w, void *hip_stream,
                      blt_ctx **out);
blt_status blt_destroy(blt_ctx *ctx);
const char *blt_last_error(const blt_ctx *ctx);

/* Make latents available to the decoder (one encoder/global pass delivers
 * them).  pytorch.kr summary, "BLT-D attention mask": every decoder row
 * reads exactly one latent (a clean byte o_{p(i)-1}, the last byte of a
 * patch o_{p(i)}, block bytes o_M), so the cross-attention softmax over its
 * single key is 1 and the read is the value path alone; it is computed here
 * once per latent for every layer (the layer equation of "BLT
 * architecture": B_l = D_{l-1} + W_o softmax(.) V).
 * For entry i: latent vector o = table + (slot[i] * seq_stride +
 * idx[i]) * d_global (device, dtype), written as latent idx[i] of sequence
 * slot[i]: cross[slot][idx][l] = W_o^c_l W_v^c_l W_lat o for every layer l.
 * slot, idx: host arrays of n entries (any n: processed max_rows at a time).
 * Errors: BLT_EINVAL for a NULL argument or a slot outside 0..max_batch-1,
 * BLT_ECAPACITY for an index outside 0..max_latents-1; nothing is enqueued
 * then. */
blt_status blt_latents_put(blt_ctx *ctx, const blt_state *st, int32_t n, const int32_t *slot,
                           const int32_t *idx, const void *table, int64_t seq_stride);

/* One decoder pass over clean rows only (prefill, autoregressive steps,
 * BLT-S drafts and the causal verification pass of BLT-S / BLT-DV).
 * pytorch.kr summary, "BLT-D inference": the clean prefix is cached, so a
 * pass computes only rows not cached yet (prefix caching); "BLT-S and
 * BLT-DV": verification runs the full model causally over the draft once,
 * which is this call over rows l..l+r; "BLT-S": each draft byte is one such
 * pass of one row.
 * For sequence b of the batch: rows start_pos[b] .. start_pos[b]+n_rows[b]-1
 * of state slot slot[b] are computed causally over the cached prefix
 * [0, start_pos[b]) and each other, and their keys/values are written to the
 * cache (a start_pos below the previous length overwrites: rollback).
 * start_pos[b] may not exceed the clean rows written so far for that slot
 * of that state (by this call or blt_decode_block_step's appended rows, on
 * this context; a state starts empty): rows past them hold no keys, and the
 * call returns BLT_EINVAL.  The count is kept per state kv buffer address.
 * Row j of sequence b has token bytes[b*n_max+j] (host) -- or, if `bytes` is
 * NULL, tokens_dev[slot[b]*n_max+j] (device int32, e.g. the argmax of a
 * previous pass) -- and reads latent lat_idx[b*n_max+j] (host).
 * Outputs (device, nullable): argmax_out[slot[b]*n_max+j] (greedy byte of the
 * row: lowest id among the largest of logits 0..255), conf_out (its
 * probability), logits_out[(slot[b]*n_max+j)*257 + v] (float32).  At most
 * max_rows rows in total; a sequence with n_rows[b] = 0 is skipped.
 * Self-attention of a bfloat16 sequence with at least 64 rows in the call
 * runs as one causal (flash) pass over its keys, tiles of 128 rows at a
 * time; shorter ones take the split-K decode kernel.  Either way a row's
 * result depends only on its own inputs and on which of the two kernels its
 * sequence took (the two agree to rounding).
 * sampling (nullable; see blt_decode_block_step): argmax_out then receives
 * each row's drawn byte (row j of sequence b draws n = draw[b]*64 + j; at
 * most 64 rows per sequence) and conf_out the model probability of it. */
typedef struct {
  float temperature;
  float top_p;
  uint64_t seed;
} blt_sampling;
blt_status blt_kv_append(blt_ctx *ctx, const blt_state *st, int32_t batch, const int32_t *slot,
                         const int32_t *start_pos, const int32_t *n_rows, int32_t n_max,
                         const uint8_t *bytes, const int32_t *tokens_dev, const int32_t *lat_idx,
                         int32_t *argmax_out, float *conf_out, float *logits_out,
                         const blt_sampling *sampling, const int32_t *draw);

/* blt_kv_append for callers that cannot allocate device memory at the time
 * of the call (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same pass, with the same arguments, results
 * and validation, but its working buffers (residual stream, queries,
 * attention partials, activations, logits, decisions and the pass's row and
 * sequence descriptors) live in one static device array of 32 MiB that the
 * library holds on each GPU until the process ends, instead of the
 * context's workspace.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine) and never captures a graph; the context must
 * already exist (blt_create allocates).  Limits, checked before anything is
 * enqueued: at most 15 rows in the call (BLT_ECAPACITY), and the pass's
 * buffers (about rows x (n_heads x ceil(max_ctx/128) x (d_model/n_heads+2) x
 * 4 + 7 x d_model x 4 + 257 x 4 + max(d_model, d_ffn, d_global) x 4) bytes)
 * within the 32 MiB (BLT_ECAPACITY).  Every call on one GPU, from any
 * context, shares that GPU's array and nothing in it needs to start at zero:
 * calls that overlap in time on one GPU (different streams or threads) race
 * and must be serialised by the caller. */
blt_status blt_kv_append_noalloc(blt_ctx *ctx, const blt_state *st, int32_t batch,
                                 const int32_t *slot, const int32_t *start_pos,
                                 const int32_t *n_rows, int32_t n_max, const uint8_t *bytes,
                                 const int32_t *tokens_dev, const int32_t *lat_idx,
                                 int32_t *argmax_out, float *conf_out, float *logits_out,
                                 const blt_sampling *sampling, const int32_t *draw);

/* One BLT-D decoder pass (pytorch.kr summary, "BLT-D inference" and
 * "BLT-D attention mask").  For sequence b: n_append[b] clean rows at
 * start_pos[b].. (tokens append_bytes[b*n_append_max+j], latents
 * append_lat[...], host) are appended to the cache as in blt_kv_append; then
 * B block rows at the following positions (start_pos[b] at most the rows
 * written so far, as in blt_kv_append), tokens block_tok[slot[b]*B+j]
 * (device int32, 256 = [MASK]) and latent block_lat[b] (host), read every
 * cached row and every block row (BIDIR) or the block rows up to themselves
 * (CAUSAL).  Block rows are not kept as clean rows (their cache rows are
 * scratch).  Then every still-masked block position is decided by `mode` /
 * `alpha` (a finite threshold; for ENTROPY a bound >= 0, +inf allowed) and
 * block_tok is updated in place; masked_left[slot[b]] (device) receives the
 * number of [MASK]s left.  Optional device outputs for block rows:
 * argmax_out/conf_out [slot[b]*B+j] (conf_out: the row's confidence, or its
 * entropy in nats under ENTROPY), logits_out [(slot[b]*B+j)*257+v].
 *
 * Sampling (pytorch.kr summary, "block unmasking strategies": EB sampling
 * combined with top-p sampling).  sampling == NULL: each position takes its
 * greedy byte.  Otherwise each block position draws its byte from the
 * nucleus of softmax(z / temperature) over bytes 0..255 (bytes ranked by
 * probability, ties by byte id; the nucleus is the shortest prefix of that
 * ranking whose mass reaches top_p; with c = u * its mass, the byte whose
 * interval of the nucleus holds c), where u in [0, 1) is the top 24 bits of
 * output n + 1 of SplitMix64 started from state seed + slot[b], over 2^24,
 * and n = draw[b] * 64 + j for block position j (draw: host, >= 0, one
 * value per sequence, e.g. its count of sampling passes so far).  The
 * position's confidence and entropy stay those of the model's distribution
 * (temperature 1): the probability of the drawn byte, and the entropy of
 * softmax(z).  Requires a bfloat16 or float32 context alike; temperature
 * > 0 and finite, 0 < top_p <= 1, draw[b] * 64 + 63 < 2^31. */
blt_status blt_decode_block_step(blt_ctx *ctx, const blt_state *st, int32_t batch,
                                 const int32_t *slot, const int32_t *start_pos,
                                 const int32_t *n_append, int32_t n_append_max,
                                 const uint8_t *append_bytes, const int32_t *append_lat,
                                 int32_t *block_tok, int32_t B, const int32_t *block_lat,
                                 float alpha, blt_unmask mode, blt_block_mask mask,
                                 int32_t *argmax_out, float *conf_out, float *logits_out,
                                 int32_t *masked_left, const blt_sampling *sampling,
                                 const int32_t *draw);

/* Greedy exact-match verification (pytorch.kr summary, "BLT-S and BLT-DV").
 * For sequence slot s = slot[b] (slot NULL: s = b): draft[s*ld_draft+j]
 * (device int32, j < r) holds the draft bytes x'_{l+1..l+r}; pred[s*ld_pred+j]
 * (device int32, j <= r) the greedy bytes y_l..y_{l+r} of the causal pass over
 * rows l..l+r.  accept_len[s] = number of leading j with draft[j] == pred[j];
 * next_byte[s] = pred[accept_len[s]]: the correction at the first mismatch,
 * or the free byte when the whole draft matched (device outputs). */
blt_status blt_verify_accept(blt_ctx *ctx, int32_t batch, const int32_t *slot, int32_t r,
                             const int32_t *draft, int32_t ld_draft, const int32_t *pred,
                             int32_t ld_pred, int32_t *accept_len, int32_t *next_byte);

/* Verification of sampled drafts by rejection sampling (pytorch.kr summary,
 * "BLT-S and BLT-DV": sampling at temperature > 0 extends the verification
 * with rejection sampling; the standard speculative-sampling rule is taken).
 * For sequence slot s = slot[b] (slot NULL: s = b): draft[s*ld_draft+j]
 * (device int32, j < r) the draft bytes; zq[(s*ld_q+j)*257+v] (device f32)
 * the logits draft byte j was drawn from; zp[(s*ld_p+j)*257+v] (j <= r) the
 * logits of causal verify row l+j.  With q_j, p_j the distributions the
 * top-p sampler draws from (`sampling`), draft byte j is kept iff
 * u_j * q_j(x) < p_j(x); at the first rejection the byte appended is drawn
 * from max(0, p_j - q_j) renormalised (bytes in id order: the first whose
 * cumulative mass exceeds u' times the total); if all r are kept it is drawn
 * from p_r as the top-p sampler draws.  u_j = draw n = draw[b]*64 + j, u' =
 * draw[b]*64 + r of the stream seed + s (as in blt_decode_block_step).
 * Outputs accept_len[s], next_byte[s] (device int32).  r < 64. */
blt_status blt_verify_sample(blt_ctx *ctx, int32_t batch, const int32_t *slot, int32_t r,
                             const int32_t *draft, int32_t ld_draft, const float *zq, int32_t ld_q,
                             const float *zp, int32_t ld_p, const blt_sampling *sampling,
                             const int32_t *draw, int32_t *accept_len, int32_t *next_byte);

/* Kernel timing with HIP events on the context's stream (profiling aid).
 * While a family is enabled, every launch of it is stamped by its own
 * dispatch (start and end events).  blt_profile_read synchronises the stream
 * and returns the launches timed so far, their summed duration and the
 * algorithmic work they must do, in `bytes`:
 *  - BLT_PROF_ATTENTION, the split-K self-attention kernel of decode passes:
 *    bytes of the key and value rows of the cache its sequences read (sum over
 *    sequences of kmax * 2 * d_model * element size; kmax = the largest key
 *    count of the sequence's rows);
 *  - BLT_PROF_ATTENTION_CAUSAL, the causal (flash) self-attention kernel of
 *    long clean-row passes (prefill): floating-point operations, sum over its
 *    rows of 4 * d_model * kend (the multiply-adds of QK^T and PV);
 *  - BLT_PROF_GEMV_MFMA / BLT_PROF_GEMV, the projections of passes of fewer
 *    than 16 rows on the MFMA GEMV (bfloat16, K <= 1536, N >= 2048: QKV, W1)
 *    and on the dot-product GEMV (the others): bytes, N*K weights + R*K
 *    activations (float32 when the RMSNorm prologue reads the residual) +
 *    R*N outputs (+ R*N float32 residual reads of a residual epilogue), in the
 *    context's element size;
 *  - BLT_PROF_GEMM, the MFMA GEMM of passes of 16 or more rows: floating-point
 *    operations, 2*N*K*R.
 * Only decoder passes are timed (not blt_latents_put).  reset != 0 clears
 * the totals.  Enabling or disabling collects pending events first. */
typedef enum {
  BLT_PROF_OFF = 0,
  BLT_PROF_ATTENTION = 1,
  BLT_PROF_ATTENTION_CAUSAL = 2,
  BLT_PROF_GEMV_MFMA = 3,
  BLT_PROF_GEMV = 4,
  BLT_PROF_GEMM = 5
} blt_prof_family;
blt_status blt_profile_enable(blt_ctx *ctx, int32_t family);
blt_status blt_profile_read(blt_ctx *ctx, uint64_t *launches, double *total_ms, double *bytes,
                            int32_t reset);

/* Replay of decoder passes from HIP graphs (off by default: where the host
 * waits for each pass's result before enqueueing the next, the graph launch
 * latency at the head of a pass outweighs the launch gaps it removes).  The kernel
 * sequence of a pass depends only on its shape (rows, sequences, the
 * attention chunk grid in buckets of 4 chunks) and on its scalar and
 * pointer arguments; the per-pass row and sequence descriptors are staged in
 * device buffers before it.  The first pass of a shape is launched directly,
 * the second is captured into a graph on a library-owned stream and every
 * later one replays that graph on the context's stream; results are the same
 * either way.  Passes while a profiling family is enabled are never replayed.
 * enable = 0 launches every pass directly and frees the cached graphs. */
blt_status blt_graphs_enable(blt_ctx *ctx, int32_t enable);

/* Keys per split-K self-attention workgroup, in chunks of 128 keys.
 * chunks = 0 (the default) lets each pass choose from its shape: a pass
 * whose chunks number at most 1024 (summed over its sequences and heads)
 * takes one chunk per workgroup; in larger ones, when sequences times heads
 * reach 256, one eight-wave workgroup per (sequence, head) takes all of its
 * keys and writes the output (no merge of partial results); otherwise the
 * workgroups of a (sequence, head) share its chunks evenly, as many as give
 * about 512 workgroups in the pass.  chunks >= 1 forces that count (on
 * four-wave workgroups).  Counts above 1 apply only to bfloat16
 * contexts with d_model / n_heads <= 64 and to passes whose split-K
 * sequences have at most 16 rows; other passes take 1.  The count changes
 * the rounding of the softmax sums, not what is computed.  BLT_EINVAL for a
 * negative count. */
blt_status blt_attention_chunks(blt_ctx *ctx, int32_t chunks);

/* Form of the causal (prefill) self-attention kernel, which takes a bf16
 * sequence's clean rows of a pass once it has at least 64 of them.  Its
 * workgroups each take a pair of 128-row tiles of one (sequence, head);
 * groups = 0 (the default) lets each pass choose from its grid: with up to
 * 2048 workgroups, eight waves in two key groups that walk alternate key
 * tiles and join their softmax states at the end; with more, four waves
 * that walk every key tile.  groups = 1 or 2 forces that form.  The form
 * changes the rounding of the softmax sums, not what is computed.
 * BLT_EINVAL for other values. */
blt_status blt_flash_key_groups(blt_ctx *ctx, int32_t groups);

/* Kernel of the bfloat16 projections of passes of 16 rows or more (the MFMA
 * GEMM path; passes of fewer rows use the GEMVs).  Two kernels: one stages
 * both operand tiles through LDS (64x64 to 128x128 tiles); the other takes
 * 64x64 tiles whose weights stream from a fragment-ordered copy straight
 * into the matrix-core operands of the one wave that uses them, with only
 * the activations staged through LDS.  form = 0 (the default) chooses by
 * shape: the weight-streaming kernel for products of at most 1024 rows
 * where the staged-tile kernel would take 128x128 tiles but fewer than 200
 * workgroups, else the staged-tile kernel.  form = 1 forces the staged-tile
 * kernel, form = 2 the weight-streaming kernel wherever it applies (K a
 * multiple of 256).  The form changes the rounding of the sums (tile and K
 * split), not what is computed.  BLT_EINVAL for other values. */
blt_status blt_gemm_form(blt_ctx *ctx, int32_t form);

/* Bandwidth proxy (wangzhan123.com Fast-BLT article, section six):
 * bytes_total = bytes_per_param * (n_dec * p_dec + n_encglob * (p_enc + p_glob)),
 * gb_per_seq = bytes_total / 1e9 / n_seq.  Host-only, exact integers;
 * BLT_EINVAL on NULL, n_seq = 0 or 64-bit overflow. */
typedef struct { uint64_t n_dec, n_encglob, n_seq; } blt_counts;
typedef struct { uint64_t p_dec, p_enc, p_glob; uint32_t bytes_per_param; } blt_params;
blt_status blt_bw_model(const blt_counts *c, const blt_params *p, uint64_t *bytes_total,
                        double *gb_per_seq);

/* ------------------------------------------------------------------------
 * Decode sessions: native host drivers of the four decoding policies over
 * the calls above (greedy BLT, BLT-D, BLT-S, BLT-DV), with the pass
 * counters of the efficiency metrics (decoder passes and encoder/global
 * passes per output sequence).  The encoder and global model are not part of
 * this library: an encoder/global pass makes the requested latents of the
 * caller's latent table available (blt_latents_put) and is counted.
 * Patch boundaries of generated bytes come from a seeded stand-in rule: a
 * new patch starts after byte x_i iff the current patch holds 8 bytes or the
 * (1 + 256*x_{i-1} + x_i)-th SplitMix64 output from the sequence's salt is 0
 * modulo 4.
 * ---------------------------------------------------------------------- */
typedef enum {
  BLT_POLICY_GREEDY = 0,
  BLT_POLICY_BLT_D = 1,
  BLT_POLICY_BLT_S = 2,
  BLT_POLICY_BLT_DV = 3
} blt_policy;

typedef struct {
  blt_policy policy;
  int32_t block;            /* B (BLT-D, BLT-DV) or draft window k (BLT-S) */
  float alpha;              /* confidence threshold, or the entropy bound for ENTROPY */
  blt_unmask unmask;
  blt_block_mask block_mask;
  int32_t n_gen;            /* bytes to generate per sequence */
  /* Sampling (temperature > 0; 0 = greedy): bytes of sequence b are drawn
   * as in blt_decode_block_step with stream seed + b, pass d of the
   * sequence's generation (its decoder passes so far) drawing n = d*64 + j.
   * Greedy BLT: each pass draws the next byte.  BLT-D: block positions draw
   * their bytes.  BLT-S: draft bytes are drawn and the draft is verified by
   * blt_verify_sample (the verify pass is pass d).  BLT-DV: the block draft
   * (any unmask rule) is verified the same way, each draft byte against the
   * distribution of the pass that committed it. */
  float temperature;
  float top_p;
  uint64_t seed;
} blt_policy_args;

typedef struct blt_session blt_session;

/* batch sequences in slots 0..batch-1.  Host inputs per sequence b:
 * prompts[b] (prompt_len[b] bytes), patch_lens[b] (n_patches[b] patch
 * lengths summing to prompt_len[b]; the prompt's last patch is complete),
 * salt[b].  latent_table: device [batch][n_latents][d_global] (dtype) holding
 * latent m of sequence b at (b * n_latents + m) * d_global. */
blt_status blt_session_create(blt_ctx *ctx, const blt_state *st, int32_t batch,
                              const uint8_t *const *prompts, const int32_t *prompt_len,
                              const int32_t *const *patch_lens, const int32_t *n_patches,
                              const uint64_t *salt, const void *latent_table, int32_t n_latents,
                              blt_session **out);
/* Prefill: latents of the prompt's patches and the cache of prompt rows
 * 0..N-2 (the last prompt byte is the first row the policy computes).
 * Counted apart from the decode counters. */
blt_status blt_session_prefill(blt_session *s);
/* Run a policy from the prefilled state until n_gen bytes per sequence are
 * committed.  May be called again: each call restarts from the prompt. */
blt_status blt_session_generate(blt_session *s, const blt_policy_args *args);
/* Generated bytes of sequence b (up to cap), decoder and encoder/global
 * passes of the last generate call, and the accepted draft lengths summed
 * over verification rounds (BLT-S, BLT-DV). */
blt_status blt_session_result(const blt_session *s, int32_t b, uint8_t *out, int32_t cap,
                              int32_t *n_out, uint64_t *n_dec, uint64_t *n_encglob,
                              uint64_t *n_rounds, uint64_t *n_accepted);
/* Device-resident BLT-D blocks (pytorch.kr summary, "BLT-D inference"):
 * with mode 1, a BLT-D generation (greedy, any unmask rule, either block
 * mask) runs its first block as above and every later block with no host
 * round trip.  On the device, per block: the stand-in patcher's state and
 * the committed bytes decide the block's encoder/global pass (the latents of
 * patches up to the last, possibly truncated, one get their cross vectors;
 * the pass is counted) and its first decoder pass (the last B+1 committed
 * bytes as clean rows with their latents, the one before the newest
 * recomputed with its final latent, then the B [MASK] rows); B decoder
 * passes follow, each counted for a sequence only while its block still has
 * a [MASK] (a pass in which no sequence has one does no work); the filled
 * block is committed and the patcher runs over its bytes.  The block's
 * launches are captured once as a HIP graph (when graphs are enabled) and
 * replayed; the bytes and counters are read back at the end.  Where every
 * pass has fewer than 16 rows (the GEMV path, whose row results do not
 * depend on the pass) results and counts equal the host-driven path's; with
 * 16 rows or more the first pass of a block holds other rows than the host
 * driver's, the matrix-core GEMMs tile and round differently, and bytes may
 * differ where two bytes tie within the rounding.  A device-resident block
 * always launches its B passes (those after the block is filled return at
 * once but are still launched), so it pays off when every pass is needed
 * and passes are short.  Mode 2 chooses: for one sequence, the first blocks
 * run host-driven, and if each of the four after the first took all B
 * decoder passes (one byte committed per pass), the rest of the generation
 * runs device-resident; else, and for more sequences, host-driven.  In
 * blocks run device-resident by mode 2, the GEMVs and the split-K attention
 * test the gate only before their first store (a closed pass still loads
 * and computes, and stores nothing), which saves the gate's round trip
 * where every pass has work.  Mode 3: device-resident after the first
 * block, like mode 1, with that late test (for callers whose passes all
 * have work).  Mode 0 (the default): host-driven blocks.  Sampled
 * generation and the other policies are unaffected.  BLT_EINVAL for other
 * modes. */
blt_status blt_session_device_blocks(blt_session *s, int32_t mode);
blt_status blt_session_destroy(blt_session *s);

#ifdef __cplusplus
}
#endif
#endif /* BLT_H */
