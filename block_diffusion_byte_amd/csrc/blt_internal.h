// Internal declarations shared by the HIP kernels (kernels.hip) and the
// C-ABI host code (blt_api.cpp, session.cpp).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/blt.h"

namespace blt {

constexpr int kVocab = 257;
constexpr int kMask = 256;
constexpr int kAttnChunk = 128;     // keys per split-K attention chunk (aligned to absolute positions)
constexpr int kMaxChunks = 128;     // chunks per sequence the fused merge handles (max_ctx <= 16384)
constexpr int kMaxBlock = 64;       // block rows per sequence handled by one wave in unmask
constexpr int kGemvRows = 16;       // rows per GEMV row block; passes with R >= 16 use MFMA (bf16)
constexpr int kFlashRows = 128;     // rows per workgroup of the causal (flash) attention kernel
constexpr int kFlashMinRows = 64;   // a bf16 sequence with this many clean rows in a pass takes it

// Token source codes in RowDesc::tok (values >= 0 are literal token ids).
constexpr int kTokFromBlock = -1;   // block_tok[blk]
constexpr int kTokFromDev = -2;     // tokens_dev[blk]

// One row of a decoder pass.
struct RowDesc {
  int32_t slot;   // state slot (sequence)
  int32_t pos;    // absolute byte position (RoPE and KV row)
  int32_t tok;    // token id or a kTokFrom* code
  int32_t blk;    // index into block_tok / tokens_dev for the kTokFrom* codes
  int32_t lat;    // latent index read by the cross-attention
  int32_t kend;   // the row attends cache rows [0, kend)
  int32_t oidx;   // index into the caller's per-row outputs, -1 for none
  int32_t attn_flash;  // 1: its sequence takes the causal kernel (no partials to merge)
  int32_t ctr;    // sampled passes: the row's draw number (block rows), -1: no draw
};

// Temperature / top-p sampling of a pass's block rows (temperature > 0).
struct SampleArgs {
  float temperature, top_p;
  uint64_t seed;    // stream of the row's sequence: seed + slot
};

// One sequence of a decoder pass.
struct SeqDesc {
  int32_t slot;
  int32_t row0, nrows;   // its rows in the pass
  int32_t kmax;          // max kend over its rows
  int32_t blk0;          // first block_tok entry of its block (-1: no block)
  int32_t blk_row0;      // pass row of its first block row
  int32_t nblk;          // block rows
  int32_t out_b;         // index of the sequence in the caller's batch
  int32_t attn_flash;    // 1: self-attention by the causal kernel (clean rows only, >= kFlashMinRows)
};

// EP_PART (MFMA GEMM only): split y's partial product to out_f32[split][R][N]
enum Epilogue { EP_STORE_F32 = 0, EP_RESID = 1, EP_SILU_ACT = 2, EP_STORE_ACT = 3, EP_ROWOFF_F32 = 4,
                EP_PART = 5 };
enum Prologue { PRO_PLAIN = 0, PRO_NORM = 1 };

// y[r][o] = sum_i W[o][i] * x[r][i] for r < R, o < N.
struct GemmArgs {
  const void *W;
  int N, K;
  int R;
  int pro;
  const void *X;           // PRO_PLAIN: activations, row r at X + (x_row_off ? x_row_off[r] : r * ldx)
  int64_t ldx;
  const int64_t *x_row_off;
  const float *H;          // PRO_NORM: x = act(gain * H[r] / rms(H[r]))
  int64_t ldh;
  const void *gain;
  float eps;
  int ep;
  float *out_f32;
  void *out_act;
  int64_t ldo;
  const int64_t *row_off;  // EP_ROWOFF_F32: out_f32[row_off[r] + off_add + o]
  int64_t off_add;
  // EP_RESID: resid[r * ldo + o] += y (+ cross[slot][lat][cross_layer][o] when cross != null)
  float *resid;
  const float *cross;
  const RowDesc *rows;
  int cross_layer, n_layers, max_lat, d;
  // QKV projection with RoPE and the KV-cache write fused into the epilogue
  // (GEMV path): outputs are taken in (j, j + d_head/2) pairs of each head.
  int qkv_rope;
  const float2 *rope_tab;
  float *q_out;
  void *kv;
  int n_heads, d_head, max_ctx, layer;   // max_ctx: cache rows, kv_rows(cfg.max_ctx)
};

// Cache rows per sequence and head: max_ctx rounded up to whole attention
// chunks, so a chunk's loads never leave its plane.
inline int kv_rows(int max_ctx) { return (max_ctx + kAttnChunk - 1) / kAttnChunk * kAttnChunk; }

// Does a pass of R rows take the GEMV path (else the MFMA GEMM)?
inline bool gemv_path(bool bf16, int R) { return !bf16 || R < kGemvRows; }

struct KVGeom {
  int n_layers, n_heads, d_head, max_ctx;  // max_ctx: cache rows, kv_rows(cfg.max_ctx)
};

// Element offset of (key, dim) in a head's V plane.  The plane is cut into
// tiles of kVTile keys, each stored [d_h][kVTile]: the kVTile keys of every
// dimension that one attention wave reads form a single contiguous block
// (d_h * kVTile elements), and 8 consecutive keys of one dimension are one
// 16-byte piece.
constexpr int kVTile = 32;
__host__ __device__ inline int64_t v_off(int key, int dim, int d_head) {
  return ((int64_t)(key / kVTile) * d_head + dim) * kVTile + key % kVTile;
}

// Kernel launchers (kernels.hip).  `bf16` selects the bfloat16 instantiations.
// A residual product (EP_RESID) on the MFMA path whose K was split: its
// partial products wait in ws[splits][R][N], and the next RMSNorm prologue
// over the same residual adds them (in split order) and the cross term.
struct SplitResid {
  float *ws = nullptr;
  size_t cap = 0;        // floats in ws
  int splits = 0;        // 0: nothing pending
  GemmArgs a{};          // the pending product's arguments
};
// sr (nullable) allows residual products to split K and carries a pending
// sum to the RMSNorm prologue that must take it; xnorm_ws holds the
// normalised activations of the MFMA path.
hipError_t launch_gemm(bool bf16, const GemmArgs &a, void *xnorm_ws, SplitResid *sr, hipStream_t s);
hipError_t launch_embed(bool bf16, const void *embed, const float *cross, const RowDesc *rows,
                        int R, int d, int n_layers, int max_lat, const int32_t *block_tok,
                        const int32_t *tokens_dev, float *h, hipStream_t s);
hipError_t launch_rope_kv(bool bf16, const float *qkv, int R, const RowDesc *rows,
                          const float2 *rope_tab, float *q_out, void *kv, KVGeom g, int layer,
                          hipStream_t s);
// ev0/ev1 (nullable) are stamped by the dispatch of the split-K partials
// kernel, or of the causal kernel when ev_flash is set.  grid_chunks = 0
// skips the split-K kernel and its merge (every sequence on the causal
// kernel); flash_tiles = 0 skips the causal kernel.  nsub: chunks of
// kAttnChunk keys per split-K workgroup (above 1 only for bf16 with d_head
// <= 64), which must be 1 when a split-K sequence has more than 16 rows; when
// one workgroup covers every chunk the kernel writes the output and no merge
// runs.  wg = 2 (bf16, d_head <= 64, at most 16 split-K rows per sequence):
// one eight-wave workgroup per (sequence, head) over all grid_chunks chunks,
// writing the output directly; nsub is then ignored.  sd_host (nullable): the
// host copy of seqs[0] for a one-sequence pass, handed to the split-K kernel
// with its launch (never for a captured launch, whose arguments would go
// stale on replay).
hipError_t launch_attention(bool bf16, const float *q, const void *kv, KVGeom g, int layer,
                            const SeqDesc *seqs, int n_seq, const SeqDesc *sd_host,
                            int grid_chunks, int nsub, int wg, int max_chunks, int flash_tiles, const RowDesc *rows, int R,
                            float *part, void *a_out, hipEvent_t ev0, hipEvent_t ev1, bool ev_flash,
                            hipStream_t s);
bool gemv_supported(bool bf16, int K);
// report_entropy: conf_out receives each row's entropy instead of its confidence.
// smp (nullable): rows with ctr >= 0 draw their byte by temperature / top-p
// sampling; confidence and entropy stay those of the model's distribution.
hipError_t launch_decide(const float *logits, int R, const RowDesc *rows, int32_t *argmax_ws,
                         float *conf_ws, float *ent_ws, int report_entropy, int32_t *argmax_out,
                         float *conf_out, float *logits_out, const SampleArgs *smp, hipStream_t s);
// mode: a blt_unmask value; alpha: the confidence threshold or the entropy bound.
hipError_t launch_unmask(const SeqDesc *seqs, int n_seq, const int32_t *argmax_ws,
                         const float *conf_ws, const float *ent_ws, int32_t *block_tok,
                         float alpha, int mode, int32_t *masked_left, hipStream_t s);
// Greedy decisions of every row and the unmasking of every sequence's block
// in one launch (block passes without sampling): one workgroup per sequence.
hipError_t launch_decide_unmask(const float *logits, int n_seq, const SeqDesc *seqs,
                                const RowDesc *rows, int32_t *argmax_ws, float *conf_ws,
                                float *ent_ws, int report_entropy, int32_t *argmax_out,
                                float *conf_out, float *logits_out, int32_t *block_tok,
                                float alpha, int mode, int32_t *masked_left, hipStream_t s);
// Rejection-sampling verification: draws[b] = the verify pass's draw index d of
// sequence b (uniforms d*64 + j and d*64 + r of the stream seed + slot).
hipError_t launch_verify_sample(int batch, const SeqDesc *seqs, const int64_t *draws, int r,
                                const int32_t *draft, int ld_draft, const float *zq, int ld_q,
                                const float *zp, int ld_p, const SampleArgs &smp,
                                int32_t *accept_len, int32_t *next_byte, hipStream_t s);
// dst = src^T, n x n elements of the context's dtype (set-up only).
hipError_t launch_transpose(bool bf16, const void *src, void *dst, int n, hipStream_t s);
hipError_t launch_verify(int batch, const SeqDesc *seqs, int r, const int32_t *draft,
                         int ld_draft, const int32_t *pred, int ld_pred, int32_t *accept_len,
                         int32_t *next_byte, hipStream_t s);

}  // namespace blt
