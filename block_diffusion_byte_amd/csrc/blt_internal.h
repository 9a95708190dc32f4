// Internal declarations shared by the HIP kernels (kernels.hip) and the
// C-ABI host code (blt_api.cpp, session.cpp).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/blt.h"
#include "desc.h"

namespace blt {

// Device buffers one decoder pass works in (the context's workspace, or the
// allocation-free entry point's static scratch array).
struct PassWs {
  float *h, *qkv, *q, *part, *logits, *conf, *ent;
  int32_t *argmax;
  void *xa, *xb;
  SeqDesc *seqs;
  RowDesc *rows;
};

// The allocation-free entry point's scratch: a file-scope device array of
// kScratchBytes, one copy per GPU.  scratch_region returns its device address
// on the current device (looked up once per device with hipGetSymbolAddress).
constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kNoAllocRows = 15;    // rows per allocation-free call (the GEMV path)
hipError_t scratch_region(void **ptr);

// EP_PART (MFMA GEMM only): split y's partial product to out_f32[split][R][N]
enum Epilogue { EP_STORE_F32 = 0, EP_RESID = 1, EP_SILU_ACT = 2, EP_STORE_ACT = 3, EP_ROWOFF_F32 = 4,
                EP_PART = 5 };
enum Prologue { PRO_PLAIN = 0, PRO_NORM = 1 };

// y[r][o] = sum_i W[o][i] * x[r][i] for r < R, o < N.
struct GemmArgs {
  const void *W;
  const void *Wf;          // W in fragment order (launch_frag_pack; nullable): the weight-streaming GEMM
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
  // device-resident passes: the number of sequences that still have masked
  // positions; when it reads 0 the kernel returns at once (nullptr: always run)
  const int32_t *gate;
  // with a gate: 1 tests it only before the kernel's first store (the GEMVs),
  // for passes the driver expects to have work
  int gate_late;
};

// Cache rows per sequence and head: max_ctx rounded up to whole attention
// chunks, so a chunk's loads never leave its plane.
inline int kv_rows(int max_ctx) { return (max_ctx + kAttnChunk - 1) / kAttnChunk * kAttnChunk; }

// Does a pass of R rows take the GEMV path (else the MFMA GEMM)?
inline bool gemv_path(bool bf16, int R) { return !bf16 || R < kGemvRows; }

struct KVGeom {
  int n_layers, n_heads, d_head, max_ctx;  // max_ctx: cache rows, kv_rows(cfg.max_ctx)
};

// Element offset of (key, dim) in a head's K plane.  The plane is cut into
// tiles of kKTile keys, each stored [d_h / 32][kKTile][32]: one 32-dimension
// slice of every key of the tile, then the next slice.  A bf16 128-byte line
// then holds one slice of two consecutive keys, so the 16-byte pieces that
// one attention load instruction takes (16 keys, one slice, four pieces per
// key) cover whole lines, and streaming (non-temporal) loads fetch each line
// once.  d_h is 32, 64 or 128 (checked at creation).
constexpr int kKTile = 32;
__host__ __device__ inline int64_t k_off(int key, int dim, int d_head) {
  return ((int64_t)(key / kKTile) * d_head + (dim / 32) * kKTile) * 32 + (key % kKTile) * 32 + dim % 32;
}

// Element offset of (key, dim) in a head's V plane.  The plane is cut into
// tiles of kVTile keys, each stored [d_h][kVTile]: the kVTile keys of every
// dimension that one attention wave reads form a single contiguous block
// (d_h * kVTile elements), and 8 consecutive keys of one dimension are one
// 16-byte piece.
constexpr int kVTile = 32;
__host__ __device__ inline int64_t v_off(int key, int dim, int d_head) {
  return ((int64_t)(key / kVTile) * d_head + dim) * kVTile + key % kVTile;
}

// Device-side state of one sequence for device-resident BLT-D blocks: the
// committed bytes live in a device array next to it, the stand-in patcher
// runs on the device after each block, and each block's encoder/global pass
// (the latents it makes available) and first decoder pass are planned there.
struct DevSeq {
  int32_t n;           // committed bytes (prompt + generated)
  int32_t patch_last;  // patch index of byte n-1
  int32_t cur_len;     // bytes of that patch so far
  int32_t ends_last;   // a patch boundary follows byte n-1
  int32_t lat_ready;   // latents 0..lat_ready-1 have cross vectors
  int32_t err;         // nonzero: a latent index or byte out of range
  uint64_t salt;
  int32_t win_patch[kMaxBlock + 1], win_ends[kMaxBlock + 1];   // bytes n-B-1 .. n-1
};

struct DevBlockArgs {
  DevSeq *st;                 // [S]
  int32_t *x;                 // committed bytes, x[b * x_stride + i]
  int x_stride;
  int S, B, causal;           // sequences (slots 0..S-1), block size, block mask
  RowDesc *rows0;             // first pass: B+1 clean rows, then B block rows, per sequence
  SeqDesc *seqs0;
  RowDesc *rows1;             // later passes: the B block rows per sequence
  SeqDesc *seqs1;
  int64_t *lat_offs;          // [2][S*(B+1)]: latent table rows, cross rows of the latents to make
  int32_t *block_tok, *masked_left, *gate, *n_eg;
  int max_latents, n_lat, d_global, n_layers, d_model;
  int64_t seq_stride;         // latent table rows per sequence
};
hipError_t launch_block_plan(const DevBlockArgs &a, hipStream_t s);
// kept[i] = logits[i] (rows of 257) for every block position i = slot*B + j
// of slots 0..n_slots-1 that was [MASK] in `before` and holds a byte in `after`.
hipError_t launch_keep_drawn(const int32_t *before, const int32_t *after, const float *logits,
                             float *kept, int n_slots, int B, hipStream_t s);
hipError_t launch_block_commit(const DevBlockArgs &a, hipStream_t s);

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
// ev0/ev1 (nullable): stamped by the dispatch of the product kernel itself
// (not of the RMSNorm launch that precedes an MFMA GEMM with a norm prologue).
// form: 0 chooses the MFMA GEMM kernel by shape (the weight-streaming kernel
// where the staged-tile kernel's 128x128 tiles would be too few, at most
// 1024 rows), 1 forces the staged-tile kernel, 2 the weight-streaming kernel
// wherever it applies.
hipError_t launch_gemm(bool bf16, const GemmArgs &a, void *xnorm_ws, SplitResid *sr, hipStream_t s,
                       hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr, int form = 0);
enum GemmKind { GEMM_KIND_GEMV_MFMA = 0, GEMM_KIND_GEMV = 1, GEMM_KIND_MFMA = 2 };
GemmKind gemm_kind(bool bf16, const GemmArgs &a);
// gate (nullable, every launcher below): see GemmArgs::gate.
hipError_t launch_embed(bool bf16, const void *embed, const float *cross, const RowDesc *rows,
                        int R, int d, int n_layers, int max_lat, const int32_t *block_tok,
                        const int32_t *tokens_dev, float *h, hipStream_t s,
                        const int32_t *gate = nullptr);
hipError_t launch_rope_kv(bool bf16, const float *qkv, int R, const RowDesc *rows,
                          const float2 *rope_tab, float *q_out, void *kv, KVGeom g, int layer,
                          hipStream_t s, const int32_t *gate = nullptr);
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
                            hipStream_t s, const int32_t *gate = nullptr, int flash_kg = 0,
                            int gate_late = 0);
bool gemv_supported(bool bf16, int K);
// report_entropy: conf_out receives each row's entropy instead of its confidence.
// smp (nullable): rows with ctr >= 0 draw their byte by temperature / top-p
// sampling; confidence and entropy stay those of the model's distribution.
hipError_t launch_decide(const float *logits, int R, const RowDesc *rows, int32_t *argmax_ws,
                         float *conf_ws, float *ent_ws, int report_entropy, int32_t *argmax_out,
                         float *conf_out, float *logits_out, const SampleArgs *smp, hipStream_t s,
                         const int32_t *gate = nullptr);
// mode: a blt_unmask value; alpha: the confidence threshold or the entropy bound.
// gate (nullable): decremented when a sequence's last [MASK] is committed;
// pass_count (nullable): pass_count[slot] += 1 for each sequence that still
// had a [MASK] when the pass began (device-resident decoder pass counter).
hipError_t launch_unmask(const SeqDesc *seqs, int n_seq, const int32_t *argmax_ws,
                         const float *conf_ws, const float *ent_ws, int32_t *block_tok,
                         float alpha, int mode, int32_t *masked_left, hipStream_t s,
                         int32_t *gate = nullptr, int32_t *pass_count = nullptr);
// Greedy decisions of every row and the unmasking of every sequence's block
// in one launch (block passes without sampling): one workgroup per sequence.
hipError_t launch_decide_unmask(const float *logits, int n_seq, const SeqDesc *seqs,
                                const RowDesc *rows, int32_t *argmax_ws, float *conf_ws,
                                float *ent_ws, int report_entropy, int32_t *argmax_out,
                                float *conf_out, float *logits_out, int32_t *block_tok,
                                float alpha, int mode, int32_t *masked_left, hipStream_t s,
                                int32_t *gate = nullptr, int32_t *pass_count = nullptr);
// Rejection-sampling verification: draws[b] = the verify pass's draw index d of
// sequence b (uniforms d*64 + j and d*64 + r of the stream seed + slot).
hipError_t launch_verify_sample(int batch, const SeqDesc *seqs, const int64_t *draws, int r,
                                const int32_t *draft, int ld_draft, const float *zq, int ld_q,
                                const float *zp, int ld_p, const SampleArgs &smp,
                                int32_t *accept_len, int32_t *next_byte, hipStream_t s);
// dst = src^T, n x n elements of the context's dtype (set-up only).
hipError_t launch_transpose(bool bf16, const void *src, void *dst, int n, hipStream_t s);
// bf16 W[N][K] -> its fragment order for the weight-streaming GEMM
// (frag_elems(N, K) elements: rows padded to a multiple of 16 with zeros).
size_t frag_elems(int N, int K);
hipError_t launch_frag_pack(const void *src, int N, int K, void *dst, hipStream_t s);
hipError_t launch_verify(int batch, const SeqDesc *seqs, int r, const int32_t *draft,
                         int ld_draft, const int32_t *pred, int ld_pred, int32_t *accept_len,
                         int32_t *next_byte, hipStream_t s);

}  // namespace blt
