// Pass descriptors and the constants they use, shared by the HIP kernels,
// the C-ABI host code and host-only test drivers (no HIP dependency).
#pragma once
#include <stdint.h>

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
  int32_t keep_kv;  // 1: the cache already holds this row's keys and values (a
                    // recomputation with an unchanged latent): they are not written
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

}  // namespace blt
