// The library-owned context behind the opaque blt_ctx handle.
#pragma once

#include <string>
#include <vector>

#include "blt_internal.h"

namespace blt {

constexpr int kRing = 8;  // pinned staging slots for per-pass descriptors

// Event pairs bracketing launches of one kernel family (profiling aid).
struct ProfRec {
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  double bytes = 0;
};

struct StageSlot {
  void *host = nullptr;
  hipEvent_t ev = nullptr;
  bool pending = false;
};

}  // namespace blt

struct blt_ctx {
  blt_config cfg;
  bool bf16 = false;
  hipStream_t stream = nullptr;
  blt_weights w;
  std::vector<blt_layer_weights> layers;
  // workspace, sized for cfg.max_rows rows
  float *h = nullptr;         // residual stream [R][d]
  float *qkv = nullptr;       // [R][3d]
  float *q = nullptr;         // RoPE'd queries [R][d]
  float *part = nullptr;      // attention chunk partials [R][H][max_chunks][dh+2]
  float *logits = nullptr;    // [R][257]
  float *rinv = nullptr;      // [R]
  float *conf_ws = nullptr;   // [R]
  int32_t *argmax_ws = nullptr;
  int *counters = nullptr;    // attention merge counters [max_batch][H], kept at zero
  void *xa = nullptr;         // GEMM activations [R][max(d, F)]
  void *xb = nullptr;         // GEMM activations [R][max(d, d_global)]
  blt::RowDesc *rows_d = nullptr;
  blt::SeqDesc *seqs_d = nullptr;
  int64_t *offs_d = nullptr;
  float2 *rope_tab = nullptr; // (cos, sin) [max_ctx][dh/2]
  int max_chunks = 0;
  blt::StageSlot ring[blt::kRing];
  int ring_next = 0;
  size_t seq_off = 0, off_off = 0;
  std::string err;
  // profiling: family being timed, event pool, pending and accumulated figures
  int prof_family = 0;
  std::vector<blt::ProfRec> prof_pool;
  size_t prof_used = 0;
  uint64_t prof_launches = 0;
  double prof_ms = 0, prof_bytes = 0;
};

namespace blt {
blt_status stage_pass(blt_ctx *c, const std::vector<RowDesc> &rows,
                      const std::vector<SeqDesc> &seqs, const std::vector<int64_t> *offs);
blt_status prof_next(blt_ctx *c, double bytes, hipEvent_t *ev0, hipEvent_t *ev1);
blt_status prof_collect(blt_ctx *c);
blt_status run_pass(blt_ctx *c, const blt_state *st, const std::vector<RowDesc> &rows,
                    const std::vector<SeqDesc> &seqs, const int32_t *block_tok,
                    const int32_t *tokens_dev, bool unmask, float alpha, int one_step,
                    int32_t *masked_left, int32_t *argmax_out, float *conf_out,
                    float *logits_out);
}  // namespace blt
