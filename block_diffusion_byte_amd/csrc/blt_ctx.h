// The library-owned context behind the opaque blt_ctx handle.
#pragma once

#include <string.h>

#include <algorithm>
#include <string>
#include <unordered_map>
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

// Everything the kernel sequence of a decoder pass depends on besides the
// staged descriptors: passes with equal keys replay one HIP graph.
struct PassKey {
  int R, S, grid_chunks, flash_tiles, unmask, mode, sample, attn_sub, attn_wg;
  uint32_t alpha_bits, temp_bits, top_p_bits;
  uint64_t seed;
  const void *kv, *cross, *block_tok, *tokens_dev, *masked_left, *argmax_out, *conf_out,
      *logits_out;
  bool operator==(const PassKey &o) const { return memcmp(this, &o, sizeof(PassKey)) == 0; }
};
struct PassKeyHash {
  size_t operator()(const PassKey &k) const {
    const unsigned char *p = (const unsigned char *)&k;
    uint64_t h = 1469598103934665603ull;  // FNV-1a over the key bytes
    for (size_t i = 0; i < sizeof(PassKey); ++i) h = (h ^ p[i]) * 1099511628211ull;
    return (size_t)h;
  }
};
struct GraphEntry {
  hipGraphExec_t exec = nullptr;  // instantiated on the second sighting of a key
};
constexpr size_t kMaxGraphs = 256;
constexpr int kMaxStates = 16;   // decode states whose written rows one context tracks

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
  blt::SplitResid split;      // split-K residual products (MFMA path)
  float *conf_ws = nullptr;   // [R]
  float *ent_ws = nullptr;    // [R] entropy of each row (nats)
  int32_t *argmax_ws = nullptr;
  void *xa = nullptr;         // GEMM activations [R][max(d, F)]
  void *xb = nullptr;         // GEMM activations [R][max(d, d_global)]
  void *cross_w = nullptr;    // [L*d][d]: W_o^c_l W_v^c_l of every layer, stacked (set-up)
  // bf16 projection weights in fragment order for the weight-streaming GEMM
  // of passes of 16 rows or more (one allocation, made at set-up; null when
  // no pass can reach 16 rows): per layer, the byte head, W_lat and C
  struct FragLayer {
    const void *wqkv = nullptr, *wo = nullptr, *w1 = nullptr, *w2 = nullptr;
  };
  void *frag = nullptr;
  std::vector<FragLayer> frag_layers;
  const void *frag_out = nullptr, *frag_lat = nullptr, *frag_cross = nullptr;
  void *desc_d = nullptr;      // per-pass descriptors: sequences, rows, row offsets
  blt::SeqDesc *seqs_d = nullptr;
  blt::RowDesc *rows_d = nullptr;
  int64_t *offs_d = nullptr;
  float2 *rope_tab = nullptr; // (cos, sin) [max_ctx][dh/2]
  int max_chunks = 0;
  blt::StageSlot ring[blt::kRing];
  int ring_next = 0;
  size_t row_off = 0, off_off = 0;  // byte offsets in desc_d and the staging slots
  std::string err;
  // replay of decoder passes from cached HIP graphs (captured on cap_stream)
  bool graphs = false;
  // split-K attention chunks per workgroup forced by blt_attention_chunks (0: per pass)
  int attn_chunks = 0;
  // key groups of the causal attention kernel forced by blt_flash_key_groups (0: per pass)
  int flash_kg = 0;
  // MFMA GEMM kernel forced by blt_gemm_form (0: by shape)
  int gemm_form = 0;
  hipStream_t cap_stream = nullptr;
  std::unordered_map<blt::PassKey, blt::GraphEntry, blt::PassKeyHash> graph_cache;
  // profiling: family being timed, event pool, pending and accumulated figures
  int prof_family = 0;
  std::vector<blt::ProfRec> prof_pool;
  size_t prof_used = 0;
  uint64_t prof_launches = 0;
  double prof_ms = 0, prof_bytes = 0;
  // clean cache rows written so far per (state, slot), keyed by the state's
  // kv buffer: a pass may start at most at that count (rows past it were
  // never written and would enter the softmax).  A fixed table sized at
  // creation, so no call allocates host memory for it.
  struct Written {
    const void *kv = nullptr;
    std::vector<int32_t> rows;   // max_batch entries
  };
  Written written[blt::kMaxStates];
  // nullptr when kMaxStates other states are already tracked
  int32_t *written_rows(const blt_state *st) {
    for (Written &wr : written)
      if (wr.kv == st->kv) return wr.rows.data();
    for (Written &wr : written)
      if (!wr.kv) {
        wr.kv = st->kv;
        std::fill(wr.rows.begin(), wr.rows.end(), 0);
        return wr.rows.data();
      }
    return nullptr;
  }
  // the pass workspace above as one view; host descriptor lists reserved at
  // creation (max_rows rows, max_batch sequences) for the allocation-free call
  blt::PassWs ws{};
  std::vector<blt::RowDesc> rows_tmp;
  std::vector<blt::SeqDesc> seqs_tmp;
  std::vector<char> seen_tmp;
};

namespace blt {
// dst (nullable): the workspace whose descriptor buffers receive the rows and
// sequences (default: the context's own descriptor buffer).
blt_status stage_pass(blt_ctx *c, const std::vector<RowDesc> &rows,
                      const std::vector<SeqDesc> &seqs, const std::vector<int64_t> *offs,
                      const PassWs *dst = nullptr);
blt_status prof_next(blt_ctx *c, double bytes, hipEvent_t *ev0, hipEvent_t *ev1);
blt_status prof_collect(blt_ctx *c);
blt_status enqueue_device_pass(blt_ctx *c, const blt_state *st, int R, int S, int grid_chunks,
                               RowDesc *rows, SeqDesc *seqs, int32_t *block_tok, float alpha,
                               int mode, int32_t *masked_left, int32_t *gate, int32_t *pass_count,
                               int rows_per_seq, hipStream_t s, bool gate_late);
blt_status latents_from_device(blt_ctx *c, const blt_state *st, int m, const int64_t *offs,
                               const void *table, hipStream_t s);
blt_status run_pass(blt_ctx *c, const blt_state *st, std::vector<RowDesc> &rows,
                    std::vector<SeqDesc> &seqs, const int32_t *block_tok,
                    const int32_t *tokens_dev, bool unmask, float alpha, int mode,
                    int32_t *masked_left, int32_t *argmax_out, float *conf_out,
                    float *logits_out, const blt_sampling *smp, const PassWs *ws_static = nullptr);
}  // namespace blt
