// C-ABI entry points: argument validation on the host, the library-owned
// workspace, and the kernel sequence of one decoder pass.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "blt_ctx.h"
#include "host_checks.h"

using namespace blt;

namespace {

bool valid_cfg(const blt_config *c, std::string *why) {
  auto bad = [&](const char *m) { *why = m; return false; };
  if (!c) return bad("config is NULL");
  if (c->dtype != BLT_F32 && c->dtype != BLT_BF16) return bad("dtype must be BLT_F32 or BLT_BF16");
  if (c->vocab != kVocab) return bad("vocab must be 257 (256 bytes + [MASK])");
  if (c->n_layers < 1 || c->d_model < 1 || c->n_heads < 1 || c->d_ffn < 1 || c->d_global < 1)
    return bad("layer/width sizes must be positive");
  if (c->d_model % c->n_heads) return bad("d_model must be a multiple of n_heads");
  const int dh = c->d_model / c->n_heads;
  if (dh != 32 && dh != 64 && dh != 128) return bad("head width must be 32, 64 or 128");
  const int epc = c->dtype == BLT_BF16 ? 8 : 4;
  const int q = 32 * epc;  // 4 waves x 8 lanes x one 16-byte chunk
  if (c->d_model % q || c->d_ffn % q || c->d_global % q)
    return bad("d_model, d_ffn and d_global must be multiples of 256 (bf16) or 128 (f32)");
  if (c->dtype == BLT_BF16 && (c->d_model % 64 || c->d_ffn % 64 || c->d_global % 64))
    return bad("bf16 widths must be multiples of 64");
  if (c->max_batch < 1 || c->max_ctx < 1 || c->max_latents < 1 || c->max_rows < 1)
    return bad("capacities must be positive");
  if (c->max_block < 1 || c->max_block > kMaxBlock) return bad("max_block must be in 1..64");
  if (!(c->rope_theta > 0.f) || !isfinite(c->rope_theta)) return bad("rope_theta must be > 0");
  if (!(c->rms_eps >= 0.f) || !isfinite(c->rms_eps)) return bad("rms_eps must be >= 0");
  if (!gemv_supported(c->dtype == BLT_BF16, c->d_model) || !gemv_supported(c->dtype == BLT_BF16, c->d_ffn) ||
      !gemv_supported(c->dtype == BLT_BF16, c->d_global))
    return bad("d_model, d_ffn, d_global: unsupported width (multiple of 256/128 with 1,2,3,4,6,8,12,16,24 chunks per lane)");
  if (c->max_ctx > kAttnChunk * kMaxChunks) return bad("max_ctx above 16384");
  return true;
}

size_t esize(const blt_config &c) { return c.dtype == BLT_BF16 ? 2 : 4; }

blt_status fail(blt_ctx *c, blt_status st, const std::string &m) {
  if (c) c->err = m;
  return st;
}

// Message without a temporary string: c->err keeps its reserved capacity.
blt_status fail(blt_ctx *c, blt_status st, const char *m) {
  if (c) c->err.assign(m);
  return st;
}

blt_status hip_fail(blt_ctx *c, hipError_t e, const char *where) {
  if (c) c->err = std::string(where) + ": " + hipGetErrorString(e);
  return BLT_EHIP;
}

#define HIP_TRY(ctx, expr)                                         \
  do {                                                             \
    hipError_t _e = (expr);                                        \
    if (_e != hipSuccess) return hip_fail((ctx), _e, #expr);       \
  } while (0)

template <typename T>
hipError_t dalloc(T **p, size_t n) {
  return hipMalloc((void **)p, std::max<size_t>(n, 1) * sizeof(T));
}

}  // namespace

namespace blt {

// Copy this pass's descriptors into a pinned staging slot and then to the
// device buffer of the same layout (sequences, rows, row offsets): one copy
// carries the sequences and the rows.  Slots rotate; a slot is reused only
// after its previous copy ended.
blt_status stage_pass(blt_ctx *c, const std::vector<RowDesc> &rows,
                      const std::vector<SeqDesc> &seqs, const std::vector<int64_t> *offs,
                      const PassWs *dst) {
#ifdef BLT_DEBUG_BOUNDS
  {
    const blt_config &g = c->cfg;
    const DescLimits lim{g.max_batch, g.max_ctx, g.max_latents, g.max_rows,
                         (int64_t)g.max_batch * g.max_block};
    char msg[160];
    if (const char *why = check_pass_descs(rows.data(), (int)rows.size(), seqs.data(),
                                           (int)seqs.size(), lim, msg, sizeof msg))
      return fail(c, BLT_EINVAL, why);
  }
#endif
  StageSlot &sl = c->ring[c->ring_next];
  c->ring_next = (c->ring_next + 1) % kRing;
  if (sl.pending) {
    HIP_TRY(c, hipEventSynchronize(sl.ev));
    sl.pending = false;
  }
  char *p = (char *)sl.host;
  const size_t rb = rows.size() * sizeof(RowDesc), sb = seqs.size() * sizeof(SeqDesc);
  const size_t ob = offs ? offs->size() * sizeof(int64_t) : 0;
  if (sb) memcpy(p, seqs.data(), sb);
  if (rb) memcpy(p + c->row_off, rows.data(), rb);
  if (ob) memcpy(p + c->off_off, offs->data(), ob);
  if (dst) {
    // another workspace's descriptor buffers: sequences and rows apart
    if (ob) return fail(c, BLT_EINVAL, "stage_pass: offsets go to the context's buffer only");
    if (sb) HIP_TRY(c, hipMemcpyAsync(dst->seqs, p, sb, hipMemcpyHostToDevice, c->stream));
    if (rb) HIP_TRY(c, hipMemcpyAsync(dst->rows, p + c->row_off, rb, hipMemcpyHostToDevice, c->stream));
  } else if (rb)
    HIP_TRY(c, hipMemcpyAsync(c->desc_d, p, c->row_off + rb, hipMemcpyHostToDevice, c->stream));
  else if (sb)
    HIP_TRY(c, hipMemcpyAsync(c->desc_d, p, sb, hipMemcpyHostToDevice, c->stream));
  if (ob)
    HIP_TRY(c, hipMemcpyAsync((char *)c->desc_d + c->off_off, p + c->off_off, ob,
                              hipMemcpyHostToDevice, c->stream));
  HIP_TRY(c, hipEventRecord(sl.ev, c->stream));
  sl.pending = true;
  return BLT_OK;
}

// Next event pair of the profiling pool (collecting first when it is full).
blt_status prof_next(blt_ctx *c, double bytes, hipEvent_t *ev0, hipEvent_t *ev1) {
  *ev0 = *ev1 = nullptr;
  if (c->prof_used == c->prof_pool.size()) {
    blt_status bs = prof_collect(c);
    if (bs != BLT_OK) return bs;
  }
  ProfRec &r = c->prof_pool[c->prof_used++];
  r.bytes = bytes;
  *ev0 = r.ev0;
  *ev1 = r.ev1;
  return BLT_OK;
}

blt_status prof_collect(blt_ctx *c) {
  if (c->prof_used == 0) return BLT_OK;
  HIP_TRY(c, hipStreamSynchronize(c->stream));
  for (size_t i = 0; i < c->prof_used; ++i) {
    float ms = 0.f;
    HIP_TRY(c, hipEventElapsedTime(&ms, c->prof_pool[i].ev0, c->prof_pool[i].ev1));
    c->prof_ms += ms;
    c->prof_bytes += c->prof_pool[i].bytes;
    c->prof_launches += 1;
  }
  c->prof_used = 0;
  return BLT_OK;
}

GemmArgs base_args(const blt_ctx *c) {
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.eps = c->cfg.rms_eps;
  a.n_layers = c->cfg.n_layers;
  a.max_lat = c->cfg.max_latents;
  a.d = c->cfg.d_model;
  return a;
}

// Arguments of the kernel sequence of one pass besides the staged descriptors.
struct PassLaunch {
  int R, S, grid_chunks, flash_tiles;
  const blt_state *st;
  const int32_t *block_tok, *tokens_dev;
  bool unmask;
  float alpha;
  int mode;                          // a blt_unmask value
  int32_t *masked_left, *argmax_out;
  float *conf_out, *logits_out;
  double split_bytes;                // per layer: K and V rows the split-K kernel's sequences read
  double flash_flops;                // per layer: the causal kernel's QK^T and PV flops
  bool sample;                       // block rows draw their bytes (smp)
  SampleArgs smp;
  int attn_sub = 1;                  // kAttnChunk-key chunks per split-K attention workgroup
  int attn_wg = 1;                   // 2: eight-wave workgroups, one per (sequence, head)
  const SeqDesc *seq1 = nullptr;     // host copy of a one-sequence pass's descriptor (direct launches)
  int32_t *gate = nullptr;           // device-resident passes: sequences with masks left (0: skip)
  int gate_late = 0;                 // 1: the streaming kernels test the gate before their stores
  int32_t *pass_count = nullptr;     // device-resident passes: decoder passes per slot
};

// Split-K attention: a pass whose chunks number at most 1024 in all takes one
// chunk per workgroup (small passes need the parallelism).  In larger ones,
// when sequences times heads reach 256, one eight-wave workgroup per
// (sequence, head) walks all of its chunks and writes the output (no
// partials, no merge); below that the workgroups of a (sequence, head) share
// its chunks evenly, as many as give about 512 in the pass: partials written
// to memory slow the key stream far beyond their size, so they take many
// chunks per workgroup.  Sequences of more than 16 split-K rows keep one
// chunk, held in registers for every 16-row group.  The choice depends on the
// pass's shape only (measured at the batch-1, batch-16 and batch-64 shapes).
static void choose_attention(const blt_ctx *c, PassLaunch &p, int grid_chunks, int split_rows) {
  p.attn_sub = 1;
  p.attn_wg = 1;
  if (!c->bf16 || c->cfg.d_model / c->cfg.n_heads > 64 || split_rows > 16 || grid_chunks <= 0) return;
  if (c->attn_chunks) {
    p.attn_sub = c->attn_chunks;
    return;
  }
  const int units = c->cfg.n_heads * p.S;
  if ((int64_t)units * grid_chunks <= 1024) return;
  if (units >= 256) {
    p.attn_sub = grid_chunks;
    p.attn_wg = 2;
    return;
  }
  const int wg = std::min(grid_chunks, std::max(1, (512 + units - 1) / units));
  p.attn_sub = (grid_chunks + wg - 1) / wg;
}

// The kernel sequence of one decoder pass over the staged rows, on stream s.
blt_status enqueue_pass(blt_ctx *c, const PassLaunch &p, hipStream_t s, const PassWs &w) {
  const blt_config &g = c->cfg;
  const int R = p.R, S = p.S, d = g.d_model, F = g.d_ffn, L = g.n_layers;
  const bool bf = c->bf16;
  const blt_state *st = p.st;
  const float *cross = (const float *)st->cross;
  HIP_TRY(c, launch_embed(bf, c->w.embed, cross, w.rows, R, d, L, g.max_latents, p.block_tok,
                          p.tokens_dev, w.h, s, p.gate));
  KVGeom geo{L, g.n_heads, d / g.n_heads, kv_rows(g.max_ctx)};
  c->split.splits = 0;               // no sum left pending by an interrupted pass
  // A projection, stamped with events when its kernel family is being timed:
  // the GEMV families count algorithmic bytes (weights, activations read,
  // outputs written, the residual read by a residual epilogue), the MFMA
  // GEMM counts flops (2 N K R).
  const size_t e = bf ? 2 : 4;
  auto gemm = [&](const GemmArgs &a) -> blt_status {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    const int fam = c->prof_family;
    if (fam == BLT_PROF_GEMV_MFMA || fam == BLT_PROF_GEMV || fam == BLT_PROF_GEMM) {
      const GemmKind k = gemm_kind(bf, a);
      if ((fam == BLT_PROF_GEMV_MFMA && k == GEMM_KIND_GEMV_MFMA) ||
          (fam == BLT_PROF_GEMV && k == GEMM_KIND_GEMV) || (fam == BLT_PROF_GEMM && k == GEMM_KIND_MFMA)) {
        double work;
        if (k == GEMM_KIND_MFMA) {
          work = 2.0 * a.N * a.K * a.R;
        } else {
          const double act = a.pro == PRO_NORM ? 4.0 : (double)e;
          const double outb = (a.ep == EP_STORE_ACT || a.ep == EP_SILU_ACT) ? (double)e : 4.0;
          work = (double)a.N * a.K * e + (double)a.R * a.K * act + (double)a.R * a.N * outb +
                 (a.ep == EP_RESID ? 4.0 * a.R * a.N : 0.0);
        }
        blt_status pb = prof_next(c, work, &e0, &e1);
        if (pb != BLT_OK) return pb;
      }
    }
    GemmArgs ag = a;
    ag.gate = p.gate;
    ag.gate_late = p.gate_late;
    HIP_TRY(c, launch_gemm(bf, ag, w.xb, &c->split, s, e0, e1, c->gemm_form));
    return BLT_OK;
  };
#define BLT_GEMM_TRY(a)                 \
  do {                                  \
    const blt_status _g = gemm(a);      \
    if (_g != BLT_OK) return _g;        \
  } while (0)
  for (int l = 0; l < L; ++l) {
    const blt_layer_weights &lw = c->layers[l];
    const blt_ctx::FragLayer *fl = c->frag ? &c->frag_layers[l] : nullptr;
    GemmArgs a = base_args(c);
    a.R = R;
    a.rows = w.rows;
    // q, k, v = W_qkv RMSNorm(h)
    a.W = lw.wqkv; a.Wf = fl ? fl->wqkv : nullptr; a.N = 3 * d; a.K = d;
    a.pro = PRO_NORM; a.H = w.h; a.ldh = d; a.gain = lw.g_attn;
    a.ep = EP_STORE_F32; a.out_f32 = w.qkv; a.ldo = 3 * d;
    // RoPE and the KV write happen in the projection's epilogue (on the
    // MFMA path when a 64-column tile holds whole heads)
    if (gemv_path(bf, R) || geo.d_head <= 64) {
      a.qkv_rope = 1; a.rope_tab = c->rope_tab; a.q_out = w.q; a.kv = st->kv;
      a.n_heads = g.n_heads; a.d_head = d / g.n_heads; a.max_ctx = kv_rows(g.max_ctx); a.layer = l;
      BLT_GEMM_TRY(a);
    } else {
      BLT_GEMM_TRY(a);
      HIP_TRY(c, launch_rope_kv(bf, w.qkv, R, w.rows, c->rope_tab, w.q, st->kv, geo, l, s, p.gate));
    }
    hipEvent_t e0 = nullptr, e1 = nullptr;
    const bool ev_flash = c->prof_family == BLT_PROF_ATTENTION_CAUSAL;
    if ((c->prof_family == BLT_PROF_ATTENTION && p.grid_chunks > 0) ||
        (ev_flash && p.flash_tiles > 0)) {
      blt_status pb = prof_next(c, ev_flash ? p.flash_flops : p.split_bytes, &e0, &e1);
      if (pb != BLT_OK) return pb;
    }
    HIP_TRY(c, launch_attention(bf, w.q, st->kv, geo, l, w.seqs, S, p.seq1, p.grid_chunks,
                                p.attn_sub, p.attn_wg, c->max_chunks,
                                p.flash_tiles, w.rows, R, w.part, w.xa, e0, e1, ev_flash, s, p.gate,
                                c->flash_kg, p.gate_late));
    // h += W_o a
    a = base_args(c); a.R = R; a.rows = w.rows;
    a.W = lw.wo; a.Wf = fl ? fl->wo : nullptr; a.N = d; a.K = d;
    a.pro = PRO_PLAIN; a.X = w.xa; a.ldx = d;
    a.ep = EP_RESID; a.resid = w.h; a.ldo = d;
    BLT_GEMM_TRY(a);
    // f = SiLU(W1 RMSNorm(h))
    a = base_args(c); a.R = R; a.rows = w.rows;
    a.W = lw.w1; a.Wf = fl ? fl->w1 : nullptr; a.N = F; a.K = d;
    a.pro = PRO_NORM; a.H = w.h; a.ldh = d; a.gain = lw.g_ffn;
    a.ep = EP_SILU_ACT; a.out_act = w.xa; a.ldo = F;
    BLT_GEMM_TRY(a);
    // h += W2 f (+ the next layer's cross-attention contribution)
    a = base_args(c); a.R = R; a.rows = w.rows;
    a.W = lw.w2; a.Wf = fl ? fl->w2 : nullptr; a.N = d; a.K = F;
    a.pro = PRO_PLAIN; a.X = w.xa; a.ldx = F;
    a.ep = EP_RESID; a.resid = w.h; a.ldo = d;
    if (l + 1 < L) { a.cross = cross; a.cross_layer = l + 1; }
    BLT_GEMM_TRY(a);
  }
  GemmArgs a = base_args(c);
  a.R = R; a.rows = w.rows;
  a.W = c->w.w_out; a.Wf = c->frag_out; a.N = kVocab; a.K = d;
  a.pro = PRO_NORM; a.H = w.h; a.ldh = d; a.gain = c->w.g_out;
  a.ep = EP_STORE_F32; a.out_f32 = w.logits; a.ldo = kVocab;
  BLT_GEMM_TRY(a);
#undef BLT_GEMM_TRY
  if (c->split.splits) return fail(c, BLT_EHIP, "enqueue_pass: a split residual sum was left pending");
  const int rep_ent = p.unmask && p.mode == BLT_UNMASK_ENTROPY;
  if (p.unmask && !p.sample) {
    HIP_TRY(c, launch_decide_unmask(w.logits, S, w.seqs, w.rows, w.argmax, w.conf,
                                    w.ent, rep_ent, p.argmax_out, p.conf_out, p.logits_out,
                                    (int32_t *)p.block_tok, p.alpha, p.mode, p.masked_left, s,
                                    p.gate, p.pass_count));
    return BLT_OK;
  }
  HIP_TRY(c, launch_decide(w.logits, R, w.rows, w.argmax, w.conf, w.ent, rep_ent,
                           p.argmax_out, p.conf_out, p.logits_out, p.sample ? &p.smp : nullptr, s,
                           p.gate));
  if (p.unmask)
    HIP_TRY(c, launch_unmask(w.seqs, S, w.argmax, w.conf, w.ent,
                             (int32_t *)p.block_tok, p.alpha, p.mode, p.masked_left, s, p.gate,
                             p.pass_count));
  return BLT_OK;
}

void drop_graphs(blt_ctx *c) {
  for (auto &kv : c->graph_cache)
    if (kv.second.exec) (void)hipGraphExecDestroy(kv.second.exec);
  c->graph_cache.clear();
}

// One decoder pass over `rows` (grouped by `seqs`): the descriptors are
// staged, then the kernel sequence is launched directly or, for a pass shape
// seen before, replayed from a cached graph (captured on the context's own
// capture stream, launched on its stream).
blt_status run_pass(blt_ctx *c, const blt_state *st, std::vector<RowDesc> &rows,
                    std::vector<SeqDesc> &seqs, const int32_t *block_tok,
                    const int32_t *tokens_dev, bool unmask, float alpha, int mode,
                    int32_t *masked_left, int32_t *argmax_out, float *conf_out,
                    float *logits_out, const blt_sampling *smp, const PassWs *ws_static) {
  // Attention path per sequence, from its own rows only: a bf16 sequence
  // whose rows in the pass are all clean (no block) and number at least
  // kFlashMinRows takes the causal kernel; every other one the split-K kernel.
  // Profiling figures per layer: the split-K kernel must read the K and V
  // rows below each of its sequences' kmax; the causal kernel does 4 d flops
  // per (row, key) pair (two multiply-adds per head dimension, QK^T and PV).
  const int d = c->cfg.d_model;
  int kmax = 0, flash_tiles = 0, split_rows = 0;
  double split_bytes = 0, flash_flops = 0;
  for (SeqDesc &sd : seqs) {
    sd.attn_flash = c->bf16 && sd.blk0 < 0 && sd.nrows >= kFlashMinRows;
    for (int r = sd.row0; r < sd.row0 + sd.nrows; ++r) {
      rows[r].attn_flash = sd.attn_flash;
      if (sd.attn_flash) flash_flops += 4.0 * d * rows[r].kend;
    }
    if (sd.attn_flash) {
      flash_tiles = std::max(flash_tiles, (sd.nrows + kFlashRows - 1) / kFlashRows);
    } else {
      kmax = std::max(kmax, sd.kmax);
      split_rows = std::max(split_rows, sd.nrows);
      split_bytes += (double)sd.kmax * 2.0 * d * (c->bf16 ? 2 : 4);
    }
  }
  blt_status bs = stage_pass(c, rows, seqs, nullptr, ws_static);
  if (bs != BLT_OK) return bs;
  PassLaunch p{(int)rows.size(), (int)seqs.size(), (kmax + kAttnChunk - 1) / kAttnChunk,
               flash_tiles, st, block_tok, tokens_dev, unmask, alpha, mode, masked_left,
               argmax_out, conf_out, logits_out, split_bytes, flash_flops, smp != nullptr,
               SampleArgs{smp ? smp->temperature : 0.f, smp ? smp->top_p : 0.f,
                          smp ? smp->seed : 0}};
  auto attn_policy = [&](int grid_chunks) { choose_attention(c, p, grid_chunks, split_rows); };
  if (ws_static || !c->graphs || c->prof_family != BLT_PROF_OFF) {
    attn_policy(p.grid_chunks);
    if (seqs.size() == 1) p.seq1 = &seqs[0];
    return enqueue_pass(c, p, c->stream, ws_static ? *ws_static : c->ws);
  }
  // chunk-grid buckets of 4 keep the number of distinct graphs small; the
  // chunks past a sequence's kmax leave at once
  p.grid_chunks = std::min((p.grid_chunks + 3) / 4 * 4, c->max_chunks);
  attn_policy(p.grid_chunks);
  PassKey key;
  memset(&key, 0, sizeof(key));
  key.R = p.R; key.S = p.S; key.grid_chunks = p.grid_chunks; key.flash_tiles = p.flash_tiles;
  key.attn_sub = p.attn_sub; key.attn_wg = p.attn_wg;
  key.unmask = unmask;
  key.mode = mode;
  memcpy(&key.alpha_bits, &alpha, sizeof(float));
  key.sample = p.sample;
  memcpy(&key.temp_bits, &p.smp.temperature, sizeof(float));
  memcpy(&key.top_p_bits, &p.smp.top_p, sizeof(float));
  key.seed = p.smp.seed;
  key.kv = st->kv; key.cross = st->cross; key.block_tok = block_tok; key.tokens_dev = tokens_dev;
  key.masked_left = masked_left; key.argmax_out = argmax_out; key.conf_out = conf_out;
  key.logits_out = logits_out;
  auto it = c->graph_cache.find(key);
  if (it == c->graph_cache.end()) {
    // first sighting: launch directly (also prepares every kernel's attributes)
    if (c->graph_cache.size() >= kMaxGraphs) drop_graphs(c);
    c->graph_cache.emplace(key, GraphEntry{});
    return enqueue_pass(c, p, c->stream, c->ws);
  }
  GraphEntry &ge = it->second;
  if (!ge.exec) {
    HIP_TRY(c, hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal));
    const blt_status ls = enqueue_pass(c, p, c->cap_stream, c->ws);
    hipGraph_t graph = nullptr;
    const hipError_t ee = hipStreamEndCapture(c->cap_stream, &graph);
    if (ls != BLT_OK || ee != hipSuccess) {
      if (graph) (void)hipGraphDestroy(graph);
      return ls != BLT_OK ? ls : hip_fail(c, ee, "hipStreamEndCapture");
    }
    const hipError_t ie = hipGraphInstantiate(&ge.exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (ie != hipSuccess) {
      ge.exec = nullptr;
      return hip_fail(c, ie, "hipGraphInstantiate");
    }
  }
  HIP_TRY(c, hipGraphLaunch(ge.exec, c->stream));
  return BLT_OK;
}

// A BLT-D block pass whose descriptors were written on the device (by the
// block plan kernel): R rows of S sequences, attention over at most
// grid_chunks chunks, every kernel gated by *gate, decoder passes counted in
// pass_count.  Nothing is staged from the host and no host copy of a
// descriptor is handed to a kernel, so the launches can be captured once and
// replayed.
blt_status enqueue_device_pass(blt_ctx *c, const blt_state *st, int R, int S, int grid_chunks,
                               RowDesc *rows, SeqDesc *seqs, int32_t *block_tok, float alpha,
                               int mode, int32_t *masked_left, int32_t *gate, int32_t *pass_count,
                               int rows_per_seq, hipStream_t s, bool gate_late) {
  PassLaunch p{R, S, grid_chunks, 0, st, block_tok, nullptr, true, alpha, mode, masked_left,
               nullptr, nullptr, nullptr, 0.0, 0.0, false, SampleArgs{0.f, 0.f, 0}};
  p.gate = gate;
  p.gate_late = gate_late ? 1 : 0;
  p.pass_count = pass_count;
  choose_attention(c, p, grid_chunks, rows_per_seq);
  PassWs w = c->ws;
  w.rows = rows;
  w.seqs = seqs;
  return enqueue_pass(c, p, s, w);
}

// The latent projections of m latents whose table rows and cross rows the
// device wrote into offs[0..m) and offs[m..2m) (an encoder/global pass
// planned on the device): o~ = W_lat o, then cross = C o~ for every layer.
blt_status latents_from_device(blt_ctx *c, const blt_state *st, int m, const int64_t *offs,
                               const void *table, hipStream_t s) {
  const blt_config &g = c->cfg;
  if (m > g.max_rows) return fail(c, BLT_ECAPACITY, "latents_from_device: more latents than max_rows");
  const int d = g.d_model, L = g.n_layers;
  GemmArgs a = base_args(c);
  a.R = m; a.W = c->w.w_lat; a.Wf = c->frag_lat; a.N = d; a.K = g.d_global;
  a.pro = PRO_PLAIN; a.X = table; a.x_row_off = offs;
  a.ep = EP_STORE_ACT; a.out_act = c->xb; a.ldo = d;
  HIP_TRY(c, launch_gemm(c->bf16, a, c->xb, nullptr, s, nullptr, nullptr, c->gemm_form));
  a = base_args(c);
  a.R = m; a.W = c->cross_w; a.Wf = c->frag_cross; a.N = L * d; a.K = d;
  a.pro = PRO_PLAIN; a.X = c->xb; a.ldx = d;
  a.ep = EP_ROWOFF_F32; a.out_f32 = (float *)st->cross; a.row_off = offs + m;
  HIP_TRY(c, launch_gemm(c->bf16, a, c->xb, nullptr, s, nullptr, nullptr, c->gemm_form));
  return BLT_OK;
}

}  // namespace blt

extern "C" {

blt_status blt_state_size(const blt_config *cfg, size_t *kv_bytes, size_t *cross_bytes) {
  std::string why;
  if (!valid_cfg(cfg, &why) || !kv_bytes || !cross_bytes) return BLT_EINVAL;
  const size_t e = esize(*cfg);
  *kv_bytes = (size_t)cfg->max_batch * cfg->n_layers * 2 * kv_rows(cfg->max_ctx) * cfg->d_model * e;
  *cross_bytes = (size_t)cfg->max_batch * cfg->max_latents * cfg->n_layers * cfg->d_model * sizeof(float);
  return BLT_OK;
}

const char *blt_last_error(const blt_ctx *ctx) { return ctx ? ctx->err.c_str() : "NULL context"; }

blt_status blt_create(const blt_config *cfg, const blt_weights *w, void *hip_stream, blt_ctx **out) {
  std::string why;
  if (!out) return BLT_EINVAL;
  *out = nullptr;
  if (!valid_cfg(cfg, &why)) {
    if (cfg && (cfg->dtype != BLT_F32 && cfg->dtype != BLT_BF16)) return BLT_EDTYPE;
    return BLT_EINVAL;
  }
  if (!w || !w->embed || !w->w_lat || !w->w_out || !w->g_out || !w->layers) return BLT_EINVAL;
  for (int l = 0; l < cfg->n_layers; ++l) {
    const blt_layer_weights &lw = w->layers[l];
    if (!lw.wv_c || !lw.wo_c || !lw.wqkv || !lw.wo || !lw.g_attn || !lw.g_ffn || !lw.w1 || !lw.w2)
      return BLT_EINVAL;
  }
  blt_ctx *c = new (std::nothrow) blt_ctx();
  if (!c) return BLT_EINVAL;
  c->cfg = *cfg;
  c->bf16 = cfg->dtype == BLT_BF16;
  c->stream = (hipStream_t)hip_stream;
  c->w = *w;
  c->layers.assign(w->layers, w->layers + cfg->n_layers);
  const int R = cfg->max_rows, d = cfg->d_model, F = cfg->d_ffn, H = cfg->n_heads;
  const int dh = d / H;
  c->max_chunks = (cfg->max_ctx + kAttnChunk - 1) / kAttnChunk;
  const size_t e = esize(*cfg);
  const size_t wide = (size_t)std::max(d, F);
  hipError_t he = hipSuccess;
  auto chk = [&](hipError_t x) { if (he == hipSuccess) he = x; };
  chk(dalloc(&c->h, (size_t)R * d));
  chk(dalloc(&c->qkv, (size_t)R * 3 * d));
  chk(dalloc(&c->q, (size_t)R * d));
  chk(dalloc(&c->part, (size_t)R * H * c->max_chunks * (dh + 2)));
  chk(dalloc(&c->logits, (size_t)R * kVocab));
  // partial products of split-K residual GEMMs (MFMA path: bf16, >= 16 rows)
  if (c->bf16 && R >= kGemvRows) {
    c->split.cap = std::min<size_t>((size_t)8 * R * d, (size_t)1 << 22);
    chk(dalloc(&c->split.ws, c->split.cap));
  }
  chk(dalloc(&c->conf_ws, (size_t)R));
  chk(dalloc(&c->ent_ws, (size_t)R));
  chk(dalloc(&c->argmax_ws, (size_t)R));
  chk(hipMalloc(&c->xa, std::max<size_t>(1, (size_t)R * wide * e)));
  chk(hipMalloc(&c->xb, std::max<size_t>(1, (size_t)R * std::max(d, cfg->d_global) * e)));
  chk(dalloc(&c->rope_tab, (size_t)cfg->max_ctx * (dh / 2)));
  chk(hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking));
  c->row_off = ((size_t)cfg->max_batch * sizeof(SeqDesc) + 255) & ~(size_t)255;
  c->off_off = (c->row_off + (size_t)R * sizeof(RowDesc) + 255) & ~(size_t)255;
  // offsets area: the two row-offset lists of a latent batch (2 per row) or
  // one draw index per sequence of a sampled verification
  const size_t stage = c->off_off + std::max<size_t>(2 * (size_t)R, cfg->max_batch) * sizeof(int64_t);
  chk(hipMalloc(&c->desc_d, stage));
  if (he == hipSuccess) {
    c->seqs_d = (SeqDesc *)c->desc_d;
    c->rows_d = (RowDesc *)((char *)c->desc_d + c->row_off);
    c->offs_d = (int64_t *)((char *)c->desc_d + c->off_off);
    c->ws = PassWs{c->h, c->qkv, c->q, c->part, c->logits, c->conf_ws, c->ent_ws, c->argmax_ws,
                   c->xa, c->xb, c->seqs_d, c->rows_d};
  }
  for (auto &wr : c->written) wr.rows.assign(cfg->max_batch, 0);
  c->rows_tmp.reserve(R);
  c->seqs_tmp.reserve(cfg->max_batch);
  c->seen_tmp.reserve(cfg->max_batch);
  c->err.reserve(512);
  for (int i = 0; i < kRing && he == hipSuccess; ++i) {
    chk(hipHostMalloc(&c->ring[i].host, stage, hipHostMallocDefault));
    chk(hipEventCreateWithFlags(&c->ring[i].ev, hipEventDisableTiming));
  }
  if (he == hipSuccess) {
    // RoPE angles pos * theta^(-2j/dh), evaluated in double precision.
    std::vector<float2> tab((size_t)cfg->max_ctx * (dh / 2));
    for (int p = 0; p < cfg->max_ctx; ++p)
      for (int j = 0; j < dh / 2; ++j) {
        const double ang = (double)p * pow((double)cfg->rope_theta, -2.0 * j / dh);
        tab[(size_t)p * (dh / 2) + j] = make_float2((float)cos(ang), (float)sin(ang));
      }
    chk(hipMemcpy(c->rope_tab, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice));
  }
  if (he == hipSuccess) {
    // The cross-attention read of one latent is W_o^c_l W_v^c_l W_lat o for
    // every layer l: the two per-layer matrices are multiplied once here,
    // C_l = W_o^c_l (W_v^c_l^T)^T by the GEMM (rows of W_o^c_l against rows of
    // the transposed W_v^c_l), stacked as [L*d][d] so that one product per
    // latent fills all its cross vectors.
    const int L = cfg->n_layers;
    void *tmp = nullptr;
    chk(hipMalloc(&c->cross_w, (size_t)L * d * d * e));
    chk(hipMalloc(&tmp, (size_t)d * d * e));
    for (int l = 0; l < L && he == hipSuccess; ++l) {
      const blt_layer_weights &lw = c->layers[l];
      chk(launch_transpose(c->bf16, lw.wv_c, tmp, d, c->stream));
      GemmArgs a = base_args(c);
      a.R = d; a.W = tmp; a.N = d; a.K = d;
      a.pro = PRO_PLAIN; a.X = lw.wo_c; a.ldx = d;
      a.ep = EP_STORE_ACT; a.out_act = (char *)c->cross_w + (size_t)l * d * d * e; a.ldo = d;
      chk(launch_gemm(c->bf16, a, c->xb, nullptr, c->stream, nullptr, nullptr, c->gemm_form));
    }
    chk(hipStreamSynchronize(c->stream));
    if (tmp) (void)hipFree(tmp);
  }
  if (he == hipSuccess && c->bf16 && cfg->max_rows >= kGemvRows) {
    // Fragment-ordered copies of the projection weights, read by the
    // weight-streaming GEMM of passes of 16 rows or more (an extra 2 bytes
    // per parameter of the decoder, W_lat and C)
    const int L = cfg->n_layers, F = cfg->d_ffn, dg = cfg->d_global;
    struct Job {
      const void *src;
      int N, K;
      const void **dst;
    };
    std::vector<Job> jobs;
    c->frag_layers.assign(L, blt_ctx::FragLayer{});
    for (int l = 0; l < L; ++l) {
      const blt_layer_weights &lw = c->layers[l];
      blt_ctx::FragLayer &fl = c->frag_layers[l];
      jobs.push_back({lw.wqkv, 3 * d, d, &fl.wqkv});
      jobs.push_back({lw.wo, d, d, &fl.wo});
      jobs.push_back({lw.w1, F, d, &fl.w1});
      jobs.push_back({lw.w2, d, F, &fl.w2});
    }
    jobs.push_back({c->w.w_out, kVocab, d, &c->frag_out});
    jobs.push_back({c->w.w_lat, d, dg, &c->frag_lat});
    jobs.push_back({c->cross_w, L * d, d, &c->frag_cross});
    size_t total = 0;
    for (const Job &j : jobs)
      if (j.K % 32 == 0) total += frag_elems(j.N, j.K);
    chk(hipMalloc(&c->frag, total * e));
    size_t off = 0;
    for (const Job &j : jobs) {
      if (he != hipSuccess || j.K % 32) continue;
      void *dst = (char *)c->frag + off * e;
      chk(launch_frag_pack(j.src, j.N, j.K, dst, c->stream));
      *j.dst = dst;
      off += frag_elems(j.N, j.K);
    }
    chk(hipStreamSynchronize(c->stream));
  }
  if (he != hipSuccess) {
    blt_destroy(c);
    return BLT_EHIP;
  }
  *out = c;
  return BLT_OK;
}

blt_status blt_destroy(blt_ctx *c) {
  if (!c) return BLT_EINVAL;
  (void)hipStreamSynchronize(c->stream);
  drop_graphs(c);
  if (c->cap_stream) (void)hipStreamDestroy(c->cap_stream);
  void *bufs[] = {c->h, c->qkv, c->q, c->part, c->logits, c->split.ws, c->conf_ws, c->ent_ws, c->argmax_ws,
                  c->xa, c->xb, c->desc_d, c->rope_tab, c->cross_w, c->frag};
  for (void *p : bufs)
    if (p) (void)hipFree(p);
  for (int i = 0; i < kRing; ++i) {
    if (c->ring[i].host) (void)hipHostFree(c->ring[i].host);
    if (c->ring[i].ev) (void)hipEventDestroy(c->ring[i].ev);
  }
  for (ProfRec &r : c->prof_pool) {
    if (r.ev0) (void)hipEventDestroy(r.ev0);
    if (r.ev1) (void)hipEventDestroy(r.ev1);
  }
  delete c;
  return BLT_OK;
}

blt_status blt_latents_put(blt_ctx *c, const blt_state *st, int32_t n, const int32_t *slot,
                           const int32_t *idx, const void *table, int64_t seq_stride) {
  if (!c) return BLT_EINVAL;
  const blt_config &g = c->cfg;
  if (!st || !st->cross || n < 0 || (n > 0 && (!slot || !idx || !table)) || seq_stride < 0)
    return fail(c, BLT_EINVAL, "blt_latents_put: bad argument");
  for (int i = 0; i < n; ++i) {
    if (slot[i] < 0 || slot[i] >= g.max_batch) return fail(c, BLT_EINVAL, "blt_latents_put: slot out of range");
    if (idx[i] < 0 || idx[i] >= g.max_latents) return fail(c, BLT_ECAPACITY, "blt_latents_put: latent index beyond max_latents");
  }
  const int d = g.d_model, L = g.n_layers;
  for (int i0 = 0; i0 < n; i0 += g.max_rows) {
    const int m = std::min(g.max_rows, n - i0);
    // staged offsets: the source rows of the latents, then their cross rows
    std::vector<int64_t> offs(2 * (size_t)m);
    for (int i = 0; i < m; ++i) {
      offs[i] = ((int64_t)slot[i0 + i] * seq_stride + idx[i0 + i]) * g.d_global;
      offs[m + i] = (((int64_t)slot[i0 + i] * g.max_latents + idx[i0 + i]) * L) * d;
    }
    std::vector<RowDesc> no_rows;
    std::vector<SeqDesc> no_seqs;
    blt_status bs = stage_pass(c, no_rows, no_seqs, &offs);
    if (bs != BLT_OK) return bs;
    // o~ = W_lat o  -> xb
    GemmArgs a = base_args(c);
    a.R = m; a.W = c->w.w_lat; a.Wf = c->frag_lat; a.N = d; a.K = g.d_global;
    a.pro = PRO_PLAIN; a.X = table; a.x_row_off = c->offs_d;
    a.ep = EP_STORE_ACT; a.out_act = c->xb; a.ldo = d;
    HIP_TRY(c, launch_gemm(c->bf16, a, c->xb, nullptr, c->stream, nullptr, nullptr, c->gemm_form));
    // cross[slot][idx][l][:] = C_l o~ for every layer at once (N = L*d)
    a = base_args(c);
    a.R = m; a.W = c->cross_w; a.Wf = c->frag_cross; a.N = L * d; a.K = d;
    a.pro = PRO_PLAIN; a.X = c->xb; a.ldx = d;
    a.ep = EP_ROWOFF_F32; a.out_f32 = (float *)st->cross; a.row_off = c->offs_d + m;
    HIP_TRY(c, launch_gemm(c->bf16, a, c->xb, nullptr, c->stream, nullptr, nullptr, c->gemm_form));
  }
  return BLT_OK;
}

static blt_status check_slots(blt_ctx *c, int32_t batch, const int32_t *slot, const char *fn) {
  const blt_config &g = c->cfg;
  char msg[160];
  if (batch < 1 || batch > g.max_batch || !slot) {
    snprintf(msg, sizeof(msg), "%s: bad batch or slot array", fn);
    return fail(c, BLT_EINVAL, (const char *)msg);
  }
  std::vector<char> &seen = c->seen_tmp;   // reserved at creation: no allocation here
  seen.assign(g.max_batch, 0);
  for (int b = 0; b < batch; ++b) {
    if (slot[b] < 0 || slot[b] >= g.max_batch) {
      snprintf(msg, sizeof(msg), "%s: slot out of range", fn);
      return fail(c, BLT_EINVAL, (const char *)msg);
    }
    if (seen[slot[b]]) {
      snprintf(msg, sizeof(msg), "%s: a slot appears twice in one pass", fn);
      return fail(c, BLT_EINVAL, (const char *)msg);
    }
    seen[slot[b]] = 1;
  }
  return BLT_OK;
}

// Validation of a sampling request shared by the decode calls.
static blt_status check_sampling(blt_ctx *c, const blt_sampling *sampling, const int32_t *draw,
                                 int32_t batch, const char *fn) {
  if (!sampling) return BLT_OK;
  if (!(sampling->temperature > 0.f) || !isfinite(sampling->temperature) ||
      !(sampling->top_p > 0.f && sampling->top_p <= 1.f) || !draw)
    return fail(c, BLT_EINVAL, std::string(fn) + ": sampling needs temperature > 0, 0 < top_p <= 1 and draw");
  for (int b = 0; b < batch; ++b)
    if (draw[b] < 0 || (int64_t)draw[b] * kMaxBlock + kMaxBlock > INT32_MAX)
      return fail(c, BLT_EINVAL, std::string(fn) + ": draw out of range");
  return BLT_OK;
}

// Rows of one blt_kv_append call; `noalloc` carves the pass workspace out of
// the static scratch array instead of the context's workspace.
static blt_status kv_append_impl(blt_ctx *c, const blt_state *st, int32_t batch, const int32_t *slot,
                                 const int32_t *start_pos, const int32_t *n_rows, int32_t n_max,
                                 const uint8_t *bytes, const int32_t *tokens_dev, const int32_t *lat_idx,
                                 int32_t *argmax_out, float *conf_out, float *logits_out,
                                 const blt_sampling *sampling, const int32_t *draw, bool noalloc) {
  if (!c) return BLT_EINVAL;
  const blt_config &g = c->cfg;
  const char *fn = noalloc ? "blt_kv_append_noalloc" : "blt_kv_append";
  if (!st || !st->kv || !st->cross) return fail(c, BLT_EINVAL, "blt_kv_append: state is NULL");
  blt_status bs = check_slots(c, batch, slot, fn);
  if (bs != BLT_OK) return bs;
  if (!start_pos || !n_rows || !lat_idx || n_max < 1 || (!bytes && !tokens_dev))
    return fail(c, BLT_EINVAL, "blt_kv_append: NULL argument or n_max < 1");
  bs = check_sampling(c, sampling, draw, batch, fn);
  if (bs != BLT_OK) return bs;
  if (sampling && n_max > kMaxBlock)
    return fail(c, BLT_EINVAL, "blt_kv_append: sampled passes take at most 64 rows per sequence");
  std::vector<RowDesc> &rows = c->rows_tmp;   // reserved at creation (max_rows, max_batch)
  std::vector<SeqDesc> &seqs = c->seqs_tmp;
  rows.clear();
  seqs.clear();
  int32_t *wr = c->written_rows(st);
  if (!wr) return fail(c, BLT_ECAPACITY, "blt_kv_append: more decode states than one context tracks (16)");
  for (int b = 0; b < batch; ++b) {
    const int n = n_rows[b], s0 = start_pos[b];
    if (n < 0 || n > n_max || s0 < 0) return fail(c, BLT_EINVAL, "blt_kv_append: bad n_rows or start_pos");
    if ((int64_t)s0 + n > g.max_ctx) return fail(c, BLT_ECAPACITY, "blt_kv_append: rows beyond max_ctx");
    if (n > 0 && s0 > wr[slot[b]])
      return fail(c, BLT_EINVAL, "blt_kv_append: start_pos beyond the rows already written for the slot");
    if (n == 0) continue;
    if ((int64_t)rows.size() + n > g.max_rows) return fail(c, BLT_ECAPACITY, "blt_kv_append: more rows than max_rows");
    if (noalloc && (int64_t)rows.size() + n > kNoAllocRows)
      return fail(c, BLT_ECAPACITY, "blt_kv_append_noalloc: more than 15 rows in one call");
    SeqDesc sd{slot[b], (int)rows.size(), n, s0 + n, -1, -1, 0, slot[b]};
    for (int j = 0; j < n; ++j) {
      const int li = lat_idx[(size_t)b * n_max + j];
      if (li < 0 || li >= g.max_latents) return fail(c, BLT_ECAPACITY, "blt_kv_append: latent index beyond max_latents");
      const int dj = slot[b] * n_max + j;  // device arrays are indexed by slot
      RowDesc rd{slot[b], s0 + j, bytes ? (int)bytes[(size_t)b * n_max + j] : kTokFromDev, dj, li,
                 s0 + j + 1, dj, 0, sampling ? draw[b] * kMaxBlock + j : -1};
      rows.push_back(rd);
    }
    seqs.push_back(sd);
  }
  if (rows.empty()) return BLT_OK;
  PassWs sw{};
  if (noalloc) {
    // the pass workspace, carved out of the static scratch array in 256-byte
    // aligned regions for this call's rows
    const size_t R = rows.size(), d = g.d_model, H = g.n_heads, dh = d / H;
    const size_t e = c->bf16 ? 2 : 4;
    size_t off = 0;
    auto take = [&](size_t bytes_) { const size_t o = off; off = (off + bytes_ + 255) & ~(size_t)255; return o; };
    const size_t o_seqs = take((size_t)g.max_batch * sizeof(SeqDesc)), o_rows = take(R * sizeof(RowDesc));
    const size_t o_h = take(R * d * 4), o_qkv = take(R * 3 * d * 4), o_q = take(R * d * 4);
    const size_t o_part = take(R * H * c->max_chunks * (dh + 2) * 4), o_lg = take(R * kVocab * 4);
    const size_t o_cf = take(R * 4), o_en = take(R * 4), o_am = take(R * 4);
    const size_t o_xa = take(R * std::max<size_t>(d, g.d_ffn) * e);
    const size_t o_xb = take(R * std::max<size_t>(d, g.d_global) * e);
    if (off > kScratchBytes)
      return fail(c, BLT_ECAPACITY, "blt_kv_append_noalloc: the pass needs more than the 32 MiB scratch array");
    void *base = nullptr;
    HIP_TRY(c, scratch_region(&base));
    char *b8 = (char *)base;
    sw = PassWs{(float *)(b8 + o_h), (float *)(b8 + o_qkv), (float *)(b8 + o_q), (float *)(b8 + o_part),
                (float *)(b8 + o_lg), (float *)(b8 + o_cf), (float *)(b8 + o_en), (int32_t *)(b8 + o_am),
                b8 + o_xa, b8 + o_xb, (SeqDesc *)(b8 + o_seqs), (RowDesc *)(b8 + o_rows)};
  }
  bs = run_pass(c, st, rows, seqs, nullptr, tokens_dev, false, 0.f, 0, nullptr, argmax_out,
                conf_out, logits_out, sampling, noalloc ? &sw : nullptr);
  if (bs == BLT_OK)
    for (const SeqDesc &sd : seqs) wr[sd.slot] = rows[sd.row0].pos + sd.nrows;
  return bs;
}

blt_status blt_kv_append(blt_ctx *c, const blt_state *st, int32_t batch, const int32_t *slot,
                         const int32_t *start_pos, const int32_t *n_rows, int32_t n_max,
                         const uint8_t *bytes, const int32_t *tokens_dev, const int32_t *lat_idx,
                         int32_t *argmax_out, float *conf_out, float *logits_out,
                         const blt_sampling *sampling, const int32_t *draw) {
  return kv_append_impl(c, st, batch, slot, start_pos, n_rows, n_max, bytes, tokens_dev, lat_idx,
                        argmax_out, conf_out, logits_out, sampling, draw, false);
}

blt_status blt_kv_append_noalloc(blt_ctx *c, const blt_state *st, int32_t batch, const int32_t *slot,
                                 const int32_t *start_pos, const int32_t *n_rows, int32_t n_max,
                                 const uint8_t *bytes, const int32_t *tokens_dev, const int32_t *lat_idx,
                                 int32_t *argmax_out, float *conf_out, float *logits_out,
                                 const blt_sampling *sampling, const int32_t *draw) {
  return kv_append_impl(c, st, batch, slot, start_pos, n_rows, n_max, bytes, tokens_dev, lat_idx,
                        argmax_out, conf_out, logits_out, sampling, draw, true);
}

blt_status blt_decode_block_step(blt_ctx *c, const blt_state *st, int32_t batch,
                                 const int32_t *slot, const int32_t *start_pos,
                                 const int32_t *n_append, int32_t n_append_max,
                                 const uint8_t *append_bytes, const int32_t *append_lat,
                                 int32_t *block_tok, int32_t B, const int32_t *block_lat,
                                 float alpha, blt_unmask mode, blt_block_mask mask,
                                 int32_t *argmax_out, float *conf_out, float *logits_out,
                                 int32_t *masked_left, const blt_sampling *sampling,
                                 const int32_t *draw) {
  if (!c) return BLT_EINVAL;
  const blt_config &g = c->cfg;
  static const char *fn = "blt_decode_block_step";
  if (!st || !st->kv || !st->cross) return fail(c, BLT_EINVAL, "blt_decode_block_step: state is NULL");
  blt_status bs = check_slots(c, batch, slot, fn);
  if (bs != BLT_OK) return bs;
  if (!start_pos || !block_tok || !block_lat || !masked_left)
    return fail(c, BLT_EINVAL, "blt_decode_block_step: NULL argument");
  if (B < 1 || B > g.max_block) return fail(c, BLT_ECAPACITY, "blt_decode_block_step: B outside 1..max_block");
  if (mode != BLT_UNMASK_THRESHOLD && mode != BLT_UNMASK_ONE_STEP && mode != BLT_UNMASK_ENTROPY)
    return fail(c, BLT_EINVAL, "blt_decode_block_step: bad unmask mode");
  if (mask != BLT_BLOCK_BIDIR && mask != BLT_BLOCK_CAUSAL) return fail(c, BLT_EINVAL, "blt_decode_block_step: bad block mask");
  if (mode == BLT_UNMASK_ENTROPY ? !(alpha >= 0.f) : !isfinite(alpha))
    return fail(c, BLT_EINVAL, "blt_decode_block_step: alpha must be finite (an entropy bound: >= 0, may be +inf)");
  if (n_append_max < 0 || (n_append_max > 0 && (!n_append || !append_bytes || !append_lat)))
    return fail(c, BLT_EINVAL, "blt_decode_block_step: bad append arguments");
  bs = check_sampling(c, sampling, draw, batch, fn);
  if (bs != BLT_OK) return bs;
  std::vector<RowDesc> rows;
  std::vector<SeqDesc> seqs;
  int32_t *wr = c->written_rows(st);
  if (!wr) return fail(c, BLT_ECAPACITY, "blt_decode_block_step: more decode states than one context tracks (16)");
  for (int b = 0; b < batch; ++b) {
    const int na = n_append_max > 0 ? n_append[b] : 0, s0 = start_pos[b];
    if (na < 0 || na > n_append_max || s0 < 0) return fail(c, BLT_EINVAL, "blt_decode_block_step: bad n_append or start_pos");
    const int64_t end = (int64_t)s0 + na + B;
    if (end > g.max_ctx) return fail(c, BLT_ECAPACITY, "blt_decode_block_step: block beyond max_ctx");
    if (s0 > wr[slot[b]])
      return fail(c, BLT_EINVAL, "blt_decode_block_step: start_pos beyond the rows already written for the slot");
    if ((int64_t)rows.size() + na + B > g.max_rows) return fail(c, BLT_ECAPACITY, "blt_decode_block_step: more rows than max_rows");
    const int bl = block_lat[b];
    if (bl < 0 || bl >= g.max_latents) return fail(c, BLT_ECAPACITY, "blt_decode_block_step: latent index beyond max_latents");
    SeqDesc sd{slot[b], (int)rows.size(), na + B, (int)end, slot[b] * B, (int)rows.size() + na, B,
               slot[b]};
    for (int j = 0; j < na; ++j) {
      const int li = append_lat[(size_t)b * n_append_max + j];
      if (li < 0 || li >= g.max_latents) return fail(c, BLT_ECAPACITY, "blt_decode_block_step: latent index beyond max_latents");
      rows.push_back(RowDesc{slot[b], s0 + j, (int)append_bytes[(size_t)b * n_append_max + j], 0, li,
                             s0 + j + 1, -1, 0, -1});
    }
    for (int j = 0; j < B; ++j) {
      const int pos = s0 + na + j;
      rows.push_back(RowDesc{slot[b], pos, kTokFromBlock, slot[b] * B + j, bl,
                             mask == BLT_BLOCK_CAUSAL ? pos + 1 : (int)end, slot[b] * B + j, 0,
                             sampling ? draw[b] * kMaxBlock + j : -1});
    }
    seqs.push_back(sd);
  }
  bs = run_pass(c, st, rows, seqs, block_tok, nullptr, true, alpha, (int)mode,
                masked_left, argmax_out, conf_out, logits_out, sampling);
  if (bs == BLT_OK)
    for (const SeqDesc &sd : seqs) wr[sd.slot] = rows[sd.row0].pos + (sd.nrows - sd.nblk);
  return bs;
}

blt_status blt_verify_accept(blt_ctx *c, int32_t batch, const int32_t *slot, int32_t r,
                             const int32_t *draft, int32_t ld_draft, const int32_t *pred,
                             int32_t ld_pred, int32_t *accept_len, int32_t *next_byte) {
  if (!c) return BLT_EINVAL;
  if (batch < 1 || batch > c->cfg.max_batch || r < 0 || !draft || !pred || !accept_len ||
      !next_byte || ld_draft < r || ld_pred < r + 1)
    return fail(c, BLT_EINVAL, "blt_verify_accept: bad argument");
  std::vector<SeqDesc> seqs(batch);
  for (int b = 0; b < batch; ++b) {
    const int s = slot ? slot[b] : b;
    if (s < 0 || s >= c->cfg.max_batch) return fail(c, BLT_EINVAL, "blt_verify_accept: slot out of range");
    seqs[b] = SeqDesc{s, 0, 0, 0, 0, 0, 0, s};
  }
  std::vector<RowDesc> no_rows;
  blt_status bs = stage_pass(c, no_rows, seqs, nullptr);
  if (bs != BLT_OK) return bs;
  HIP_TRY(c, launch_verify(batch, c->seqs_d, r, draft, ld_draft, pred, ld_pred, accept_len,
                           next_byte, c->stream));
  return BLT_OK;
}

blt_status blt_verify_sample(blt_ctx *c, int32_t batch, const int32_t *slot, int32_t r,
                             const int32_t *draft, int32_t ld_draft, const float *zq, int32_t ld_q,
                             const float *zp, int32_t ld_p, const blt_sampling *sampling,
                             const int32_t *draw, int32_t *accept_len, int32_t *next_byte) {
  if (!c) return BLT_EINVAL;
  static const char *fn = "blt_verify_sample";
  if (batch < 1 || batch > c->cfg.max_batch || r < 0 || r >= kMaxBlock || !draft || !zq || !zp ||
      !accept_len || !next_byte || !sampling || ld_draft < r || ld_q < r || ld_p < r + 1)
    return fail(c, BLT_EINVAL, "blt_verify_sample: bad argument (r must be below 64)");
  blt_status bs = check_sampling(c, sampling, draw, batch, fn);
  if (bs != BLT_OK) return bs;
  std::vector<SeqDesc> seqs(batch);
  std::vector<int64_t> draws(batch);
  for (int b = 0; b < batch; ++b) {
    const int s = slot ? slot[b] : b;
    if (s < 0 || s >= c->cfg.max_batch) return fail(c, BLT_EINVAL, "blt_verify_sample: slot out of range");
    seqs[b] = SeqDesc{s, 0, 0, 0, 0, 0, 0, s};
    draws[b] = draw[b];
  }
  std::vector<RowDesc> no_rows;
  bs = stage_pass(c, no_rows, seqs, &draws);
  if (bs != BLT_OK) return bs;
  const SampleArgs smp{sampling->temperature, sampling->top_p, sampling->seed};
  HIP_TRY(c, launch_verify_sample(batch, c->seqs_d, c->offs_d, r, draft, ld_draft, zq, ld_q, zp, ld_p,
                                  smp, accept_len, next_byte, c->stream));
  return BLT_OK;
}

blt_status blt_profile_enable(blt_ctx *c, int32_t family) {
  if (!c) return BLT_EINVAL;
  if (family < BLT_PROF_OFF || family > BLT_PROF_GEMM)
    return fail(c, BLT_EINVAL, "blt_profile_enable: unknown kernel family");
  if (family != BLT_PROF_OFF && c->prof_pool.empty()) {
    c->prof_pool.resize(4096);
    for (ProfRec &r : c->prof_pool) {
      HIP_TRY(c, hipEventCreate(&r.ev0));
      HIP_TRY(c, hipEventCreate(&r.ev1));
    }
  }
  blt_status bs = prof_collect(c);
  c->prof_family = family;
  return bs;
}

blt_status blt_graphs_enable(blt_ctx *c, int32_t enable) {
  if (!c) return BLT_EINVAL;
  if (!enable) drop_graphs(c);
  c->graphs = enable != 0;
  return BLT_OK;
}

blt_status blt_attention_chunks(blt_ctx *c, int32_t chunks) {
  if (!c) return BLT_EINVAL;
  if (chunks < 0) return fail(c, BLT_EINVAL, "blt_attention_chunks: chunks must be >= 0");
  c->attn_chunks = chunks;
  return BLT_OK;
}

blt_status blt_flash_key_groups(blt_ctx *c, int32_t groups) {
  if (!c) return BLT_EINVAL;
  if (groups < 0 || groups > 2) return fail(c, BLT_EINVAL, "blt_flash_key_groups: groups must be 0, 1 or 2");
  if (groups != c->flash_kg) drop_graphs(c);   // captured passes keep the form they were captured with
  c->flash_kg = groups;
  return BLT_OK;
}

blt_status blt_gemm_form(blt_ctx *c, int32_t form) {
  if (!c) return BLT_EINVAL;
  if (form < 0 || form > 2) return fail(c, BLT_EINVAL, "blt_gemm_form: form must be 0, 1 or 2");
  if (form != c->gemm_form) drop_graphs(c);   // captured passes keep the kernels they were captured with
  c->gemm_form = form;
  return BLT_OK;
}

blt_status blt_profile_read(blt_ctx *c, uint64_t *launches, double *total_ms, double *bytes,
                            int32_t reset) {
  if (!c || !launches || !total_ms || !bytes) return BLT_EINVAL;
  blt_status bs = prof_collect(c);
  if (bs != BLT_OK) return bs;
  *launches = c->prof_launches;
  *total_ms = c->prof_ms;
  *bytes = c->prof_bytes;
  if (reset) {
    c->prof_launches = 0;
    c->prof_ms = c->prof_bytes = 0;
  }
  return BLT_OK;
}

blt_status blt_bw_model(const blt_counts *cn, const blt_params *p, uint64_t *bytes_total,
                        double *gb_per_seq) {
  if (!cn || !p || !bytes_total || cn->n_seq == 0) return BLT_EINVAL;
  uint64_t a, b, eg, sum, tot;
  if (__builtin_mul_overflow(cn->n_dec, p->p_dec, &a)) return BLT_EINVAL;
  if (__builtin_add_overflow(p->p_enc, p->p_glob, &eg)) return BLT_EINVAL;
  if (__builtin_mul_overflow(cn->n_encglob, eg, &b)) return BLT_EINVAL;
  if (__builtin_add_overflow(a, b, &sum)) return BLT_EINVAL;
  if (__builtin_mul_overflow(sum, (uint64_t)p->bytes_per_param, &tot)) return BLT_EINVAL;
  *bytes_total = tot;
  if (gb_per_seq) *gb_per_seq = (double)tot / 1e9 / (double)cn->n_seq;
  return BLT_OK;
}

}  // extern "C"
