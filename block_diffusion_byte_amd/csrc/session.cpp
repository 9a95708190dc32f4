// Native host drivers of the decoding policies (greedy BLT, BLT-D, BLT-S,
// BLT-DV) over the decoder-step calls, with the pass counters of the
// efficiency metrics.  Sequences of a batch advance independently inside
// lock-step passes: a sequence whose block is full, or that has produced its
// bytes, leaves the following passes.
//
// Policies (pytorch.kr Fast-BLT summary):
//  * greedy BLT: one decoder pass per byte over the newest byte's row; before
//    a row that ends a patch, an encoder/global pass delivers that patch's
//    latent ("BLT architecture": the global model runs once per patch).
//  * BLT-D ("BLT-D inference"): per block an encoder/global pass, then
//    x' = [x; MASK x B] and decoder passes until the block is filled.  Block
//    rows and the last prefix byte read the last latent o_M; cached rows whose
//    latent changed are recomputed (rollback to the first of them).
//  * BLT-S ("BLT-S"): k autoregressive draft passes without the
//    encoder/global model, one encoder/global pass over the draft, one causal
//    pass over rows l..l+k, greedy exact-match acceptance.
//  * BLT-DV ("BLT-DV"): an encoder/global pass and a BLT-D block draft, an
//    encoder/global pass over the draft, a causal pass, the same acceptance.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "blt_ctx.h"
#include "host_patcher.h"

using namespace blt;

namespace {

struct SeqState {
  std::vector<uint8_t> prompt;
  std::vector<int32_t> plens;
  uint64_t salt = 0;
  std::vector<uint8_t> x;
  Seg seg;
  int cache_len = 0;
  std::vector<int32_t> ctau;    // latent each cached row was computed with
  int lat_ready = 0;            // latents 0..lat_ready-1 have cross vectors
  int avail = -1;               // newest latent the decoder may read
  uint64_t n_dec = 0, n_eg = 0, rounds = 0, accepted = 0;
  // prefilled snapshot
  Seg seg0;
  int cache0 = 0, lat0 = 0, avail0 = -1;
  std::vector<int32_t> ctau0;
};

}  // namespace

struct blt_session {
  blt_ctx *ctx = nullptr;
  blt_state st{};
  int batch = 0;
  const void *table = nullptr;
  int n_lat = 0;
  std::vector<SeqState> seqs;
  bool prefilled = false;
  int32_t *dev = nullptr;       // device scratch (ints)
  int32_t *host = nullptr;      // pinned mirror (mapped into the device's address space)
  int32_t *host_dev = nullptr;  // the mirror's device address
  size_t dev_n = 0;
  // device regions (offsets into dev)
  size_t o_blk = 0, o_masked = 0, o_draft = 0, o_pred = 0, o_acc = 0, o_next = 0;
  int W = 0;                    // per-slot width of the draft / pred regions
  // sampled drafts: logits each draft byte was drawn from, [slot][W][257],
  // and the verify rows' logits, [slot][W][257] (device f32)
  float *zq = nullptr, *zp = nullptr;
  int32_t *blk_before = nullptr;  // block tokens before a sampled draft pass [slot][B]
  // sampling of the current generate call (temperature 0: greedy)
  blt_sampling smp{0.f, 1.f, 0};
  bool sampled = false;
  // device-resident BLT-D blocks (blt_session_device_blocks): 0 off, 1 on,
  // 2 chosen from the first host-driven blocks, 3 on with the streaming
  // kernels testing the gate late
  int device_blocks = 0;
  struct DevBufs {
    int B = 0;                       // block size the buffers were laid out for
    DevSeq *st = nullptr;
    int32_t *x = nullptr;            // [batch][max_ctx]
    RowDesc *rows0 = nullptr, *rows1 = nullptr;
    SeqDesc *seqs0 = nullptr, *seqs1 = nullptr;
    int64_t *lat_offs = nullptr;
    int32_t *ints = nullptr;         // gate, then pass counts, n_eg and masked counts [batch] each
  } db;
};

namespace {

blt_status sfail(blt_session *s, blt_status st, const std::string &m) {
  s->ctx->err = m;
  return st;
}

#define S_TRY(expr)                          \
  do {                                       \
    blt_status _b = (expr);                  \
    if (_b != BLT_OK) return _b;             \
  } while (0)

#define S_HIP(s, expr)                                                          \
  do {                                                                          \
    hipError_t _e = (expr);                                                     \
    if (_e != hipSuccess)                                                       \
      return sfail((s), BLT_EHIP, std::string(#expr) + ": " + hipGetErrorString(_e)); \
  } while (0)

// One encoder/global pass for each listed sequence: latents up to `upto[i]`
// become readable (cross vectors computed for the new ones) and it counts.
blt_status encglob(blt_session *s, const std::vector<int> &who, const std::vector<int> &upto) {
  std::vector<int32_t> slot, idx;
  for (size_t i = 0; i < who.size(); ++i) {
    SeqState &q = s->seqs[who[i]];
    if (upto[i] >= s->n_lat || upto[i] >= s->ctx->cfg.max_latents)
      return sfail(s, BLT_ECAPACITY, "session: sequence needs more latents than the table holds");
    for (int m = q.lat_ready; m <= upto[i]; ++m) {
      slot.push_back(who[i]);
      idx.push_back(m);
    }
    q.lat_ready = std::max(q.lat_ready, upto[i] + 1);
    q.n_eg += 1;
  }
  if (slot.empty()) return BLT_OK;
  return blt_latents_put(s->ctx, &s->st, (int)slot.size(), slot.data(), idx.data(), s->table,
                         s->n_lat);
}

blt_status readback(blt_session *s, size_t off, size_t n) {
  S_HIP(s, hipMemcpyAsync(s->host + off, s->dev + off, n * sizeof(int32_t), hipMemcpyDeviceToHost,
                          s->ctx->stream));
  S_HIP(s, hipStreamSynchronize(s->ctx->stream));
  return BLT_OK;
}

// Small per-pass results (masked counts, greedy bytes, acceptance) are
// written by the kernels straight into the pinned mirror, which the device
// reaches through its mapping: reading them needs only the stream to drain.
int32_t *mapped(blt_session *s, size_t off) { return s->host_dev + off; }

blt_status drain(blt_session *s) {
  S_HIP(s, hipStreamSynchronize(s->ctx->stream));
  return BLT_OK;
}

// Wait for per-sequence results the pass's last kernel writes into the
// mapped mirror: each listed entry was set to -1 before the pass, so the
// host can go on as soon as every entry has been written, without waiting
// for the stream's completion to be signalled.  A bounded spin; past it (or
// on a stream error) the stream is synchronised as usual.
blt_status await_mapped(blt_session *s, size_t off, const std::vector<int> &who) {
  volatile int32_t *h = s->host + off;
  for (long spin = 0; spin < (1l << 22); ++spin) {
    bool all = true;
    for (int b : who)
      if (h[b] < 0) { all = false; break; }
    if (all) return BLT_OK;
    if ((spin & 4095) == 4095 && hipStreamQuery(s->ctx->stream) != hipErrorNotReady) break;
  }
  return drain(s);
}

blt_status upload(blt_session *s, size_t off, size_t n) {
  S_HIP(s, hipMemcpyAsync(s->dev + off, s->host + off, n * sizeof(int32_t), hipMemcpyHostToDevice,
                          s->ctx->stream));
  return BLT_OK;
}

// Draw index of each listed sequence's next decoder pass: its decoder
// passes so far in this generation.
std::vector<int32_t> draws_of(blt_session *s, const std::vector<int> &who) {
  std::vector<int32_t> d;
  for (int b : who) d.push_back((int32_t)s->seqs[b].n_dec);
  return d;
}

void commit(SeqState &q, uint8_t b, int n_gen) {
  if ((int)(q.x.size() - q.prompt.size()) >= n_gen) return;
  q.seg.push(q.salt, q.x.back(), b);
  q.x.push_back(b);
}

bool done(const SeqState &q, int n_gen) { return (int)(q.x.size() - q.prompt.size()) >= n_gen; }

void free_dev_blocks(blt_session *s) {
  void *p[] = {s->db.st, s->db.x, s->db.rows0, s->db.rows1, s->db.seqs0, s->db.seqs1, s->db.lat_offs,
               s->db.ints};
  for (void *q : p)
    if (q) (void)hipFree(q);
  s->db = blt_session::DevBufs{};
}

// ---------------------------------------------------------------- greedy
blt_status run_greedy(blt_session *s, int n_gen) {
  const int W = s->W;
  while (true) {
    std::vector<int> act;
    for (int b = 0; b < s->batch; ++b)
      if (!done(s->seqs[b], n_gen)) act.push_back(b);
    if (act.empty()) return BLT_OK;
    std::vector<int> eg_who, eg_upto;
    std::vector<int32_t> slot, start, nrow, lat;
    std::vector<uint8_t> bytes;
    for (int b : act) {
      SeqState &q = s->seqs[b];
      const size_t i = q.x.size() - 1;
      const int tau = q.seg.causal_target(i);
      if (tau > q.avail) {
        q.avail = q.seg.last_complete;
        eg_who.push_back(b);
        eg_upto.push_back(q.avail);
      }
      slot.push_back(b);
      start.push_back((int32_t)i);
      nrow.push_back(1);
      lat.push_back(tau);
      bytes.push_back(q.x[i]);
    }
    S_TRY(encglob(s, eg_who, eg_upto));
    const std::vector<int32_t> dw = draws_of(s, act);
    for (int b : act) s->host[s->o_pred + b] = -1;
    S_TRY(blt_kv_append(s->ctx, &s->st, (int)act.size(), slot.data(), start.data(), nrow.data(), 1,
                        bytes.data(), nullptr, lat.data(), mapped(s, s->o_pred), nullptr, nullptr,
                        s->sampled ? &s->smp : nullptr, s->sampled ? dw.data() : nullptr));
    S_TRY(await_mapped(s, s->o_pred, act));
    for (size_t k = 0; k < act.size(); ++k) {
      SeqState &q = s->seqs[act[k]];
      q.cache_len = start[k] + 1;
      q.ctau.resize(q.cache_len);
      q.ctau[start[k]] = lat[k];
      q.n_dec += 1;
      commit(q, (uint8_t)s->host[s->o_pred + act[k]], n_gen);
    }
    (void)W;
  }
}

// ---------------------------------------------------------------- BLT-D block
// One block for every sequence in `act`: encoder/global pass, then passes
// until no [MASK] is left.  The filled block is left in host[o_blk + slot*B].
blt_status block_draft(blt_session *s, const std::vector<int> &act, const blt_policy_args &pa) {
  const int B = pa.block;
  std::vector<int> eg_upto;
  for (int b : act) {
    SeqState &q = s->seqs[b];
    q.avail = q.seg.last_target();
    eg_upto.push_back(q.avail);
  }
  S_TRY(encglob(s, act, eg_upto));
  // first pass: clean rows from the first row whose latent changed (or is
  // not cached yet) to the last prefix byte, then the block
  std::vector<int32_t> slot, start, nap, blat;
  std::vector<std::vector<int32_t>> reqs(act.size());
  int na_max = 0;
  for (size_t k = 0; k < act.size(); ++k) {
    SeqState &q = s->seqs[act[k]];
    const int n = (int)q.x.size();
    std::vector<int32_t> &req = reqs[k];
    req.resize(n);
    for (int i = 0; i < n - 1; ++i) req[i] = q.seg.causal_target(i);
    req[n - 1] = q.seg.last_target();
    int first = q.cache_len;
    for (int i = 0; i < q.cache_len; ++i)
      if (q.ctau[i] != req[i]) { first = i; break; }
    slot.push_back(act[k]);
    start.push_back(first);
    nap.push_back(n - first);
    blat.push_back(q.seg.last_target());
    na_max = std::max(na_max, n - first);
    for (int j = 0; j < B; ++j) s->host[s->o_blk + (size_t)act[k] * B + j] = kMask;
  }
  std::vector<uint8_t> abytes((size_t)act.size() * std::max(na_max, 1), 0);
  std::vector<int32_t> alat((size_t)act.size() * std::max(na_max, 1), 0);
  for (size_t k = 0; k < act.size(); ++k) {
    SeqState &q = s->seqs[act[k]];
    for (int j = 0; j < nap[k]; ++j) {
      abytes[k * na_max + j] = q.x[start[k] + j];
      alat[k * na_max + j] = reqs[k][start[k] + j];
    }
  }
  S_TRY(upload(s, s->o_blk, (size_t)s->batch * B));
  const blt_unmask um = pa.unmask;
  std::vector<int> cur = act;
  std::vector<int32_t> cslot = slot, cstart = start, cnap = nap, cblat = blat;
  bool first_pass = true;
  // sampled passes: stream seed + b, draw = the sequence's decoder passes so
  // far; each block position keeps in zq[slot][j] the logits of the pass that
  // committed it (the distribution its byte was drawn from, which a BLT-DV
  // draft is verified against): the pass writes every block row's logits to
  // zp and the positions it committed are copied to zq
  const int nslot = s->ctx->cfg.max_batch;
  while (!cur.empty()) {
    const std::vector<int32_t> cdraw = draws_of(s, cur);
    for (int b : cur) s->host[s->o_masked + b] = -1;
    if (s->sampled)
      S_HIP(s, hipMemcpyAsync(s->blk_before, s->dev + s->o_blk, sizeof(int32_t) * (size_t)nslot * B,
                              hipMemcpyDeviceToDevice, s->ctx->stream));
    S_TRY(blt_decode_block_step(s->ctx, &s->st, (int)cur.size(), cslot.data(), cstart.data(),
                                first_pass ? cnap.data() : nullptr, first_pass ? na_max : 0,
                                first_pass ? abytes.data() : nullptr,
                                first_pass ? alat.data() : nullptr, s->dev + s->o_blk, B,
                                cblat.data(), pa.alpha, um, pa.block_mask, nullptr, nullptr,
                                s->sampled ? s->zp : nullptr, mapped(s, s->o_masked),
                                s->sampled ? &s->smp : nullptr,
                                s->sampled ? cdraw.data() : nullptr));
    if (s->sampled)
      S_HIP(s, launch_keep_drawn(s->blk_before, s->dev + s->o_blk, s->zp, s->zq, nslot, B,
                                 s->ctx->stream));
    S_TRY(await_mapped(s, s->o_masked, cur));
    if (first_pass) {
      for (size_t k = 0; k < act.size(); ++k) {
        SeqState &q = s->seqs[act[k]];
        const int n = (int)q.x.size();
        q.ctau.resize(n);
        for (int i = start[k]; i < n; ++i) q.ctau[i] = reqs[k][i];
        q.cache_len = n;
      }
    }
    std::vector<int> nxt;
    std::vector<int32_t> ns, nst, nbl;
    for (size_t k = 0; k < cur.size(); ++k) {
      SeqState &q = s->seqs[cur[k]];
      q.n_dec += 1;
      if (s->host[s->o_masked + cur[k]] > 0) {
        nxt.push_back(cur[k]);
        ns.push_back(cslot[k]);
        nst.push_back((int32_t)q.x.size());
        nbl.push_back(cblat[k]);
      }
    }
    cur.swap(nxt);
    cslot.swap(ns);
    cstart.swap(nst);
    cblat.swap(nbl);
    first_pass = false;
  }
  return readback(s, s->o_blk, (size_t)s->batch * B);
}

blt_status run_blt_d_device(blt_session *s, const blt_policy_args &pa);

// Host-driven blocks the automatic choice of device-resident blocks watches
// before it decides.
constexpr int kAutoBlocks = 4;

blt_status run_blt_d(blt_session *s, const blt_policy_args &pa) {
  bool first = true;
  // automatic choice: device-resident blocks pay for every one of a block's B
  // passes, including those a block no longer needs (their kernels return at
  // once, but are still launched), so they are taken only when every watched
  // block needed all B passes (one byte committed per pass); and only for one
  // sequence, whose short passes make the host's turn-around between them a
  // visible share (with 16 sequences a pass is long, and the device block's
  // extra work, B+1 rows recomputed and B+1 latent requests, outweighs it)
  int watched = 0;
  bool every_pass_needed = true;
  std::vector<uint64_t> n_dec0(s->batch);
  while (true) {
    std::vector<int> act;
    for (int b = 0; b < s->batch; ++b)
      if (!done(s->seqs[b], pa.n_gen)) act.push_back(b);
    if (act.empty()) return BLT_OK;
    const blt_config &g = s->ctx->cfg;
    // after the first block (which appends the prompt's pending byte alone),
    // every block of every sequence has the same shape: the rest runs on the
    // device when it fits the context's rows
    const bool dev = s->device_blocks == 1 || s->device_blocks == 3 ||
                     (s->device_blocks == 2 && s->batch == 1 && watched >= kAutoBlocks &&
                      every_pass_needed);
    if (!first && dev && !s->sampled && (int)act.size() == s->batch &&
        s->ctx->prof_family == BLT_PROF_OFF && s->batch * (2 * pa.block + 1) <= g.max_rows &&
        s->batch * (pa.block + 1) <= g.max_rows)
      return run_blt_d_device(s, pa);
    for (int b : act) n_dec0[b] = s->seqs[b].n_dec;
    S_TRY(block_draft(s, act, pa));
    // the first block may be shorter (the prompt's pending byte); later ones
    // are watched
    if (!first) {
      for (int b : act)
        if (s->seqs[b].n_dec - n_dec0[b] != (uint64_t)pa.block) every_pass_needed = false;
      ++watched;
    }
    first = false;
    for (int b : act)
      for (int j = 0; j < pa.block; ++j)
        commit(s->seqs[b], (uint8_t)s->host[s->o_blk + (size_t)b * pa.block + j], pa.n_gen);
  }
}

// ---------------------------------------------------------------- device-resident blocks
// The remaining BLT-D blocks of every sequence with no host round trip: per
// block the plan kernel (encoder/global pass and the first pass's rows), the
// latent projections, B decoder passes (a pass with no [MASK] left in any
// sequence returns at once in every kernel and is not counted) and the
// commit kernel (bytes and the stand-in patcher).  One block is captured as a
// HIP graph and replayed; the host reads the bytes and counters back once.
blt_status run_blt_d_device(blt_session *s, const blt_policy_args &pa) {
  blt_ctx *c = s->ctx;
  const blt_config &g = c->cfg;
  const int S = s->batch, B = pa.block, X = g.max_ctx;
  const int gen0 = (int)(s->seqs[0].x.size() - s->seqs[0].prompt.size());
  const int nb = (pa.n_gen - gen0 + B - 1) / B;
  if (nb <= 0) return BLT_OK;
  auto &db = s->db;
  if (db.B != B) {
    free_dev_blocks(s);
    auto ok = [](hipError_t e) { return e == hipSuccess; };
    if (!ok(hipMalloc(&db.st, sizeof(DevSeq) * S)) || !ok(hipMalloc(&db.x, sizeof(int32_t) * (size_t)S * X)) ||
        !ok(hipMalloc(&db.rows0, sizeof(RowDesc) * (size_t)S * (2 * B + 1))) ||
        !ok(hipMalloc(&db.rows1, sizeof(RowDesc) * (size_t)S * B)) ||
        !ok(hipMalloc(&db.seqs0, sizeof(SeqDesc) * S)) || !ok(hipMalloc(&db.seqs1, sizeof(SeqDesc) * S)) ||
        !ok(hipMalloc(&db.lat_offs, sizeof(int64_t) * 2 * (size_t)S * (B + 1))) ||
        !ok(hipMalloc(&db.ints, sizeof(int32_t) * (1 + 3 * (size_t)S)))) {
      free_dev_blocks(s);
      return sfail(s, BLT_EHIP, "session: device block buffers could not be allocated");
    }
    db.B = B;
  }
  // each sequence's state after the host's first block
  std::vector<DevSeq> st(S);
  std::vector<int32_t> xs((size_t)S * X, 0), ints(1 + 2 * (size_t)S, 0);
  int n_max = 0;
  for (int b = 0; b < S; ++b) {
    SeqState &q = s->seqs[b];
    const int n = (int)q.x.size();
    // after a block the cache holds its prefix rows 0..n-B-1 (the last of
    // them read the block's latent and is recomputed by the next block)
    if (n < B + 1 || q.cache_len != n - B)
      return sfail(s, BLT_EINVAL, "session: device blocks need a filled first block");
    DevSeq &d = st[b];
    memset(&d, 0, sizeof(d));
    d.n = n;
    d.patch_last = q.seg.patch.back();
    d.cur_len = q.seg.cur_len;
    d.ends_last = q.seg.ends.back();
    d.lat_ready = q.lat_ready;
    d.salt = q.salt;
    for (int j = 0; j <= B; ++j) {
      d.win_patch[j] = q.seg.patch[n - B - 1 + j];
      d.win_ends[j] = q.seg.ends[n - B - 1 + j];
    }
    for (int i = 0; i < n; ++i) xs[(size_t)b * X + i] = q.x[i];
    n_max = std::max(n_max, n);
  }
  if (n_max + (int64_t)nb * B > X) return sfail(s, BLT_ECAPACITY, "session: device blocks beyond max_ctx");
  hipStream_t hs = c->stream;
  S_HIP(s, hipMemcpyAsync(db.st, st.data(), sizeof(DevSeq) * S, hipMemcpyHostToDevice, hs));
  S_HIP(s, hipMemcpyAsync(db.x, xs.data(), sizeof(int32_t) * xs.size(), hipMemcpyHostToDevice, hs));
  S_HIP(s, hipMemcpyAsync(db.ints, ints.data(), sizeof(int32_t) * ints.size(), hipMemcpyHostToDevice, hs));
  int32_t *gate = db.ints, *pass_count = db.ints + 1, *n_eg = db.ints + 1 + S;
  // the per-pass masked counts stay on the device (no host reads them here;
  // in host-mapped memory every unmask kernel would wait for its PCIe write)
  int32_t *masked_dev = db.ints + 1 + 2 * S;
  DevBlockArgs a{db.st, db.x, X, S, B, pa.block_mask == BLT_BLOCK_CAUSAL ? 1 : 0, db.rows0, db.seqs0,
                 db.rows1, db.seqs1, db.lat_offs, s->dev + s->o_blk, masked_dev, gate, n_eg,
                 g.max_latents, s->n_lat, g.d_global, g.n_layers, g.d_model, (int64_t)s->n_lat};
  // attention over the longest context of the last block
  const int grid_chunks = (n_max + nb * B + kAttnChunk - 1) / kAttnChunk;
  // chosen automatically, the blocks are known to need all their passes (or
  // the caller says so, mode 3): the streaming kernels then test the gate
  // only before their stores
  const bool late = s->device_blocks == 2 || s->device_blocks == 3;
  auto enqueue_block = [&](hipStream_t q) -> blt_status {
    S_HIP(s, launch_block_plan(a, q));
    S_TRY(latents_from_device(c, &s->st, S * (B + 1), db.lat_offs, s->table, q));
    for (int p = 0; p < B; ++p)
      S_TRY(enqueue_device_pass(c, &s->st, S * (p ? B : 2 * B + 1), S, grid_chunks, p ? db.rows1 : db.rows0,
                                p ? db.seqs1 : db.seqs0, s->dev + s->o_blk, pa.alpha, (int)pa.unmask,
                                masked_dev, gate, pass_count, p ? B : 2 * B + 1, q,
                                late));
    S_HIP(s, launch_block_commit(a, q));
    return BLT_OK;
  };
  // the block is captured once and replayed; without a graph it is enqueued directly
  hipGraphExec_t exec = nullptr;
  if (c->graphs) {
    hipGraph_t graph = nullptr;
    if (hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal) == hipSuccess) {
      const blt_status ls = enqueue_block(c->cap_stream);
      const hipError_t ee = hipStreamEndCapture(c->cap_stream, &graph);
      if (ls != BLT_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        return ls;
      }
      if (ee == hipSuccess && graph && hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess)
        exec = nullptr;
      if (graph) (void)hipGraphDestroy(graph);
    }
  }
  for (int k = 0; k < nb; ++k) {
    if (exec) {
      const hipError_t e = hipGraphLaunch(exec, hs);
      if (e != hipSuccess) {
        (void)hipGraphExecDestroy(exec);
        return sfail(s, BLT_EHIP, std::string("hipGraphLaunch: ") + hipGetErrorString(e));
      }
    } else {
      S_TRY(enqueue_block(hs));
    }
  }
  if (exec) (void)hipGraphExecDestroy(exec);
  S_HIP(s, hipMemcpyAsync(st.data(), db.st, sizeof(DevSeq) * S, hipMemcpyDeviceToHost, hs));
  S_HIP(s, hipMemcpyAsync(xs.data(), db.x, sizeof(int32_t) * xs.size(), hipMemcpyDeviceToHost, hs));
  S_HIP(s, hipMemcpyAsync(ints.data(), db.ints, sizeof(int32_t) * ints.size(), hipMemcpyDeviceToHost, hs));
  S_HIP(s, hipStreamSynchronize(hs));
  int32_t *wr = c->written_rows(&s->st);
  for (int b = 0; b < S; ++b) {
    SeqState &q = s->seqs[b];
    if (st[b].err) return sfail(s, BLT_ECAPACITY, "session: a device block read a latent or byte out of range");
    const int keep = std::min(st[b].n, (int)q.prompt.size() + pa.n_gen);
    q.x.assign(xs.begin() + (size_t)b * X, xs.begin() + (size_t)b * X + keep);
    q.n_dec += (uint64_t)ints[1 + b];
    q.n_eg += (uint64_t)ints[1 + S + b];
    q.lat_ready = st[b].lat_ready;
    q.cache_len = st[b].n - B;      // clean rows the last block's first pass wrote
    if (wr) wr[b] = q.cache_len;
  }
  return BLT_OK;
}

// ---------------------------------------------------------------- verification
// Causal pass over rows l..l+r of each sequence's draft, then greedy
// exact-match acceptance on the device.  draft_dev holds the draft bytes at
// [slot*ld + j]; draft_host[k] the same bytes on the host.
blt_status verify_round(blt_session *s, const std::vector<int> &act,
                        const std::vector<std::vector<uint8_t>> &draft_host, int r,
                        const int32_t *draft_dev, int ld_draft, int n_gen, int ld_q) {
  const int n_max = r + 1;
  std::vector<int32_t> slot, start, nrow, lat((size_t)act.size() * n_max), eg_upto;
  std::vector<uint8_t> bytes((size_t)act.size() * n_max);
  std::vector<Seg> dseg(act.size());
  for (size_t k = 0; k < act.size(); ++k) {
    SeqState &q = s->seqs[act[k]];
    const size_t l = q.x.size() - 1;
    Seg sg = q.seg;   // segmentation of the draft continues from the committed bytes
    uint8_t prev = q.x[l];
    for (int j = 0; j < r; ++j) {
      sg.push(q.salt, prev, draft_host[k][j]);
      prev = draft_host[k][j];
    }
    int need = -1;
    for (int j = 0; j <= r; ++j) {
      lat[k * n_max + j] = sg.causal_target(l + j);
      need = std::max(need, lat[k * n_max + j]);
      bytes[k * n_max + j] = j == 0 ? q.x[l] : draft_host[k][j - 1];
    }
    eg_upto.push_back(std::max(need, q.avail));
    slot.push_back(act[k]);
    start.push_back((int32_t)l);
    nrow.push_back(n_max);
    dseg[k] = sg;
  }
  S_TRY(encglob(s, act, eg_upto));
  const std::vector<int32_t> dw = draws_of(s, act);
  S_TRY(blt_kv_append(s->ctx, &s->st, (int)act.size(), slot.data(), start.data(), nrow.data(),
                      n_max, bytes.data(), nullptr, lat.data(), s->dev + s->o_pred, nullptr,
                      s->sampled ? s->zp : nullptr, nullptr, nullptr));
  for (int b : act) s->host[s->o_acc + b] = s->host[s->o_next + b] = -1;
  if (s->sampled)
    S_TRY(blt_verify_sample(s->ctx, (int)act.size(), slot.data(), r, draft_dev, ld_draft, s->zq,
                            ld_q, s->zp, n_max, &s->smp, dw.data(), mapped(s, s->o_acc),
                            mapped(s, s->o_next)));
  else
    S_TRY(blt_verify_accept(s->ctx, (int)act.size(), slot.data(), r, draft_dev, ld_draft,
                            s->dev + s->o_pred, n_max, mapped(s, s->o_acc), mapped(s, s->o_next)));
  S_TRY(await_mapped(s, s->o_acc, act));
  S_TRY(await_mapped(s, s->o_next, act));
  for (size_t k = 0; k < act.size(); ++k) {
    SeqState &q = s->seqs[act[k]];
    const int l = (int)q.x.size() - 1;
    const int a = s->host[s->o_acc + act[k]];
    const uint8_t nb = (uint8_t)s->host[s->o_next + act[k]];
    q.n_dec += 1;
    q.rounds += 1;
    q.accepted += (uint64_t)a;
    // rows l..l+a were computed from accepted bytes with their final latents
    q.cache_len = l + a + 1;
    q.ctau.resize(q.cache_len);
    for (int j = 0; j <= a; ++j) q.ctau[l + j] = lat[k * n_max + j];
    for (int j = 0; j < a; ++j) commit(q, draft_host[k][j], n_gen);
    // the encoder/global pass saw the draft: patches completed within the
    // accepted bytes have valid latents, the appended byte was never seen
    q.avail = q.seg.last_complete;
    commit(q, nb, n_gen);
  }
  return BLT_OK;
}

blt_status run_blt_s(blt_session *s, const blt_policy_args &pa) {
  const int k = pa.block, W = k + 1;
  while (true) {
    std::vector<int> act;
    for (int b = 0; b < s->batch; ++b)
      if (!done(s->seqs[b], pa.n_gen)) act.push_back(b);
    if (act.empty()) return BLT_OK;
    std::vector<int32_t> slot(act.begin(), act.end()), nrow(act.size(), 1), lat, start;
    std::vector<uint8_t> first_bytes;
    for (int b : act) {
      SeqState &q = s->seqs[b];
      // Draft rows read the newest latent available: the cap min(target,
      // avail) always equals avail, since avail is the newest complete patch
      // before the draft and every draft row's own target is at least that.
      if (q.avail < 0 || q.avail >= q.lat_ready)
        return sfail(s, BLT_EINVAL, "session: draft latent has no cross vectors");
      lat.push_back(q.avail);
      first_bytes.push_back(q.x.back());
    }
    // draft pass j writes its greedy byte to draft[slot*W + j] and reads the
    // previous one from there: no host round trip between draft passes
    int32_t *dr = s->dev + s->o_draft;
    for (int j = 0; j < k; ++j) {
      start.clear();
      for (int b : act) start.push_back((int32_t)(s->seqs[b].x.size() - 1 + j));
      std::vector<uint8_t> hb(first_bytes);
      std::vector<int32_t> lt(lat);
      // host arrays are [batch][n_max]; one row per sequence at column 0
      std::vector<uint8_t> hb2((size_t)act.size() * W, 0);
      std::vector<int32_t> lt2((size_t)act.size() * W, 0);
      for (size_t i = 0; i < act.size(); ++i) {
        hb2[i * W] = hb[i];
        lt2[i * W] = lt[i];
      }
      // sampled: the drawn byte goes to draft[slot*W + j] and the row's
      // logits to zq[slot][j]
      const std::vector<int32_t> dw = draws_of(s, act);
      S_TRY(blt_kv_append(s->ctx, &s->st, (int)act.size(), slot.data(), start.data(), nrow.data(),
                          W, j == 0 ? hb2.data() : nullptr, j == 0 ? nullptr : dr + (j - 1),
                          lt2.data(), dr + j, nullptr, s->sampled ? s->zq + (size_t)j * 257 : nullptr,
                          s->sampled ? &s->smp : nullptr, s->sampled ? dw.data() : nullptr));
      for (int b : act) s->seqs[b].n_dec += 1;
    }
    S_TRY(readback(s, s->o_draft, (size_t)s->batch * W));
    std::vector<std::vector<uint8_t>> dh(act.size(), std::vector<uint8_t>(k));
    for (size_t i = 0; i < act.size(); ++i)
      for (int j = 0; j < k; ++j) dh[i][j] = (uint8_t)s->host[s->o_draft + (size_t)act[i] * W + j];
    S_TRY(verify_round(s, act, dh, k, dr, W, pa.n_gen, W));
  }
}

blt_status run_blt_dv(blt_session *s, const blt_policy_args &pa) {
  const int B = pa.block;
  while (true) {
    std::vector<int> act;
    for (int b = 0; b < s->batch; ++b)
      if (!done(s->seqs[b], pa.n_gen)) act.push_back(b);
    if (act.empty()) return BLT_OK;
    S_TRY(block_draft(s, act, pa));
    std::vector<std::vector<uint8_t>> dh(act.size(), std::vector<uint8_t>(B));
    for (size_t i = 0; i < act.size(); ++i)
      for (int j = 0; j < B; ++j) dh[i][j] = (uint8_t)s->host[s->o_blk + (size_t)act[i] * B + j];
    S_TRY(verify_round(s, act, dh, B, s->dev + s->o_blk, B, pa.n_gen, B));
  }
}

}  // namespace

extern "C" {

blt_status blt_session_create(blt_ctx *ctx, const blt_state *st, int32_t batch,
                              const uint8_t *const *prompts, const int32_t *prompt_len,
                              const int32_t *const *patch_lens, const int32_t *n_patches,
                              const uint64_t *salt, const void *latent_table, int32_t n_latents,
                              blt_session **out) {
  if (!ctx || !out) return BLT_EINVAL;
  *out = nullptr;
  const blt_config &g = ctx->cfg;
  auto bad = [&](const char *m) { ctx->err = m; return BLT_EINVAL; };
  if (!st || !st->kv || !st->cross) return bad("blt_session_create: state is NULL");
  if (batch < 1 || batch > g.max_batch) return bad("blt_session_create: batch outside 1..max_batch");
  if (!prompts || !prompt_len || !patch_lens || !n_patches || !salt || !latent_table || n_latents < 1)
    return bad("blt_session_create: NULL argument");
  blt_session *s = new (std::nothrow) blt_session();
  if (!s) return BLT_EINVAL;
  s->ctx = ctx;
  s->st = *st;
  s->batch = batch;
  s->table = latent_table;
  s->n_lat = n_latents;
  s->seqs.resize(batch);
  for (int b = 0; b < batch; ++b) {
    SeqState &q = s->seqs[b];
    if (!prompts[b] || !patch_lens[b] || prompt_len[b] < 1 || n_patches[b] < 1) {
      delete s;
      return bad("blt_session_create: empty prompt or segmentation");
    }
    q.prompt.assign(prompts[b], prompts[b] + prompt_len[b]);
    q.plens.assign(patch_lens[b], patch_lens[b] + n_patches[b]);
    int64_t tot = 0;
    for (int v : q.plens) {
      if (v < 1) { delete s; return bad("blt_session_create: patch length < 1"); }
      tot += v;
    }
    if (tot != prompt_len[b]) { delete s; return bad("blt_session_create: patch lengths do not sum to the prompt length"); }
    if (prompt_len[b] > g.max_ctx) { delete s; ctx->err = "blt_session_create: prompt longer than max_ctx"; return BLT_ECAPACITY; }
    q.salt = salt[b];
  }
  const int wmax = g.max_block + 1;
  s->W = wmax;
  s->o_blk = 0;
  s->o_masked = s->o_blk + (size_t)g.max_batch * g.max_block;
  s->o_draft = s->o_masked + g.max_batch;
  s->o_pred = s->o_draft + (size_t)g.max_batch * wmax;
  s->o_acc = s->o_pred + (size_t)g.max_batch * wmax;
  s->o_next = s->o_acc + g.max_batch;
  s->dev_n = s->o_next + g.max_batch;
  const size_t zn = (size_t)g.max_batch * wmax * 257;
  if (hipMalloc(&s->zq, zn * sizeof(float)) != hipSuccess ||
      hipMalloc(&s->zp, zn * sizeof(float)) != hipSuccess ||
      hipMalloc(&s->blk_before, sizeof(int32_t) * (size_t)g.max_batch * g.max_block) != hipSuccess ||
      hipMalloc(&s->dev, s->dev_n * sizeof(int32_t)) != hipSuccess ||
      hipHostMalloc(&s->host, s->dev_n * sizeof(int32_t), hipHostMallocMapped) != hipSuccess ||
      hipHostGetDevicePointer((void **)&s->host_dev, s->host, 0) != hipSuccess) {
    blt_session_destroy(s);
    ctx->err = "blt_session_create: allocation failed";
    return BLT_EHIP;
  }
  *out = s;
  return BLT_OK;
}

blt_status blt_session_prefill(blt_session *s) {
  if (!s) return BLT_EINVAL;
  const blt_config &g = s->ctx->cfg;
  std::vector<int> who, upto;
  for (int b = 0; b < s->batch; ++b) {
    SeqState &q = s->seqs[b];
    q.seg.init_prompt(q.plens);
    q.lat_ready = 0;
    q.avail = q.seg.last_complete;
    who.push_back(b);
    upto.push_back(q.avail);
  }
  S_TRY(encglob(s, who, upto));
  for (int b = 0; b < s->batch; ++b) {
    SeqState &q = s->seqs[b];
    const int n = (int)q.prompt.size() - 1;   // the last prompt byte stays pending
    q.ctau.assign(n, 0);
    for (int i = 0; i < n; ++i) q.ctau[i] = q.seg.causal_target(i);
    for (int c0 = 0; c0 < n; c0 += g.max_rows) {
      const int m = std::min(g.max_rows, n - c0);
      std::vector<int32_t> lat(q.ctau.begin() + c0, q.ctau.begin() + c0 + m);
      int32_t slot = b, start = c0, nrow = m;
      S_TRY(blt_kv_append(s->ctx, &s->st, 1, &slot, &start, &nrow, m, q.prompt.data() + c0,
                          nullptr, lat.data(), nullptr, nullptr, nullptr, nullptr, nullptr));
    }
    q.cache_len = n;
    q.seg0 = q.seg;
    q.cache0 = n;
    q.ctau0 = q.ctau;
    q.lat0 = q.lat_ready;
    q.avail0 = q.avail;
  }
  S_HIP(s, hipStreamSynchronize(s->ctx->stream));
  s->prefilled = true;
  return BLT_OK;
}

blt_status blt_session_generate(blt_session *s, const blt_policy_args *pa) {
  if (!s || !pa) return BLT_EINVAL;
  const blt_config &g = s->ctx->cfg;
  if (!s->prefilled) return sfail(s, BLT_EINVAL, "blt_session_generate: call blt_session_prefill first");
  if (pa->n_gen < 0) return sfail(s, BLT_EINVAL, "blt_session_generate: n_gen < 0");
  if (pa->block < 1 || pa->block > g.max_block)
    return sfail(s, BLT_ECAPACITY, "blt_session_generate: block outside 1..max_block");
  if (!(pa->temperature >= 0.f) || !isfinite(pa->temperature))
    return sfail(s, BLT_EINVAL, "blt_session_generate: temperature must be finite and >= 0");
  s->sampled = pa->temperature > 0.f;
  s->smp = blt_sampling{pa->temperature, pa->top_p, pa->seed};
  if (s->sampled && (pa->policy == BLT_POLICY_BLT_S || pa->policy == BLT_POLICY_BLT_DV) &&
      pa->block >= kMaxBlock)
    return sfail(s, BLT_EINVAL, "blt_session_generate: sampled verification needs a draft below 64 bytes");
  for (SeqState &q : s->seqs) {
    if ((int64_t)q.prompt.size() + pa->n_gen + 2 * pa->block + 1 > g.max_ctx)
      return sfail(s, BLT_ECAPACITY, "blt_session_generate: prompt + n_gen + block exceeds max_ctx");
    q.x = q.prompt;
    q.seg = q.seg0;
    q.cache_len = q.cache0;
    q.ctau = q.ctau0;
    q.lat_ready = q.lat0;
    q.avail = q.avail0;
    q.n_dec = q.n_eg = q.rounds = q.accepted = 0;
  }
  switch (pa->policy) {
    case BLT_POLICY_GREEDY: return run_greedy(s, pa->n_gen);
    case BLT_POLICY_BLT_D: return run_blt_d(s, *pa);
    case BLT_POLICY_BLT_S: return run_blt_s(s, *pa);
    case BLT_POLICY_BLT_DV: return run_blt_dv(s, *pa);
  }
  return sfail(s, BLT_EINVAL, "blt_session_generate: unknown policy");
}

blt_status blt_session_result(const blt_session *s, int32_t b, uint8_t *out, int32_t cap,
                              int32_t *n_out, uint64_t *n_dec, uint64_t *n_encglob,
                              uint64_t *n_rounds, uint64_t *n_accepted) {
  if (!s || b < 0 || b >= s->batch || cap < 0 || (cap > 0 && !out)) return BLT_EINVAL;
  const SeqState &q = s->seqs[b];
  const int n = (int)(q.x.size() - q.prompt.size());
  const int m = std::min(n, cap);
  if (m > 0) memcpy(out, q.x.data() + q.prompt.size(), (size_t)m);
  if (n_out) *n_out = n;
  if (n_dec) *n_dec = q.n_dec;
  if (n_encglob) *n_encglob = q.n_eg;
  if (n_rounds) *n_rounds = q.rounds;
  if (n_accepted) *n_accepted = q.accepted;
  return BLT_OK;
}

blt_status blt_session_device_blocks(blt_session *s, int32_t mode) {
  if (!s) return BLT_EINVAL;
  if (mode < 0 || mode > 3) return sfail(s, BLT_EINVAL, "blt_session_device_blocks: mode must be 0..3");
  s->device_blocks = mode;
  return BLT_OK;
}

blt_status blt_session_destroy(blt_session *s) {
  if (!s) return BLT_EINVAL;
  if (s->ctx) (void)hipStreamSynchronize(s->ctx->stream);
  if (s->dev) (void)hipFree(s->dev);
  if (s->zq) (void)hipFree(s->zq);
  if (s->zp) (void)hipFree(s->zp);
  if (s->blk_before) (void)hipFree(s->blk_before);
  if (s->host) (void)hipHostFree(s->host);
  free_dev_blocks(s);
  delete s;
  return BLT_OK;
}

}  // extern "C"
