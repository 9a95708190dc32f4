// Descriptor checks of the bounds-checking debug build (BLT_DEBUG_BOUNDS):
// every row and sequence a decoder pass stages is checked against the
// context's geometry before it is copied to the device, so a driver whose
// bookkeeping goes wrong fails with a message instead of sending a kernel
// out of its buffers.  No HIP dependency: host-only test drivers build it
// under the sanitizers.
#pragma once
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "desc.h"

namespace blt {

struct DescLimits {
  int max_batch, max_ctx, max_latents, max_rows;
  int64_t block_entries;   // block_tok entries a kTokFromBlock row may name
};

// nullptr when the pass is in range, else a message (in msg) naming the
// first violation.  Invariants: every row names a slot, a position below
// max_ctx and a latent below max_latents, attends at least itself (pos <
// kend <= max_ctx), takes a byte or MASK or names a token source; every
// sequence's rows are contiguous and carry its slot, its kmax is their
// largest kend, its block rows (if any) lie inside its rows; with sequences
// present every row belongs to exactly one; no two rows write one cache row.
inline const char *check_pass_descs(const RowDesc *rows, int n_rows, const SeqDesc *seqs,
                                    int n_seqs, const DescLimits &g, char *msg, size_t cap) {
  auto bad = [&](const char *what, int i) {
    snprintf(msg, cap, "debug bounds: %s (index %d)", what, i);
    return (const char *)msg;
  };
  if (n_rows < 0 || n_rows > g.max_rows) return bad("row count outside 0..max_rows", n_rows);
  if (n_seqs < 0 || n_seqs > std::max(g.max_batch, 1)) return bad("sequence count above max_batch", n_seqs);
  std::vector<std::pair<int64_t, int>> writes;
  writes.reserve(n_rows);
  for (int i = 0; i < n_rows; ++i) {
    const RowDesc &r = rows[i];
    if (r.slot < 0 || r.slot >= g.max_batch) return bad("row slot outside 0..max_batch", i);
    if (r.pos < 0 || r.pos >= g.max_ctx) return bad("row position outside 0..max_ctx", i);
    if (r.kend <= r.pos || r.kend > g.max_ctx) return bad("row kend outside pos+1..max_ctx", i);
    if (r.lat < 0 || r.lat >= g.max_latents) return bad("row latent outside 0..max_latents", i);
    if (r.tok > kMask || (r.tok < 0 && r.tok != kTokFromBlock && r.tok != kTokFromDev))
      return bad("row token neither a byte, MASK nor a token source", i);
    if (r.tok < 0 && r.blk < 0) return bad("row token source index negative", i);
    if (r.tok == kTokFromBlock && r.blk >= g.block_entries) return bad("row block index beyond block_tok", i);
    if (r.oidx < -1) return bad("row output index below -1", i);
    if (r.ctr < -1) return bad("row draw number below -1", i);
    if ((r.attn_flash & ~1) || (r.keep_kv & ~1)) return bad("row flag not 0 or 1", i);
    if (!r.keep_kv) writes.emplace_back((int64_t)r.slot * g.max_ctx + r.pos, i);
  }
  std::sort(writes.begin(), writes.end());
  for (size_t i = 1; i < writes.size(); ++i)
    if (writes[i].first == writes[i - 1].first) return bad("two rows write one cache row", writes[i].second);
  std::vector<int> owner(n_seqs > 0 ? n_rows : 0, -1);
  for (int s = 0; s < n_seqs; ++s) {
    const SeqDesc &q = seqs[s];
    if (q.slot < 0 || q.slot >= g.max_batch) return bad("sequence slot outside 0..max_batch", s);
    if (q.out_b < 0 || q.out_b >= g.max_batch) return bad("sequence batch index outside 0..max_batch", s);
    if (q.row0 < 0 || q.nrows < 0 || q.row0 + q.nrows > n_rows) return bad("sequence rows outside the pass", s);
    if (q.attn_flash & ~1) return bad("sequence flag not 0 or 1", s);
    int kmax = 0;
    for (int i = q.row0; i < q.row0 + q.nrows; ++i) {
      if (owner[i] >= 0) return bad("row in two sequences", i);
      owner[i] = s;
      if (rows[i].slot != q.slot) return bad("row slot differs from its sequence's", i);
      if (rows[i].attn_flash != q.attn_flash) return bad("row attention kernel differs from its sequence's", i);
      kmax = std::max(kmax, rows[i].kend);
    }
    if (q.nrows > 0 && q.kmax != kmax) return bad("sequence kmax is not its rows' largest kend", s);
    if (q.nblk < 0) return bad("sequence block row count negative", s);
    if (q.nblk > 0) {
      if (q.blk0 < 0 || q.blk_row0 < q.row0 || q.blk_row0 + q.nblk > q.row0 + q.nrows)
        return bad("sequence block rows outside its rows", s);
      if ((int64_t)q.blk0 + q.nblk > g.block_entries) return bad("sequence block beyond block_tok", s);
    }
  }
  for (size_t i = 0; i < owner.size(); ++i)
    if (owner[i] < 0) return bad("row in no sequence", (int)i);
  return nullptr;
}

}  // namespace blt
