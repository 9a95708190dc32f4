// Host-only driver over the library's HIP-free host logic (the stand-in
// patcher and the debug build's descriptor checks), built by the CPU tests
// with AddressSanitizer and UndefinedBehaviorSanitizer.  Test infrastructure.
//
// stdin, one case per line:
//   P salt n_lens lens... n_x x... t
//       prints the state after the prompt's segmentation, then the state of
//       a copy taken after pushing bytes n_prompt..t-1 and continued with the
//       rest (the draft rounds continue a copy), then the state after
//       pushing every byte after the prompt
//   D max_batch max_ctx max_latents max_rows block_entries n_rows (10 ints per row)...
//     n_seqs (9 ints per sequence)...
//       prints "ok" or the checker's message
#include <stdio.h>

#include <string>
#include <vector>

#include "../../block_diffusion_byte_amd/csrc/host_checks.h"
#include "../../block_diffusion_byte_amd/csrc/host_patcher.h"

using namespace blt;

static void print_seg(const Seg &s) {
  printf("S %d %d", s.cur_len, s.last_complete);
  for (size_t i = 0; i < s.patch.size(); ++i) printf(" %d:%d", s.patch[i], (int)s.ends[i]);
  printf("\n");
}

int main() {
  char kind[4];
  while (scanf("%3s", kind) == 1) {
    if (kind[0] == 'P') {
      unsigned long long salt;
      int nl, nx, t;
      if (scanf("%llu %d", &salt, &nl) != 2) return 2;
      std::vector<int32_t> lens(nl);
      int n_prompt = 0;
      for (auto &v : lens) {
        if (scanf("%d", &v) != 1) return 2;
        n_prompt += v;
      }
      if (scanf("%d", &nx) != 1) return 2;
      std::vector<int> x(nx);
      for (auto &v : x)
        if (scanf("%d", &v) != 1) return 2;
      if (scanf("%d", &t) != 1) return 2;
      Seg s;
      s.init_prompt(lens);
      print_seg(s);
      for (int i = n_prompt; i < t; ++i) s.push(salt, (uint8_t)x[i - 1], (uint8_t)x[i]);
      Seg c = s;
      for (int i = t; i < nx; ++i) c.push(salt, (uint8_t)x[i - 1], (uint8_t)x[i]);
      print_seg(c);
      for (int i = t; i < nx; ++i) s.push(salt, (uint8_t)x[i - 1], (uint8_t)x[i]);
      print_seg(s);
    } else if (kind[0] == 'D') {
      DescLimits g{};
      long long be;
      int nr, ns;
      if (scanf("%d %d %d %d %lld %d", &g.max_batch, &g.max_ctx, &g.max_latents, &g.max_rows, &be, &nr) != 6)
        return 2;
      g.block_entries = be;
      std::vector<RowDesc> rows(nr);
      for (auto &r : rows)
        if (scanf("%d %d %d %d %d %d %d %d %d %d", &r.slot, &r.pos, &r.tok, &r.blk, &r.lat, &r.kend,
                  &r.oidx, &r.attn_flash, &r.ctr, &r.keep_kv) != 10)
          return 2;
      if (scanf("%d", &ns) != 1) return 2;
      std::vector<SeqDesc> seqs(ns);
      for (auto &q : seqs)
        if (scanf("%d %d %d %d %d %d %d %d %d", &q.slot, &q.row0, &q.nrows, &q.kmax, &q.blk0, &q.blk_row0,
                  &q.nblk, &q.out_b, &q.attn_flash) != 9)
          return 2;
      char msg[160];
      const char *why = check_pass_descs(rows.data(), nr, seqs.data(), ns, g, msg, sizeof msg);
      printf("%s\n", why ? why : "ok");
    } else {
      return 2;
    }
    fflush(stdout);
  }
  return 0;
}
