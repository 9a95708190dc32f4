// Native decode sessions through the C-ABI from a plain C++ program (test
// infrastructure): the checked library builds run here without Python or
// torch in the process, the sanitized one with this driver built under the
// same sanitizers.
//
//   session_driver <case_dir>
//
// case_dir/case.txt:
//   n_layers d_model n_heads d_ffn d_global dtype max_batch max_ctx max_latents max_rows max_block rope_theta rms_eps
//   batch n_latents
//   per sequence: prompt_len n_patches salt / the prompt's bytes / its patch lengths
//   n_runs, then per run: policy block alpha unmask device_blocks temperature top_p seed n_gen
// case_dir/<name>.bin: weights in the device dtype (embed, w_lat, w_out, g_out,
//   L<l>_<wv_c|wo_c|wqkv|wo|g_attn|g_ffn|w1|w2>) and latents ([batch][n_latents][d_global]).
// stdout, per run and sequence: "R run b n n_dec n_eg rounds accepted byte..."
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

#include <string>
#include <vector>

#include "../../include/blt.h"

static std::string g_dir;

static void die(const char *what, const char *detail = "") {
  fprintf(stderr, "session_driver: %s %s\n", what, detail);
  exit(1);
}

static void *upload(const std::string &name, size_t *bytes_out = nullptr) {
  const std::string path = g_dir + "/" + name + ".bin";
  FILE *f = fopen(path.c_str(), "rb");
  if (!f) die("cannot open", path.c_str());
  fseek(f, 0, SEEK_END);
  const long n = ftell(f);
  fseek(f, 0, SEEK_SET);
  std::vector<char> buf((size_t)n);
  if (n > 0 && fread(buf.data(), 1, (size_t)n, f) != (size_t)n) die("short read", path.c_str());
  fclose(f);
  void *d = nullptr;
  if (hipMalloc(&d, n > 0 ? (size_t)n : 1) != hipSuccess) die("hipMalloc failed for", path.c_str());
  if (n > 0 && hipMemcpy(d, buf.data(), (size_t)n, hipMemcpyHostToDevice) != hipSuccess)
    die("hipMemcpy failed for", path.c_str());
  if (bytes_out) *bytes_out = (size_t)n;
  return d;
}

#define CHECK(ctx, call)                                                                      \
  do {                                                                                        \
    blt_status _s = (call);                                                                   \
    if (_s != BLT_OK) {                                                                       \
      fprintf(stderr, "session_driver: %s -> %d: %s\n", #call, (int)_s,                       \
              (ctx) ? blt_last_error(ctx) : "");                                              \
      exit(1);                                                                                \
    }                                                                                         \
  } while (0)

int main(int argc, char **argv) {
  if (argc != 2) die("usage: session_driver <case_dir>");
  g_dir = argv[1];
  FILE *f = fopen((g_dir + "/case.txt").c_str(), "r");
  if (!f) die("cannot open case.txt");
  blt_config cfg{};
  int dtype = 0;
  if (fscanf(f, "%d %d %d %d %d %d %d %d %d %d %d %f %f", &cfg.n_layers, &cfg.d_model, &cfg.n_heads,
             &cfg.d_ffn, &cfg.d_global, &dtype, &cfg.max_batch, &cfg.max_ctx, &cfg.max_latents,
             &cfg.max_rows, &cfg.max_block, &cfg.rope_theta, &cfg.rms_eps) != 13)
    die("bad config line");
  cfg.vocab = 257;
  cfg.dtype = dtype ? BLT_BF16 : BLT_F32;
  int batch = 0, n_lat = 0;
  if (fscanf(f, "%d %d", &batch, &n_lat) != 2 || batch < 1 || batch > cfg.max_batch) die("bad batch line");
  std::vector<std::vector<uint8_t>> prompts(batch);
  std::vector<std::vector<int32_t>> plens(batch);
  std::vector<uint64_t> salts(batch);
  for (int b = 0; b < batch; ++b) {
    int n = 0, np = 0;
    unsigned long long salt = 0;
    if (fscanf(f, "%d %d %llu", &n, &np, &salt) != 3 || n < 1 || np < 1) die("bad sequence line");
    salts[b] = salt;
    prompts[b].resize(n);
    plens[b].resize(np);
    for (auto &v : prompts[b]) {
      int x;
      if (fscanf(f, "%d", &x) != 1) die("bad prompt");
      v = (uint8_t)x;
    }
    for (auto &v : plens[b])
      if (fscanf(f, "%d", &v) != 1) die("bad patch lengths");
  }
  int n_runs = 0;
  if (fscanf(f, "%d", &n_runs) != 1) die("bad run count");
  struct Run {
    int policy, block, unmask, device, n_gen;
    float alpha, temperature, top_p;
    unsigned long long seed;
  };
  std::vector<Run> runs(n_runs);
  for (auto &r : runs)
    if (fscanf(f, "%d %d %f %d %d %f %f %llu %d", &r.policy, &r.block, &r.alpha, &r.unmask, &r.device,
               &r.temperature, &r.top_p, &r.seed, &r.n_gen) != 9)
      die("bad run line");
  fclose(f);

  void *embed = upload("embed"), *w_lat = upload("w_lat"), *w_out = upload("w_out"), *g_out = upload("g_out");
  std::vector<blt_layer_weights> layers(cfg.n_layers);
  const char *names[8] = {"wv_c", "wo_c", "wqkv", "wo", "g_attn", "g_ffn", "w1", "w2"};
  for (int l = 0; l < cfg.n_layers; ++l) {
    void *p[8];
    for (int k = 0; k < 8; ++k) p[k] = upload("L" + std::to_string(l) + "_" + names[k]);
    layers[l] = blt_layer_weights{p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]};
  }
  const blt_weights w{embed, w_lat, w_out, g_out, layers.data()};
  void *table = upload("latents");

  std::vector<const uint8_t *> pp(batch);
  std::vector<const int32_t *> pl(batch);
  std::vector<int32_t> plen(batch), npat(batch);
  for (int b = 0; b < batch; ++b) {
    pp[b] = prompts[b].data();
    pl[b] = plens[b].data();
    plen[b] = (int32_t)prompts[b].size();
    npat[b] = (int32_t)plens[b].size();
  }
  for (int ri = 0; ri < n_runs; ++ri) {
    const Run &r = runs[ri];
    blt_config c = cfg;
    c.max_block = r.block;                   // as the Python sessions size it
    size_t kvb = 0, crb = 0;
    CHECK(nullptr, blt_state_size(&c, &kvb, &crb));
    blt_state st{};
    if (hipMalloc(&st.kv, kvb) != hipSuccess || hipMalloc(&st.cross, crb) != hipSuccess)
      die("state hipMalloc failed");
    blt_ctx *ctx = nullptr;
    CHECK(nullptr, blt_create(&c, &w, nullptr, &ctx));
    blt_session *s = nullptr;
    CHECK(ctx, blt_session_create(ctx, &st, batch, pp.data(), plen.data(), pl.data(), npat.data(),
                                  salts.data(), table, n_lat, &s));
    CHECK(ctx, blt_session_device_blocks(s, r.device));
    CHECK(ctx, blt_session_prefill(s));
    blt_policy_args a{};
    a.policy = (blt_policy)r.policy;
    a.block = r.block;
    a.alpha = r.alpha;
    a.unmask = (blt_unmask)r.unmask;
    a.block_mask = BLT_BLOCK_BIDIR;
    a.n_gen = r.n_gen;
    a.temperature = r.temperature;
    a.top_p = r.top_p;
    a.seed = r.seed;
    CHECK(ctx, blt_session_generate(s, &a));
    for (int b = 0; b < batch; ++b) {
      std::vector<uint8_t> out((size_t)r.n_gen + 1);
      int32_t n = 0;
      uint64_t nd = 0, ne = 0, nr = 0, na = 0;
      CHECK(ctx, blt_session_result(s, b, out.data(), r.n_gen, &n, &nd, &ne, &nr, &na));
      printf("R %d %d %d %llu %llu %llu %llu", ri, b, n, (unsigned long long)nd, (unsigned long long)ne,
             (unsigned long long)nr, (unsigned long long)na);
      for (int i = 0; i < n && i < r.n_gen; ++i) printf(" %d", out[i]);
      printf("\n");
    }
    CHECK(ctx, blt_session_destroy(s));
    CHECK(ctx, blt_destroy(ctx));
    if (hipFree(st.kv) != hipSuccess || hipFree(st.cross) != hipSuccess) die("hipFree failed");
  }
  fflush(stdout);
  // the weights are released with the process
  return 0;
}
