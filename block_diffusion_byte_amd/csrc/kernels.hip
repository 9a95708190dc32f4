// HIP kernels of the Fast-BLT local byte decoder step, written for gfx950
// (CDNA4: wave64, MFMA, 160 KB LDS per CU).
//
// Decoder layer (pytorch.kr Fast-BLT summary, BLT architecture, the layer
// equation): residual += cross-attention read of one latent, then a pre-norm
// self-attention and FFN transformer layer; a final RMSNorm and the 257-way
// byte head.  Decisions (block unmasking strategies; BLT-S/BLT-DV
// verification) run on the device too.
//
// Numerics: the residual stream, softmax statistics and logits are float32;
// in the bf16 configuration every GEMM input (weights and the normalised or
// attention/FFN activations) and the KV cache are bfloat16, products are
// accumulated in float32.  Every reduction has an order fixed by the data
// layout alone (never by how many rows share a pass), so a row's results do
// not depend on the other rows of its pass: the GEMV path splits K over
// lanes and waves identically for any row count, and attention splits keys
// into chunks aligned to absolute positions merged in chunk order.
#include <hip/hip_runtime.h>
#include <math.h>

#include "blt_internal.h"

namespace blt {

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);                                              // nearest, ties to even
  return (uint16_t)(u >> 16);
}

template <bool BF> struct Act;
template <> struct Act<true> {
  using T = uint16_t;
  static constexpr int EPC = 8;  // elements per 16-byte chunk
};
template <> struct Act<false> {
  using T = float;
  static constexpr int EPC = 4;
};

__device__ __forceinline__ float to_f(uint16_t v) { return bf2f(v); }
__device__ __forceinline__ float to_f(float v) { return v; }
template <typename T> __device__ __forceinline__ T from_f(float f);
template <> __device__ __forceinline__ uint16_t from_f<uint16_t>(float f) { return f2bf(f); }
template <> __device__ __forceinline__ float from_f<float>(float f) { return f; }

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <bool BF> __device__ __forceinline__ float dot_chunk(uint4 w, uint4 x, float acc);
template <> __device__ __forceinline__ float dot_chunk<true>(uint4 w, uint4 x, float acc) {
  acc = dot2(w.x, x.x, acc);
  acc = dot2(w.y, x.y, acc);
  acc = dot2(w.z, x.z, acc);
  acc = dot2(w.w, x.w, acc);
  return acc;
}
template <> __device__ __forceinline__ float dot_chunk<false>(uint4 w, uint4 x, float acc) {
  acc = fmaf(__uint_as_float(w.x), __uint_as_float(x.x), acc);
  acc = fmaf(__uint_as_float(w.y), __uint_as_float(x.y), acc);
  acc = fmaf(__uint_as_float(w.z), __uint_as_float(x.z), acc);
  acc = fmaf(__uint_as_float(w.w), __uint_as_float(x.w), acc);
  return acc;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// Load the 16-byte chunk `c` of activation row `rr`, applying the RMSNorm
// prologue when requested.
template <bool BF>
__device__ __forceinline__ uint4 load_x_chunk(const GemmArgs &a, int rr, int c, float rinv) {
  using T = typename Act<BF>::T;
  constexpr int EPC = Act<BF>::EPC;
  if (a.pro == PRO_PLAIN) {
    const T *row = (const T *)a.X + (a.x_row_off ? a.x_row_off[rr] : (int64_t)rr * a.ldx);
    return *(const uint4 *)(row + (int64_t)c * EPC);
  }
  const float *hr = a.H + (int64_t)rr * a.ldh + (int64_t)c * EPC;
  const T *g = (const T *)a.gain + (int64_t)c * EPC;
  uint4 gv = *(const uint4 *)g;
  if constexpr (BF) {
    float4 h0 = *(const float4 *)hr, h1 = *(const float4 *)(hr + 4);
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
    const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float g0 = __uint_as_float(gw[i] << 16), g1 = __uint_as_float(gw[i] & 0xffff0000u);
      uint32_t lo = f2bf(g0 * hv[2 * i] * rinv), hi = f2bf(g1 * hv[2 * i + 1] * rinv);
      o[i] = lo | (hi << 16);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
  } else {
    float4 h0 = *(const float4 *)hr;
    return make_uint4(__float_as_uint(__uint_as_float(gv.x) * h0.x * rinv),
                      __float_as_uint(__uint_as_float(gv.y) * h0.y * rinv),
                      __float_as_uint(__uint_as_float(gv.z) * h0.z * rinv),
                      __float_as_uint(__uint_as_float(gv.w) * h0.w * rinv));
  }
}

template <bool BF>
__device__ __forceinline__ void epilogue(const GemmArgs &a, int r, int o, float y) {
  using T = typename Act<BF>::T;
  switch (a.ep) {
    case EP_STORE_F32:
      a.out_f32[(int64_t)r * a.ldo + o] = y;
      break;
    case EP_RESID: {
      float c = 0.f;
      if (a.cross) {
        const RowDesc rd = a.rows[r];
        c = a.cross[(((int64_t)rd.slot * a.max_lat + rd.lat) * a.n_layers + a.cross_layer) * a.d + o];
      }
      a.resid[(int64_t)r * a.ldo + o] += y + c;
      break;
    }
    case EP_SILU_ACT:
      ((T *)a.out_act)[(int64_t)r * a.ldo + o] = from_f<T>(y / (1.f + expf(-y)));
      break;
    case EP_STORE_ACT:
      ((T *)a.out_act)[(int64_t)r * a.ldo + o] = from_f<T>(y);
      break;
    case EP_ROWOFF_F32:
      a.out_f32[a.row_off[r] + a.off_add + o] = y;
      break;
  }
}

// ---------------------------------------------------------------------------
// GEMV for passes of a few rows (weight-streaming bound).
//
// A workgroup (4 waves) owns 8 output rows.  Lanes are grouped by 8: group g
// of every wave reads output row o0+g, 128 contiguous bytes per load, so
// each load instruction of a wave streams 8 full cache lines.  The K axis is
// split into 4 contiguous quarters, one per wave; inside a quarter lane s of
// a group takes the 16-byte chunks s, s+8, s+16, ... in ascending order.
// Partial sums are reduced in the group by xor-shuffles (1, 2, 4) and then
// over the 4 waves in wave order.  That order depends on K only.
// Activations are staged in LDS (all groups of a wave read the same chunk:
// broadcast), in tiles of at most kTQ chunks per quarter; the tile size only
// decides when activations are staged, never the accumulation order.
template <bool BF, int RB>
__global__ __launch_bounds__(256) void k_gemv(GemmArgs a) {
  constexpr int EPC = Act<BF>::EPC;
  constexpr int kTQ = RB <= 8 ? 64 : 32;
  __shared__ uint4 xs[RB * 4 * kTQ];
  __shared__ float red[4][RB][8];
  __shared__ float rinv_s[RB];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 3, s = lane & 7;
  const int o = blockIdx.x * 8 + g;
  const bool o_ok = o < a.N;
  const int KC = a.K / EPC, Q = KC / 4, TQ = Q < kTQ ? Q : kTQ;
  const uint4 *wrow = (const uint4 *)((const char *)a.W + (int64_t)(o_ok ? o : 0) * a.K * (BF ? 2 : 4)) + w * Q;

  for (int rb = 0; rb < a.R; rb += RB) {
    const int nr = min(RB, a.R - rb);
    if (a.pro == PRO_NORM) {
      for (int r = w; r < nr; r += 4) {
        const float *hr = a.H + (int64_t)(rb + r) * a.ldh;
        float ss = 0.f;
        for (int k = lane; k < a.K; k += 64) ss = fmaf(hr[k], hr[k], ss);
        ss = wave_sum(ss);
        if (lane == 0) rinv_s[r] = 1.f / sqrtf(ss / (float)a.K + a.eps);
      }
      __syncthreads();
    }
    float acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[r] = 0.f;

    for (int t0 = 0; t0 < Q; t0 += TQ) {
      const int tq = min(TQ, Q - t0);
      for (int i = tid; i < nr * 4 * tq; i += 256) {
        const int r = i / (4 * tq), rem = i - r * 4 * tq, ww = rem / tq, j = rem - ww * tq;
        xs[(r * 4 + ww) * kTQ + j] =
            load_x_chunk<BF>(a, rb + r, ww * Q + t0 + j, a.pro == PRO_NORM ? rinv_s[r] : 1.f);
      }
      __syncthreads();
      if (o_ok) {
        uint4 wv[kTQ / 8];
#pragma unroll
        for (int u = 0; u < kTQ / 8; ++u) {
          const int j = s + 8 * u;
          if (j < tq) wv[u] = wrow[t0 + j];
        }
#pragma unroll
        for (int u = 0; u < kTQ / 8; ++u) {
          const int j = s + 8 * u;
          if (j < tq) {
#pragma unroll
            for (int r = 0; r < RB; ++r)
              if (r < nr) acc[r] = dot_chunk<BF>(wv[u], xs[(r * 4 + w) * kTQ + j], acc[r]);
          }
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      float v = acc[r];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      if (s == 0 && r < nr) red[w][r][g] = v;
    }
    __syncthreads();
    for (int i = tid; i < nr * 8; i += 256) {
      const int r = i >> 3, gg = i & 7, oo = blockIdx.x * 8 + gg;
      if (oo < a.N) {
        const float y = ((red[0][r][gg] + red[1][r][gg]) + red[2][r][gg]) + red[3][r][gg];
        epilogue<BF>(a, rb + r, oo, y);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// MFMA GEMM (bf16 x bf16 -> f32) for passes of >= 16 rows: Y[R][N] = X[R][K] W[N][K]^T.
// 64x64 output tile per workgroup, K step 64 through LDS; each wave owns a
// 32x32 quarter as 2x2 tiles of v_mfma_f32_16x16x32_bf16.
constexpr int kBM = 64, kBN = 64, kBK = 64, kLdsK = kBK + 8;

__global__ __launch_bounds__(256) void k_gemm_mfma(GemmArgs a) {
  __shared__ uint16_t xs[kBM * kLdsK];
  __shared__ uint16_t ws[kBN * kLdsK];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int n0 = blockIdx.x * kBN, m0 = blockIdx.y * kBM;
  const int wr = (w >> 1) * 32, wc = (w & 1) * 32;
  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const uint16_t *X = (const uint16_t *)a.X;
  const uint16_t *W = (const uint16_t *)a.W;
  for (int k0 = 0; k0 < a.K; k0 += kBK) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + u * 256, row = idx >> 3, kc = idx & 7;
      const int rr = m0 + row, nn = n0 + row;
      uint4 xv = make_uint4(0, 0, 0, 0), wv = make_uint4(0, 0, 0, 0);
      if (rr < a.R) {
        const uint16_t *xr = X + (a.x_row_off ? a.x_row_off[rr] : (int64_t)rr * a.ldx);
        xv = *(const uint4 *)(xr + k0 + kc * 8);
      }
      if (nn < a.N) wv = *(const uint4 *)(W + (int64_t)nn * a.K + k0 + kc * 8);
      *(uint4 *)&xs[row * kLdsK + kc * 8] = xv;
      *(uint4 *)&ws[row * kLdsK + kc * 8] = wv;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kBK; ks += 32) {
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint4 v = *(const uint4 *)&xs[(wr + i * 16 + (l & 15)) * kLdsK + ks + 8 * (l >> 4)];
        af[i] = __builtin_bit_cast(bf16x8_t, v);
        uint4 u = *(const uint4 *)&ws[(wc + i * 16 + (l & 15)) * kLdsK + ks + 8 * (l >> 4)];
        bfr[i] = __builtin_bit_cast(bf16x8_t, u);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wr + i * 16 + 4 * (l >> 4) + v;
        const int n = n0 + wc + j * 16 + (l & 15);
        if (m < a.R && n < a.N) epilogue<true>(a, m, n, acc[i][j][v]);
      }
}

// RMSNorm rows into an activation buffer (MFMA path prologue).
template <bool BF>
__global__ __launch_bounds__(256) void k_rmsnorm_act(const float *H, int64_t ldh, const void *gain,
                                                     int K, float eps, void *out) {
  using T = typename Act<BF>::T;
  __shared__ float part[4];
  const int r = blockIdx.x, t = threadIdx.x;
  const float *hr = H + (int64_t)r * ldh;
  float ss = 0.f;
  for (int k = t; k < K; k += 256) ss = fmaf(hr[k], hr[k], ss);
  ss = wave_sum(ss);
  if ((t & 63) == 0) part[t >> 6] = ss;
  __syncthreads();
  const float tot = ((part[0] + part[1]) + part[2]) + part[3];
  const float rinv = 1.f / sqrtf(tot / (float)K + eps);
  const T *g = (const T *)gain;
  T *o = (T *)out + (int64_t)r * K;
  for (int k = t; k < K; k += 256) o[k] = from_f<T>(to_f(g[k]) * hr[k] * rinv);
}

// ---------------------------------------------------------------------------
// h[r] = E[tok_r] + cross contribution of layer 0 for the row's latent.
template <bool BF>
__global__ __launch_bounds__(256) void k_embed(const void *embed, const float *cross,
                                               const RowDesc *rows, int d, int n_layers,
                                               int max_lat, const int32_t *block_tok,
                                               const int32_t *tokens_dev, float *h) {
  using T = typename Act<BF>::T;
  const int r = blockIdx.x;
  const RowDesc rd = rows[r];
  int tok = rd.tok;
  if (tok == kTokFromBlock) tok = block_tok[rd.blk];
  else if (tok == kTokFromDev) tok = tokens_dev[rd.blk];
  tok = tok < 0 ? 0 : (tok > kMask ? kMask : tok);
  const T *e = (const T *)embed + (int64_t)tok * d;
  const float *c = cross + ((int64_t)rd.slot * max_lat + rd.lat) * n_layers * d;
  for (int k = threadIdx.x; k < d; k += 256) h[(int64_t)r * d + k] = to_f(e[k]) + c[k];
}

// RoPE on q and k at the row's absolute position (rotate-half pairs (j, j+dh/2),
// angles from a float2 (cos, sin) table), q kept in f32, k and v written to the
// cache row `pos` of the row's sequence.
template <bool BF>
__global__ __launch_bounds__(256) void k_rope_kv(const float *qkv, const RowDesc *rows,
                                                 const float2 *rope_tab, float *q_out, void *kvp,
                                                 KVGeom g, int layer) {
  using T = typename Act<BF>::T;
  const int r = blockIdx.x;
  const RowDesc rd = rows[r];
  const int dh = g.d_head, half = dh >> 1, d = g.n_heads * dh;
  const float *src = qkv + (int64_t)r * 3 * d;
  const int64_t plane = (int64_t)g.max_ctx * dh;
  T *kv = (T *)kvp;
  for (int p = threadIdx.x; p < d / 2; p += 256) {
    const int hh = p / half, j = p - hh * half;
    const float2 cs = rope_tab[(int64_t)rd.pos * half + j];
    const int lo = hh * dh + j, hi = lo + half;
    const float q1 = src[lo], q2 = src[hi];
    q_out[(int64_t)r * d + lo] = q1 * cs.x - q2 * cs.y;
    q_out[(int64_t)r * d + hi] = q2 * cs.x + q1 * cs.y;
    const float k1 = src[d + lo], k2 = src[d + hi];
    const int64_t kb = ((((int64_t)rd.slot * g.n_layers + layer) * 2 + 0) * g.n_heads + hh) * plane +
                       (int64_t)rd.pos * dh;
    const int64_t vb = kb + (int64_t)g.n_heads * plane;
    kv[kb + j] = from_f<T>(k1 * cs.x - k2 * cs.y);
    kv[kb + j + half] = from_f<T>(k2 * cs.x + k1 * cs.y);
    kv[vb + j] = from_f<T>(src[2 * d + lo]);
    kv[vb + j + half] = from_f<T>(src[2 * d + hi]);
  }
}

// ---------------------------------------------------------------------------
// Split-K attention.  Workgroup (chunk c, head h, sequence b) owns keys
// [c*256, c*256+256) of that sequence and every row of it in the pass; row r
// reads keys [0, kend_r).  Thread t holds key c*256+t in registers, scores are
// staged in LDS, the softmax statistics of the chunk are (max, sum), and
// P.V is summed by (dim, key-partition) threads.  Output per (row, head,
// chunk): the unnormalised o[dh], m, l.
template <bool BF, int DH>
__global__ __launch_bounds__(256) void k_attn_partial(const float *q, const void *kvp, KVGeom g,
                                                      int layer, const SeqDesc *seqs,
                                                      const RowDesc *rows, float *part,
                                                      int max_chunks) {
  using T = typename Act<BF>::T;
  constexpr int CK = kAttnChunk, RG = 16, NP = 256 / DH, KPP = CK / NP;
  __shared__ float qs[RG][DH];
  __shared__ float ps[RG][CK];
  __shared__ float op[NP][RG][DH];
  __shared__ float redm[RG][4], reds[RG][4];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const SeqDesc sd = seqs[b];
  const int key0 = c * CK;
  if (key0 >= sd.kmax) return;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int d = g.n_heads * DH;
  const int64_t plane = (int64_t)g.max_ctx * DH;
  const T *Kb = (const T *)kvp + ((((int64_t)sd.slot * g.n_layers + layer) * 2 + 0) * g.n_heads + h) * plane;
  const T *Vb = Kb + (int64_t)g.n_heads * plane;
  const int j = key0 + t;
  float kr[DH];
  if (j < sd.kmax) {
    const uint4 *kp = (const uint4 *)(Kb + (int64_t)j * DH);
    constexpr int EPC = Act<BF>::EPC;
#pragma unroll
    for (int u = 0; u < DH / EPC; ++u) {
      const uint4 v = kp[u];
      if constexpr (BF) {
        const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kr[u * 8 + 2 * i] = __uint_as_float(vv[i] << 16);
          kr[u * 8 + 2 * i + 1] = __uint_as_float(vv[i] & 0xffff0000u);
        }
      } else {
        kr[u * 4 + 0] = __uint_as_float(v.x);
        kr[u * 4 + 1] = __uint_as_float(v.y);
        kr[u * 4 + 2] = __uint_as_float(v.z);
        kr[u * 4 + 3] = __uint_as_float(v.w);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < DH; ++e) kr[e] = 0.f;
  }
  const float scale = 1.f / sqrtf((float)DH);
  const int e = t % DH, kp = t / DH;

  for (int rg = 0; rg < sd.nrows; rg += RG) {
    const int nr = min(RG, sd.nrows - rg);
    for (int i = t; i < nr * DH; i += 256) {
      const int r = i / DH, ee = i - r * DH;
      qs[r][ee] = q[(int64_t)(sd.row0 + rg + r) * d + h * DH + ee];
    }
    __syncthreads();
    for (int r = 0; r < nr; ++r) {
      const int kend = rows[sd.row0 + rg + r].kend;
      float s = -INFINITY;
      if (j < kend) {
        float acc = 0.f;
#pragma unroll
        for (int ee = 0; ee < DH; ++ee) acc = fmaf(qs[r][ee], kr[ee], acc);
        s = acc * scale;
      }
      ps[r][t] = s;
      const float m = wave_max(s);
      if (lane == 0) redm[r][w] = m;
    }
    __syncthreads();
    for (int r = 0; r < nr; ++r) {
      const float m = fmaxf(fmaxf(redm[r][0], redm[r][1]), fmaxf(redm[r][2], redm[r][3]));
      const float s = ps[r][t];
      const float p = (s == -INFINITY) ? 0.f : expf(s - m);
      ps[r][t] = p;
      const float sum = wave_sum(p);
      if (lane == 0) reds[r][w] = sum;
    }
    __syncthreads();
    float o[RG];
#pragma unroll
    for (int r = 0; r < RG; ++r) o[r] = 0.f;
    for (int jj = kp * KPP; jj < (kp + 1) * KPP; ++jj) {
      const int jg = key0 + jj;
      if (jg >= sd.kmax) break;
      const float v = to_f(Vb[(int64_t)jg * DH + e]);
#pragma unroll
      for (int r = 0; r < RG; ++r)
        if (r < nr) o[r] = fmaf(ps[r][jj], v, o[r]);
    }
#pragma unroll
    for (int r = 0; r < RG; ++r)
      if (r < nr) op[kp][r][e] = o[r];
    __syncthreads();
    for (int i = t; i < nr * DH; i += 256) {
      const int r = i / DH, ee = i - r * DH;
      const int row = sd.row0 + rg + r;
      if (rows[row].kend <= key0) continue;
      float acc = 0.f;
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) acc += op[pp][r][ee];
      float *dst = part + (((int64_t)row * g.n_heads + h) * max_chunks + c) * (DH + 2);
      dst[ee] = acc;
      if (ee == 0) {
        dst[DH] = fmaxf(fmaxf(redm[r][0], redm[r][1]), fmaxf(redm[r][2], redm[r][3]));
        dst[DH + 1] = ((reds[r][0] + reds[r][1]) + reds[r][2]) + reds[r][3];
      }
    }
    __syncthreads();
  }
}

// Merge the chunks of (row, head) in chunk order and write the attention
// output as a GEMM activation.
template <bool BF, int DH>
__global__ void k_attn_merge(const float *part, const RowDesc *rows, int n_heads, int max_chunks,
                             void *a_out) {
  using T = typename Act<BF>::T;
  const int r = blockIdx.x, h = blockIdx.y, e = threadIdx.x;
  const int nc = (rows[r].kend + kAttnChunk - 1) / kAttnChunk;
  const float *base = part + ((int64_t)r * n_heads + h) * max_chunks * (DH + 2);
  float m = -INFINITY;
  for (int c = 0; c < nc; ++c) m = fmaxf(m, base[c * (DH + 2) + DH]);
  float l = 0.f, o = 0.f;
  for (int c = 0; c < nc; ++c) {
    const float f = expf(base[c * (DH + 2) + DH] - m);
    l = fmaf(base[c * (DH + 2) + DH + 1], f, l);
    o = fmaf(base[c * (DH + 2) + e], f, o);
  }
  ((T *)a_out)[(int64_t)r * n_heads * DH + h * DH + e] = from_f<T>(o / l);
}

// ---------------------------------------------------------------------------
// Greedy byte and confidence of each row: max over logits 0..255 (the [MASK]
// logit takes no part), lowest id on ties, conf = 1 / sum exp(z - max).
__global__ __launch_bounds__(64) void k_decide(const float *logits, const RowDesc *rows,
                                               int32_t *argmax_ws, float *conf_ws,
                                               int32_t *argmax_out, float *conf_out,
                                               float *logits_out) {
  const int r = blockIdx.x, l = threadIdx.x;
  const float *z = logits + (int64_t)r * kVocab;
  float best = -INFINITY;
  int bi = 0x7fffffff;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = l + 64 * i;
    const float v = z[j];
    if (v > best) { best = v; bi = j; }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ob = __shfl_xor(best, m, 64);
    const int oi = __shfl_xor(bi, m, 64);
    if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += expf(z[l + 64 * i] - best);
  s = wave_sum(s);
  const int oidx = rows[r].oidx;
  if (l == 0) {
    argmax_ws[r] = bi;
    conf_ws[r] = 1.f / s;
    if (oidx >= 0) {
      if (argmax_out) argmax_out[oidx] = bi;
      if (conf_out) conf_out[oidx] = 1.f / s;
    }
  }
  if (oidx >= 0 && logits_out)
    for (int j = l; j < kVocab; j += 64) logits_out[(int64_t)oidx * kVocab + j] = z[j];
}

// Confidence-threshold unmasking with the forced single commit, or one-step
// filling; one wave per sequence, lane j = block position j.
__global__ __launch_bounds__(64) void k_unmask(const SeqDesc *seqs, const int32_t *argmax_ws,
                                               const float *conf_ws, int32_t *block_tok,
                                               float alpha, int one_step, int32_t *masked_left) {
  const SeqDesc sd = seqs[blockIdx.x];
  if (sd.nblk <= 0) return;
  const int j = threadIdx.x;
  const bool active = j < sd.nblk;
  const int tok = active ? block_tok[sd.blk0 + j] : 0;
  const bool masked = active && tok == kMask;
  const float c = masked ? conf_ws[sd.blk_row0 + j] : -1.f;
  bool commit = masked && (one_step || c > alpha);
  const unsigned long long mm = __ballot(masked);
  unsigned long long cm = __ballot(commit);
  if (cm == 0ull && mm != 0ull) {
    const float best = wave_max(c);
    const unsigned long long cand = __ballot(masked && c == best);
    commit = (j == __ffsll((long long)cand) - 1);
    cm = __ballot(commit);
  }
  if (commit) block_tok[sd.blk0 + j] = argmax_ws[sd.blk_row0 + j];
  if (j == 0) masked_left[sd.out_b] = __popcll(mm) - __popcll(cm);
}

// Greedy exact-match acceptance: leading draft bytes equal to the prediction
// made one position earlier; the prediction at the first mismatch (or after
// the last draft byte) is appended.
__global__ void k_verify(int batch, const SeqDesc *seqs, int r, const int32_t *draft, int ld_draft,
                         const int32_t *pred, int ld_pred, int32_t *accept_len,
                         int32_t *next_byte) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  const int s = seqs[b].slot;
  const int32_t *dr = draft + (int64_t)s * ld_draft;
  const int32_t *pr = pred + (int64_t)s * ld_pred;
  int a = 0;
  while (a < r && dr[a] == pr[a]) ++a;
  accept_len[s] = a;
  next_byte[s] = pr[a];
}

template <bool BF>
hipError_t gemv_dispatch(const GemmArgs &a, hipStream_t s) {
  const dim3 grid((a.N + 7) / 8);
  if (a.R <= 1) hipLaunchKernelGGL((k_gemv<BF, 1>), grid, dim3(256), 0, s, a);
  else if (a.R <= 2) hipLaunchKernelGGL((k_gemv<BF, 2>), grid, dim3(256), 0, s, a);
  else if (a.R <= 4) hipLaunchKernelGGL((k_gemv<BF, 4>), grid, dim3(256), 0, s, a);
  else if (a.R <= 8) hipLaunchKernelGGL((k_gemv<BF, 8>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_gemv<BF, 16>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(bool bf16, const GemmArgs &a, float * /*rinv_ws*/, void *xnorm_ws,
                       hipStream_t s) {
  if (a.R <= 0) return hipSuccess;
  if (!bf16) return gemv_dispatch<false>(a, s);
  if (a.R < kGemvRows) return gemv_dispatch<true>(a, s);
  GemmArgs b = a;
  if (a.pro == PRO_NORM) {
    hipLaunchKernelGGL((k_rmsnorm_act<true>), dim3(a.R), dim3(256), 0, s, a.H, a.ldh, a.gain, a.K,
                       a.eps, xnorm_ws);
    b.pro = PRO_PLAIN;
    b.X = xnorm_ws;
    b.ldx = a.K;
    b.x_row_off = nullptr;
  }
  hipLaunchKernelGGL(k_gemm_mfma, dim3((a.N + kBN - 1) / kBN, (a.R + kBM - 1) / kBM), dim3(256), 0,
                     s, b);
  return hipGetLastError();
}

hipError_t launch_embed(bool bf16, const void *embed, const float *cross, const RowDesc *rows,
                        int R, int d, int n_layers, int max_lat, const int32_t *block_tok,
                        const int32_t *tokens_dev, float *h, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL((k_embed<true>), dim3(R), dim3(256), 0, s, embed, cross, rows, d, n_layers,
                       max_lat, block_tok, tokens_dev, h);
  else
    hipLaunchKernelGGL((k_embed<false>), dim3(R), dim3(256), 0, s, embed, cross, rows, d, n_layers,
                       max_lat, block_tok, tokens_dev, h);
  return hipGetLastError();
}

hipError_t launch_rope_kv(bool bf16, const float *qkv, int R, const RowDesc *rows,
                          const float2 *rope_tab, float *q_out, void *kv, KVGeom g, int layer,
                          hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL((k_rope_kv<true>), dim3(R), dim3(256), 0, s, qkv, rows, rope_tab, q_out, kv,
                       g, layer);
  else
    hipLaunchKernelGGL((k_rope_kv<false>), dim3(R), dim3(256), 0, s, qkv, rows, rope_tab, q_out, kv,
                       g, layer);
  return hipGetLastError();
}

template <bool BF, int DH>
static void attn_launch(const float *q, const void *kv, KVGeom g, int layer, const SeqDesc *seqs,
                        int n_seq, int max_chunks, const RowDesc *rows, int R, float *part,
                        void *a_out, hipStream_t s) {
  hipLaunchKernelGGL((k_attn_partial<BF, DH>), dim3(max_chunks, g.n_heads, n_seq), dim3(256), 0, s,
                     q, kv, g, layer, seqs, rows, part, max_chunks);
  hipLaunchKernelGGL((k_attn_merge<BF, DH>), dim3(R, g.n_heads), dim3(DH), 0, s, part, rows,
                     g.n_heads, max_chunks, a_out);
}

hipError_t launch_attention(bool bf16, const float *q, const void *kv, KVGeom g, int layer,
                            const SeqDesc *seqs, int n_seq, int max_chunks, const RowDesc *rows,
                            int R, float *part, void *a_out, hipStream_t s) {
  switch (g.d_head) {
    case 32:
      if (bf16) attn_launch<true, 32>(q, kv, g, layer, seqs, n_seq, max_chunks, rows, R, part, a_out, s);
      else attn_launch<false, 32>(q, kv, g, layer, seqs, n_seq, max_chunks, rows, R, part, a_out, s);
      break;
    case 64:
      if (bf16) attn_launch<true, 64>(q, kv, g, layer, seqs, n_seq, max_chunks, rows, R, part, a_out, s);
      else attn_launch<false, 64>(q, kv, g, layer, seqs, n_seq, max_chunks, rows, R, part, a_out, s);
      break;
    case 128:
      if (bf16) attn_launch<true, 128>(q, kv, g, layer, seqs, n_seq, max_chunks, rows, R, part, a_out, s);
      else attn_launch<false, 128>(q, kv, g, layer, seqs, n_seq, max_chunks, rows, R, part, a_out, s);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decide(const float *logits, int R, const RowDesc *rows, int32_t *argmax_ws,
                         float *conf_ws, int32_t *argmax_out, float *conf_out, float *logits_out,
                         hipStream_t s) {
  hipLaunchKernelGGL(k_decide, dim3(R), dim3(64), 0, s, logits, rows, argmax_ws, conf_ws,
                     argmax_out, conf_out, logits_out);
  return hipGetLastError();
}

hipError_t launch_unmask(const SeqDesc *seqs, int n_seq, const int32_t *argmax_ws,
                         const float *conf_ws, int32_t *block_tok, float alpha, int one_step,
                         int32_t *masked_left, hipStream_t s) {
  hipLaunchKernelGGL(k_unmask, dim3(n_seq), dim3(64), 0, s, seqs, argmax_ws, conf_ws, block_tok,
                     alpha, one_step, masked_left);
  return hipGetLastError();
}

hipError_t launch_verify(int batch, const SeqDesc *seqs, int r, const int32_t *draft,
                         int ld_draft, const int32_t *pred, int ld_pred, int32_t *accept_len,
                         int32_t *next_byte, hipStream_t s) {
  hipLaunchKernelGGL(k_verify, dim3((batch + 63) / 64), dim3(64), 0, s, batch, seqs, r, draft,
                     ld_draft, pred, ld_pred, accept_len, next_byte);
  return hipGetLastError();
}

}  // namespace blt
