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
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <type_traits>

#include <mutex>

#include "blt_internal.h"

namespace blt {

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Device-resident passes gate every kernel on a count of sequences with
// masks left (0: the kernel returns at once).  Each gated kernel has two
// instantiations: GT launches with the gate pointer; the ungated one, for
// host-driven passes, does not load it, so its first kernel-argument loads
// are not held behind that pointer's (about 0.25 us per launch measured).
template <bool GT> __device__ __forceinline__ bool gate_closed(const int32_t *gate) {
  if constexpr (GT) return *gate == 0;
  else return false;
}

// The same gate read late, for the kernels of a decoder pass that stream
// large operands (the GEMVs and the split-K attention) when the driver
// expects every pass to have work: GT = 2 loads the gate at entry but tests
// it only after the kernel's loads and products, before its first global
// store, so its round trip overlaps theirs instead of holding them back
// (measured 0.2-0.4 us per launch).  A closed pass then loads and computes
// (its operands are valid: the pass's descriptors stay in place) and stores
// nothing.  GT = 1 tests at entry, GT = 0 has no gate.
template <int GT> __device__ __forceinline__ bool gate_closed_entry(const int32_t *gate) {
  if constexpr (GT == 1) return *gate == 0;
  else return false;
}
template <int GT> __device__ __forceinline__ int gate_open_late(const int32_t *gate) {
  // a scalar load among the kernel-argument loads (as a vector load the
  // compiler moved it to a scalar register at once and waited for it there)
  if constexpr (GT == 2) return *gate;
  else return 1;
}

__device__ __forceinline__ float bf2f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);   // v_cvt_pk_bf16_f32: nearest, ties to even
}
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
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

// Cross-lane exchange inside 16-lane rows through DPP operand modifiers (a
// VALU operand, no LDS round trip).  Applied in this order, the four moves
// pair lane i with i^1, i^2, then the other quad and the other half of its
// row: after step k every lane of an aligned group of 2^k lanes holds the
// group's reduction, bit-identical across the group (+ and max commute).
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7-i of its 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <- lane 15-i of its 16 lanes

template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL> __device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}

// Sum / max over aligned groups of G lanes (G = 1, 2, 4, 8, 16).
template <int G> __device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp_f<kDppXor1>(v);
  if constexpr (G >= 4) v += dpp_f<kDppXor2>(v);
  if constexpr (G >= 8) v += dpp_f<kDppHalfMirror>(v);
  if constexpr (G >= 16) v += dpp_f<kDppMirror>(v);
  return v;
}
template <int G> __device__ __forceinline__ float group_max(float v) {
  if constexpr (G >= 2) v = fmaxf(v, dpp_f<kDppXor1>(v));
  if constexpr (G >= 4) v = fmaxf(v, dpp_f<kDppXor2>(v));
  if constexpr (G >= 8) v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  if constexpr (G >= 16) v = fmaxf(v, dpp_f<kDppMirror>(v));
  return v;
}

__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Whole-wave sum / max, wave-uniform result: 16-lane rows, then the four
// row totals in a fixed order.
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = group_max<16>(v);
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// The residual-update operands of output o of row r: the current residual
// and (with a cross table) the next layer's cross-attention contribution.
struct ResidEpi {
  float h, c;
};

__device__ __forceinline__ ResidEpi resid_operands(const GemmArgs &a, int r, int o) {
  ResidEpi e{a.resid[(int64_t)r * a.ldo + o], 0.f};
  if (a.cross) {
    const RowDesc rd = a.rows[r];
    e.c = a.cross[(((int64_t)rd.slot * a.max_lat + rd.lat) * a.n_layers + a.cross_layer) * a.d + o];
  }
  return e;
}

template <bool BF>
__device__ __forceinline__ void epilogue(const GemmArgs &a, int r, int o, float y, const ResidEpi &re) {
  using T = typename Act<BF>::T;
  switch (a.ep) {
    case EP_STORE_F32:
      a.out_f32[(int64_t)r * a.ldo + o] = y;
      break;
    case EP_RESID:
      a.resid[(int64_t)r * a.ldo + o] = re.h + (y + (a.cross ? re.c : 0.f));
      break;
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
// A workgroup is 4 waves sharing RPW = 64/G output rows: the G lanes of a
// group read 16*G contiguous bytes of their row per load instruction.  The K
// axis is split into four contiguous quarters, one per wave, and lane s of a
// group takes the chunks s, s+G, s+2G, ... (NC of them) of its quarter.  All
// of a lane's weight chunks are loaded at kernel entry, before activations are
// staged, so the whole weight slice is in flight at once.  Partial sums are
// reduced over the group by xor-shuffles and then over the 4 waves in wave
// order: the order depends on K and G only, never on the number of rows, so
// a row's result does not depend on the rows it shares a pass with.
// Activation rows are staged in LDS, RB rows at a time; with the RMSNorm
// prologue the staged values are gain*h and the row's 1/rms scales the dot
// product afterwards.
__device__ __forceinline__ int qkv_rope_row(const GemmArgs &a, int i) {
  // Output i of the QKV+RoPE GEMV: consecutive outputs pair (j, j + dh/2) of
  // one head so both halves of a rotation land in the same workgroup.
  const int half = a.d_head >> 1, p = i >> 1, which = i & 1;
  const int hd = a.d >> 1, sec = p / hd, pp = p - sec * hd, hh = pp / half, j = pp - hh * half;
  return sec * a.d + hh * a.d_head + j + which * half;
}

// Position, slot and rotation (cos, sin) of one output pair of the fused
// QKV projection: what its epilogue needs besides the two dot products.
struct QkvEpi {
  int pos, slot;
  float2 cs;
  int keep_kv;   // the row's keys and values stay as cached
};

// Column j (within its head half) of the pair whose first output is i0.
__device__ __forceinline__ int qkv_pair_j(const GemmArgs &a, int i0) {
  const int half = a.d_head >> 1, p = i0 >> 1, hd = a.d >> 1;
  const int pp = p - (p / hd) * hd;
  return pp - (pp / half) * half;
}

// Epilogue of the fused QKV projection: RoPE on q and k of one (j, j+dh/2)
// pair at the row's position, q kept in f32, k and v written to the cache.
template <bool BF>
__device__ __forceinline__ void qkv_rope_store(const GemmArgs &a, int r, int i0, float y0, float y1,
                                               const QkvEpi &e) {
  using T = typename Act<BF>::T;
  const int half = a.d_head >> 1, p = i0 >> 1;
  const int hd = a.d >> 1, sec = p / hd, pp = p - sec * hd, hh = pp / half, j = pp - hh * half;
  const int lo = hh * a.d_head + j;
  const float2 cs = e.cs;
  if (sec == 0) {
    a.q_out[(int64_t)r * a.d + lo] = y0 * cs.x - y1 * cs.y;
    a.q_out[(int64_t)r * a.d + lo + half] = y1 * cs.x + y0 * cs.y;
    return;
  }
  if (e.keep_kv) return;
  const int64_t plane = (int64_t)a.max_ctx * a.d_head;
  const int64_t head = (((int64_t)e.slot * a.n_layers + a.layer) * 2 + (sec - 1)) * a.n_heads + hh;
  T *kv = (T *)a.kv;
  if (sec == 1) {
    kv[head * plane + k_off(e.pos, j, a.d_head)] = from_f<T>(y0 * cs.x - y1 * cs.y);
    kv[head * plane + k_off(e.pos, j + half, a.d_head)] = from_f<T>(y1 * cs.x + y0 * cs.y);
  } else {
    kv[head * plane + v_off(e.pos, j, a.d_head)] = from_f<T>(y0);
    kv[head * plane + v_off(e.pos, j + half, a.d_head)] = from_f<T>(y1);
  }
}

// The same epilogue for a pair addressed by its natural QKV column n (the
// first half of a head; the second is n + d_h/2), as the MFMA path lays out
// its outputs: q kept in f32 (RoPE), k (RoPE) and v written to the cache.
template <bool BF>
__device__ __forceinline__ void qkv_rope_store_col(const GemmArgs &a, int r, int n, float y0,
                                                   float y1, int pos, int slot, float2 cs,
                                                   int keep_kv) {
  using T = typename Act<BF>::T;
  const int half = a.d_head >> 1, sec = n / a.d, c = n - sec * a.d;
  const int hh = c / a.d_head, j = c - hh * a.d_head;
  if (sec == 0) {
    a.q_out[(int64_t)r * a.d + c] = y0 * cs.x - y1 * cs.y;
    a.q_out[(int64_t)r * a.d + c + half] = y1 * cs.x + y0 * cs.y;
    return;
  }
  if (keep_kv) return;
  const int64_t plane = (int64_t)a.max_ctx * a.d_head;
  const int64_t head = (((int64_t)slot * a.n_layers + a.layer) * 2 + (sec - 1)) * a.n_heads + hh;
  T *kv = (T *)a.kv;
  if (sec == 1) {
    kv[head * plane + k_off(pos, j, a.d_head)] = from_f<T>(y0 * cs.x - y1 * cs.y);
    kv[head * plane + k_off(pos, j + half, a.d_head)] = from_f<T>(y1 * cs.x + y0 * cs.y);
  } else {
    kv[head * plane + v_off(pos, j, a.d_head)] = from_f<T>(y0);
    kv[head * plane + v_off(pos, j + half, a.d_head)] = from_f<T>(y1);
  }
}

// Raw activation data of one 16-byte staged chunk: the chunk itself (plain
// input) or the f32 residual values it is made from (RMSNorm prologue).
template <bool BF, int PRO> struct StageRaw;
template <bool BF> struct StageRaw<BF, PRO_PLAIN> { uint4 v; };
template <> struct StageRaw<true, PRO_NORM> { float4 h0, h1; };
template <> struct StageRaw<false, PRO_NORM> { float4 h0; };

template <bool BF, int PRO>
__device__ __forceinline__ void stage_load(const GemmArgs &a, int rr, int c, StageRaw<BF, PRO> &st) {
  using T = typename Act<BF>::T;
  constexpr int EPC = Act<BF>::EPC;
  if constexpr (PRO == PRO_PLAIN) {
    const T *row = (const T *)a.X + (a.x_row_off ? a.x_row_off[rr] : (int64_t)rr * a.ldx);
    st.v = *(const uint4 *)(row + (int64_t)c * EPC);
  } else {
    const float *hr = a.H + (int64_t)rr * a.ldh + (int64_t)c * EPC;
    st.h0 = *(const float4 *)hr;
    if constexpr (BF) st.h1 = *(const float4 *)(hr + 4);
  }
}

// The staged chunk (gain * h for the RMSNorm prologue) and the sum of
// squares of its residual values, accumulated in element order.
template <bool BF, int PRO>
__device__ __forceinline__ uint4 stage_value(const StageRaw<BF, PRO> &st, uint4 gv, float &ss) {
  if constexpr (PRO == PRO_PLAIN) {
    return st.v;
  } else if constexpr (BF) {
    const float hv[8] = {st.h0.x, st.h0.y, st.h0.z, st.h0.w, st.h1.x, st.h1.y, st.h1.z, st.h1.w};
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ss = fmaf(hv[2 * i], hv[2 * i], ss);
      ss = fmaf(hv[2 * i + 1], hv[2 * i + 1], ss);
      o[i] = f2bf2(__uint_as_float(gw[i] << 16) * hv[2 * i],
                   __uint_as_float(gw[i] & 0xffff0000u) * hv[2 * i + 1]);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
  } else {
    ss = fmaf(st.h0.x, st.h0.x, ss);
    ss = fmaf(st.h0.y, st.h0.y, ss);
    ss = fmaf(st.h0.z, st.h0.z, ss);
    ss = fmaf(st.h0.w, st.h0.w, ss);
    return make_uint4(__float_as_uint(__uint_as_float(gv.x) * st.h0.x),
                      __float_as_uint(__uint_as_float(gv.y) * st.h0.y),
                      __float_as_uint(__uint_as_float(gv.z) * st.h0.z),
                      __float_as_uint(__uint_as_float(gv.w) * st.h0.w));
  }
}

template <bool BF, int G, int NC, int RB, int PRO, int GT>
__global__ __launch_bounds__(256) void k_gemv(GemmArgs a) {
  if (gate_closed_entry<GT>(a.gate)) return;
  const int open = gate_open_late<GT>(a.gate);   // GT = 2: tested before the first store
  constexpr int EPC = Act<BF>::EPC;
  constexpr int RPW = 64 / G;
  constexpr int Q = NC * G, KC = 4 * Q;      // chunks per wave quarter, per row
  constexpr int K = KC * EPC;
  constexpr int CPT = (KC + 255) / 256;      // staged chunks per thread per row
  extern __shared__ uint4 xs[];              // [RB][KC] staged activation rows
  __shared__ float red[4][RB][RPW];
  __shared__ float ssq[4][RB];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane / G, s = lane - g * G;
  const int i = blockIdx.x * RPW + g;        // this group's output (logical index)
  const int ic = min(i, a.N - 1);
  const int orow = a.qkv_rope ? qkv_rope_row(a, ic) : ic;
  const uint4 *wrow = (const uint4 *)a.W + (int64_t)orow * KC + w * Q + s;
  static_assert(RB * RPW <= 256, "one epilogue item per thread and row block");
  uint4 gv[CPT];
  StageRaw<BF, PRO> raw[RB][CPT];
  uint4 wv[NC];
  int rb = 0, nr = min(RB, a.R);
  // Activation loads first (small, cache-resident), then the epilogue
  // operands of this thread's output item, then the weight slice: waiting
  // for the activations leaves every weight load in flight.  Loads that
  // need a loaded row descriptor go out after the weights, so that the dot
  // products never wait for them.
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int c = min(tid + 256 * k, KC - 1);
    if constexpr (PRO == PRO_NORM) gv[k] = *(const uint4 *)((const typename Act<BF>::T *)a.gain + c * EPC);
#pragma unroll
    for (int r = 0; r < RB; ++r)
      if (r < 4 || r < nr) stage_load<BF, PRO>(a, min(r, nr - 1), c, raw[r][k]);  // uniform skip
  }
  // epilogue item of this thread: (row er, output pair ep0) for the fused
  // QKV projection, (row er, output eo) otherwise; clamped so loads are safe
  const int er = a.qkv_rope ? tid / (RPW / 2) : tid / RPW;
  const int erc = min(er, nr - 1);
  const int ep0 = blockIdx.x * RPW + 2 * (tid - er * (RPW / 2));
  const int eo = blockIdx.x * RPW + (tid - er * RPW), eoc = min(eo, a.N - 1);
  // Unconditional loads through uniform pointer selects (the weights stand
  // in for unused operands), so no branch forces an early wait.
  const bool need_row = a.qkv_rope || (a.ep == EP_RESID && a.cross);
  const int4 *rowp = need_row ? (const int4 *)(a.rows + erc) : (const int4 *)a.W;
  const int4 rlo = rowp[0], rhi = rowp[1];        // slot pos tok blk | lat kend oidx attn_flash
  const int2 *rxp = need_row ? (const int2 *)((const int *)(a.rows + erc) + 8) : (const int2 *)a.W;
  const int2 rx = rxp[0];                         // ctr keep_kv
  const float *resp = a.ep == EP_RESID ? a.resid + (int64_t)erc * a.ldo + eoc : (const float *)a.W;
  ResidEpi re{*resp, 0.f};
#pragma unroll
  for (int u = 0; u < NC; ++u) wv[u] = wrow[u * G];
  // keep every use of the loaded descriptors below the weight loads
  __builtin_amdgcn_sched_barrier(0);
  QkvEpi qe{rlo.y, rlo.x, make_float2(1.f, 0.f), a.qkv_rope ? rx.y : 0};
  {
    const int64_t ci = (((int64_t)rlo.x * a.max_lat + rhi.x) * a.n_layers + a.cross_layer) * a.d + eoc;
    const int64_t ti = (int64_t)rlo.y * (a.d_head >> 1) + qkv_pair_j(a, min(ep0, a.N - 2));
    const float2 *csp = a.qkv_rope ? a.rope_tab + ti : (const float2 *)a.W;
    const float *crp = a.ep == EP_RESID && a.cross ? a.cross + ci : (const float *)a.W;
    // consumed only by the epilogue of the matching kind
    qe.cs = *csp;
    re.c = *crp;
  }

  while (true) {
    // Thread tid stages chunks tid, tid+256, ... of every row: the same
    // chunks for every row, so each row's sum of squares has one order.
    float ssr[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      ssr[r] = 0.f;
      if (r >= 4 && r >= nr) continue;       // uniform: rows past the pass
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        float ssk = 0.f;                     // squares of this chunk, in element order
        const uint4 v = stage_value<BF, PRO>(raw[r][k], gv[k], ssk);
        const bool valid = tid + 256 * k < KC; // clamped duplicates add nothing
        ssr[r] += valid ? ssk : 0.f;
        if (valid) xs[r * KC + tid + 256 * k] = v;
      }
    }
    if constexpr (PRO == PRO_NORM) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        if (r >= 4 && r >= nr) continue;
        const float v = wave_sum(ssr[r]);
        if (lane == 0) ssq[w][r] = v;
      }
    }
    __syncthreads();
    // RQ rows at a time: independent accumulation chains and reductions
    // overlap, while only RQ*NC staged chunks are live next to the weights
    // (rows past the last are clamped re-reads whose results are dropped)
    constexpr int RQ = NC <= 4 ? 4 : (NC <= 8 ? 2 : 1);
    for (int r0 = 0; r0 < nr; r0 += RQ) {
      float v[RQ];
#pragma unroll
      for (int j = 0; j < RQ; ++j) v[j] = 0.f;
#pragma unroll
      for (int u = 0; u < NC; ++u)
#pragma unroll
        for (int j = 0; j < RQ; ++j)
          v[j] = dot_chunk<BF>(wv[u], xs[min(r0 + j, nr - 1) * KC + w * Q + s + u * G], v[j]);
#pragma unroll
      for (int j = 0; j < RQ; ++j) v[j] = group_sum<G>(v[j]);
      if (s == 0) {
#pragma unroll
        for (int j = 0; j < RQ; ++j)
          if (r0 + j < nr) red[w][r0 + j][g] = v[j];
      }
    }
    __syncthreads();
    if (!open) return;                       // uniform: a closed device-resident pass
    // one epilogue item per thread; the first row block uses the operands
    // loaded at entry, later blocks load their own
    if (a.qkv_rope) {
      const int r = er, gg = 2 * (tid - er * (RPW / 2)), i0 = ep0;
      if (r < nr && i0 + 1 < a.N) {
        float y0 = ((red[0][r][gg] + red[1][r][gg]) + red[2][r][gg]) + red[3][r][gg];
        float y1 = ((red[0][r][gg + 1] + red[1][r][gg + 1]) + red[2][r][gg + 1]) + red[3][r][gg + 1];
        if constexpr (PRO == PRO_NORM) {
          const float rinv = 1.f / sqrtf((((ssq[0][r] + ssq[1][r]) + ssq[2][r]) + ssq[3][r]) / (float)K + a.eps);
          y0 *= rinv;
          y1 *= rinv;
        }
        if (rb > 0) {
          const RowDesc rd = a.rows[rb + r];
          qe.pos = rd.pos;
          qe.slot = rd.slot;
          qe.keep_kv = rd.keep_kv;
          qe.cs = a.rope_tab[(int64_t)rd.pos * (a.d_head >> 1) + qkv_pair_j(a, i0)];
        }
        qkv_rope_store<BF>(a, rb + r, i0, y0, y1, qe);
      }
    } else {
      const int r = er, gg = tid - er * RPW, oo = eo;
      if (r < nr && oo < a.N) {
        float y = ((red[0][r][gg] + red[1][r][gg]) + red[2][r][gg]) + red[3][r][gg];
        if constexpr (PRO == PRO_NORM)
          y *= 1.f / sqrtf((((ssq[0][r] + ssq[1][r]) + ssq[2][r]) + ssq[3][r]) / (float)K + a.eps);
        if (rb > 0 && a.ep == EP_RESID) re = resid_operands(a, rb + r, oo);
        epilogue<BF>(a, rb + r, oo, y, re);
      }
    }
    rb += RB;
    if (rb >= a.R) break;
    nr = min(RB, a.R - rb);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int c = min(tid + 256 * k, KC - 1);
#pragma unroll
      for (int r = 0; r < RB; ++r)
        if (r < 4 || r < nr) stage_load<BF, PRO>(a, rb + min(r, nr - 1), c, raw[r][k]);
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA GEMM (bf16 x bf16 -> f32) for passes of >= 16 rows: Y[R][N] = X[R][K] W[N][K]^T.
//
// BM x BN output tile per workgroup of 8 waves: a WM x WN grid of wave tiles
// of 16x16 v_mfma_f32_16x16x32_bf16 blocks, and KH groups of waves that
// split each 64-wide K step between them (KH = 2: two 32-wide halves, the
// groups' sums added through LDS after the loop), so every SIMD runs two
// waves that hide each other's LDS and MFMA latencies.  The global loads of
// step k+2 are issued while step k computes (two register slots) and each
// step's tile is stored to one of two LDS buffers, so the load latency
// overlaps the MFMAs of the steps before.  An LDS tile row holds its eight
// 16-byte chunks XOR-swizzled by the row index, so the 16 lanes that read one
// chunk column of 16 rows hit distinct banks.  Workgroups are dispatched
// round-robin over the 8 XCDs; tiles are numbered so that the workgroups of
// one XCD take a contiguous run of them (all row tiles of consecutive column
// tiles) and share those W tiles in the XCD's L2.
constexpr int kGemmBK = 64;

// f(integral_constant<int, I>) for I = 0..N-1: indices stay compile-time
// constants, so register arrays indexed by them are never spilled.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

template <int BM, int BN, int WM, int WN, int KH, bool GT>
__global__ __launch_bounds__(512) void k_gemm_mfma(GemmArgs a) {
  if (gate_closed<GT>(a.gate)) return;
  constexpr int NT = 512, P = 2;                    // threads; register slots of prefetched steps
  constexpr int CH = kGemmBK / 8;                   // 16-byte chunks per tile row
  constexpr int LA = BM * CH / NT, LB = BN * CH / NT;  // chunks per thread per step
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;  // 16x16 tiles per wave
  constexpr int KSUB = 2 / KH;                      // 32-wide k-steps per group and step
  static_assert(WM * WN * KH == 8 && LA >= 1 && LB >= 1, "8 waves");
  // operand tiles (two buffers each); after the K loop the same LDS holds
  // the second group's sums and then the f32 output tile of the QKV+RoPE epilogue
  __shared__ __align__(16) u32x4_t smem[2 * BM * CH + 2 * BN * CH];
  static_assert(BM * BN * 4 <= (int)sizeof(smem), "output tile fits the operand buffers");
  u32x4_t (*sa)[BM * CH] = reinterpret_cast<u32x4_t (*)[BM * CH]>(smem);
  u32x4_t (*sb)[BN * CH] = reinterpret_cast<u32x4_t (*)[BN * CH]>(smem + 2 * BM * CH);
  const int t = threadIdx.x, w = t >> 6, l = t & 63;
  const int kg = w / (WM * WN), wt = w % (WM * WN);   // K group, wave tile
  const int mt = (a.R + BM - 1) / BM, nt = (a.N + BN - 1) / BN, ntiles = mt * nt;
  // XCD x = blockIdx % 8 takes tiles [x * (ntiles/8) + min(x, ntiles%8), ...)
  const int xcd = (int)blockIdx.x & 7;
  const int tile = xcd * (ntiles >> 3) + min(xcd, ntiles & 7) + ((int)blockIdx.x >> 3);
  const int m0 = (tile % mt) * BM, n0 = (tile / mt) * BN;
  // split-K: workgroup row y of the grid takes K steps [y nk, (y+1) nk)
  const int nk = a.K / kGemmBK / (int)gridDim.y;   // a multiple of P (checked at launch)
  const int64_t k0 = (int64_t)blockIdx.y * nk * kGemmBK;
  const uint16_t *X = (const uint16_t *)a.X + k0, *W = (const uint16_t *)a.W + k0;
  // this thread's chunks of each step: tile chunk q = t + NT i (row q / CH,
  // column q % CH); rows past the matrix edge re-read its last row
  const uint16_t *ga[LA], *gb[LB];
  int sla[LA], slb[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int q = t + NT * i, r = q / CH, c = q % CH, rr = min(m0 + r, a.R - 1);
    ga[i] = X + (a.x_row_off ? a.x_row_off[rr] : (int64_t)rr * a.ldx) + c * 8;
    sla[i] = r * CH + (c ^ (r & 7));
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int q = t + NT * i, r = q / CH, c = q % CH, nn = min(n0 + r, a.N - 1);
    gb[i] = W + (int64_t)nn * a.K + c * 8;
    slb[i] = r * CH + (c ^ (r & 7));
  }
  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int wr = (wt / WN) * (BM / WM), wc = (wt % WN) * (BN / WN);
  u32x4_t xa[P][LA], xb[P][LB];              // register slots: step s waits in slot s % P

  auto load = [&](u32x4_t (&ra)[LA], u32x4_t (&rb)[LB], int kt) {
    kt = min(kt, nk - 1);                    // past the end: harmless re-reads
    static_for<0, LA>([&](auto i) { ra[i] = *(const u32x4_t *)(ga[i] + kt * kGemmBK); });
    static_for<0, LB>([&](auto i) { rb[i] = *(const u32x4_t *)(gb[i] + kt * kGemmBK); });
  };
  auto store = [&](u32x4_t *s_a, u32x4_t *s_b, const u32x4_t (&ra)[LA], const u32x4_t (&rb)[LB]) {
    static_for<0, LA>([&](auto i) { s_a[sla[i]] = ra[i]; });
    static_for<0, LB>([&](auto i) { s_b[slb[i]] = rb[i]; });
  };
  auto compute = [&](const u32x4_t *s_a, const u32x4_t *s_b) {
#pragma unroll
    for (int ss = 0; ss < KSUB; ++ss) {
      const int c = (kg * KSUB + ss) * 4 + (l >> 4);
      bf16x8_t af[TM], bw[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wr + i * 16 + (l & 15);
        af[i] = __builtin_bit_cast(bf16x8_t, s_a[r * CH + (c ^ (r & 7))]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wc + j * 16 + (l & 15);
        bw[j] = __builtin_bit_cast(bf16x8_t, s_b[r * CH + (c ^ (r & 7))]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bw[j], acc[i][j], 0, 0, 0);
    }
  };

  // steps 0..P-1 in flight, step 0 staged in LDS buffer 0 and slot 0 refilled
  static_for<0, P>([&](auto j) { load(xa[j], xb[j], j); });
  store(sa[0], sb[0], xa[0], xb[0]);
  load(xa[0], xb[0], P);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += P) {
    // step kt+j computes from buffer j&1 while steps kt+j+1 .. kt+j+P load;
    // step kt+j+1 moves from its slot to the other buffer, and the slot
    // takes step kt+j+1+P
    static_for<0, P>([&](auto j) {
      constexpr int jn = (decltype(j)::value + 1) % P;
      compute(sa[decltype(j)::value & 1], sb[decltype(j)::value & 1]);
      store(sa[(decltype(j)::value + 1) & 1], sb[(decltype(j)::value + 1) & 1], xa[jn], xb[jn]);
      load(xa[jn], xb[jn], kt + decltype(j)::value + 1 + P);
      __syncthreads();
    });
  }
  // acc[i][j][v]: row wr+16i+4(l/16)+v, column wc+16j+l%16 of the tile; with
  // two K groups the second's sums join the first's (a fixed order)
  const bool lead = KH == 1 || kg == 0;
  if constexpr (KH == 2) {
    float *red = reinterpret_cast<float *>(smem);
    if (!lead) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) red[((wt * TM + i) * TN + j) * 256 + v * 64 + l] = acc[i][j][v];
    }
    __syncthreads();
    if (lead) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[i][j][v] += red[((wt * TM + i) * TN + j) * 256 + v * 64 + l];
    }
  }
  if (a.qkv_rope) {
    // QKV projection with RoPE and the KV write: the tile goes through LDS
    // so each thread can take (j, j + d_h/2) pairs of one head (the tile's
    // columns start on a head boundary: BN is a multiple of d_h)
    float *ct = reinterpret_cast<float *>(smem);
    if (KH == 2) __syncthreads();            // the sums above are read
    if (lead) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            ct[(wr + i * 16 + 4 * (l >> 4) + v) * BN + wc + j * 16 + (l & 15)] = acc[i][j][v];
    }
    __syncthreads();
    const int half = a.d_head >> 1;
    for (int it = t; it < BM * (BN / 2); it += NT) {
      const int rr = it / (BN / 2), pc = it - rr * (BN / 2);
      const int c = (pc / half) * a.d_head + pc % half;   // first column of the pair
      const int m = m0 + rr, n = n0 + c;
      if (m >= a.R || n >= a.N) continue;
      const RowDesc rd = a.rows[m];
      qkv_rope_store_col<true>(a, m, n, ct[rr * BN + c], ct[rr * BN + c + half], rd.pos, rd.slot,
                               a.rope_tab[(int64_t)rd.pos * half + (n % a.d_head)], rd.keep_kv);
    }
    return;
  }
  if (!lead) return;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wr + i * 16 + 4 * (l >> 4) + v;
        const int n = n0 + wc + j * 16 + (l & 15);
        if (m >= a.R || n >= a.N) continue;
        if (a.ep == EP_PART)                 // this split's partial product
          a.out_f32[((int64_t)blockIdx.y * a.R + m) * a.N + n] = acc[i][j][v];
        else
          epilogue<true>(a, m, n, acc[i][j][v],
                         a.ep == EP_RESID ? resid_operands(a, m, n) : ResidEpi{0.f, 0.f});
      }
}

// ---------------------------------------------------------------------------
// Weight-streaming MFMA GEMM for decode passes (16 to 1024 rows):
// Y[R][N] = X[R][K] W[N][K]^T, bf16 x bf16 -> f32.
//
// A workgroup of 4 waves takes a 16*TM-row x 64*TN-column tile; wave w owns
// columns [16*TN*w, 16*TN*(w+1)) of it over all 16*TM rows, so every weight
// fragment is used by exactly one wave and is loaded straight from memory
// into the B-operand registers (lane l: column l%16, the 8 consecutive k of
// group l/16), PB 64-wide K steps ahead of the MFMAs that use them, from a
// copy of the weights in fragment order (`k_frag_pack`) where each wave's
// load instruction covers 1 KB of consecutive memory.  Only the
// activations, which all four waves use, go through LDS: chunks of KCS K
// steps, two buffers, rows padded by 16 bytes (the 16 lanes that read one
// k-piece of 16 rows hit distinct banks), one barrier per chunk; the next
// chunk's activations are loaded into registers while the current one is
// computed.  Each output element is one fixed-order chain of MFMAs over its
// K range; split-K (gridDim.y > 1) writes partial products as the staged-tile
// kernel does.  Workgroups of one XCD take consecutive tiles, row tiles
// fastest, so the row tiles of a column tile share its weights in that XCD's
// L2.  Launched as 64x64 tiles with four steps in flight and two-step chunks
// (170 registers, 35 KB of LDS: three workgroups per CU).  Measured at 576
// rows (batch-64 decode): the L2 serves about 85% of the requests and the
// weights are fetched from HBM about once, so these products are bound by how
// fast the L2 delivers re-read tiles to the CUs, which grows with the
// workgroups resident per CU (3.5 TB/s with one 64x256 tile per CU, 7-9
// TB/s with two or three 64x64 tiles); wider tiles (64x128, 64x256), deeper
// prefetch (8 steps) and four-step chunks were slower.  In row-major weight
// order (each load instruction half of 16 lines) it ran about 2x slower.
template <int TM, int TN, int PB, int KCS, bool GT>
__global__ __launch_bounds__(256) void k_gemm_bs(GemmArgs a) {
  if (gate_closed<GT>(a.gate)) return;
  constexpr int NT = 256, BM = 16 * TM, BN = 64 * TN;
  constexpr int CP = KCS * 8;                  // 16-byte k-pieces per row of a chunk
  constexpr int PR = CP + 1;                   // LDS row pitch in pieces (one of padding)
  constexpr int LA = BM * CP / NT;             // chunk pieces loaded per thread
  constexpr int ABUF = BM * PR;                // pieces per chunk buffer
  constexpr int SMEM = (2 * ABUF * 16 > BM * BN * 4 ? 2 * ABUF * 16 : BM * BN * 4) / 16;
  static_assert(PB % KCS == 0 && (BM * CP) % NT == 0 && LA >= 1, "tile shape");
  __shared__ __align__(16) u32x4_t smem[SMEM];
  const int t = threadIdx.x, w = t >> 6, l = t & 63;
  const int mt = (a.R + BM - 1) / BM, nt = (a.N + BN - 1) / BN, ntiles = mt * nt;
  const int xcd = (int)blockIdx.x & 7;
  const int tile = xcd * (ntiles >> 3) + min(xcd, ntiles & 7) + ((int)blockIdx.x >> 3);
  const int m0 = (tile % mt) * BM, n0 = (tile / mt) * BN;
  const int nk = a.K / kGemmBK / (int)gridDim.y;   // a multiple of PB (checked at launch)
  const int nch = nk / KCS;
  const int64_t k0 = (int64_t)blockIdx.y * nk * kGemmBK;
  const uint16_t *X = (const uint16_t *)a.X + k0;
  // chunk piece q = t + NT i of this thread: row q / CP, piece q % CP;
  // rows past the matrix edge re-read its last row (their results are dropped)
  const uint16_t *ga[LA];
  int sla[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int q = t + NT * i, r = q / CP, p = q % CP, rr = min(m0 + r, a.R - 1);
    ga[i] = X + (a.x_row_off ? a.x_row_off[rr] : (int64_t)rr * a.ldx) + p * 8;
    sla[i] = r * PR + p;
  }
  // weights in fragment order (a.Wf): the B operand of column block ct and
  // 32-deep k block kb is the 1 KB at ((ct * K/32 + kb) * 64) * 8 elements;
  // blocks past the matrix edge re-read its last block
  const int wc = w * 16 * TN, nct = (a.N + 15) / 16;
  const uint16_t *gb[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int ct = min((n0 + wc) / 16 + j, nct - 1);
    gb[j] = (const uint16_t *)a.Wf + ((int64_t)ct * (a.K / 32) + k0 / 32) * 512 + l * 8;
  }
  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t ra[LA];                              // the next chunk's activations
  u32x4_t rb[PB][TN][2];                       // weights of steps kt .. kt+PB-1, slot kt % PB

  auto load_a = [&](int c) {
    c = min(c, nch - 1);                       // past the end: harmless re-reads
    static_for<0, LA>([&](auto i) { ra[i] = *(const u32x4_t *)(ga[i] + (int64_t)c * KCS * kGemmBK); });
  };
  auto store_a = [&](int buf) {
    static_for<0, LA>([&](auto i) { smem[buf * ABUF + sla[i]] = ra[i]; });
  };
  auto load_b = [&](auto slot, int kt) {
    kt = min(kt, nk - 1);
    static_for<0, TN>([&](auto j) {
      rb[slot][j][0] = *(const u32x4_t *)(gb[j] + (int64_t)kt * 1024);
      rb[slot][j][1] = *(const u32x4_t *)(gb[j] + (int64_t)kt * 1024 + 512);
    });
  };
  auto compute = [&](int buf, int s, auto slot) {
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      bf16x8_t af[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = __builtin_bit_cast(bf16x8_t, smem[buf * ABUF + (16 * i + (l & 15)) * PR + s * 8 + ss * 4 + (l >> 4)]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              af[i], __builtin_bit_cast(bf16x8_t, rb[slot][j][ss]), acc[i][j], 0, 0, 0);
    }
  };

  // chunk 0's activations first, so staging them waits for nothing else
  load_a(0);
  static_for<0, PB>([&](auto j) { load_b(j, decltype(j)::value); });
  store_a(0);
  load_a(1);
  __syncthreads();
  for (int kt0 = 0; kt0 < nk; kt0 += PB) {
    static_for<0, PB>([&](auto j) {
      constexpr int s = decltype(j)::value;
      const int c = kt0 / KCS + s / KCS;       // chunk of step kt0 + s
      compute(c & 1, s % KCS, j);
      load_b(j, kt0 + s + PB);
      if constexpr (s % KCS == KCS - 1) {
        // chunk c is done: chunk c+1 goes to the other buffer (last read by
        // chunk c-1, before the previous barrier), chunk c+2 is fetched
        store_a((c + 1) & 1);
        load_a(c + 2);
        __syncthreads();
      }
    });
  }
  // acc[i][j][v]: row 16i+4(l/16)+v, column wc+16j+l%16 of the tile
  if (a.qkv_rope) {
    // QKV projection with RoPE and the KV write through an f32 tile in LDS
    // (the tile's columns start on a head boundary: BN is a multiple of d_h)
    float *ct = reinterpret_cast<float *>(smem);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) ct[(i * 16 + 4 * (l >> 4) + v) * BN + wc + j * 16 + (l & 15)] = acc[i][j][v];
    __syncthreads();
    const int half = a.d_head >> 1;
    for (int it = t; it < BM * (BN / 2); it += NT) {
      const int rr = it / (BN / 2), pc = it - rr * (BN / 2);
      const int c = (pc / half) * a.d_head + pc % half;   // first column of the pair
      const int m = m0 + rr, n = n0 + c;
      if (m >= a.R || n >= a.N) continue;
      const RowDesc rd = a.rows[m];
      qkv_rope_store_col<true>(a, m, n, ct[rr * BN + c], ct[rr * BN + c + half], rd.pos, rd.slot,
                               a.rope_tab[(int64_t)rd.pos * half + (n % a.d_head)], rd.keep_kv);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + i * 16 + 4 * (l >> 4) + v;
        const int n = n0 + wc + j * 16 + (l & 15);
        if (m >= a.R || n >= a.N) continue;
        if (a.ep == EP_PART)                 // this split's partial product
          a.out_f32[((int64_t)blockIdx.y * a.R + m) * a.N + n] = acc[i][j][v];
        else
          epilogue<true>(a, m, n, acc[i][j][v],
                         a.ep == EP_RESID ? resid_operands(a, m, n) : ResidEpi{0.f, 0.f});
      }
}

// RMSNorm rows into an activation buffer (MFMA path prologue).  SPLITS > 0:
// a split-K residual product is pending (partial products p.out_f32[split][R][K],
// its cross term per p.cross): the row first takes h += (sum + cross), the
// partials added in split order, as the product's own epilogue would.  Each
// thread takes elements t + 256 i of blocks of 2048, every load of a block
// issued before the first is used.
template <bool BF, int SPLITS, bool GT>
__global__ __launch_bounds__(256) void k_rmsnorm_act(float *H, int64_t ldh, const void *gain,
                                                     int K, float eps, void *out, GemmArgs p) {
  if (gate_closed<GT>(p.gate)) return;
  using T = typename Act<BF>::T;
  constexpr int E = 8;                       // elements per thread and block
  constexpr int NS = SPLITS > 0 ? SPLITS : 1;
  __shared__ float part[4];
  const int r = blockIdx.x, t = threadIdx.x;
  float *hr = H + (int64_t)r * ldh;
  RowDesc rd{};
  if (SPLITS > 0 && p.cross) rd = p.rows[r];   // first, so it lands while the rest is in flight
  float ss = 0.f, v[E];
  for (int kb = 0; kb < K; kb += 256 * E) {
    float hv[E], y[E][NS], cv[E];
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int k = min(kb + t + 256 * i, K - 1);   // past the row: re-reads, dropped below
      hv[i] = hr[k];
      if constexpr (SPLITS > 0) {
#pragma unroll
        for (int sp = 0; sp < SPLITS; ++sp) y[i][sp] = p.out_f32[((int64_t)sp * p.R + r) * K + k];
      }
    }
    if constexpr (SPLITS > 0) {
      const float *cr =
          p.cross ? p.cross + (((int64_t)rd.slot * p.max_lat + rd.lat) * p.n_layers + p.cross_layer) * p.d
                  : nullptr;
#pragma unroll
      for (int i = 0; i < E; ++i) cv[i] = cr ? cr[min(kb + t + 256 * i, K - 1)] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int k = kb + t + 256 * i;
      float x = hv[i];
      if constexpr (SPLITS > 0) {
        float sum = y[i][0];
#pragma unroll
        for (int sp = 1; sp < SPLITS; ++sp) sum += y[i][sp];
        x = x + (sum + cv[i]);
        if (k < K) hr[k] = x;
      }
      v[i] = x;
      if (k < K) ss = fmaf(x, x, ss);
    }
  }
  ss = wave_sum(ss);
  if ((t & 63) == 0) part[t >> 6] = ss;
  __syncthreads();
  const float tot = ((part[0] + part[1]) + part[2]) + part[3];
  const float rinv = 1.f / sqrtf(tot / (float)K + eps);
  const T *g = (const T *)gain;
  T *o = (T *)out + (int64_t)r * K;
  for (int kb = 0; kb < K; kb += 256 * E) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int k = kb + t + 256 * i;
      // one block: the values are still in registers; else this thread's own writes
      if (k < K) o[k] = from_f<T>(to_f(g[k]) * (K <= 256 * E ? v[i] : hr[k]) * rinv);
    }
  }
}

// ---------------------------------------------------------------------------
// h[r] = E[tok_r] + cross contribution of layer 0 for the row's latent.
template <bool BF, bool GT>
__global__ __launch_bounds__(256) void k_embed(const void *embed, const float *cross,
                                               const RowDesc *rows, int d, int n_layers,
                                               int max_lat, const int32_t *block_tok,
                                               const int32_t *tokens_dev, float *h,
                                               const int32_t *gate) {
  if (gate_closed<GT>(gate)) return;   // device-resident pass with nothing left to do
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
template <bool BF, bool GT>
__global__ __launch_bounds__(256) void k_rope_kv(const float *qkv, const RowDesc *rows,
                                                 const float2 *rope_tab, float *q_out, void *kvp,
                                                 KVGeom g, int layer, const int32_t *gate) {
  if (gate_closed<GT>(gate)) return;   // device-resident pass with nothing left to do
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
    if (rd.keep_kv) continue;
    const float k1 = src[d + lo], k2 = src[d + hi];
    const int64_t kb = ((((int64_t)rd.slot * g.n_layers + layer) * 2 + 0) * g.n_heads + hh) * plane;
    const int64_t vb = ((((int64_t)rd.slot * g.n_layers + layer) * 2 + 1) * g.n_heads + hh) * plane;
    kv[kb + k_off(rd.pos, j, dh)] = from_f<T>(k1 * cs.x - k2 * cs.y);
    kv[kb + k_off(rd.pos, j + half, dh)] = from_f<T>(k2 * cs.x + k1 * cs.y);
    kv[vb + v_off(rd.pos, j, dh)] = from_f<T>(src[2 * d + lo]);
    kv[vb + v_off(rd.pos, j + half, dh)] = from_f<T>(src[2 * d + hi]);
  }
}

// ---------------------------------------------------------------------------
// Split-K attention partials.
//
// Cache layout per (sequence, layer, head): K in tiles of 32 positions,
// [max_ctx / 32][d_head / 32][32][32] (k_off: 32-dimension slices of the
// tile's keys), and V transposed in tiles of 32 positions,
// [max_ctx / 32][d_head][32] (v_off), so that both products below read
// their operands straight from HBM with 16-byte loads that cover whole
// 128-byte lines, and a wave's 32 keys of K and of V are each one
// contiguous block.  The bf16 kernel streams both with non-temporal loads:
// every line is read once per pass.
//
// Workgroup (chunk c, head h, sequence b) owns keys [c*128, c*128+128) of
// that sequence, for every row of the sequence in the pass; row r reads keys
// [0, kend_r).  For each row it writes the chunk's unnormalised output
// o = sum_k exp(s_k - m) v_k with m = max_k s_k and l = sum_k exp(s_k - m).
// Keys past a row's kend contribute exact zeros, so a row's partials depend
// only on its own query and keys (never on the other rows of the pass).
constexpr int kCK = kAttnChunk;

// Row reductions over the four 16-lane groups of a wave (lanes l, l^16, l^32,
// l^48 hold the same row): two cross-lane swaps, no LDS.
__device__ __forceinline__ float max_lane_groups(float x) {
  // max over lanes l, l^16, l^32, l^48 (the four lane groups of a 16-lane row)
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float sum_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// ---------------------------------------------------------------------------
// GEMV on MFMA for bfloat16 passes of 1..15 rows (weight-streaming bound).
//
// A workgroup of 4 waves takes 16 output columns; wave w takes K quarter w
// in 32-wide steps of v_mfma_f32_16x16x32_bf16, with the activations as the A
// operand (lane l: row l%16, k 8(l/16)..+8; rows past the pass are zeros and
// read nothing) and the weight rows as the B operand (lane l: column l%16),
// so each lane's weight piece is 16 contiguous bytes and SB steps' pieces are
// in flight at once.  The four waves' 16x16 sums are added through LDS in
// wave order.  With the RMSNorm prologue the A operand is gain*h rounded to
// bf16, each lane sums the squares of the h values it loads (in step order),
// lane groups and waves add them in a fixed order, and the row's 1/rms
// scales its outputs.  A row's result does not depend on the other rows of
// the pass: the MFMA keeps rows apart and no order depends on the row count.
// Its cost hardly grows with the row count (a cold pass of 1 to 9 rows at the
// 1B-class shapes runs in the time of a plain read of the weights).
template <int PRO, int SB, int GT>
__global__ __launch_bounds__(256) void k_gemv_mfma(GemmArgs a) {
  if (gate_closed_entry<GT>(a.gate)) return;
  const int open = gate_open_late<GT>(a.gate);   // GT = 2: tested before the first store
  const int t = threadIdx.x, w = t >> 6, l = t & 63, lr = l & 15, lq = l >> 4;
  const int n0 = blockIdx.x * 16;
  const int kq = a.K / 4, steps = kq / 32;  // this wave's K range in 32-wide steps (a multiple of SB)
  const int kw = w * kq + 8 * lq;
  const bool live = lr < a.R;
  const int row = min(lr, a.R - 1);
  // the lane's weight row: output column n0 + lr (QKV+RoPE: the permuted row
  // that keeps both halves of a rotation pair in one workgroup)
  const int col = min(n0 + lr, a.N - 1);
  const uint16_t *wp =
      (const uint16_t *)a.W + (int64_t)(a.qkv_rope ? qkv_rope_row(a, col) : col) * a.K + kw;
  const uint16_t *xp = nullptr, *gp = nullptr;
  const float *hp = nullptr;
  if constexpr (PRO == PRO_PLAIN) {
    xp = (const uint16_t *)a.X + (a.x_row_off ? a.x_row_off[row] : (int64_t)row * a.ldx) + kw;
  } else {
    hp = a.H + (int64_t)row * a.ldh + kw;
    gp = (const uint16_t *)a.gain + kw;
  }
  // QKV + RoPE epilogue operands of this thread's output (row t/16, the pair
  // at column n0 + t%16): the row's position and slot go out first, the
  // rotation's cos/sin right after the first weight loads, so that neither
  // dependent load is waited for after the products
  const int erow = min(t >> 4, a.R - 1);
  int epos = 0, eslot = 0, ekeep = 0;
  float2 ecs = make_float2(1.f, 0.f);
  if (a.qkv_rope) {
    epos = a.rows[erow].pos;
    eslot = a.rows[erow].slot;
    ekeep = a.rows[erow].keep_kv;
  }
  __builtin_amdgcn_sched_barrier(0);
  __shared__ float red[4][16][17];
  __shared__ float ssq[4][16];
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  for (int s0 = 0; s0 < steps; s0 += SB) {
    u32x4_t wv[SB], xv[SB], gv[SB];
    float4 h0[SB], h1[SB];
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      const int k = (s0 + j) * 32;
      wv[j] = *(const u32x4_t *)(wp + k);
      if constexpr (PRO == PRO_PLAIN) {
        xv[j] = live ? *(const u32x4_t *)(xp + k) : u32x4_t{0u, 0u, 0u, 0u};
      } else {
        h0[j] = live ? *(const float4 *)(hp + k) : make_float4(0.f, 0.f, 0.f, 0.f);
        h1[j] = live ? *(const float4 *)(hp + k + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        gv[j] = *(const u32x4_t *)(gp + k);
      }
    }
    if (a.qkv_rope && s0 == 0) {
      __builtin_amdgcn_sched_barrier(0);
      ecs = a.rope_tab[(int64_t)epos * (a.d_head >> 1) + qkv_pair_j(a, min(n0 + (t & 15), a.N - 2))];
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      u32x4_t av;
      if constexpr (PRO == PRO_PLAIN) {
        av = xv[j];
      } else {
        const float hv[8] = {h0[j].x, h0[j].y, h0[j].z, h0[j].w, h1[j].x, h1[j].y, h1[j].z, h1[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ss = fmaf(hv[2 * i], hv[2 * i], ss);
          ss = fmaf(hv[2 * i + 1], hv[2 * i + 1], ss);
          av[i] = f2bf2(__uint_as_float(gv[j][i] << 16) * hv[2 * i],
                        __uint_as_float(gv[j][i] & 0xffff0000u) * hv[2 * i + 1]);
        }
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                     __builtin_bit_cast(bf16x8_t, wv[j]), acc, 0, 0, 0);
    }
  }
  // acc[v]: row 4(l/16)+v, column l%16 of the tile
#pragma unroll
  for (int v = 0; v < 4; ++v) red[w][4 * lq + v][lr] = acc[v];
  if constexpr (PRO == PRO_NORM) {
    ss = sum_lane_groups(ss);               // the four lane groups holding row lr
    if (lq == 0) ssq[w][lr] = ss;
  }
  __syncthreads();
  if (!open) return;                        // uniform: a closed device-resident pass
  const int r = t >> 4, c = t & 15;         // one output per thread: row r, column n0 + c
  if (r >= a.R) return;
  float rinv = 1.f;
  if constexpr (PRO == PRO_NORM)
    rinv = 1.f / sqrtf((((ssq[0][r] + ssq[1][r]) + ssq[2][r]) + ssq[3][r]) / (float)a.K + a.eps);
  auto out = [&](int cc) {
    return (((red[0][r][cc] + red[1][r][cc]) + red[2][r][cc]) + red[3][r][cc]) * rinv;
  };
  if (a.qkv_rope) {
    // outputs (n0+c, n0+c+1), c even: the (j, j + d_h/2) pair of one head
    const int i0 = n0 + c;
    if ((c & 1) || i0 + 1 >= a.N) return;
    qkv_rope_store<true>(a, r, i0, out(c), out(c + 1), QkvEpi{epos, eslot, ecs, ekeep});
    return;
  }
  const int n = n0 + c;
  if (n >= a.N) return;
  epilogue<true>(a, r, n, out(c), a.ep == EP_RESID ? resid_operands(a, r, n) : ResidEpi{0.f, 0.f});
}


// bfloat16: a workgroup takes nsub consecutive chunks of kCK keys of one
// (sequence, head) (PIPE: nsub > 1), each wave 32 keys of every chunk, and up
// to 16 rows at a time.  Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_16x16x32_bf16; the K rows are fed to the two 16-key score tiles
// permuted (row m of tile t is key 8(m/4) + 4t + m%4) so that lane group q
// ends up holding keys 8q..8q+7 of the wave's 32 for row lr: exactly the
// B-operand layout of O^T += V^T P^T with k-slot 8q+i = key 8q+i, so the V
// operand of lane (dim, q) is one 16-byte piece of the transposed V tile and
// the output O^T[dim][row] keeps each row's values in the lanes that hold
// its running max and sum (the rescale between chunks is lane-local).  The
// loads of chunk i+1 are issued before chunk i is computed; the softmax runs
// in base-2 units (one multiply and one exp2 per score) over all the
// workgroup's chunks, P is split into bf16 hi and lo parts (two MFMAs per
// output tile, about 16 significant bits), and the four waves' (o, m, l) are
// combined through LDS in wave order into one partial per workgroup (m
// stored in natural-log units) or, when one workgroup covers all of a
// sequence's keys (direct), into the normalised output itself.  Partials
// written to HBM slow the key stream far beyond their size, so large passes
// take many chunks per workgroup; one chunk keeps the most workgroups for
// small passes, and stays in registers for every group of 16 rows.  WG = 2:
// eight waves in two groups that take alternate chunks (group 0 the even
// ones), so one workgroup covers a (sequence, head) with twice the loads in
// flight; their eight (o, m, l) are combined the same way.
template <int DH, bool PIPE, int WG, int GT>
__global__ __launch_bounds__(256 * WG) void k_attn_mfma(const float *q, const void *kvp, KVGeom g,
                                                        int layer, const SeqDesc *seqs,
                                                        const RowDesc *rows, float *part,
                                                        int max_chunks, int chunks_per_wg,
                                                        int direct, void *a_out, SeqDesc sd_arg,
                                                        int use_sd_arg, const int32_t *gate) {
  if (gate_closed_entry<GT>(gate)) return;
  const int open = gate_open_late<GT>(gate);  // GT = 2: tested before the first store
  constexpr int NSUB = PIPE ? 2 : 1;          // > 1: the prefetching loop
  constexpr int NWV = 4 * WG;                 // waves
  constexpr int KS = DH / 32;                 // k-steps of the score product
  constexpr int DT = DH / 16;                 // 16-dim output tiles of P.V
  constexpr int KW = 32;                      // keys per wave and chunk
  constexpr int OST = DH + 4;                 // LDS row stride of the wave outputs
  __shared__ float ow[NWV][16 * OST];
  __shared__ float mw[NWV][16], lw[NWV][16];
  __shared__ int kends[16];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  // a single sequence's descriptor may come with the launch: the key and
  // query loads then need no memory round trip before them
  const SeqDesc sd = use_sd_arg ? sd_arg : seqs[b];
  const int key0 = c * kCK * chunks_per_wg;
  if (key0 >= sd.kmax || sd.attn_flash) return;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, lr = lane & 15, lq = lane >> 4;
  // chunk group (chunks grp, grp + WG, ...) and 32-key slice of the wave
  const int grp = WG == 1 ? 0 : w >> 2, wq = WG == 1 ? w : w & 3;
  const int d = g.n_heads * DH;
  const int64_t plane = (int64_t)g.max_ctx * DH;
  const uint16_t *Kp =
      (const uint16_t *)kvp + ((((int64_t)sd.slot * g.n_layers + layer) * 2 + 0) * g.n_heads + h) * plane;
  const uint16_t *Vt = Kp + (int64_t)g.n_heads * plane;
  const int klast = sd.kmax - 1;              // every cache row below kmax holds data
  // chunks holding keys (one without PIPE: the launcher passes chunks_per_wg = 1)
  const int nsub = PIPE ? min(chunks_per_wg, (sd.kmax - key0 + kCK - 1) / kCK) : 1;

  // K (A operand: key kw0 + 8(lr/4) + 4kt + lr%4, dims 32ks+8lq..+8) and the
  // raw V pieces (dims 16dt+lr, keys kw0+8lq..+8) of one chunk; key indices
  // are clamped into the written cache rows
  auto load = [&](int kw0, bf16x8_t (&ka)[2][KS], u32x4_t (&vg)[DT]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = min(kw0 + 8 * (lr >> 2) + 4 * kt + (lr & 3), klast);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        ka[kt][ks] = __builtin_bit_cast(
            bf16x8_t, __builtin_nontemporal_load((const u32x4_t *)(Kp + k_off(key, 32 * ks + 8 * lq, DH))));
    }
    const int va = min(kw0 + 8 * lq, klast & ~7);   // a group clamped here lies wholly past kmax
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      vg[dt] = __builtin_nontemporal_load((const u32x4_t *)(Vt + v_off(va, 16 * dt + lr, DH)));
  };
  int nr = min(16, sd.nrows);
  float4 qf[KS][2];
  {
    const float *qr = q + (int64_t)(sd.row0 + min(lr, nr - 1)) * d + h * DH + 8 * lq;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks][0] = *(const float4 *)(qr + 32 * ks);
      qf[ks][1] = *(const float4 *)(qr + 32 * ks + 4);
    }
  }
  int my_kend = rows[sd.row0 + min(lr, nr - 1)].kend;
  bf16x8_t ka[2][KS], kn[2][KS];
  u32x4_t vg[DT], vn[DT];
  if (grp < nsub) load(key0 + kCK * grp + wq * KW, ka, vg);
  const float c2 = 1.4426950408889634f / sqrtf((float)DH);   // log2(e) / sqrt(d_h)

  for (int rg = 0;;) {
    if (t < 16) kends[t] = rows[sd.row0 + rg + min(t, nr - 1)].kend;
    bf16x8_t qb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8_t v;
      v[0] = (__bf16)qf[ks][0].x; v[1] = (__bf16)qf[ks][0].y;
      v[2] = (__bf16)qf[ks][0].z; v[3] = (__bf16)qf[ks][0].w;
      v[4] = (__bf16)qf[ks][1].x; v[5] = (__bf16)qf[ks][1].y;
      v[6] = (__bf16)qf[ks][1].z; v[7] = (__bf16)qf[ks][1].w;
      qb[ks] = v;
    }
    float m = -INFINITY, lp = 0.f;            // running max (base 2) and sum of row lr
    f32x4_t o[DT];                            // o[dt][v]: row lr, dim 16dt+4lq+v
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int sb = grp; sb < nsub; sb += WG) {
      const int kw0 = key0 + kCK * sb + wq * KW;
      if (NSUB > 1 && sb + WG < nsub) load(kw0 + WG * kCK, kn, vn);
      const int kq = kw0 + 8 * lq;            // the lane group's first key
      // S^T tiles: acc[kt][v] = score of key kq+4kt+v for row lr
      f32x4_t acc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        acc[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kt][ks], qb[ks], acc[kt], 0, 0, 0);
      }
      float sv[8];
      float mt = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int key = kq + 4 * kt + v;
          const float x = key < my_kend ? acc[kt][v] * c2 : -INFINITY;
          sv[kt * 4 + v] = x;
          mt = fmaxf(mt, x);
        }
      mt = max_lane_groups(mt);               // the four lane groups holding row lr
      const float m_new = fmaxf(m, mt);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
      m = m_new;
      float ps = 0.f;
      bf16x8_t pa_hi, pa_lo;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pv = sv[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[i] - m_new);
        ps += pv;
        const __bf16 hb = (__bf16)pv;
        pa_hi[i] = hb;
        pa_lo[i] = (__bf16)(pv - (float)hb);
      }
      lp = lp * alpha + ps;
      // V operand (k-slot 8q+i = key kq+i); keys at or past kmax (never
      // written) become 0
      bf16x8_t vb[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        u32x4_t x = vg[dt];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = kq + 2 * i < sd.kmax ? (x[i] & 0xffffu) : 0u;
          const uint32_t hi = kq + 2 * i + 1 < sd.kmax ? (x[i] & 0xffff0000u) : 0u;
          x[i] = lo | hi;
        }
        vb[dt] = __builtin_bit_cast(bf16x8_t, x);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        o[dt] = o[dt] * alpha;
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb[dt], pa_hi, o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb[dt], pa_lo, o[dt], 0, 0, 0);
      }
      if constexpr (NSUB > 1) {              // past the last chunk: unused
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) ka[kt][ks] = kn[kt][ks];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vg[dt] = vn[dt];
      }
    }
    const float l = sum_lane_groups(lp);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int v = 0; v < 4; ++v) ow[w][lr * OST + 16 * dt + 4 * lq + v] = o[dt][v];
    if (lq == 0) {
      mw[w][lr] = m;
      lw[w][lr] = l;
    }
    __syncthreads();
    if (!open) return;                        // uniform: a closed device-resident pass
    for (int i = t; i < nr * DH; i += 256 * WG) {
      const int r = i / DH, e = i - r * DH;
      if (kends[r] <= key0) continue;
      float M = -INFINITY;
#pragma unroll
      for (int x = 0; x < NWV; ++x) M = fmaxf(M, mw[x][r]);
      float O = 0.f, L = 0.f;                 // in wave order
#pragma unroll
      for (int x = 0; x < NWV; ++x) {
        const float f = mw[x][r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[x][r] - M);
        O += f * ow[x][r * OST + e];
        L += f * lw[x][r];
      }
      if (direct) {                           // every key of the row: the output itself
        ((uint16_t *)a_out)[(int64_t)(sd.row0 + rg + r) * d + h * DH + e] = f2bf(O / L);
        continue;
      }
      float *dst = part + (((int64_t)(sd.row0 + rg + r) * g.n_heads + h) * max_chunks + c) * (DH + 2);
      dst[e] = O;
      if (e == 0) {
        dst[DH] = M * 0.6931471805599453f;    // natural-log units for the merge
        dst[DH + 1] = L;
      }
    }
    rg += 16;
    if (rg >= sd.nrows) break;
    nr = min(16, sd.nrows - rg);
    {
      const float *qr = q + (int64_t)(sd.row0 + rg + min(lr, nr - 1)) * d + h * DH + 8 * lq;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qf[ks][0] = *(const float4 *)(qr + 32 * ks);
        qf[ks][1] = *(const float4 *)(qr + 32 * ks + 4);
      }
    }
    my_kend = rows[sd.row0 + rg + min(lr, nr - 1)].kend;
    // the first chunk again (one chunk per workgroup keeps it in registers)
    if constexpr (NSUB > 1)
      if (grp < nsub) load(key0 + kCK * grp + wq * KW, ka, vg);
    __syncthreads();                          // LDS of this row group fully read
  }
}

// Causal attention for long runs of clean rows (prompt prefill, KV rebuild):
// the keys of every row are a prefix [0, kend) of its sequence's cache, so
// one pass over the keys serves a whole tile of rows with an online softmax
// (a reference max and a running sum per row, the accumulator rescaled when
// the max outgrows the reference by 2^8) and the normalised output is written
// straight to the activations, with no partials and no merge.
//
// Row tiles hold kFlashRows = 128 consecutive rows of a sequence in the pass,
// 32 per wave in two groups of 16.  Under the causal mask tile i reads about
// i + 1 key tiles, so workgroup (p, head h, sequence b) takes the pair of row
// tiles n-1-p and p, which balances the work of the workgroups; the
// workgroups of one XCD take consecutive (pair, head) items, so they share
// their heads' keys and values in that XCD's L2.  For each row
// tile it walks the keys below the tile's largest kend in tiles of KT keys
// staged through LDS (double-buffered: the next tile's loads are in flight
// during the current tile's products).  Same MFMA formulation as the split-K
// kernel: S^T = K Q^T, with the K rows fed permuted, leaves each lane with
// the scores of one row for 8 consecutive keys of each 32, which are already
// the B operand of O^T += V^T P^T (P rounded to bf16 for the
// product, its sum kept in f32: the kernel is bound by its MFMA and softmax
// work, and the hi + lo split of the split-K kernel would double the P.V
// products), and the lane's O^T entries belong to that same row, so the softmax
// bookkeeping is lane-local apart from the row max over the four lane groups
// (two permlane swaps).  Each K and V operand read from LDS serves both row
// groups.  Scores are taken in base-2 units (times log2(e) / sqrt(d_h)), so
// each probability is one fma and one exp2.  A row's result depends only on
// its own query and kend: keys past kend get probability exactly 0 and leave
// the row's statistics unchanged, whatever the other rows of the tile read.
// Cache rows at or past the sequence's kmax are never written and are staged
// as zeros.
template <int DH, int KG, bool GT>
__global__ __launch_bounds__(256 * KG) void k_attn_flash(const float *q, const void *kvp, KVGeom g,
                                                    int layer, const SeqDesc *seqs,
                                                    const RowDesc *rows, void *a_out,
                                                    const int32_t *gate) {
  if (gate_closed<GT>(gate)) return;   // device-resident pass with nothing left to do
  constexpr int KS = DH / 32;                 // k-steps of the score product
  constexpr int DT = DH / 16;                 // 16-dim output tiles
  constexpr int KT = DH <= 64 ? 64 : 32;      // keys per LDS tile
  constexpr int N16 = KT / 16;                // 16-key score tiles per LDS tile
  constexpr int NJ = KT / 32;                 // 32-key slot groups of the P.V product
  constexpr int KST = DH + 8;                 // LDS row strides (elements), +16 bytes
  constexpr int VST = KT + 8;
  constexpr int NK = KT * DH / 8 / 256;       // 16-byte pieces per thread per tile, K and V each
  static_assert(NK >= 1 && KT * DH / 8 == NK * 256, "tile must split evenly over 256 threads");
  static_assert(kFlashRows == 128, "4 waves x 2 groups x 16 rows");
  static_assert(KG == 1 || KG == 2, "one or two key groups");
  // key group kg (KG = 2: eight waves) walks the key tiles kg, kg + KG, ...
  // through its own two LDS buffers
  constexpr int BUF = KT * KST + DH * VST;    // one buffer: a K tile, then a V^T tile
  __shared__ __align__(16) uint16_t smem[KG * 2 * BUF];
  auto kt_s = [&](int grp, int buf) { return smem + (grp * 2 + buf) * BUF; };
  auto vt_s = [&](int grp, int buf) { return smem + (grp * 2 + buf) * BUF + KT * KST; };
  __shared__ int kend_s[kFlashRows];
  // Workgroups are dispatched round-robin over the 8 XCDs, each with its own
  // L2: workgroup i (linear index) runs on XCD i % 8, which takes a
  // contiguous run of the (pair, head, sequence) items, so the workgroups of
  // one XCD share a few heads' keys and values in its L2 instead of every
  // XCD streaming all of them.
  const int gx = (int)gridDim.x, gy = (int)gridDim.y;
  const int total = gx * gy * (int)gridDim.z;
  const int lin = (int)blockIdx.x + gx * ((int)blockIdx.y + gy * (int)blockIdx.z);
  const int xcd = lin & 7;
  const int item = xcd * (total >> 3) + min(xcd, total & 7) + (lin >> 3);
  const int h = (item / gx) % gy, b = item / (gx * gy);
  const SeqDesc sd = seqs[b];
  if (!sd.attn_flash) return;
  const int ntile = (sd.nrows + kFlashRows - 1) / kFlashRows;
  const int pr = item % gx;
  if (pr >= (ntile + 1) / 2) return;
  const int kg = (int)threadIdx.x >> 8, t = (int)threadIdx.x & 255;   // key group, thread in it
  const int lane = t & 63, w = t >> 6, lr = lane & 15, lq = lane >> 4;
  const int d = g.n_heads * DH;
  const int64_t plane = (int64_t)g.max_ctx * DH;
  const uint16_t *Kp =
      (const uint16_t *)kvp + ((((int64_t)sd.slot * g.n_layers + layer) * 2 + 0) * g.n_heads + h) * plane;
  const uint16_t *Vt = Kp + (int64_t)g.n_heads * plane;
  const int kmax = sd.kmax;
  const float c2 = 1.4426950408889634f / sqrtf((float)DH);   // log2(e) / sqrt(d_h)
  // Keys of the score tiles: row m of 16-key tile k16 is key 32 (k16/2) +
  // 8 (m/4) + 4 (k16%2) + m%4 of the LDS tile, so that after S^T = K Q^T
  // lane group q holds keys 8q..8q+7 of each 32-key group for its row: the
  // B-operand layout of O^T += V^T P^T with k-slot 8q+i = key 8q+i, and the V
  // operand of a lane is one 16-byte piece.
  auto kperm = [](int k16, int m) { return 32 * (k16 >> 1) + 8 * (m >> 2) + 4 * (k16 & 1) + (m & 3); };

  // staging: thread t moves NK 16-byte pieces of K (stored [key][dim] in
  // LDS) and of V^T ([dim][key]) per tile; pieces past kmax become zeros.  V piece i is
  // dimension vdim(i), keys 8 vpiece(i)..+8 of the tile: consecutive pieces
  // run through the V plane's memory in order (its 32-key tiles are
  // [dim][32 keys])
  auto vdim = [](int i) { return (i % (DH * 4)) >> 2; };
  auto vpiece = [](int i) { return 4 * (i / (DH * 4)) + (i & 3); };
  // K piece i is the i-th 16-byte piece of the tile's K memory (whole 32-key
  // tiles of k_off): key kkey(i), dimensions kdim(i)..+8
  auto kkey = [](int i) { return 32 * (i / (4 * DH)) + (i % 128) / 4; };
  auto kdim = [](int i) { return 32 * ((i % (4 * DH)) / 128) + 8 * (i % 4); };
  u32x4_t kr[NK], vr[NK];
  auto load = [&](int tk) {
    const int key0 = tk * KT;
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const int i = t + 256 * j;
      kr[j] = *(const u32x4_t *)(Kp + (int64_t)key0 * DH + 8 * i);
      const int dd = vdim(i), vp = vpiece(i);
      vr[j] = *(const u32x4_t *)(Vt + v_off(key0 + 8 * vp, dd, DH));
    }
  };
  auto store = [&](int tk, int buf) {
    const int key0 = tk * KT;
    if (key0 + KT <= kmax) {                   // uniform: the whole tile lies below kmax
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        const int i = t + 256 * j;
        *(u32x4_t *)(kt_s(kg, buf) + kkey(i) * KST + kdim(i)) = kr[j];
        *(u32x4_t *)(vt_s(kg, buf) + vdim(i) * VST + 8 * vpiece(i)) = vr[j];
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const int i = t + 256 * j;
      const int kk = kkey(i);
      u32x4_t kv = kr[j];
      if (key0 + kk >= kmax) kv = u32x4_t{0u, 0u, 0u, 0u};
      *(u32x4_t *)(kt_s(kg, buf) + kk * KST + kdim(i)) = kv;
      const int dd = vdim(i), vp = vpiece(i);
      u32x4_t vv = vr[j];
      const int k0 = key0 + 8 * vp;
      if (k0 + 8 > kmax) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = k0 + 2 * e < kmax ? (vv[e] & 0xffffu) : 0u;
          const uint32_t hi = k0 + 2 * e + 1 < kmax ? (vv[e] & 0xffff0000u) : 0u;
          vv[e] = lo | hi;
        }
      }
      *(u32x4_t *)(vt_s(kg, buf) + dd * VST + 8 * vp) = vv;
    }
  };

  for (int half = 0; half < 2; ++half) {
    const int tile = half ? pr : ntile - 1 - pr;
    if (half && tile >= ntile - 1 - pr) break;   // odd tile count: the middle tile runs alone
    const int r0 = tile * kFlashRows;
    const int nr = min(kFlashRows, sd.nrows - r0);
    if (half) __syncthreads();                   // LDS of the first row tile fully read
    if (kg == 0 && t < kFlashRows) kend_s[t] = rows[sd.row0 + r0 + min(t, nr - 1)].kend;
    // the lane's rows: 32 w + 16 g + lr of the tile (clamped into the tile's rows)
    bf16x8_t qb[2][KS];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int row = sd.row0 + r0 + min(32 * w + 16 * gi + lr, nr - 1);
      const float *qr = q + (int64_t)row * d + h * DH + 8 * lq;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const float4 a = *(const float4 *)(qr + 32 * ks), c = *(const float4 *)(qr + 32 * ks + 4);
        bf16x8_t v;
        v[0] = (__bf16)a.x; v[1] = (__bf16)a.y; v[2] = (__bf16)a.z; v[3] = (__bf16)a.w;
        v[4] = (__bf16)c.x; v[5] = (__bf16)c.y; v[6] = (__bf16)c.z; v[7] = (__bf16)c.w;
        qb[gi][ks] = v;
      }
    }
    __syncthreads();
    int my_kend[2];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) my_kend[gi] = kend_s[min(32 * w + 16 * gi + lr, nr - 1)];
    // largest kend of the tile, largest and smallest of the wave's rows
    int kend_wg = 0, kend_hi = 0, kend_lo = 0x7fffffff;
    for (int i = 0; i < nr; ++i) {
      const int k = kend_s[i];
      kend_wg = max(kend_wg, k);
      if ((i >> 5) == w) {
        kend_hi = max(kend_hi, k);
        kend_lo = min(kend_lo, k);
      }
    }
    const int ntk = (kend_wg + KT - 1) / KT;

    f32x4_t o[2][DT];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[gi][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

    if (kg < ntk) {
      load(kg);
      store(kg, 0);
    }
    __syncthreads();
    // every key group runs the same number of steps (barriers line up); a
    // group whose tile lies past the last one idles in that step
    for (int it = 0; it * KG < ntk; ++it) {
      const int tk = it * KG + kg;
      const int buf = it & 1;
      const int key0 = tk * KT;
      if (tk + KG < ntk) load(tk + KG);
      if (tk < ntk && key0 < kend_hi) {       // wave-uniform: some row of the wave reads these keys
        // S^T for both row groups; every K operand read once
        f32x4_t acc[2][N16];
#pragma unroll
        for (int k16 = 0; k16 < N16; ++k16) {
          bf16x8_t ka[KS];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            ka[ks] = *(const bf16x8_t *)(kt_s(kg, buf) + kperm(k16, lr) * KST + 32 * ks + 8 * lq);
#pragma unroll
          for (int gi = 0; gi < 2; ++gi) {
            acc[gi][k16] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
              acc[gi][k16] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks], qb[gi][ks], acc[gi][k16], 0, 0, 0);
          }
        }
        // acc[g][k16][v]: raw score of key key0 + 16 k16 + 4 lq + v for the
        // lane's row of group g; masking only where the tile reaches past the
        // smallest kend of the wave's rows
        if (key0 + KT > kend_lo) {
#pragma unroll
          for (int gi = 0; gi < 2; ++gi)
#pragma unroll
            for (int k16 = 0; k16 < N16; ++k16)
#pragma unroll
              for (int v = 0; v < 4; ++v)
                if (key0 + kperm(k16, 4 * lq + v) >= my_kend[gi]) acc[gi][k16][v] = -INFINITY;
        }
        u32x4_t ph[2][NJ];
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
          float sv[KT / 4];                   // the lane's scores, read once from the accumulators
#pragma unroll
          for (int k16 = 0; k16 < N16; ++k16)
#pragma unroll
            for (int v = 0; v < 4; ++v) sv[4 * k16 + v] = acc[gi][k16][v];
          float mt = -INFINITY;
#pragma unroll
          for (int i = 0; i < KT / 4; ++i) mt = fmaxf(mt, sv[i]);
          // The reference max m moves only when a row's max exceeds it by 8
          // (base-2 units): the probabilities exp2(s c - m) stay <= 256, exact
          // in f32 and as bf16 operands, the numerator and the denominator
          // share the scale, and the output is rescaled rarely.  A row whose
          // keys all lie past its kend so far (m = -inf: the second key
          // group's first tiles) takes m = 0 in the exponent, so its masked
          // scores give exp2(-inf) = 0 and not exp2(-inf + inf).
          const float m_tile = max_lane_groups(mt) * c2;
          const bool grow = m_tile > m_run[gi] + 8.f;
          const float m_new = grow ? m_tile : m_run[gi];
          const float alpha = grow ? __builtin_amdgcn_exp2f(m_run[gi] - m_new) : 1.f;
          m_run[gi] = m_new;
          const float m_exp = m_new == -INFINITY ? 0.f : m_new;
          float ps = 0.f;
#pragma unroll
          for (int i = 0; i < KT / 4; i += 2) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[i], c2, -m_exp));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[i + 1], c2, -m_exp));
            ps += p0 + p1;
            ph[gi][i / 8][(i % 8) / 2] = f2bf2(p0, p1);
          }
          l_run[gi] = l_run[gi] * alpha + ps;
          if (__ballot(grow)) {               // the reference max moved for some row of the wave
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[gi][dt] = o[gi][dt] * alpha;
          }
        }
        // O^T += V^T P^T: slot group j holds k-slots 8 lq + i <-> keys
        // 32 j + 8 lq + i, one 16-byte piece of the V^T tile; every V operand read once
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const bf16x8_t va = *(const bf16x8_t *)(vt_s(kg, buf) + (16 * dt + lr) * VST + 32 * j + 8 * lq);
#pragma unroll
            for (int gi = 0; gi < 2; ++gi) {
              o[gi][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  va, __builtin_bit_cast(bf16x8_t, ph[gi][j]), o[gi][dt], 0, 0, 0);
            }
          }
      }
      if (tk + KG < ntk) store(tk + KG, buf ^ 1);
      __syncthreads();
    }
    if constexpr (KG == 2) {
      // the second key group's (o, m, l) join the first's through LDS (the
      // operand buffers are free after the last barrier): o = o0 a0 + o1 a1,
      // l = l0 a0 + l1 a1 with a_i = exp2(m_i - max(m0, m1)); m0 is finite
      // (key 0 is the first group's), a group without keys has m = -inf, a = 0
      float *xs = reinterpret_cast<float *>(smem);
      constexpr int NV = 2 * DT * 4 + 4;     // floats per lane
      static_assert(256 * NV * 4 <= (int)sizeof(smem), "exchange fits the operand buffers");
      float *mine = xs + (size_t)t * NV;
      if (kg == 1) {
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int v = 0; v < 4; ++v) mine[(gi * DT + dt) * 4 + v] = o[gi][dt][v];
          mine[2 * DT * 4 + gi] = m_run[gi];
          mine[2 * DT * 4 + 2 + gi] = l_run[gi];
        }
      }
      __syncthreads();
      if (kg == 0) {
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
          const float m1 = mine[2 * DT * 4 + gi], l1 = mine[2 * DT * 4 + 2 + gi];
          const float mx = fmaxf(m_run[gi], m1);
          const float a0 = __builtin_amdgcn_exp2f(m_run[gi] - mx), a1 = __builtin_amdgcn_exp2f(m1 - mx);
          l_run[gi] = l_run[gi] * a0 + l1 * a1;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int v = 0; v < 4; ++v) o[gi][dt][v] = o[gi][dt][v] * a0 + mine[(gi * DT + dt) * 4 + v] * a1;
        }
      }
    }
    // o[g][dt][v]: unnormalised output of the lane's row of group g, dim 16 dt + 4 lq + v
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      if (kg != 0) break;
      const float L = sum_lane_groups(l_run[gi]);
      const int wr = 32 * w + 16 * gi + lr;
      if (wr < nr) {
        uint16_t *dst = (uint16_t *)a_out + (int64_t)(sd.row0 + r0 + wr) * d + h * DH + 4 * lq;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          uint2 pk;
          pk.x = f2bf2(o[gi][dt][0] / L, o[gi][dt][1] / L);
          pk.y = f2bf2(o[gi][dt][2] / L, o[gi][dt][3] / L);
          *(uint2 *)(dst + 16 * dt) = pk;
        }
      }
    }
  }
}

// float32: keys staged in LDS, two threads per key for the scores (one DPP
// exchange), softmax statistics by 16-lane groups, P.V by (dim, key
// partition) threads with the thread's V column (a row of the transposed V)
// in registers.
template <int DH, bool GT>
__global__ __launch_bounds__(256) void k_attn_f32(const float *q, const void *kvp, KVGeom g,
                                                  int layer, const SeqDesc *seqs,
                                                  const RowDesc *rows, float *part,
                                                  int max_chunks, const int32_t *gate) {
  if (gate_closed<GT>(gate)) return;   // device-resident pass with nothing left to do
  constexpr int RG = 16;                              // rows per row group
  constexpr int ROWB = DH * 4;                        // bytes of one key row
  constexpr int LDB = ROWB + 16;                      // padded LDS row stride (bytes)
  constexpr int CPR = ROWB / 16;                      // 16-byte chunks per key row
  constexpr int HCH = CPR / 2;                        // chunks per half row
  constexpr int NP = 256 / DH, KPP = kCK / NP;        // P.V key partitions
  constexpr int PER = kCK * CPR / 256;                // K chunks per thread
  constexpr int QPT = RG * DH / 256;                  // q elements per thread
  __shared__ __align__(16) char ks[kCK * LDB];        // K rows, then P.V partials
  __shared__ __align__(16) float qs[RG][DH];
  __shared__ __align__(16) float ps[RG][kCK];         // scores, then probabilities
  __shared__ float redm[RG], reds[RG];
  __shared__ int kends[RG];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const SeqDesc sd = seqs[b];
  const int key0 = c * kCK;
  if (key0 >= sd.kmax) return;
  const int t = threadIdx.x;
  const int d = g.n_heads * DH;
  const int64_t plane = (int64_t)g.max_ctx * DH;
  const float *Kp = (const float *)kvp + ((((int64_t)sd.slot * g.n_layers + layer) * 2 + 0) * g.n_heads + h) * plane;
  const float *Vt = Kp + (int64_t)g.n_heads * plane;
  const int nkeys = min(kCK, sd.kmax - key0);

  int nr = min(RG, sd.nrows);
  float qv[QPT];
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int idx = t + 256 * k, r = idx / DH, ee = idx - r * DH;
    qv[k] = q[(int64_t)(sd.row0 + min(r, nr - 1)) * d + h * DH + ee];
  }
  const int my_kend = rows[sd.row0 + min(t & (RG - 1), nr - 1)].kend;
  uint4 kr[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int idx = t + u * 256, key = idx / CPR, cc = idx - key * CPR;
    kr[u] = *(const uint4 *)(Kp + k_off(key0 + min(key, nkeys - 1), 4 * cc, DH));   // 4 floats
  }
  const int kk = t >> 1, hf = t & 1;                  // score phase: key kk, half hf
  const int e = t % DH, kp = t / DH;                  // P.V phase: dim e, partition kp
  // this thread's V column over its key partition (a row of the transposed V)
  float vcol[KPP];
#pragma unroll
  for (int j = 0; j < KPP; ++j)
    vcol[j] = Vt[v_off(key0 + min(kp * KPP + j, nkeys - 1), e, DH)];
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int idx = t + 256 * k, r = idx / DH, ee = idx - r * DH;
    qs[r][ee] = qv[k];
  }
  if (t < RG) kends[t] = my_kend;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int idx = t + u * 256, key = idx / CPR, cc = idx - key * CPR;
    *(uint4 *)(ks + key * LDB + cc * 16) = kr[u];
  }
  const float scale = 1.f / sqrtf((float)DH);
  __syncthreads();

  for (int rg = 0;;) {
    uint4 kh[HCH];
#pragma unroll
    for (int u = 0; u < HCH; ++u) kh[u] = *(const uint4 *)(ks + kk * LDB + (hf * HCH + u) * 16);
    for (int r0 = 0; r0 < nr; r0 += 4) {
      float acc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = 0.f;
#pragma unroll
      for (int u = 0; u < HCH; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[j] = dot_chunk<false>(kh[u], *(const uint4 *)((const char *)&qs[min(r0 + j, nr - 1)][0] +
                                                            (hf * HCH + u) * 16), acc[j]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] = group_sum<2>(acc[j]);
        const int r = r0 + j;
        if (hf == 0 && r < nr) ps[r][kk] = (key0 + kk < kends[r]) ? acc[j] * scale : -INFINITY;
      }
    }
    __syncthreads();
    {
      // softmax statistics: 16 threads per row, 8 keys each
      const int r = t >> 4, sl = t & 15;
      float sv[kCK / 16];
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < kCK / 16; ++j) {
        sv[j] = ps[r][sl * (kCK / 16) + j];
        m = fmaxf(m, sv[j]);
      }
      m = group_max<16>(m);
      float l = 0.f;
#pragma unroll
      for (int j = 0; j < kCK / 16; ++j) {
        const float p = (sv[j] == -INFINITY) ? 0.f : expf(sv[j] - m);
        l += p;
        if (r < nr) ps[r][sl * (kCK / 16) + j] = p;
      }
      l = group_sum<16>(l);
      if (sl == 0) {
        redm[r] = m;
        reds[r] = l;
      }
    }
    __syncthreads();                                  // K rows are free: reuse for partials
    float *op = (float *)ks;                          // [NP][RG][DH]
    for (int r0 = 0; r0 < nr; r0 += 4) {
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = 0.f;
#pragma unroll
      for (int j = 0; j < KPP; j += 4)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 p4 = *(const float4 *)&ps[min(r0 + i, RG - 1)][kp * KPP + j];
          o[i] = fmaf(p4.x, vcol[j], o[i]);
          o[i] = fmaf(p4.y, vcol[j + 1], o[i]);
          o[i] = fmaf(p4.z, vcol[j + 2], o[i]);
          o[i] = fmaf(p4.w, vcol[j + 3], o[i]);
        }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (r0 + i < nr) op[(kp * RG + r0 + i) * DH + e] = o[i];
    }
    __syncthreads();
    for (int i = t; i < nr * DH; i += 256) {
      const int r = i / DH, ee = i - r * DH;
      const int row = sd.row0 + rg + r;
      if (kends[r] <= key0) continue;
      float acc = 0.f;
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) acc += op[(pp * RG + r) * DH + ee];
      float *dst = part + (((int64_t)row * g.n_heads + h) * max_chunks + c) * (DH + 2);
      dst[ee] = acc;
      if (ee == 0) {
        dst[DH] = redm[r];
        dst[DH + 1] = reds[r];
      }
    }
    rg += RG;
    if (rg >= sd.nrows) break;
    // next row group: its q rows and kends; the K rows come back from global
    __syncthreads();
    nr = min(RG, sd.nrows - rg);
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int idx = t + 256 * k, r = idx / DH, ee = idx - r * DH;
      qs[r][ee] = q[(int64_t)(sd.row0 + rg + min(r, nr - 1)) * d + h * DH + ee];
    }
    if (t < RG) kends[t] = rows[sd.row0 + rg + min(t, nr - 1)].kend;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = t + u * 256, key = idx / CPR, cc = idx - key * CPR;
      *(uint4 *)(ks + key * LDB + cc * 16) = *(const uint4 *)(Kp + k_off(key0 + min(key, nkeys - 1), 4 * cc, DH));
    }
    __syncthreads();
  }
}

// Merge of the chunk partials of (row, head) in chunk order; chunk c's
// partial sits at [row][h][c][d_h + 2].  Every load is addressed by the
// pass's chunk count gc alone (chunks past the row's own count are read but
// weighted by an exact 0), so the partial outputs of the first PRE chunks,
// the statistics and the row descriptor are all in flight at once; chunks
// past PRE follow 32 at a time.
template <bool BF, int DH, int PRE, bool GT>
__global__ __launch_bounds__(64) void k_attn_merge(const float *part, const RowDesc *rows,
                                                   int n_heads, int max_chunks, int gc, int ck,
                                                   void *a_out, const int32_t *gate) {
  if (gate_closed<GT>(gate)) return;   // device-resident pass with nothing left to do
  using T = typename Act<BF>::T;
  static_assert(PRE % 32 == 0 || PRE < 32, "later chunks go 32 at a time");
  constexpr int EPL = (DH + 63) / 64;       // output dims per lane
  __shared__ float fw[kMaxChunks];
  const int row = blockIdx.x, h = blockIdx.y, l = threadIdx.x;
  const float *pb = part + ((int64_t)row * n_heads + h) * max_chunks * (DH + 2);
  // the lanes of a chunk read one contiguous row of the partials
  float ov[EPL][PRE];
#pragma unroll
  for (int j = 0; j < EPL; ++j)
#pragma unroll
    for (int u = 0; u < PRE; ++u) ov[j][u] = pb[min(u, gc - 1) * (DH + 2) + min(l + 64 * j, DH - 1)];
  const int c0 = min(l, gc - 1), c1 = min(l + 64, gc - 1);
  const float m0 = pb[c0 * (DH + 2) + DH], m1 = pb[c1 * (DH + 2) + DH];
  const float l0 = pb[c0 * (DH + 2) + DH + 1], l1 = pb[c1 * (DH + 2) + DH + 1];
  const RowDesc rd = rows[row];
  const int nc = (rd.kend + ck - 1) / ck;   // chunks of ck keys holding the row's keys
  // chunk weights f_c = exp(m_c - M) and L = sum_c l_c f_c, one chunk per lane
  const bool ok0 = l < nc, ok1 = l + 64 < nc;
  const float M = wave_max(fmaxf(ok0 ? m0 : -INFINITY, ok1 ? m1 : -INFINITY));
  const float f0 = ok0 ? expf(m0 - M) : 0.f, f1 = ok1 ? expf(m1 - M) : 0.f;
  const float L = wave_sum((ok0 ? l0 : 0.f) * f0 + (ok1 ? l1 : 0.f) * f1);
  fw[l] = f0;
  fw[l + 64] = f1;
  __syncthreads();
  // O[e] = sum_c o_c[e] f_c in chunk order
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = l + 64 * j;
    float O = 0.f;
#pragma unroll
    for (int u = 0; u < PRE; ++u) O = fmaf(u < nc ? ov[j][u] : 0.f, fw[u], O);
    for (int cb = PRE; cb < gc; cb += 32) {
      float ol[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) ol[u] = pb[min(cb + u, gc - 1) * (DH + 2) + min(e, DH - 1)];
#pragma unroll
      for (int u = 0; u < 32; ++u)
        O = fmaf(cb + u < nc ? ol[u] : 0.f, fw[min(cb + u, kMaxChunks - 1)], O);
    }
    if (e < DH && !rd.attn_flash)             // else written by the causal kernel
      ((T *)a_out)[(int64_t)row * n_heads * DH + h * DH + e] = from_f<T>(O / L);
  }
}

// ---------------------------------------------------------------------------
// Greedy byte and confidence of each row: max over logits 0..255 (the [MASK]
// logit takes no part), lowest id on ties, conf = 1 / sum exp(z - max).
// One wave decides row r (lane l = threadIdx.x & 63).
__device__ __forceinline__ void decide_row(int r, const float *logits, const RowDesc *rows,
                                           int32_t *argmax_ws, float *conf_ws, float *ent_ws,
                                           int report_entropy, int32_t *argmax_out,
                                           float *conf_out, float *logits_out) {
  const int l = threadIdx.x & 63;
  const float *z = logits + (int64_t)r * kVocab;
  float best = -INFINITY;
  int bi = 0x7fffffff;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = l + 64 * i;
    const float v = z[j];
    if (v > best) { best = v; bi = j; }
  }
  // (max, lowest index) over each 16-lane row by DPP, then over the rows
#define BLT_ARGMAX_STEP(ctrl)                                            \
  {                                                                     \
    const float ob = dpp_f<ctrl>(best);                                 \
    const int oi = dpp_i<ctrl>(bi);                                     \
    if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }   \
  }
  BLT_ARGMAX_STEP(kDppXor1) BLT_ARGMAX_STEP(kDppXor2)
  BLT_ARGMAX_STEP(kDppHalfMirror) BLT_ARGMAX_STEP(kDppMirror)
#undef BLT_ARGMAX_STEP
  {
    float bv = lane_f(best, 0);
    int bx = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
    for (int q = 16; q < 64; q += 16) {
      const float ob = lane_f(best, q);
      const int oi = __builtin_amdgcn_readlane(bi, q);
      if (ob > bv || (ob == bv && oi < bx)) { bv = ob; bx = oi; }
    }
    best = bv;
    bi = bx;
  }
  // S = sum_b e_b and T = sum_b e_b (z_b - max) with e_b = exp(z_b - max):
  // conf = 1 / S, entropy = ln S - T / S (nats)
  float s = 0.f, tz = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x = z[l + 64 * i] - best;
    const float e = expf(x);
    s += e;
    tz = fmaf(e, x, tz);
  }
  s = wave_sum(s);
  tz = wave_sum(tz);
  const float ent = logf(s) - tz / s;
  const int oidx = rows[r].oidx;
  if (l == 0) {
    argmax_ws[r] = bi;
    conf_ws[r] = 1.f / s;
    ent_ws[r] = ent;
    if (oidx >= 0) {
      if (argmax_out) argmax_out[oidx] = bi;
      if (conf_out) conf_out[oidx] = report_entropy ? ent : 1.f / s;
    }
  }
  if (oidx >= 0 && logits_out)
    for (int j = l; j < kVocab; j += 64) logits_out[(int64_t)oidx * kVocab + j] = z[j];
}

template <bool GT>
__global__ __launch_bounds__(64) void k_decide(const float *logits, const RowDesc *rows,
                                               int32_t *argmax_ws, float *conf_ws, float *ent_ws,
                                               int report_entropy, int32_t *argmax_out,
                                               float *conf_out, float *logits_out,
                                               const int32_t *gate) {
  if (gate_closed<GT>(gate)) return;   // device-resident pass with nothing left to do
  decide_row(blockIdx.x, logits, rows, argmax_ws, conf_ws, ent_ws, report_entropy, argmax_out,
             conf_out, logits_out);
}

// Sampled decisions (temperature / top-p, the stochastic variant paired
// with EB sampling): one workgroup per row, thread j = byte j.  The greedy
// byte, confidence and entropy are those of k_decide (model distribution);
// a row with a draw number ctr >= 0 then takes instead the byte drawn from
// the nucleus of softmax(z / T): with e_j = exp((z_j - max) / T), the mass
// ranked before byte j (larger e, or equal e and lower id) is summed in
// byte order, the nucleus is the bytes with e_j > 0 whose preceding mass is
// below top_p * sum(e), and the draw is the nucleus byte of largest rank
// whose preceding mass is <= u * (nucleus mass).  u is the top 24 bits of
// SplitMix64 output ctr + 1 from state seed + slot (Steele, Lea and Flood,
// 2014), over 2^24.  Its confidence is the model probability of the drawn
// byte.
__device__ __forceinline__ uint64_t splitmix64_nth(uint64_t seed, uint64_t n) {
  uint64_t x = seed + 0x9E3779B97F4A7C15ull * n;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

// Sum and max over the 256 threads: each wave, then the four waves in order.
__device__ __forceinline__ float block_sum256(float v, float *red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}
__device__ __forceinline__ float block_max256(float v, float *red) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

template <bool GT>
__global__ __launch_bounds__(256) void k_decide_sample(const float *logits, const RowDesc *rows,
                                                      int32_t *argmax_ws, float *conf_ws,
                                                      float *ent_ws, int report_entropy,
                                                      int32_t *argmax_out, float *conf_out,
                                                      float *logits_out, SampleArgs smp,
                                                      const int32_t *gate) {
  if (gate_closed<GT>(gate)) return;   // device-resident pass with nothing left to do
  __shared__ float ew[256];
  __shared__ float red[4];
  __shared__ float pick_e;
  const int r = blockIdx.x, t = threadIdx.x;
  const RowDesc rd = rows[r];
  const float *zr = logits + (int64_t)r * kVocab;
  const float z = zr[t];
  // greedy byte: the largest logit, lowest id on ties
  const float best = block_max256(z, red);
  const float bi = block_max256(z == best ? -(float)t : -INFINITY, red);
  int choice = (int)-bi;
  const float x = z - best, e = expf(x);
  const float s = block_sum256(e, red);
  const float tz = block_sum256(e * x, red);
  const float ent = logf(s) - tz / s;
  float conf = 1.f / s;
  if (rd.ctr >= 0) {
    const float eT = expf(x / smp.temperature);
    ew[t] = eT;
    const float sT = block_sum256(eT, red);   // its barriers also publish ew
    float before = 0.f;
    int rank = 0;
    for (int k = 0; k < 256; ++k) {
      const float ek = ew[k];
      const bool prior = ek > eT || (ek == eT && k < t);
      before += prior ? ek : 0.f;
      rank += prior;
    }
    const bool in = before < smp.top_p * sT && eT > 0.f;
    const float mass = block_sum256(in ? eT : 0.f, red);
    const uint64_t bits = splitmix64_nth(smp.seed + (uint64_t)rd.slot, (uint64_t)rd.ctr + 1) >> 40;
    const float c = (float)bits * (1.f / 16777216.f) * mass;
    const bool cand = in && before <= c;
    const float top = block_max256(cand ? (float)rank : -1.f, red);
    choice = (int)block_max256(cand && (float)rank == top ? (float)t : -1.f, red);
    if (t == choice) pick_e = e;
    __syncthreads();
    conf = pick_e / s;
  }
  if (t == 0) {
    argmax_ws[r] = choice;
    conf_ws[r] = conf;
    ent_ws[r] = ent;
    if (rd.oidx >= 0) {
      if (argmax_out) argmax_out[rd.oidx] = choice;
      if (conf_out) conf_out[rd.oidx] = report_entropy ? ent : conf;
    }
  }
  if (rd.oidx >= 0 && logits_out)
    for (int j = t; j < kVocab; j += 256) logits_out[(int64_t)rd.oidx * kVocab + j] = zr[j];
}

// dst = src^T for an n x n matrix (set-up only: the cross-attention weights).
template <typename T>
__global__ __launch_bounds__(256) void k_transpose(const T *src, T *dst, int n) {
  const int64_t total = (int64_t)n * n;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / n, c = i - r * n;
    dst[c * n + r] = src[i];
  }
}

// Unmasking after a pass; one wave per sequence, lane j = block position j.
// THRESHOLD: masked positions with conf > alpha, or if none the most
// confident one (lowest position on ties); ONE_STEP: every masked position;
// ENTROPY: masked positions ranked by entropy (ties by position), committed
// in rank order while the running entropy sum stays <= alpha (the bound
// gamma), at least the first.
// One wave unmasks the block of sequence sd (lane j = block position j).
__device__ __forceinline__ void unmask_seq(const SeqDesc &sd, const int32_t *argmax_ws,
                                           const float *conf_ws, const float *ent_ws,
                                           int32_t *block_tok, float alpha, int mode,
                                           int32_t *masked_left, int32_t *gate,
                                           int32_t *pass_count) {
  if (sd.nblk <= 0) return;
  const int j = threadIdx.x & 63;
  const bool active = j < sd.nblk;
  const int tok = active ? block_tok[sd.blk0 + j] : 0;
  const bool masked = active && tok == kMask;
  const unsigned long long mm = __ballot(masked);
  unsigned long long cm = 0ull;
  if (mode == BLT_UNMASK_ENTROPY) {
    const float e = masked ? ent_ws[sd.blk_row0 + j] : INFINITY;
    int rank = 0;                                   // masked positions ahead of this one
    for (int i = 0; i < 64; ++i) {
      const float ei = lane_f(e, i);
      rank += ((mm >> i) & 1ull) && (ei < e || (ei == e && i < j));
    }
    float sum = 0.f;
    const int nm = __popcll(mm);
    for (int k = 0; k < nm; ++k) {                  // uniform walk in rank order
      const int who = __ffsll((long long)__ballot(masked && rank == k)) - 1;
      sum += lane_f(e, who);
      if (k > 0 && !(sum <= alpha)) break;
      cm |= 1ull << who;
    }
  } else {
    const float c = masked ? conf_ws[sd.blk_row0 + j] : -1.f;
    cm = __ballot(masked && (mode == BLT_UNMASK_ONE_STEP || c > alpha));
    if (cm == 0ull && mm != 0ull) {
      const float best = wave_max(c);
      const unsigned long long cand = __ballot(masked && c == best);
      cm = 1ull << (__ffsll((long long)cand) - 1);
    }
  }
  if ((cm >> j) & 1ull) block_tok[sd.blk0 + j] = argmax_ws[sd.blk_row0 + j];
  const int left = __popcll(mm) - __popcll(cm);
  if (j == 0) {
    masked_left[sd.out_b] = left;
    // device-resident blocks: a pass counts for a sequence that still had a
    // [MASK]; the gate drops when its last one is committed
    if (pass_count && mm != 0ull) pass_count[sd.slot] += 1;
    if (gate && mm != 0ull && left == 0) atomicSub(gate, 1);
  }
}

template <bool GT>
__global__ __launch_bounds__(64) void k_unmask(const SeqDesc *seqs, const int32_t *argmax_ws,
                                               const float *conf_ws, const float *ent_ws,
                                               int32_t *block_tok, float alpha, int mode,
                                               int32_t *masked_left, int32_t *gate,
                                               int32_t *pass_count) {
  if (gate_closed<GT>(gate)) return;
  unmask_seq(seqs[blockIdx.x], argmax_ws, conf_ws, ent_ws, block_tok, alpha, mode, masked_left,
             gate, pass_count);
}

// Decisions and unmasking of a block pass in one launch: workgroup b takes
// sequence b, its four waves decide the sequence's rows (row0 + w, + 4, ...)
// exactly as k_decide does, then wave 0 unmasks its block.
template <bool GT>
__global__ __launch_bounds__(256) void k_decide_unmask(const float *logits, const SeqDesc *seqs,
                                                      const RowDesc *rows, int32_t *argmax_ws,
                                                      float *conf_ws, float *ent_ws,
                                                      int report_entropy, int32_t *argmax_out,
                                                      float *conf_out, float *logits_out,
                                                      int32_t *block_tok, float alpha, int mode,
                                                      int32_t *masked_left, int32_t *gate,
                                                      int32_t *pass_count) {
  if (gate_closed<GT>(gate)) return;
  const SeqDesc sd = seqs[blockIdx.x];
  const int w = threadIdx.x >> 6;
  for (int r = sd.row0 + w; r < sd.row0 + sd.nrows; r += 4)
    decide_row(r, logits, rows, argmax_ws, conf_ws, ent_ws, report_entropy, argmax_out, conf_out,
               logits_out);
  __syncthreads();                            // the rows' decisions are visible to wave 0
  if (w == 0) unmask_seq(sd, argmax_ws, conf_ws, ent_ws, block_tok, alpha, mode, masked_left, gate,
                         pass_count);
}

// Probability of byte t (this thread's) under the distribution the top-p
// sampler draws from, for the logits row zr: the nucleus of softmax(z / T),
// renormalised; 0 outside it.  All 256 threads of the workgroup take part.
// ew, red: LDS scratch (256 and 4 floats).
__device__ float nucleus_prob(const float *zr, float temperature, float top_p, float *ew,
                              float *red) {
  const int t = threadIdx.x;
  const float z = zr[t];
  const float best = block_max256(z, red);
  const float eT = expf((z - best) / temperature);
  ew[t] = eT;
  const float sT = block_sum256(eT, red);      // its barriers also publish ew
  float before = 0.f;
  for (int k = 0; k < 256; ++k) {
    const float ek = ew[k];
    before += (ek > eT || (ek == eT && k < t)) ? ek : 0.f;
  }
  const bool in = before < top_p * sT && eT > 0.f;
  const float mass = block_sum256(in ? eT : 0.f, red);
  __syncthreads();                            // ew fully read before the next use
  return in ? eT / mass : 0.f;
}

// Rejection-sampling verification of sampled drafts (speculative sampling):
// workgroup b takes sequence b, thread t byte t.  For draft byte j (in
// order) with draft distribution q (from the logits it was drawn from) and
// target p (from verify row j): kept iff u_j * q(x) < p(x); at the first
// rejection the appended byte is drawn from max(0, p - q) renormalised,
// bytes in id order; after a full acceptance it is drawn from the last
// target as the top-p sampler draws (bytes ranked by probability, ties by
// id).  u_j: draw d*64 + j, the appended byte's uniform: draw d*64 + r, of
// the stream seed + slot (SplitMix64 as in k_decide_sample), d = draws[b].
__global__ __launch_bounds__(256) void k_verify_sample(const SeqDesc *seqs, const int64_t *draws,
                                                      int r, const int32_t *draft, int ld_draft,
                                                      const float *zq, int ld_q, const float *zp,
                                                      int ld_p, SampleArgs smp,
                                                      int32_t *accept_len, int32_t *next_byte) {
  __shared__ float ew[256];
  __shared__ float red[4];
  __shared__ float px, qx;
  const int t = threadIdx.x;
  const int s = seqs[blockIdx.x].slot;
  const uint64_t stream = smp.seed + (uint64_t)s, base = (uint64_t)draws[blockIdx.x] * kMaxBlock;
  const float u_next = (float)(splitmix64_nth(stream, base + r + 1) >> 40) * (1.f / 16777216.f);
  for (int j = 0; j < r; ++j) {
    const int x = draft[(int64_t)s * ld_draft + j];
    const float q = nucleus_prob(zq + ((int64_t)s * ld_q + j) * kVocab, smp.temperature, smp.top_p, ew, red);
    const float p = nucleus_prob(zp + ((int64_t)s * ld_p + j) * kVocab, smp.temperature, smp.top_p, ew, red);
    if (t == x) {
      qx = q;
      px = p;
    }
    __syncthreads();
    const float u = (float)(splitmix64_nth(stream, base + j + 1) >> 40) * (1.f / 16777216.f);
    if (u * qx < px) {                          // kept (uniform branch)
      __syncthreads();                          // px, qx read before the next draft byte
      continue;
    }
    // residual max(0, p - q): the first byte, in id order, whose cumulative
    // residual mass exceeds u_next times the total
    const float res = fmaxf(p - q, 0.f);
    ew[t] = res;
    const float total = block_sum256(res, red);
    float cum = 0.f;
    for (int k = 0; k <= t; ++k) cum += ew[k];
    const float c = u_next * total;
    const float pick = -block_max256(cum > c ? -(float)t : -256.f, red);
    if (t == 0) {
      accept_len[s] = j;
      next_byte[s] = min((int)pick, 255);
    }
    return;
  }
  // all r kept: the free byte from the last target, ranked draw
  const float p = nucleus_prob(zp + ((int64_t)s * ld_p + r) * kVocab, smp.temperature, smp.top_p, ew, red);
  ew[t] = p;
  __syncthreads();
  float before = 0.f;
  int rank = 0;
  for (int k = 0; k < 256; ++k) {
    const float pk = ew[k];
    const bool prior = pk > p || (pk == p && k < t);
    before += prior ? pk : 0.f;
    rank += prior;
  }
  const bool cand = p > 0.f && before <= u_next;
  const float top = block_max256(cand ? (float)rank : -1.f, red);
  const float pick = block_max256(cand && (float)rank == top ? (float)t : -1.f, red);
  if (t == 0) {
    accept_len[s] = r;
    next_byte[s] = (int)pick;
  }
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

template <bool BF, int G, int NC, int RB, int PRO>
hipError_t gemv_launch(const GemmArgs &a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  constexpr int KC = 4 * NC * G;
  if (a.K != KC * Act<BF>::EPC) return hipErrorInvalidValue;
  const size_t lds = (size_t)RB * KC * 16;
  // gate form: 0 none, 1 tested at entry, 2 tested before the stores (bf16
  // passes the driver expects to have work)
  const int gt = a.gate == nullptr ? 0 : (BF && a.gate_late ? 2 : 1);
  const void *fn = gt == 2   ? (const void *)k_gemv<BF, G, NC, RB, PRO, BF ? 2 : 1>
                   : gt == 1 ? (const void *)k_gemv<BF, G, NC, RB, PRO, 1>
                             : (const void *)k_gemv<BF, G, NC, RB, PRO, 0>;
  static bool attr[3] = {false, false, false};
  if (!attr[gt]) {
    // allow dynamic LDS up to the 160 KB of a gfx950 CU, less the static part
    hipFuncAttributes fa;
    hipError_t e = hipFuncGetAttributes(&fa, fn);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                            160 * 1024 - (int)fa.sharedSizeBytes);
    if (e != hipSuccess) return e;
    attr[gt] = true;
  }
  constexpr int RPW = 64 / G;
  const dim3 grid((a.N + RPW - 1) / RPW);
  if (gt == 2)
    hipExtLaunchKernelGGL((k_gemv<BF, G, NC, RB, PRO, BF ? 2 : 1>), grid, dim3(256), lds, s, ev0, ev1, 0, a);
  else if (gt == 1)
    hipExtLaunchKernelGGL((k_gemv<BF, G, NC, RB, PRO, 1>), grid, dim3(256), lds, s, ev0, ev1, 0, a);
  else
    hipExtLaunchKernelGGL((k_gemv<BF, G, NC, RB, PRO, 0>), grid, dim3(256), lds, s, ev0, ev1, 0, a);
  return hipGetLastError();
}

// Lanes per output row: 16 for narrow matrices (more workgroups), else 8.
template <bool BF> int gemv_lanes(const GemmArgs &a) {
  constexpr int EPC = Act<BF>::EPC;
  return (!a.qkv_rope && a.N <= 2048 && a.K % (EPC * 64) == 0) ? 16 : 8;
}

template <bool BF, int G, int NC>
hipError_t gemv_rows(const GemmArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  // rows per block: 4, 8 or 16, the smallest that holds the pass (more rows
  // loop over blocks of 16); narrow-K matrices only, so the 16-row staging
  // fits the register budget
  constexpr bool wide16 = NC <= 8;
  if (a.pro == PRO_NORM) {
    if (a.R <= 4) return gemv_launch<BF, G, NC, 4, PRO_NORM>(a, s, e0, e1);
    if (a.R <= 8 || !wide16) return gemv_launch<BF, G, NC, 8, PRO_NORM>(a, s, e0, e1);
    return gemv_launch<BF, G, NC, wide16 ? 16 : 8, PRO_NORM>(a, s, e0, e1);
  }
  if (a.R <= 4) return gemv_launch<BF, G, NC, 4, PRO_PLAIN>(a, s, e0, e1);
  if (a.R <= 8 || !wide16) return gemv_launch<BF, G, NC, 8, PRO_PLAIN>(a, s, e0, e1);
  return gemv_launch<BF, G, NC, wide16 ? 16 : 8, PRO_PLAIN>(a, s, e0, e1);
}

template <bool BF>
hipError_t gemv_dispatch(const GemmArgs &a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  constexpr int EPC = Act<BF>::EPC;
  const int G = gemv_lanes<BF>(a), NC = a.K / (EPC * G * 4);
#define BLT_GEMV_CASE(g, nc) \
  if (G == g && NC == nc) return gemv_rows<BF, g, nc>(a, s, e0, e1);
  BLT_GEMV_CASE(8, 1) BLT_GEMV_CASE(8, 2) BLT_GEMV_CASE(8, 3) BLT_GEMV_CASE(8, 4)
  BLT_GEMV_CASE(8, 6) BLT_GEMV_CASE(8, 8) BLT_GEMV_CASE(8, 12) BLT_GEMV_CASE(8, 16)
  BLT_GEMV_CASE(16, 1) BLT_GEMV_CASE(16, 2) BLT_GEMV_CASE(16, 3) BLT_GEMV_CASE(16, 4)
  BLT_GEMV_CASE(16, 6) BLT_GEMV_CASE(16, 8) BLT_GEMV_CASE(16, 12)
#undef BLT_GEMV_CASE
  return hipErrorInvalidValue;
}

}  // namespace

bool gemv_supported(bool bf16, int K) {
  // chunk counts instantiated by gemv_dispatch for 8 lanes per row
  const int epc = bf16 ? 8 : 4;
  if (K % (32 * epc)) return false;
  const int nc = K / (32 * epc);
  return nc == 1 || nc == 2 || nc == 3 || nc == 4 || nc == 6 || nc == 8 || nc == 12 || nc == 16 ||
         nc == 24;  // 24: only as a 16-lane matrix (12 chunks per lane)
}

// K splits of a residual product on the MFMA path: the fewest that give at
// least 512 workgroups (about two per CU) with every split a multiple of four
// K steps, within the partials' workspace.
static int resid_splits(const GemmArgs &a, int tiles, size_t cap) {
  int best = 1;
  for (int sp = 2; sp <= 8; ++sp) {
    if (tiles * best >= 512) break;
    if (a.K % (sp * 4 * kGemmBK)) continue;
    if ((size_t)sp * a.R * a.N > cap) break;
    best = sp;
  }
  return best;
}

// Which kernel launch_gemm runs for these arguments (the choice depends on
// the matrix and, for the MFMA GEMM, on the row count only).
GemmKind gemm_kind(bool bf16, const GemmArgs &a) {
  if (!bf16 || a.R < kGemvRows)
    return (bf16 && a.K <= 1536 && a.K % 128 == 0 && a.N >= 2048) ? GEMM_KIND_GEMV_MFMA : GEMM_KIND_GEMV;
  return GEMM_KIND_MFMA;
}

// K splits of a product on the weight-streaming GEMM (64x64 tiles, four K
// steps of weights in flight): a residual product takes the fewest that give
// at least 400 workgroups, within the partials' workspace; 0 where the kernel
// does not apply (no fragment-ordered weights, over 1024 rows unless forced,
// K splits not in whole groups of four steps).
static int bs_splits(const GemmArgs &a, bool may_split, size_t cap, bool forced) {
  if (!a.Wf || (a.R > 1024 && !forced) || a.K % (4 * kGemmBK)) return 0;
  const int tiles = ((a.R + 63) / 64) * ((a.N + 63) / 64);
  int best = 1;
  for (int sp = 2; sp <= (may_split ? 8 : 1) && tiles * best < 400; ++sp) {
    if (a.K % (sp * 4 * kGemmBK)) continue;
    if ((size_t)sp * a.R * a.N > cap) break;
    best = sp;
  }
  return best;
}

hipError_t launch_gemm(bool bf16, const GemmArgs &a, void *xnorm_ws, SplitResid *sr,
                       hipStream_t s, hipEvent_t ev0, hipEvent_t ev1, int form) {
  if (a.R <= 0) return hipSuccess;
  const bool pending = sr && sr->splits > 0;
  // a pending sum is taken only by the RMSNorm prologue over its residual,
  // and nothing may write that residual first
  if (pending && ((a.pro == PRO_NORM && (a.H != sr->a.resid || a.R != sr->a.R || a.K != sr->a.N)) ||
                  (a.ep == EP_RESID && a.resid == sr->a.resid)))
    return hipErrorInvalidValue;
  if (!bf16 || a.R < kGemvRows) {
    if (pending) return hipErrorInvalidValue;
    // bfloat16: the MFMA GEMV for K <= 1536 and N >= 2048 (QKV, W1, the
    // cross-vector product).  With longer rows or fewer columns its
    // workgroups of 16 columns are too few for the weight stream and the
    // dot-product GEMV is faster (measured: K = 2048 and 4096; W_o and the
    // head in decode passes).  The choice depends on the matrix only, never
    // on the row count.
    if (bf16 && a.K <= 1536 && a.K % 128 == 0 && a.N >= 2048) {
      const int steps = a.K / 128;
      const dim3 g((a.N + 15) / 16);
#define BLT_GEMV_MFMA_GT(SB, GT)                                                                 \
  if (a.pro == PRO_NORM)                                                                         \
    hipExtLaunchKernelGGL((k_gemv_mfma<PRO_NORM, SB, GT>), g, dim3(256), 0, s, ev0, ev1, 0, a);  \
  else hipExtLaunchKernelGGL((k_gemv_mfma<PRO_PLAIN, SB, GT>), g, dim3(256), 0, s, ev0, ev1, 0, a);
#define BLT_GEMV_MFMA(SB)                                                                        \
  if (a.gate && a.gate_late) { BLT_GEMV_MFMA_GT(SB, 2) }                                       \
  else if (a.gate) { BLT_GEMV_MFMA_GT(SB, 1) } else { BLT_GEMV_MFMA_GT(SB, 0) }
      if (steps % 8 == 0) { BLT_GEMV_MFMA(8) }
      else if (steps % 4 == 0) { BLT_GEMV_MFMA(4) }
      else if (steps % 2 == 0) { BLT_GEMV_MFMA(2) }
      else { BLT_GEMV_MFMA(1) }
#undef BLT_GEMV_MFMA
#undef BLT_GEMV_MFMA_GT
      return hipGetLastError();
    }
    return bf16 ? gemv_dispatch<true>(a, s, ev0, ev1) : gemv_dispatch<false>(a, s, ev0, ev1);
  }
  GemmArgs b = a;
  if (a.pro == PRO_NORM) {
    float *H = const_cast<float *>(a.H);
    const GemmArgs &pa = pending ? sr->a : a;
#define BLT_NORM(SP)                                                                             \
  if (pa.gate)                                                                                   \
    hipLaunchKernelGGL((k_rmsnorm_act<true, SP, true>), dim3(a.R), dim3(256), 0, s, H, a.ldh,    \
                       a.gain, a.K, a.eps, xnorm_ws, pa);                                        \
  else                                                                                           \
    hipLaunchKernelGGL((k_rmsnorm_act<true, SP, false>), dim3(a.R), dim3(256), 0, s, H, a.ldh,   \
                       a.gain, a.K, a.eps, xnorm_ws, pa);
    switch (pending ? sr->splits : 0) {
      case 0: BLT_NORM(0) break;
      case 2: BLT_NORM(2) break;
      case 3: BLT_NORM(3) break;
      case 4: BLT_NORM(4) break;
      case 5: BLT_NORM(5) break;
      case 6: BLT_NORM(6) break;
      case 7: BLT_NORM(7) break;
      case 8: BLT_NORM(8) break;
      default: return hipErrorInvalidValue;
    }
#undef BLT_NORM
    if (pending) sr->splits = 0;
    b.pro = PRO_PLAIN;
    b.X = xnorm_ws;
    b.ldx = a.K;
    b.x_row_off = nullptr;
  }
  const int t64 = ((a.R + 63) / 64) * ((a.N + 63) / 64);
  // A residual product with too few tiles to fill the chip splits K; its
  // sum is left to the RMSNorm prologue that follows it
  const bool may_split = sr && sr->ws && a.ep == EP_RESID;
  int splits = may_split ? resid_splits(a, t64, sr->cap) : 1;
  const int t128 = ((a.R + 127) / 128) * ((a.N + 127) / 128);
  const int t64w = ((a.R + 63) / 64) * ((a.N + 127) / 128);
  // Where the staged-tile kernel would take 128x128 tiles but get fewer
  // than 200 workgroups (decode passes of 512-1024 rows), the weight-
  // streaming kernel's 64x64 tiles run about 3.5x as many and finish
  // sooner (576 rows: QKV 36.0 -> 29.3 us, W_o and W2 25.2 -> 17.7 us;
  // W1, with 240 such tiles, stays: 26.1 us against 32.3).  form 2 forces
  // it wherever it applies, form 1 never takes it.
  const bool big = t128 * splits >= 176;
  const int bsp = form == 1 ? 0 : bs_splits(a, may_split, may_split ? sr->cap : 0, form == 2);
  if (bsp > 0 && (form == 2 || (big && t128 * splits < 200))) {
    if (bsp > 1) {
      b.ep = EP_PART;
      b.out_f32 = sr->ws;
      sr->a = b;
      sr->splits = bsp;
    }
    const dim3 g(((a.R + 63) / 64) * ((a.N + 63) / 64), bsp);
    if (b.gate) hipExtLaunchKernelGGL((k_gemm_bs<4, 1, 4, 2, true>), g, dim3(256), 0, s, ev0, ev1, 0, b);
    else hipExtLaunchKernelGGL((k_gemm_bs<4, 1, 4, 2, false>), g, dim3(256), 0, s, ev0, ev1, 0, b);
    return hipGetLastError();
  }
  if (b.K % (splits * 2 * kGemmBK)) return hipErrorInvalidValue;  // K steps in pairs per split
  if (splits > 1) {
    b.ep = EP_PART;
    b.out_f32 = sr->ws;
    sr->a = b;                               // the norm reads the partials at b.out_f32
    sr->splits = splits;
  }
  // the largest tile that still gives about 150-180 workgroups (measured at
  // the batch-16, batch-64 and prefill shapes)
#define BLT_GEMM(BM, BN, WM, WN, KH, T)                                                           \
  if (b.gate)                                                                                     \
    hipExtLaunchKernelGGL((k_gemm_mfma<BM, BN, WM, WN, KH, true>), dim3(T, splits), dim3(512), 0, \
                          s, ev0, ev1, 0, b);                                                     \
  else                                                                                            \
    hipExtLaunchKernelGGL((k_gemm_mfma<BM, BN, WM, WN, KH, false>), dim3(T, splits), dim3(512), 0, \
                          s, ev0, ev1, 0, b);
  if (t128 * splits >= 176) { BLT_GEMM(128, 128, 2, 4, 1, t128) }
  else if (t64w * splits >= 150) { BLT_GEMM(64, 128, 2, 4, 1, t64w) }
  else { BLT_GEMM(64, 64, 2, 2, 2, t64) }
#undef BLT_GEMM
  return hipGetLastError();
}

hipError_t launch_embed(bool bf16, const void *embed, const float *cross, const RowDesc *rows,
                        int R, int d, int n_layers, int max_lat, const int32_t *block_tok,
                        const int32_t *tokens_dev, float *h, hipStream_t s, const int32_t *gate) {
#define BLT_EMBED(BF, GT)                                                                        \
  hipLaunchKernelGGL((k_embed<BF, GT>), dim3(R), dim3(256), 0, s, embed, cross, rows, d, n_layers, \
                     max_lat, block_tok, tokens_dev, h, gate);
  if (bf16) {
    if (gate) { BLT_EMBED(true, true) } else { BLT_EMBED(true, false) }
  } else {
    if (gate) { BLT_EMBED(false, true) } else { BLT_EMBED(false, false) }
  }
#undef BLT_EMBED
  return hipGetLastError();
}

hipError_t launch_rope_kv(bool bf16, const float *qkv, int R, const RowDesc *rows,
                          const float2 *rope_tab, float *q_out, void *kv, KVGeom g, int layer,
                          hipStream_t s, const int32_t *gate) {
#define BLT_ROPE(BF, GT)                                                                         \
  hipLaunchKernelGGL((k_rope_kv<BF, GT>), dim3(R), dim3(256), 0, s, qkv, rows, rope_tab, q_out, kv, \
                     g, layer, gate);
  if (bf16) {
    if (gate) { BLT_ROPE(true, true) } else { BLT_ROPE(true, false) }
  } else {
    if (gate) { BLT_ROPE(false, true) } else { BLT_ROPE(false, false) }
  }
#undef BLT_ROPE
  return hipGetLastError();
}

template <bool BF, int DH>
static void attn_launch(const float *q, const void *kv, KVGeom g, int layer, const SeqDesc *seqs,
                        int n_seq, const SeqDesc *sd_host, int grid_chunks, int nsub, int wg,
                        int max_chunks, int flash_tiles,
                        const RowDesc *rows, int R, float *part, void *a_out, hipEvent_t ev0,
                        hipEvent_t ev1, bool ev_flash, hipStream_t s, const int32_t *gate,
                        int flash_kg, int gate_late) {
  if constexpr (BF) {
    if (flash_tiles > 0) {
      const dim3 fg((flash_tiles + 1) / 2, g.n_heads, n_seq);   // pairs of row tiles
      // up to 2048 workgroups: eight waves in two key groups (two waves per
      // SIMD with one workgroup per CU); measured 8-25% faster from 128 to
      // 1024 workgroups, equal at 512-3072, 6% slower at 49152 (64 prompts
      // of 8192 rows).  The choice depends on the grid only (flash_kg > 0
      // forces a form).
      const bool two = flash_kg ? flash_kg == 2 : (int64_t)fg.x * fg.y * fg.z <= 2048;
      hipEvent_t e0 = ev_flash ? ev0 : nullptr, e1 = ev_flash ? ev1 : nullptr;
#define BLT_FLASH(KG, GT)                                                                         \
  hipExtLaunchKernelGGL((k_attn_flash<DH, KG, GT>), fg, dim3(256 * KG), 0, s, e0, e1, 0, q, kv, g, \
                        layer, seqs, rows, a_out, gate);
      if (two) {
        if (gate) { BLT_FLASH(2, true) } else { BLT_FLASH(2, false) }
      } else {
        if (gate) { BLT_FLASH(1, true) } else { BLT_FLASH(1, false) }
      }
#undef BLT_FLASH
    }
  }
  if (ev_flash) ev0 = ev1 = nullptr;
  if (grid_chunks <= 0) return;
  if (!BF || DH > 64 || nsub < 1) nsub = 1;
  if (!BF || DH > 64) wg = 1;
  if (wg == 2) nsub = grid_chunks;
  const int gc = (grid_chunks + nsub - 1) / nsub;   // workgroups (partials) per (sequence, head)
  const dim3 grid(gc, g.n_heads, n_seq);
  // one workgroup per (sequence, head): the output is written directly
  const int direct = gc == 1;
  const SeqDesc sd_arg = sd_host && n_seq == 1 ? *sd_host : SeqDesc{};
  const int use_sd_arg = sd_host && n_seq == 1;
  // with events: stamped by the dispatch itself at the kernel's start and end
  if constexpr (BF) {
#define BLT_SPLITK_GT(PIPE, WG, GT)                                                               \
  if (ev0)                                                                                        \
    hipExtLaunchKernelGGL((k_attn_mfma<DH, PIPE, WG, GT>), grid, dim3(256 * WG), 0, s, ev0, ev1, \
                          0, q, kv, g, layer, seqs, rows, part, max_chunks, nsub, direct, a_out,  \
                          sd_arg, use_sd_arg, gate);                                              \
  else                                                                                            \
    hipLaunchKernelGGL((k_attn_mfma<DH, PIPE, WG, GT>), grid, dim3(256 * WG), 0, s, q, kv, g,     \
                       layer, seqs, rows, part, max_chunks, nsub, direct, a_out, sd_arg,          \
                       use_sd_arg, gate);
#define BLT_SPLITK(PIPE, WG)                                                                      \
  if (gate && gate_late) { BLT_SPLITK_GT(PIPE, WG, 2) }                                            \
  else if (gate) { BLT_SPLITK_GT(PIPE, WG, 1) } else { BLT_SPLITK_GT(PIPE, WG, 0) }
    if constexpr (DH <= 64) {
      if (wg == 2) { BLT_SPLITK(true, 2) }
      else if (nsub > 1) { BLT_SPLITK(true, 1) }
      else { BLT_SPLITK(false, 1) }
    } else {
      BLT_SPLITK(false, 1)
    }
#undef BLT_SPLITK
#undef BLT_SPLITK_GT
  } else {
#define BLT_F32(GT)                                                                               \
  if (ev0)                                                                                        \
    hipExtLaunchKernelGGL((k_attn_f32<DH, GT>), grid, dim3(256), 0, s, ev0, ev1, 0, q, kv, g,     \
                          layer, seqs, rows, part, max_chunks, gate);                             \
  else                                                                                            \
    hipLaunchKernelGGL((k_attn_f32<DH, GT>), grid, dim3(256), 0, s, q, kv, g, layer, seqs, rows,  \
                       part, max_chunks, gate);
    if (gate) { BLT_F32(true) } else { BLT_F32(false) }
#undef BLT_F32
  }
  if (BF && direct) return;                 // no partials to merge
  // the merge takes its first 16 (or 64) chunks in one round of loads
#define BLT_MERGE(PRE, GT)                                                                        \
  hipLaunchKernelGGL((k_attn_merge<BF, DH, PRE, GT>), dim3(R, g.n_heads), dim3(64), 0, s, part,  \
                     rows, g.n_heads, max_chunks, gc, kCK * nsub, a_out, gate);
  constexpr int PRE_WIDE = DH > 64 ? 32 : 64;
  if (gc <= 16) {
    if (gate) { BLT_MERGE(16, true) } else { BLT_MERGE(16, false) }
  } else {
    if (gate) { BLT_MERGE(PRE_WIDE, true) } else { BLT_MERGE(PRE_WIDE, false) }
  }
#undef BLT_MERGE
}

hipError_t launch_attention(bool bf16, const float *q, const void *kv, KVGeom g, int layer,
                            const SeqDesc *seqs, int n_seq, const SeqDesc *sd_host,
                            int grid_chunks, int nsub, int wg, int max_chunks, int flash_tiles, const RowDesc *rows, int R,
                            float *part, void *a_out, hipEvent_t ev0, hipEvent_t ev1, bool ev_flash,
                            hipStream_t s, const int32_t *gate, int flash_kg, int gate_late) {
  if (flash_tiles > 0 && !bf16) return hipErrorInvalidValue;   // the causal kernel is bf16 only
#define BLT_ATTN(dh)                                                                              \
  if (bf16) attn_launch<true, dh>(q, kv, g, layer, seqs, n_seq, sd_host, grid_chunks, nsub, wg,   \
                                  max_chunks, flash_tiles, rows, R, part, a_out, ev0, ev1,        \
                                  ev_flash, s, gate, flash_kg, gate_late);                        \
  else attn_launch<false, dh>(q, kv, g, layer, seqs, n_seq, sd_host, grid_chunks, nsub, wg,       \
                              max_chunks, flash_tiles, rows, R, part, a_out, ev0, ev1, ev_flash, s, \
                              gate, flash_kg, gate_late);
  switch (g.d_head) {
    case 32: BLT_ATTN(32) break;
    case 64: BLT_ATTN(64) break;
    case 128: BLT_ATTN(128) break;
    default: return hipErrorInvalidValue;
  }
#undef BLT_ATTN
  return hipGetLastError();
}

hipError_t launch_decide(const float *logits, int R, const RowDesc *rows, int32_t *argmax_ws,
                         float *conf_ws, float *ent_ws, int report_entropy, int32_t *argmax_out,
                         float *conf_out, float *logits_out, const SampleArgs *smp, hipStream_t s,
                         const int32_t *gate) {
#define BLT_DECIDE_SAMPLE(GT)                                                                     \
  hipLaunchKernelGGL(k_decide_sample<GT>, dim3(R), dim3(256), 0, s, logits, rows, argmax_ws,      \
                     conf_ws, ent_ws, report_entropy, argmax_out, conf_out, logits_out, *smp, gate);
#define BLT_DECIDE(GT)                                                                            \
  hipLaunchKernelGGL(k_decide<GT>, dim3(R), dim3(64), 0, s, logits, rows, argmax_ws, conf_ws,     \
                     ent_ws, report_entropy, argmax_out, conf_out, logits_out, gate);
  if (smp) {
    if (gate) { BLT_DECIDE_SAMPLE(true) } else { BLT_DECIDE_SAMPLE(false) }
  } else {
    if (gate) { BLT_DECIDE(true) } else { BLT_DECIDE(false) }
  }
#undef BLT_DECIDE_SAMPLE
#undef BLT_DECIDE
  return hipGetLastError();
}

hipError_t launch_decide_unmask(const float *logits, int n_seq, const SeqDesc *seqs,
                                const RowDesc *rows, int32_t *argmax_ws, float *conf_ws,
                                float *ent_ws, int report_entropy, int32_t *argmax_out,
                                float *conf_out, float *logits_out, int32_t *block_tok,
                                float alpha, int mode, int32_t *masked_left, hipStream_t s,
                                int32_t *gate, int32_t *pass_count) {
#define BLT_DECIDE_UNMASK(GT)                                                                     \
  hipLaunchKernelGGL(k_decide_unmask<GT>, dim3(n_seq), dim3(256), 0, s, logits, seqs, rows,       \
                     argmax_ws, conf_ws, ent_ws, report_entropy, argmax_out, conf_out, logits_out, \
                     block_tok, alpha, mode, masked_left, gate, pass_count);
  if (gate) { BLT_DECIDE_UNMASK(true) } else { BLT_DECIDE_UNMASK(false) }
#undef BLT_DECIDE_UNMASK
  return hipGetLastError();
}

hipError_t launch_verify_sample(int batch, const SeqDesc *seqs, const int64_t *draws, int r,
                                const int32_t *draft, int ld_draft, const float *zq, int ld_q,
                                const float *zp, int ld_p, const SampleArgs &smp,
                                int32_t *accept_len, int32_t *next_byte, hipStream_t s) {
  hipLaunchKernelGGL(k_verify_sample, dim3(batch), dim3(256), 0, s, seqs, draws, r, draft, ld_draft,
                     zq, ld_q, zp, ld_p, smp, accept_len, next_byte);
  return hipGetLastError();
}

hipError_t launch_transpose(bool bf16, const void *src, void *dst, int n, hipStream_t s) {
  const int blocks = (int)std::min<int64_t>(((int64_t)n * n + 255) / 256, 4096);
  if (bf16)
    hipLaunchKernelGGL(k_transpose<uint16_t>, dim3(blocks), dim3(256), 0, s, (const uint16_t *)src,
                       (uint16_t *)dst, n);
  else
    hipLaunchKernelGGL(k_transpose<float>, dim3(blocks), dim3(256), 0, s, (const float *)src,
                       (float *)dst, n);
  return hipGetLastError();
}

// Fragment order of a bf16 matrix W[N][K] for the weight-streaming GEMM:
// piece p = (ct * K/32 + kb) * 64 + l holds W[16 ct + l % 16][32 kb + 8 (l / 16) + e],
// e = 0..7 (zeros past row N), so the B operand of one 16-column, 32-deep
// MFMA block is 1 KB of consecutive memory, lane l's 16 bytes at 16 l.
__global__ void k_frag_pack(const uint16_t *src, int N, int K, uint16_t *dst, int64_t pieces) {
  const int KB = K / 32;
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < pieces;
       p += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(p & 63);
    const int64_t rest = p >> 6;
    const int kb = (int)(rest % KB), ct = (int)(rest / KB);
    const int n = 16 * ct + (l & 15), k = 32 * kb + 8 * (l >> 4);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (n < N) v = *(const uint4 *)(src + (int64_t)n * K + k);
    *(uint4 *)(dst + p * 8) = v;
  }
}

size_t frag_elems(int N, int K) { return (size_t)((N + 15) / 16) * 16 * K; }

hipError_t launch_frag_pack(const void *src, int N, int K, void *dst, hipStream_t s) {
  if (K % 32) return hipErrorInvalidValue;
  const int64_t pieces = (int64_t)((N + 15) / 16) * (K / 32) * 64;
  const int blocks = (int)std::min<int64_t>((pieces + 255) / 256, 8192);
  hipLaunchKernelGGL(k_frag_pack, dim3(blocks), dim3(256), 0, s, (const uint16_t *)src, N, K,
                     (uint16_t *)dst, pieces);
  return hipGetLastError();
}

hipError_t launch_unmask(const SeqDesc *seqs, int n_seq, const int32_t *argmax_ws,
                         const float *conf_ws, const float *ent_ws, int32_t *block_tok, float alpha,
                         int mode, int32_t *masked_left, hipStream_t s, int32_t *gate,
                         int32_t *pass_count) {
#define BLT_UNMASK(GT)                                                                            \
  hipLaunchKernelGGL(k_unmask<GT>, dim3(n_seq), dim3(64), 0, s, seqs, argmax_ws, conf_ws, ent_ws, \
                     block_tok, alpha, mode, masked_left, gate, pass_count);
  if (gate) { BLT_UNMASK(true) } else { BLT_UNMASK(false) }
#undef BLT_UNMASK
  return hipGetLastError();
}

hipError_t launch_verify(int batch, const SeqDesc *seqs, int r, const int32_t *draft,
                         int ld_draft, const int32_t *pred, int ld_pred, int32_t *accept_len,
                         int32_t *next_byte, hipStream_t s) {
  hipLaunchKernelGGL(k_verify, dim3((batch + 63) / 64), dim3(64), 0, s, batch, seqs, r, draft,
                     ld_draft, pred, ld_pred, accept_len, next_byte);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Draft distributions of sampled BLT-DV blocks: after each pass, a position
// committed by it (masked before, a byte after) keeps the logits of that
// pass, the distribution its byte was drawn from.  Block (slot, j) per
// workgroup; logits and kept rows both at (slot * B + j) * 257.
__global__ __launch_bounds__(64) void k_keep_drawn(const int32_t *before, const int32_t *after,
                                                   const float *logits, float *kept, int B) {
  const int i = blockIdx.x;                  // slot * B + j
  if (before[i] != kMask || after[i] == kMask) return;
  for (int v = threadIdx.x; v < kVocab; v += 64) kept[(int64_t)i * kVocab + v] = logits[(int64_t)i * kVocab + v];
}

hipError_t launch_keep_drawn(const int32_t *before, const int32_t *after, const float *logits,
                             float *kept, int n_slots, int B, hipStream_t s) {
  if (n_slots * B <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_keep_drawn, dim3(n_slots * B), dim3(64), 0, s, before, after, logits, kept, B);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Device-resident BLT-D blocks (pytorch.kr summary, "BLT-D inference": per
// block one encoder/global pass, then decoder passes until the block is
// filled; "BLT-D attention mask" for the latent each row reads).  One thread
// per sequence; sequence b sits in state slot b.

// Plan of a block: its encoder/global pass (latents lat_ready .. M of the
// last, possibly truncated, patch M; the remaining of the B+1 requests repeat
// M, which recomputes the same values), the first pass's rows (the last B+1
// committed bytes as clean rows with their causal latents -- the newest byte
// reads o_M as the last byte of the truncated patch, the one before it is
// recomputed with its now final latent -- and the B [MASK] rows reading o_M)
// and the later passes' rows (the block rows alone).
__global__ void k_block_plan(DevBlockArgs a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b == 0) *a.gate = a.S;                 // every sequence starts with B masks
  if (b >= a.S) return;
  DevSeq &q = a.st[b];
  const int B = a.B, n = q.n, M = q.patch_last;
  const int r0 = b * (2 * B + 1);
  const int32_t *xs = a.x + (int64_t)b * a.x_stride;
  for (int j = 0; j <= B; ++j) {
    const int i = n - B - 1 + j;
    const int tgt = j == B ? M : (q.win_ends[j] ? q.win_patch[j] : q.win_patch[j] - 1);
    // the oldest of them read its patch's latent as the last prefix byte of
    // the previous block: unchanged when a boundary follows it, and then its
    // cached keys and values stay (as a host-driven block leaves them)
    a.rows0[r0 + j] = RowDesc{b, i, xs[i], 0, tgt, i + 1, -1, 0, -1, j == 0 && q.win_ends[0] ? 1 : 0};
  }
  for (int j = 0; j < B; ++j) {
    const int pos = n + j;
    const RowDesc rd{b, pos, kTokFromBlock, b * B + j, M, a.causal ? pos + 1 : n + B, b * B + j, 0, -1, 0};
    a.rows0[r0 + B + 1 + j] = rd;
    a.rows1[b * B + j] = rd;
    a.block_tok[b * B + j] = kMask;
  }
  a.seqs0[b] = SeqDesc{b, r0, 2 * B + 1, n + B, b * B, r0 + B + 1, B, b, 0};
  a.seqs1[b] = SeqDesc{b, b * B, B, n + B, b * B, b * B, B, b, 0};
  a.masked_left[b] = B;
  const int m0 = q.lat_ready;
  if (M - m0 + 1 > B + 1) q.err = 2;
  for (int e = 0; e <= B; ++e) {
    int idx = min(m0 + e, M);
    if (idx < 0 || idx >= a.n_lat || idx >= a.max_latents) {
      q.err = 1;
      idx = 0;
    }
    a.lat_offs[b * (B + 1) + e] = ((int64_t)b * a.seq_stride + idx) * a.d_global;
    a.lat_offs[(int64_t)a.S * (B + 1) + b * (B + 1) + e] =
        ((int64_t)b * a.max_latents + idx) * a.n_layers * a.d_model;
  }
  q.lat_ready = max(m0, M + 1);
  a.n_eg[b] += 1;
}

// Commit of a filled block: its bytes join the sequence and the stand-in
// patcher decides, byte by byte, where patches end (a new patch starts after
// byte x_i iff the current one holds 8 bytes or the (1 + 256 x_{i-1} +
// x_i)-th SplitMix64 output from the sequence's salt is 0 modulo 4).
__global__ void k_block_commit(DevBlockArgs a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.S) return;
  DevSeq &q = a.st[b];
  const int B = a.B;
  int32_t *xs = a.x + (int64_t)b * a.x_stride;
  q.win_patch[0] = q.patch_last;
  q.win_ends[0] = q.ends_last;
  for (int j = 0; j < B; ++j) {
    int byte = a.block_tok[b * B + j];
    if (byte < 0 || byte > 255) {
      q.err = 3;
      byte = 0;
    }
    const int prev = xs[q.n - 1 + j];
    const bool fresh = q.ends_last != 0;
    const int p = q.patch_last + (fresh ? 1 : 0);
    q.cur_len = fresh ? 1 : q.cur_len + 1;
    const bool e = q.cur_len >= 8 || (splitmix64_nth(q.salt, 1 + 256ull * prev + byte) & 3ull) == 0;
    xs[q.n + j] = byte;
    q.patch_last = p;
    q.ends_last = e;
    q.win_patch[j + 1] = p;
    q.win_ends[j + 1] = e;
  }
  q.n += B;
}

hipError_t launch_block_plan(const DevBlockArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_block_plan, dim3((a.S + 63) / 64), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_block_commit(const DevBlockArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_block_commit, dim3((a.S + 63) / 64), dim3(64), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point (blt_kv_append_noalloc): one
// static device array per GPU.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in symbol); it asks for the device
// address, which differs per GPU, once per device with that device current.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_region(void **ptr) {
  static std::mutex mu;
  static void *addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace blt
