"""Python binding of libblt (the MI355X Fast-BLT local byte decoder step).

Argument marshalling only: every function here has the name of the C entry
point it calls, turns torch tensors into device pointers and Python
sequences into host arrays, and raises ``BltError`` on a non-zero status.
All computation happens in the HIP library; there is no fallback.  PyTorch
provides device memory and the stream.

``Decoder`` is a small holder that keeps the weight and state tensors alive
next to the context that points at them.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# BLT_LIB=debug loads the bounds-checking build (libblt_debug.so), BLT_LIB=asan
# the host-sanitized one (libblt_asan.so; the process must preload the
# sanitizer runtime); unset: the release build.
_VARIANT = os.environ.get("BLT_LIB", "")
if _VARIANT not in ("", "release", "debug", "asan"):
    raise ImportError(f"BLT_LIB={_VARIANT!r}: expected release, debug or asan")
LIB_PATH = os.path.join(_HERE, "libblt.so" if _VARIANT in ("", "release") else f"libblt_{_VARIANT}.so")

BLT_OK, BLT_EINVAL, BLT_ECAPACITY, BLT_EDTYPE, BLT_EHIP, BLT_ENOTIMPL = 0, -1, -2, -3, -4, -5
BLT_F32, BLT_BF16 = 0, 1
BLT_UNMASK_THRESHOLD, BLT_UNMASK_ONE_STEP, BLT_UNMASK_ENTROPY = 0, 1, 2
BLT_BLOCK_BIDIR, BLT_BLOCK_CAUSAL = 0, 1
BLT_POLICY_GREEDY, BLT_POLICY_BLT_D, BLT_POLICY_BLT_S, BLT_POLICY_BLT_DV = 0, 1, 2, 3
BLT_PROF_OFF, BLT_PROF_ATTENTION, BLT_PROF_ATTENTION_CAUSAL = 0, 1, 2
BLT_PROF_GEMV_MFMA, BLT_PROF_GEMV, BLT_PROF_GEMM = 3, 4, 5
MASK = 256
VOCAB = 257

EXPORTS = [
    "blt_state_size", "blt_create", "blt_destroy", "blt_last_error", "blt_latents_put",
    "blt_kv_append", "blt_decode_block_step", "blt_verify_accept", "blt_verify_sample", "blt_bw_model",
    "blt_session_create", "blt_session_prefill", "blt_session_generate", "blt_session_result",
    "blt_session_destroy", "blt_profile_enable", "blt_profile_read", "blt_graphs_enable",
    "blt_attention_chunks", "blt_kv_append_noalloc", "blt_session_device_blocks",
    "blt_flash_key_groups", "blt_gemm_form",
]


class BltError(RuntimeError):
    def __init__(self, fn, status, msg=""):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class blt_config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("d_ffn", C.c_int32), ("vocab", C.c_int32), ("d_global", C.c_int32),
                ("max_batch", C.c_int32), ("max_ctx", C.c_int32), ("max_latents", C.c_int32),
                ("max_rows", C.c_int32), ("max_block", C.c_int32), ("dtype", C.c_int32),
                ("rope_theta", C.c_float), ("rms_eps", C.c_float)]


class blt_layer_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in
                ("wv_c", "wo_c", "wqkv", "wo", "g_attn", "g_ffn", "w1", "w2")]


class blt_weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("w_lat", C.c_void_p), ("w_out", C.c_void_p),
                ("g_out", C.c_void_p), ("layers", C.POINTER(blt_layer_weights))]


class blt_state(C.Structure):
    _fields_ = [("kv", C.c_void_p), ("cross", C.c_void_p)]


class blt_counts(C.Structure):
    _fields_ = [("n_dec", C.c_uint64), ("n_encglob", C.c_uint64), ("n_seq", C.c_uint64)]


class blt_params(C.Structure):
    _fields_ = [("p_dec", C.c_uint64), ("p_enc", C.c_uint64), ("p_glob", C.c_uint64),
                ("bytes_per_param", C.c_uint32)]


class blt_policy_args(C.Structure):
    _fields_ = [("policy", C.c_int32), ("block", C.c_int32), ("alpha", C.c_float),
                ("unmask", C.c_int32), ("block_mask", C.c_int32), ("n_gen", C.c_int32),
                ("temperature", C.c_float), ("top_p", C.c_float), ("seed", C.c_uint64)]


class blt_sampling(C.Structure):
    _fields_ = [("temperature", C.c_float), ("top_p", C.c_float), ("seed", C.c_uint64)]


_lib = None


def lib():
    """Load libblt.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m block_diffusion_byte_amd.build"
                              f"{' --variant ' + _VARIANT if _VARIANT not in ('', 'release') else ''}`")
        L = C.CDLL(LIB_PATH)
        P, I32, I64, F = C.c_void_p, C.c_int32, C.c_int64, C.c_float
        sig = {
            "blt_state_size": [P, P, P],
            "blt_create": [P, P, P, P],
            "blt_destroy": [P],
            "blt_latents_put": [P, P, I32, P, P, P, I64],
            "blt_kv_append": [P, P, I32, P, P, P, I32, P, P, P, P, P, P, P, P],
            "blt_kv_append_noalloc": [P, P, I32, P, P, P, I32, P, P, P, P, P, P, P, P],
            "blt_decode_block_step": [P, P, I32, P, P, P, I32, P, P, P, I32, P, F, I32, I32,
                                      P, P, P, P, P, P],
            "blt_verify_accept": [P, I32, P, I32, P, I32, P, I32, P, P],
            "blt_verify_sample": [P, I32, P, I32, P, I32, P, I32, P, I32, P, P, P, P],
            "blt_bw_model": [P, P, P, P],
            "blt_session_create": [P, P, I32, P, P, P, P, P, P, I32, P],
            "blt_session_prefill": [P],
            "blt_session_generate": [P, P],
            "blt_session_result": [P, I32, P, I32, P, P, P, P, P],
            "blt_session_destroy": [P],
            "blt_session_device_blocks": [P, I32],
            "blt_profile_enable": [P, I32],
            "blt_profile_read": [P, P, P, P, I32],
            "blt_graphs_enable": [P, I32],
            "blt_attention_chunks": [P, I32],
            "blt_flash_key_groups": [P, I32],
            "blt_gemm_form": [P, I32],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = C.c_int
        L.blt_last_error.argtypes = [P]
        L.blt_last_error.restype = C.c_char_p
        _lib = L
    return _lib


def _check(fn, st, ctx=None):
    if st != BLT_OK:
        msg = lib().blt_last_error(ctx).decode() if ctx else ""
        raise BltError(fn, st, msg)


def _ptr(t):
    """Device pointer of a torch tensor (or None -> NULL)."""
    if t is None:
        return None
    return C.c_void_p(t.data_ptr())


def _i32(seq):
    a = np.ascontiguousarray(np.asarray(seq, dtype=np.int32))
    return a, a.ctypes.data_as(C.c_void_p)


def _u8(seq):
    a = np.ascontiguousarray(np.asarray(seq, dtype=np.uint8))
    return a, a.ctypes.data_as(C.c_void_p)


def blt_state_size(cfg: blt_config):
    kv, cr = C.c_size_t(), C.c_size_t()
    _check("blt_state_size", lib().blt_state_size(C.byref(cfg), C.byref(kv), C.byref(cr)))
    return kv.value, cr.value


def blt_create(cfg: blt_config, weights: blt_weights, stream_ptr: int):
    ctx = C.c_void_p()
    _check("blt_create", lib().blt_create(C.byref(cfg), C.byref(weights), C.c_void_p(stream_ptr),
                                          C.byref(ctx)))
    return ctx


def blt_destroy(ctx):
    _check("blt_destroy", lib().blt_destroy(ctx))


def blt_latents_put(ctx, state: blt_state, slot, idx, table, seq_stride: int):
    s, sp = _i32(slot)
    i, ip = _i32(idx)
    _check("blt_latents_put", lib().blt_latents_put(ctx, C.byref(state), len(s), sp, ip,
                                                    _ptr(table), seq_stride), ctx)


def _sampling(sampling, draw):
    smp = smpp = dr = drp = None
    if sampling is not None:
        smp = blt_sampling(C.c_float(sampling[0]), C.c_float(sampling[1]), int(sampling[2]))
        smpp = C.byref(smp)
    if draw is not None:
        dr, drp = _i32(draw)
    return (smp, dr), smpp, drp


def blt_kv_append(ctx, state, slot, start_pos, n_rows, n_max, lat_idx, bytes_=None,
                  tokens_dev=None, argmax_out=None, conf_out=None, logits_out=None, sampling=None,
                  draw=None, noalloc=False):
    """sampling: None (greedy) or (temperature, top_p, seed); draw: one draw
    index per sequence (required with sampling).  noalloc: call
    blt_kv_append_noalloc (the pass works in the library's static scratch
    array; at most 15 rows)."""
    fn = "blt_kv_append_noalloc" if noalloc else "blt_kv_append"
    keep, smpp, drp = _sampling(sampling, draw)
    s, sp = _i32(slot)
    st, stp = _i32(start_pos)
    n, np_ = _i32(n_rows)
    li, lip = _i32(np.asarray(lat_idx).reshape(-1))
    b = None
    bp = None
    if bytes_ is not None:
        b, bp = _u8(np.asarray(bytes_).reshape(-1))
    _check(fn, getattr(lib(), fn)(
        ctx, C.byref(state), len(s), sp, stp, np_, n_max, bp, _ptr(tokens_dev), lip,
        _ptr(argmax_out), _ptr(conf_out), _ptr(logits_out), smpp, drp), ctx)


def blt_decode_block_step(ctx, state, slot, start_pos, block_tok, B, block_lat, alpha,
                          mode=BLT_UNMASK_THRESHOLD, mask=BLT_BLOCK_BIDIR, n_append=None,
                          n_append_max=0, append_bytes=None, append_lat=None, argmax_out=None,
                          conf_out=None, logits_out=None, masked_left=None, sampling=None,
                          draw=None):
    """sampling: None (greedy) or (temperature, top_p, seed); draw: one draw
    index per sequence (required with sampling)."""
    s, sp = _i32(slot)
    smp = smpp = dr = drp = None
    if sampling is not None:
        smp = blt_sampling(C.c_float(sampling[0]), C.c_float(sampling[1]), int(sampling[2]))
        smpp = C.byref(smp)
    if draw is not None:
        dr, drp = _i32(draw)
    st, stp = _i32(start_pos)
    bl, blp = _i32(block_lat)
    keep = []
    nap = abp = alp = None
    if n_append_max > 0:
        a, nap = _i32(n_append)
        ab, abp = _u8(np.asarray(append_bytes).reshape(-1))
        al, alp = _i32(np.asarray(append_lat).reshape(-1))
        keep += [a, ab, al]
    _check("blt_decode_block_step", lib().blt_decode_block_step(
        ctx, C.byref(state), len(s), sp, stp, nap, n_append_max, abp, alp, _ptr(block_tok), B,
        blp, C.c_float(alpha), mode, mask, _ptr(argmax_out), _ptr(conf_out), _ptr(logits_out),
        _ptr(masked_left), smpp, drp), ctx)


def blt_verify_sample(ctx, r, draft, ld_draft, zq, ld_q, zp, ld_p, sampling, draw, accept_len,
                      next_byte, slot=None, batch=None):
    """Rejection-sampling verification; sampling = (temperature, top_p, seed),
    draw: the verify pass's draw index per sequence."""
    keep, smpp, drp = _sampling(sampling, draw)
    sp = None
    if slot is not None:
        sl, sp = _i32(slot)
        batch = len(sl)
    _check("blt_verify_sample", lib().blt_verify_sample(
        ctx, batch, sp, r, _ptr(draft), ld_draft, _ptr(zq), ld_q, _ptr(zp), ld_p, smpp, drp,
        _ptr(accept_len), _ptr(next_byte)), ctx)


def blt_verify_accept(ctx, r, draft, ld_draft, pred, ld_pred, accept_len, next_byte, slot=None,
                      batch=None):
    sp = None
    if slot is not None:
        s, sp = _i32(slot)
        batch = len(s)
    _check("blt_verify_accept", lib().blt_verify_accept(
        ctx, batch, sp, r, _ptr(draft), ld_draft, _ptr(pred), ld_pred, _ptr(accept_len),
        _ptr(next_byte)), ctx)


def blt_graphs_enable(ctx, enable):
    _check("blt_graphs_enable", lib().blt_graphs_enable(ctx, 1 if enable else 0), ctx)


def blt_attention_chunks(ctx, chunks):
    _check("blt_attention_chunks", lib().blt_attention_chunks(ctx, chunks), ctx)


def blt_flash_key_groups(ctx, groups):
    _check("blt_flash_key_groups", lib().blt_flash_key_groups(ctx, groups), ctx)


def blt_gemm_form(ctx, form):
    _check("blt_gemm_form", lib().blt_gemm_form(ctx, form), ctx)


def blt_profile_enable(ctx, family):
    _check("blt_profile_enable", lib().blt_profile_enable(ctx, family), ctx)


def blt_profile_read(ctx, reset=False):
    n, ms, by = C.c_uint64(), C.c_double(), C.c_double()
    _check("blt_profile_read", lib().blt_profile_read(ctx, C.byref(n), C.byref(ms), C.byref(by),
                                                      1 if reset else 0), ctx)
    return n.value, ms.value, by.value


def blt_bw_model(n_dec, n_encglob, n_seq, p_dec, p_enc, p_glob, bytes_per_param=2):
    c = blt_counts(n_dec, n_encglob, n_seq)
    p = blt_params(p_dec, p_enc, p_glob, bytes_per_param)
    tot, gb = C.c_uint64(), C.c_double()
    _check("blt_bw_model", lib().blt_bw_model(C.byref(c), C.byref(p), C.byref(tot), C.byref(gb)))
    return tot.value, gb.value


def blt_session_create(ctx, state, prompts, patch_lens, salts, latent_table, n_latents):
    batch = len(prompts)
    pr = [np.ascontiguousarray(np.asarray(p, dtype=np.uint8)) for p in prompts]
    pl = [np.ascontiguousarray(np.asarray(p, dtype=np.int32)) for p in patch_lens]
    pp = (C.c_void_p * batch)(*[a.ctypes.data for a in pr])
    lp = (C.c_void_p * batch)(*[a.ctypes.data for a in pl])
    plen, plenp = _i32([len(a) for a in pr])
    npt, nptp = _i32([len(a) for a in pl])
    salt = np.ascontiguousarray(np.asarray([s & (2 ** 64 - 1) for s in salts], dtype=np.uint64))
    out = C.c_void_p()
    _check("blt_session_create", lib().blt_session_create(
        ctx, C.byref(state), batch, pp, plenp, lp, nptp, salt.ctypes.data_as(C.c_void_p),
        _ptr(latent_table), n_latents, C.byref(out)), ctx)
    return out


def blt_session_prefill(ctx, sess):
    _check("blt_session_prefill", lib().blt_session_prefill(sess), ctx)


def blt_session_generate(ctx, sess, policy, block, alpha, n_gen, unmask=BLT_UNMASK_THRESHOLD,
                         block_mask=BLT_BLOCK_BIDIR, temperature=0.0, top_p=1.0, seed=0):
    a = blt_policy_args(policy, block, alpha, unmask, block_mask, n_gen, temperature, top_p, seed)
    _check("blt_session_generate", lib().blt_session_generate(sess, C.byref(a)), ctx)


def blt_session_device_blocks(ctx, sess, mode=1):
    """BLT-D blocks after the first one: 0 (or False) host-driven, 1 (or True)
    on the device, 2 chosen from the first blocks (see blt.h)."""
    _check("blt_session_device_blocks", lib().blt_session_device_blocks(sess, int(mode)), ctx)


def blt_session_result(sess, b, cap):
    buf = (C.c_uint8 * max(cap, 1))()
    n = C.c_int32()
    nd, ne, nr, na = C.c_uint64(), C.c_uint64(), C.c_uint64(), C.c_uint64()
    _check("blt_session_result", lib().blt_session_result(
        sess, b, buf, cap, C.byref(n), C.byref(nd), C.byref(ne), C.byref(nr), C.byref(na)))
    return {"out": bytes(buf[:min(n.value, cap)]), "n": n.value, "n_dec": nd.value,
            "n_eg": ne.value, "rounds": nr.value, "accepted": na.value}


def blt_session_destroy(sess):
    _check("blt_session_destroy", lib().blt_session_destroy(sess))


def decoder_params(n_layers, d_model, d_ffn, d_global, vocab=VOCAB):
    """Parameters of the local decoder as configured here, the P_dec of the
    bandwidth proxy: byte embedding and head (vocab x d each), latent
    projection (d x d_global), per layer the cross-attention q/k/v/o and
    self-attention q/k/v/o projections (8 d^2), the two FFN matrices (2 d F)
    and two RMSNorm gains, and the final gain."""
    d, F, L = d_model, d_ffn, n_layers
    return 2 * vocab * d + d * d_global + L * (8 * d * d + 2 * d * F + 2 * d) + d


def streamed_params(n_layers, d_model, d_ffn, vocab=VOCAB):
    """Weights one decoder pass reads: per layer W_qkv, W_o, W1, W2, and the
    byte head (the cross-attention products are applied once per latent)."""
    d, F, L = d_model, d_ffn, n_layers
    return L * (4 * d * d + 2 * d * F) + vocab * d


def latent_params(n_layers, d_model, d_global):
    """Weights one blt_latents_put batch reads: W_lat and the stacked
    per-layer cross products W_o^c W_v^c."""
    return d_model * d_global + n_layers * d_model * d_model


class Decoder:
    """Weights and decode state on the GPU, with a libblt context over them."""

    def __init__(self, weights: Dict, *, n_layers, d_model, n_heads, d_ffn, d_global, dtype,
                 max_batch, max_ctx, max_latents, max_rows, max_block, rope_theta=10000.0,
                 rms_eps=1e-5, device="cuda"):
        import torch
        self.torch_dtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.cfg = blt_config(n_layers, d_model, n_heads, d_ffn, VOCAB, d_global, max_batch,
                              max_ctx, max_latents, max_rows, max_block,
                              BLT_BF16 if dtype == "bf16" else BLT_F32, rope_theta, rms_eps)
        lib()  # fail loudly before allocating anything

        def dev(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(
                device=device, dtype=self.torch_dtype)

        self.t = {k: dev(weights[k]) for k in ("embed", "w_lat", "w_out", "g_out")}
        self.lt = [{k: dev(lw[k]) for k in ("wv_c", "wo_c", "wqkv", "wo", "g_attn", "g_ffn",
                                             "w1", "w2")} for lw in weights["layers"]]
        self._layers = (blt_layer_weights * n_layers)(*[
            blt_layer_weights(*[lw[k].data_ptr() for k in ("wv_c", "wo_c", "wqkv", "wo",
                                                          "g_attn", "g_ffn", "w1", "w2")])
            for lw in self.lt])
        self.weights = blt_weights(self.t["embed"].data_ptr(), self.t["w_lat"].data_ptr(),
                                   self.t["w_out"].data_ptr(), self.t["g_out"].data_ptr(),
                                   C.cast(self._layers, C.POINTER(blt_layer_weights)))
        kvb, crb = blt_state_size(self.cfg)
        self.kv = torch.empty(kvb, dtype=torch.uint8, device=device)
        self.cross = torch.empty(crb, dtype=torch.uint8, device=device)
        self.state = blt_state(self.kv.data_ptr(), self.cross.data_ptr())
        self.stream = torch.cuda.current_stream(device)
        self.ctx = blt_create(self.cfg, self.weights, self.stream.cuda_stream)

    def close(self):
        if self.ctx:
            blt_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
