"""Decoder forward pass with explicit masks, float64 (oracle; test infrastructure only).

The local decoder of BLT (pytorch.kr Fast-BLT summary, "BLT architecture"
section, the layer equation): each layer first adds a cross-attention read of
the global model's patch latents to the residual stream, B_l = D_{l-1} +
W_o softmax(Q K^T / sqrt(d_k)) V, and then applies an ordinary decoder
transformer layer, D_l = DecoderTransformerLayer(B_l).

Readings where the pages are silent (each listed in the design notes):
  * the transformer layer is pre-norm: RMSNorm -> causal/block self-attention
    with RoPE -> residual, then RMSNorm -> W2 SiLU(W1 .) -> residual; a final
    RMSNorm feeds an untied 257-way head.  No biases.  eps = 1e-5.
  * one shared latent projection W_lat (d x d_global) maps o_m to the
    decoder width; per layer W_q^c, W_k^c, W_v^c, W_o^c are d x d and the
    cross query is not normalised.
  * RoPE uses the original byte positions (BLT-D training, block
    construction: each block byte keeps its original index for RoPE), the
    rotate-half pairing (i, i + d_h/2), theta = 10000, 0-based positions.
"""
from __future__ import annotations

import numpy as np


def as64(w):
    """Recursively convert a weight dict (bltgen layout) to float64 arrays."""
    if isinstance(w, dict):
        return {k: as64(v) for k, v in w.items()}
    if isinstance(w, list):
        return [as64(v) for v in w]
    return np.asarray(w, dtype=np.float64)


def rms_norm(x, g, eps):
    """g * x / sqrt(mean(x^2) + eps) over the last axis."""
    return g * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def silu(x):
    return x / (1.0 + np.exp(-x))


def rope(x, pos, theta):
    """Rotate-half RoPE.  x: [n, H, d_h]; pos: [n] absolute byte positions.

    Pair (j, j + d_h/2) is rotated by the angle pos * theta^(-2j/d_h).
    """
    dh = x.shape[-1]
    half = dh // 2
    freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / dh)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * freq[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def masked_attention(q, k, v, allow):
    """Multi-head softmax attention with an explicit boolean mask.

    q: [n, H, dh]; k, v: [m, H, dh]; allow: [n, m] (row i may read key j).
    Returns [n, H, dh].  Every row must be allowed at least one key.
    """
    n, H, dh = q.shape
    m = k.shape[0]
    kt = np.ascontiguousarray(k.transpose(1, 2, 0))      # [H, dh, m]
    vh = np.ascontiguousarray(v.transpose(1, 0, 2))      # [H, m, dh]
    out = np.empty((n, H, dh))
    step = max(1, int(2e7 // max(1, H * m)))             # bound the score tensor
    for i0 in range(0, n, step):
        i1 = min(n, i0 + step)
        qh = np.ascontiguousarray(q[i0:i1].transpose(1, 0, 2))   # [H, r, dh]
        s = (qh @ kt) / np.sqrt(dh)                       # [H, r, m]
        s = np.where(allow[None, i0:i1, :], s, -np.inf)
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=-1, keepdims=True)
        out[i0:i1] = (p @ vh).transpose(1, 0, 2)
    return out


def latent_keys_values(W, lw, latents, idx):
    """Cross-attention keys and values of the latents ``idx`` for one layer.

    o~_m = W_lat o_m, k_m = W_k^c o~_m, v_m = W_v^c o~_m.
    """
    ot = latents[idx] @ W["w_lat"].T
    return ot @ lw["wk_c"].T, ot @ lw["wv_c"].T


def cross_attention(W, lw, h, latents, lat_sets, n_heads):
    """General multi-head cross-attention of each row to its allowed latents.

    lat_sets: list (one per row) of latent indices the row may attend.  In the
    BLT-D masks every row reads exactly one latent (pytorch.kr summary, "BLT-D
    attention mask": prefix byte i reads o_{p(i)-1}, the last byte of a patch
    reads o_{p(i)}, block bytes read only o_M); the softmax is still taken
    over the allowed set, so a wider set would be handled the same way.
    """
    n, d = h.shape
    dh = d // n_heads
    smax = max(len(s) for s in lat_sets)
    idx = np.zeros((n, smax), dtype=np.int64)
    ok = np.zeros((n, smax), dtype=bool)
    for i, s in enumerate(lat_sets):
        idx[i, :len(s)] = s
        ok[i, :len(s)] = True
    uniq, inv = np.unique(idx, return_inverse=True)
    kl, vl = latent_keys_values(W, lw, latents, uniq)
    kr = kl[inv.reshape(n, smax)].reshape(n, smax, n_heads, dh)
    vr = vl[inv.reshape(n, smax)].reshape(n, smax, n_heads, dh)
    q = (h @ lw["wq_c"].T).reshape(n, n_heads, dh)
    s = np.einsum("ihd,ishd->ihs", q, kr) / np.sqrt(dh)
    s = np.where(ok[:, None, :], s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    a = np.einsum("ihs,ishd->ihd", p, vr).reshape(n, d)
    return a @ lw["wo_c"].T


def self_attention_qkv(lw, h, pos, n_heads, eps, theta):
    """Pre-norm q, k, v of the rows, with RoPE applied to q and k."""
    n, d = h.shape
    dh = d // n_heads
    u = rms_norm(h, lw["g_attn"], eps)
    qkv = u @ lw["wqkv"].T
    q = rope(qkv[:, :d].reshape(n, n_heads, dh), pos, theta)
    k = rope(qkv[:, d:2 * d].reshape(n, n_heads, dh), pos, theta)
    v = qkv[:, 2 * d:].reshape(n, n_heads, dh)
    return q, k, v


def ffn(lw, h, eps):
    """W2 SiLU(W1 RMSNorm(h))."""
    return silu(rms_norm(h, lw["g_ffn"], eps) @ lw["w1"].T) @ lw["w2"].T


def head(W, h, eps):
    """Final RMSNorm and the 257-way byte head: fp64 logits."""
    return rms_norm(h, W["g_out"], eps) @ W["w_out"].T


def forward(W, wl, latents, tokens, pos, lat_sets, allow):
    """No-cache decoder forward over ``n`` rows with an explicit [n, n] mask.

    tokens: ids 0..256 (256 = [MASK]); pos: absolute byte positions;
    lat_sets: per-row allowed latent indices; allow[i, j]: row i reads row j.
    Returns the [n, 257] logits.
    """
    tokens = np.asarray(tokens)
    h = W["embed"][tokens].copy()
    for lw in W["layers"]:
        h = h + cross_attention(W, lw, h, latents, lat_sets, wl.n_heads)
        q, k, v = self_attention_qkv(lw, h, pos, wl.n_heads, wl.rms_eps, wl.rope_theta)
        a = masked_attention(q, k, v, allow).reshape(h.shape)
        h = h + a @ lw["wo"].T
        h = h + ffn(lw, h, wl.rms_eps)
    return head(W, h, wl.rms_eps)


def blt_d_mask(n_prefix, n_block, block_causal=False):
    """Self-attention mask of the BLT-D decoder input x' = [x; block].

    pytorch.kr summary, "BLT-D attention mask": prefix positions attend
    causally; block positions attend each other bidirectionally and read the
    whole clean prefix; a prefix position never reads a block position.  With
    ``block_causal`` the block is causal as well (the same weights run as an
    autoregressive model, used for verification).
    """
    n = n_prefix + n_block
    allow = np.zeros((n, n), dtype=bool)
    for i in range(n):
        if i < n_prefix:
            allow[i, : i + 1] = True
        else:
            allow[i, :n_prefix] = True
            if block_causal:
                allow[i, n_prefix: i + 1] = True
            else:
                allow[i, n_prefix:] = True
    return allow
