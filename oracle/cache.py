"""Decoder forward over a clean-prefix KV cache (oracle; test infrastructure only).

pytorch.kr Fast-BLT summary, "BLT-D inference": the clean prefix (and all
latents but the last) can be cached, so each step recomputes only the last
latent and the current block.  This module keeps, per layer, the RoPE'd keys
and the values of the clean rows already seen, and runs new rows against
them.  It must reproduce ``model.forward`` with the explicit BLT-D mask; the
tests check exactly that.

Rows of one call are ``n_append`` clean rows followed by block rows, at
consecutive positions starting at ``start``.  The clean rows are causal; block
rows read the whole prefix and every block row (bidirectional) or the block
rows up to themselves (causal).  Block rows never enter the cache: their keys
and values are recomputed on every pass.  Calling with ``start`` below the
current length truncates the cache there first (rollback).
"""
from __future__ import annotations

import numpy as np

from . import model


class CachedDecoder:
    def __init__(self, W, wl, latents, capacity):
        self.W = W
        self.wl = wl
        self.latents = latents
        H, dh = wl.n_heads, wl.d_model // wl.n_heads
        self.K = [np.zeros((capacity, H, dh)) for _ in range(wl.n_layers)]
        self.V = [np.zeros((capacity, H, dh)) for _ in range(wl.n_layers)]
        self.length = 0
        self.tau = np.full(capacity, -1, dtype=np.int64)   # target each cached row used

    def run(self, tokens, start, targets, n_append, block_causal=False):
        """Run rows at positions start.. and return their [n, 257] logits."""
        wl, W = self.wl, self.W
        tokens = np.asarray(tokens, dtype=np.int64)
        n = len(tokens)
        if not (0 <= start <= self.length):
            raise ValueError("start must lie within the cached prefix")
        if start + n > self.K[0].shape[0]:
            raise ValueError("cache capacity exceeded")
        pos = start + np.arange(n)
        cur = model.blt_d_mask(n_append, n - n_append, block_causal)
        allow = np.concatenate([np.ones((n, start), dtype=bool), cur], axis=1)
        lat_sets = [[int(t)] for t in targets]
        h = W["embed"][tokens].copy()
        for li, lw in enumerate(W["layers"]):
            h = h + model.cross_attention(W, lw, h, self.latents, lat_sets, wl.n_heads)
            q, k, v = model.self_attention_qkv(lw, h, pos, wl.n_heads, wl.rms_eps, wl.rope_theta)
            keys = np.concatenate([self.K[li][:start], k], axis=0)
            vals = np.concatenate([self.V[li][:start], v], axis=0)
            a = model.masked_attention(q, keys, vals, allow).reshape(h.shape)
            h = h + a @ lw["wo"].T
            h = h + model.ffn(lw, h, wl.rms_eps)
            self.K[li][start:start + n_append] = k[:n_append]
            self.V[li][start:start + n_append] = v[:n_append]
        self.length = start + n_append
        self.tau[start:start + n_append] = np.asarray(targets[:n_append], dtype=np.int64)
        return model.head(W, h, wl.rms_eps)

    def truncate(self, length):
        if length > self.length:
            raise ValueError("cannot extend by truncation")
        self.length = length
