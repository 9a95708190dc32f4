"""Helpers shared by the GPU tests: build a Decoder for a workload and replay
oracle pass traces through the C-ABI (teacher forcing)."""
from __future__ import annotations

import sys

import numpy as np

import bltgen
from oracle import decide, loops, model, patcher

FP32_REL = 1e-4       # fp32 path: max|dz| <= 1e-4 * max|z_oracle| per row
BF16_ABS = 2e-2       # bf16 path: max|dz| <= 2e-2
GAP_MARGIN = {"fp32": 1e-4, "bf16": 4e-2}    # decisions compared only outside these bands
CONF_MARGIN = {"fp32": 1e-5, "bf16": 1e-2}
FALLBACK_REL = {"fp32": 1e-5, "bf16": 5e-2}   # relative gap of the two most confident positions


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def decoder_for(wl, w, max_batch=None, max_rows=256, device="cuda:0"):
    import block_diffusion_byte_amd as blt
    return blt.Decoder(w, n_layers=wl.n_layers, d_model=wl.d_model, n_heads=wl.n_heads,
                       d_ffn=wl.d_ffn, d_global=wl.d_global, dtype=wl.dtype,
                       max_batch=max_batch or wl.batch, max_ctx=wl.max_ctx,
                       max_latents=wl.n_latents, max_rows=max_rows, max_block=max(wl.block, 1),
                       rope_theta=wl.rope_theta, rms_eps=wl.rms_eps, device=device)


def oracle_inputs(wl, w, seq=0):
    W = model.as64(w)
    inp = bltgen.make_sequence_inputs(wl, seq)
    inp64 = dict(inp, latents=inp["latents"].astype(np.float64))
    return W, inp, inp64


def logits_ok(got, ref, dtype):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref).max(axis=-1)
    if dtype == "fp32":
        tol = FP32_REL * np.abs(ref).max(axis=-1)
    else:
        tol = np.full(err.shape, BF16_ABS)
    return bool((err <= tol).all()), float(err.max()), float(tol.min())


class Replayer:
    """Replays an oracle trace on the GPU for one sequence in state slot 0."""

    def __init__(self, dec, wl, inp, slot=0):
        import torch
        import block_diffusion_byte_amd as blt
        self.blt, self.torch = blt, torch
        self.dec, self.wl, self.slot = dec, wl, slot
        dev = dec.kv.device
        self.table = torch.from_numpy(inp["latents"]).to(dev, dec.torch_dtype)
        mb = dec.cfg.max_batch
        B = max(wl.block, 1)
        self.B = B
        self.block_tok = torch.full((mb * B,), 256, dtype=torch.int32, device=dev)
        self.masked = torch.zeros(mb, dtype=torch.int32, device=dev)
        W = max(B + 1, 2)
        self.W = W
        self.argmax = torch.zeros(mb * max(W, dec.cfg.max_rows), dtype=torch.int32, device=dev)
        self.conf = torch.zeros(mb * max(W, dec.cfg.max_rows), dtype=torch.float32, device=dev)
        self.logits = torch.zeros(mb * max(W, dec.cfg.max_rows) * 257, dtype=torch.float32, device=dev)
        # every latent of the table gets its cross vectors
        n = wl.n_latents
        blt.blt_latents_put(dec.ctx, dec.state, [slot] * n, list(range(n)), self.table, 0)

    def prefill(self, inp):
        x = [int(b) for b in inp["prompt"]]
        patch, ends = patcher.segment(x, inp["prompt_patches"], inp["salt"])
        n = len(x) - 1
        taus = [patcher.causal_target(patch, ends, i) for i in range(n)]
        mr = self.dec.cfg.max_rows
        for c0 in range(0, n, mr):
            m = min(mr, n - c0)
            self.blt.blt_kv_append(self.dec.ctx, self.dec.state, [self.slot], [c0], [m], m,
                                   taus[c0:c0 + m], bytes_=x[c0:c0 + m])

    def rows(self, rec):
        """Run a clean-row pass; return (logits [n, 257], argmax [n])."""
        n = len(rec["tokens"])
        self.blt.blt_kv_append(self.dec.ctx, self.dec.state, [self.slot], [rec["start"]], [n], n,
                               rec["targets"], bytes_=rec["tokens"], argmax_out=self.argmax,
                               logits_out=self.logits)
        self.torch.cuda.synchronize()
        base = self.slot * n
        z = self.logits[base * 257:(base + n) * 257].view(n, 257).cpu().numpy()
        return z, self.argmax[base:base + n].cpu().numpy()

    def block(self, rec, alpha, one_step):
        """Run a BLT-D pass from the oracle's block state; return logits of
        the block rows, argmax, conf and the block after the commit."""
        B, na = len(rec["block_before"]), rec["n_append"]
        s = self.slot
        self.block_tok[s * B:(s + 1) * B] = self.torch.tensor(rec["block_before"], dtype=self.torch.int32)
        self.blt.blt_decode_block_step(
            self.dec.ctx, self.dec.state, [s], [rec["start"]], self.block_tok, B,
            [rec["targets"][na]], alpha,
            mode=self.blt.BLT_UNMASK_ONE_STEP if one_step else self.blt.BLT_UNMASK_THRESHOLD,
            mask=self.blt.BLT_BLOCK_CAUSAL if rec["block_causal"] else self.blt.BLT_BLOCK_BIDIR,
            n_append=[na], n_append_max=na, append_bytes=rec["tokens"][:na] if na else None,
            append_lat=rec["targets"][:na] if na else None, argmax_out=self.argmax,
            conf_out=self.conf, logits_out=self.logits, masked_left=self.masked)
        self.torch.cuda.synchronize()
        z = self.logits[s * B * 257:(s + 1) * B * 257].view(B, 257).cpu().numpy()
        return (z, self.argmax[s * B:(s + 1) * B].cpu().numpy(),
                self.conf[s * B:(s + 1) * B].cpu().numpy(),
                self.block_tok[s * B:(s + 1) * B].cpu().numpy(), int(self.masked[s].item()))


def replay_and_compare(dec, wl, inp, run, alpha, one_step, dtype):
    """Teacher-forced replay of every pass of an oracle run.  Returns
    (worst logit error, decisions compared, decisions skipped as near-ties)."""
    rp = Replayer(dec, wl, inp)
    rp.prefill(inp)
    worst, compared, skipped = 0.0, 0, 0
    gapm, confm = GAP_MARGIN[dtype], CONF_MARGIN[dtype]
    for k, rec in enumerate(run.passes):
        if rec["kind"] == "block":
            z, am, conf, after, left = rp.block(rec, alpha, one_step)
            na = rec["n_append"]
            ok, err, tol = logits_ok(z, rec["logits"][na:], dtype)
            assert ok, f"pass {k}: block logits err {err} > tol {tol}"
            worst = max(worst, err)
            masked = [j for j, t in enumerate(rec["block_before"]) if t == 256]
            near = any(rec["gap"][j] <= gapm or (not one_step and abs(rec["conf"][j] - alpha) <= confm)
                       for j in masked)
            cs = sorted((rec["conf"][j] for j in masked), reverse=True)
            if not one_step and cs and cs[0] <= alpha and len(cs) > 1:
                # forced single commit: the two most confident positions must be apart
                near = near or (cs[0] - cs[1]) <= FALLBACK_REL[dtype] * cs[0]
            if near:
                skipped += 1
                continue
            for j in masked:
                assert am[j] == rec["choice"][j], f"pass {k} pos {j}: argmax {am[j]} vs {rec['choice'][j]}"
                assert abs(conf[j] - rec["conf"][j]) <= max(confm, 1e-6)
            assert list(after) == rec["block_after"], f"pass {k}: block {list(after)} vs {rec['block_after']}"
            assert left == sum(1 for t in rec["block_after"] if t == 256)
            compared += 1
        else:
            z, am = rp.rows(rec)
            ok, err, tol = logits_ok(z, rec["logits"], dtype)
            assert ok, f"pass {k} ({rec['kind']}): logits err {err} > tol {tol}"
            worst = max(worst, err)
            for j, (g, c) in enumerate(zip(rec["gap"], rec["choice"])):
                if g > gapm:
                    assert am[j] == c, f"pass {k} row {j}: argmax {am[j]} vs {c}"
                    compared += 1
                else:
                    skipped += 1
    return worst, compared, skipped
