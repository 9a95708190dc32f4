"""Helpers shared by the GPU tests: build a Decoder for a workload and replay
oracle pass traces through the C-ABI (teacher forcing)."""
from __future__ import annotations

import sys

import numpy as np

import bltgen
from oracle import decide, loops, model, patcher

FP32_REL = 1e-4       # fp32 path: max|dz| <= 1e-4 * max|z_oracle| per row
BF16_ABS = 2e-2       # bf16 path: max|dz| <= 2e-2
CONF_MARGIN = {"fp32": 1e-5, "bf16": 1e-2}   # confidence tolerance (absolute)
ENT_TOL = {"fp32": 1e-4, "bf16": 5e-2}       # entropy tolerance (nats, absolute)


def unmask_mode(unmask):
    """"threshold" / "one_step" / "entropy" from a mode name or a one_step flag."""
    if isinstance(unmask, str):
        return unmask
    return "one_step" if unmask else "threshold"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# Fraction of bf16 decisions that must be decidable beyond the measured
# GPU-oracle differences (and so compared exactly).  With the 1B-class logit
# spread (std ~0.6 over 256 bytes, top-2 gap ~0.2) and bf16 logit errors of
# ~1e-2, about one greedy decision in seven falls inside twice the row error.
COVERAGE_FLOOR = 0.7


def assert_coverage(name, compared, skipped, floor=COVERAGE_FLOOR):
    """Enough decisions were compared exactly (not skipped as near-ties)."""
    tot = compared + skipped
    frac = compared / tot if tot else 0.0
    assert compared > 0 and frac >= floor, \
        f"{name}: only {compared} of {tot} decisions compared ({skipped} near-ties skipped), below {floor:.0%}"
    return frac


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


def logits_ok(got, ref, dtype, scale=1.0):
    """Logits within the path's tolerance.  scale: the head-weight scale of
    the decoder (logits and their rounding errors grow with it in proportion,
    so the bf16 bound is BF16_ABS * scale)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref).max(axis=-1)
    if dtype == "fp32":
        tol = FP32_REL * np.abs(ref).max(axis=-1)
    else:
        tol = np.full(err.shape, BF16_ABS * scale)
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

    def rows(self, rec, sampling=None, draw=None):
        """Run a clean-row pass; return (logits [n, 257], argmax [n]) (the
        drawn bytes when sampling)."""
        n = len(rec["tokens"])
        self.blt.blt_kv_append(self.dec.ctx, self.dec.state, [self.slot], [rec["start"]], [n], n,
                               rec["targets"], bytes_=rec["tokens"], argmax_out=self.argmax,
                               logits_out=self.logits, sampling=sampling,
                               draw=None if draw is None else [draw])
        self.torch.cuda.synchronize()
        base = self.slot * n
        z = self.logits[base * 257:(base + n) * 257].view(n, 257).cpu().numpy()
        return z, self.argmax[base:base + n].cpu().numpy()

    def block(self, rec, alpha, unmask, sampling=None, draw=None):
        """Run a BLT-D pass from the oracle's block state; return logits of
        the block rows, argmax (the drawn bytes when sampling), conf (entropy
        under "entropy") and the block after the commit."""
        B, na = len(rec["block_before"]), rec["n_append"]
        s = self.slot
        self.block_tok[s * B:(s + 1) * B] = self.torch.tensor(rec["block_before"], dtype=self.torch.int32)
        mode = {"threshold": self.blt.BLT_UNMASK_THRESHOLD, "one_step": self.blt.BLT_UNMASK_ONE_STEP,
                "entropy": self.blt.BLT_UNMASK_ENTROPY}[unmask_mode(unmask)]
        self.blt.blt_decode_block_step(
            self.dec.ctx, self.dec.state, [s], [rec["start"]], self.block_tok, B,
            [rec["targets"][na]], alpha,
            mode=mode,
            mask=self.blt.BLT_BLOCK_CAUSAL if rec["block_causal"] else self.blt.BLT_BLOCK_BIDIR,
            n_append=[na], n_append_max=na, append_bytes=rec["tokens"][:na] if na else None,
            append_lat=rec["targets"][:na] if na else None, argmax_out=self.argmax,
            conf_out=self.conf, logits_out=self.logits, masked_left=self.masked,
            sampling=sampling, draw=None if draw is None else [draw])
        self.torch.cuda.synchronize()
        z = self.logits[s * B * 257:(s + 1) * B * 257].view(B, 257).cpu().numpy()
        return (z, self.argmax[s * B:(s + 1) * B].cpu().numpy(),
                self.conf[s * B:(s + 1) * B].cpu().numpy(),
                self.block_tok[s * B:(s + 1) * B].cpu().numpy(), int(self.masked[s].item()))


def _row_err(got, ref):
    return np.abs(np.asarray(got, dtype=np.float64) - np.asarray(ref, dtype=np.float64)).max(axis=-1)


def _entropy_commit_decidable(rec, ent, alpha):
    """Is the oracle's entropy-bounded commit decided beyond the measured
    entropy differences?  The committed set must be separated from the
    other masked positions, and the running sums must clear gamma on both
    sides of the cut."""
    before = [int(t) for t in rec["block_before"]]
    masked = [j for j, t in enumerate(before) if t == 256]
    rent = list(rec["entropy"])
    d = {j: abs(float(ent[j]) - rent[j]) + 1e-6 for j in masked}
    after = [int(t) for t in rec["block_after"]]
    S = [j for j in masked if after[j] != 256]
    O = [j for j in masked if after[j] == 256]
    if O and max(rent[j] + d[j] for j in S) >= min(rent[j] - d[j] for j in O):
        return False
    tot, err = sum(rent[j] for j in S), sum(d[j] for j in S)
    if len(S) > 1 and tot + err > alpha:
        return False
    if O:
        nxt = min(O, key=lambda j: (rent[j], j))
        if tot + rent[nxt] - err - d[nxt] <= alpha:
            return False
    return True


def check_block_pass(k, rec, z, am, conf, after, left, alpha, one_step, dtype, scale=1.0):
    """Compare one BLT-D pass of the GPU (block-row logits z, argmax, conf,
    block after the commit, masked count) with the oracle's record.

    Logits must lie within the path's tolerance.  A decision is compared
    wherever the oracle's margin exceeds the measured GPU-oracle difference
    of what decides it, so that both sides must agree: a position's greedy
    byte when its top-2 logit gap exceeds twice the row's largest logit
    difference; the commit when every confidence is farther from alpha than
    its own difference and, for a forced single commit, the two most
    confident position stays ahead of every other beyond their differences.
    Under "entropy" (one_step may name the mode) conf holds the GPU's
    entropies; see _entropy_commit_decidable.
    Returns (logit error, decisions compared, decisions skipped)."""
    mode = unmask_mode(one_step)
    one_step = mode == "one_step"
    na = int(rec["n_append"])
    zr = np.asarray(rec["logits"])[na:]
    ok, err, tol = logits_ok(z, zr, dtype, scale)
    assert ok, f"pass {k}: block logits err {err} > tol {tol}"
    rowerr = _row_err(z, zr)
    before = [int(t) for t in rec["block_before"]]
    choice, rconf, gap = list(rec["choice"]), list(rec["conf"]), list(rec["gap"])
    masked = [j for j, t in enumerate(before) if t == 256]
    if mode == "entropy":
        rent = list(rec["entropy"])
        for j in masked:
            assert abs(float(conf[j]) - rent[j]) <= ENT_TOL[dtype] * scale, \
                f"pass {k} pos {j}: entropy {conf[j]} vs {rent[j]}"
        dconf = {j: 0.0 for j in masked}
    else:
        dconf = {j: abs(float(conf[j]) - rconf[j]) for j in masked}
    compared = skipped = 0
    for j in masked:
        assert dconf[j] <= max(CONF_MARGIN[dtype] * scale, 1e-6), f"pass {k} pos {j}: conf {conf[j]} vs {rconf[j]}"
        if gap[j] > 2.0 * rowerr[j] + 1e-6:
            assert am[j] == choice[j], f"pass {k} pos {j}: argmax {am[j]} vs {choice[j]}"
            compared += 1
        else:
            skipped += 1
    near = any(gap[j] <= 2.0 * rowerr[j] + 1e-6 for j in masked)
    if one_step:
        # the one-step rule commits every masked position whatever the
        # confidences: the commit set is always decided, and each committed
        # byte is compared wherever that byte is decidable
        rafter = [int(t) for t in rec["block_after"]]
        assert left == 0 and all(int(t) != 256 for t in after), f"pass {k}: one-step block not filled"
        for j in masked:
            if gap[j] > 2.0 * rowerr[j] + 1e-6:
                assert int(after[j]) == rafter[j], f"pass {k} pos {j}: committed {after[j]} vs {rafter[j]}"
        return err, compared + 1, skipped
    if mode == "entropy":
        near = near or not _entropy_commit_decidable(rec, conf, alpha)
    else:
        near = near or any(abs(rconf[j] - alpha) <= dconf[j] + 1e-7 for j in masked)
        order = sorted(masked, key=lambda j: -rconf[j])
        if order and rconf[order[0]] <= alpha and len(order) > 1:
            # the most confident position must stay ahead of every other one
            j0 = order[0]
            near = near or any(rconf[j0] - dconf[j0] <= rconf[j] + dconf[j] + 1e-7 for j in order[1:])
    if near:
        return err, compared, skipped + 1
    rafter = [int(t) for t in rec["block_after"]]
    assert list(after) == rafter, f"pass {k}: block {list(after)} vs {rafter}"
    assert left == sum(1 for t in rafter if t == 256)
    return err, compared + 1, skipped


def check_rows_pass(k, rec, z, am, dtype, scale=1.0):
    """Compare a clean-row pass (draft, verify or greedy rows) with the
    oracle's record: logits within tolerance, each row's greedy byte where
    the oracle's top-2 gap exceeds twice the row's largest logit difference.
    Returns (logit error, decisions compared, skipped)."""
    ok, err, tol = logits_ok(z, rec["logits"], dtype, scale)
    assert ok, f"pass {k}: logits err {err} > tol {tol}"
    rowerr = _row_err(z, rec["logits"])
    compared = skipped = 0
    for j, (g, c) in enumerate(zip(rec["gap"], rec["choice"])):
        if g > 2.0 * rowerr[j] + 1e-6:
            assert am[j] == c, f"pass {k} row {j}: argmax {am[j]} vs {c}"
            compared += 1
        else:
            skipped += 1
    return err, compared, skipped


def replay_and_compare(dec, wl, inp, run, alpha, one_step, dtype):
    """Teacher-forced replay of every pass of an oracle run.  Returns
    (worst logit error, decisions compared, decisions skipped as near-ties)."""
    rp = Replayer(dec, wl, inp)
    rp.prefill(inp)
    worst, compared, skipped = 0.0, 0, 0
    for k, rec in enumerate(run.passes):
        if rec["kind"] == "block":
            z, am, conf, after, left = rp.block(rec, alpha, one_step)
            err, c, sk = check_block_pass(k, rec, z, am, conf, after, left, alpha, one_step, dtype,
                                          wl.head_scale)
            worst = max(worst, err)
            compared += c
            skipped += sk
        else:
            z, am = rp.rows(rec)
            err, c, sk = check_rows_pass(k, rec, z, am, dtype, wl.head_scale)
            worst = max(worst, err)
            compared += c
            skipped += sk
    return worst, compared, skipped
