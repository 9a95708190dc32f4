"""GPU parity at the full workload sizes, in the benchmark's launch configuration.

Every sequence of a workload's batch gets its own prompt, latents and state
slot, is prefilled the way the native decode driver does it (latents of the
prompt's patches, one cache append per sequence in chunks of max_rows), and
the first-round passes run for the whole batch in one call per pass, as the
driver issues them.  The sampled sequences are teacher-forced from the
float64 oracle's traces in tests/golden/fullsize_*.npz (written by
tests/golden/make_fullsize.py, which calls only the oracle) and compared:
bf16 logits within 2e-2 of the oracle, decisions exactly wherever the
oracle's margins lie outside the bf16 rounding band.  The other sequences
run on the GPU's own decisions; they are there so that every pass has the
benchmark's row count and attention grid.
"""
import importlib.util
import os
from types import SimpleNamespace

import numpy as np
import pytest

import bltgen
from oracle import patcher
from tests.gpu_util import (assert_coverage, check_block_pass, check_rows_pass, decoder_for,
                            replay_and_compare, say)

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
BLOCK, DRAFT, VERIFY = 0, 1, 2


KIND_NAMES = {0: "block", 1: "draft", 2: "verify", 3: "ar"}


def _golden_plan():
    spec = importlib.util.spec_from_file_location("make_fullsize", os.path.join(GOLD, "make_fullsize.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _as_run(recs):
    """Golden records in the form the single-sequence replayer takes."""
    passes = []
    for r in recs:
        d = dict(r)
        d["kind"] = KIND_NAMES[int(r["kind"])]
        for key in ("start", "n_append"):
            d[key] = int(r[key])
        for key in ("tokens", "targets", "choice", "block_before", "block_after"):
            if key in r:
                d[key] = [int(v) for v in r[key]]
        if "block_causal" in r:
            d["block_causal"] = bool(int(r["block_causal"]))
        passes.append(d)
    return SimpleNamespace(passes=passes)


def _gold(wl):
    z = np.load(os.path.join(GOLD, f"fullsize_{wl.name}.npz"))
    recs = {}
    for s in (int(v) for v in z["seqs"]):
        ps = []
        for i in range(int(z["n_passes"])):
            p = f"s{s}_p{i}_"
            ps.append({k[len(p):]: z[k] for k in z.files if k.startswith(p)})
        recs[s] = ps
    return recs


class FullBatch:
    def __init__(self, wl):
        import torch
        import block_diffusion_byte_amd as blt
        self.torch, self.blt, self.wl = torch, blt, wl
        self.b, self.B = wl.batch, max(wl.block, 1)
        self.max_rows = max(1024, wl.batch * (2 * wl.block + 2), wl.prompt_len)   # as bench.py
        self.dec = decoder_for(wl, bltgen.make_weights(wl), max_batch=self.b, max_rows=self.max_rows)
        dev = "cuda:0"
        inps = [bltgen.make_sequence_inputs(wl, s) for s in range(self.b)]
        self.table = torch.from_numpy(np.stack([i["latents"] for i in inps])).to(dev, self.dec.torch_dtype)
        self.x, self.seg = [], []
        slots, idx = [], []
        for s, inp in enumerate(inps):
            x = [int(v) for v in inp["prompt"]]
            patch, ends = patcher.segment(x, inp["prompt_patches"], inp["salt"])
            self.x.append(x)
            self.seg.append((patch, ends, inp["prompt_patches"], inp["salt"]))
            # latents through a few patches past the prompt's last: verification
            # rows over a draft may read patches the draft completes (two
            # rounds of up to B + 1 bytes each)
            m = min(patcher.last_target(patch) + 2 * (self.B + 1) + 1, wl.n_latents - 1)
            slots += [s] * (m + 1)
            idx += list(range(m + 1))
        blt.blt_latents_put(self.dec.ctx, self.dec.state, slots, idx, self.table, wl.n_latents)
        for s, x in enumerate(self.x):
            patch, ends = self.seg[s][:2]
            n = len(x) - 1                                   # the last prompt byte stays pending
            taus = [patcher.causal_target(patch, ends, i) for i in range(n)]
            for c0 in range(0, n, self.max_rows):
                m = min(self.max_rows, n - c0)
                blt.blt_kv_append(self.dec.ctx, self.dec.state, [s], [c0], [m], m, taus[c0:c0 + m],
                                  bytes_=x[c0:c0 + m])
        W = self.B + 1
        self.W = W
        self.block_tok = torch.full((self.b * self.B,), 256, dtype=torch.int32, device=dev)
        self.masked = torch.zeros(self.b, dtype=torch.int32, device=dev)
        self.argmax = torch.zeros(self.b * W, dtype=torch.int32, device=dev)
        self.conf = torch.zeros(self.b * W, dtype=torch.float32, device=dev)
        self.logits = torch.zeros(self.b * W * 257, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

    def close(self):
        self.dec.close()

    def last_target(self, s):
        return patcher.last_target(self.seg[s][0])

    def block_pass(self, first, forced, alpha, one_step):
        """One BLT-D pass of every sequence's first block.  first: the pending
        last prompt byte is appended (reading the last, possibly truncated,
        patch) in front of the block.  forced: {slot: block tokens before the
        pass} for the teacher-forced sequences."""
        blt, torch, B = self.blt, self.torch, self.B
        for s, bb in forced.items():
            self.block_tok[s * B:(s + 1) * B] = torch.tensor([int(t) for t in bb], dtype=torch.int32)
        if first:
            starts = [len(x) - 1 for x in self.x]
            kw = dict(n_append=[1] * self.b, n_append_max=1, append_bytes=[x[-1] for x in self.x],
                      append_lat=[self.last_target(s) for s in range(self.b)])
        else:
            starts = [len(x) for x in self.x]
            kw = {}
        blt.blt_decode_block_step(
            self.dec.ctx, self.dec.state, list(range(self.b)), starts, self.block_tok, B,
            [self.last_target(s) for s in range(self.b)], alpha,
            mode=blt.BLT_UNMASK_ONE_STEP if one_step else blt.BLT_UNMASK_THRESHOLD,
            mask=blt.BLT_BLOCK_BIDIR, argmax_out=self.argmax, conf_out=self.conf,
            logits_out=self.logits, masked_left=self.masked, **kw)
        torch.cuda.synchronize()
        z = self.logits.view(-1, 257)[:self.b * B].cpu().numpy().reshape(self.b, B, 257)
        am = self.argmax[:self.b * B].cpu().numpy().reshape(self.b, B)
        cf = self.conf[:self.b * B].cpu().numpy().reshape(self.b, B)
        blk = self.block_tok.cpu().numpy().reshape(self.b, B)
        return z, am, cf, blk, self.masked.cpu().numpy()

    def block_pass_rec(self, rec, alpha, one_step):
        """One BLT-D pass of sequence 0 (batch 1) as the oracle's record has it:
        its clean rows first (the pending prompt byte, or a rollback and the
        previous block's bytes), then the block."""
        blt, torch, B = self.blt, self.torch, self.B
        assert self.b == 1
        na = int(rec["n_append"])
        self.block_tok[:B] = torch.tensor([int(t) for t in rec["block_before"]], dtype=torch.int32)
        kw = {}
        if na:
            kw = dict(n_append=[na], n_append_max=na, append_bytes=[int(t) for t in rec["tokens"][:na]],
                      append_lat=[int(t) for t in rec["targets"][:na]])
        blt.blt_decode_block_step(
            self.dec.ctx, self.dec.state, [0], [int(rec["start"])], self.block_tok, B,
            [int(rec["targets"][na])], alpha,
            mode=blt.BLT_UNMASK_ONE_STEP if one_step else blt.BLT_UNMASK_THRESHOLD,
            mask=blt.BLT_BLOCK_BIDIR, argmax_out=self.argmax, conf_out=self.conf,
            logits_out=self.logits, masked_left=self.masked, **kw)
        torch.cuda.synchronize()
        z = self.logits.view(-1, 257)[:B].cpu().numpy().reshape(1, B, 257)
        am = self.argmax[:B].cpu().numpy().reshape(1, B)
        cf = self.conf[:B].cpu().numpy().reshape(1, B)
        blk = self.block_tok.cpu().numpy().reshape(1, B)
        return z, am, cf, blk, self.masked.cpu().numpy()

    def rows_pass(self, forced, fallback):
        """Clean rows of every sequence in one cache append (draft rows or a
        verification).  forced: {slot: (start, tokens, targets)}; the other
        sequences take fallback(slot) -> (start, tokens, targets), all with
        the same row count."""
        rows = {s: forced[s] if s in forced else fallback(s) for s in range(self.b)}
        n = len(rows[0][1])
        assert all(len(r[1]) == n for r in rows.values())
        self.blt.blt_kv_append(
            self.dec.ctx, self.dec.state, list(range(self.b)), [int(rows[s][0]) for s in range(self.b)],
            [n] * self.b, n, [int(t) for s in range(self.b) for t in rows[s][2]],
            bytes_=[int(t) for s in range(self.b) for t in rows[s][1]], argmax_out=self.argmax,
            logits_out=self.logits)
        self.torch.cuda.synchronize()
        z = self.logits.view(-1, 257)[:self.b * n].cpu().numpy().reshape(self.b, n, 257)
        am = self.argmax[:self.b * n].cpu().numpy().reshape(self.b, n)
        return z, am

    def verify_rows(self, s, draft):
        """Rows l..l+r of sequence s over the draft (l = its last prompt byte)."""
        x = self.x[s] + [int(t) for t in draft]
        patch, ends = patcher.segment(x, self.seg[s][2], self.seg[s][3])
        l = len(self.x[s]) - 1
        return l, x[l:], [patcher.causal_target(patch, ends, i) for i in range(l, len(x))]


def _summary(name, worst, compared, skipped):
    say(f"{name}: worst logit err {worst:.3g}, {compared} decisions compared, {skipped} near-ties skipped")
    assert_coverage(name, compared, skipped)


def test_fullsize_bltd4_batch1_first_block():
    """BLT-D-4 at the 1B-class shape, batch 1, 4096-byte prompt: every pass
    of the first block and the second block's first pass (the last prompt
    row rolled back to its causal latent and recomputed with the block's
    committed bytes in front of the new block)."""
    wl = bltgen.WORKLOADS[1]
    gold = _gold(wl)
    fb = FullBatch(wl)
    worst, comp, skip = 0.0, 0, 0
    try:
        assert len(gold[0]) >= 5 and int(gold[0][4]["n_append"]) > 1      # reaches block 2
        for k in range(len(gold[0])):
            rec = gold[0][k]
            assert int(rec["kind"]) == BLOCK
            z, am, cf, blk, left = fb.block_pass_rec(rec, wl.alpha, False)
            err, c, sk = check_block_pass(k, rec, z[0], am[0], cf[0], blk[0], left[0], wl.alpha, False, "bf16")
            worst, comp, skip = max(worst, err), comp + c, skip + sk
    finally:
        fb.close()
    _summary(wl.name, worst, comp, skip)


def test_fullsize_bltd16_batch16_first_passes():
    """BLT-D-16, alpha 0.9, batch 16: the first two passes of the first block
    of all 16 sequences, sequences 0 and 15 against the oracle."""
    wl = bltgen.WORKLOADS[2]
    gold = _gold(wl)
    fb = FullBatch(wl)
    worst, comp, skip = 0.0, 0, 0
    try:
        for k in range(len(gold[0])):
            forced = {s: gold[s][k]["block_before"] for s in gold}
            z, am, cf, blk, left = fb.block_pass(k == 0, forced, wl.alpha, False)
            for s in gold:
                rec = gold[s][k]
                err, c, sk = check_block_pass(k, rec, z[s], am[s], cf[s], blk[s], left[s], wl.alpha,
                                              False, "bf16")
                worst, comp, skip = max(worst, err), comp + c, skip + sk
    finally:
        fb.close()
    _summary(wl.name, worst, comp, skip)


def test_fullsize_blts8_batch1_first_round():
    """BLT-S k=8, batch 1: the eight draft passes (stale latents past the
    patch boundary) and the causal verification pass of the first two
    rounds (the second starts from the accepted bytes and the appended one)."""
    wl = bltgen.WORKLOADS[3]
    gold = _gold(wl)
    fb = FullBatch(wl)
    worst, comp, skip = 0.0, 0, 0
    try:
        assert len(gold[0]) == 18 and int(gold[0][17]["kind"]) == VERIFY
        for k, rec in enumerate(gold[0]):
            assert int(rec["kind"]) in (DRAFT, VERIFY)
            z, am = fb.rows_pass({0: (rec["start"], rec["tokens"], rec["targets"])}, None)
            err, c, sk = check_rows_pass(k, rec, z[0], am[0], "bf16")
            worst, comp, skip = max(worst, err), comp + c, skip + sk
    finally:
        fb.close()
    _summary(wl.name, worst, comp, skip)


def test_fullsize_bltdv8_batch64_first_round():
    """BLT-DV-8 one-step at the larger decoder (d 1536, 24 heads), batch 64,
    8192-byte prompts: the one-step draft pass and the verification pass of
    all 64 sequences, sequences 0, 21, 42 and 63 against the oracle."""
    wl = bltgen.WORKLOADS[4]
    gold = _gold(wl)
    fb = FullBatch(wl)
    worst, comp, skip = 0.0, 0, 0
    try:
        rec0 = {s: gold[s][0] for s in gold}
        assert all(int(r["kind"]) == BLOCK for r in rec0.values())
        z, am, cf, blk, left = fb.block_pass(True, {s: r["block_before"] for s, r in rec0.items()},
                                             wl.alpha, True)
        for s, rec in rec0.items():
            err, c, sk = check_block_pass(0, rec, z[s], am[s], cf[s], blk[s], left[s], wl.alpha, True, "bf16")
            worst, comp, skip = max(worst, err), comp + c, skip + sk
        rec1 = {s: gold[s][1] for s in gold}
        assert all(int(r["kind"]) == VERIFY for r in rec1.values())
        z, am = fb.rows_pass({s: (r["start"], r["tokens"], r["targets"]) for s, r in rec1.items()},
                             lambda s: fb.verify_rows(s, blk[s]))
        for s, rec in rec1.items():
            err, c, sk = check_rows_pass(1, rec, z[s], am[s], "bf16")
            worst, comp, skip = max(worst, err), comp + c, skip + sk
    finally:
        fb.close()
    _summary(wl.name, worst, comp, skip)


@pytest.mark.parametrize("key", ["long_fp32", "long_bf16"])
def test_max_context_first_block(key):
    """Prompts that fill the cache's 16384 rows (128 attention chunks, the
    most the merge takes): every pass of the first block, float32 tiny
    decoder (BLT-D-4, threshold) and 2-layer bfloat16 decoder (BLT-D-16, one
    step, the MFMA path), teacher-forced from the oracle."""
    wl = _golden_plan().LONG[key]
    assert wl.max_ctx > 16256 and wl.max_ctx <= 16384
    gold = _gold(wl)
    w = bltgen.make_weights(wl)
    inp = bltgen.make_sequence_inputs(wl, 0)
    dec = decoder_for(wl, w, max_batch=1, max_rows=1024)
    dtype = "fp32" if wl.dtype == "fp32" else "bf16"
    try:
        worst, comp, skip = replay_and_compare(dec, wl, inp, _as_run(gold[0]), wl.alpha,
                                               wl.unmask == "one_step", dtype)
    finally:
        dec.close()
    _summary(wl.name, worst, comp, skip)
