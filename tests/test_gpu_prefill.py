"""GPU parity of long clean-row passes (prompt prefill, KV rebuild) and of the
split-K decode attention at each chunk count per workgroup, against the CPU
oracle.

A bf16 sequence with at least 64 clean rows in a pass takes the causal
(flash) attention kernel; shorter ones and block passes take the split-K
kernel.  These tests append ragged runs of rows (tiles of 64 with a partial
last tile, a cached prefix before the run, two sequences of different lengths
in one pass, and a pass that mixes both kernels), with the causal kernel in
each of its forms (four waves, or two key groups whose softmax states join
at the end), and compare every row's
logits with the float64 oracle's cached decoder (bf16 tolerance: 2e-2
absolute), and every greedy byte whose oracle top-2 gap is outside the
rounding band.

The split-K kernel walks one or more chunks of 128 keys per workgroup (all
of a sequence's chunks, with the output written directly and no merge, when
one workgroup covers them); the last test forces several counts on short
appends after contexts whose chunk counts are not multiples of them (one
sequence shorter than a whole workgroup's span), with 1 to 9 rows per
sequence whose key counts differ.  The last test takes a batch wide enough
(sequences x heads = 256) for the eight-wave workgroup per (sequence, head),
with ragged contexts and appends.
"""
import numpy as np
import pytest

import bltgen
from oracle import cache, patcher
from tests.gpu_util import BF16_ABS, decoder_for, logits_ok, oracle_inputs, say

pytestmark = pytest.mark.gpu

MINI = bltgen.WORKLOADS[1].replace(name="mini_prefill_bf16", n_layers=2, d_model=256, n_heads=4,
                                   d_ffn=1024, d_global=512, prompt_len=600, prompt_patches=150,
                                   n_gen=8, block=4, batch=2)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    import block_diffusion_byte_amd as blt
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    blt.lib()
    yield


class _Seq:
    """One sequence: its oracle cached decoder, bytes and causal targets."""

    def __init__(self, wl, w, s):
        W, inp, inp64 = oracle_inputs(wl, w, seq=s)
        self.inp = inp
        self.x = [int(b) for b in inp["prompt"]]
        patch, ends = patcher.segment(self.x, inp["prompt_patches"], inp["salt"])
        self.tau = [patcher.causal_target(patch, ends, i) for i in range(len(self.x) - 1)]
        self.oracle = cache.CachedDecoder(W, wl, inp64["latents"], len(self.x) + 8)

    def expect(self, start, n):
        return self.oracle.run(self.x[start:start + n], start, self.tau[start:start + n], n)


def _check(got, ref, tag):
    ok, err, tol = logits_ok(got, ref, "bf16")
    # greedy bytes wherever the oracle's top-2 gap clears twice the tolerance
    top2 = np.sort(ref[:, :256], axis=1)[:, -2:]
    sure = (top2[:, 1] - top2[:, 0]) > 2 * BF16_ABS
    am_ref = np.argmax(ref[:, :256], axis=1)
    am_got = np.argmax(got[:, :256], axis=1)
    say(f"{tag}: {len(ref)} rows, worst logit err {err:.3g} (tol {tol:.3g}), "
        f"{int(sure.sum())} greedy bytes compared")
    assert ok, f"{tag}: logits err {err} > {tol}"
    assert np.array_equal(am_ref[sure], am_got[sure]), tag


def _append(blt, torch, dec, seqs, plan, z):
    """One kv_append pass: plan = [(slot, start, n)]; returns per-slot logits."""
    n_max = max(n for _, _, n in plan)
    slots = [s for s, _, _ in plan]
    lat = np.zeros((len(plan), n_max), dtype=np.int64)
    byt = np.zeros((len(plan), n_max), dtype=np.int64)
    for i, (s, st, n) in enumerate(plan):
        lat[i, :n] = seqs[s].tau[st:st + n]
        byt[i, :n] = seqs[s].x[st:st + n]
    blt.blt_kv_append(dec.ctx, dec.state, slots, [st for _, st, _ in plan], [n for _, _, n in plan],
                      n_max, lat, bytes_=byt, logits_out=z)
    torch.cuda.synchronize()
    out = {}
    for s, st, n in plan:
        base = s * n_max
        out[s] = z[base * 257:(base + n) * 257].view(n, 257).cpu().numpy().astype(np.float64)
    return out


@pytest.mark.parametrize("groups", [0, 1, 2])
def test_causal_kernel_ragged_tiles_prefix_and_mixed_passes(groups):
    """groups: the causal kernel's form (0: chosen per pass, 1: four waves
    over every key tile, 2: two key groups of four waves)."""
    import torch
    import block_diffusion_byte_amd as blt
    wl = MINI
    w = bltgen.make_weights(wl, gains="random")
    seqs = [_Seq(wl, w, s) for s in range(2)]
    dec = decoder_for(wl, w, max_batch=2, max_rows=512)
    try:
        blt.blt_flash_key_groups(dec.ctx, groups)
        for s in range(2):
            table = torch.from_numpy(seqs[s].inp["latents"]).to("cuda:0", dec.torch_dtype)
            blt.blt_latents_put(dec.ctx, dec.state, [s] * wl.n_latents, list(range(wl.n_latents)),
                                table, 0)
        z = torch.zeros(2 * 512 * 257, device="cuda:0")
        # pass 1: both sequences on the causal kernel, 150 rows (two full
        # tiles and a partial one) and 70 rows (one full tile and 6 rows)
        got = _append(blt, torch, dec, seqs, [(0, 0, 150), (1, 0, 70)], z)
        _check(got[0], seqs[0].expect(0, 150), "seq 0 rows 0..149 (causal kernel)")
        _check(got[1], seqs[1].expect(0, 70), "seq 1 rows 0..69 (causal kernel)")
        # pass 2: 229 rows after a 150-row prefix (causal kernel) beside
        # 10 rows of the other sequence (split-K kernel) in the same pass
        got = _append(blt, torch, dec, seqs, [(0, 150, 229), (1, 70, 10)], z)
        _check(got[0], seqs[0].expect(150, 229), "seq 0 rows 150..378 after a prefix (causal kernel)")
        _check(got[1], seqs[1].expect(70, 10), "seq 1 rows 70..79 (split-K kernel, mixed pass)")
        # pass 3: exactly one tile; then a rollback that rewrites the tail
        got = _append(blt, torch, dec, seqs, [(1, 80, 64)], z)
        _check(got[1], seqs[1].expect(80, 64), "seq 1 rows 80..143 (one full tile)")
        seqs[0].oracle.truncate(300)
        got = _append(blt, torch, dec, seqs, [(0, 300, 299)], z)
        _check(got[0], seqs[0].expect(300, 299), "seq 0 rows 300..598 after truncation to 300")
        # pass 5: 100 rows after a 40-row prefix: the first wave's rows read
        # 41..72 keys, so the second key group's first tile (keys 64..127)
        # lies wholly past the kend of some of them
        seqs[1].oracle.truncate(40)
        got = _append(blt, torch, dec, seqs, [(1, 40, 100)], z)
        _check(got[1], seqs[1].expect(40, 100), "seq 1 rows 40..139 after truncation to 40")
        with pytest.raises(blt.BltError):
            blt.blt_flash_key_groups(dec.ctx, 3)
    finally:
        dec.close()


def test_causal_kernel_matches_split_k_pass_by_pass():
    """The same rows through both kernels (one 200-row pass vs passes of 50
    rows): the logits agree within the bf16 tolerance."""
    import torch
    import block_diffusion_byte_amd as blt
    wl = MINI
    w = bltgen.make_weights(wl, gains="random")
    seqs = [_Seq(wl, w, 0)]
    res = []
    for chunk in (200, 50):
        dec = decoder_for(wl, w, max_batch=2, max_rows=256)
        try:
            table = torch.from_numpy(seqs[0].inp["latents"]).to("cuda:0", dec.torch_dtype)
            blt.blt_latents_put(dec.ctx, dec.state, [0] * wl.n_latents, list(range(wl.n_latents)),
                                table, 0)
            z = torch.zeros(2 * 256 * 257, device="cuda:0")
            parts = [_append(blt, torch, dec, seqs, [(0, c0, chunk)], z)[0] for c0 in range(0, 200, chunk)]
            res.append(np.concatenate(parts))
        finally:
            dec.close()
    err = np.abs(res[0] - res[1]).max()
    say(f"causal kernel vs split-K over 200 rows: max logit difference {err:.3g}")
    assert err <= BF16_ABS


LONG = MINI.replace(name="mini_chunks_bf16", prompt_len=1400, prompt_patches=350, batch=3)


def test_split_k_chunks_per_workgroup_match_the_oracle():
    """Appends of 9, 1 and 6 rows after 700-, 1030- and 1385-byte contexts
    (6, 9 and 12 chunks of keys) with 1, 3, 4, 8 and 64 chunks per workgroup
    (64: one workgroup per sequence and head, no merge), and the default
    choice: every row's logits match the oracle, and the counts
    agree with each other within the same bf16 tolerance (the attention
    output is rounded to bfloat16, so a different summation order can move
    it by one bf16 step, and the logits by a few thousandths)."""
    import torch
    import block_diffusion_byte_amd as blt
    wl = LONG
    w = bltgen.make_weights(wl, gains="random")
    seqs = [_Seq(wl, w, s) for s in range(3)]
    ctx = [700, 1030, 1385]
    n_new = [9, 1, 6]
    dec = decoder_for(wl, w, max_batch=3, max_rows=1400)
    try:
        for s in range(3):
            table = torch.from_numpy(seqs[s].inp["latents"]).to("cuda:0", dec.torch_dtype)
            blt.blt_latents_put(dec.ctx, dec.state, [s] * wl.n_latents, list(range(wl.n_latents)),
                                table, 0)
        z = torch.zeros(3 * 1400 * 257, device="cuda:0")
        for s in range(3):   # contexts through the causal kernel, one sequence at a time
            _append(blt, torch, dec, seqs, [(s, 0, ctx[s])], z)
            seqs[s].expect(0, ctx[s])
        ref = {s: seqs[s].expect(ctx[s], n_new[s]) for s in range(3)}
        plan = [(s, ctx[s], n_new[s]) for s in range(3)]
        got = {}
        for chunks in (1, 3, 4, 8, 64, 0):
            blt.blt_attention_chunks(dec.ctx, chunks)
            got[chunks] = _append(blt, torch, dec, seqs, plan, z)   # rewrites the same rows
            for s in range(3):
                _check(got[chunks][s], ref[s], f"{chunks} chunks per workgroup, seq {s}")
        for chunks in (3, 4, 8, 64, 0):
            err = max(np.abs(got[chunks][s] - got[1][s]).max() for s in range(3))
            say(f"{chunks} vs 1 chunks per workgroup: max logit difference {err:.3g}")
            assert err <= BF16_ABS
        with pytest.raises(blt.BltError):
            blt.blt_attention_chunks(dec.ctx, -1)
    finally:
        dec.close()


WIDE = MINI.replace(name="mini_wide_bf16", d_model=512, n_heads=8, prompt_len=900, prompt_patches=225,
                    batch=32)


def test_eight_wave_attention_ragged_batch_matches_the_oracle():
    """32 sequences x 8 heads (256 pairs): a split-K pass of more than 1024
    chunks in all takes one eight-wave workgroup per (sequence, head) with
    the output written directly.  Contexts of 260..880 bytes (3 to 7 chunks,
    odd and even counts, so the two wave groups get unequal shares) and
    appends of 1 to 9 rows: every row's logits match the oracle, and agree
    with one chunk per workgroup (partials and the merge kernel) within the
    same bf16 tolerance; graph replays of the pass match it exactly."""
    import torch
    import block_diffusion_byte_amd as blt
    wl = WIDE
    w = bltgen.make_weights(wl, gains="random")
    n = wl.batch
    seqs = [_Seq(wl, w, s) for s in range(n)]
    ctx = [260 + 20 * s for s in range(n)]
    n_new = [1 + s % 9 for s in range(n)]
    dec = decoder_for(wl, w, max_batch=n, max_rows=max(ctx))
    try:
        for s in range(n):
            table = torch.from_numpy(seqs[s].inp["latents"]).to("cuda:0", dec.torch_dtype)
            blt.blt_latents_put(dec.ctx, dec.state, [s] * wl.n_latents, list(range(wl.n_latents)),
                                table, 0)
        z = torch.zeros(n * max(ctx) * 257, device="cuda:0")
        for s in range(n):   # contexts through the causal kernel, one sequence at a time
            _append(blt, torch, dec, seqs, [(s, 0, ctx[s])], z)
            seqs[s].expect(0, ctx[s])
        ref = {s: seqs[s].expect(ctx[s], n_new[s]) for s in range(n)}
        plan = [(s, ctx[s], n_new[s]) for s in range(n)]
        got = {}
        for chunks in (0, 1):   # the shape's own choice (eight waves), then one chunk
            blt.blt_attention_chunks(dec.ctx, chunks)
            got[chunks] = _append(blt, torch, dec, seqs, plan, z)   # rewrites the same rows
            for s in range(n):
                _check(got[chunks][s], ref[s], f"{chunks} chunks per workgroup, seq {s}")
        err = max(np.abs(got[0][s] - got[1][s]).max() for s in range(n))
        say(f"eight-wave vs one chunk per workgroup: max logit difference {err:.3g}")
        assert err <= BF16_ABS
        # graph capture and replay of the same pass (its chunk grid rounded
        # up to a bucket) reproduce the direct launch bit for bit
        blt.blt_attention_chunks(dec.ctx, 0)
        blt.blt_graphs_enable(dec.ctx, True)
        for rep in range(3):     # direct, captured, replayed
            again = _append(blt, torch, dec, seqs, plan, z)
            for s in range(n):
                assert np.array_equal(again[s], got[0][s]), (rep, s)
        blt.blt_graphs_enable(dec.ctx, False)
    finally:
        dec.close()
