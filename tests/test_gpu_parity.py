"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

Teacher-forced replays run every pass of an oracle trace on the GPU from the
oracle's own state (same rows, same block tokens) and compare logits within
the tolerance of the path (fp32: 1e-4 relative to the row's largest logit;
bf16: 2e-2 absolute) and every decision whose oracle margin is outside the
rounding band.  Session tests run the native decode drivers free-running and
compare bytes and pass counts exactly (fp32) or against the GPU itself
(BLT-S must reproduce greedy decoding byte for byte).
"""
import numpy as np
import pytest

import bltgen
from oracle import loops
from tests.gpu_util import assert_coverage, decoder_for, oracle_inputs, replay_and_compare, say

pytestmark = pytest.mark.gpu

MINI_BF16 = bltgen.WORKLOADS[1].replace(n_layers=2, d_model=256, n_heads=4, d_ffn=1024,
                                        d_global=512, prompt_len=300, prompt_patches=80,
                                        n_gen=40, block=4)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    import block_diffusion_byte_amd as blt
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    blt.lib()
    yield


def _replay(wl, policy, n_gen, gains="random", floor=None, **kw):
    w = bltgen.make_weights(wl, gains=gains)
    W, inp, inp64 = oracle_inputs(wl, w)
    if policy == "blt_d":
        run = loops.blt_d(W, wl, inp64, n_gen, kw["B"], kw["alpha"], kw.get("one_step", False),
                          kw.get("causal", False), trace=True, unmask=kw.get("unmask"))
    elif policy == "blt_s":
        run = loops.blt_s(W, wl, inp64, n_gen, kw["k"], trace=True)
    elif policy == "blt_dv":
        run = loops.blt_dv(W, wl, inp64, n_gen, kw["B"], kw["alpha"], kw.get("one_step", True),
                           trace=True)
    else:
        run = loops.greedy(W, wl, inp64, n_gen, trace=True)
    wl2 = wl.replace(block=max(wl.block, kw.get("B", 0), kw.get("k", 0)))
    dec = decoder_for(wl2, w, max_batch=1, max_rows=64)
    try:
        worst, comp, skip = replay_and_compare(dec, wl2, inp, run, kw.get("alpha", 0.0),
                                               kw.get("unmask") or kw.get("one_step", policy == "blt_dv"),
                                               wl.dtype)
    finally:
        dec.close()
    say(f"{wl.name} {policy}: {len(run.passes)} passes, worst logit err {worst:.3g}, "
        f"{comp} decisions compared, {skip} near-ties skipped")
    if floor is None:
        assert_coverage(f"{wl.name} {policy}", comp, skip)
    else:
        assert_coverage(f"{wl.name} {policy}", comp, skip, floor)
    return worst


def test_tiny_fp32_blt_d_teacher_forced():
    wl = bltgen.WORKLOADS[0]
    _replay(wl, "blt_d", wl.n_gen, B=4, alpha=0.7)


def test_tiny_fp32_blt_d_causal_block_teacher_forced():
    wl = bltgen.WORKLOADS[0]
    _replay(wl, "blt_d", 24, B=4, alpha=0.7, causal=True)


def test_tiny_fp32_peaked_multi_commit_teacher_forced():
    wl = bltgen.WORKLOADS[0].replace(head_scale=12.0)
    _replay(wl, "blt_d", 48, gains="ones", B=4, alpha=0.7)


def test_tiny_fp32_blt_s_teacher_forced():
    wl = bltgen.WORKLOADS[0]
    _replay(wl, "blt_s", 32, k=8)


def test_tiny_fp32_blt_dv_teacher_forced():
    wl = bltgen.WORKLOADS[0]
    _replay(wl, "blt_dv", 24, B=8, alpha=0.7, one_step=True)


def test_mini_bf16_block16_mfma_teacher_forced():
    # 16 block rows plus the appended clean rows: the projections run on MFMA
    wl = MINI_BF16.replace(block=16, alpha=0.9)
    _replay(wl, "blt_d", 32, B=16, alpha=0.9)


def test_mini_bf16_blt_s_teacher_forced():
    _replay(MINI_BF16, "blt_s", 24, k=8)


def test_mini_bf16_blt_dv_teacher_forced():
    wl = MINI_BF16.replace(block=8)
    _replay(wl, "blt_dv", 24, B=8, alpha=0.7, one_step=True)


def test_mini_bf16_multi_commit_unscaled_head_teacher_forced():
    """Passes that commit several block positions with the byte head as
    stated (no scaling), so the logits are held to the plain 2e-2 bf16 bound:
    the threshold rule at alpha 0.005 (every confidence of this decoder,
    0.008-0.011, lies above it: four commits per pass) and entropy-bounded
    unmasking with gamma 12 nats (entropies ~5.5: two of eight per pass)."""
    _replay(MINI_BF16, "blt_d", 24, B=4, alpha=0.005)
    _replay(MINI_BF16.replace(block=8), "blt_d", 24, B=8, alpha=12.0, unmask="entropy")


@pytest.mark.parametrize("dtype,d_model,n_heads", [("bf16", 256, 2), ("bf16", 256, 8),
                                                   ("fp32", 128, 2), ("fp32", 256, 2)])
def test_head_widths_teacher_forced(dtype, d_model, n_heads):
    """Head widths 128, 32 (bf16) and 64, 128 (f32) besides the workloads'
    64 (bf16) and 32 (f32): the cache's K tiles hold 4, 1 and 2 slices of
    32 dimensions, the causal prefill kernel takes 32-key tiles at d_h 128,
    and the split-K kernels their one-chunk forms.  The 300-byte prompt is
    prefilled by the causal kernel (bf16) and every later pass reads the
    cache through the split-K kernels, over ten blocks.  Every row's logits
    are held to the path's bound; of the argmax decisions at least 60% must
    lie outside the rounding band and be compared (this random two-head
    decoder at d_h 128 leaves 67%, the workloads' decoders 70% or more)."""
    base = MINI_BF16 if dtype == "bf16" else bltgen.WORKLOADS[0]
    wl = base.replace(name=f"{dtype}_dh{d_model // n_heads}", d_model=d_model, n_heads=n_heads,
                      prompt_len=300, prompt_patches=80)
    _replay(wl, "blt_d", 40, B=4, alpha=0.7, floor=0.6)


def test_tiny_fp32_entropy_bounded_teacher_forced():
    """Entropy-bounded unmasking (gamma 4 nats, B 8, peaked head: passes
    commit 1 to 5 positions), float32 GEMV path."""
    wl = bltgen.WORKLOADS[0].replace(head_scale=12.0)
    _replay(wl, "blt_d", 32, B=8, alpha=4.0, unmask="entropy")


def test_mini_bf16_entropy_bounded_block16_teacher_forced():
    """Entropy-bounded unmasking, B 16 on the bf16 MFMA path."""
    wl = MINI_BF16.replace(head_scale=12.0, block=16)
    _replay(wl, "blt_d", 32, B=16, alpha=4.0, unmask="entropy")


# ---------------------------------------------------------------- sessions
def _session(wl, w, inps, policy, n_gen, block, alpha, unmask=0, mask=0, max_rows=64,
             graphs=True, repeats=1, between=None, device=False):
    """Run a native decode session; with repeats > 1 the generation is rerun
    from the same prefill (calling `between` in between) and every run's
    results are returned."""
    import torch
    import block_diffusion_byte_amd as blt
    dec = decoder_for(wl.replace(block=block), w, max_batch=len(inps), max_rows=max_rows)
    blt.blt_graphs_enable(dec.ctx, graphs)
    table = torch.from_numpy(np.stack([i["latents"] for i in inps])).to("cuda:0", dec.torch_dtype)
    sess = blt.blt_session_create(dec.ctx, dec.state, [i["prompt"] for i in inps],
                                  [i["prompt_patches"] for i in inps], [i["salt"] for i in inps],
                                  table, wl.n_latents)
    runs = []
    try:
        if device:
            blt.blt_session_device_blocks(dec.ctx, sess, int(device))
        blt.blt_session_prefill(dec.ctx, sess)
        for k in range(repeats):
            if k and between:
                between()
            blt.blt_session_generate(dec.ctx, sess, policy, block, alpha, n_gen, unmask, mask)
            runs.append([blt.blt_session_result(sess, b, n_gen) for b in range(len(inps))])
    finally:
        blt.blt_session_destroy(sess)
        dec.close()
    return runs if repeats > 1 else runs[0]


@pytest.mark.parametrize("block", [4, 16])
def test_graph_replays_match_direct_launches(block):
    """Passes replayed from cached HIP graphs (GEMV path at block 4, MFMA path
    at block 16) give the same bytes and counts as direct launches, on every
    rerun, with unrelated eager GPU work and synchronisations in between."""
    import torch
    import block_diffusion_byte_amd as blt
    wl = MINI_BF16.replace(head_scale=12.0)
    w = bltgen.make_weights(wl)
    inps = [bltgen.make_sequence_inputs(wl, b) for b in range(2)]

    def eager_work():
        x = torch.randn(512, 512, device="cuda:0")
        (x @ x).sum().item()
        torch.cuda.synchronize()

    ref = _session(wl, w, inps, blt.BLT_POLICY_BLT_D, 40, block, 0.5, graphs=False)
    runs = _session(wl, w, inps, blt.BLT_POLICY_BLT_D, 40, block, 0.5, graphs=True, repeats=4,
                    between=eager_work)
    for k, got in enumerate(runs):
        for b in range(len(inps)):
            assert got[b]["out"] == ref[b]["out"], f"run {k} seq {b}: bytes differ"
            assert (got[b]["n_dec"], got[b]["n_eg"]) == (ref[b]["n_dec"], ref[b]["n_eg"])
    say(f"block {block}: 4 graph runs identical to direct launches, n_dec {[r['n_dec'] for r in ref]}")


@pytest.mark.parametrize("policy", ["greedy", "blt_d", "blt_s", "blt_dv"])
def test_tiny_fp32_sessions_match_oracle_exactly(policy):
    import block_diffusion_byte_amd as blt
    wl = bltgen.WORKLOADS[0]
    w = bltgen.make_weights(wl, gains="random")
    n_gen = 40
    inps, refs = [], []
    for seq in range(3):
        W, inp, inp64 = oracle_inputs(wl, w, seq)
        inps.append(inp)
        if policy == "greedy":
            refs.append(loops.greedy(W, wl, inp64, n_gen))
        elif policy == "blt_d":
            refs.append(loops.blt_d(W, wl, inp64, n_gen, 4, 0.7))
        elif policy == "blt_s":
            refs.append(loops.blt_s(W, wl, inp64, n_gen, 8))
        else:
            refs.append(loops.blt_dv(W, wl, inp64, n_gen, 8, 0.7, one_step=True))
    pid = {"greedy": blt.BLT_POLICY_GREEDY, "blt_d": blt.BLT_POLICY_BLT_D,
           "blt_s": blt.BLT_POLICY_BLT_S, "blt_dv": blt.BLT_POLICY_BLT_DV}[policy]
    block = {"greedy": 1, "blt_d": 4, "blt_s": 8, "blt_dv": 8}[policy]
    unmask = blt.BLT_UNMASK_ONE_STEP if policy == "blt_dv" else blt.BLT_UNMASK_THRESHOLD
    got = _session(wl, w, inps, pid, n_gen, block, 0.7, unmask)
    for b, (g, r) in enumerate(zip(got, refs)):
        assert list(g["out"]) == r.out, f"seq {b}: bytes differ"
        assert (g["n_dec"], g["n_eg"]) == (r.n_dec, r.n_eg), f"seq {b}: counts differ"
        if r.accept:
            assert g["rounds"] == len(r.accept) and g["accepted"] == sum(r.accept)
    say(f"{policy}: 3 sequences x {n_gen} bytes identical; n_dec {[g['n_dec'] for g in got]}")


# (policy, block or draft window, alpha or entropy bound, unmask, causal block mask, head scale)
EDGE_BLOCKS = {
    "blt_d_b1": ("blt_d", 1, 0.7, "threshold", False, 1.0),
    "blt_d_b1_causal": ("blt_d", 1, 0.7, "threshold", True, 1.0),
    "blt_d_b64": ("blt_d", 64, 0.7, "threshold", False, 1.0),
    "blt_d_b64_causal_one_step": ("blt_d", 64, 0.7, "one_step", True, 1.0),
    "blt_d_b64_entropy_peaked": ("blt_d", 64, 10.0, "entropy", False, 12.0),
    "blt_s_k1": ("blt_s", 1, 0.0, "threshold", False, 1.0),
    "blt_dv_b1": ("blt_dv", 1, 0.7, "one_step", False, 1.0),
    "blt_dv_b64": ("blt_dv", 64, 0.7, "one_step", False, 1.0),
}


@pytest.mark.parametrize("case", sorted(EDGE_BLOCKS))
def test_tiny_fp32_degenerate_and_largest_blocks_match_oracle(case):
    """The smallest and the largest block / draft window (1 and 64 positions,
    the most one unmask wave takes) in native sessions: bytes, decoder and
    encoder/global passes, rounds and accepted bytes equal the oracle's
    (pytorch.kr summary, "BLT-D inference", "BLT-S and BLT-DV").  With 40
    bytes to generate, a 64-position block over-fills the generation and is
    truncated after its passes are counted; with B = 1 every pass commits
    its one position.  The entropy-bounded case takes the peaked head
    (x12), whose entropies are spread far beyond float32 rounding, so every
    ranking of the 64 positions is decided.  The latent tables and caches
    are sized for 40 + 2 x 64 bytes, as a drafted block past the 40 bytes
    completes patches of its own."""
    import block_diffusion_byte_amd as blt
    policy, B, alpha, unmask, causal, scale = EDGE_BLOCKS[case]
    n_gen = 40
    wl = bltgen.WORKLOADS[0].replace(block=B, n_gen=n_gen + 2 * B, head_scale=scale)
    w = bltgen.make_weights(wl, gains="random")
    inps, refs = [], []
    for seq in range(3):
        W, inp, inp64 = oracle_inputs(wl, w, seq)
        inps.append(inp)
        if policy == "blt_d":
            refs.append(loops.blt_d(W, wl, inp64, n_gen, B, alpha, block_causal=causal, unmask=unmask))
        elif policy == "blt_s":
            refs.append(loops.blt_s(W, wl, inp64, n_gen, B))
        else:
            refs.append(loops.blt_dv(W, wl, inp64, n_gen, B, alpha, unmask=unmask))
    pid = {"blt_d": blt.BLT_POLICY_BLT_D, "blt_s": blt.BLT_POLICY_BLT_S, "blt_dv": blt.BLT_POLICY_BLT_DV}[policy]
    um = {"threshold": blt.BLT_UNMASK_THRESHOLD, "one_step": blt.BLT_UNMASK_ONE_STEP,
          "entropy": blt.BLT_UNMASK_ENTROPY}[unmask]
    mask = blt.BLT_BLOCK_CAUSAL if causal else blt.BLT_BLOCK_BIDIR
    got = _session(wl, w, inps, pid, n_gen, B, alpha, um, mask, max_rows=3 * (2 * B + 2))
    for b, (g, r) in enumerate(zip(got, refs)):
        assert list(g["out"]) == r.out, f"seq {b}: bytes differ"
        assert (g["n_dec"], g["n_eg"]) == (r.n_dec, r.n_eg), f"seq {b}: counts differ"
        if r.accept:
            assert g["rounds"] == len(r.accept) and g["accepted"] == sum(r.accept)
    say(f"{case}: 3 sequences x {n_gen} bytes identical; n_dec {[g['n_dec'] for g in got]}")


@pytest.mark.parametrize("dmode", [1, 3])
@pytest.mark.parametrize("case", ["threshold", "peaked", "entropy", "one_step", "causal"])
def test_tiny_fp32_device_blocks_match_oracle_exactly(case, dmode):
    """BLT-D with every block after the first planned, decoded, committed and
    patched on the device (one captured graph per block, one readback at the
    end): 3 sequences, bytes and decoder / encoder-global pass counts equal
    to the oracle's, for the threshold rule (one commit per pass), the peaked
    head (several commits per pass, so later passes of a block do no work),
    entropy-bounded and one-step unmasking, and the causal block mask.  Device
    mode 3 runs the same with the streaming kernels testing the gate only before
    their stores: the passes of a block that no longer needs them (peaked,
    entropy, one-step) load and compute and must store nothing."""
    import block_diffusion_byte_amd as blt
    wl = bltgen.WORKLOADS[0]
    B, alpha, unmask, mode, causal = 4, 0.7, None, blt.BLT_UNMASK_THRESHOLD, False
    if case in ("peaked", "entropy"):
        wl = wl.replace(head_scale=12.0)
    if case == "entropy":
        B, alpha, unmask, mode = 8, 4.0, "entropy", blt.BLT_UNMASK_ENTROPY
    if case == "one_step":
        unmask, mode = "one_step", blt.BLT_UNMASK_ONE_STEP
    if case == "causal":
        causal = True
    w = bltgen.make_weights(wl, gains="random")
    n_gen = 40
    inps, refs = [], []
    for seq in range(3):
        W, inp, inp64 = oracle_inputs(wl, w, seq)
        inps.append(inp)
        refs.append(loops.blt_d(W, wl, inp64, n_gen, B, alpha, block_causal=causal, unmask=unmask))
    got = _session(wl, w, inps, blt.BLT_POLICY_BLT_D, n_gen, B, alpha, mode,
                   blt.BLT_BLOCK_CAUSAL if causal else blt.BLT_BLOCK_BIDIR, device=dmode)
    for b, (g, r) in enumerate(zip(got, refs)):
        assert list(g["out"]) == r.out, f"seq {b}: bytes differ"
        assert (g["n_dec"], g["n_eg"]) == (r.n_dec, r.n_eg), f"seq {b}: counts differ"
    say(f"device blocks mode {dmode} ({case}): 3 x {n_gen} bytes identical to the oracle; "
        f"n_dec {[g['n_dec'] for g in got]}")


@pytest.mark.parametrize("case", ["threshold", "peaked"])
def test_tiny_fp32_auto_blocks_match_oracle_exactly(case):
    """Blocks driven by the driver's own choice (mode 2), one sequence per
    session: the first blocks run host-driven; with the threshold rule every
    pass commits one byte, so after four watched blocks the rest of the
    10-block generation runs device-resident; with the peaked head passes
    commit several bytes and the blocks stay host-driven.  Either way each of
    3 sequences' bytes and pass counts equal the oracle's; a mode outside 0..3
    is refused."""
    import block_diffusion_byte_amd as blt
    wl = bltgen.WORKLOADS[0]
    if case == "peaked":
        wl = wl.replace(head_scale=12.0)
    w = bltgen.make_weights(wl, gains="random")
    n_gen, B, alpha = 40, 4, 0.7
    inps, refs = [], []
    for seq in range(3):
        W, inp, inp64 = oracle_inputs(wl, w, seq)
        inps.append(inp)
        refs.append(loops.blt_d(W, wl, inp64, n_gen, B, alpha))
    got = [_session(wl, w, [inp], blt.BLT_POLICY_BLT_D, n_gen, B, alpha, device=2)[0] for inp in inps]
    for b, (g, r) in enumerate(zip(got, refs)):
        assert list(g["out"]) == r.out, f"seq {b}: bytes differ"
        assert (g["n_dec"], g["n_eg"]) == (r.n_dec, r.n_eg), f"seq {b}: counts differ"
    say(f"auto blocks ({case}): 3 x {n_gen} bytes identical to the oracle; n_dec {[g['n_dec'] for g in got]}")
    import torch
    dec = decoder_for(wl, w, max_batch=1, max_rows=64)
    try:
        table = torch.from_numpy(np.stack([inps[0]["latents"]])).to("cuda:0", dec.torch_dtype)
        sess = blt.blt_session_create(dec.ctx, dec.state, [inps[0]["prompt"]], [inps[0]["prompt_patches"]],
                                      [inps[0]["salt"]], table, wl.n_latents)
        try:
            with pytest.raises(blt.BltError):
                blt.blt_session_device_blocks(dec.ctx, sess, 4)
        finally:
            blt.blt_session_destroy(sess)
    finally:
        dec.close()


@pytest.mark.parametrize("mode", [1, 3])
@pytest.mark.parametrize("graphs", [True, False])
def test_bf16_device_blocks_equal_host_blocks(graphs, mode):
    """bfloat16 decoder, 2 sequences: the device-resident blocks give exactly
    the bytes and counts of the host-driven blocks (the recomputed prefix row
    reads the same latent through the same kernels, and a row's result does
    not depend on the rows beside it).  The peaked head commits several bytes
    per pass, so blocks end before their last passes: mode 3 runs those
    closed passes through the bf16 GEMVs and split-K attention that test the
    gate only before their stores, which must leave every result as mode 1
    and the host driver do."""
    import block_diffusion_byte_amd as blt
    wl = MINI_BF16.replace(head_scale=12.0)
    w = bltgen.make_weights(wl)
    inps = [bltgen.make_sequence_inputs(wl, b) for b in range(2)]
    host = _session(wl, w, inps, blt.BLT_POLICY_BLT_D, 40, 4, 0.5, graphs=graphs)
    dev = _session(wl, w, inps, blt.BLT_POLICY_BLT_D, 40, 4, 0.5, graphs=graphs, device=mode)
    for b in range(2):
        assert dev[b]["out"] == host[b]["out"], f"seq {b}: bytes differ"
        assert (dev[b]["n_dec"], dev[b]["n_eg"]) == (host[b]["n_dec"], host[b]["n_eg"])
    say(f"bf16 device blocks mode {mode} (graphs {graphs}) equal host blocks; n_dec {[r['n_dec'] for r in dev]}")


def test_tiny_fp32_entropy_bounded_session_exact():
    """The native BLT-D driver with entropy-bounded unmasking reproduces the
    oracle's bytes and pass counts exactly (3 sequences, gamma 4 nats)."""
    import block_diffusion_byte_amd as blt
    wl = bltgen.WORKLOADS[0].replace(head_scale=12.0)
    w = bltgen.make_weights(wl, gains="random")
    inps, refs = [], []
    for seq in range(3):
        W, inp, inp64 = oracle_inputs(wl, w, seq)
        inps.append(inp)
        refs.append(loops.blt_d(W, wl, inp64, 40, 8, 4.0, unmask="entropy"))
    got = _session(wl, w, inps, blt.BLT_POLICY_BLT_D, 40, 8, 4.0, blt.BLT_UNMASK_ENTROPY)
    for b, (g, r) in enumerate(zip(got, refs)):
        assert list(g["out"]) == r.out, f"seq {b}: bytes differ"
        assert (g["n_dec"], g["n_eg"]) == (r.n_dec, r.n_eg), f"seq {b}: counts differ"
    assert min(r.n_dec for r in refs) < 40
    say(f"EB sessions: n_dec {[g['n_dec'] for g in got]} for 40 bytes")


def test_tiny_fp32_peaked_session_multi_commit_exact():
    import block_diffusion_byte_amd as blt
    wl = bltgen.WORKLOADS[0].replace(head_scale=12.0)
    w = bltgen.make_weights(wl)
    W, inp, inp64 = oracle_inputs(wl, w)
    ref = loops.blt_d(W, wl, inp64, 48, 4, 0.7)
    got = _session(wl, w, [inp], blt.BLT_POLICY_BLT_D, 48, 4, 0.7)[0]
    assert list(got["out"]) == ref.out and (got["n_dec"], got["n_eg"]) == (ref.n_dec, ref.n_eg)
    assert ref.n_dec < 48
    say(f"peaked BLT-D: {ref.n_dec} passes for 48 bytes")


def test_blt_s_equals_greedy_on_gpu_full_size():
    """BLT-S with k=8 at the 1B-class decoder shape (4096-byte Zipf prompt,
    2048 bytes) reproduces greedy decoding byte for byte on the GPU."""
    import block_diffusion_byte_amd as blt
    wl = bltgen.WORKLOADS[3]
    w = bltgen.make_weights(wl)
    inp = bltgen.make_sequence_inputs(wl, 0)
    n_gen = wl.n_gen
    g = _session(wl, w, [inp], blt.BLT_POLICY_GREEDY, n_gen, 8, 0.0, max_rows=1024)[0]
    s = _session(wl, w, [inp], blt.BLT_POLICY_BLT_S, n_gen, 8, 0.0, max_rows=1024)[0]
    assert g["out"] == s["out"] and len(s["out"]) == n_gen
    assert g["n_dec"] == n_gen
    assert s["n_dec"] == s["rounds"] * 9 and s["n_eg"] == s["rounds"]
    say(f"BLT-S k=8: {n_gen} bytes identical to greedy; decoder passes {s['n_dec']} vs {g['n_dec']}, "
        f"encoder/global passes {s['n_eg']} vs {g['n_eg']}, mean accepted {s['accepted'] / s['rounds']:.2f}")


def test_row_result_does_not_depend_on_the_pass():
    """A row's logits are bit-identical whether it is appended alone or with
    eight other rows in one pass (GEMVs on MFMA and on dot products, split-K
    attention): the property BLT-S relies on to reproduce greedy decoding,
    checked directly at the 1B-class decoder width (d_model 1024, so every
    GEMV kernel of the batch-1 path runs)."""
    import torch
    import block_diffusion_byte_amd as blt
    wl = bltgen.WORKLOADS[1].replace(n_layers=2, prompt_len=160, prompt_patches=40, n_gen=8, block=4)
    w = bltgen.make_weights(wl, gains="random")
    inp = bltgen.make_sequence_inputs(wl, 0)
    lat = [min(i // 4, 39) for i in range(160)]
    outs = []
    for split in (False, True):
        dec = decoder_for(wl, w, max_batch=1, max_rows=160)
        try:
            table = torch.from_numpy(inp["latents"]).to("cuda:0", dec.torch_dtype)
            blt.blt_latents_put(dec.ctx, dec.state, [0] * 40, list(range(40)), table, 0)
            z = torch.zeros(160 * 257, device="cuda:0")
            # a 100-row prefix (causal kernel), then rows 100..108 in one pass or one by one
            blt.blt_kv_append(dec.ctx, dec.state, [0], [0], [100], 100, lat[:100],
                              bytes_=inp["prompt"][:100], logits_out=z)
            got = []
            starts = [(100 + j, 1) for j in range(9)] if split else [(100, 9)]
            for st, n in starts:
                blt.blt_kv_append(dec.ctx, dec.state, [0], [st], [n], n, lat[st:st + n],
                                  bytes_=inp["prompt"][st:st + n], logits_out=z)
                torch.cuda.synchronize()
                got.append(z[:n * 257].view(n, 257).cpu().numpy().copy())
            outs.append(np.concatenate(got))
        finally:
            dec.close()
    assert np.array_equal(outs[0], outs[1]), np.abs(outs[0] - outs[1]).max()
    say("9 rows in one pass vs one by one: logits bit-identical")


def test_pass_is_deterministic():
    import torch
    import block_diffusion_byte_amd as blt
    wl = MINI_BF16
    w = bltgen.make_weights(wl)
    inp = bltgen.make_sequence_inputs(wl, 0)
    outs = []
    for _ in range(2):
        dec = decoder_for(wl, w, max_batch=1, max_rows=64)
        table = torch.from_numpy(inp["latents"]).to("cuda:0", dec.torch_dtype)
        blt.blt_latents_put(dec.ctx, dec.state, [0] * 20, list(range(20)), table, 0)
        z = torch.zeros(64 * 257, device="cuda:0")
        blt.blt_kv_append(dec.ctx, dec.state, [0], [0], [40], 40, [min(i // 4, 19) for i in range(40)],
                          bytes_=inp["prompt"][:40], logits_out=z)
        torch.cuda.synchronize()
        outs.append(z.cpu().numpy())
        dec.close()
    assert np.array_equal(outs[0], outs[1])


def test_argument_errors_enqueue_nothing():
    import torch
    import block_diffusion_byte_amd as blt
    wl = bltgen.WORKLOADS[0]
    w = bltgen.make_weights(wl)
    dec = decoder_for(wl, w, max_batch=2, max_rows=16)
    bt = torch.full((8,), 256, dtype=torch.int32, device="cuda:0")
    ml = torch.zeros(2, dtype=torch.int32, device="cuda:0")
    try:
        cases = [
            (dict(B=5), blt.BLT_ECAPACITY),                        # B > max_block
            (dict(start=[wl.max_ctx - 2]), blt.BLT_ECAPACITY),     # block beyond max_ctx
            (dict(lat=[wl.n_latents]), blt.BLT_ECAPACITY),         # latent out of range
            (dict(slot=[0, 0], start=[0, 0], lat=[0, 0]), blt.BLT_EINVAL),  # duplicate slot
            (dict(alpha=float("nan")), blt.BLT_EINVAL),
        ]
        for kw, code in cases:
            with pytest.raises(blt.BltError) as ei:
                blt.blt_decode_block_step(dec.ctx, dec.state, kw.get("slot", [0]), kw.get("start", [0]),
                                          bt, kw.get("B", 4), kw.get("lat", [0]), kw.get("alpha", 0.7),
                                          masked_left=ml)
            assert ei.value.status == code
        with pytest.raises(blt.BltError):
            blt.blt_kv_append(dec.ctx, dec.state, [0], [0], [17], 17, [0] * 17, bytes_=[1] * 17)
        # a pass may not start past the rows written for its slot: nothing
        # is cached yet, so start 1 is rejected before anything runs; after
        # 3 rows, start 3 is accepted and start 4 rejected, for both calls
        for call in ("append", "block"):
            def run(start, n=1):
                if call == "append":
                    blt.blt_kv_append(dec.ctx, dec.state, [1], [start], [n], n, [0] * n,
                                      bytes_=[7] * n)
                else:
                    blt.blt_decode_block_step(dec.ctx, dec.state, [1], [start], bt, 4, [0], 0.7,
                                              masked_left=ml)
            with pytest.raises(blt.BltError) as ei:
                run(4 if call == "block" else 1)
            assert ei.value.status == blt.BLT_EINVAL
        blt.blt_kv_append(dec.ctx, dec.state, [1], [0], [3], 3, [0] * 3, bytes_=[7] * 3)
        blt.blt_kv_append(dec.ctx, dec.state, [1], [3], [1], 1, [0], bytes_=[7])
        blt.blt_decode_block_step(dec.ctx, dec.state, [1], [4], bt, 4, [0], 0.7, masked_left=ml)
        for bad in (5, 9):
            with pytest.raises(blt.BltError) as ei:
                blt.blt_kv_append(dec.ctx, dec.state, [1], [bad], [1], 1, [0], bytes_=[7])
            assert ei.value.status == blt.BLT_EINVAL
        # empty inputs: an append of no rows and a latent upload of no
        # entries are accepted and do nothing (slot 0 still has no rows, so
        # start 1 stays rejected); a pass over no sequences is refused
        blt.blt_kv_append(dec.ctx, dec.state, [0, 1], [0, 0], [0, 0], 1, [0, 0], bytes_=[0, 0])
        blt.blt_latents_put(dec.ctx, dec.state, [], [], torch.zeros(1, device="cuda:0"), 0)
        with pytest.raises(blt.BltError) as ei:
            blt.blt_kv_append(dec.ctx, dec.state, [0], [1], [1], 1, [0], bytes_=[7])
        assert ei.value.status == blt.BLT_EINVAL
        with pytest.raises(blt.BltError) as ei:
            blt.blt_decode_block_step(dec.ctx, dec.state, [], [], bt, 4, [], 0.7, masked_left=ml)
        assert ei.value.status == blt.BLT_EINVAL
        torch.cuda.synchronize()
    finally:
        dec.close()
