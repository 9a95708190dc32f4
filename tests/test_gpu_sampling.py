"""GPU parity of sampled BLT-D (temperature and top-p sampling combined with
the unmask rules) against the CPU oracle.

Teacher-forced replays run each pass of an oracle trace on the GPU from the
oracle's own block state and check, per block position:
  * the logits, within the path's tolerance;
  * the drawn byte against the oracle's sampler applied to the GPU's own
    logits (the sampling logic, to float32 rounding: compared where that
    draw's margin exceeds 1e-5), and against the oracle's draw wherever the
    oracle's margin exceeds the probability error the logit tolerance allows;
  * the confidence (the model probability of the drawn byte) or entropy;
  * the commit: the oracle's unmask rule applied to the GPU's draws and
    confidences must give the GPU's block, unless a confidence lies within
    1e-5 of the threshold (or an entropy prefix sum within 1e-4 of gamma).
Native sessions are checked for determinism per seed and for the greedy
limit; options the library does not implement fail with BLT_ENOTIMPL.
"""
import numpy as np
import pytest

import bltgen
from oracle import decide, loops
from tests.gpu_util import (BF16_ABS, FP32_REL, Replayer, decoder_for, logits_ok, oracle_inputs,
                            say)

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


def _rule(block, choice, conf, ent, alpha, unmask):
    if unmask == "entropy":
        return decide.unmask_commit_entropy(block, choice, ent, alpha)[0]
    return decide.unmask_commit(block, choice, conf, alpha, unmask == "one_step")[0]


def _near_threshold(block, conf, ent, alpha, unmask):
    masked = [j for j, t in enumerate(block) if t == decide.MASK]
    if unmask == "threshold":
        return any(abs(conf[j] - alpha) < 1e-5 for j in masked)
    if unmask == "entropy":
        srt = sorted(ent[j] for j in masked)
        return any(abs(c - alpha) < 1e-4 for c in np.cumsum(srt))
    return False


def _replay_sampled(wl, unmask, alpha, sampling, n_gen=32, B=4):
    import torch
    w = bltgen.make_weights(wl, gains="random")
    W, inp, inp64 = oracle_inputs(wl, w)
    run = loops.blt_d(W, wl, inp64, n_gen, B, alpha, unmask=unmask, sampling=sampling, trace=True)
    temp, top_p, seed = sampling
    dec = decoder_for(wl.replace(block=B), w, max_batch=1, max_rows=256)
    scale = wl.head_scale
    stats = dict(drawn=0, vs_oracle=0, commits=0, worst=0.0)
    try:
        rp = Replayer(dec, wl, inp)
        rp.prefill(inp)
        for d, rec in enumerate(run.passes):
            z, am, cf, after, left = rp.block(rec, alpha, unmask, sampling=sampling, draw=d)
            na = rec["n_append"]
            ref = np.asarray(rec["logits"])[na:]
            ok, err, tol = logits_ok(z, ref, wl.dtype, scale)
            assert ok, f"pass {d}: logits err {err} > {tol}"
            stats["worst"] = max(stats["worst"], err)
            conf, ent = [0.0] * B, [0.0] * B
            for j in range(B):
                # logit error bound eps of the path -> probability error <= 2 eps / T
                eps = FP32_REL * np.abs(ref[j][:256]).max() if wl.dtype == "fp32" else BF16_ABS * scale
                prob_tol = 2.5 * eps / temp
                u = decide.uniform(seed, d * loops.MAX_BLOCK + j)
                assert u == rec["u"][j]
                b, _, e, margin = decide.sample_top_p(z[j], temp, top_p, u)
                zj = np.asarray(z[j][:256], dtype=np.float64)
                q = np.exp(zj - zj.max())
                conf[j], ent[j] = float(q[am[j]] / q.sum()), e
                if margin > 1e-5:
                    assert am[j] == b, f"pass {d} pos {j}: drew {am[j]}, sampler on its logits {b}"
                    stats["drawn"] += 1
                if rec["gap"][j] > prob_tol:
                    assert am[j] == rec["choice"][j], f"pass {d} pos {j}: drew {am[j]}, oracle {rec['choice'][j]}"
                    stats["vs_oracle"] += 1
                want = ent[j] if unmask == "entropy" else conf[j]
                assert abs(cf[j] - want) <= 1e-4 * max(1.0, abs(want)), (d, j, cf[j], want)
            if not _near_threshold(rec["block_before"], conf, ent, alpha, unmask):
                exp_after = _rule(rec["block_before"], list(am), conf, ent, alpha, unmask)
                assert list(after) == exp_after, f"pass {d}: block {list(after)} vs rule {exp_after}"
                stats["commits"] += 1
            assert left == sum(1 for t in after if t == decide.MASK)
    finally:
        dec.close()
    say(f"{wl.name} sampled BLT-D ({unmask}, T={temp}, top_p={top_p}): {len(run.passes)} passes, "
        f"worst logit err {stats['worst']:.3g}, {stats['drawn']} draws vs the sampler on GPU logits, "
        f"{stats['vs_oracle']} vs the oracle's draws, {stats['commits']} commits checked")
    assert stats["drawn"] > 0 and stats["commits"] > 0
    return stats


@pytest.mark.parametrize("unmask,alpha", [("threshold", 0.3), ("entropy", 3.0), ("one_step", 0.0)])
def test_tiny_fp32_sampled_blt_d_teacher_forced(unmask, alpha):
    wl = bltgen.WORKLOADS[0].replace(head_scale=12.0)
    st = _replay_sampled(wl, unmask, alpha, (0.8, 0.9, 1234))
    assert st["vs_oracle"] > 0


def test_mini_bf16_sampled_blt_d_entropy_teacher_forced():
    wl = MINI_BF16.replace(head_scale=12.0)
    _replay_sampled(wl, "entropy", 3.0, (1.0, 0.8, 77), n_gen=24)


def _replay_verify(wl, policy, r, sampling, n_gen=24, unmask="one_step", alpha=0.0):
    """Teacher-forced replay of a sampled BLT-S (drafts of r bytes) or
    one-step BLT-DV (blocks of r) oracle trace: draft passes draw on the GPU,
    the verify pass runs the causal rows, then blt_verify_sample decides
    from the GPU's own draft and verify logits.  The decision (accepted count
    and appended byte) is compared with the oracle's rule applied to the
    GPU's logits wherever that margin exceeds 1e-5, and with the oracle's own
    decision wherever its margin exceeds the probability error the logit
    tolerance allows."""
    import torch
    import block_diffusion_byte_amd as blt
    w = bltgen.make_weights(wl, gains="random")
    W, inp, inp64 = oracle_inputs(wl, w)
    temp, top_p, seed = sampling
    if policy == "blt_s":
        run = loops.blt_s(W, wl, inp64, n_gen, r, trace=True, sampling=sampling)
    else:
        run = loops.blt_dv(W, wl, inp64, n_gen, r, alpha, one_step=unmask == "one_step", unmask=unmask,
                           trace=True, sampling=sampling)
    dec = decoder_for(wl.replace(block=r), w, max_batch=1, max_rows=256)
    dev = "cuda:0"
    zq_d = torch.zeros((r, 257), dtype=torch.float32, device=dev)
    zp_d = torch.zeros((r + 1, 257), dtype=torch.float32, device=dev)
    draft_d = torch.zeros(r, dtype=torch.int32, device=dev)
    acc_d = torch.zeros(1, dtype=torch.int32, device=dev)
    nxt_d = torch.zeros(1, dtype=torch.int32, device=dev)
    stats = dict(rounds=0, vs_rule=0, vs_oracle=0, worst=0.0)
    try:
        rp = Replayer(dec, wl, inp)
        rp.prefill(inp)
        zq = []
        for d, rec in enumerate(run.passes):
            if rec["kind"] == "draft":
                z, am = rp.rows(rec, sampling=sampling, draw=d)
                zq.append(z[0])
                if rec["gap"][0] > 2.5 * FP32_REL * np.abs(np.asarray(rec["logits"])[0]).max() / temp:
                    assert am[0] == rec["choice"][0], f"pass {d}: drew {am[0]}, oracle {rec['choice'][0]}"
                continue
            if rec["kind"] == "block":
                # each position's draft distribution: the logits of the pass that committed it
                z, am, _, after, _ = rp.block(rec, alpha, unmask, sampling=sampling, draw=d)
                if not zq:
                    zq = [None] * r
                for j in range(r):
                    if rec["block_before"][j] == decide.MASK and rec["block_after"][j] != decide.MASK:
                        zq[j] = z[j]
                continue
            # verify pass: rows l..l+r, then the rejection-sampling decision
            z, _ = rp.rows(rec)
            ref = np.asarray(rec["logits"])
            ok, err, tol = logits_ok(z, ref, wl.dtype, wl.head_scale)
            assert ok, f"pass {d}: logits err {err} > {tol}"
            stats["worst"] = max(stats["worst"], err)
            draft = [int(t) for t in rec["tokens"][1:]]
            zq_d.copy_(torch.from_numpy(np.stack(zq)).float())
            zp_d.copy_(torch.from_numpy(z[:r + 1]).float())
            draft_d.copy_(torch.tensor(draft, dtype=torch.int32))
            blt.blt_verify_sample(dec.ctx, r, draft_d, r, zq_d, r, zp_d, r + 1, sampling, [d], acc_d,
                                  nxt_d, slot=[0])
            torch.cuda.synchronize()
            got = (int(acc_d.item()), int(nxt_d.item()))
            q = [decide.sampling_dist(zq[j], temp, top_p) for j in range(r)]
            p = [decide.sampling_dist(z[j], temp, top_p) for j in range(r + 1)]
            a, b, margin = decide.verify_sample(draft, q, p, rec["u_acc"], rec["u_next"])
            if margin > 1e-5:
                assert got == (a, b), f"pass {d}: GPU {got}, rule on GPU logits {(a, b)}"
                stats["vs_rule"] += 1
            eps = FP32_REL * np.abs(ref).max()
            if rec["margin"] > 4 * 2.5 * eps / temp:
                assert got == (rec["accept"], rec["next"]), f"pass {d}: GPU {got}, oracle {(rec['accept'], rec['next'])}"
                stats["vs_oracle"] += 1
            stats["rounds"] += 1
            zq = []
    finally:
        dec.close()
    say(f"sampled {policy} {unmask} (r={r}, T={temp}, top_p={top_p}): {stats['rounds']} verifications, worst logit "
        f"err {stats['worst']:.3g}, {stats['vs_rule']} decisions vs the rule on GPU logits, "
        f"{stats['vs_oracle']} vs the oracle's")
    assert stats["vs_rule"] > 0 and stats["vs_oracle"] > 0


@pytest.mark.parametrize("policy,r", [("blt_s", 4), ("blt_dv", 4)])
def test_tiny_fp32_rejection_sampling_verify_teacher_forced(policy, r):
    wl = bltgen.WORKLOADS[0].replace(head_scale=12.0)
    _replay_verify(wl, policy, r, (0.8, 0.9, 4321))


@pytest.mark.parametrize("unmask,alpha", [("threshold", 0.3), ("entropy", 3.0)])
def test_tiny_fp32_sampled_blt_dv_multi_pass_drafts_teacher_forced(unmask, alpha):
    """Sampled BLT-DV whose block draft takes several passes (threshold or
    entropy-bounded unmasking): every draft byte is verified against the
    distribution of the pass that committed it (the oracle's blt_dv with
    sampling), by blt_verify_sample from the GPU's own logits."""
    wl = bltgen.WORKLOADS[0].replace(head_scale=12.0)
    _replay_verify(wl, "blt_dv", 4, (0.8, 0.9, 4321), unmask=unmask, alpha=alpha)


def _session(wl, w, inps, n_gen, block, alpha, unmask, temp, top_p, seed, policy=None):
    import torch
    import block_diffusion_byte_amd as blt
    dec = decoder_for(wl.replace(block=block), w, max_batch=len(inps), max_rows=64)
    table = torch.from_numpy(np.stack([i["latents"] for i in inps])).to("cuda:0", dec.torch_dtype)
    sess = blt.blt_session_create(dec.ctx, dec.state, [i["prompt"] for i in inps],
                                  [i["prompt_patches"] for i in inps], [i["salt"] for i in inps],
                                  table, wl.n_latents)
    try:
        blt.blt_session_prefill(dec.ctx, sess)
        blt.blt_session_generate(dec.ctx, sess, blt.BLT_POLICY_BLT_D if policy is None else policy,
                                 block, alpha, n_gen, unmask, temperature=temp, top_p=top_p, seed=seed)
        return [blt.blt_session_result(sess, b, n_gen) for b in range(len(inps))]
    finally:
        blt.blt_session_destroy(sess)
        dec.close()


def test_sampled_sessions_are_seeded_and_reach_the_greedy_limit():
    import block_diffusion_byte_amd as blt
    wl = bltgen.WORKLOADS[0].replace(head_scale=12.0)
    w = bltgen.make_weights(wl, gains="random")
    inps = [bltgen.make_sequence_inputs(wl, b) for b in range(3)]
    E = blt.BLT_UNMASK_ENTROPY
    a = _session(wl, w, inps, 40, 4, 3.0, E, 0.8, 0.9, 5)
    b = _session(wl, w, inps, 40, 4, 3.0, E, 0.8, 0.9, 5)
    c = _session(wl, w, inps, 40, 4, 3.0, E, 0.8, 0.9, 6)
    assert [r["out"] for r in a] == [r["out"] for r in b]
    assert [r["out"] for r in a] != [r["out"] for r in c]
    assert all(r["n"] == 40 for r in a)
    g = _session(wl, w, inps, 40, 4, 3.0, E, 0.0, 1.0, 0)
    lim = _session(wl, w, inps, 40, 4, 3.0, E, 1.0, 1e-7, 5)
    assert [(r["out"], r["n_dec"]) for r in lim] == [(r["out"], r["n_dec"]) for r in g]
    # the oracle's greedy EB run agrees with the greedy session
    W, _, inp64 = oracle_inputs(wl, w, 0)
    ref = loops.blt_d(W, wl, inp64, 40, 4, 3.0, unmask="entropy")
    assert list(g[0]["out"]) == ref.out
    say(f"sampled sessions: seeded, n_dec {[r['n_dec'] for r in a]}; top_p -> 0 equals greedy")


@pytest.mark.parametrize("policy", ["greedy", "blt_s", "blt_dv", "blt_dv_threshold", "blt_dv_entropy"])
def test_sampled_verified_sessions_are_seeded_and_reach_the_greedy_limit(policy):
    """Sampled greedy BLT, BLT-S and BLT-DV sessions (one-step, threshold and
    entropy-bounded drafts; rejection-sampling verification): a seed
    reproduces its bytes, another seed gives others, and a vanishing top_p
    gives the greedy session exactly."""
    import block_diffusion_byte_amd as blt
    wl = bltgen.WORKLOADS[0].replace(head_scale=12.0)
    w = bltgen.make_weights(wl, gains="random")
    inps = [bltgen.make_sequence_inputs(wl, b) for b in range(3)]
    pid = {"greedy": blt.BLT_POLICY_GREEDY, "blt_s": blt.BLT_POLICY_BLT_S}.get(policy, blt.BLT_POLICY_BLT_DV)
    block = {"greedy": 1, "blt_s": 4}.get(policy, 4)
    O, alpha = blt.BLT_UNMASK_ONE_STEP, 0.0
    if policy == "blt_dv_threshold":
        O, alpha = blt.BLT_UNMASK_THRESHOLD, 0.3
    if policy == "blt_dv_entropy":
        O, alpha = blt.BLT_UNMASK_ENTROPY, 3.0
    a = _session(wl, w, inps, 32, block, alpha, O, 0.8, 0.9, 5, policy=pid)
    b = _session(wl, w, inps, 32, block, alpha, O, 0.8, 0.9, 5, policy=pid)
    c = _session(wl, w, inps, 32, block, alpha, O, 0.8, 0.9, 6, policy=pid)
    assert [r["out"] for r in a] == [r["out"] for r in b]
    assert [r["out"] for r in a] != [r["out"] for r in c]
    assert all(r["n"] == 32 for r in a)
    g = _session(wl, w, inps, 32, block, alpha, O, 0.0, 1.0, 0, policy=pid)
    lim = _session(wl, w, inps, 32, block, alpha, O, 1.0, 1e-7, 5, policy=pid)
    assert [(r["out"], r["n_dec"], r["accepted"]) for r in lim] == \
        [(r["out"], r["n_dec"], r["accepted"]) for r in g]
    say(f"sampled {policy} sessions: seeded; top_p -> 0 equals greedy; n_dec {[r['n_dec'] for r in a]}")


@pytest.mark.parametrize("unmask,alpha", [("threshold", 0.3), ("entropy", 3.0)])
def test_tiny_fp32_sampled_blt_dv_session_matches_oracle(unmask, alpha):
    """The native driver's sampled BLT-DV with multi-pass drafts (each draft
    byte verified against the distribution of the pass that committed it, as
    kept on the device) reproduces the oracle's sampled blt_dv: bytes,
    decoder / encoder-global passes and accepted draft bytes (float32: the
    sampler's and the acceptance test's margins lie far outside the path's
    rounding for these draws)."""
    import block_diffusion_byte_amd as blt
    wl = bltgen.WORKLOADS[0].replace(head_scale=12.0)
    w = bltgen.make_weights(wl, gains="random")
    smp = (0.8, 0.9, 5)
    inps, refs = [], []
    for seq in range(3):
        W, inp, inp64 = oracle_inputs(wl, w, seq)
        inps.append(inp)
        refs.append(loops.blt_dv(W, wl, inp64, 32, 4, alpha, one_step=False, unmask=unmask,
                                 sampling=(smp[0], smp[1], smp[2] + seq)))
    mode = blt.BLT_UNMASK_ENTROPY if unmask == "entropy" else blt.BLT_UNMASK_THRESHOLD
    got = _session(wl, w, inps, 32, 4, alpha, mode, smp[0], smp[1], smp[2], policy=blt.BLT_POLICY_BLT_DV)
    for b, (g, r) in enumerate(zip(got, refs)):
        assert list(g["out"]) == r.out, f"seq {b}: bytes differ"
        assert (g["n_dec"], g["n_eg"], g["accepted"]) == (r.n_dec, r.n_eg, sum(r.accept)), f"seq {b}"
    say(f"sampled BLT-DV {unmask} sessions equal the oracle: n_dec {[g['n_dec'] for g in got]}, "
        f"accepted {[g['accepted'] for g in got]}")


def test_sampling_argument_errors():
    import block_diffusion_byte_amd as blt
    wl = bltgen.WORKLOADS[0]
    w = bltgen.make_weights(wl)
    inps = [bltgen.make_sequence_inputs(wl, 0)]
    with pytest.raises(blt.BltError) as ei:
        _session(wl, w, inps, 8, 4, 0.7, 0, 1.0, 0.0, 1)
    assert ei.value.status == blt.BLT_EINVAL


def test_verify_sample_batch_above_twice_max_rows():
    """blt_verify_sample stages one draw index per sequence: a batch of 64 on
    a context of max_rows 16 (more sequences than the latent-offset lists
    hold) must stay within the staging area and decide every sequence as
    the oracle's rule does on the same float32 logits."""
    import torch
    import block_diffusion_byte_amd as blt
    wl = bltgen.WORKLOADS[0]
    w = bltgen.make_weights(wl)
    batch, r, temp, top_p, seed = 64, 4, 0.9, 0.95, 77
    dec = decoder_for(wl.replace(block=r), w, max_batch=batch, max_rows=16)
    rng = np.random.default_rng(5)
    zq = (3.0 * rng.standard_normal((batch, r, 257))).astype(np.float32)
    zp = (3.0 * rng.standard_normal((batch, r + 1, 257))).astype(np.float32)
    draft = rng.integers(0, 256, (batch, r)).astype(np.int32)
    # half the drafts copy the verify rows' top byte, so acceptances happen
    draft[::2] = np.argmax(zp[::2, :r, :256], axis=2)
    draws = [int(v) for v in rng.integers(0, 1000, batch)]
    dev = "cuda:0"
    acc = torch.full((batch,), -1, dtype=torch.int32, device=dev)
    nxt = torch.full((batch,), -1, dtype=torch.int32, device=dev)
    try:
        blt.blt_verify_sample(dec.ctx, r, torch.from_numpy(draft).to(dev), r,
                              torch.from_numpy(zq).to(dev), r, torch.from_numpy(zp).to(dev), r + 1,
                              (temp, top_p, seed), draws, acc, nxt, slot=list(range(batch)))
        torch.cuda.synchronize()
        got_a, got_n = acc.cpu().numpy(), nxt.cpu().numpy()
    finally:
        dec.close()
    compared = accepted = 0
    for s in range(batch):
        q = [decide.sampling_dist(zq[s, j].astype(np.float64), temp, top_p) for j in range(r)]
        p = [decide.sampling_dist(zp[s, j].astype(np.float64), temp, top_p) for j in range(r + 1)]
        u_acc = [decide.uniform(seed + s, draws[s] * loops.MAX_BLOCK + j) for j in range(r)]
        u_next = decide.uniform(seed + s, draws[s] * loops.MAX_BLOCK + r)
        a, b, margin = decide.verify_sample(list(draft[s]), q, p, u_acc, u_next)
        if margin > 1e-5:
            assert (int(got_a[s]), int(got_n[s])) == (a, b), f"sequence {s}"
            compared += 1
            accepted += a
    say(f"verify_sample batch {batch} on max_rows 16: {compared} of {batch} decisions compared, "
        f"{accepted} draft bytes accepted")
    assert compared >= batch // 2 and accepted > 0
