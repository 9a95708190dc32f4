"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a
closed form, a textbook or library routine in a special case, brute force
on tiny inputs, an invariant, or a value the pages print.  They are chosen
so that a plausible slip (a dropped term, a wrong sign or index, a
transposed operand) fails at least one of them.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

import bltgen
from oracle import cache, decide, loops, model, patcher, proxy

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MICRO = bltgen.WORKLOADS[0].replace(n_layers=2, d_model=32, n_heads=2, d_ffn=64, d_global=16,
                                    prompt_len=12, prompt_patches=5, n_gen=16)


def micro(gains="random", **kw):
    wl = MICRO.replace(**kw)
    W = model.as64(bltgen.make_weights(wl, gains=gains))
    inp = bltgen.make_sequence_inputs(wl, 0)
    inp["latents"] = inp["latents"].astype(np.float64)
    return wl, W, inp


# ---------------------------------------------------------------- attention
def brute_attention(q, k, v, allow):
    n, H, dh = q.shape
    out = np.zeros_like(q)
    for h in range(H):
        for i in range(n):
            js = [j for j in range(k.shape[0]) if allow[i, j]]
            sc = [sum(q[i, h, e] * k[j, h, e] for e in range(dh)) / dh ** 0.5 for j in js]
            mx = max(sc)
            w = [np.exp(s - mx) for s in sc]
            tot = sum(w)
            for j, wj in zip(js, w):
                out[i, h] += (wj / tot) * v[j, h]
    return out


def test_masked_attention_matches_brute_force():
    rng = np.random.default_rng(1)
    for n, m, H, dh in [(5, 7, 2, 4), (9, 9, 3, 2), (1, 4, 1, 8)]:
        q, k, v = (rng.standard_normal((x, H, dh)) for x in (n, m, m))
        allow = rng.random((n, m)) < 0.5
        allow[np.arange(n), rng.integers(0, m, n)] = True
        np.testing.assert_allclose(model.masked_attention(q, k, v, allow),
                                   brute_attention(q, k, v, allow), rtol=1e-12, atol=1e-12)


def test_masked_attention_matches_torch_sdpa():
    rng = np.random.default_rng(2)
    n, H, dh = 11, 3, 8
    q, k, v = (rng.standard_normal((n, H, dh)) for _ in range(3))
    allow = model.blt_d_mask(7, 4)
    ref = Fnn.scaled_dot_product_attention(
        torch.tensor(q).transpose(0, 1), torch.tensor(k).transpose(0, 1),
        torch.tensor(v).transpose(0, 1), attn_mask=torch.tensor(allow)).transpose(0, 1).numpy()
    np.testing.assert_allclose(model.masked_attention(q, k, v, allow), ref, rtol=1e-12, atol=1e-12)


def test_blt_d_mask_structure():
    a = model.blt_d_mask(3, 2)
    # prefix causal, prefix never reads the block; block reads prefix + whole block
    assert a.tolist() == [
        [1, 0, 0, 0, 0], [1, 1, 0, 0, 0], [1, 1, 1, 0, 0], [1, 1, 1, 1, 1], [1, 1, 1, 1, 1]]
    c = model.blt_d_mask(3, 2, block_causal=True)
    assert c.tolist() == np.tril(np.ones((5, 5), dtype=bool)).tolist()


# ---------------------------------------------------------------- RoPE / norms
def test_rope_is_complex_rotation_of_half_pairs():
    rng = np.random.default_rng(3)
    n, H, dh, theta = 6, 2, 8, 10000.0
    x = rng.standard_normal((n, H, dh))
    pos = np.array([0, 1, 5, 77, 1000, 4095])
    got = model.rope(x, pos, theta)
    half = dh // 2
    z = x[..., :half] + 1j * x[..., half:]
    for j in range(half):
        z[..., j] *= np.exp(1j * pos[:, None] * theta ** (-2.0 * j / dh))
    np.testing.assert_allclose(got, np.concatenate([z.real, z.imag], -1), atol=1e-12)


def test_rope_identity_at_zero_and_relative():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 16))
    k = rng.standard_normal((1, 1, 16))
    np.testing.assert_array_equal(model.rope(q, [0], 1e4), q)
    s = [float((model.rope(q, [p + c], 1e4) * model.rope(k, [3 + c], 1e4)).sum())
         for p, c in [(9, 0), (9, 17), (9, 1234)]]
    assert np.allclose(s, s[0], atol=1e-10)


def test_rms_norm_matches_torch_and_invariants():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 32)) * 3
    g = rng.uniform(0.5, 1.5, 32)
    ref = Fnn.rms_norm(torch.tensor(x), (32,), weight=torch.tensor(g), eps=1e-5).numpy()
    np.testing.assert_allclose(model.rms_norm(x, g, 1e-5), ref, rtol=1e-12)
    u = model.rms_norm(x, np.ones(32), 0.0)
    np.testing.assert_allclose(np.sqrt((u ** 2).mean(-1)), 1.0, rtol=1e-12)


# ---------------------------------------------------------------- cross-attention
def test_single_key_cross_attention_closed_form():
    wl, W, inp = micro()
    lw = W["layers"][1]
    rng = np.random.default_rng(6)
    h = rng.standard_normal((4, wl.d_model))
    taus = [0, 3, 3, 1]
    got = model.cross_attention(W, lw, h, inp["latents"], [[t] for t in taus], wl.n_heads)
    for i, t in enumerate(taus):
        ot = np.einsum("oi,i->o", W["w_lat"], inp["latents"][t])
        want = np.einsum("oi,i->o", lw["wo_c"], np.einsum("oi,i->o", lw["wv_c"], ot))
        np.testing.assert_allclose(got[i], want, rtol=1e-11, atol=1e-12)


def test_multi_latent_cross_attention_matches_torch_sdpa():
    wl, W, inp = micro()
    lw = W["layers"][0]
    rng = np.random.default_rng(7)
    h = rng.standard_normal((3, wl.d_model))
    sets = [[0, 1, 2], [2, 4, 5], [1, 2, 3]]
    got = model.cross_attention(W, lw, h, inp["latents"], sets, wl.n_heads)
    H, dh = wl.n_heads, wl.d_head
    for i, s in enumerate(sets):
        ot = inp["latents"][s] @ W["w_lat"].T
        q = torch.tensor(h[i] @ lw["wq_c"].T).view(1, H, 1, dh)
        k = torch.tensor(ot @ lw["wk_c"].T).view(len(s), H, dh).permute(1, 0, 2)[None]
        v = torch.tensor(ot @ lw["wv_c"].T).view(len(s), H, dh).permute(1, 0, 2)[None]
        a = Fnn.scaled_dot_product_attention(q, k, v).reshape(-1).numpy()
        np.testing.assert_allclose(got[i], lw["wo_c"] @ a, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- full forward special cases
def _zero(W, keys):
    W = {k: v for k, v in W.items()}
    W["layers"] = [{k: (np.zeros_like(v) if k in keys else v) for k, v in lw.items()}
                   for lw in W["layers"]]
    return W


def _run_forward(W, wl, inp, toks, taus, allow):
    return model.forward(W, wl, inp["latents"], toks, np.arange(len(toks)), [[t] for t in taus], allow)


def test_forward_all_outputs_zero_is_head_of_embedding():
    wl, W, inp = micro()
    Wz = _zero(W, {"wo_c", "wo", "w2"})
    toks = [3, 250, 256, 256]
    z = _run_forward(Wz, wl, inp, toks, [0, 1, 1, 1], model.blt_d_mask(2, 2))
    e = W["embed"][toks]
    u = W["g_out"] * e / np.sqrt((e * e).mean(-1, keepdims=True) + wl.rms_eps)
    np.testing.assert_allclose(z, np.einsum("vi,ri->rv", W["w_out"], u), rtol=1e-11, atol=1e-13)


def test_forward_cross_only_closed_form():
    wl, W, inp = micro()
    Wz = _zero(W, {"wo", "w2"})
    toks, taus = [7, 9, 256], [0, 2, 4]
    z = _run_forward(Wz, wl, inp, toks, taus, model.blt_d_mask(2, 1))
    for i, (t, tau) in enumerate(zip(toks, taus)):
        h = W["embed"][t].copy()
        ot = np.einsum("oi,i->o", W["w_lat"], inp["latents"][tau])
        for lw in W["layers"]:
            h += np.einsum("oi,i->o", lw["wo_c"], np.einsum("oi,i->o", lw["wv_c"], ot))
        u = W["g_out"] * h / np.sqrt((h * h).mean() + wl.rms_eps)
        np.testing.assert_allclose(z[i], np.einsum("vi,i->v", W["w_out"], u), rtol=1e-10, atol=1e-12)


def test_forward_ffn_only_closed_form():
    wl, W, inp = micro()
    Wz = _zero(W, {"wo_c", "wo"})
    toks = [1, 2, 256, 256]
    z = _run_forward(Wz, wl, inp, toks, [0, 0, 0, 0], model.blt_d_mask(2, 2))
    h = W["embed"][toks].copy()
    for lw in W["layers"]:
        u = lw["g_ffn"] * h / np.sqrt((h * h).mean(-1, keepdims=True) + wl.rms_eps)
        a = np.einsum("fi,ri->rf", lw["w1"], u)
        h = h + np.einsum("of,rf->ro", lw["w2"], a * torch.sigmoid(torch.tensor(a)).numpy())
    u = W["g_out"] * h / np.sqrt((h * h).mean(-1, keepdims=True) + wl.rms_eps)
    np.testing.assert_allclose(z, np.einsum("vi,ri->rv", W["w_out"], u), rtol=1e-10, atol=1e-12)


def test_forward_one_self_attention_layer_matches_torch():
    """One layer, cross-attention and FFN outputs zeroed: the layer reduces to
    RMSNorm -> RoPE'd SDPA under the BLT-D mask -> W_o, checked against torch
    routines and the complex form of RoPE."""
    wl, W, inp = micro(n_layers=1)
    Wz = _zero(W, {"wo_c", "w2"})
    toks = [5, 6, 7, 256, 256, 256]
    n_pre = 3
    allow = model.blt_d_mask(n_pre, 3)
    pos = np.array([40, 41, 42, 43, 44, 45])
    z = model.forward(Wz, wl, inp["latents"], toks, pos, [[0]] * 6, allow)
    lw = W["layers"][0]
    d, H, dh = wl.d_model, wl.n_heads, wl.d_head
    e = torch.tensor(W["embed"][toks])
    u = Fnn.rms_norm(e, (d,), weight=torch.tensor(lw["g_attn"]), eps=wl.rms_eps)
    qkv = Fnn.linear(u, torch.tensor(lw["wqkv"]))

    def rot(x):
        x = x.view(6, H, dh)
        zc = torch.complex(x[..., :dh // 2], x[..., dh // 2:])
        f = wl.rope_theta ** (-2.0 * torch.arange(dh // 2, dtype=torch.float64) / dh)
        zc = zc * torch.polar(torch.ones(6, 1, dh // 2, dtype=torch.float64),
                              torch.tensor(pos, dtype=torch.float64)[:, None, None] * f)
        return torch.cat([zc.real, zc.imag], -1).transpose(0, 1)

    q, k = rot(qkv[:, :d]), rot(qkv[:, d:2 * d])
    v = qkv[:, 2 * d:].view(6, H, dh).transpose(0, 1)
    a = Fnn.scaled_dot_product_attention(q, k, v, attn_mask=torch.tensor(allow))
    h = e + Fnn.linear(a.transpose(0, 1).reshape(6, d), torch.tensor(lw["wo"]))
    want = Fnn.linear(Fnn.rms_norm(h, (d,), weight=torch.tensor(W["g_out"]), eps=wl.rms_eps),
                      torch.tensor(W["w_out"])).numpy()
    np.testing.assert_allclose(z, want, rtol=1e-10, atol=1e-12)


def test_mask_semantics_prefix_blind_to_block():
    wl, W, inp = micro()
    taus = [0, 1, 1, 2, 2, 2, 2]
    base = [10, 20, 30, 256, 256, 256, 256]
    alt = [10, 20, 30, 256, 77, 256, 256]
    for causal in (False, True):
        allow = model.blt_d_mask(3, 4, causal)
        z0 = _run_forward(W, wl, inp, base, taus, allow)
        z1 = _run_forward(W, wl, inp, alt, taus, allow)
        np.testing.assert_array_equal(z0[:3], z1[:3])           # prefix never sees the block
        if causal:
            np.testing.assert_array_equal(z0[3], z1[3])          # earlier block row blind
        else:
            assert np.abs(z0[3] - z1[3]).max() > 1e-6           # bidirectional block


def test_cached_forward_equals_no_cache():
    wl, W, inp = micro()
    rng = np.random.default_rng(8)
    x = list(rng.integers(0, 256, 20))
    taus = list(np.minimum(np.arange(20) // 3, 6))
    for causal in (False, True):
        c = cache.CachedDecoder(W, wl, inp["latents"], 64)
        c.run(x[:9], 0, taus[:9], 9)
        # pass with 3 append rows and a 4-row block (two masked)
        blk = [256, 42, 256, 17]
        z = c.run(x[9:12] + blk, 9, taus[9:12] + [5] * 4, 3, block_causal=causal)
        full = _run_forward(W, wl, inp, x[:12] + blk, taus[:12] + [5] * 4, model.blt_d_mask(12, 4, causal))
        np.testing.assert_allclose(z, full[9:], rtol=1e-10, atol=1e-12)
        # block-only pass after the append
        z = c.run(blk, 12, [5] * 4, 0, block_causal=causal)
        np.testing.assert_allclose(z, full[12:], rtol=1e-10, atol=1e-12)
        # rollback: recompute row 11 with another target, then append
        t2 = taus[:11] + [6, 6, 6]
        z = c.run(x[11:14], 11, t2[11:14], 3)
        full2 = _run_forward(W, wl, inp, x[:14], t2, model.blt_d_mask(14, 0))
        np.testing.assert_allclose(z, full2[11:], rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- decisions
def test_byte_choice_ties_mask_and_confidence():
    z = np.zeros(257)
    z[[5, 9]] = 2.0
    z[256] = 50.0                      # [MASK] logit never chosen
    b, conf, gap = decide.byte_choice(z)
    assert b == 5 and gap == 0.0
    p = torch.softmax(torch.tensor(z[:256]), 0).numpy()
    assert abs(conf - p.max()) < 1e-15
    b, conf, _ = decide.byte_choice(np.zeros(257))
    assert b == 0 and abs(conf - 1 / 256) < 1e-15


def test_unmask_rules():
    M = decide.MASK
    blk, ch = decide.unmask_commit([M, 3, M, M], [9, 9, 8, 7], [0.7, 0.99, 0.71, 0.9], 0.7)
    assert blk == [M, 3, 8, 7] and ch == [2, 3]          # strict '>' alpha, committed untouched
    blk, ch = decide.unmask_commit([M, M, M], [1, 2, 3], [0.2, 0.5, 0.5], 0.7)
    assert blk == [M, 2, M] and ch == [1]                 # fallback: most confident, lowest pos
    blk, ch = decide.unmask_commit([M, 4, M], [1, 2, 3], [0.0, 0.0, 0.0], 0.7, one_step=True)
    assert blk == [1, 4, 3]


def test_entropy_closed_forms_and_library():
    """Entropy of the byte distribution: scipy's entropy of the softmax over
    bytes 0..255; uniform -> ln 256, two tied bytes -> ln 2, one-hot -> 0;
    the [MASK] logit never counts."""
    from scipy.stats import entropy as sp_entropy
    rng = np.random.default_rng(7)
    for _ in range(5):
        z = rng.normal(0, 3, 257)
        p = np.exp(z[:256] - z[:256].max())
        assert decide.entropy(z) == pytest.approx(sp_entropy(p / p.sum()), rel=1e-12, abs=1e-12)
        z2 = z.copy()
        z2[256] = 1e3
        assert decide.entropy(z2) == decide.entropy(z)
    assert decide.entropy(np.zeros(257)) == pytest.approx(np.log(256), rel=1e-14)
    two = np.full(257, -1e9)
    two[[3, 200]] = 5.0
    assert decide.entropy(two) == pytest.approx(np.log(2), rel=1e-14)
    one = np.zeros(257)
    one[17] = 1e4
    assert decide.entropy(one) == 0.0


def test_entropy_bounded_unmask_rules():
    M = decide.MASK
    # ranked 1 (0.1), 2 (0.3), 0 (0.5): cumulative 0.1, 0.4, 0.9
    blk, ch = decide.unmask_commit_entropy([M, M, M], [7, 8, 9], [0.5, 0.1, 0.3], 0.45)
    assert blk == [M, 8, 9] and ch == [1, 2]
    blk, ch = decide.unmask_commit_entropy([M, M, M], [7, 8, 9], [0.5, 0.1, 0.3], 0.05)
    assert blk == [M, 8, M] and ch == [1]                 # at least one commit
    blk, ch = decide.unmask_commit_entropy([M, 4, M], [7, 8, 9], [0.2, 0.0, 0.2], 0.3)
    assert blk == [7, 4, M] and ch == [0]                 # equal entropies: lower position first
    blk, ch = decide.unmask_commit_entropy([M, 4, M], [7, 8, 9], [0.2, 0.0, 0.2], np.inf)
    assert blk == [7, 4, 9]


def test_entropy_bounded_unmask_is_the_largest_subset_within_gamma():
    """Brute force over every subset of the masked positions (B <= 6): the
    number committed is the largest size of a subset whose entropies sum to
    at most gamma (at least 1), and the committed positions are the lowest-
    entropy ones."""
    M = decide.MASK
    rng = np.random.default_rng(11)
    for _ in range(300):
        B = int(rng.integers(1, 7))
        block = [M if rng.random() < 0.8 else 5 for _ in range(B)]
        masked = [i for i in range(B) if block[i] == M]
        ent = list(np.round(rng.exponential(0.7, B), 2))   # rounded: ties happen
        gamma = float(rng.choice([0.0, rng.uniform(0, 3), np.inf]))
        out, ch = decide.unmask_commit_entropy(block, list(range(10, 10 + B)), ent, gamma)
        if not masked:
            assert ch == [] and out == block
            continue
        best = max((len(S) for r in range(len(masked) + 1) for S in itertools.combinations(masked, r)
                    if sum(ent[i] for i in S) <= gamma), default=0)
        assert len(ch) == max(best, 1)
        worst_in = max(ent[i] for i in ch)
        assert all(ent[i] >= worst_in for i in masked if i not in ch)
        assert all(out[i] == 10 + i for i in ch) and all(out[i] == block[i] for i in range(B) if i not in ch)


def test_verify_exhaustive_against_greedy_continuation():
    """r <= 3, 2-symbol alphabet: the committed bytes are exactly the first
    a + 1 bytes of the greedy continuation, and a is the longest draft prefix
    equal to it (the exactness guarantee of greedy verification)."""
    for r in range(1, 4):
        for table in itertools.product([0, 1], repeat=2 ** (r + 1)):
            f = lambda prefix: table[int("1" + "".join(map(str, prefix)), 2) % len(table)]
            for draft in itertools.product([0, 1], repeat=r):
                pred = [f(list(draft[:j])) for j in range(r + 1)]
                a, nxt = decide.verify_accept(list(draft), pred)
                greedy = []
                for _ in range(r + 1):
                    greedy.append(f(greedy))
                assert list(draft[:a]) + [nxt] == greedy[:a + 1]
                assert a == r or draft[a] != greedy[a]


def test_verify_special_cases():
    assert decide.verify_accept([4, 5, 6], [4, 5, 6, 7]) == (3, 7)   # all match + free byte
    assert decide.verify_accept([9, 5, 6], [4, 5, 6, 7]) == (0, 4)   # first wrong -> correction


# ---------------------------------------------------------------- patcher
def test_splitmix64_reference_vector():
    with open(os.path.join(GOLDEN, "splitmix64.json")) as f:
        g = json.load(f)
    assert [patcher.splitmix64_nth(g["seed"], i + 1) for i in range(3)] == [int(v, 16) for v in g["outputs"]]


def test_uniform_draws_are_published_splitmix64_outputs():
    """decide.uniform(seed, k) is the top 24 bits of SplitMix64 output k + 1,
    over 2^24: pinned to the published outputs from state 0."""
    with open(os.path.join(GOLDEN, "splitmix64.json")) as f:
        g = json.load(f)
    for k, v in enumerate(g["outputs"]):
        assert decide.uniform(g["seed"], k) == (int(v, 16) >> 40) / 2.0 ** 24
    u = [decide.uniform(7, k) for k in range(4096)]
    assert min(u) >= 0.0 and max(u) < 1.0 and abs(np.mean(u) - 0.5) < 0.02


def _logits_of(p):
    z = np.full(257, -1e4)
    for b, q in p.items():
        z[b] = np.log(q)
    return z


def test_top_p_worked_distributions():
    """Dyadic probabilities make every interval boundary exact: with p =
    (1/2, 1/4, 1/8, 1/8) on bytes 0..3, u in [0, 1/2) picks 0, [1/2, 3/4)
    picks 1, and so on; top_p = 0.7 keeps bytes 0 and 1 (the mass before
    byte 2 is 3/4 >= 0.7), whose mass 3/4 scales u.  Equal probabilities
    rank by byte id.  [MASK] never takes part."""
    z = _logits_of({0: 0.5, 1: 0.25, 2: 0.125, 3: 0.125})
    for u, full, cut in [(0.0, 0, 0), (0.4999, 0, 0), (0.5, 1, 0), (0.6666, 1, 0), (0.6667, 1, 1),
                         (0.7499, 1, 1), (0.75, 2, 1), (0.8749, 2, 1), (0.875, 3, 1), (0.9999, 3, 1)]:
        assert decide.sample_top_p(z, 1.0, 1.0, u)[0] == full, u
        assert decide.sample_top_p(z, 1.0, 0.7, u)[0] == cut, u
    b, pb, ent, _ = decide.sample_top_p(z, 1.0, 1.0, 0.8)
    assert b == 2 and abs(pb - 0.125) < 1e-12 and abs(ent - 1.75 * np.log(2)) < 1e-9
    # temperature 1/2 squares and renormalises the probabilities for the draw
    # (0.5^2, 0.25^2, 2 x 0.125^2 over 11/32: 8/11, 2/11, 1/22, 1/22) but the
    # confidence and entropy stay the model's
    for u, want in [(0.72, 0), (0.73, 1), (0.9, 1), (0.91, 2), (0.954, 2), (0.955, 3)]:
        b, pb, ent, _ = decide.sample_top_p(z, 0.5, 1.0, u)
        assert b == want, u
        assert abs(pb - [0.5, 0.25, 0.125, 0.125][b]) < 1e-12 and abs(ent - 1.75 * np.log(2)) < 1e-9
    tie = _logits_of({200: 0.25, 3: 0.25, 9: 0.25, 7: 0.25})
    tie[256] = 50.0                                   # a huge [MASK] logit changes nothing
    assert [decide.sample_top_p(tie, 1.0, 1.0, u)[0] for u in (0.1, 0.3, 0.6, 0.9)] == [3, 7, 9, 200]
    assert [decide.sample_top_p(tie, 1.0, 0.5, u)[0] for u in (0.1, 0.6)] == [3, 7]


def test_top_p_limits_are_greedy():
    """A vanishing top_p keeps only the most probable byte (lowest id on
    ties), and a vanishing temperature puts all mass on it: both give the
    greedy byte for every u."""
    rng = np.random.default_rng(5)
    for _ in range(20):
        z = rng.normal(0, 2, 257)
        g = decide.byte_choice(z)[0]
        for u in (0.0, 0.37, 0.999):
            assert decide.sample_top_p(z, 1.0, 1e-9, u)[0] == g
            assert decide.sample_top_p(z, 1e-3, 1.0, u)[0] == g
    z = np.zeros(257)
    assert [decide.sample_top_p(z, 1.0, 1e-9, u)[0] for u in (0.0, 0.99)] == [0, 0]


@pytest.mark.parametrize("top_p", [1.0, 0.9, 0.5])
def test_top_p_nucleus_and_frequencies(top_p):
    """On a grid of u the sampler only visits the nucleus -- the smallest set
    of most probable bytes whose mass reaches top_p, found here by a sort of
    (-p, byte id) -- and each nucleus byte with frequency p_b / mass(nucleus)
    to within the grid step."""
    rng = np.random.default_rng(11)
    z = rng.normal(0, 1.5, 257)
    y = z[:256] / 0.8
    p = np.exp(y - y.max())
    p /= p.sum()
    rank = np.lexsort((np.arange(256), -p))
    k = int(np.searchsorted(np.cumsum(p[rank]), top_p - 1e-15)) + 1
    nucleus = rank[:min(k, 256)]
    mass = p[nucleus].sum()
    n = 8192
    hits = np.zeros(256)
    for i in range(n):
        hits[decide.sample_top_p(z, 0.8, top_p, (i + 0.5) / n)[0]] += 1
    assert set(np.flatnonzero(hits)) <= set(nucleus.tolist())
    assert np.abs(hits[nucleus] / n - p[nucleus] / mass).max() <= 1.0 / n + 1e-12


def test_sampling_dist_is_the_renormalised_nucleus():
    z = _logits_of({0: 0.5, 1: 0.25, 2: 0.125, 3: 0.125})
    assert np.allclose(decide.sampling_dist(z, 1.0, 1.0)[:4], [0.5, 0.25, 0.125, 0.125])
    assert np.allclose(decide.sampling_dist(z, 1.0, 0.7)[:4], [2 / 3, 1 / 3, 0, 0])
    assert np.allclose(decide.sampling_dist(z, 0.5, 1.0)[:4], [8 / 11, 2 / 11, 1 / 22, 1 / 22])
    assert decide.sampling_dist(z, 1.0, 1.0)[4:].max() < 1e-100


def test_verify_sample_worked_example():
    """Draft q = (1/2, 1/4, 1/8, 1/8), target p uniform on bytes 0..3: byte 0
    is kept iff u < p/q = 1/2; the residual max(0, p - q) = (0, 0, 1/8, 1/8)
    splits at u_next = 1/2; byte 2 (p/q = 2) is always kept; after a full
    acceptance the free byte is drawn from the last target (ties by id)."""
    q = np.zeros(256); q[:4] = [0.5, 0.25, 0.125, 0.125]
    p = np.zeros(256); p[:4] = 0.25
    assert decide.verify_sample([0], [q], [p, p], [0.49], 0.9)[:2] == (1, 3)
    assert decide.verify_sample([0], [q], [p, p], [0.51], 0.49)[:2] == (0, 2)
    assert decide.verify_sample([0], [q], [p, p], [0.51], 0.51)[:2] == (0, 3)
    assert decide.verify_sample([2, 0], [q, q], [p, p, p], [0.999, 0.7], 0.3)[:2] == (1, 2)
    assert decide.verify_sample([2, 2], [q, q], [p, p, p], [0.999, 0.999], 0.3)[:2] == (2, 1)


def test_verify_sample_keeps_the_target_distribution():
    """Speculative sampling emits the target distribution: with the draft
    byte drawn from q, the first emitted byte follows p exactly, and after a
    full acceptance the free byte follows the next target.  Checked by
    enumerating the draft byte (weight q) over a grid of both uniforms."""
    rng = np.random.default_rng(21)
    zq = np.full(257, -1e4); zp = np.full(257, -1e4); zn = np.full(257, -1e4)
    zq[:6] = rng.normal(0, 1, 6); zp[:6] = rng.normal(0, 1, 6); zn[:6] = rng.normal(0, 1, 6)
    q = decide.sampling_dist(zq, 1.0, 0.9)
    p = decide.sampling_dist(zp, 0.7, 1.0)
    pn = decide.sampling_dist(zn, 1.0, 1.0)
    n = 96
    first = np.zeros(256)
    free = np.zeros(256)
    accepted = 0.0
    for x in np.flatnonzero(q):
        for i in range(n):
            for k in range(n):
                a, b, _ = decide.verify_sample([x], [q], [p, pn], [(i + 0.5) / n], (k + 0.5) / n)
                w = q[x] / n / n
                if a == 1:
                    first[x] += w
                    free[b] += w
                    accepted += w
                else:
                    first[b] += w
    assert np.abs(first - p).max() < 3.0 / n
    assert np.abs(free / accepted - pn).max() < 3.0 / n


def test_verify_sample_greedy_limit_is_exact_match():
    """With one-hot distributions (a vanishing top_p) rejection sampling is
    the greedy exact-match rule, correction and free byte included."""
    rng = np.random.default_rng(8)
    for _ in range(30):
        r = 4
        zq = rng.normal(0, 1, (r, 257))
        zp = rng.normal(0, 1, (r + 1, 257))
        y = [decide.byte_choice(zp[j])[0] for j in range(r + 1)]
        draft = [decide.byte_choice(zq[j])[0] for j in range(r)]
        for j in range(r):
            if rng.random() < 0.6:
                draft[j] = y[j]
        q = [decide.sampling_dist(zq[j], 1.0, 1e-9) for j in range(r)]
        for j in range(r):                        # the draft's own one-hot distribution
            q[j] = np.eye(256)[draft[j]]
        p = [decide.sampling_dist(zp[j], 1.0, 1e-9) for j in range(r + 1)]
        got = decide.verify_sample(draft, q, p, list(rng.random(r)), float(rng.random()))[:2]
        assert got == decide.verify_accept(draft, y)


def test_targets_worked_example():
    with open(os.path.join(GOLDEN, "targets_example.json")) as f:
        g = json.load(f)
    patch, ends = patcher.segment([0] * sum(g["patch_lengths"]), g["patch_lengths"], 0)
    assert [patcher.causal_target(patch, ends, i) for i in range(len(patch))] == g["targets"]
    assert patcher.last_target(patch) == g["last_target"]


def test_patcher_rule_statistics_and_causality():
    rng = np.random.default_rng(9)
    x = list(rng.integers(0, 256, 4000))
    patch, ends = patcher.segment(x, [1, 3], 12345)
    lens = np.bincount(patch)
    assert lens.max() <= 8 and 3.0 < lens[2:-1].mean() < 4.5
    y = list(x)
    y[3000] = (y[3000] + 1) % 256
    p2, e2 = patcher.segment(y, [1, 3], 12345)
    assert (e2[:3000] == ends[:3000]).all() and (p2[:3001] == patch[:3001]).all()


# ---------------------------------------------------------------- loops
@pytest.fixture(scope="module")
def tiny():
    wl = bltgen.WORKLOADS[0]
    W = model.as64(bltgen.make_weights(wl, gains="random"))
    inp = bltgen.make_sequence_inputs(wl, 0)
    inp["latents"] = inp["latents"].astype(np.float64)
    return wl, W, inp


def test_blt_s_equals_greedy_for_every_k(tiny):
    wl, W, inp = tiny
    g = loops.greedy(W, wl, inp, 48)
    assert g.n_dec == 48
    for k in (1, 2, 3, 5, 8):
        s = loops.blt_s(W, wl, inp, 48, k)
        assert s.out == g.out
        assert s.n_dec == len(s.accept) * (k + 1) and s.n_eg == len(s.accept)


def test_blt_d_block1_is_masked_row_greedy_for_any_alpha(tiny):
    wl, W, inp = tiny
    ref = loops.masked_row_greedy(W, wl, inp, 12)
    for alpha in (0.0, 0.7, 1.0):
        for causal in (False, True):
            r = loops.blt_d(W, wl, inp, 12, 1, alpha, block_causal=causal)
            assert r.out == ref and r.n_dec == 12 and r.n_eg == 12


def test_blt_d_alpha_extremes(tiny):
    wl, W, inp = tiny
    r = loops.blt_d(W, wl, inp, 32, 4, 1.0)
    assert r.n_dec == 32 and r.n_eg == 8                 # one commit per pass
    lo = loops.blt_d(W, wl, inp, 32, 4, 1.0 / 512)
    one = loops.blt_d(W, wl, inp, 32, 4, 0.7, one_step=True)
    assert lo.out == one.out and lo.n_dec == 8 == one.n_dec


def test_blt_d_entropy_bound_extremes(tiny):
    """Entropy-bounded unmasking: an unbounded gamma fills the block in one
    pass (= one-step); gamma = 0 commits one position per pass; with B = 1
    every rule is the masked-row greedy decoder."""
    wl, W, inp = tiny
    inf = loops.blt_d(W, wl, inp, 32, 4, np.inf, unmask="entropy")
    one = loops.blt_d(W, wl, inp, 32, 4, 0.7, one_step=True)
    assert inf.out == one.out and inf.n_dec == one.n_dec == 8
    zero = loops.blt_d(W, wl, inp, 32, 4, 0.0, unmask="entropy", trace=True)
    assert zero.n_dec == 32 and all(len(p["chosen"]) == 1 for p in zero.passes)
    for p in zero.passes:               # the committed position has the lowest entropy
        masked = [j for j, t in enumerate(p["block_before"]) if t == decide.MASK]
        assert p["entropy"][p["chosen"][0]] == min(p["entropy"][j] for j in masked)
    ref = loops.masked_row_greedy(W, wl, inp, 12)
    assert loops.blt_d(W, wl, inp, 12, 1, 0.5, unmask="entropy").out == ref


def test_sampled_blt_d_limits_and_determinism(tiny):
    """Sampled BLT-D: a vanishing top_p or temperature is greedy BLT-D (same
    bytes, same passes) under every unmask rule; a fixed seed reproduces the
    run; the draws follow the counter layout (pass d, position j -> d*64+j)."""
    wl, W, inp = tiny
    for mode, alpha in (("threshold", 0.7), ("entropy", 2.0), ("one_step", 0.0)):
        g = loops.blt_d(W, wl, inp, 24, 4, alpha, unmask=mode)
        for smp in ((1.0, 1e-9, 3), (1e-4, 1.0, 4)):
            r = loops.blt_d(W, wl, inp, 24, 4, alpha, unmask=mode, sampling=smp)
            assert r.out == g.out and r.n_dec == g.n_dec, (mode, smp)
    a = loops.blt_d(W, wl, inp, 24, 4, 2.0, unmask="entropy", sampling=(1.0, 0.9, 99), trace=True)
    b = loops.blt_d(W, wl, inp, 24, 4, 2.0, unmask="entropy", sampling=(1.0, 0.9, 99))
    g = loops.blt_d(W, wl, inp, 24, 4, 2.0, unmask="entropy")
    assert a.out == b.out and a.out != g.out
    for d, rec in enumerate(a.passes):
        assert rec["u"] == [decide.uniform(99, d * loops.MAX_BLOCK + j) for j in range(4)]


def test_sampled_blt_s_and_dv_limits_and_determinism(tiny):
    """Sampled BLT-S / BLT-DV (drafts drawn, rejection-sampling verification):
    a vanishing top_p reproduces greedy BLT-S (= greedy BLT) and greedy
    BLT-DV exactly; a seed reproduces its run; the verify draws follow the
    counter layout (pass d: d*64 + j, appended byte d*64 + r)."""
    wl, W, inp = tiny
    g = loops.greedy(W, wl, inp, 24)
    gs = loops.blt_s(W, wl, inp, 24, 4)
    gdv = loops.blt_dv(W, wl, inp, 24, 4, 0.7, one_step=True)
    lim_s = loops.blt_s(W, wl, inp, 24, 4, sampling=(1.0, 1e-9, 5))
    lim_dv = loops.blt_dv(W, wl, inp, 24, 4, 0.7, one_step=True, sampling=(1.0, 1e-9, 5))
    assert lim_s.out == gs.out == g.out and lim_s.n_dec == gs.n_dec and lim_s.accept == gs.accept
    assert lim_dv.out == gdv.out and lim_dv.n_dec == gdv.n_dec and lim_dv.accept == gdv.accept
    a = loops.blt_s(W, wl, inp, 24, 4, sampling=(1.0, 0.9, 7), trace=True)
    b = loops.blt_s(W, wl, inp, 24, 4, sampling=(1.0, 0.9, 7))
    assert a.out == b.out and a.out != g.out and len(a.out) == 24
    for d, rec in enumerate(a.passes):
        if rec["kind"] == "draft":
            assert rec["u"] == decide.uniform(7, d * loops.MAX_BLOCK)
        else:
            r = len(rec["tokens"]) - 1
            assert rec["u_acc"] == [decide.uniform(7, d * loops.MAX_BLOCK + j) for j in range(r)]
            assert rec["u_next"] == decide.uniform(7, d * loops.MAX_BLOCK + r)
    c = loops.blt_dv(W, wl, inp, 24, 4, 0.7, one_step=True, sampling=(1.0, 0.9, 7))
    assert len(c.out) == 24 and c.out != gdv.out


def test_blt_d_peaked_head_commits_several_per_pass():
    wl = bltgen.WORKLOADS[0].replace(head_scale=12.0)
    W = model.as64(bltgen.make_weights(wl))
    inp = bltgen.make_sequence_inputs(wl, 0)
    r = loops.blt_d(W, wl, inp, 32, 4, 0.7, trace=True)
    assert r.n_dec < 32 and max(len(p["chosen"]) for p in r.passes) > 1


def test_blt_dv_counts(tiny):
    wl, W, inp = tiny
    r = loops.blt_dv(W, wl, inp, 24, 8, 0.7, one_step=True)
    rounds = len(r.accept)
    assert r.n_eg == 2 * rounds and r.n_dec == 2 * rounds
    assert len(r.out) == 24


# ---------------------------------------------------------------- proxy
def test_proxy_worked_example():
    with open(os.path.join(GOLDEN, "proxy_example.json")) as f:
        g = json.load(f)
    gb = proxy.proxy_gb_per_seq(g["n_dec"], g["n_eg"], 1, g["p_dec"], g["p_enc"], g["p_glob"])
    assert float(gb) == g["gb"]


def test_decoder_param_count():
    assert proxy.decoder_params(bltgen.WORKLOADS[1]) == 153_637_888


# ---------------------------------------------------------------- BLT-S bookkeeping
class _ScriptedDecoder:
    """Stand-in for the cached decoder in the loops (same interface): row i
    with token x_i and latent target t predicts stream[i+1] when x_i is the
    stream's byte and t is row i's causal target in the stream's own
    segmentation, else (stream[i+1] + 1) mod 256.  A draft row that reads a
    stale latent therefore drafts a wrong byte, so accept lengths and pass
    counts expose which latent every row read."""
    stream = None
    ctarget = None

    def __init__(self, W, wl, latents, capacity):
        self.length = 0
        self.tau = np.full(capacity, -1, dtype=np.int64)

    def run(self, tokens, start, targets, n_append, block_causal=False):
        n = len(tokens)
        z = np.zeros((n, 257))
        for j in range(n):
            i = start + j
            right = int(tokens[j]) == self.stream[i] and int(targets[j]) == self.ctarget[i]
            z[j, self.stream[i + 1] if right else (self.stream[i + 1] + 1) % 256] = 1.0
        self.length = start + n_append
        return z

    def truncate(self, length):
        self.length = length


def test_blt_s_latent_bookkeeping_worked_example(monkeypatch):
    """Hand-worked BLT-S rounds (k = 4) on a segmentation whose patch
    boundaries fall inside drafts and on appended bytes: every draft row reads
    the newest latent produced before the round (stale past the boundary),
    the verify rows read their causal targets over the draft, and after a
    round only patches ending inside the accepted bytes are available (the
    appended correction or free byte was never seen by the encoder/global
    pass).  Dropping the stale cap, or counting the appended byte's patch as
    available, changes the accept lengths."""
    with open(os.path.join(GOLDEN, "blts_targets_example.json")) as f:
        g = json.load(f)
    stream = g["prompt"] + g["continuation"] + g["extension"]
    patch, ends = patcher.segment(stream, g["prompt_patches"], g["salt"])
    assert [int(i) for i in np.flatnonzero(ends)] == g["patch_ends"]
    # causal targets written from the definition: byte i reads the latent of
    # the previous patch, the last byte of a patch reads its own
    pe = set(g["patch_ends"])
    ctarget = []
    for i in range(len(stream)):
        p = sum(1 for e in pe if e < i)
        ctarget.append(p if i in pe else p - 1)
    _ScriptedDecoder.stream, _ScriptedDecoder.ctarget = stream, ctarget
    monkeypatch.setattr(loops, "CachedDecoder", _ScriptedDecoder)
    wl = bltgen.WORKLOADS[0]
    inp = {"prompt": np.array(g["prompt"]), "prompt_patches": np.array(g["prompt_patches"]),
           "salt": g["salt"], "latents": None}
    n_gen, k = len(g["continuation"]), g["k"]
    run = loops.blt_s(None, wl, inp, n_gen, k, trace=True)
    assert run.out == g["continuation"]                     # identical to greedy decoding
    assert run.accept == [r["accept"] for r in g["rounds"]]
    assert (run.n_dec, run.n_eg) == (g["n_dec"], g["n_eg"])
    recs = run.passes
    assert len(recs) == len(g["rounds"]) * (k + 1)
    for ri, r in enumerate(g["rounds"]):
        drafts, ver = recs[ri * (k + 1):ri * (k + 1) + k], recs[ri * (k + 1) + k]
        assert [d["kind"] for d in drafts] == ["draft"] * k and ver["kind"] == "verify"
        assert [d["start"] for d in drafts] == [r["l"] + j for j in range(k)]
        assert [d["targets"] for d in drafts] == [[r["draft_target"]]] * k, f"round {ri}"
        a = r["accept"]
        assert ver["start"] == r["l"] and ver["targets"][:a + 1] == r["verify_targets"], f"round {ri}"
        assert (ver["accept"], ver["next"]) == (a, r["next"])


def test_blt_s_bookkeeping_matches_greedy_targets_on_the_tiny_model(tiny):
    """On the real tiny decoder: BLT-S verify rows of the accepted prefix read
    the same latents the greedy decoder's rows read for those positions."""
    wl, W, inp = tiny
    g = loops.greedy(W, wl, inp, 40, trace=True)
    s = loops.blt_s(W, wl, inp, 40, 4, trace=True)
    assert s.out == g.out
    gt = {rec["start"]: rec["targets"][0] for rec in g.passes}
    checked = 0
    for rec in s.passes:
        if rec["kind"] == "verify":
            for j in range(rec["accept"] + 1):
                pos = rec["start"] + j
                if pos in gt:
                    assert rec["targets"][j] == gt[pos]
                    checked += 1
    assert checked > 20


# ---------------------------------------------------------------- full layer composition
def _torch_decoder(W, wl, latents, toks, pos, taus, allow):
    """Independent composition with torch routines of the BLT decoder layer
    (pytorch.kr summary, "BLT architecture": the cross-attention residual
    B_l = D_{l-1} + W_o^c softmax(.) V, then D_l = DecoderTransformerLayer(B_l),
    pre-norm self-attention then pre-norm FFN); every sublayer active."""
    t = lambda a: torch.tensor(np.asarray(a), dtype=torch.float64)
    d, H = wl.d_model, wl.n_heads
    dh = d // H
    n = len(toks)
    h = t(W["embed"])[torch.tensor(toks)]
    o = t(latents)[torch.tensor(taus)]                       # each row's single latent
    f = wl.rope_theta ** (-2.0 * torch.arange(dh // 2, dtype=torch.float64) / dh)
    rot = torch.polar(torch.ones(n, 1, dh // 2, dtype=torch.float64),
                      t(pos)[:, None, None] * f)

    def rope(x):
        x = x.view(n, H, dh)
        zc = torch.complex(x[..., :dh // 2], x[..., dh // 2:]) * rot
        return torch.cat([zc.real, zc.imag], -1).transpose(0, 1)

    for lw in W["layers"]:
        # cross-attention: SDPA over the one allowed latent key per row
        ot = Fnn.linear(o, t(W["w_lat"]))
        qc = Fnn.linear(h, t(lw["wq_c"])).view(n, H, 1, dh)
        kc = Fnn.linear(ot, t(lw["wk_c"])).view(n, H, 1, dh)
        vc = Fnn.linear(ot, t(lw["wv_c"])).view(n, H, 1, dh)
        c = Fnn.scaled_dot_product_attention(qc, kc, vc).reshape(n, d)
        h = h + Fnn.linear(c, t(lw["wo_c"]))
        u = Fnn.rms_norm(h, (d,), weight=t(lw["g_attn"]), eps=wl.rms_eps)
        qkv = Fnn.linear(u, t(lw["wqkv"]))
        q, k = rope(qkv[:, :d]), rope(qkv[:, d:2 * d])
        v = qkv[:, 2 * d:].reshape(n, H, dh).transpose(0, 1)
        a = Fnn.scaled_dot_product_attention(q, k, v, attn_mask=torch.tensor(allow))
        h = h + Fnn.linear(a.transpose(0, 1).reshape(n, d), t(lw["wo"]))
        u = Fnn.rms_norm(h, (d,), weight=t(lw["g_ffn"]), eps=wl.rms_eps)
        h = h + Fnn.linear(Fnn.silu(Fnn.linear(u, t(lw["w1"]))), t(lw["w2"]))
    u = Fnn.rms_norm(h, (d,), weight=t(W["g_out"]), eps=wl.rms_eps)
    return Fnn.linear(u, t(W["w_out"])).numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_two_layer_forward_every_sublayer_matches_torch_composition(causal):
    """Two layers with cross-attention, self-attention and FFN all active
    (random gains, random weights scaled up so every sublayer moves the
    logits): the oracle's forward equals the torch composition; and each
    sublayer matters (zeroing its output projection moves the logits), so a
    reordered or dropped sublayer fails this pin."""
    wl, W, inp = micro(n_layers=2)
    for lw in W["layers"]:
        for key in ("wo_c", "wv_c", "wqkv", "wo", "w1", "w2"):
            lw[key] = lw[key] * 8.0
    toks = [5, 200, 17, 256, 31, 256]
    pos = np.array([7, 8, 9, 10, 11, 12])
    taus = [1, 1, 2, 3, 3, 3]
    allow = model.blt_d_mask(3, 3, causal)
    z = model.forward(W, wl, inp["latents"], toks, pos, [[t] for t in taus], allow)
    want = _torch_decoder(W, wl, inp["latents"], toks, pos, taus, allow)
    np.testing.assert_allclose(z, want, rtol=1e-10, atol=1e-11)
    for key in ("wo_c", "wo", "w2"):
        zz = model.forward(_zero(W, {key}), wl, inp["latents"], toks, pos, [[t] for t in taus], allow)
        assert np.abs(zz - z).max() > 1e-3 * np.abs(z).max(), key
