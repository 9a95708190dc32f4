"""Per-pass decisions (oracle; test infrastructure only).

  * byte_choice: the greedy byte and its confidence from one row's logits;
  * unmask_commit: confidence-threshold unmasking with the forced fallback,
    or one-step filling;
  * entropy / unmask_commit_entropy: entropy-bounded (EB) unmasking;
  * verify_accept: the greedy exact-match verification of a draft;
  * uniform / sample_top_p: temperature and top-p (nucleus) sampling of a
    position's byte, the stochastic variant the pages pair with EB sampling;
  * sampling_dist / verify_sample: verification of sampled drafts by
    rejection sampling (the extension to temperature > 0 the pages mention).
"""
from __future__ import annotations

import numpy as np

from . import patcher

MASK = 256


def byte_choice(z):
    """Greedy byte and confidence of one row of 257 logits.

    A masked slot is filled with a byte, so the [MASK] logit (id 256) takes
    no part.  Confidence is the largest predicted probability (pytorch.kr
    Fast-BLT summary, "block unmasking strategies": the maximum predicted
    probability of a position is its confidence).  Ties go to the lowest
    byte id.  Returns (byte, confidence, top-2 logit gap).
    """
    z = np.asarray(z, dtype=np.float64)[:256]
    m = z.max()
    b = int(np.flatnonzero(z == m)[0])
    conf = 1.0 / np.exp(z - m).sum()
    rest = np.delete(z, b)
    return b, float(conf), float(m - rest.max())


def unmask_commit(block, choice, conf, alpha, one_step=False):
    """Commit block positions after one decoder pass.

    block: current block tokens (256 = still masked); choice/conf: per block
    position greedy byte and confidence from this pass.  Rule (pytorch.kr
    summary, "block unmasking strategies"): every masked position whose
    confidence exceeds alpha is committed at once; if none does, the single
    most confident masked position is committed so decoding always advances
    (ties to the lowest position).  One-step diffusion fills every masked
    position in a single pass (the BLT-DV one-step draft).  Committed
    positions stay committed.  Returns (new block, committed positions).
    """
    block = list(block)
    masked = [i for i, t in enumerate(block) if t == MASK]
    if not masked:
        return block, []
    if one_step:
        chosen = masked
    else:
        chosen = [i for i in masked if conf[i] > alpha]
        if not chosen:
            best = max(conf[i] for i in masked)
            chosen = [min(i for i in masked if conf[i] == best)]
    for i in chosen:
        block[i] = int(choice[i])
    return block, chosen


def entropy(z):
    """Entropy in nats of the byte distribution of one row of 257 logits.

    The distribution is the softmax over bytes 0..255 ([MASK] takes no part,
    as for the greedy byte): H = -sum_b p_b log p_b.
    """
    z = np.asarray(z, dtype=np.float64)[:256]
    p = np.exp(z - z.max())
    p = p / p.sum()
    nz = p[p > 0]
    return float(-(nz * np.log(nz)).sum())


def unmask_commit_entropy(block, choice, ent, gamma):
    """Entropy-bounded unmasking after one decoder pass.

    pytorch.kr summary, "block unmasking strategies" (EB sampling): the
    masked positions are ranked by the entropy of their prediction, lowest
    first, and the largest set of them whose summed entropy does not exceed
    gamma is decoded at once.  Readings: equal entropies rank by position;
    the entropies are summed in rank order; at least the lowest-entropy
    position is committed, so decoding always advances (as the forced commit
    of the threshold rule).  Committed positions take their greedy byte and
    stay committed.  Returns (new block, committed positions in order).
    """
    block = list(block)
    masked = [i for i, t in enumerate(block) if t == MASK]
    if not masked:
        return block, []
    order = sorted(masked, key=lambda i: (ent[i], i))
    total, n = 0.0, 0
    for i in order:
        total += ent[i]
        if total > gamma:
            break
        n += 1
    chosen = sorted(order[:max(n, 1)])
    for i in chosen:
        block[i] = int(choice[i])
    return block, chosen


def verify_accept(draft, pred):
    """Greedy exact-match verification.

    draft: the r draft bytes x'_{l+1..l+r}; pred: the r+1 greedy predictions
    y_l..y_{l+r}, pred[j] being the byte the causal pass predicts after
    position l+j.  Walking i = l+1..l+r, a draft byte is accepted while it
    equals the prediction made at the position before it; at the first
    mismatch the prediction replaces it and the walk stops; if every draft
    byte matches, the prediction after the last one is a free extra byte
    (pytorch.kr summary, "BLT-S and BLT-DV": the shared verification steps).
    Returns (accepted count a, the byte appended after them).
    """
    r = len(draft)
    if len(pred) != r + 1:
        raise ValueError("need r + 1 predictions")
    a = 0
    while a < r and int(draft[a]) == int(pred[a]):
        a += 1
    return a, int(pred[a])


def uniform(seed, counter):
    """A uniform number in [0, 1) with 24 random bits for draw ``counter``
    (>= 0) of the stream ``seed``: the top 24 bits of output counter + 1 of
    SplitMix64 started from state ``seed`` (Steele, Lea and Flood, 2014),
    divided by 2^24 (exact in float32 and float64)."""
    return (patcher.splitmix64_nth(seed, counter + 1) >> 40) / float(1 << 24)


def sample_top_p(z, temperature, top_p, u):
    """Temperature and top-p (nucleus) sampling of one masked position.

    pytorch.kr summary, "block unmasking strategies": EB sampling can be
    combined with top-p sampling to control the diversity of the output; the
    pages give no further detail, so the plainest reading of nucleus
    sampling is taken:
      p_b = softmax(z_b / temperature) over bytes 0..255 ([MASK] excluded);
      bytes ranked by p descending, equal probabilities by byte id;
      the nucleus is the shortest prefix of that ranking whose mass reaches
      top_p (a byte belongs to it iff the mass ranked before it is below
      top_p; bytes of probability 0 never do);
      with c = u * (mass of the nucleus), the chosen byte is the last byte
      of the nucleus, in rank order, whose preceding mass is <= c (the byte
      whose interval [before, before + p) of the nucleus holds c).
    Temperature and top-p shape only the draw: the position's confidence is
    the model's probability of the drawn byte and its entropy that of the
    model's distribution (temperature 1, as in greedy decoding), so the
    unmask rules judge positions the same way and the limits top_p -> 0 or
    temperature -> 0 are greedy decoding.
    Returns (byte, model probability of the byte, model entropy in nats,
    margin): margin is the smallest distance, in probability, between a
    quantity that decides the draw and its threshold (c to the chosen
    interval's ends, and the preceding mass of the nucleus' last byte and of
    the first byte left out to top_p); a computation whose probabilities are
    off by less than the margin draws the same byte.
    """
    z = np.asarray(z, dtype=np.float64)[:256]
    q = np.exp(z - z.max())
    q = q / q.sum()
    nz = q[q > 0]
    ent = float(-(nz * np.log(nz)).sum())
    y = z / float(temperature)
    e = np.exp(y - y.max())
    p = e / e.sum()
    order = sorted(range(256), key=lambda b: (-p[b], b))
    before = np.concatenate([[0.0], np.cumsum([p[b] for b in order])[:-1]])
    inside = [i for i in range(256) if before[i] < top_p and p[order[i]] > 0]
    n = len(inside)                     # the nucleus is order[:n]
    mass = float(sum(p[order[i]] for i in range(n)))
    c = u * mass
    k = max(i for i in range(n) if before[i] <= c)
    b = order[k]
    margin = min(c - before[k], before[k] + p[b] - c, top_p - before[n - 1])
    if n < 256:
        margin = min(margin, before[n] - top_p)
    return b, float(q[b]), ent, float(margin)


def sampling_dist(z, temperature, top_p):
    """The distribution sample_top_p draws from: softmax(z / temperature)
    over bytes 0..255 restricted to the nucleus and renormalised (0 outside
    it).  Returns a float64 vector of 256 probabilities."""
    y = np.asarray(z, dtype=np.float64)[:256] / float(temperature)
    e = np.exp(y - y.max())
    p = e / e.sum()
    order = sorted(range(256), key=lambda b: (-p[b], b))
    before = 0.0
    d = np.zeros(256)
    for b in order:
        if before < top_p and p[b] > 0:
            d[b] = p[b]
        before += p[b]
    return d / d.sum()


def verify_sample(draft, q, p, u_acc, u_next):
    """Rejection-sampling verification of a sampled draft.

    pytorch.kr summary, "BLT-S and BLT-DV": sampling at temperature > 0
    extends the shared verification by rejection sampling (mentioned, not
    evaluated, and not spelled out there).  The plainest reading is the
    standard speculative-sampling rule.  draft: the r draft bytes
    x'_{l+1..l+r}; q[j]: the distribution draft byte j was drawn from; p[j]
    (j = 0..r): the target distribution of the byte after verify row l+j
    (sampling_dist of that row's logits).  For j = 0, 1, ...: x = draft[j]
    is accepted iff u_acc[j] * q[j][x] < p[j][x] (probability
    min(1, p/q)); at the first rejection the appended byte is drawn from
    max(0, p[j] - q[j]) renormalised, walking bytes in id order (the first
    byte whose cumulative residual mass exceeds u_next times the total); if
    every draft byte is accepted, the free byte is drawn from p[r] as
    sample_top_p draws (bytes ranked by probability, ties by id, the first
    whose cumulative mass exceeds u_next).  Returns (accepted count a,
    appended byte, margin): margin is the smallest distance, in
    probability, between a quantity that decided the outcome and its
    threshold.
    """
    r = len(draft)
    if len(q) != r or len(p) != r + 1:
        raise ValueError("need r draft distributions and r + 1 target distributions")
    margin = np.inf
    for j in range(r):
        x = int(draft[j])
        qj, pj = np.asarray(q[j], dtype=np.float64), np.asarray(p[j], dtype=np.float64)
        t = u_acc[j] * qj[x]
        margin = min(margin, abs(pj[x] - t))
        if t < pj[x]:
            continue
        res = np.maximum(pj - qj, 0.0)
        cum = np.cumsum(res)
        c = u_next * cum[-1]
        b = int(np.flatnonzero(cum > c)[0])
        lo = cum[b - 1] if b > 0 else 0.0
        return j, b, float(min(margin, c - lo, cum[b] - c))
    pr = np.asarray(p[r], dtype=np.float64)
    order = sorted(range(256), key=lambda b: (-pr[b], b))
    cum = np.cumsum([pr[b] for b in order])
    k = int(np.flatnonzero(cum > u_next)[0])
    lo = cum[k - 1] if k > 0 else 0.0
    return r, order[k], float(min(margin, u_next - lo, cum[k] - u_next))
