"""Write the full-size golden traces used by tests/test_gpu_fullsize.py.

For each full-size workload, the float64 CPU oracle (oracle/) runs the
workload's decode policy on a few sampled sequences of the batch (seeded
synthetic inputs from bltgen) just long enough to cover its first round,
with pass tracing on, and the first passes of that trace are stored (into
the second block or round where the plan says so):
rows, latent targets, logits, greedy choices, confidences, top-2 gaps and
the block or acceptance decisions.  Nothing here calls the HIP path.

    python tests/golden/make_fullsize.py [workload ...]

Output: tests/golden/fullsize_<workload name>.npz (a few hundred KB in all).
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import bltgen  # noqa: E402
from oracle import loops, model  # noqa: E402

# workload index -> (sampled sequences, bytes to generate, passes kept)
PLAN = {
    1: ([0], 8, 5),        # BLT-D-4, batch 1: the first block and the second block's first
                           # pass (rollback of the last prompt row, the block's bytes appended)
    2: ([0, 15], 16, 2),   # BLT-D-16, batch 16: the first two block passes
    3: ([0], 10, 18),      # BLT-S k=8, batch 1: two rounds of 8 draft passes and a verification
    4: ([0, 21, 42, 63], 1, 2),   # BLT-DV-8 one-step, batch 64: draft pass and verification
}
KINDS = {"block": 0, "draft": 1, "verify": 2, "ar": 3}

# Maximum-context cases: prompts that fill the cache's 16384 rows (128
# attention chunks) for the float32 tiny decoder and a 2-layer bfloat16 one;
# the first block of BLT-D-4 (threshold) and BLT-D-16 (one step).
LONG = {
    "long_fp32": bltgen.WORKLOADS[0].replace(name="tiny_bltd4_fp32_b1_ctx16k", prompt_len=16350,
                                             prompt_patches=4100, n_gen=8),
    "long_bf16": bltgen.WORKLOADS[1].replace(name="mini_bltd16_bf16_b1_ctx16k", n_layers=2,
                                             d_model=256, n_heads=4, d_ffn=1024, d_global=512,
                                             prompt_len=16320, prompt_patches=4000, n_gen=16,
                                             block=16, unmask="one_step"),
}


def path_for(wl):
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), f"fullsize_{wl.name}.npz")


def make(k):
    if k in LONG:
        wl, (seqs, n_gen, keep) = LONG[k], ([0], LONG[k].block, 99)
    else:
        wl = bltgen.WORKLOADS[k]
        seqs, n_gen, keep = PLAN[k]
    W = model.as64(bltgen.make_weights(wl))
    out = {"workload": np.int64(k if isinstance(k, int) else -1), "seqs": np.asarray(seqs, dtype=np.int64),
           "n_passes": np.int64(keep)}
    for s in seqs:
        t0 = time.perf_counter()
        inp = bltgen.make_sequence_inputs(wl, s)
        inp = dict(inp, latents=inp["latents"].astype(np.float64))
        run = loops.run_policy(W, wl, inp, trace=True, n_gen=n_gen)
        keep = min(keep, len(run.passes)) if k in LONG else keep
        out["n_passes"] = np.int64(keep)
        assert len(run.passes) >= keep, (wl.name, s, len(run.passes))
        for i, rec in enumerate(run.passes[:keep]):
            p = f"s{s}_p{i}_"
            out[p + "kind"] = np.int64(KINDS[rec["kind"]])
            out[p + "start"] = np.int64(rec["start"])
            out[p + "n_append"] = np.int64(rec["n_append"])
            out[p + "tokens"] = np.asarray(rec["tokens"], dtype=np.int64)
            out[p + "targets"] = np.asarray(rec["targets"], dtype=np.int64)
            out[p + "logits"] = np.asarray(rec["logits"], dtype=np.float64)
            out[p + "choice"] = np.asarray(rec["choice"], dtype=np.int64)
            out[p + "gap"] = np.asarray(rec["gap"], dtype=np.float64)
            if rec["kind"] == "block":
                out[p + "conf"] = np.asarray(rec["conf"], dtype=np.float64)
                out[p + "block_before"] = np.asarray(rec["block_before"], dtype=np.int64)
                out[p + "block_after"] = np.asarray(rec["block_after"], dtype=np.int64)
                out[p + "block_causal"] = np.int64(bool(rec["block_causal"]))
            if rec["kind"] == "verify":
                out[p + "accept"] = np.int64(rec["accept"])
                out[p + "next"] = np.int64(rec["next"])
        print(f"{wl.name} seq {s}: {len(run.passes)} passes traced, kept {keep}, "
              f"{time.perf_counter() - t0:.1f} s", flush=True)
    np.savez_compressed(path_for(wl), **out)


if __name__ == "__main__":
    for a in sys.argv[1:] or [str(k) for k in sorted(PLAN)] + sorted(LONG):
        make(a if a in LONG else int(a))
