"""A fixed set of native decode sessions (test infrastructure for
tests/test_gpu_checked_builds.py).

run_all() runs them through the Python binding (the release library) and
write_cases() writes them out for tests/host/session_driver.cpp, a plain C++
program over the C-ABI, so the checked library builds run the same sessions
in a process without Python or torch.  The weights, prompts and latents come
from bltgen's seeded generators; bfloat16 values are rounded by torch exactly
as the binding rounds them on upload.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import bltgen  # noqa: E402

TINY = bltgen.WORKLOADS[0]
# a 2-layer bfloat16 decoder whose block passes of 2 x 17 rows take the MFMA GEMM
MINI = bltgen.WORKLOADS[1].replace(name="mini_bf16", n_layers=2, d_model=256, n_heads=4, d_ffn=1024,
                                   d_global=512, prompt_len=96, prompt_patches=24, head_scale=12.0)
BATCH, N_GEN, MAX_ROWS = 2, 24, 128
POLICY = {"greedy": 0, "blt_d": 1, "blt_s": 2, "blt_dv": 3}

# workload -> runs (name, policy, block, alpha, unmask, device blocks, (temperature, top_p, seed))
CASES = [
    (TINY, [("greedy", "greedy", 4, 0.7, 0, False, None),
            ("blt_d_threshold", "blt_d", 4, 0.7, 0, False, None),
            ("blt_d_device_blocks", "blt_d", 4, 0.7, 0, True, None),
            ("blt_d_entropy", "blt_d", 8, 1.5, 2, False, None),
            ("blt_s", "blt_s", 4, 0.0, 0, False, None),
            ("blt_dv_one_step", "blt_dv", 4, 0.7, 1, False, None),
            ("blt_dv_sampled", "blt_dv", 4, 0.7, 0, False, (0.8, 0.9, 1234))]),
    (MINI, [("mini_bf16_blt_d_b16", "blt_d", 16, 0.5, 0, False, None)]),
]


def _inputs(wl):
    return bltgen.make_weights(wl), [bltgen.make_sequence_inputs(wl, b) for b in range(BATCH)]


def run_all():
    """{run name: [per sequence: out, n, n_dec, n_eg, rounds, accepted]} via the binding."""
    import torch
    import block_diffusion_byte_amd as blt
    res = {}
    for wl, runs in CASES:
        w, inps = _inputs(wl)
        for name, policy, block, alpha, unmask, device, smp in runs:
            print(f"case {name}", file=sys.stderr, flush=True)
            dec = blt.Decoder(w, n_layers=wl.n_layers, d_model=wl.d_model, n_heads=wl.n_heads,
                              d_ffn=wl.d_ffn, d_global=wl.d_global, dtype=wl.dtype, max_batch=BATCH,
                              max_ctx=wl.max_ctx, max_latents=wl.n_latents, max_rows=MAX_ROWS,
                              max_block=block, rope_theta=wl.rope_theta, rms_eps=wl.rms_eps,
                              device="cuda:0")
            table = torch.from_numpy(np.stack([i["latents"] for i in inps])).to("cuda:0", dec.torch_dtype)
            sess = blt.blt_session_create(dec.ctx, dec.state, [i["prompt"] for i in inps],
                                          [i["prompt_patches"] for i in inps], [i["salt"] for i in inps],
                                          table, wl.n_latents)
            try:
                blt.blt_session_device_blocks(dec.ctx, sess, device)
                blt.blt_session_prefill(dec.ctx, sess)
                kw = {} if smp is None else {"temperature": smp[0], "top_p": smp[1], "seed": smp[2]}
                blt.blt_session_generate(dec.ctx, sess, POLICY[policy], block, alpha, N_GEN, unmask, **kw)
                out = [blt.blt_session_result(sess, b, N_GEN) for b in range(BATCH)]
            finally:
                blt.blt_session_destroy(sess)
                dec.close()
            res[name] = [[list(r["out"]), r["n"], r["n_dec"], r["n_eg"], r["rounds"], r["accepted"]]
                         for r in out]
    return res


def _dtype_bytes(a, bf16):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().tobytes() if bf16 else t.numpy().tobytes()


def write_cases(root):
    """One case folder per workload under root; returns [(folder, run names)]."""
    out = []
    for k, (wl, runs) in enumerate(CASES):
        d = os.path.join(root, f"case{k}")
        os.makedirs(d, exist_ok=True)
        w, inps = _inputs(wl)
        bf = wl.dtype == "bf16"
        for key in ("embed", "w_lat", "w_out", "g_out"):
            open(os.path.join(d, key + ".bin"), "wb").write(_dtype_bytes(w[key], bf))
        for l, lw in enumerate(w["layers"]):
            for key in ("wv_c", "wo_c", "wqkv", "wo", "g_attn", "g_ffn", "w1", "w2"):
                open(os.path.join(d, f"L{l}_{key}.bin"), "wb").write(_dtype_bytes(lw[key], bf))
        open(os.path.join(d, "latents.bin"), "wb").write(
            _dtype_bytes(np.stack([i["latents"] for i in inps]), bf))
        lines = [f"{wl.n_layers} {wl.d_model} {wl.n_heads} {wl.d_ffn} {wl.d_global} {int(bf)} {BATCH} "
                 f"{wl.max_ctx} {wl.n_latents} {MAX_ROWS} 0 {wl.rope_theta!r} {wl.rms_eps!r}",
                 f"{BATCH} {wl.n_latents}"]
        for i in inps:
            lines += [f"{len(i['prompt'])} {len(i['prompt_patches'])} {int(i['salt'])}",
                      " ".join(str(int(x)) for x in i["prompt"]),
                      " ".join(str(int(x)) for x in i["prompt_patches"])]
        lines.append(str(len(runs)))
        for name, policy, block, alpha, unmask, device, smp in runs:
            t, p, s = smp if smp else (0.0, 1.0, 0)
            lines.append(f"{POLICY[policy]} {block} {alpha!r} {unmask} {int(device)} {t!r} {p!r} {s} {N_GEN}")
        open(os.path.join(d, "case.txt"), "w").write("\n".join(lines) + "\n")
        out.append((d, [r[0] for r in runs]))
    return out


def parse_driver(stdout, names):
    """The driver's lines as run_all() returns them, for the runs `names`."""
    res = {n: [None] * BATCH for n in names}
    for line in stdout.splitlines():
        f = line.split()
        if not f or f[0] != "R":
            continue
        ri, b, n = int(f[1]), int(f[2]), int(f[3])
        res[names[ri]][b] = [[int(x) for x in f[8:]], n, int(f[4]), int(f[5]), int(f[6]), int(f[7])]
    return res
