"""Decoded bytes/s of the Fast-BLT local byte decoder step on one MI355X.

One step = one full generation of the workload's bytes from its prefilled
prompt through the native decode driver (every decoder pass, the stand-in
encoder/global passes with their latent projections, unmasking and commit).
Inputs (weights, latents, prompts) are seeded synthetic data resident in HBM
before the timed region; the prefill is not timed.

Default workload: BLT-D-4, bf16, batch 1, 9 layers, d 1024, 16 heads, FFN
4096, 4096-byte Zipf(1.1) prompt with 1024 patches, 1024 bytes generated.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PROFILE_MD = os.path.join(ROOT, "profiles", "k_attn_mfma_bltd4_bf16_b1_ctx4096.md")
KERNELS_SRC = os.path.join(ROOT, "block_diffusion_byte_amd", "csrc", "kernels.hip")


def kernel_source_sha256(name):
    """sha256 of one kernel's definition in kernels.hip: from its template
    line to the closing brace at the start of a line."""
    import hashlib
    src = open(KERNELS_SRC).read()
    i = src.index(f"void {name}(")
    i = src.rindex("template", 0, i)
    j = src.index("\n}\n", i) + 3
    return hashlib.sha256(src[i:j].encode()).hexdigest()


def measured_traffic(workload_index):
    """HBM bytes per attention launch from the committed rocprofv3 PMC summary
    (FETCH_SIZE + WRITE_SIZE scaled by a plain copy), or None when the summary
    is for another workload or the kernel's source changed since it was taken."""
    if workload_index != 1 or not os.path.exists(PROFILE_MD):
        return None
    fields = {}
    for line in open(PROFILE_MD):
        if ":" in line and not line.startswith(("#", "-", "|", "`")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("k_attn_mfma_source_sha256") != kernel_source_sha256("k_attn_mfma"):
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", type=int, default=1, help="index of the workload (0..4)")
    ap.add_argument("--cpu-bytes", type=int, default=None,
                    help="bytes the CPU oracle decodes for the baseline (default: per workload)")
    ap.add_argument("--cpu-ctx", type=int, default=2048, help="context bytes of the CPU sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB ten times (the "
                         "reference kernel for scaling HBM traffic counters) and exit")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--max-rows", type=int, default=0,
                    help="rows per decoder pass (default: the whole prompt, so prefill is one pass)")
    ap.add_argument("--no-graphs", action="store_true",
                    help="launch every decoder pass directly instead of replaying HIP graphs")
    return ap.parse_args()


def policy_id(blt, wl):
    return {"blt_d": blt.BLT_POLICY_BLT_D, "blt_s": blt.BLT_POLICY_BLT_S,
            "blt_dv": blt.BLT_POLICY_BLT_DV}[wl.policy]


def cpu_baseline(wl, w, n_bytes, ctx):
    """The oracle, as it stands, on a bounded sample of the same workload:
    sequence 0 only, decoding after an untimed prefill."""
    import numpy as np
    import bltgen
    from oracle import loops, model
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    W = model.as64(w)
    inp = bltgen.make_sequence_inputs(wl, 0)
    inp["latents"] = inp["latents"].astype(np.float64)
    # The oracle's prefill is quadratic in single-threaded NumPy; the sample
    # decodes after the first whole patches of the prompt up to ctx bytes.
    lens = np.asarray(inp["prompt_patches"])
    keep = int(np.searchsorted(np.cumsum(lens), ctx, side="right"))
    keep = max(keep, 1)
    n_ctx = int(lens[:keep].sum())
    inp = dict(inp, prompt=inp["prompt"][:n_ctx], prompt_patches=lens[:keep])
    t0 = time.perf_counter()
    ref = loops.run_policy(W, wl, inp, n_gen=n_bytes)
    t_all = time.perf_counter() - t0
    t_pre = ref.prefill_s
    t_dec = max(t_all - t_pre, 1e-9)
    return {"value": n_bytes / t_dec, "unit": "bytes/s", "cores": int(cores), "kind": "oracle",
            "sample": f"sequence 0 of the same workload, context cut to the first {n_ctx} prompt bytes "
                      f"({keep} patches), {n_bytes} bytes decoded: {ref.n_dec} decoder passes in "
                      f"{t_dec:.1f} s (prefill {t_pre:.1f} s, untimed)"}


def prefill_report(rows, seconds, max_rows, launches, ms, flops):
    """Prompt prefill: rows per second, and the causal attention kernel's
    achieved bf16 MFMA rate (algorithmic flops / event-timed duration)."""
    avg_us = 1e3 * ms / max(launches, 1)
    fpl = flops / max(launches, 1)
    tflops = fpl / (avg_us * 1e-6) / 1e12 if launches else 0.0
    return {"rows": rows, "seconds": seconds, "rows_per_s": rows / seconds,
            "rows_per_pass": max_rows,
            "roofline": {"bound": "mfma", "kernel": "k_attn_flash (causal attention, MFMA bf16)",
                         "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "launches": launches,
                         "avg_us": avg_us, "flops_per_launch": fpl}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the decoder path runs on a single GPU); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 20
        x = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        y = torch.empty_like(x)
        x.fill_(1)
        for _ in range(10):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "launches": 10}))
        return

    import bltgen
    import block_diffusion_byte_amd as blt
    from oracle import proxy

    wl = bltgen.WORKLOADS[args.workload]
    dev = "cuda:0"
    w = bltgen.make_weights(wl)
    inps = [bltgen.make_sequence_inputs(wl, b) for b in range(wl.batch)]
    # one prefill pass per prompt (the causal kernel wants long passes), and
    # room for the largest decode pass
    max_rows = args.max_rows or max(1024, wl.batch * (2 * wl.block + 2), wl.prompt_len)
    dec = blt.Decoder(w, n_layers=wl.n_layers, d_model=wl.d_model, n_heads=wl.n_heads,
                      d_ffn=wl.d_ffn, d_global=wl.d_global, dtype=wl.dtype, max_batch=wl.batch,
                      max_ctx=wl.max_ctx, max_latents=wl.n_latents, max_rows=max_rows,
                      max_block=wl.block, rope_theta=wl.rope_theta, rms_eps=wl.rms_eps, device=dev)
    if args.no_graphs:
        blt.blt_graphs_enable(dec.ctx, False)
    table = torch.empty((wl.batch, wl.n_latents, wl.d_global), dtype=dec.torch_dtype, device=dev)
    for b, inp in enumerate(inps):
        table[b].copy_(torch.from_numpy(inp["latents"]))
    sess = blt.blt_session_create(dec.ctx, dec.state, [i["prompt"] for i in inps],
                                  [i["prompt_patches"] for i in inps], [i["salt"] for i in inps],
                                  table, wl.n_latents)
    # Prefill (the prompts' clean rows through blt_kv_append): once to warm
    # up, once timed, once with the causal attention kernel's launches
    # stamped by HIP events (its average duration and algorithmic flops).
    blt.blt_session_prefill(dec.ctx, sess)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    blt.blt_session_prefill(dec.ctx, sess)
    torch.cuda.synchronize()
    t_prefill = time.perf_counter() - t0
    blt.blt_profile_enable(dec.ctx, blt.BLT_PROF_ATTENTION_CAUSAL)
    blt.blt_profile_read(dec.ctx, reset=True)
    blt.blt_session_prefill(dec.ctx, sess)
    pf_launches, pf_ms, pf_flops = blt.blt_profile_read(dec.ctx, reset=True)
    blt.blt_profile_enable(dec.ctx, blt.BLT_PROF_OFF)
    prefill_rows = sum(len(i["prompt"]) - 1 for i in inps)
    unmask = blt.BLT_UNMASK_ONE_STEP if wl.unmask == "one_step" else blt.BLT_UNMASK_THRESHOLD
    pid = policy_id(blt, wl)

    def step():
        blt.blt_session_generate(dec.ctx, sess, pid, wl.block, wl.alpha, wl.n_gen, unmask)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # Same steps again with the attention kernel bracketed by HIP events on the
    # library's stream: its average launch duration and algorithmic bytes.
    blt.blt_profile_enable(dec.ctx, blt.BLT_PROF_ATTENTION)
    blt.blt_profile_read(dec.ctx, reset=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed_prof = time.perf_counter() - t1
    launches, kern_ms, kern_bytes = blt.blt_profile_read(dec.ctx, reset=True)
    blt.blt_profile_enable(dec.ctx, blt.BLT_PROF_OFF)
    avg_us = 1e3 * kern_ms / max(launches, 1)
    bytes_per_launch = kern_bytes / max(launches, 1)
    achieved = bytes_per_launch / (avg_us * 1e-6) / 1e9
    res = [blt.blt_session_result(sess, b, wl.n_gen) for b in range(wl.batch)]
    total_bytes = sum(r["n"] for r in res) * args.steps
    n_dec = sum(r["n_dec"] for r in res)
    n_eg = sum(r["n_eg"] for r in res)
    p_dec = proxy.decoder_params(wl)
    gb_counted = blt.blt_bw_model(n_dec, n_eg, wl.batch, p_dec, wl.p_enc, wl.p_glob)[1]
    gb_pages = blt.blt_bw_model(n_dec, n_eg, wl.batch, 160_000_000, wl.p_enc, wl.p_glob)[1]

    out = {
        "metric": "decoded bytes/sec",
        "value": total_bytes / elapsed,
        "unit": "bytes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * elapsed / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,0.02) decoder weights, N(0,1) latents, Zipf/uniform byte prompts)",
        "config": {"workload": wl.name, "policy": wl.policy, "batch": wl.batch, "block": wl.block,
                   "alpha": wl.alpha, "layers": wl.n_layers, "d_local": wl.d_model,
                   "heads": wl.n_heads, "ffn": wl.d_ffn, "d_global": wl.d_global,
                   "prompt_bytes": wl.prompt_len, "latents": wl.prompt_patches,
                   "bytes_generated": wl.n_gen},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(args.workload),
                     "kernel": "k_attn_mfma (split-K attention partials, MFMA)",
                     "launches": launches, "avg_us": avg_us, "bytes_per_launch": bytes_per_launch,
                     "ms_per_step_with_events": 1e3 * elapsed_prof / args.steps},
        "counters": {"decoder_passes_per_seq": n_dec / wl.batch,
                     "encglob_passes_per_seq": n_eg / wl.batch,
                     "proxy_gb_per_seq_counted_params": gb_counted,
                     "proxy_gb_per_seq_pages_params": gb_pages,
                     "prefill_s": t_prefill},
        "prefill": prefill_report(prefill_rows, t_prefill, max_rows, pf_launches, pf_ms, pf_flops),
    }
    if not args.no_cpu:
        n_cpu = args.cpu_bytes or {0: 64, 1: 128, 2: 128, 3: 128, 4: 48}[args.workload]
        out["cpu_baseline"] = cpu_baseline(wl, w, n_cpu, args.cpu_ctx)
    blt.blt_session_destroy(sess)
    dec.close()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
