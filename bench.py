"""Decoded bytes/s of the Fast-BLT local byte decoder step on one MI355X.

One step = one full generation of the workload's bytes from its prefilled
prompt through the native decode driver (every decoder pass, the stand-in
encoder/global passes with their latent projections, unmasking and commit).
Inputs (weights, latents, prompts) are seeded synthetic data resident in HBM
before the timed region; the prefill is not timed.

Main line (the metric at batch 1): BLT-D-4, bf16, batch 1, 9 layers, d 1024,
16 heads, FFN 4096, 4096-byte Zipf(1.1) prompt with 1024 patches, 1024 bytes
generated.  Further legs in the same JSON line: "batch64" (BLT-DV-8 one-step,
bf16, batch 64, d 1536, 8192-byte prompts: the metric at batch 64) and
"peaked" (the batch-1 workload with the byte head scaled x12, so passes
commit several block positions).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1] [--no-legs] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E (published)
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PAGES_P_DEC = 160_000_000        # decoder size the pages use for the proxy (both scales)
KERNELS_SRC = os.path.join(ROOT, "block_diffusion_byte_amd", "csrc", "kernels.hip")
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_sha256(name):
    """sha256 of one kernel's definition in kernels.hip: from its template
    line to the closing brace at the start of a line."""
    import hashlib
    src = open(KERNELS_SRC).read()
    i = src.index(f"void {name}(")
    i = src.rindex("template", 0, i)
    j = src.index("\n}\n", i) + 3
    return hashlib.sha256(src[i:j].encode()).hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` at `workload` from a committed
    rocprofv3 PMC summary (FETCH_SIZE + WRITE_SIZE scaled by a plain copy),
    or None when there is none or the kernel's source changed since."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "-", "|", "`", " ")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get(f"{kernel}_source_sha256") != kernel_source_sha256(kernel):
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", type=int, default=1, help="index of the main workload (0..4)")
    ap.add_argument("--no-legs", action="store_true", help="only the main workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-prof", action="store_true", help="skip the event-timed kernel passes")
    ap.add_argument("--cpu-bytes", type=int, default=16,
                    help="bytes the CPU oracle decodes with all threads (half that with one thread)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB ten times (the "
                         "reference kernel for scaling HBM traffic counters) and exit")
    ap.add_argument("--blocks", choices=("auto", "host", "device"), default="auto",
                    help="how BLT-D blocks are driven (blt_session_device_blocks): chosen by the "
                         "driver from the first blocks (auto), host-driven, or device-resident; "
                         "the other ways are timed beside the main one")
    ap.add_argument("--plain", action="store_true",
                    help="only the timed generations of the main workload: no prefill timing, no "
                         "comparison with the other block driver, no event-timed passes, no legs, "
                         "no CPU baseline (the program that hardware-counter runs profile)")
    ap.add_argument("--no-graphs", action="store_true",
                    help="launch every decoder pass directly instead of replaying HIP graphs")
    ap.add_argument("--gemm-form", type=int, default=0, choices=(0, 1, 2),
                    help="MFMA GEMM kernel of passes of 16 rows or more: 0 by shape, 1 staged "
                         "operand tiles, 2 streamed weights (blt_gemm_form)")
    return ap.parse_args()


def policy_id(blt, wl):
    return {"blt_d": blt.BLT_POLICY_BLT_D, "blt_s": blt.BLT_POLICY_BLT_S,
            "blt_dv": blt.BLT_POLICY_BLT_DV}[wl.policy]


def pct(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))]


# kernel families the library can stamp with HIP events, with their bound
FAMILIES = {
    "k_attn_mfma": ("BLT_PROF_ATTENTION", "hbm", "split-K decode self-attention (MFMA)"),
    "k_gemv_mfma": ("BLT_PROF_GEMV_MFMA", "hbm", "GEMV on MFMA (QKV, W1 of passes < 16 rows)"),
    "k_gemv": ("BLT_PROF_GEMV", "hbm", "dot-product GEMV (W_o, W2, head of passes < 16 rows)"),
    "k_gemm_mfma": ("BLT_PROF_GEMM", "mfma",
                    "MFMA GEMMs (k_gemm_mfma, k_gemm_bs: projections of passes >= 16 rows)"),
}


BLOCK_MODES = {"host": 0, "device": 1, "auto": 2}


def run_leg(blt, torch, wl, steps, warmup, families, no_graphs=False, prefill_report=False,
            blocks="auto", compare=False, gemm_form=0):
    """Time `steps` generations of workload `wl` (after `warmup` untimed ones),
    then one event-timed generation per kernel family.  blocks: how BLT-D
    blocks after the first are driven (blt_session_device_blocks: host-driven,
    device-resident, or chosen by the driver from the first blocks); compare:
    also time the same steps with the blocks driven each other way."""
    import bltgen
    dev = "cuda:0"
    w = bltgen.make_weights(wl)
    inps = [bltgen.make_sequence_inputs(wl, b) for b in range(wl.batch)]
    # one prefill pass per prompt (the causal kernel wants long passes), and
    # room for the largest decode pass
    max_rows = max(1024, wl.batch * (2 * wl.block + 2), wl.prompt_len)
    dec = blt.Decoder(w, n_layers=wl.n_layers, d_model=wl.d_model, n_heads=wl.n_heads,
                      d_ffn=wl.d_ffn, d_global=wl.d_global, dtype=wl.dtype, max_batch=wl.batch,
                      max_ctx=wl.max_ctx, max_latents=wl.n_latents, max_rows=max_rows,
                      max_block=wl.block, rope_theta=wl.rope_theta, rms_eps=wl.rms_eps, device=dev)
    del w
    if no_graphs:
        blt.blt_graphs_enable(dec.ctx, False)
    blt.blt_gemm_form(dec.ctx, gemm_form)
    table = torch.empty((wl.batch, wl.n_latents, wl.d_global), dtype=dec.torch_dtype, device=dev)
    for b, inp in enumerate(inps):
        table[b].copy_(torch.from_numpy(inp["latents"]))
    sess = blt.blt_session_create(dec.ctx, dec.state, [i["prompt"] for i in inps],
                                  [i["prompt_patches"] for i in inps], [i["salt"] for i in inps],
                                  table, wl.n_latents)
    out = {}
    try:
        blt.blt_session_prefill(dec.ctx, sess)
        torch.cuda.synchronize()
        if prefill_report:
            t0 = time.perf_counter()
            blt.blt_session_prefill(dec.ctx, sess)
            torch.cuda.synchronize()
            t_pf = time.perf_counter() - t0
            blt.blt_profile_enable(dec.ctx, blt.BLT_PROF_ATTENTION_CAUSAL)
            blt.blt_profile_read(dec.ctx, reset=True)
            blt.blt_session_prefill(dec.ctx, sess)
            n, ms, fl = blt.blt_profile_read(dec.ctx, reset=True)
            blt.blt_profile_enable(dec.ctx, blt.BLT_PROF_OFF)
            rows = sum(len(i["prompt"]) - 1 for i in inps)
            avg_us = 1e3 * ms / max(n, 1)
            tf = (fl / max(n, 1)) / (avg_us * 1e-6) / 1e12 if n else 0.0
            out["prefill"] = {
                "rows": rows, "seconds": t_pf, "rows_per_s": rows / t_pf, "rows_per_pass": max_rows,
                "roofline": {"bound": "mfma", "kernel": "k_attn_flash (causal attention, MFMA bf16)",
                             "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": tf / MFMA_BF16_PEAK_TFLOPS, "launches": n, "avg_us": avg_us,
                             "flops_per_launch": fl / max(n, 1)}}
        unmask = {"one_step": blt.BLT_UNMASK_ONE_STEP, "entropy": blt.BLT_UNMASK_ENTROPY}.get(
            wl.unmask, blt.BLT_UNMASK_THRESHOLD)
        pid = policy_id(blt, wl)
        mode = BLOCK_MODES[blocks] if wl.policy == "blt_d" else 0
        blt.blt_session_device_blocks(dec.ctx, sess, mode)

        def step():
            blt.blt_session_generate(dec.ctx, sess, pid, wl.block, wl.alpha, wl.n_gen, unmask)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        times = []
        for _ in range(steps):
            t0 = time.perf_counter()
            step()
            torch.cuda.synchronize()
            times.append(time.perf_counter() - t0)
        elapsed = sum(times)
        res = [blt.blt_session_result(sess, b, wl.n_gen) for b in range(wl.batch)]
        if compare and wl.policy == "blt_d":
            # the same steps with the blocks driven each other way
            for other in ("host", "device"):
                if other == blocks:
                    continue
                blt.blt_session_device_blocks(dec.ctx, sess, BLOCK_MODES[other])
                step()
                t0 = time.perf_counter()
                for _ in range(steps):
                    step()
                torch.cuda.synchronize()
                th = (time.perf_counter() - t0) / steps
                hres = [blt.blt_session_result(sess, b, wl.n_gen) for b in range(wl.batch)]
                out["host_driven_blocks" if other == "host" else "device_resident_blocks"] = {
                    "value": sum(r["n"] for r in hres) / th, "ms_per_step": 1e3 * th,
                    "same_bytes_and_counts": all(h["out"] == r["out"] and h["n_dec"] == r["n_dec"] and
                                                 h["n_eg"] == r["n_eg"] for h, r in zip(hres, res))}
            blt.blt_session_device_blocks(dec.ctx, sess, mode)
        n_bytes = sum(r["n"] for r in res)
        n_dec = sum(r["n_dec"] for r in res)
        n_eg = sum(r["n_eg"] for r in res)
        # one event-timed step per kernel family: launches, duration, work
        kern = {}
        for name in families:
            fam = getattr(blt, FAMILIES[name][0])
            blt.blt_profile_enable(dec.ctx, fam)
            blt.blt_profile_read(dec.ctx, reset=True)
            step()
            n, ms, work = blt.blt_profile_read(dec.ctx, reset=True)
            blt.blt_profile_enable(dec.ctx, blt.BLT_PROF_OFF)
            if n == 0:
                continue
            bound = FAMILIES[name][1]
            avg_us = 1e3 * ms / n
            per = work / n
            ach = per / (avg_us * 1e-6) / (1e9 if bound == "hbm" else 1e12)
            peak = HBM_PEAK_GBS if bound == "hbm" else MFMA_BF16_PEAK_TFLOPS
            kern[name] = {"bound": bound, "what": FAMILIES[name][2], "launches_per_step": n,
                          "ms_per_step": ms, "avg_us": avg_us,
                          ("bytes_per_launch" if bound == "hbm" else "flops_per_launch"): per,
                          "achieved": ach, "peak": peak,
                          "unit": "GB/s" if bound == "hbm" else "TFLOP/s", "frac": ach / peak}
        e = 2 if wl.dtype == "bf16" else 4
        step_s = elapsed / steps
        # whole-step algorithmic HBM bytes: weights each decoder pass streams,
        # K/V rows the attention kernel reads (its profile counts them per
        # launch), K/V rows written, weights of the latent projections
        passes = kern["k_attn_mfma"]["launches_per_step"] / wl.n_layers if "k_attn_mfma" in kern else None
        step_bytes = None
        if passes is not None:
            kv_read = kern["k_attn_mfma"]["bytes_per_launch"] * kern["k_attn_mfma"]["launches_per_step"]
            wbytes = passes * blt.streamed_params(wl.n_layers, wl.d_model, wl.d_ffn) * e
            lat_calls = n_eg / wl.batch   # lock-step: one latent batch per encoder/global round
            lbytes = lat_calls * blt.latent_params(wl.n_layers, wl.d_model, wl.d_global) * e
            kv_write = n_bytes * wl.n_layers * 2 * wl.d_model * e   # committed rows enter the cache
            step_bytes = wbytes + kv_read + lbytes + kv_write
            ach = step_bytes / step_s / 1e9
            out["step_roofline"] = {
                "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": ach / HBM_PEAK_GBS, "bytes_per_step": step_bytes,
                "passes_per_step": passes, "us_per_pass": 1e6 * step_s / passes,
                "bytes_per_pass": step_bytes / passes,
                "what": "whole generation: decoder weights per pass + K/V read and written + latent projections, "
                        "over the step's wall time"}
        if kern:
            dom = max(kern, key=lambda k: kern[k]["ms_per_step"])
            d = kern[dom]
            out["roofline"] = {"bound": d["bound"], "achieved": d["achieved"], "peak": d["peak"],
                               "unit": d["unit"], "frac": d["frac"],
                               "traffic": measured_traffic(dom, wl.name) if d["bound"] == "hbm" else None,
                               "kernel": dom, "what": d["what"], "avg_us": d["avg_us"],
                               "launches_per_step": d["launches_per_step"],
                               "dominant_by": "event-timed GPU time per step among the timed families"}
        p_dec = blt.decoder_params(wl.n_layers, wl.d_model, wl.d_ffn, wl.d_global)
        out.update({
            "value": n_bytes / step_s, "ms_per_step": 1e3 * step_s,
            "ms_per_step_p10": 1e3 * pct(times, 0.1), "ms_per_step_p50": 1e3 * pct(times, 0.5),
            "ms_per_step_p90": 1e3 * pct(times, 0.9), "steps": steps, "warmup": warmup,
            "kernels": kern,
            "counters": {
                "decoder_passes_per_seq": n_dec / wl.batch, "encglob_passes_per_seq": n_eg / wl.batch,
                "p_dec_counted": p_dec,
                "proxy_gb_per_seq_counted_params": blt.blt_bw_model(n_dec, n_eg, wl.batch, p_dec,
                                                                     wl.p_enc, wl.p_glob)[1],
                "proxy_gb_per_seq_pages_params": blt.blt_bw_model(n_dec, n_eg, wl.batch, PAGES_P_DEC,
                                                                   wl.p_enc, wl.p_glob)[1]},
            "blocks": blocks if wl.policy == "blt_d" else None,
            "blocks_note": ("auto: one sequence whose watched blocks took every pass runs the rest "
                            "device-resident with the gate tested before each store; "
                            "device_resident_blocks: mode 1, the gate tested at entry")
            if wl.policy == "blt_d" else None,
            "config": {"workload": wl.name, "policy": wl.policy, "batch": wl.batch, "block": wl.block,
                       "alpha": wl.alpha, "unmask": wl.unmask, "layers": wl.n_layers,
                       "d_local": wl.d_model, "heads": wl.n_heads, "ffn": wl.d_ffn,
                       "d_global": wl.d_global, "prompt_bytes": wl.prompt_len,
                       "latents": wl.prompt_patches, "bytes_generated": wl.n_gen,
                       "head_scale": wl.head_scale}})
    finally:
        blt.blt_session_destroy(sess)
        dec.close()
        del table
        torch.cuda.empty_cache()
    return out


def cpu_baseline(wl, n_all, n_one):
    """The oracle, as it stands, on a bounded sample of the same workload:
    sequence 0 with its full prompt (the prefill untimed), decoding n_all
    bytes with every BLAS thread, then, from the same prefilled cache,
    n_one bytes with one thread."""
    import numpy as np
    import bltgen
    from oracle import loops, model
    from threadpoolctl import threadpool_info, threadpool_limits
    W = model.as64(bltgen.make_weights(wl))
    inp = bltgen.make_sequence_inputs(wl, 0)
    inp["latents"] = inp["latents"].astype(np.float64)
    cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [os.cpu_count()])
    s = loops._Seq(W, wl, inp)
    run = loops.Run(out=[])
    t0 = time.perf_counter()
    s.prefill(run)
    t_pre = time.perf_counter() - t0
    x0, n0 = list(s.x), s.cache.length

    def decode(n_bytes):
        s.x, passes = list(x0), 0
        s.cache.truncate(n0)
        t = time.perf_counter()
        while len(s.x) - s.n_prompt < n_bytes:
            before = run.n_dec
            s.x.extend(loops._block_passes(s, run, wl.block, wl.alpha, wl.unmask, False, False)[0])
            passes += run.n_dec - before
        return time.perf_counter() - t, passes

    t_all, p_all = decode(n_all)
    with threadpool_limits(limits=1):
        t_one, p_one = decode(n_one)
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": n_all / t_all, "unit": "bytes/s", "cores": int(cores), "kind": "oracle",
            "host": {"cpu_model": cpu_model, "nproc": os.cpu_count(),
                     "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None},
            "sample": f"sequence 0 of {wl.name} with its full {len(x0)}-byte prompt (prefill {t_pre:.1f} s, "
                      f"untimed): {n_all} bytes ({p_all} decoder passes) in {t_all:.1f} s on {cores} threads",
            "single_thread": {"value": n_one / t_one, "unit": "bytes/s", "cores": 1,
                              "sample": f"{n_one} bytes ({p_one} decoder passes) in {t_one:.1f} s from the "
                                        f"same prefilled cache"}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the decoder path runs on a single GPU); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
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

    wl = bltgen.WORKLOADS[args.workload]
    if args.plain:
        args.no_prof = args.no_legs = args.no_cpu = True
    small = ["k_attn_mfma", "k_gemv_mfma", "k_gemv"]
    fams = [] if args.no_prof else (small if wl.batch * (wl.block + 1) < 16 else ["k_attn_mfma", "k_gemm_mfma"])
    main_leg = run_leg(blt, torch, wl, args.steps, args.warmup, fams, args.no_graphs,
                       prefill_report=not args.plain, blocks=args.blocks,
                       compare=not args.plain, gemm_form=args.gemm_form)
    out = {
        "metric": "decoded bytes/sec",
        "value": main_leg["value"],
        "unit": "bytes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_leg["ms_per_step"],
        "ms_per_step_p10": main_leg["ms_per_step_p10"],
        "ms_per_step_p90": main_leg["ms_per_step_p90"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,0.02) decoder weights, N(0,1) latents, Zipf/uniform byte prompts)",
        "config": main_leg["config"],
    }
    for k in ("roofline", "step_roofline", "kernels", "counters", "prefill", "blocks", "blocks_note",
              "host_driven_blocks", "device_resident_blocks"):
        if k in main_leg:
            out[k] = main_leg[k]
    if not args.no_legs and args.workload == 1:
        legs = {}
        legs["batch64"] = run_leg(blt, torch, bltgen.WORKLOADS[4], 1, 1,
                                  [] if args.no_prof else ["k_attn_mfma", "k_gemm_mfma"], args.no_graphs,
                                  gemm_form=args.gemm_form)
        legs["peaked"] = run_leg(blt, torch, wl.replace(head_scale=12.0), max(1, args.steps // 2), 1,
                                 [] if args.no_prof else ["k_attn_mfma"], args.no_graphs,
                                 blocks=args.blocks, compare=True, gemm_form=args.gemm_form)
        out["legs"] = legs
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_bytes, max(1, args.cpu_bytes // 2))
    print(json.dumps(out))


if __name__ == "__main__":
    main()
