"""blt_kv_append_noalloc (working buffers in the library's static scratch
array) against blt_kv_append on the same rows: outputs and cache contents
bit-identical, over consecutive calls whose second is smaller, for float32
and bfloat16 decoders; oversized calls are rejected."""
import numpy as np
import pytest

import bltgen
from tests.gpu_util import decoder_for, say

pytestmark = pytest.mark.gpu

BF16_MINI = bltgen.WORKLOADS[1].replace(n_layers=2, d_model=256, n_heads=4, d_ffn=1024, d_global=512,
                                        prompt_len=64, prompt_patches=16, n_gen=16, block=4)


@pytest.mark.parametrize("wl", [bltgen.WORKLOADS[0], BF16_MINI], ids=["tiny_fp32", "mini_bf16"])
def test_noalloc_append_equals_append(wl):
    import torch
    import block_diffusion_byte_amd as blt
    w = bltgen.make_weights(wl, gains="random")
    inp = bltgen.make_sequence_inputs(wl, 0)
    dec = decoder_for(wl, w, max_batch=2, max_rows=64)
    dec.kv.zero_()   # rows never written compare equal too
    dev = "cuda:0"
    n_max = 16
    x = [int(v) for v in inp["prompt"]] + [int(v) for v in np.random.default_rng(3).integers(0, 256, 64)]
    lat = [min(i // 4, wl.n_latents - 1) for i in range(len(x))]
    try:
        table = torch.from_numpy(inp["latents"]).to(dev, dec.torch_dtype)
        for slot in (0, 1):
            blt.blt_latents_put(dec.ctx, dec.state, [slot] * wl.n_latents, list(range(wl.n_latents)),
                                table, 0)
        outs = {}
        for slot, noalloc in ((0, False), (1, True)):
            outs[slot] = []
            z = torch.full((2 * n_max * 257,), float("nan"), device=dev)
            am = torch.full((2 * n_max,), -1, dtype=torch.int32, device=dev)
            cf = torch.full((2 * n_max,), float("nan"), device=dev)
            # prefill 30 rows in two calls of 15, then 9 rows, then (smaller) 2 rows
            for start, n in ((0, 15), (15, 15), (30, 9), (39, 2)):
                blt.blt_kv_append(dec.ctx, dec.state, [slot], [start], [n], n_max,
                                  np.array([lat[start:start + n] + [0] * (n_max - n)]),
                                  bytes_=np.array([x[start:start + n] + [0] * (n_max - n)]),
                                  argmax_out=am, conf_out=cf, logits_out=z, noalloc=noalloc)
                torch.cuda.synchronize()
                base = slot * n_max
                outs[slot].append((z[base * 257:(base + n) * 257].cpu().numpy().copy(),
                                   am[base:base + n].cpu().numpy().copy(),
                                   cf[base:base + n].cpu().numpy().copy()))
        for (z0, a0, c0), (z1, a1, c1) in zip(outs[0], outs[1]):
            assert np.isfinite(z0).all()
            assert np.array_equal(z0, z1) and np.array_equal(a0, a1) and np.array_equal(c0, c1)
        # the cache rows the two slots hold are identical too
        kv = dec.kv.view(torch.uint8).view(2, -1)
        assert torch.equal(kv[0], kv[1])
        # a batch of both slots in one allocation-free call, against the same call on the context's workspace
        res = []
        for noalloc in (False, True):
            z = torch.zeros(2 * n_max * 257, device=dev)
            blt.blt_kv_append(dec.ctx, dec.state, [0, 1], [41, 41], [3, 3], n_max,
                              np.array([lat[41:44] + [0] * 13] * 2), bytes_=np.array([x[41:44] + [0] * 13] * 2),
                              logits_out=z, noalloc=noalloc)
            torch.cuda.synchronize()
            res.append(z.cpu().numpy())
        assert np.array_equal(res[0], res[1])
        # limits: 16 rows are rejected before anything is enqueued
        with pytest.raises(blt.BltError) as ei:
            blt.blt_kv_append(dec.ctx, dec.state, [0], [44], [16], 16, np.array([lat[44:60]]),
                              bytes_=np.array([x[44:60]]), noalloc=True)
        assert ei.value.status == blt.BLT_ECAPACITY
    finally:
        dec.close()
    say(f"{wl.name}: allocation-free appends bit-identical to blt_kv_append over 4 calls and a 2-sequence call")
