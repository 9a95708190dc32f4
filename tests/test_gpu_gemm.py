"""GPU parity of the two MFMA GEMM kernels of bf16 passes of 16 rows or more,
against the CPU oracle.

Passes of 16 rows or more take their projections (QKV with RoPE and the KV
write, W_o and W2 with the residual, W1 with SiLU, the byte head, the latent
projections) on the MFMA GEMM path, in one of two kernels: one that stages
both operand tiles through LDS, and one that streams the weights straight
into the matrix-core operands of the one wave that uses them (the default up
to 1024 rows).  Each test forces one kernel with `blt_gemm_form` and runs
clean-row passes whose row counts are not multiples of the 64-row tile (220,
50 and 300 rows, two sequences in one pass), after a latent upload of 150
latents per sequence (the latent projections on the GEMM path); the byte
head's 257 columns leave a ragged last column tile, and W2 (K = 1024) is
split over K with the partial sums added by the next RMSNorm launch.  Every
row's logits are compared with the float64 oracle's cached decoder (bf16
tolerance: 2e-2 absolute), and every greedy byte whose oracle top-2 gap is
outside the rounding band.
"""
import pytest

import bltgen
from tests.gpu_util import decoder_for
from tests.test_gpu_prefill import MINI, _append, _check, _Seq

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    import block_diffusion_byte_amd as blt
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    blt.lib()
    yield


@pytest.mark.parametrize("form", [0, 1, 2])
def test_gemm_kernels_ragged_passes_match_oracle(form):
    """form: 0 chosen by shape, 1 staged operand tiles, 2 streamed weights."""
    import torch
    import block_diffusion_byte_amd as blt
    wl = MINI
    w = bltgen.make_weights(wl, gains="random")
    seqs = [_Seq(wl, w, s) for s in range(2)]
    dec = decoder_for(wl, w, max_batch=2, max_rows=512)
    try:
        blt.blt_gemm_form(dec.ctx, form)
        for s in range(2):
            table = torch.from_numpy(seqs[s].inp["latents"]).to("cuda:0", dec.torch_dtype)
            blt.blt_latents_put(dec.ctx, dec.state, [s] * wl.n_latents, list(range(wl.n_latents)),
                                table, 0)
        z = torch.zeros(2 * 512 * 257, device="cuda:0")
        got = _append(blt, torch, dec, seqs, [(0, 0, 150), (1, 0, 70)], z)
        _check(got[0], seqs[0].expect(0, 150), f"form {form}: seq 0 rows 0..149 (220-row pass)")
        _check(got[1], seqs[1].expect(0, 70), f"form {form}: seq 1 rows 0..69 (220-row pass)")
        got = _append(blt, torch, dec, seqs, [(0, 150, 40), (1, 70, 10)], z)
        _check(got[0], seqs[0].expect(150, 40), f"form {form}: seq 0 rows 150..189 (50-row pass)")
        _check(got[1], seqs[1].expect(70, 10), f"form {form}: seq 1 rows 70..79 (50-row pass)")
        got = _append(blt, torch, dec, seqs, [(0, 190, 300)], z)
        _check(got[0], seqs[0].expect(190, 300), f"form {form}: seq 0 rows 190..489 (300-row pass)")
        with pytest.raises(blt.BltError):
            blt.blt_gemm_form(dec.ctx, 3)
    finally:
        dec.close()
