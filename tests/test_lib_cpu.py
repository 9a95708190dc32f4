"""Host-side checks of the C-ABI library (no GPU work is launched)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import bltgen
import block_diffusion_byte_amd as blt
from oracle import proxy

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "blt.h")


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:blt_status|const char \*)\s*(blt_\w+)\s*\(", src, re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 14
    L = blt.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(names) == sorted(blt.EXPORTS)


def test_bw_model_matches_oracle_proxy():
    rng = np.random.default_rng(0)
    for _ in range(50):
        nd, ne, ns = (int(v) for v in rng.integers(1, 10 ** 6, 3))
        wl = bltgen.WORKLOADS[int(rng.integers(0, 5))]
        pd = proxy.decoder_params(wl)
        tot, gb = blt.blt_bw_model(nd, ne, ns, pd, wl.p_enc, wl.p_glob)
        assert tot == proxy.proxy_bytes(nd, ne, pd, wl.p_enc, wl.p_glob)
        assert gb == pytest.approx(float(proxy.proxy_gb_per_seq(nd, ne, ns, pd, wl.p_enc, wl.p_glob)),
                                   rel=1e-15)


def test_bw_model_rejects_overflow_and_zero_sequences():
    with pytest.raises(blt.BltError):
        blt.blt_bw_model(2 ** 63, 1, 1, 4, 1, 1)
    with pytest.raises(blt.BltError):
        blt.blt_bw_model(1, 1, 0, 1, 1, 1)


def _cfg(**kw):
    base = dict(n_layers=2, d_model=128, n_heads=4, d_ffn=512, vocab=257, d_global=256,
                max_batch=2, max_ctx=128, max_latents=64, max_rows=32, max_block=4,
                dtype=blt.BLT_F32, rope_theta=10000.0, rms_eps=1e-5)
    base.update(kw)
    return blt.blt_config(**base)


def test_state_size_formula():
    kv, cr = blt.blt_state_size(_cfg())
    assert kv == 2 * 2 * 2 * 128 * 128 * 4
    assert cr == 2 * 64 * 2 * 128 * 4
    kv, _ = blt.blt_state_size(_cfg(dtype=blt.BLT_BF16, d_model=256, d_ffn=512, d_global=256))
    assert kv == 2 * 2 * 2 * 128 * 256 * 2


@pytest.mark.parametrize("kw", [dict(vocab=256), dict(d_model=130), dict(n_heads=3),
                                dict(max_block=65), dict(max_rows=0), dict(rope_theta=-1.0),
                                dict(d_ffn=100)])
def test_invalid_configs_are_rejected_before_any_device_work(kw):
    with pytest.raises(blt.BltError):
        blt.blt_state_size(_cfg(**kw))
    ctx = C.c_void_p()
    w = blt.blt_weights()
    st = blt.lib().blt_create(C.byref(_cfg(**kw)), C.byref(w), None, C.byref(ctx))
    assert st in (blt.BLT_EINVAL, blt.BLT_EDTYPE) and not ctx.value


def test_null_context_and_weights():
    L = blt.lib()
    assert L.blt_destroy(None) == blt.BLT_EINVAL
    assert L.blt_verify_accept(None, 1, None, 1, None, 1, None, 2, None, None) == blt.BLT_EINVAL
    ctx = C.c_void_p()
    assert L.blt_create(C.byref(_cfg()), None, None, C.byref(ctx)) == blt.BLT_EINVAL
    assert L.blt_last_error(None) == b"NULL context"
    # the tuning controls and the session switches refuse a NULL context or session
    assert L.blt_attention_chunks(None, 1) == blt.BLT_EINVAL
    assert L.blt_flash_key_groups(None, 2) == blt.BLT_EINVAL
    assert L.blt_gemm_form(None, 1) == blt.BLT_EINVAL
    assert L.blt_graphs_enable(None, 1) == blt.BLT_EINVAL
    assert L.blt_profile_enable(None, 1) == blt.BLT_EINVAL
    assert L.blt_session_device_blocks(None, 1) == blt.BLT_EINVAL
    assert L.blt_session_destroy(None) == blt.BLT_EINVAL
