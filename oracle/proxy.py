"""Parameter-load bandwidth proxy (oracle; test infrastructure only).

wangzhan123.com Fast-BLT article, section six (why bandwidth rather than
wall-clock): total memory traffic in GB = b x [decoder forward passes x
decoder parameters + encoder/global forward passes x (encoder parameters +
global parameters)] / 10^9, with b = 2 bytes per 16-bit parameter.  The
pytorch.kr summary ("evaluation tasks and efficiency metrics") defines the
pass counts as averages per output sequence and states the same b = 2.
"""
from __future__ import annotations

from fractions import Fraction


def proxy_bytes(n_dec, n_eg, p_dec, p_enc, p_glob, b=2):
    """Exact integer byte count summed over the counted passes."""
    return b * (n_dec * p_dec + n_eg * (p_enc + p_glob))


def proxy_gb_per_seq(n_dec, n_eg, n_seq, p_dec, p_enc, p_glob, b=2):
    """GB per output sequence, as an exact fraction."""
    return Fraction(proxy_bytes(n_dec, n_eg, p_dec, p_enc, p_glob, b), 10 ** 9 * n_seq)


def decoder_params(wl, with_cross_qk=True):
    """Parameter count of the synthetic decoder (embedding, latent projection,
    per-layer cross and self attention, RMSNorm gains, FFN, final norm, head)."""
    d, F, dg, L, V = wl.d_model, wl.d_ffn, wl.d_global, wl.n_layers, 257
    per_layer = (4 if with_cross_qk else 2) * d * d + 4 * d * d + 2 * d * F + 2 * d
    return V * d + d * dg + L * per_layer + V * d + d
