"""Asymmetric-axis (KIVI) against same-axis grouped quantization: error on
synthetic data (test infrastructure and a measurement, CPU only).

"KV Cache Quantization Strategies", Step 2: Keys share a range per channel
over the tokens (scale [..., 1, head_dim]) and Values per token (scale
[..., tokens, 1]); the table's third row, one fixed-size local group, is
simple but need not fit the K/V distributions.  Its section 5.1 runs the
HQQ cache with groups of 64 along head_dim for both K and V, and states that
this setting does not test whether the asymmetric axes beat the same axis.
This module measures that on the synthetic workloads: Keys with a few
channels ten times larger (the outlier channels the per-channel Key scale is
for), Values N(0, 1).

Both schemes take the same codec steps (oracle.codec); KIVI's Key scale is
per channel over each ``segment`` of tokens (the library's whole-group
flushes), its Value scale per token.  Errors are against the unquantized
inputs, in float64: per-element RMS of K and V, and the max-abs / RMS error
of single-query decode attention (oracle.attention.attention_rows) over all
tokens.  Scale bytes are fp16 per token per head.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_rows
from .codec import (quantize_grouped_per_token, quantize_key_per_channel, quantize_value_per_token,
                    restore, restore_grouped_per_token)


def kivi_restored(k, v, qmax: int, segment: int, eps: float = 1e-8):
    """K per channel over each segment of tokens, V per token; restored float64."""
    B, H, T, D = k.shape
    k_hat = np.empty((B, H, T, D))
    for t0 in range(0, T, segment):
        codes, scale = quantize_key_per_channel(k[:, :, t0:t0 + segment], qmax, eps, "fp16")
        k_hat[:, :, t0:t0 + segment] = restore(codes, scale, eps, np.float64)
    codes, scale = quantize_value_per_token(v, qmax, eps, "fp16")
    return k_hat, restore(codes, scale, eps, np.float64)


def same_axis_restored(k, v, qmax: int, group: int, eps: float = 1e-8):
    """K and V per token in runs of ``group`` channels; restored float64."""
    out = []
    for x in (k, v):
        codes, scale = quantize_grouped_per_token(x, group, qmax, eps, "fp16")
        out.append(restore_grouped_per_token(codes, scale, eps, np.float64))
    return out[0], out[1]


def attention_error(k, v, k_hat, v_hat, q, sigma: float):
    """(max-abs, RMS) of decode attention with restored K/V against exact K/V.
    q: [B, Hq, D]; K/V heads are shared by Hq / Hkv query heads."""
    B, Hq, D = q.shape
    H = k.shape[1]
    g = Hq // H
    errs = []
    for b in range(B):
        for h in range(H):
            rows = np.asarray(q[b, h * g:(h + 1) * g], np.float64)
            ref = attention_rows(rows, k[b, h], v[b, h], sigma)
            got = attention_rows(rows, k_hat[b, h], v_hat[b, h], sigma)
            errs.append(got - ref)
    e = np.stack(errs)
    return float(np.abs(e).max()), float(np.sqrt(np.mean(e ** 2)))


def compare(k, v, q, qmax: int = 7, segment: int = 128, group: int = 64, sigma=None):
    """Both schemes on one input: dict scheme -> error and metadata figures."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    D = k.shape[-1]
    sigma = 1.0 / np.sqrt(D) if sigma is None else sigma
    res = {}
    for name, (k_hat, v_hat), scale_bytes in (
            ("kivi", kivi_restored(k, v, qmax, segment), 2.0 * D / segment + 2.0),
            ("same_axis", same_axis_restored(k, v, qmax, group), 2.0 * 2 * D / group)):
        mx, rms = attention_error(k, v, k_hat, v_hat, q, sigma)
        res[name] = {
            "k_rms": float(np.sqrt(np.mean((k_hat - k) ** 2))),
            "v_rms": float(np.sqrt(np.mean((v_hat - v) ** 2))),
            "attn_max_abs": mx, "attn_rms": rms,
            "scale_bytes_per_token_head": scale_bytes,
        }
    return res


def main():
    """The study on the Llama-3-8B decode distributions (2 sequences, 4096 tokens)."""
    import json

    import kvq_synth as ks
    w = ks.small(ks.LLAMA3_DECODE, batch=2)
    s = ks.Stream(w, seed=0)
    k, v = ks.kv_pair(s, w.prefill)
    q = ks.decode_query(s)
    for bits, qmax in ((4, 7), (2, 1), (8, 127)):
        r = compare(k.float().numpy(), v.float().numpy(), q.float().numpy(), qmax=qmax)
        print(json.dumps({"code_bits": bits, "qmax": qmax, **r}))


if __name__ == "__main__":
    main()
