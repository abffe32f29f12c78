"""The feed-forward sublayer's input in the oracle's "bf16" mode: the row that enters the gate and
up projections is rounded to the nearest bf16 value, and nothing else inside the sublayer is.

Pinned against a closed form written here with plain NumPy (no oracle helper): a one-layer
drafter whose attention sublayer adds nothing (zero O projection) and whose two-tap conv is off
maps the embedded block rows h to h + W_down (silu(W_gate bf16(y)) * (W_up bf16(y))),
y = RMSNorm(h) * g ("Architecture", flowchart "Drafter": the backbone's MLP sublayer; the
precision of activations is not fixed by the pages).  Rounding is round-to-nearest-even to 8
significant bits, done here through frexp / rint.  The unrounded closed form must match mode
"exact", and each form must miss the other mode's result by far more than the tolerance.  CPU only.
"""
import math

import numpy as np

from block_diffusion_draft_inject_amd import synth
from oracle import dflash_oracle as O

TOL = 1e-12   # relative to the largest |h|


def _setup():
    cfg = synth.WORKLOADS["tiny_fp32"].replace(n_layers=1, use_conv=0)
    w = synth.make_weights(cfg)
    W = {k: v.values.astype(np.float64) for k, v in w.items() if k != "layers"}
    W["layers"] = [{k: v.values.astype(np.float64) for k, v in lw.items()} for lw in w["layers"]]
    W["layers"][0]["wo"] = np.zeros_like(W["layers"][0]["wo"])   # the attention sublayer adds zero
    return cfg, W


def _bf16(x):
    """Nearest value with 8 significant bits, ties to even (x finite, nonzero or zero)."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))        # x = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def _closed_form(cfg, W, anchor, round_input):
    K, d = cfg.block_size, cfg.hidden
    lw = W["layers"][0]
    ids = [anchor] + [cfg.mask_id] * (K - 1)
    out = np.zeros((K, d))
    for t in range(K):
        h = W["embed"][ids[t]]
        ms = math.fsum(float(x) * float(x) for x in h) / d
        y = h / math.sqrt(ms + cfg.rms_eps) * lw["mlp_norm"]
        if round_input:
            y = _bf16(y)
        g = np.array([math.fsum(lw["w_gate"][j] * y) for j in range(cfg.ffn)])
        u = np.array([math.fsum(lw["w_up"][j] * y) for j in range(cfg.ffn)])
        s = g / (1.0 + np.exp(-g)) * u
        m = np.array([math.fsum(lw["w_down"][i] * s) for i in range(d)])
        out[t] = h + m
    return out


def test_bf16_rounding_helper_is_nearest_even():
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 3.0 + 2.0 ** -7, 0.0, 1e-30])
    assert np.array_equal(_bf16(x), np.array([1.0, 1.0 + 2.0 ** -6, -1.0, 3.0, 0.0, _bf16(1e-30)]))
    assert np.array_equal(_bf16(x), O.bf16_round(x))


def test_mlp_input_rounded_in_bf16_mode():
    cfg, W = _setup()
    cache = O.DraftCache(cfg.n_layers)
    got = O.draft_block(cfg, W, cache, 5, "bf16")["residual"]
    ref = _closed_form(cfg, W, 5, round_input=True)
    scale = np.max(np.abs(ref))
    assert np.max(np.abs(got - ref)) <= TOL * scale
    # planted: the same sublayer without the rounding (mode "exact") misses by far more
    plain = O.draft_block(cfg, W, cache, 5, "exact")["residual"]
    assert np.max(np.abs(plain - ref)) > 1e6 * TOL * scale


def test_mlp_input_not_rounded_in_exact_mode():
    cfg, W = _setup()
    cache = O.DraftCache(cfg.n_layers)
    got = O.draft_block(cfg, W, cache, 5, "exact")["residual"]
    ref = _closed_form(cfg, W, 5, round_input=False)
    scale = np.max(np.abs(ref))
    assert np.max(np.abs(got - ref)) <= TOL * scale
    rounded = _closed_form(cfg, W, 5, round_input=True)
    assert np.max(np.abs(got - rounded)) > 1e6 * TOL * scale
