"""Pins of the oracle's per-channel two-tap conv ("Architecture", section "Problem 2 -- Suffix decay
is local": a two-tap dynamic depthwise convolution whose coefficients combine a learned base kernel
with a correction computed from the current hidden state, one correction shared per 16 channels).
CPU only."""
import math

import numpy as np
import pytest

from block_diffusion_draft_inject_amd import synth
from oracle import dflash_oracle as O


def _closed_form(x, base, wc, G):
    """Element by element: out[t][c] = s(base0[c] + <W[c // G], x_t>) x_t[c]
    + s(base1[c] + <W[d/G + c // G], x_t>) x_{t-1}[c], with x_{-1} = 0 and s the logistic function."""
    K, d = x.shape
    ng = d // G
    out = np.zeros((K, d))
    for t in range(K):
        corr = [math.fsum(wc[j] * x[t]) for j in range(2 * ng)]
        for c in range(d):
            k0 = 1.0 / (1.0 + math.exp(-(base[0][c] + corr[c // G])))
            k1 = 1.0 / (1.0 + math.exp(-(base[1][c] + corr[ng + c // G])))
            out[t, c] = k0 * x[t, c] + (k1 * x[t - 1, c] if t else 0.0)
    return out


def _draw(K=6, d=64, G=16, seed=0, scale=0.5):
    g = np.random.default_rng(seed)
    return g.standard_normal((K, d)), g.standard_normal((2, d)) * scale, g.standard_normal((2 * d // G, d)) * 0.3


@pytest.mark.parametrize("G", [16, 8, 64])
def test_grouped_conv_closed_form(G):
    x, base, wc = _draw(G=G)
    ref = _closed_form(x, base, wc, G)
    assert np.max(np.abs(O.two_tap_conv_grouped(x, base, wc, G) - ref)) < 1e-14


def test_grouped_conv_pin_rejects_wrong_group_index(monkeypatch):
    """A correction indexed c mod (d/G) (groups interleaved instead of runs of G channels) misses
    the closed form by O(1)."""
    x, base, wc = _draw()

    def interleaved(x, base, wc, group):
        d = x.shape[1]
        ng = d // group
        corr = x @ wc.T
        idx = np.arange(d) % ng
        k0 = O.sigmoid(base[0][None, :] + corr[:, idx])
        k1 = O.sigmoid(base[1][None, :] + corr[:, ng + idx])
        prev = np.zeros_like(x)
        prev[1:] = x[:-1]
        return k0 * x + k1 * prev

    monkeypatch.setattr(O, "two_tap_conv_grouped", interleaved)
    err = np.max(np.abs(O.two_tap_conv_grouped(x, base, wc, 16) - _closed_form(x, base, wc, 16)))
    assert err > 1e-2, err


def test_one_group_with_constant_base_is_the_scalar_form():
    """G = d with base_j[c] = b_j for every channel: one correction per tap, i.e. the configs'
    scalar per-position taps k_t = sigmoid(W_c x_t + b_c)."""
    x, _, _ = _draw(d=48, G=48)
    g = np.random.default_rng(3)
    w = g.standard_normal((2, 48)) * 0.2
    b = np.array([0.3, -0.7])
    grouped = O.two_tap_conv_grouped(x, np.repeat(b[:, None], 48, axis=1), w, 48)
    assert np.max(np.abs(grouped - O.two_tap_conv(x, w, b))) < 1e-15


def test_channels_of_a_group_share_the_correction_and_keep_their_base():
    """Zero correction weights: every channel's coefficients are its own sigmoid(base); a correction
    that moves only group 1 changes exactly channels 16..31."""
    x, base, _ = _draw(d=64)
    zero = np.zeros((8, 64))
    out = O.two_tap_conv_grouped(x, base, zero, 16)
    k0, k1 = O.sigmoid(base[0]), O.sigmoid(base[1])
    prev = np.vstack([np.zeros(64), x[:-1]])
    assert np.allclose(out, k0 * x + k1 * prev, atol=1e-15)
    w1 = zero.copy()
    w1[1] = 1.0               # tap 0 correction of group 1 (channels 16..31) reads sum(x_t)
    moved = O.two_tap_conv_grouped(x, base, w1, 16) != out
    assert moved[:, 16:32].all() and not moved[:, :16].any() and not moved[:, 32:].any()


def test_grouped_conv_is_causal_and_slot_zero_has_no_predecessor():
    x, base, wc = _draw()
    a = O.two_tap_conv_grouped(x, base, wc, 16)
    x2 = x.copy()
    x2[3] += 1.0
    d = O.two_tap_conv_grouped(x2, base, wc, 16) - a
    assert np.all(d[:3] == 0) and np.any(d[3] != 0) and np.any(d[4] != 0) and np.all(d[5] == 0)
    one = O.two_tap_conv_grouped(x[:1], base, wc, 16)
    assert np.allclose(one[0], O.sigmoid(base[0] + np.repeat(wc[:4] @ x[0], 16)) * x[0], atol=1e-15)


def test_parameter_count_at_the_pages_width():
    """The shapes give 20 convs x (2 d^2/16 + 2 d) parameters: 16,486,400 at a drafter width of
    2560 (5 layers, 4 convs each), the page's "+16.5M params".  (The width 2560 is not stated on
    the pages: a consistency check of the shapes, not a pin of the oracle's values.)"""
    cfg = synth.WORKLOADS["b1_k16"].replace(hidden=2560, conv_group=16)
    shapes = synth.layer_shapes(cfg)
    per_layer = sum(int(np.prod(s)) for n, s in shapes.items() if n.startswith("conv_"))
    total = cfg.n_layers * per_layer
    assert total == 16_486_400 and round(total / 1e6, 1) == 16.5


def test_draft_with_one_group_equals_scalar_draft():
    """End to end: the tiny drafter with conv_group = d and every base row constant equals the
    scalar-conv drafter with those constants as biases."""
    cfg = synth.WORKLOADS["tiny_fp32"]
    w = synth.make_weights(cfg)
    W = {k: v.values.astype(np.float64) for k, v in w.items() if k != "layers"}
    W["layers"] = [{k: v.values.astype(np.float64) for k, v in lw.items()} for lw in w["layers"]]
    Wg = dict(W)
    Wg["layers"] = []
    for lw in W["layers"]:
        lw = dict(lw)
        for nm in ("attn_pre", "attn_post", "mlp_pre", "mlp_post"):
            lw[f"conv_{nm}_b"] = np.repeat(lw[f"conv_{nm}_b"][:, None], cfg.hidden, axis=1)
        Wg["layers"].append(lw)
    cache = O.DraftCache(cfg.n_layers)
    pos = np.arange(0, 20)
    O.inject(cfg, W, cache, pos, synth.target_states(cfg, 0, pos).values, "exact")
    a = O.draft_block(cfg, W, cache, 3, "exact")["logits"]
    b = O.draft_block(cfg.replace(conv_group=cfg.hidden), Wg, cache, 3, "exact")["logits"]
    assert np.max(np.abs(a - b)) < 1e-12
    # and the per-16-channel drafter differs from it
    cg = cfg.replace(conv_group=16)
    wg = synth.make_weights(cg)
    Wc = {k: v.values.astype(np.float64) for k, v in wg.items() if k != "layers"}
    Wc["layers"] = [{k: v.values.astype(np.float64) for k, v in lw.items()} for lw in wg["layers"]]
    assert Wc["layers"][0]["conv_mlp_pre_w"].shape == (2 * cfg.hidden // 16, cfg.hidden)
    assert Wc["layers"][0]["conv_mlp_pre_b"].shape == (2, cfg.hidden)
    c = O.draft_block(cg, Wc, cache, 3, "exact")["logits"]
    assert np.all(np.isfinite(c)) and np.max(np.abs(c - a)) > 1e-3
