"""Pins for the CPU oracle: checks against library routines, closed forms, invariants the
pages fix, brute force, and the pages' worked example.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

from block_diffusion_draft_inject_amd import synth
from oracle import dflash_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------- helpers

def tiny(**kw):
    base = synth.WORKLOADS["tiny_fp32"]
    return base.replace(**kw) if kw else base


def weights64(cfg, **kw):
    w = synth.make_weights(cfg, **kw)
    out = {k: v.values.astype(np.float64) for k, v in w.items() if k != "layers"}
    out["layers"] = [{k: v.values.astype(np.float64) for k, v in lw.items()} for lw in w["layers"]]
    return out


def fill_cache(cfg, W, L, first=0, seq=0, mode="exact", states_fn=None):
    cache = O.DraftCache(cfg.n_layers)
    pos = np.arange(first, L)
    st = synth.target_states(cfg, seq, pos).values if states_fn is None else states_fn(pos)
    O.inject(cfg, W, cache, pos, st, mode)
    return cache


# ---------------------------------------------------------------- numeric primitives

def test_bf16_round_matches_torch_rne():
    g = np.random.default_rng(1)
    x = g.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # exact halfway cases: bf16 value + half an ulp, both even and odd lower neighbours
    base = torch.tensor(g.standard_normal(1000).astype(np.float32)).to(torch.bfloat16).float().numpy()
    e = np.floor(np.log2(np.abs(base)))
    half = (2.0 ** (e - 8)).astype(np.float32)
    ties = (base + np.sign(base) * half).astype(np.float32)
    x = np.concatenate([x, ties, np.float32([0.0, -0.0, 1.0, -1.0, 65504.0, 1e-30])])
    ours = O.bf16_round(x.astype(np.float64))
    ref = torch.tensor(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_rms_norm_closed_forms():
    g = np.random.default_rng(2)
    x = g.standard_normal((5, 64)) * 7.0
    y = O.rms_norm(x, np.ones(64), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, atol=1e-14)
    assert np.allclose(O.rms_norm(3.5 * x, np.ones(64), 0.0), y, atol=1e-14)
    gain = g.standard_normal(64)
    assert np.allclose(O.rms_norm(x, gain, 0.0), y * gain, atol=1e-14)
    # eps: a constant row c has rms c, so output = c / sqrt(c^2 + eps)
    c = 0.01
    out = O.rms_norm(np.full((1, 8), c), np.ones(8), 1e-6)
    assert np.allclose(out, c / math.sqrt(c * c + 1e-6), atol=1e-15)


def test_rope_matches_complex_rotation():
    """Rotate-half RoPE equals multiplying z_i = x_i + i*x_{i+h} by exp(i * p * theta^(-2i/d))."""
    g = np.random.default_rng(3)
    dh, theta = 64, 10000.0
    x = g.standard_normal((7, dh))
    pos = np.array([0, 1, 5, 100, 1023, 32767, 40000])
    y = O.rope(x, pos, theta)
    h = dh // 2
    z = x[:, :h] + 1j * x[:, h:]
    freqs = np.array([theta ** (-2.0 * i / dh) for i in range(h)])
    zr = z * np.exp(1j * pos[:, None] * freqs[None, :])
    assert np.allclose(y[:, :h], zr.real, atol=1e-12)
    assert np.allclose(y[:, h:], zr.imag, atol=1e-12)
    assert np.array_equal(O.rope(x[:1], np.array([0]), theta), x[:1])


def test_rope_is_relative():
    g = np.random.default_rng(4)
    q, k = g.standard_normal((2, 128))
    for p, s in [(5, 3), (1030, 7), (32767, 31744)]:
        base = O.rope(q[None], np.array([p]), 1e4) @ O.rope(k[None], np.array([s]), 1e4).T
        for delta in (1, 977, 20000):
            sh = O.rope(q[None], np.array([p + delta]), 1e4) @ O.rope(k[None], np.array([s + delta]), 1e4).T
            assert abs(sh[0, 0] - base[0, 0]) < 1e-10


def test_sigmoid_silu_special_values():
    assert O.sigmoid(0.0) == 0.5
    assert abs(O.sigmoid(40.0) - 1.0) < 1e-15
    assert O.silu(0.0) == 0.0
    assert abs(O.silu(30.0) - 30.0) < 1e-9
    assert abs(O.silu(-30.0)) < 1e-9
    # silu(x) - silu(-x) = x
    x = np.linspace(-5, 5, 11)
    assert np.allclose(O.silu(x) - O.silu(-x), x, atol=1e-14)


def test_two_tap_conv_structure():
    """With W_c = 0 the taps are the constants sigmoid(b); the second tap reads the previous
    row, slot 0 reads zero."""
    g = np.random.default_rng(5)
    x = g.standard_normal((6, 32))
    b = np.array([0.3, -1.2])
    y = O.two_tap_conv(x, np.zeros((2, 32)), b)
    k0, k1 = 1 / (1 + math.exp(-0.3)), 1 / (1 + math.exp(1.2))
    assert np.allclose(y[0], k0 * x[0], atol=1e-15)
    for t in range(1, 6):
        assert np.allclose(y[t], k0 * x[t] + k1 * x[t - 1], atol=1e-15)
    # taps (1, 0) reduce to no conv
    y = O.two_tap_conv(x, np.zeros((2, 32)), np.array([60.0, -60.0]))
    assert np.allclose(y, x, atol=1e-12)
    assert np.array_equal(O.two_tap_conv(x, np.zeros((2, 32)), b, use_conv=False), x)
    # causal: row t depends only on rows <= t
    x2 = x.copy()
    x2[4] += 1.0
    w = g.standard_normal((2, 32))
    d = O.two_tap_conv(x2, w, b) - O.two_tap_conv(x, w, b)
    assert np.all(d[:4] == 0) and np.any(d[4] != 0) and np.any(d[5] != 0)


def test_attention_matches_torch_sdpa_gqa():
    g = np.random.default_rng(6)
    K, nh, nkv, dh, nk = 8, 16, 4, 32, 50
    q = g.standard_normal((K, nh, dh))
    k = g.standard_normal((nk, nkv, dh))
    v = g.standard_normal((nk, nkv, dh))
    ours = O._attention(q, k, v, nkv)
    tq = torch.tensor(q).permute(1, 0, 2)[None]
    tk = torch.tensor(k).permute(1, 0, 2)[None]
    tv = torch.tensor(v).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, enable_gqa=True)
    assert np.allclose(ours, ref[0].permute(1, 0, 2).numpy(), atol=1e-12)
    # n_kv == n_h is plain multi-head attention
    k16 = g.standard_normal((nk, nh, dh))
    v16 = g.standard_normal((nk, nh, dh))
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, torch.tensor(k16).permute(1, 0, 2)[None], torch.tensor(v16).permute(1, 0, 2)[None])
    assert np.allclose(O._attention(q, k16, v16, nh), ref[0].permute(1, 0, 2).numpy(), atol=1e-12)


def test_topk_matches_stable_argsort():
    g = np.random.default_rng(7)
    v = np.round(g.standard_normal(5000), 2)     # many exact ties
    ref = np.argsort(-v, kind="stable")[:16]
    assert np.array_equal(O.topk_desc(v, 16), ref)


# ---------------------------------------------------------------- injection

def test_inject_chunking_and_scale_invariance():
    cfg = tiny()
    W = weights64(cfg)
    pos = np.arange(0, 24)
    st = synth.target_states(cfg, 0, pos).values
    whole = O.DraftCache(cfg.n_layers)
    O.inject(cfg, W, whole, pos, st, "exact")
    parts = O.DraftCache(cfg.n_layers)
    for a, b in [(0, 5), (5, 6), (6, 24)]:
        O.inject(cfg, W, parts, pos[a:b], st[a:b], "exact")
    assert whole.length == parts.length == 24
    for l in range(cfg.n_layers):
        for p in range(24):
            assert np.allclose(whole.k[l][p], parts.k[l][p], atol=1e-12)
            assert np.allclose(whole.v[l][p], parts.v[l][p], atol=1e-12)
    # RMSNorm of the concatenation: scaling the states changes nothing (eps is tiny vs rms 1)
    sc = O.DraftCache(cfg.n_layers)
    O.inject(cfg, W, sc, pos, 4.0 * st, "exact")
    for l in range(cfg.n_layers):
        assert np.allclose(sc.v[l][3], whole.v[l][3], rtol=1e-5)
        assert np.allclose(sc.k[l][3], whole.k[l][3], rtol=1e-5)


def test_inject_gain_placement_and_rope_pairs():
    """Concat-norm gain scales V linearly but not K (the per-head k-norm removes scale);
    RoPE after the k-norm keeps each rotated pair's norm equal to the gained normed pair."""
    cfg = tiny()
    W = weights64(cfg)
    pos = np.array([0, 3, 77])
    st = synth.target_states(cfg, 0, pos).values
    a = O.DraftCache(cfg.n_layers)
    O.inject(cfg, W, a, pos, st, "exact")
    W2 = dict(W)
    W2["concat_norm"] = 2.0 * W["concat_norm"]
    b = O.DraftCache(cfg.n_layers)
    O.inject(cfg, W2, b, pos, st, "exact")
    h = cfg.head_dim // 2
    for l in range(cfg.n_layers):
        for p in pos:
            assert np.allclose(b.v[l][p], 2.0 * a.v[l][p], atol=1e-12)
            assert np.allclose(b.k[l][p], a.k[l][p], atol=1e-9)
        # rebuild the pre-rotation normed key of position 77 from its position-0 twin:
        # at p=0 RoPE is the identity, so K(0) = gain * xhat(0)
    st0 = np.repeat(st[2:3], 2, axis=0)
    c = O.DraftCache(cfg.n_layers)
    O.inject(cfg, W, c, np.array([0, 77]), st0, "exact")
    for l in range(cfg.n_layers):
        k0, k77 = c.k[l][0], c.k[l][77]
        pair0 = k0[:, :h] ** 2 + k0[:, h:] ** 2
        pair77 = k77[:, :h] ** 2 + k77[:, h:] ** 2
        assert np.allclose(pair0, pair77, atol=1e-12)
        assert not np.allclose(k0, k77)


# ---------------------------------------------------------------- draft pass invariants

def test_window_excludes_old_positions():
    """Tokens outside the sliding window do not affect the draft (bitwise)."""
    cfg = tiny(window=16)
    W = weights64(cfg)
    L = 40
    a = fill_cache(cfg, W, L)
    def perturbed(pos):
        st = synth.target_states(cfg, 0, pos).values.copy()
        st[pos < L - cfg.window] += 5.0
        return st
    b = fill_cache(cfg, W, L, states_fn=perturbed)
    ra = O.draft_block(cfg, W, a, 17, "exact")
    rb = O.draft_block(cfg, W, b, 17, "exact")
    assert np.array_equal(ra["logits"], rb["logits"])
    # and a perturbation inside the window does change them
    def perturbed_in(pos):
        st = synth.target_states(cfg, 0, pos).values.copy()
        st[pos == L - 3] += 5.0
        return st
    c = fill_cache(cfg, W, L, states_fn=perturbed_in)
    assert not np.allclose(O.draft_block(cfg, W, c, 17, "exact")["logits"], ra["logits"])


def test_block_is_non_causal():
    """Changing a later block slot changes the logits of earlier slots."""
    cfg = tiny()
    W = weights64(cfg)
    cache = fill_cache(cfg, W, 32)
    ids = np.full(cfg.block_size, cfg.mask_id)
    ids[0] = 11
    ra = O.draft_block(cfg, W, cache, 11, "exact", block_ids=ids)
    ids2 = ids.copy()
    ids2[-1] = 5
    rb = O.draft_block(cfg, W, cache, 11, "exact", block_ids=ids2)
    assert np.max(np.abs(ra["logits"][0] - rb["logits"][0])) > 1e-6
    # with the default block the result equals passing the ids explicitly
    rc = O.draft_block(cfg, W, cache, 11, "exact")
    assert np.array_equal(rc["logits"], ra["logits"])


def test_positions_enter_only_relatively():
    """Shifting every position by the same offset leaves the draft unchanged (RoPE is
    relative), so a context at 32768 behaves like the same window content at 1024."""
    cfg = tiny(window=16)
    W = weights64(cfg)
    L, shift = 24, 32768 - 24
    st = synth.target_states(cfg, 0, np.arange(L - 16, L)).values
    a = O.DraftCache(cfg.n_layers)
    O.inject(cfg, W, a, np.arange(L - 16, L), st, "exact")
    b = O.DraftCache(cfg.n_layers)
    O.inject(cfg, W, b, np.arange(L - 16, L) + shift, st, "exact")
    ra = O.draft_block(cfg, W, a, 9, "exact")
    rb = O.draft_block(cfg, W, b, 9, "exact")
    assert np.allclose(ra["logits"], rb["logits"], atol=1e-9)


def test_conv_off_equals_unit_taps():
    cfg = tiny()
    W = weights64(cfg)
    cache = fill_cache(cfg, W, 20)
    off = O.draft_block(cfg.replace(use_conv=False), W, cache, 3, "exact")
    W1 = dict(W)
    W1["layers"] = []
    for lw in W["layers"]:
        lw = dict(lw)
        for nm in ("attn_pre", "attn_post", "mlp_pre", "mlp_post"):
            lw[f"conv_{nm}_w"] = np.zeros_like(lw[f"conv_{nm}_w"])
            lw[f"conv_{nm}_b"] = np.array([80.0, -80.0])
        W1["layers"].append(lw)
    unit = O.draft_block(cfg, W1, cache, 3, "exact")
    assert np.allclose(off["logits"], unit["logits"], atol=1e-10)


def test_empty_context_and_bf16_mode_close_to_exact():
    cfg = tiny()
    W = weights64(cfg)
    empty = O.DraftCache(cfg.n_layers)
    r = O.draft_block(cfg, W, empty, 5, "exact")
    assert np.all(np.isfinite(r["logits"]))
    cache = fill_cache(cfg, W, 40)
    cache_b = fill_cache(cfg, W, 40, mode="bf16")
    ex = O.draft_block(cfg, W, cache, 5, "exact")
    bf = O.draft_block(cfg, W, cache_b, 5, "bf16")
    err = np.max(np.abs(ex["logits"] - bf["logits"]))
    assert 0 < err < 0.05


def test_topk_output_consistent_with_logits():
    cfg = tiny()
    W = weights64(cfg)
    r = O.draft_block(cfg, W, fill_cache(cfg, W, 10), 1, "exact")
    for t in range(cfg.block_size - 1):
        ref = np.argsort(-r["logits"][t], kind="stable")[:16]
        assert np.array_equal(r["topk_ids"][t], ref)
        assert np.array_equal(r["topk_logits"][t], r["logits"][t][ref])


# ---------------------------------------------------------------- selector

def _lattice(cfg, seed, stress=True):
    W = weights64(cfg, selector_stress=stress)
    g = np.random.default_rng(seed)
    km1 = cfg.block_size - 1
    ids = np.stack([g.choice(cfg.vocab - 1, 16, replace=False) for _ in range(km1)])
    logits = -np.sort(-g.standard_normal((km1, 16)), axis=1)
    hf = g.standard_normal((cfg.block_size, cfg.hidden))
    return W, ids, logits, hf


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_viterbi_matches_brute_force(K, seed):
    cfg = tiny(block_size=K)
    W, ids, logits, hf = _lattice(cfg, seed)
    S = O.pair_scores(cfg, W, 7, ids, logits, hf)
    allp = O.brute_force_paths(S)
    assert len(allp) == 16 ** (K - 1)
    res = O.select_path(cfg, W, 7, ids, logits, hf, "viterbi")
    assert list(res["path_idx"]) == list(allp[0][1])
    assert abs(res["score"] - allp[0][0]) < 1e-12
    second = allp[1][0] if len(allp) > 1 else -np.inf
    assert abs(res["margin"] - (allp[0][0] - second)) < 1e-12
    assert np.array_equal(res["path_ids"], ids[np.arange(K - 1), res["path_idx"]])


def test_greedy_walk_against_enumeration():
    """Greedy: each step takes the best successor of the previous pick; check step by step
    against the full enumeration restricted to the chosen prefix."""
    cfg = tiny(block_size=4)
    W, ids, logits, hf = _lattice(cfg, 3)
    S = O.pair_scores(cfg, W, 7, ids, logits, hf)
    res = O.select_path(cfg, W, 7, ids, logits, hf, "greedy")
    prefix, a, gaps = [], 0, []
    for t in range(3):
        succ = sorted(range(16), key=lambda b: (-S[t][a, b], b))
        prefix.append(succ[0])
        gaps.append(S[t][a, succ[0]] - S[t][a, succ[1]])
        a = succ[0]
    assert list(res["path_idx"]) == prefix
    assert abs(res["margin"] - min(gaps)) < 1e-12
    vit = O.select_path(cfg, W, 7, ids, logits, hf, "viterbi")
    assert res["score"] <= vit["score"] + 1e-12


def test_selector_without_pair_term_is_per_position_argmax():
    cfg = tiny(block_size=8)
    W, ids, logits, hf = _lattice(cfg, 4)
    W0 = dict(W)
    W0["sel_A"] = np.zeros_like(W["sel_A"])
    for mode in ("viterbi", "greedy"):
        r = O.select_path(cfg, W0, 7, ids, logits, hf, mode)
        assert list(r["path_idx"]) == [0] * 7
        assert abs(r["score"] - logits[:, 0].sum()) < 1e-12
    # the gate: W_H = 0 gives H = 1/2 everywhere
    Wh = dict(W)
    Wh["sel_WH"] = np.zeros_like(W["sel_WH"])
    S = O.pair_scores(cfg, Wh, 7, ids, logits, hf)
    pair = 0.5 * (W["sel_A"][ids[0]] * W["sel_B"][ids[1]]).sum(1)
    assert np.allclose(S[1][np.arange(16), np.arange(16)] - logits[1], pair, atol=1e-12)


# ---------------------------------------------------------------- verification

def test_verify_full_accept_and_first_reject():
    K = 16
    g = np.random.default_rng(8)
    d = g.integers(0, 1000, K - 1)
    tgt = np.concatenate([d, [42]])
    n, com, nxt = O.verify_greedy(d, tgt)
    assert n == K - 1 and nxt == 42 and list(com) == list(d) + [42]
    tgt2 = tgt.copy()
    tgt2[0] = d[0] + 1
    n, com, nxt = O.verify_greedy(d, tgt2)
    assert n == 0 and nxt == d[0] + 1 and com[0] == d[0] + 1 and np.all(com[1:] == -1)
    tgt3 = tgt.copy()
    tgt3[5] = d[5] + 3
    n, com, nxt = O.verify_greedy(d, tgt3)
    assert n == 5 and list(com[:6]) == list(d[:5]) + [d[5] + 3]


def test_expected_acceptance_statistics():
    """E[tau] = 1 + sum_i p^i for per-position match probability p (3.1412 at K=8, p=0.7)."""
    cfg = synth.WORKLOADS["b32_k8_conv"].replace(batch=20000)
    match, alt, last = synth.match_draws(cfg, 0)
    g = np.random.default_rng(9)
    draft = g.integers(0, cfg.vocab, (cfg.batch, 7))
    tgt = synth.stand_in_target(draft, match, alt, last, cfg.vocab)
    taus = np.array([O.verify_greedy(draft[b], tgt[b])[0] + 1 for b in range(cfg.batch)])
    exp = 1 + sum(0.7 ** i for i in range(1, 8))
    assert abs(exp - 3.1412) < 1e-4
    assert abs(taus.mean() - exp) < 4 * taus.std() / math.sqrt(cfg.batch)


def test_recall_table_reproduces_printed_acceptance():
    """The pages' recall table: acceptance length = 1 + sum_i prod_{j<=i} r_j gives the
    printed 4.27 (Recall@1) and 6.79 (Recall@16); simulating greedy verification with those
    position-conditional acceptance rates gives the same mean.

    The recalls are printed to 0.1 percent, so the formula is evaluated at both ends of each
    recall's rounding interval; the printed length (two decimals) must fall in that range."""
    fx = json.load(open(os.path.join(HERE, "golden", "recall_table.json")))
    half = fx["recall_printed_to_percent"] / 2 / 100
    last_digit = 10.0 ** -fx["acceptance_printed_decimals"]
    for key, printed in (("recall_at_1_percent", fx["acceptance_length_printed"]["recall_at_1"]),
                         ("recall_at_16_percent", fx["acceptance_length_printed"]["recall_at_16"])):
        r = [x / 100 for x in fx[key]]
        lo = O.expected_tau([x - half for x in r])
        hi = O.expected_tau([x + half for x in r])
        assert lo - last_digit <= printed <= hi
        g = np.random.default_rng(10)
        n = 40000
        draft = g.integers(0, 100, (n, len(r)))
        hit = g.random((n, len(r))) < np.array(r)
        tgt = np.where(hit, draft, draft + 1)
        tgt = np.concatenate([tgt, np.zeros((n, 1), dtype=tgt.dtype)], axis=1)
        taus = np.array([O.verify_greedy(draft[i], tgt[i])[0] + 1 for i in range(n)])
        assert lo - 4 * taus.std() / math.sqrt(n) <= taus.mean() <= hi + 4 * taus.std() / math.sqrt(n)


def test_target_for_tau_yields_requested_tau():
    cfg = synth.WORKLOADS["b32_k16_incremental"]
    tau = synth.tau_draws(cfg, 3)
    _, alt, last = synth.match_draws(cfg, 3)
    g = np.random.default_rng(11)
    draft = g.integers(0, cfg.vocab, (cfg.batch, 15))
    tgt = synth.target_for_tau(draft, tau, alt, last, cfg.vocab)
    got = np.array([O.verify_greedy(draft[b], tgt[b])[0] + 1 for b in range(cfg.batch)])
    assert np.array_equal(got, tau)


# ---------------------------------------------------------------- planted mistakes are caught

def test_planted_mistakes_fail_pins():
    """A conv tap that reads the next row instead of the previous one, or a causal mask inside
    the block, would each break a pin above; check that the pins notice such edits."""
    cfg = tiny()
    W = weights64(cfg)
    cache = fill_cache(cfg, W, 20)
    ref = O.draft_block(cfg, W, cache, 3, "exact")["logits"]
    orig = O.two_tap_conv
    try:
        def swapped(x, w, b, use_conv=True):
            x = O.as64(x)
            k = O.sigmoid(x @ O.as64(w).T + O.as64(b))
            nxt = np.zeros_like(x)
            nxt[:-1] = x[1:]
            return k[:, 0:1] * x + k[:, 1:2] * nxt
        O.two_tap_conv = swapped
        bad = O.draft_block(cfg, W, cache, 3, "exact")["logits"]
        assert not np.allclose(bad, ref)
    finally:
        O.two_tap_conv = orig
    orig_att = O._attention
    try:
        def causal(q, k, v, n_kv):
            K = q.shape[0]
            n = k.shape[0]
            out = np.empty_like(q)
            for i in range(q.shape[1]):
                j = (i * n_kv) // q.shape[1]
                s = q[:, i, :] @ k[:, j, :].T / math.sqrt(q.shape[2])
                s = s + np.triu(np.full((K, n), -np.inf), n - K + 1)
                p = np.exp(s - s.max(1, keepdims=True))
                out[:, i, :] = (p / p.sum(1, keepdims=True)) @ v[:, j, :]
            return out
        O._attention = causal
        ids = np.full(cfg.block_size, cfg.mask_id)
        ids[0] = 3
        a = O.draft_block(cfg, W, cache, 3, "exact", block_ids=ids)["logits"]
        ids[-1] = 9
        b = O.draft_block(cfg, W, cache, 3, "exact", block_ids=ids)["logits"]
        assert np.array_equal(a[0], b[0])   # the non-causality pin would fail on this oracle
    finally:
        O._attention = orig_att


def test_synthetic_inputs_are_deterministic():
    cfg = tiny()
    a = synth.make_weights(cfg)
    b = synth.make_weights(cfg)
    assert np.array_equal(a["fc"].storage, b["fc"].storage)
    assert np.array_equal(a["layers"][1]["w_down"].storage, b["layers"][1]["w_down"].storage)
    s1 = synth.target_states(cfg, 0, [3, 4, 5]).values
    s2 = synth.target_states(cfg, 0, [5]).values
    assert np.array_equal(s1[2], s2[0])
    gains = a["layers"][0]["attn_norm"].values
    assert abs(gains.mean() - 1.0) < 0.01 and gains.std() > 0.01


# --------------------------------------------------------------------------------------
# sampling walk and rejection-sampling verification
# --------------------------------------------------------------------------------------

def _softmax(z):
    e = np.exp(z - np.max(z))
    return e / e.sum()


def test_inverse_cdf_boundaries():
    w = np.array([0.0, 0.25, 0.0, 0.5, 0.25])
    assert O.inverse_cdf(w, 0.0) == 1          # first index with positive weight
    assert O.inverse_cdf(w, 0.2499) == 1
    assert O.inverse_cdf(w, 0.25) == 3         # the boundary belongs to the next interval
    assert O.inverse_cdf(w, 0.7499) == 3
    assert O.inverse_cdf(w, 0.75) == 4
    assert O.inverse_cdf(w, 0.999999) == 4


def test_sample_walk_joint_distribution():
    """Empirical joint distribution of two sampled picks equals softmax(S_1/T) x softmax(S_2[b1]/T)."""
    rng = np.random.default_rng(11)
    T = 0.7
    S = [rng.normal(size=(1, 4)), rng.normal(size=(4, 4)) * 1.5]
    exact = np.outer(_softmax(S[0][0] / T), np.ones(4)) * np.stack([_softmax(S[1][a] / T) for a in range(4)])
    N = 40000
    U = rng.random((N, 2))
    counts = np.zeros((4, 4))
    for u in U:
        idx, qp, qc = O.sample_walk(S, u, T)
        counts[idx[0], idx[1]] += 1
    emp = counts / N
    sigma = np.sqrt(exact * (1 - exact) / N)
    assert np.all(np.abs(emp - exact) < 5 * sigma + 1e-12)
    # the reported probabilities are the conditionals used for the draw
    idx, qp, qc = O.sample_walk(S, [0.3, 0.8], T)
    assert np.allclose(qc[0], _softmax(S[0][0] / T)) and np.allclose(qc[1], _softmax(S[1][idx[0]] / T))
    assert qp[0] == qc[0][idx[0]] and qp[1] == qc[1][idx[1]]


def test_sample_walk_temperature_limits():
    rng = np.random.default_rng(5)
    S = [rng.normal(size=(1, 16))] + [rng.normal(size=(16, 16)) for _ in range(4)]
    # a very low temperature reduces sampling to the greedy walk (any uniform)
    greedy_idx, _, _ = O.greedy_walk(S)
    for u in ([0.01] * 5, [0.5] * 5, [0.99] * 5):
        idx, _, _ = O.sample_walk(S, u, 1e-4)
        assert list(idx) == list(greedy_idx)
    # a very high temperature makes every candidate equally likely: u picks floor(16 u)
    idx, qp, _ = O.sample_walk(S, [0.0, 0.07, 0.5, 0.93, 0.999], 1e6)
    assert list(idx) == [0, 1, 8, 14, 15]
    assert np.allclose(qp, 1 / 16, rtol=1e-4)


def test_nucleus_closed_forms():
    """Top-p by hand: keep the most probable entries until their mass reaches top_p (the entry
    that crosses it stays), ties ranked by index, then renormalise."""
    q = np.array([0.1, 0.5, 0.3, 0.1])
    assert np.allclose(O.nucleus(q, 0.75), [0, 0.625, 0.375, 0])      # 0.5 < 0.75 -> 0.3 stays
    assert np.allclose(O.nucleus(q, 0.4), [0, 1, 0, 0])               # the top entry alone reaches 0.4
    assert np.allclose(O.nucleus(q, 0.85), [0.1, 0.5, 0.3, 0] / np.float64(0.9))   # tie 0.1/0.1 -> index 0
    assert np.allclose(O.nucleus(q, 1.0), q)
    t = np.array([0.3, 0.3, 0.2, 0.2])
    assert np.allclose(O.nucleus(t, 0.5), [0.5, 0.5, 0, 0])
    assert np.allclose(O.nucleus(t, 0.65), [0.375, 0.375, 0.25, 0])
    assert np.allclose(O.nucleus(t, 1e-9), [1, 0, 0, 0])


def test_sample_walk_top_p():
    rng = np.random.default_rng(9)
    S = [rng.normal(size=(1, 16)) * 2] + [rng.normal(size=(16, 16)) * 2 for _ in range(3)]
    # a vanishing nucleus keeps only the most probable successor: the greedy walk, q = 1
    g, _, _ = O.greedy_walk(S)
    for u in (0.0, 0.5, 0.999):
        idx, qp, qc = O.sample_walk(S, [u] * 4, 1.0, top_p=1e-9)
        assert list(idx) == list(g) and np.allclose(qp, 1.0)
    # the picks never leave the nucleus, and the reported q is the cut distribution
    U = rng.random((2000, 4))
    for u in U[:200]:
        idx, qp, qc = O.sample_walk(S, u, 0.8, top_p=0.6)
        for t in range(4):
            assert qc[t][idx[t]] > 0 and qp[t] == qc[t][idx[t]] and abs(qc[t].sum() - 1) < 1e-12
    # first pick: empirical distribution equals the cut distribution
    want = O.nucleus(np.exp(S[0][0] / 0.8 - np.max(S[0][0] / 0.8)) / np.exp(S[0][0] / 0.8 - np.max(S[0][0] / 0.8)).sum(),
                     0.6)
    counts = np.bincount([O.sample_walk(S, u, 0.8, top_p=0.6)[0][0] for u in U], minlength=16) / len(U)
    assert np.all(np.abs(counts - want) < 5 * np.sqrt(want * (1 - want) / len(U)) + 1e-12)


def _drafter_and_target():
    """Tiny vocabulary: slot 1 and slot 2 candidates with fixed drafter probabilities (slot 2's
    independent of the slot-1 pick here), and target distributions for slots 1, 2 and the bonus."""
    cand = np.array([[0, 2, 4], [1, 2, 5]])
    q = np.array([[0.5, 0.3, 0.2], [0.6, 0.25, 0.15]])
    p = np.array([[0.10, 0.05, 0.40, 0.15, 0.20, 0.10],
                  [0.05, 0.30, 0.05, 0.20, 0.15, 0.25],
                  [0.30, 0.10, 0.10, 0.10, 0.20, 0.20]])
    return cand, q, p


def test_rejection_verification_is_lossless():
    """Whatever the drafter proposes, the committed tokens follow the target: the first one is
    distributed as p_1; the second (given the first draft was accepted) as p_2; the third
    (given both were accepted) as the bonus distribution p_3."""
    cand, q, p = _drafter_and_target()
    rng = np.random.default_rng(7)
    N = 60000
    first = np.zeros(6)
    second = np.zeros(6)
    third = np.zeros(6)
    n1 = n2 = 0
    for _ in range(N):
        j1 = O.inverse_cdf(q[0], rng.random())
        j2 = O.inverse_cdf(q[1], rng.random())
        draft = [cand[0][j1], cand[1][j2]]
        n, com, nxt = O.verify_rejection(draft, [q[0][j1], q[1][j2]], cand, q, p, rng.random(2), rng.random())
        first[com[0]] += 1
        if n >= 1:
            second[com[1]] += 1
            n1 += 1
        if n == 2:
            third[com[2]] += 1
            n2 += 1
        assert nxt == com[n]
    for emp, cnt, target in ((first / N, N, p[0]), (second / n1, n1, p[1]), (third / n2, n2, p[2])):
        sigma = np.sqrt(target * (1 - target) / cnt)
        assert np.all(np.abs(emp - target) < 5 * sigma)
    # acceptance rate of slot 1 = sum_v min(p_1(v), q_1(v)) (the overlap of the two)
    overlap = sum(min(p[0][v], q[0][j]) for j, v in enumerate(cand[0]))
    assert abs(n1 / N - overlap) < 5 * math.sqrt(overlap * (1 - overlap) / N)


def test_rejection_verification_special_cases():
    cand, q, p = _drafter_and_target()
    # target equal to the drafter on slot 1: the draft is always accepted
    p_eq = p.copy()
    p_eq[0] = 0.0
    p_eq[0][cand[0]] = q[0]
    for u in (0.0, 0.5, 0.999999):
        n, com, _ = O.verify_rejection([cand[0][1], cand[1][0]], [q[0][1], q[1][0]], cand, q, p_eq, [u, 0.0], 0.3)
        assert n >= 1
    # a draft the target gives zero probability is always rejected, never re-drawn
    p_z = p.copy()
    p_z[0][4] = 0.0
    p_z[0] /= p_z[0].sum()
    for u_res in np.linspace(0, 0.999, 25):
        n, com, _ = O.verify_rejection([4, 1], [q[0][2], q[1][0]], cand, q, p_z, [0.0, 0.0], u_res)
        assert n == 0 and com[0] != 4 and list(com[1:]) == [-1, -1]
    # all accepted: the bonus comes from the last row
    n, com, nxt = O.verify_rejection([0, 1], [q[0][0], q[1][0]], cand, q, p, [0.0, 0.0], 0.0)
    assert n == 2 and list(com) == [0, 1, 0] and nxt == 0
    # an unnormalised slot-1 row that q covers everywhere: max(0, p - q) has no mass, so the token is
    # drawn from p_1 itself (mass 0.1 on token 0, 0.2 on token 4: u < 1/3 gives 0, above gives 4)
    p_u = p.copy()
    p_u[0] = 0.0
    p_u[0][0], p_u[0][4] = 0.1, 0.2
    for u_res, want in ((0.0, 0), (0.3333, 0), (0.3334, 4), (0.99, 4)):
        n, com, nxt = O.verify_rejection([2, 1], [q[0][1], q[1][0]], cand, q, p_u, [0.5, 0.0], u_res)
        assert n == 0 and nxt == want and list(com) == [want, -1, -1]


# ---------------------------------------------------------------------------------------------
# FP8 weight-only lm_head: E4M3 codes and per-row power-of-two scales
# ---------------------------------------------------------------------------------------------

def test_e4m3_codes_match_torch_float8():
    """The oracle's E4M3 rounding equals torch's float8_e4m3fn conversion (round to nearest,
    ties to even) on values with the bf16 significand width, on every midpoint between two
    neighbouring codes (the ties), and on every code value itself."""
    import torch
    rng = np.random.default_rng(8)
    vals = O.e4m3_value(np.array([c for c in range(256) if (c & 0x7F) != 0x7F]))
    mids = (vals[:-1] + vals[1:]) / 2
    mids = mids[np.abs(mids) <= 448]
    x = rng.uniform(-448, 448, 20000) * np.exp2(-rng.integers(0, 20, 20000))
    x = O.bf16_round(x)
    for arr in (x, vals, mids):
        ours = O.e4m3_code(arr)
        ref = torch.tensor(arr, dtype=torch.float64).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(ours, ref)


def test_e4m3_values_match_torch_float8():
    import torch
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(O.e4m3_value(codes), ref)
    assert O.e4m3_value(np.array([0x7E]))[0] == 448.0 and O.e4m3_value(np.array([0x01]))[0] == 2.0 ** -9


def test_fp8_rows_scale_and_error_bound():
    """Each row's largest magnitude lands in (224, 448] after its power-of-two scale; every
    dequantised weight is within half a code step of the weight (relative 2^-4 for normals,
    2^-10 absolute for subnormals, scaled); an all-zero row stays zero; signs are kept."""
    rng = np.random.default_rng(9)
    W = O.bf16_round(rng.normal(0, 0.02, (40, 256)))
    W[3] = 0.0
    W[5] *= 1e-3
    W[7, :] = -W[7, :]
    codes, scales = O.quantize_fp8_rows(W)
    D = O.dequantize_fp8_rows(codes, scales)
    for r in range(W.shape[0]):
        amax = np.max(np.abs(W[r]))
        if amax == 0:
            assert np.all(D[r] == 0) and scales[r] == 1.0
            continue
        a = amax / scales[r]
        assert 224 < a <= 448, (r, a)
        x = np.abs(W[r]) / scales[r]
        step = np.where(x >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(x, 2.0 ** -6))) - 3), 2.0 ** -9)
        assert np.all(np.abs(W[r] - D[r]) <= step / 2 * scales[r] * (1 + 1e-12)), r
        assert np.all((np.sign(D[r]) == np.sign(W[r])) | (D[r] == 0))


def test_fp8_row_exponent_closed_form():
    for amax, k in ((448.0, 0), (448.5, 1), (224.0, -1), (224.0001, 0), (1.0, -8), (0.03125, -13), (0.0, 0)):
        assert O.fp8_row_exponent(amax) == k, (amax, k)
