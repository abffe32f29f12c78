"""CPU oracle for the DFlash drafter block pass -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy.  Only the tests, the smoke check and the benchmark's
cpu_baseline leg may import this module; the library never does, and this module
imports nothing from the library.

What it computes, and where the pages say so:

* KV injection -- "Z Lab releases DFlash 2 for Qwen 3.8 27B" (llms.blog), section
  "Persistent Conditioning Through Target KV Injection": tapped target hidden states
  are concatenated, RMS-normalised, projected to the drafter width, and pushed
  through every draft layer's own K and V projections into that layer's KV cache.
  "Architecture" (kb.ekarisky.com, DFlash 2), Component Breakdown row "KV injection
  path" and "Internals Worth Knowing": projection ahead of the draft pass, with norm
  and RoPE applied to the projected keys.
* Single-pass block draft -- "Architecture", Component Breakdown rows "DFlash drafter
  backbone" (5 layers, sliding window 1024) and "Block attention mask" (slot 0 holds
  the anchor, slots 1..K-1 start as MASK, attention non-causal inside the block).
* Two-tap dynamic convolution -- "Architecture", section "Problem 2 -- Suffix decay
  is local": Conv(x)_t = k_t0 * x_t + k_t1 * x_{t-1}, around every attention and MLP
  sublayer, the first position reading the last verified token.  Two forms: the configs'
  scalar taps per position, and the page's per-channel coefficients (a learned base per
  channel plus a correction from the current row shared per 16 channels).
* Shared lm_head and top-16 candidates -- "Architecture", flowchart "Drafter" and the
  sequence diagram "One Cycle, Step by Step".
* Path selector -- "Architecture", section "Problem 1 -- Independent picks are
  incoherent": S_t(a, b) = U_t(b) + < A(a) * H(h_t), B(b) >.
* Greedy verification -- "Architecture", section "Speculative Decoding Context" and the
  sequence diagram: accept the longest valid prefix plus one bonus token.
* Sampling walk and rejection-sampling verification -- "Architecture", section "Problem 1"
  (sampling draws from the same pair scores; rejection sampling restores the exact target
  distribution), flowchart "Verification" and section "Speculative Decoding Context"
  (rejection sampling makes the scheme lossless).

Readings taken where the pages are silent (each also listed in the design notes):
RMSNorm over the whole concatenation then the fc projection, no bias; K/V of the
context are W_k c and W_v c with no extra input norm; per-head RMSNorm on q and k
then rotate-half RoPE (theta 10000) at absolute positions; context token j sits at
position j, the anchor at L (the current length), slot t at L+t; every block query
sees the last min(L, W) injected positions plus all K block slots; conv taps are
per-position scalars k_t = sigmoid(W_c x_t + b_c) (the 2048 -> 2 sigmoid-gated form),
slot 0 reads a zero predecessor; H(h) = sigmoid(W_H h) with h the final-normed
hidden at the candidate's slot; A and B are [V][r] tables; logits only for slots
1..K-1; top-16 ordered by (logit descending, id ascending).

Rounding points ("mode"):
  "exact"  -- everything float64.
  "bf16"   -- the drafter stores its KV cache in bf16: the context K/V written by
              injection and the block's own k/v (after per-head norm and RoPE) are rounded
              to bf16 (nearest, ties to even).  The shared lm_head is a bf16 product: its
              input, the final-normed hidden h_f of slots 1..K-1, is rounded to bf16 too
              (the returned h_final, which the selector reads, is not).  Weights and target
              states are bf16 inputs; every other value (activations, accumulations,
              softmax, logits, selector) stays float64.
"""
from __future__ import annotations

import itertools
import math

import numpy as np

F64 = np.float64


# --------------------------------------------------------------------------------------
# numeric helpers
# --------------------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Nearest bfloat16 value (8 exponent bits, 7 stored mantissa bits), ties to even.

    Works on the float64 bit pattern: drop the low 45 of the 52 mantissa bits with
    round-to-nearest-even.  Valid for magnitudes in bf16's normal range, which is all
    this oracle produces."""
    x = np.ascontiguousarray(x, dtype=F64)
    b = x.view(np.uint64)
    drop = np.uint64(45)
    half_minus_one = np.uint64((1 << 44) - 1)
    lsb = (b >> drop) & np.uint64(1)
    r = (b + half_minus_one + lsb) & ~np.uint64((1 << 45) - 1)
    return r.view(F64)


def _rounder(mode: str):
    if mode == "bf16":
        return bf16_round
    if mode == "exact":
        return lambda v: np.asarray(v, dtype=F64)
    raise ValueError(mode)


def as64(a) -> np.ndarray:
    return np.asarray(a, dtype=F64)


def rms_norm(x, gain, eps):
    """RMSNorm: x / sqrt(mean(x^2) + eps) * gain over the last axis."""
    x = as64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * as64(gain)


def sigmoid(x):
    x = as64(x)
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    x = as64(x)
    return x * sigmoid(x)


def rope(x, pos, theta):
    """Rotate-half rotary embedding on the last axis (size d_h) at integer positions `pos`.

    Pair (x_i, x_{i+d_h/2}) is rotated by angle pos * theta^(-2i/d_h)."""
    x = as64(x)
    dh = x.shape[-1]
    half = dh // 2
    inv = theta ** (-(np.arange(half, dtype=F64) * 2.0) / dh)
    ang = as64(pos)[..., None] * inv
    shape = ang.shape[:-1] + (1,) * (x.ndim - ang.ndim) + (half,)
    ang = ang.reshape(shape)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def two_tap_conv(x, w, b, use_conv=True):
    """Conv(x)_t = k_t0 * x_t + k_t1 * x_{t-1} over the rows of one block (x: [K][d]).

    k_t = sigmoid(W_c x_t + b_c) in R^2 (per-position taps from the current row).
    Slot 0 has no predecessor inside the block: x_{-1} = 0."""
    x = as64(x)
    if not use_conv:
        return x
    k = sigmoid(x @ as64(w).T + as64(b))          # [K][2]
    prev = np.zeros_like(x)
    prev[1:] = x[:-1]
    return k[:, 0:1] * x + k[:, 1:2] * prev


def two_tap_conv_grouped(x, base, wc, group):
    """Per-channel (depthwise) two-tap conv over the rows of one block (x: [K][d]):
    Conv(x)_t = k_t0 * x_t + k_t1 * x_{t-1} with coefficient vectors k_tj in R^d,

        k_tj[c] = sigmoid(base_j[c] + corr_tj[c // group]),   corr_tj = W_j x_t in R^(d / group),

    a learned base kernel per channel and tap plus a correction from the current row shared by
    each run of `group` consecutive channels ("Architecture", section "Problem 2 -- Suffix decay
    is local": one correction per 16 channels).  base: [2][d]; wc: [2 * d / group][d], tap 0's
    correction rows first.  Slot 0 has no predecessor inside the block: x_{-1} = 0."""
    x = as64(x)
    d = x.shape[1]
    ng = d // group
    corr = x @ as64(wc).T                                            # [K][2 * ng]
    base = as64(base)
    k0 = sigmoid(base[0][None, :] + np.repeat(corr[:, :ng], group, axis=1))
    k1 = sigmoid(base[1][None, :] + np.repeat(corr[:, ng:], group, axis=1))
    prev = np.zeros_like(x)
    prev[1:] = x[:-1]
    return k0 * x + k1 * prev


def sublayer_conv(cfg, x, w, b):
    """The conv of one sublayer boundary in the drafter's configured form: none, the scalar
    per-position taps (w: [2][d], b: [2]) or the per-channel form (cfg.conv_group > 0: w is the
    correction matrix [2 d / G][d], b the base kernel [2][d])."""
    if not cfg.use_conv:
        return as64(x)
    if getattr(cfg, "conv_group", 0):
        return two_tap_conv_grouped(x, b, w, cfg.conv_group)
    return two_tap_conv(x, w, b, True)


def topk_desc(values, k):
    """Indices of the k largest values, ordered by (value descending, index ascending)."""
    values = as64(values)
    order = np.lexsort((np.arange(values.size), -values))
    return order[:k]


# --------------------------------------------------------------------------------------
# the drafter's KV cache: by absolute position, no ring
# --------------------------------------------------------------------------------------

class DraftCache:
    """K/V of one sequence for every draft layer, keyed by absolute position."""

    def __init__(self, n_layers):
        self.k = [dict() for _ in range(n_layers)]
        self.v = [dict() for _ in range(n_layers)]
        self.length = 0          # anchor position of the next draft = one past the last injected

    def positions(self):
        return sorted(self.k[0].keys())


def inject(cfg, W, cache: DraftCache, positions, states, mode="bf16"):
    """Project target states of `positions` into every layer's cache.

    u = concat of the tapped states (one row per position); u_bar = RMSNorm(u) * g_in;
    c = W_fc u_bar; for each layer l: K_l = RoPE_p(RMSNorm_head(W_k^l c) * g_k^l),
    V_l = W_v^l c.  The cache length becomes max(position) + 1."""
    R = _rounder(mode)
    positions = np.asarray(positions, dtype=np.int64).reshape(-1)
    if positions.size == 0:
        return
    u = as64(states).reshape(positions.size, cfg.concat_width)
    u_bar = rms_norm(u, W["concat_norm"], cfg.rms_eps)
    c = u_bar @ as64(W["fc"]).T
    nkv, dh = cfg.n_kv_heads, cfg.head_dim
    for l, lw in enumerate(W["layers"]):
        k = (c @ as64(lw["wk"]).T).reshape(-1, nkv, dh)
        k = R(rope(rms_norm(k, lw["k_norm"], cfg.rms_eps), positions[:, None], cfg.rope_theta))
        v = R((c @ as64(lw["wv"]).T).reshape(-1, nkv, dh))
        for i, p in enumerate(positions):
            cache.k[l][int(p)] = k[i]
            cache.v[l][int(p)] = v[i]
    cache.length = max(cache.length, int(positions.max()) + 1)


def _attention(q, k, v, n_kv):
    """Softmax attention of every query row over every key row, per head, with GQA.

    q: [K][n_h][d_h]; k, v: [n_keys][n_kv][d_h].  Query head i reads kv head
    floor(i * n_kv / n_h).  Scale 1/sqrt(d_h).  No mask: every query sees every key."""
    K, nh, dh = q.shape
    out = np.empty_like(q)
    for i in range(nh):
        j = (i * n_kv) // nh
        s = q[:, i, :] @ k[:, j, :].T / math.sqrt(dh)     # [K][n_keys]
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, i, :] = p @ v[:, j, :]
    return out


def draft_block(cfg, W, cache: DraftCache, anchor, mode="bf16", block_ids=None, keep_logits=True):
    """One forward pass over the block [anchor, MASK, ..., MASK] at positions L..L+K-1.

    Returns dict with h_final [K][d], logits [K-1][V] (slots 1..K-1), topk_ids/topk_logits
    [K-1][topk].  `block_ids` overrides the block's token ids (used by invariant tests)."""
    R = _rounder(mode)
    K, d, nh, nkv, dh = cfg.block_size, cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    L = cache.length
    ids = np.full(K, cfg.mask_id, dtype=np.int64)
    ids[0] = anchor
    if block_ids is not None:
        ids = np.asarray(block_ids, dtype=np.int64)
    pos = L + np.arange(K)
    ctx = [p for p in range(max(0, L - cfg.window), L) if p in cache.k[0]]
    h = as64(W["embed"])[ids]                                   # residual stream [K][d]
    for l, lw in enumerate(W["layers"]):
        # attention sublayer
        z = rms_norm(h, lw["attn_norm"], cfg.rms_eps)
        y = sublayer_conv(cfg, z, lw["conv_attn_pre_w"], lw["conv_attn_pre_b"])
        q = (y @ as64(lw["wq"]).T).reshape(K, nh, dh)
        k = (y @ as64(lw["wk"]).T).reshape(K, nkv, dh)
        v = (y @ as64(lw["wv"]).T).reshape(K, nkv, dh)
        q = rope(rms_norm(q, lw["q_norm"], cfg.rms_eps), pos[:, None], cfg.rope_theta)
        k = R(rope(rms_norm(k, lw["k_norm"], cfg.rms_eps), pos[:, None], cfg.rope_theta))
        v = R(v)
        if ctx:
            keys = np.concatenate([np.stack([cache.k[l][p] for p in ctx]), k])
            vals = np.concatenate([np.stack([cache.v[l][p] for p in ctx]), v])
        else:
            keys, vals = k, v
        o = _attention(q, keys, vals, nkv).reshape(K, nh * dh)
        a = o @ as64(lw["wo"]).T
        h = h + sublayer_conv(cfg, a, lw["conv_attn_post_w"], lw["conv_attn_post_b"])
        # feed-forward sublayer
        z = rms_norm(h, lw["mlp_norm"], cfg.rms_eps)
        y = sublayer_conv(cfg, z, lw["conv_mlp_pre_w"], lw["conv_mlp_pre_b"])
        s = silu(y @ as64(lw["w_gate"]).T) * (y @ as64(lw["w_up"]).T)
        m = s @ as64(lw["w_down"]).T
        h = h + sublayer_conv(cfg, m, lw["conv_mlp_post_w"], lw["conv_mlp_post_b"])
    h_final = rms_norm(h, W["final_norm"], cfg.rms_eps)
    logits = R(h_final[1:]) @ as64(W["lm_head"]).T              # [K-1][V]; bf16 input in mode "bf16"
    tk = cfg.topk
    ids_out = np.stack([topk_desc(row, tk) for row in logits]).astype(np.int64)
    vals_out = np.take_along_axis(logits, ids_out, axis=1)
    out = dict(h_final=h_final, topk_ids=ids_out, topk_logits=vals_out, residual=h)
    if keep_logits:
        out["logits"] = logits
    return out


# --------------------------------------------------------------------------------------
# path selector
# --------------------------------------------------------------------------------------

def pair_scores(cfg, W, anchor, topk_ids, topk_logits, h_final):
    """S_t(a, b) = U_t(b) + sum_j A[a, j] * H_t[j] * B[b, j] for t = 1..K-1.

    H_t = sigmoid(W_H h_t), h_t the final-normed hidden of slot t.  Predecessors of slot 1
    are just the anchor; of slot t >= 2 the candidates of slot t-1.
    Returns a list: S[0] has shape [1][k], S[t-1] for t >= 2 has shape [k][k]."""
    A, B, WH = as64(W["sel_A"]), as64(W["sel_B"]), as64(W["sel_WH"])
    topk_ids = np.asarray(topk_ids, dtype=np.int64)
    U = as64(topk_logits)
    S = []
    for t in range(1, cfg.block_size):
        gate = sigmoid(WH @ as64(h_final[t]))
        prev = np.array([anchor]) if t == 1 else topk_ids[t - 2]
        pair = (A[prev] * gate) @ B[topk_ids[t - 1]].T
        S.append(U[t - 1][None, :] + pair)
    return S


def _path_better(s1, p1, s2, p2):
    """Total order on (score, candidate-index path): higher score first, then the
    lexicographically smaller index path."""
    return s1 > s2 or (s1 == s2 and tuple(p1) < tuple(p2))


def viterbi_2best(S):
    """Max-scoring path through the lattice, keeping the two best partial paths per state.

    Returns (best_path_indices, best_score, second_score).  second_score is -inf when the
    lattice has a single path."""
    n = len(S)
    k = S[0].shape[1]
    # lists[b] = up to two (score, path) entries, best first
    lists = [[(S[0][0, b], (b,))] for b in range(k)]
    for t in range(1, n):
        new = []
        for b in range(k):
            cands = []
            for a in range(k):
                for sc, path in lists[a]:
                    cands.append((sc + S[t][a, b], path + (b,)))
            best = []
            for c in cands:
                best.append(c)
                best.sort(key=lambda e: (-e[0], e[1]))
                best = best[:2]
            new.append(best)
        lists = new
    final = [e for lst in lists for e in lst]
    final.sort(key=lambda e: (-e[0], e[1]))
    second = final[1][0] if len(final) > 1 else -np.inf
    return list(final[0][1]), final[0][0], second


def greedy_walk(S):
    """Follow the best successor from the anchor; margin = smallest best-minus-second gap."""
    path, score, margin = [], 0.0, np.inf
    a = 0
    for t in range(len(S)):
        row = S[t][a]
        order = topk_desc(row, row.size)
        b = int(order[0])
        if row.size > 1:
            margin = min(margin, row[order[0]] - row[order[1]])
        path.append(b)
        score += row[b]
        a = b
    return path, score, margin


def select_path(cfg, W, anchor, topk_ids, topk_logits, h_final, mode="viterbi"):
    """Returns dict(path_idx, path_ids [K-1], score, margin)."""
    S = pair_scores(cfg, W, anchor, topk_ids, topk_logits, h_final)
    if mode == "viterbi":
        idx, best, second = viterbi_2best(S)
        margin = best - second
    elif mode == "greedy":
        idx, best, margin = greedy_walk(S)
    else:
        raise ValueError(mode)
    ids = np.asarray(topk_ids, dtype=np.int64)
    path_ids = np.array([ids[t, idx[t]] for t in range(len(idx))], dtype=np.int64)
    return dict(path_idx=np.array(idx), path_ids=path_ids, score=best, margin=margin)


def brute_force_paths(S):
    """Every path's score, best first (same total order as viterbi_2best).  Tiny lattices only."""
    k = S[0].shape[1]
    out = []
    for path in itertools.product(range(k), repeat=len(S)):
        sc = S[0][0, path[0]] + sum(S[t][path[t - 1], path[t]] for t in range(1, len(S)))
        out.append((sc, path))
    out.sort(key=lambda e: (-e[0], e[1]))
    return out


# --------------------------------------------------------------------------------------
# verification
# --------------------------------------------------------------------------------------

def verify_greedy(draft, target):
    """Greedy longest-prefix verification of one block.

    draft: d_1..d_{K-1}; target: g_0..g_{K-1}, g_i the target's argmax after slot i.
    n = largest m with d_i == g_{i-1} for all i <= m; tau = n + 1 committed tokens
    (the accepted drafts plus the bonus g_n).  Returns (n, committed [K] padded with -1,
    next_anchor = g_n)."""
    draft = [int(x) for x in draft]
    target = [int(x) for x in target]
    K = len(target)
    n = 0
    while n < K - 1 and draft[n] == target[n]:
        n += 1
    committed = draft[:n] + [target[n]] + [-1] * (K - 1 - n)
    return n, np.array(committed, dtype=np.int64), target[n]


# --------------------------------------------------------------------------------------
# sampling walk and rejection-sampling verification
# --------------------------------------------------------------------------------------

def inverse_cdf(weights, u):
    """Smallest index i with u * sum(weights) < sum(weights[:i + 1]) (u in [0, 1)); the last
    index with positive weight if rounding leaves none."""
    w = np.asarray(weights, dtype=F64)
    c = np.cumsum(w)
    target = u * c[-1]
    hit = np.nonzero(target < c)[0]
    if hit.size:
        return int(hit[0])
    return int(np.nonzero(w > 0)[0][-1])


def nucleus(q, top_p):
    """Top-p truncation of a distribution: rank the entries by probability (descending, ties to
    the lower index), keep every entry whose preceding mass in that ranking is below top_p (so
    the entry that crosses top_p stays), zero the rest and renormalise.  top_p >= 1 keeps all."""
    q = np.asarray(q, dtype=F64)
    if top_p >= 1.0:
        return q / q.sum()
    order = sorted(range(len(q)), key=lambda i: (-q[i], i))
    keep = np.zeros(len(q), dtype=bool)
    before = 0.0
    for i in order:
        if before < top_p:
            keep[i] = True
        before += q[i]
    r = np.where(keep, q, 0.0)
    return r / r.sum()


def sample_walk(S, uniforms, temperature, top_p=1.0):
    """Sampling walk over the candidate lattice.  At slot t the candidate b is drawn from the
    conditional distribution q_t(b) = softmax_b(S_t(a, b) / T) given the previous pick a (the
    anchor for slot 1), cut to its top-p nucleus (nucleus()), by inverse CDF in candidate order
    with the supplied uniform u_t.

    Returns (idx [K-1], q_path [K-1] = q_t(picked), q_cand [K-1][16] = q_t over the slot's
    candidates given the previous pick, after the cut)."""
    idx, q_path, q_cand = [], [], []
    a = 0
    for t, St in enumerate(S):
        z = np.asarray(St[a], dtype=F64) / temperature
        q = np.exp(z - z.max())
        q = nucleus(q / q.sum(), top_p)
        b = inverse_cdf(q, float(uniforms[t]))
        idx.append(b)
        q_path.append(q[b])
        q_cand.append(q)
        a = b
    return np.array(idx), np.array(q_path), np.array(q_cand)


def verify_rejection(draft, q_path, cand_ids, q_cand, target_probs, u_accept, u_resample):
    """Rejection-sampling verification of one block (speculative sampling).

    draft d_1..d_{K-1} with the drafter's probabilities q_i(d_i) (q_path) and its full
    distribution at slot i, q_i(v) = q_cand[i-1][j] for v = cand_ids[i-1][j], else 0;
    target_probs [K][V]: p_i for slot i at row i-1, the bonus distribution p_K at row K-1.
    Draft i is accepted iff u_i < p_i(d_i) / q_i(d_i), in order, up to the first rejection.
    At a rejection at slot i the committed token is drawn from r(v) = max(0, p_i(v) - q_i(v))
    (normalised); if every draft is accepted a bonus token is drawn from p_K.  Both draws use
    u_resample by inverse CDF in token order.  Returns (n, committed [K] padded with -1,
    next_anchor) like verify_greedy."""
    draft = [int(x) for x in draft]
    K = len(draft) + 1
    p = np.asarray(target_probs, dtype=F64)
    n = 0
    while n < K - 1 and u_accept[n] * q_path[n] < p[n, draft[n]]:
        n += 1
    if n < K - 1:
        r = p[n].copy()
        for j, v in enumerate(cand_ids[n]):
            r[int(v)] = max(0.0, p[n, int(v)] - float(q_cand[n][j]))
        if r.sum() <= 0:
            r = p[n].copy()
    else:
        r = p[K - 1].copy()
    tok = inverse_cdf(r, float(u_resample))
    committed = draft[:n] + [tok] + [-1] * (K - 1 - n)
    return n, np.array(committed, dtype=np.int64), tok


# --------------------------------------------------------------------------------------
# FP8 weight-only lm_head (a NEXT-step option, not part of the pages' pass)
# --------------------------------------------------------------------------------------
# The pages run drafts with quantised weights on one backend ("z-lab/dflash" README mirror,
# section "MLX (Apple Silicon)": 4-bit draft weights); they fix no format.  The format here
# is the OCP 8-bit floating point E4M3 encoding (bias 7, 3 mantissa bits, no infinities,
# largest finite 448, subnormals m * 2^-9), one code per weight, with one power-of-two scale
# per weight row: the row's largest magnitude maps into (224, 448].  Rounding is to the
# nearest code, ties to even.  A row whose largest magnitude is below 2^-64 is stored as zero.

E4M3_MAX = 448.0
FP8_ZERO_ROW = 2.0 ** -64


def fp8_row_exponent(amax):
    """Smallest integer k with amax <= 448 * 2^k (0 for a row stored as zero)."""
    amax = float(amax)
    if amax < FP8_ZERO_ROW:
        return 0
    k = math.frexp(amax)[1] - 9
    while amax > math.ldexp(E4M3_MAX, k):
        k += 1
    while amax <= math.ldexp(E4M3_MAX, k - 1):
        k -= 1
    return k


def e4m3_code(x):
    """E4M3 code (uint8) of the nearest representable value to each x (|x| <= 448, ties to
    even).  The sign bit of x is kept, so a negative x that rounds to zero gives -0 (0x80)."""
    x = np.asarray(x, dtype=F64)
    a = np.abs(x)
    assert np.all(a <= E4M3_MAX)
    codes = np.zeros(x.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormals (and zero): multiples of 2^-9; 8 * 2^-9 is the smallest normal, code 0x08
    codes[sub] = np.rint(a[sub] * 512.0).astype(np.int64)
    # normals: a = 2^f * mant, mant in [1, 2), f = floor(log2 a); 8 mantissa steps per binade
    an = a[~sub]
    f = np.frexp(an)[1] - 1
    m = np.rint((np.ldexp(an, -f) - 1.0) * 8.0).astype(np.int64)   # 0..8
    e = f + 7 + (m == 8)
    m = np.where(m == 8, 0, m)
    codes[~sub] = (e << 3) | m
    return (codes | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def e4m3_value(codes):
    """Value of each E4M3 code (the NaN codes 0x7F / 0xFF are not produced and not accepted)."""
    c = np.asarray(codes).astype(np.int64)
    assert not np.any((c & 0x7F) == 0x7F)
    e, m = (c >> 3) & 15, c & 7
    mag = np.where(e == 0, np.ldexp(m.astype(F64), -9), np.ldexp(1.0 + m / 8.0, e - 7))
    return np.where(c >> 7, -mag, mag)


def quantize_fp8_rows(W):
    """Per-row power-of-two scale and E4M3 codes of a weight matrix W [rows][cols] (the bf16
    values as float64).  Returns (codes uint8 [rows][cols], scales float64 [rows] = 2^k)."""
    W = np.asarray(W, dtype=F64)
    amax = np.max(np.abs(W), axis=1) if W.shape[1] else np.zeros(W.shape[0])
    zero = amax < FP8_ZERO_ROW
    k = np.array([fp8_row_exponent(a) for a in amax], dtype=np.int64)
    scales = np.where(zero, 1.0, np.ldexp(1.0, k))
    X = np.where(zero[:, None], np.where(np.signbit(W), -0.0, 0.0), np.ldexp(W, -k[:, None]))
    return e4m3_code(X), scales


def dequantize_fp8_rows(codes, scales):
    """The weights the codes stand for: value(code) * scale of the row (exact in float64)."""
    return e4m3_value(codes) * np.asarray(scales, dtype=F64)[:, None]


# --------------------------------------------------------------------------------------
# MXFP4 weight-only drafts (a NEXT-step option, not part of the pages' pass)
# --------------------------------------------------------------------------------------
# The pages run 4-bit drafts on one backend ("z-lab/dflash" README mirror, section "MLX (Apple
# Silicon)") and fix no format.  The format here is the OCP Microscaling MXFP4 encoding: along each
# weight row, blocks of 32 consecutive weights share one scale 2^s, stored as an 8-bit exponent
# byte s + 127 (E8M0); each weight is a 4-bit E2M1 element (sign bit, 2 exponent bits, 1 mantissa
# bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).  The block's largest magnitude a sets
# s = floor(log2 a) - 2, 2 being the exponent of the largest element magnitude 6 = 1.5 * 2^2, so a
# lands in [4, 8) * 2^s.  Each element is the E2M1 magnitude nearest to |w| / 2^s (ties to the even
# code, i.e. mantissa bit 0), magnitudes above 6 saturate to 6, and the sign bit is w's (so -0 is
# code 8).  A block whose largest magnitude is below 2^-64 is stored as zero codes with scale 1.
# Two elements per byte: element 2j in the low nibble, element 2j + 1 in the high one.

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
MX_BLOCK = 32
MX_ZERO_BLOCK = 2.0 ** -64


def e2m1_code(x):
    """4-bit E2M1 code (0..15) of each x: the nearest magnitude (ties to the even code, saturating
    at 6) with bit 3 the sign bit of x."""
    x = np.asarray(x, dtype=F64)
    a = np.minimum(np.abs(x), 6.0)
    dist = np.abs(a[..., None] - E2M1_MAG)
    nearest = dist == dist.min(axis=-1, keepdims=True)         # one code, or two at a midpoint
    idx = np.arange(8)
    even = np.where(nearest & (idx % 2 == 0), idx, 99).min(axis=-1)
    code = np.where(even < 99, even, np.where(nearest, idx, 99).min(axis=-1))
    return code | (np.signbit(x).astype(np.int64) << 3)


def e2m1_value(codes):
    """Value of each 4-bit E2M1 code."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAG[c & 7]
    return np.where(c & 8, -mag, mag)


def mx_block_exponent(amax):
    """s = floor(log2 amax) - 2 for one block (0 for a block stored as zero)."""
    amax = float(amax)
    if amax < MX_ZERO_BLOCK:
        return 0
    return math.frexp(amax)[1] - 3          # frexp: amax = m 2^e, m in [0.5, 1): floor(log2) = e - 1


def quantize_mxfp4_rows(W):
    """MXFP4 codes and block scales of W [rows][cols] (cols a multiple of 32; the bf16 values as
    float64).  Returns (codes uint8 [rows][cols/2], element 2j in the low nibble of byte j;
    scale bytes uint8 [rows][cols/32] = s + 127)."""
    W = np.asarray(W, dtype=F64)
    rows, cols = W.shape
    assert cols % MX_BLOCK == 0
    blocks = W.reshape(rows, cols // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(blocks), axis=-1)
    s = np.array([[mx_block_exponent(a) for a in r] for r in amax], dtype=np.int64).reshape(amax.shape)
    assert np.all((s + 127 >= 1) & (s + 127 <= 254))
    codes = e2m1_code(np.ldexp(blocks, -s[..., None])).reshape(rows, cols)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, (s + 127).astype(np.uint8)


def dequantize_mxfp4_rows(packed, scale_bytes):
    """The weights MXFP4 codes stand for: value(element) * 2^(scale byte - 127), exact in float64."""
    packed = np.asarray(packed).astype(np.int64)
    rows = packed.shape[0]
    codes = np.stack([packed & 15, packed >> 4], axis=-1).reshape(rows, -1)
    cols = codes.shape[1]
    sc = np.ldexp(1.0, np.asarray(scale_bytes).astype(np.int64) - 127)      # [rows][cols/32]
    return (e2m1_value(codes).reshape(rows, cols // MX_BLOCK, MX_BLOCK) * sc[..., None]).reshape(rows, cols)


def expected_tau(match_probs):
    """E[tau] when draft i is accepted with conditional probability r_i given all earlier
    ones were: 1 + sum_i prod_{j<=i} r_j (the bonus token always counts)."""
    acc, total = 1.0, 1.0
    for r in match_probs:
        acc *= r
        total += acc
    return total
