"""Seeded synthetic inputs for the drafter block pass.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  The CPU oracle and the HIP path are both fed from here
(tests and the benchmark call it, then hand the arrays to each side).

Every draw comes from a Philox counter generator keyed on (seed, name), so any
one tensor, or the target states of any one (sequence, position), can be
regenerated on its own without drawing everything before it.

Workload shapes follow the pages' drafters: "Architecture" (kb.ekarisky.com,
DFlash 2), Component Breakdown table -- about 2B parameters, 5 layers,
sliding window 1024, anchor in slot 0 and MASK in slots 1..K-1; block 8
(7 drafts) in the H200 benchmark table and block 16 as the default in
"DFlash Deep Dive" section 2.
"""
from __future__ import annotations

import dataclasses
import zlib
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class DraftConfig:
    """Shape of one synthetic drafter plus the workload it is run on."""
    name: str
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    n_taps: int
    target_hidden: int
    block_size: int
    sel_rank: int
    mask_id: int
    dtype: str                    # "f32" or "bf16": storage of weights, states, activations
    batch: int
    window: int = 1024
    topk: int = 16
    use_conv: bool = True
    conv_group: int = 0           # 0: scalar conv taps per position; G > 0: per-channel taps, one
                                  # correction per G channels (conv weights [2 d/G][d], bases [2][d])
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    weight_std: float = 0.02
    seed: int = 0
    # workload description (not part of the model)
    context: tuple = (1024, 1024)  # inclusive range of per-sequence context lengths L
    window_only_states: bool = False  # only the last `window` positions get target states
    match_prob: float | None = 0.7   # stand-in target: P(draft i == target argmax) per position
    cycles: int = 1
    tau_uniform: bool = False        # incremental workload: tau ~ U{1..K} per cycle

    @property
    def concat_width(self) -> int:
        return self.n_taps * self.target_hidden

    @property
    def q_width(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_width(self) -> int:
        return self.n_kv_heads * self.head_dim

    def replace(self, **kw) -> "DraftConfig":
        return dataclasses.replace(self, **kw)


def _big(name: str, **kw) -> DraftConfig:
    base = dict(n_layers=5, hidden=2048, n_heads=16, n_kv_heads=4, head_dim=128, ffn=6144,
                vocab=151936, n_taps=5, target_hidden=5120, sel_rank=16, mask_id=151935,
                dtype="bf16")
    base.update(kw)
    return DraftConfig(name=name, **base)


# The five workloads.  Names say what they are.
WORKLOADS = {
    # tiny fp32 drafter: 2 layers, hidden 256, 4 heads x 64, SwiGLU 768, vocab 4096,
    # 3 taps x 512 -> 256, context 128, K=8, batch 1, selector rank 8
    "tiny_fp32": DraftConfig(
        name="tiny_fp32", n_layers=2, hidden=256, n_heads=4, n_kv_heads=4, head_dim=64, ffn=768,
        vocab=4096, n_taps=3, target_hidden=512, block_size=8, sel_rank=8, mask_id=4095,
        dtype="f32", batch=1, context=(128, 128), match_prob=None),
    # 5-layer bf16 drafter, batch 1, K=16, full 1024 window of context
    "b1_k16": _big("b1_k16", block_size=16, batch=1, context=(1024, 1024)),
    # same drafter, K=8, batch 32, ragged contexts 512..4096, two-tap conv, 0.7 match rule
    "b32_k8_conv": _big("b32_k8_conv", block_size=8, batch=32, context=(512, 4096)),
    # incremental injection: batch 32, K=16, 2048-token prefixes, 64 cycles, tau ~ U{1..16}
    "b32_k16_incremental": _big("b32_k16_incremental", block_size=16, batch=32,
                                context=(2048, 2048), cycles=64, tau_uniform=True, match_prob=None),
    # long context, high batch: batch 64, context 32768, only the last 1024 positions matter
    "b64_k16_long": _big("b64_k16_long", block_size=16, batch=64, context=(32768, 32768),
                         window_only_states=True),
}


def _key(seed: int, *parts) -> int:
    h = 0
    for p in parts:
        h = zlib.crc32(repr(p).encode(), h)
    return (int(seed) << 64) | h


def rng(seed: int, *parts) -> np.random.Generator:
    """Independent Philox stream for one named draw."""
    return np.random.Generator(np.random.Philox(key=_key(seed, *parts)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns the uint16 bit patterns.

    Used only to define the stored inputs (bf16 weights and states)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Tensor:
    """A stored input: its values (float32, exactly the stored values) and the storage bits."""
    values: np.ndarray            # float32 array holding exactly what is stored
    storage: np.ndarray           # float32 array (f32 configs) or uint16 bf16 bits (bf16 configs)


def _store(x32: np.ndarray, dtype: str) -> Tensor:
    if dtype == "f32":
        x32 = np.ascontiguousarray(x32, dtype=np.float32)
        return Tensor(values=x32, storage=x32)
    bits = f32_to_bf16_bits(x32)
    return Tensor(values=bf16_bits_to_f32(bits), storage=bits)


def _normal(cfg: DraftConfig, name, shape, std, mean=0.0) -> Tensor:
    g = rng(cfg.seed, cfg.vocab, cfg.hidden, name)
    x = g.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return _store(x, cfg.dtype)


LAYER_TENSORS = ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "mlp_norm",
                 "w_gate", "w_up", "w_down",
                 "conv_attn_pre_w", "conv_attn_pre_b", "conv_attn_post_w", "conv_attn_post_b",
                 "conv_mlp_pre_w", "conv_mlp_pre_b", "conv_mlp_post_w", "conv_mlp_post_b")


def layer_shapes(cfg: DraftConfig) -> dict:
    d, f = cfg.hidden, cfg.ffn
    cw, cb = ((2 * d // cfg.conv_group, d), (2, d)) if cfg.conv_group else ((2, d), (2,))
    return {
        "attn_norm": (d,), "wq": (cfg.q_width, d), "wk": (cfg.kv_width, d), "wv": (cfg.kv_width, d),
        "q_norm": (cfg.head_dim,), "k_norm": (cfg.head_dim,), "wo": (d, cfg.q_width),
        "mlp_norm": (d,), "w_gate": (f, d), "w_up": (f, d), "w_down": (d, f),
        "conv_attn_pre_w": cw, "conv_attn_pre_b": cb,
        "conv_attn_post_w": cw, "conv_attn_post_b": cb,
        "conv_mlp_pre_w": cw, "conv_mlp_pre_b": cb,
        "conv_mlp_post_w": cw, "conv_mlp_post_b": cb,
    }


def global_shapes(cfg: DraftConfig) -> dict:
    return {
        "embed": (cfg.vocab, cfg.hidden), "lm_head": (cfg.vocab, cfg.hidden),
        "concat_norm": (cfg.concat_width,), "fc": (cfg.hidden, cfg.concat_width),
        "final_norm": (cfg.hidden,), "sel_A": (cfg.vocab, cfg.sel_rank),
        "sel_B": (cfg.vocab, cfg.sel_rank), "sel_WH": (cfg.sel_rank, cfg.hidden),
    }


def _is_gain(name: str) -> bool:
    return name.endswith("norm")


def make_weights(cfg: DraftConfig, selector_stress: bool = False) -> dict:
    """Random-init drafter: matrices, embeddings, conv and selector parameters ~ N(0, std);
    norm gains ~ 1 + N(0, std) so that a kernel ignoring a gain is caught.

    selector_stress draws A, B ~ N(0, 1) so that the pair term dominates the drafter logits."""
    s = cfg.weight_std
    w = {}
    for name, shape in global_shapes(cfg).items():
        std = 1.0 if (selector_stress and name in ("sel_A", "sel_B")) else s
        w[name] = _normal(cfg, name, shape, std, mean=1.0 if _is_gain(name) else 0.0)
    w["layers"] = []
    for l in range(cfg.n_layers):
        lw = {}
        for name, shape in layer_shapes(cfg).items():
            lw[name] = _normal(cfg, ("layer", l, name), shape, s, mean=1.0 if _is_gain(name) else 0.0)
        w["layers"].append(lw)
    return w


def conv_tensors(cfg: DraftConfig) -> list:
    """The conv parameters of every layer alone (the same draws make_weights makes for them), so
    that drafters differing only in conv form can share every other tensor."""
    s = cfg.weight_std
    shapes = layer_shapes(cfg)
    return [{n: _normal(cfg, ("layer", l, n), shp, s) for n, shp in shapes.items() if n.startswith("conv_")}
            for l in range(cfg.n_layers)]


def target_states(cfg: DraftConfig, seq: int, positions) -> Tensor:
    """Tapped target hidden states, N(0,1), one row of n_taps*target_hidden per (seq, position).

    Row (seq, p) is the same whichever batch of positions asks for it."""
    positions = np.asarray(positions, dtype=np.int64).reshape(-1)
    out = np.empty((positions.size, cfg.concat_width), dtype=np.float32)
    for i, p in enumerate(positions):
        out[i] = rng(cfg.seed, cfg.concat_width, "state", int(seq), int(p)).standard_normal(
            cfg.concat_width, dtype=np.float32)
    return _store(out, cfg.dtype)


def context_lengths(cfg: DraftConfig) -> np.ndarray:
    lo, hi = cfg.context
    if lo == hi:
        return np.full(cfg.batch, lo, dtype=np.int64)
    return rng(cfg.seed, "ctxlen", cfg.batch).integers(lo, hi + 1, size=cfg.batch)


def first_state_position(cfg: DraftConfig, L: int) -> int:
    """First position that receives a target state when the context has length L."""
    return max(0, L - cfg.window) if cfg.window_only_states else 0


def anchors(cfg: DraftConfig, cycle: int = 0) -> np.ndarray:
    """Anchor (last verified) token per sequence, uniform on [0, V-2] (never MASK)."""
    return rng(cfg.seed, "anchor", cycle, cfg.batch).integers(0, cfg.vocab - 1, size=cfg.batch).astype(np.int32)


def match_draws(cfg: DraftConfig, cycle: int = 0):
    """Random numbers of the stand-in target for one cycle.

    Returns (match [B][K-1] bool, alt_offset [B][K-1] int in [1, V-1], last [B] int in [0, V-1]).
    Position i matches the draft with probability match_prob; otherwise the target's argmax is
    (d_i + alt_offset) mod V, which never equals d_i."""
    K = cfg.block_size
    g = rng(cfg.seed, "match", cycle, cfg.batch)
    p = 0.7 if cfg.match_prob is None else cfg.match_prob
    match = g.random((cfg.batch, K - 1)) < p
    alt = g.integers(1, cfg.vocab, size=(cfg.batch, K - 1))
    last = g.integers(0, cfg.vocab, size=cfg.batch)
    return match, alt, last


def tau_draws(cfg: DraftConfig, cycle: int) -> np.ndarray:
    """Incremental workload: committed tokens per cycle, uniform on {1..K}."""
    return rng(cfg.seed, "tau", cycle, cfg.batch).integers(1, cfg.block_size + 1, size=cfg.batch)


def stand_in_target(draft: np.ndarray, match: np.ndarray, alt: np.ndarray, last: np.ndarray,
                    vocab: int) -> np.ndarray:
    """Target argmax per block slot built from a draft path and pre-drawn randomness.

    g[i-1] = d[i] where match[i-1] else (d[i] + alt[i-1]) mod V, for i = 1..K-1; g[K-1] = last.
    This stands in for a target model's verify pass (which needs weights this repo does not have)."""
    draft = np.asarray(draft, dtype=np.int64)
    B, km1 = draft.shape
    g = np.empty((B, km1 + 1), dtype=np.int32)
    g[:, :km1] = np.where(match, draft, (draft + alt) % vocab)
    g[:, km1] = last
    return g


def target_for_tau(draft: np.ndarray, tau: np.ndarray, alt: np.ndarray, last: np.ndarray,
                   vocab: int) -> np.ndarray:
    """Target argmax that makes greedy verification commit exactly tau[b] tokens."""
    draft = np.asarray(draft, dtype=np.int64)
    B, km1 = draft.shape
    idx = np.arange(km1)[None, :]
    match = idx < (np.asarray(tau)[:, None] - 1)
    return stand_in_target(draft, match, alt, last, vocab)


# ------------------------------------------------------------------------------ sampling stages

def lattice(cfg: DraftConfig, n: int, tag: int = 0):
    """A candidate lattice as the lm_head stage hands it to the selector, drawn directly.

    Returns (topk_ids [n][K-1][16] int32, distinct per slot, in [0, V-2]; topk_logits
    [n][K-1][16] float32, descending: a N(8, 2) head minus cumulative Exp(mean 0.4) gaps, the
    shape of a peaked lm_head row's top 16; h_final [n][K][hidden] float32 ~ N(0, 1), the
    spread of a final-normed hidden row)."""
    K, d = cfg.block_size, cfg.hidden
    g = rng(cfg.seed, "lattice", tag, n, K, d)
    ids = np.empty((n, K - 1, 16), dtype=np.int32)
    for b in range(n):
        for t in range(K - 1):
            ids[b, t] = g.choice(cfg.vocab - 1, size=16, replace=False)
    head = g.normal(8.0, 2.0, size=(n, K - 1, 1))
    gaps = g.exponential(0.4, size=(n, K - 1, 16))
    gaps[..., 0] = 0.0
    logits = (head - np.cumsum(gaps, axis=-1)).astype(np.float32)
    h_final = g.standard_normal((n, K, d), dtype=np.float32)
    return ids, logits, h_final


def sampling_uniforms(cfg: DraftConfig, n: int, tag: int = 0):
    """Uniform [0, 1) draws of one sampled cycle: (walk [n][K-1], accept [n][K-1], resample [n]),
    float32."""
    K = cfg.block_size
    g = rng(cfg.seed, "uniforms", tag, n, K)
    walk = g.random((n, K - 1), dtype=np.float32)
    acc = g.random((n, K - 1), dtype=np.float32)
    res = g.random(n, dtype=np.float32)
    return walk, acc, res


def target_probs(cfg: DraftConfig, cand_ids: np.ndarray, tag: int = 0, cand_mass: float = 0.7) -> np.ndarray:
    """Stand-in target distributions for one block, [n][K][V] float32, rows summing to 1.

    Row i-1 (slot i) puts about cand_mass on the drafter's 16 candidates of slot i (Gamma(1)
    weights) and the rest on the whole vocabulary (Gamma(0.05) weights: a few tokens hold most
    of it); the bonus row K-1 has only the vocabulary-wide part."""
    cand_ids = np.asarray(cand_ids)
    n, km1, _ = cand_ids.shape
    V = cfg.vocab
    g = rng(cfg.seed, "target_probs", tag, n, km1 + 1, V)
    out = np.empty((n, km1 + 1, V), dtype=np.float64)
    for b in range(n):
        for i in range(km1 + 1):
            bg = g.gamma(0.05, size=V)
            bg *= (1.0 - cand_mass if i < km1 else 1.0) / bg.sum()
            if i < km1:
                c = g.gamma(1.0, size=16)
                bg[cand_ids[b, i]] += cand_mass * c / c.sum()
            out[b, i] = bg
    return out.astype(np.float32)
