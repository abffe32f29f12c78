"""Thin ctypes binding of libdflash (include/dflash.h): the same entry points, argument
marshalling only.  Every step of the drafter pass runs in the HIP library; PyTorch only
provides device memory and streams.

Loading fails loudly if the library has not been built (build.py / __graft_entry__.build()).
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_double, c_float, c_int32, c_int64, c_size_t, c_uint64, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdflash.so")

DFLASH_OK = 0
DFLASH_F32, DFLASH_BF16 = 0, 1
SELECT_VITERBI, SELECT_GREEDY = 0, 1

# order of per-layer tensors (dflash_layer_tensor)
LAYER_TENSORS = ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "mlp_norm",
                 "w_gate", "w_up", "w_down",
                 "conv_attn_pre_w", "conv_attn_pre_b", "conv_attn_post_w", "conv_attn_post_b",
                 "conv_mlp_pre_w", "conv_mlp_pre_b", "conv_mlp_post_w", "conv_mlp_post_b")


class dflash_config(Structure):
    _fields_ = [(n, c_int32) for n in ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "ffn", "vocab",
                                       "n_taps", "target_hidden", "block_size", "window", "topk", "sel_rank",
                                       "mask_id", "use_conv")] + [
        ("rms_eps", c_float), ("rope_theta", c_float), ("dtype", c_int32), ("conv_group", c_int32)]


class dflash_weights(Structure):
    _fields_ = [(n, c_void_p) for n in ("embed", "lm_head", "concat_norm", "fc", "final_norm",
                                        "sel_A", "sel_B", "sel_WH")] + [("layers", POINTER(c_void_p))]


class dflash_kv_layout(Structure):
    _fields_ = [(n, c_size_t) for n in ("k_offset", "v_offset", "seq_len_offset", "seq_base_offset",
                                        "device_error_offset", "total_bytes")]


class DflashError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib = None


def lib():
    """The loaded libdflash (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libdflash is not built ({LIB_PATH} missing); run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    H = c_void_p
    sigs = {
        "dflash_config_check": (c_int32, [POINTER(dflash_config)]),
        "dflash_kv_cache_bytes": (c_size_t, [POINTER(dflash_config), c_int32]),
        "dflash_kv_cache_layout": (c_int32, [POINTER(dflash_config), c_int32, POINTER(dflash_kv_layout)]),
        "dflash_workspace_bytes": (c_size_t, [POINTER(dflash_config), c_int32, c_int32, c_int32]),
        "dflash_create": (c_int32, [POINTER(dflash_config), POINTER(dflash_weights), c_int32, c_int32, c_int32,
                                    c_void_p, c_size_t, c_void_p, c_size_t, POINTER(H)]),
        "dflash_destroy": (c_int32, [H]),
        "dflash_reset_seqs": (c_int32, [H, c_int32, c_void_p, c_void_p]),
        "dflash_inject_kv": (c_int32, [H, c_int32, c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p]),
        "dflash_draft_block": (c_int32, [H, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p]),
        "dflash_draft_block_static": (c_int32, [H, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                                c_void_p, c_void_p]),
        "dflash_select_path": (c_int32, [H, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                                         c_void_p, c_void_p, c_void_p]),
        "dflash_select_sample": (c_int32, [H, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_float, c_float,
                                           c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
        "dflash_verify_rejection": (c_int32, [c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                              c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                              c_void_p]),
        "dflash_verify_greedy": (c_int32, [c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                           c_void_p, c_void_p]),
        "dflash_synth_target_argmax": (c_int32, [c_int32, c_int32, c_int32, c_void_p, c_float, c_uint64, c_void_p,
                                                 c_void_p, c_void_p]),
        "dflash_quantize_fp8_rows": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
        "dflash_set_lm_head_fp8": (c_int32, [H, c_void_p, c_void_p]),
        "dflash_quantize_mxfp4_rows": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
        "dflash_set_lm_head_mxfp4": (c_int32, [H, c_void_p, c_void_p]),
        "dflash_set_mlp_fp8": (c_int32, [H, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
        "dflash_set_mlp_mxfp4": (c_int32, [H, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
        "dflash_set_attn_fp8": (c_int32, [H, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
        "dflash_set_inject_fp8": (c_int32, [H, c_void_p, c_void_p, c_void_p, c_void_p]),
        "dflash_set_attn_mxfp4": (c_int32, [H, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
        "dflash_set_inject_mxfp4": (c_int32, [H, c_void_p, c_void_p, c_void_p, c_void_p]),
        "dflash_block_weights": (c_int32, [c_void_p, c_int64, c_int64, c_void_p, c_void_p]),
        "dflash_set_blocked_weights": (c_int32, [H, POINTER(dflash_weights)]),
        "dflash_timing_enable": (c_int32, [H, c_int32]),
        "dflash_timing_read": (c_int32, [H, POINTER(c_double), POINTER(c_int32)]),
        "dflash_get_device_error": (c_int32, [H, POINTER(c_int32)]),
        "dflash_status_string": (c_char_p, [c_int32]),
        "dflash_last_error": (c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


EXPORTED = ("dflash_config_check", "dflash_kv_cache_bytes", "dflash_kv_cache_layout", "dflash_workspace_bytes",
            "dflash_create", "dflash_destroy", "dflash_reset_seqs", "dflash_inject_kv", "dflash_draft_block",
            "dflash_draft_block_static", "dflash_select_path", "dflash_select_sample", "dflash_verify_rejection", "dflash_verify_greedy",
            "dflash_synth_target_argmax", "dflash_quantize_fp8_rows", "dflash_set_lm_head_fp8", "dflash_set_mlp_fp8",
            "dflash_quantize_mxfp4_rows", "dflash_set_lm_head_mxfp4", "dflash_set_mlp_mxfp4",
            "dflash_set_attn_fp8", "dflash_set_inject_fp8", "dflash_set_attn_mxfp4", "dflash_set_inject_mxfp4",
            "dflash_block_weights", "dflash_set_blocked_weights", "dflash_timing_enable",
            "dflash_timing_read", "dflash_get_device_error", "dflash_status_string", "dflash_last_error")


def check(fn_name, status):
    if status != DFLASH_OK:
        msg = lib().dflash_last_error().decode(errors="replace")
        raise DflashError(fn_name, status, msg)


def make_config(cfg) -> dflash_config:
    """dflash_config from any object with the drafter's fields (e.g. synth.DraftConfig)."""
    return dflash_config(
        n_layers=cfg.n_layers, hidden=cfg.hidden, n_heads=cfg.n_heads, n_kv_heads=cfg.n_kv_heads,
        head_dim=cfg.head_dim, ffn=cfg.ffn, vocab=cfg.vocab, n_taps=cfg.n_taps, target_hidden=cfg.target_hidden,
        block_size=cfg.block_size, window=cfg.window, topk=cfg.topk, sel_rank=cfg.sel_rank, mask_id=cfg.mask_id,
        use_conv=int(bool(cfg.use_conv)), rms_eps=cfg.rms_eps, rope_theta=cfg.rope_theta,
        dtype=DFLASH_BF16 if cfg.dtype == "bf16" else DFLASH_F32, conv_group=int(getattr(cfg, "conv_group", 0)))


def ptr(t) -> int | None:
    """Device (or host) address of a tensor, None for None."""
    return None if t is None else t.data_ptr()


# ------------------------------------------------------------------ entry points, same names

def dflash_config_check(cfg):
    c = make_config(cfg)
    return lib().dflash_config_check(ctypes.byref(c))


def dflash_kv_cache_bytes(cfg, max_seqs):
    c = make_config(cfg)
    return lib().dflash_kv_cache_bytes(ctypes.byref(c), max_seqs)


def dflash_kv_cache_layout(cfg, max_seqs) -> dflash_kv_layout:
    c = make_config(cfg)
    out = dflash_kv_layout()
    check("dflash_kv_cache_layout", lib().dflash_kv_cache_layout(ctypes.byref(c), max_seqs, ctypes.byref(out)))
    return out


def dflash_workspace_bytes(cfg, max_seqs, max_batch, max_inject_rows):
    c = make_config(cfg)
    return lib().dflash_workspace_bytes(ctypes.byref(c), max_seqs, max_batch, max_inject_rows)


def dflash_verify_greedy(n_seq, block_size, draft_ids, target_argmax, n_accepted, n_commit, committed, next_anchor,
                         stream=None):
    check("dflash_verify_greedy", lib().dflash_verify_greedy(
        n_seq, block_size, ptr(draft_ids), ptr(target_argmax), ptr(n_accepted), ptr(n_commit), ptr(committed),
        ptr(next_anchor), stream))


def dflash_verify_rejection(n_seq, block_size, vocab, draft_ids, q_path, topk_ids, q_cand, target_probs, u_accept,
                            u_resample, n_accepted, n_commit, committed, next_anchor, stream=None):
    check("dflash_verify_rejection", lib().dflash_verify_rejection(
        n_seq, block_size, vocab, ptr(draft_ids), ptr(q_path), ptr(topk_ids), ptr(q_cand), ptr(target_probs),
        ptr(u_accept), ptr(u_resample), ptr(n_accepted), ptr(n_commit), ptr(committed), ptr(next_anchor), stream))


def dflash_block_weights(src, dst, stream=None):
    """16-row-blocked copy (same size, bf16) of a row-major bf16 matrix [rows][cols] into dst."""
    rows, cols = src.shape
    check("dflash_block_weights", lib().dflash_block_weights(ptr(src), rows, cols, ptr(dst), stream))


def dflash_quantize_mxfp4_rows(src, codes, scales, stream=None):
    """MXFP4 codes [rows][cols/2] (uint8) and block scale bytes [rows][cols/32] (uint8) of a bf16 matrix."""
    rows, cols = src.shape
    check("dflash_quantize_mxfp4_rows", lib().dflash_quantize_mxfp4_rows(ptr(src), rows, cols, ptr(codes), ptr(scales),
                                                                         stream))


def dflash_synth_target_argmax(n_seq, block_size, vocab, draft_ids, match_prob, seed, counter, target_argmax,
                               stream=None):
    check("dflash_synth_target_argmax", lib().dflash_synth_target_argmax(
        n_seq, block_size, vocab, ptr(draft_ids), match_prob, seed, ptr(counter), ptr(target_argmax), stream))


def dflash_quantize_fp8_rows(src, codes, row_scales, stream=None):
    """E4M3 codes and per-row power-of-two scales of a bf16 matrix src [rows][cols] (device)."""
    rows, cols = src.shape
    check("dflash_quantize_fp8_rows", lib().dflash_quantize_fp8_rows(ptr(src), rows, cols, ptr(codes), ptr(row_scales),
                                                                     stream))


class Drafter:
    """One libdflash handle plus the caller-owned device buffers it borrows.

    `weights` maps the tensor names of synth.global_shapes / LAYER_TENSORS to device tensors
    (layers: a list of per-layer dicts).  All methods enqueue on `stream` (a raw hipStream_t
    address, None = default stream) and return immediately."""

    def __init__(self, cfg, weights, max_seqs, max_batch, max_inject_rows=1024, device="cuda", kv_from=None):
        """kv_from: another Drafter of the same config and max_seqs whose KV cache this handle
        shares (each handle keeps its own workspace)."""
        import torch
        self.cfg = cfg
        self.c = make_config(cfg)
        st = lib().dflash_config_check(ctypes.byref(self.c))
        check("dflash_config_check", st)
        self.weights = weights  # keep alive
        self.max_seqs, self.max_batch, self.max_inject_rows = max_seqs, max_batch, max_inject_rows
        self.kv_layout = dflash_kv_cache_layout(cfg, max_seqs)
        if kv_from is not None:
            if kv_from.max_seqs != max_seqs or kv_from.kv_layout.total_bytes != self.kv_layout.total_bytes:
                raise ValueError("kv_from must have the same config and max_seqs")
            self.kv = kv_from.kv
        else:
            self.kv = torch.zeros(self.kv_layout.total_bytes, dtype=torch.uint8, device=device)
        nbytes = dflash_workspace_bytes(cfg, max_seqs, max_batch, max_inject_rows)
        if nbytes == 0:
            raise DflashError("dflash_workspace_bytes", -1, "invalid sizes")
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        w = dflash_weights()
        for name in ("embed", "lm_head", "concat_norm", "fc", "final_norm", "sel_A", "sel_B", "sel_WH"):
            setattr(w, name, weights[name].data_ptr())
        flat = []
        for lw in weights["layers"]:
            flat += [lw[n].data_ptr() for n in LAYER_TENSORS]
        self._layers = (c_void_p * len(flat))(*flat)
        w.layers = ctypes.cast(self._layers, POINTER(c_void_p))
        self._w = w
        h = c_void_p()
        check("dflash_create", lib().dflash_create(ctypes.byref(self.c), ctypes.byref(w), max_seqs, max_batch,
                                                   max_inject_rows, self.kv.data_ptr(), self.kv.numel(),
                                                   self.ws.data_ptr(), self.ws.numel(), ctypes.byref(h)))
        self.h = h

    def dflash_set_lm_head_fp8(self, codes, row_scales):
        """Use E4M3 lm_head codes [V][d] with their row scales [V] (None, None: the bf16 lm_head)."""
        self._lm_fp8 = (codes, row_scales)   # keep alive
        check("dflash_set_lm_head_fp8", lib().dflash_set_lm_head_fp8(self.h, ptr(codes), ptr(row_scales)))

    def dflash_set_lm_head_mxfp4(self, codes, scales):
        """Use MXFP4 codes [vocab][hidden/2] with block scale bytes [vocab][hidden/32] for the lm_head
        (None, None: back to bf16)."""
        self._lm_fp4 = (codes, scales)   # keep alive
        check("dflash_set_lm_head_mxfp4", lib().dflash_set_lm_head_mxfp4(self.h, ptr(codes), ptr(scales)))

    def dflash_set_mlp_fp8(self, layer, gate_up_codes, gate_up_scales, down_codes, down_scales):
        """Use E4M3 codes for layer's MLP: stacked [gate; up] [2 ffn][d] and down [d][ffn], with row
        scales (all None: the bf16 matrices)."""
        if not hasattr(self, "_mlp_fp8"):
            self._mlp_fp8 = {}
        self._mlp_fp8[layer] = (gate_up_codes, gate_up_scales, down_codes, down_scales)   # keep alive
        check("dflash_set_mlp_fp8", lib().dflash_set_mlp_fp8(self.h, layer, ptr(gate_up_codes), ptr(gate_up_scales),
                                                             ptr(down_codes), ptr(down_scales)))

    def dflash_set_mlp_mxfp4(self, layer, gate_up_codes, gate_up_scales, down_codes, down_scales):
        """Use MXFP4 codes for layer's MLP: stacked [gate; up] [2 ffn][d/2] and down [d][ffn/2], with
        block scale bytes [rows][cols/32] (all None: the bf16 matrices)."""
        if not hasattr(self, "_mlp_fp8"):
            self._mlp_fp8 = {}
        self._mlp_fp8[layer] = (gate_up_codes, gate_up_scales, down_codes, down_scales)   # keep alive
        check("dflash_set_mlp_mxfp4", lib().dflash_set_mlp_mxfp4(self.h, layer, ptr(gate_up_codes),
                                                                 ptr(gate_up_scales), ptr(down_codes),
                                                                 ptr(down_scales)))

    def dflash_set_attn_fp8(self, layer, qkv_codes, qkv_scales, o_codes, o_scales):
        """Use E4M3 codes for layer's stacked [wq; wk; wv] and wo (all None: bf16)."""
        if not hasattr(self, "_attn_fp8"):
            self._attn_fp8 = {}
        self._attn_fp8[layer] = (qkv_codes, qkv_scales, o_codes, o_scales)   # keep alive
        check("dflash_set_attn_fp8", lib().dflash_set_attn_fp8(self.h, layer, ptr(qkv_codes), ptr(qkv_scales),
                                                               ptr(o_codes), ptr(o_scales)))

    def dflash_set_inject_fp8(self, fc_codes, fc_scales, kv_codes, kv_scales):
        """Use E4M3 codes for W_fc and the stacked per-layer [wk; wv] (all None: bf16)."""
        self._inj_fp8 = (fc_codes, fc_scales, kv_codes, kv_scales)   # keep alive
        check("dflash_set_inject_fp8", lib().dflash_set_inject_fp8(self.h, ptr(fc_codes), ptr(fc_scales),
                                                                   ptr(kv_codes), ptr(kv_scales)))

    def dflash_set_attn_mxfp4(self, layer, qkv_codes, qkv_scales, o_codes, o_scales):
        """Use MXFP4 codes and block scale bytes for layer's stacked [wq; wk; wv] and wo (all None: bf16)."""
        if not hasattr(self, "_attn_fp8"):
            self._attn_fp8 = {}
        self._attn_fp8[layer] = (qkv_codes, qkv_scales, o_codes, o_scales)   # keep alive
        check("dflash_set_attn_mxfp4", lib().dflash_set_attn_mxfp4(self.h, layer, ptr(qkv_codes), ptr(qkv_scales),
                                                                   ptr(o_codes), ptr(o_scales)))

    def dflash_set_blocked_weights(self, blocked):
        """Register blocked copies (dflash_block_weights) of the bf16 weight matrices: a dict with
        optional "lm_head", "fc" and "layers" (one dict per layer with any of wq, wk, wv, wo, w_gate,
        w_up, w_down); None removes them."""
        if blocked is None:
            self._blocked = None
            check("dflash_set_blocked_weights", lib().dflash_set_blocked_weights(self.h, None))
            return
        bw = dflash_weights()
        for name in ("lm_head", "fc"):
            if blocked.get(name) is not None:
                setattr(bw, name, blocked[name].data_ptr())
        keep = [bw]
        if blocked.get("layers") is not None:
            if len(blocked["layers"]) != self.c.n_layers:
                raise ValueError("blocked['layers'] needs one dict per layer")
            flat = [(lw[n].data_ptr() if lw.get(n) is not None else None) for lw in blocked["layers"]
                    for n in LAYER_TENSORS]
            arr = (c_void_p * len(flat))(*flat)
            bw.layers = ctypes.cast(arr, POINTER(c_void_p))
            keep.append(arr)
        self._blocked = (blocked, keep)   # keep alive
        check("dflash_set_blocked_weights", lib().dflash_set_blocked_weights(self.h, ctypes.byref(bw)))

    def dflash_set_inject_mxfp4(self, fc_codes, fc_scales, kv_codes, kv_scales):
        """Use MXFP4 codes and block scale bytes for W_fc and the stacked per-layer [wk; wv] (all None: bf16)."""
        self._inj_fp8 = (fc_codes, fc_scales, kv_codes, kv_scales)   # keep alive
        check("dflash_set_inject_mxfp4", lib().dflash_set_inject_mxfp4(self.h, ptr(fc_codes), ptr(fc_scales),
                                                                       ptr(kv_codes), ptr(kv_scales)))

    def close(self):
        if self.h:
            check("dflash_destroy", lib().dflash_destroy(self.h))
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- views of the KV region (for tests)
    def kv_views(self):
        import torch
        c, L = self.cfg, self.kv_layout
        dt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
        es = 2 if c.dtype == "bf16" else 4
        shape = (c.n_layers, self.max_seqs, c.n_kv_heads, c.window, c.head_dim)
        n = 1
        for s in shape:
            n *= s
        k = self.kv[L.k_offset:L.k_offset + n * es].view(dt).view(shape)
        v = self.kv[L.v_offset:L.v_offset + n * es].view(dt).view(shape)
        sl = self.kv[L.seq_len_offset:L.seq_len_offset + 4 * self.max_seqs].view(torch.int32)
        sb = self.kv[L.seq_base_offset:L.seq_base_offset + 4 * self.max_seqs].view(torch.int32)
        return k, v, sl, sb

    # -- entry points
    def dflash_reset_seqs(self, seq_ids, stream=None):
        check("dflash_reset_seqs", lib().dflash_reset_seqs(self.h, seq_ids.numel(), ptr(seq_ids), stream))

    def dflash_inject_kv(self, seq_ids, n_new, max_new, target_hidden, start_pos=None, stream=None):
        check("dflash_inject_kv", lib().dflash_inject_kv(self.h, seq_ids.numel(), ptr(seq_ids), ptr(start_pos),
                                                         ptr(n_new), max_new, ptr(target_hidden), stream))

    def dflash_draft_block(self, seq_ids, anchor_ids, topk_ids, topk_logits, h_final, logits=None, stream=None):
        check("dflash_draft_block", lib().dflash_draft_block(self.h, seq_ids.numel(), ptr(seq_ids), ptr(anchor_ids),
                                                             ptr(topk_ids), ptr(topk_logits), ptr(h_final),
                                                             ptr(logits), stream))

    def dflash_draft_block_static(self, seq_ids, anchor_ids, topk_ids, topk_logits, h_final, logits=None, stream=None):
        check("dflash_draft_block_static", lib().dflash_draft_block_static(
            self.h, seq_ids.numel(), ptr(seq_ids), ptr(anchor_ids), ptr(topk_ids), ptr(topk_logits), ptr(h_final),
            ptr(logits), stream))

    def dflash_select_path(self, anchor_ids, topk_ids, topk_logits, h_final, mode, path_ids, path_score=None,
                           margin=None, stream=None):
        check("dflash_select_path", lib().dflash_select_path(self.h, anchor_ids.numel(), ptr(anchor_ids),
                                                             ptr(topk_ids), ptr(topk_logits), ptr(h_final), mode,
                                                             ptr(path_ids), ptr(path_score), ptr(margin), stream))

    def dflash_select_sample(self, anchor_ids, topk_ids, topk_logits, h_final, temperature, top_p, uniforms, path_ids,
                             q_path, q_cand=None, stream=None):
        check("dflash_select_sample", lib().dflash_select_sample(self.h, anchor_ids.numel(), ptr(anchor_ids),
                                                                 ptr(topk_ids), ptr(topk_logits), ptr(h_final),
                                                                 float(temperature), float(top_p), ptr(uniforms),
                                                                 ptr(path_ids), ptr(q_path), ptr(q_cand), stream))

    def dflash_timing_enable(self, capacity):
        check("dflash_timing_enable", lib().dflash_timing_enable(self.h, capacity))

    def dflash_timing_read(self):
        tot, n = c_double(), c_int32()
        check("dflash_timing_read", lib().dflash_timing_read(self.h, ctypes.byref(tot), ctypes.byref(n)))
        return tot.value, n.value

    def dflash_get_device_error(self):
        code = c_int32()
        check("dflash_get_device_error", lib().dflash_get_device_error(self.h, ctypes.byref(code)))
        return code.value

    # -- output allocation helper
    def outputs(self, n_seq, logits=False):
        import torch
        c = self.cfg
        dev = self.kv.device
        dt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
        K = c.block_size
        out = dict(
            topk_ids=torch.empty((n_seq, K - 1, 16), dtype=torch.int32, device=dev),
            topk_logits=torch.empty((n_seq, K - 1, 16), dtype=torch.float32, device=dev),
            h_final=torch.empty((n_seq, K, c.hidden), dtype=torch.float32, device=dev),
            logits=torch.empty((n_seq, K - 1, c.vocab), dtype=torch.float32, device=dev) if logits else None,
        )
        return out


def upload_weights(w_np, dtype: str, device="cuda"):
    """Copies synth.make_weights(...) output (storage arrays) to device tensors."""
    import numpy as np
    import torch

    def up(t):
        a = t.storage
        if dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    out = {k: up(v) for k, v in w_np.items() if k != "layers"}
    out["layers"] = [{k: up(v) for k, v in lw.items()} for lw in w_np["layers"]]
    return out
