"""Host-side checks of the C ABI: the library loads without a GPU, exports every symbol the
header declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

from block_diffusion_draft_inject_amd import binding as B
from block_diffusion_draft_inject_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libdflash not built")


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "dflash.h")).read()
    return sorted(set(re.findall(r"DFLASH_API\s+[\w\s\*]+?\b(dflash_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) >= 17
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(B.EXPORTED) == names


def test_config_check_accepts_workloads_and_rejects_bad_shapes():
    for name, cfg in synth.WORKLOADS.items():
        assert B.dflash_config_check(cfg) == 0, (name, B.lib().dflash_last_error())
    base = synth.WORKLOADS["b1_k16"]
    assert B.dflash_config_check(base.replace(topk=8)) == -3
    assert B.dflash_config_check(base.replace(head_dim=64)) == -3          # bf16 attention needs 128
    assert B.dflash_config_check(base.replace(block_size=1)) == -3
    assert B.dflash_config_check(base.replace(n_kv_heads=3)) == -3
    assert B.dflash_config_check(base.replace(block_size=32)) == -3        # 4 heads/group * 32 > 64
    assert B.dflash_config_check(base.replace(mask_id=151936)) == -1
    # the O and down projections' k-splits must fit the sublayer epilogue (K <= 16384)
    assert B.dflash_config_check(base.replace(ffn=16384)) == 0
    assert B.dflash_config_check(base.replace(ffn=16384 + 128)) == -3
    assert B.dflash_config_check(base.replace(n_heads=132, n_kv_heads=4)) == -3   # 132 x 128 > 16384
    assert B.lib().dflash_config_check(None) == -1
    assert b"NULL" in B.lib().dflash_last_error()


def test_sizes():
    cfg = synth.WORKLOADS["b1_k16"]
    kv = B.dflash_kv_cache_layout(cfg, 4)
    one = 5 * 4 * 4 * 1024 * 128 * 2
    assert kv.k_offset == 0 and kv.v_offset >= one and kv.seq_len_offset >= kv.v_offset + one
    assert kv.total_bytes == B.dflash_kv_cache_bytes(cfg, 4)
    assert B.dflash_workspace_bytes(cfg, 4, 2, 64) > 0
    assert B.dflash_workspace_bytes(cfg, 4, 0, 64) == 0
    assert B.dflash_kv_cache_bytes(cfg.replace(topk=3), 4) == 0
    # a bigger batch needs at least as much workspace
    assert B.dflash_workspace_bytes(cfg, 64, 64, 1024) >= B.dflash_workspace_bytes(cfg, 4, 2, 64)


def _fake_handle(cfg, max_seqs=4, max_batch=2, rows=64):
    """A handle over fake (never dereferenced) device addresses: creation is host-only."""
    L = B.lib()
    c = B.make_config(cfg)
    w = B.dflash_weights()
    for i, n in enumerate(("embed", "lm_head", "concat_norm", "fc", "final_norm", "sel_A", "sel_B", "sel_WH")):
        setattr(w, n, 0x1000 * (i + 1))
    flat = (ctypes.c_void_p * (cfg.n_layers * len(B.LAYER_TENSORS)))(*[0x100000 + 16 * i for i in range(
        cfg.n_layers * len(B.LAYER_TENSORS))])
    w.layers = ctypes.cast(flat, ctypes.POINTER(ctypes.c_void_p))
    kvb = B.dflash_kv_cache_bytes(cfg, max_seqs)
    wsb = B.dflash_workspace_bytes(cfg, max_seqs, max_batch, rows)
    h = ctypes.c_void_p()
    st = L.dflash_create(ctypes.byref(c), ctypes.byref(w), max_seqs, max_batch, rows, 0x7000000, kvb, 0x9000000,
                         wsb, ctypes.byref(h))
    return st, h, (c, w, flat), kvb, wsb


def test_create_validates_before_any_device_call():
    cfg = synth.WORKLOADS["tiny_fp32"]
    st, h, keep, kvb, wsb = _fake_handle(cfg)
    assert st == 0, B.lib().dflash_last_error()
    L = B.lib()
    # too-small buffers
    c, w, _ = keep
    h2 = ctypes.c_void_p()
    assert L.dflash_create(ctypes.byref(c), ctypes.byref(w), 4, 2, 64, 0x7000000, kvb - 1, 0x9000000, wsb,
                           ctypes.byref(h2)) == -2
    assert L.dflash_create(ctypes.byref(c), ctypes.byref(w), 4, 2, 64, 0x7000000, kvb, 0x9000000, wsb - 1,
                           ctypes.byref(h2)) == -2
    assert L.dflash_create(ctypes.byref(c), ctypes.byref(w), 4, 2, 64, None, kvb, 0x9000000, wsb,
                           ctypes.byref(h2)) == -1
    w.fc = None
    assert L.dflash_create(ctypes.byref(c), ctypes.byref(w), 4, 2, 64, 0x7000000, kvb, 0x9000000, wsb,
                           ctypes.byref(h2)) == -1
    # entry points reject host-checkable problems without enqueueing anything
    fake = 0x5000
    assert L.dflash_draft_block(h, 3, fake, fake, fake, fake, fake, None, None) == -2      # n_seq > max_batch
    assert L.dflash_draft_block(h, 0, fake, fake, fake, fake, fake, None, None) == -2
    assert L.dflash_draft_block(h, 1, None, fake, fake, fake, fake, None, None) == -1
    assert L.dflash_inject_kv(h, 5, fake, None, fake, 4, fake, None) == -2                  # n_seq > max_seqs
    assert L.dflash_inject_kv(h, 1, None, None, fake, 4, fake, None) == -1
    assert L.dflash_inject_kv(h, 1, fake, None, fake, -1, fake, None) == -1
    assert L.dflash_inject_kv(h, 0, None, None, None, 4, None, None) == 0                   # nothing to do
    assert L.dflash_select_path(h, 1, fake, fake, fake, fake, 7, fake, None, None, None) == -1
    assert L.dflash_select_path(h, 3, fake, fake, fake, fake, 0, fake, None, None, None) == -2
    assert L.dflash_verify_greedy(2, 8, None, fake, fake, None, fake, fake, None) == -1
    assert L.dflash_verify_greedy(2, 1, fake, fake, fake, None, fake, fake, None) == -1
    assert L.dflash_verify_greedy(0, 8, None, None, None, None, None, None, None) == 0
    assert L.dflash_synth_target_argmax(2000, 8, 100, fake, 0.7, 0, fake, fake, None) == -2
    assert L.dflash_synth_target_argmax(2, 8, 100, fake, 1.5, 0, fake, fake, None) == -1
    assert L.dflash_timing_enable(h, -1) == -1
    assert L.dflash_quantize_mxfp4_rows(fake, 4, 48, fake, fake, None) == -1            # cols not a multiple of 32
    assert L.dflash_quantize_mxfp4_rows(None, 4, 64, fake, fake, None) == -1
    assert L.dflash_quantize_mxfp4_rows(None, 0, 64, None, None, None) == 0             # nothing to do
    assert L.dflash_set_lm_head_mxfp4(h, fake, None) == -1
    assert L.dflash_set_lm_head_mxfp4(h, fake, fake) == -3                              # fp32 drafter
    assert L.dflash_set_lm_head_mxfp4(h, None, None) == 0
    assert L.dflash_set_mlp_mxfp4(h, 0, fake, fake, fake, None) == -1                  # three of four set
    assert L.dflash_set_mlp_mxfp4(h, 9, None, None, None, None) == -1                  # no such layer
    assert L.dflash_set_mlp_mxfp4(h, 0, fake, fake, fake, fake) == -3                  # fp32 drafter
    assert L.dflash_set_mlp_mxfp4(h, 0, None, None, None, None) == 0
    assert L.dflash_set_attn_mxfp4(h, 0, fake, fake, None, fake) == -1                 # three of four set
    assert L.dflash_set_attn_mxfp4(h, -1, None, None, None, None) == -1                # no such layer
    assert L.dflash_set_attn_mxfp4(h, 0, fake, fake, fake, fake) == -3                 # fp32 drafter
    assert L.dflash_set_attn_mxfp4(h, 0, None, None, None, None) == 0
    assert L.dflash_set_inject_mxfp4(h, fake, None, fake, fake) == -1
    assert L.dflash_set_inject_mxfp4(h, fake, fake, fake, fake) == -3                  # fp32 drafter
    assert L.dflash_set_inject_mxfp4(h, None, None, None, None) == 0
    assert L.dflash_destroy(h) == 0


def test_status_strings():
    L = B.lib()
    for s in (0, -1, -2, -3, -4, -5):
        assert L.dflash_status_string(s)


def test_quantised_lm_head_row_limit_precedes_any_device_work():
    """MXFP4 (and E4M3) weights run at every row count.  The MXFP4 tiles stage the block scales of
    at most 2048 k per workgroup, so an MXFP4 lm_head over a wider hidden size runs on the skinny
    top-16 kernels, which keep one work counter per 64-row tile, 64 counters in all: a draft of
    more than 4096 rows with it is refused before anything is enqueued (on a handle over
    never-dereferenced fake device addresses the call returns -3 instead of touching the device)."""
    cfg = synth.WORKLOADS["b1_k16"].replace(hidden=2560, name="b1_k16_h2560")
    st, h, keep, kvb, wsb = _fake_handle(cfg, max_seqs=260, max_batch=257, rows=64)
    assert st == 0, B.lib().dflash_last_error()
    L = B.lib()
    fake = 0x5000
    assert L.dflash_set_lm_head_mxfp4(h, fake, fake) == 0
    assert L.dflash_draft_block(h, 257, fake, fake, fake, fake, fake, None, None) == -3     # 4112 rows
    assert b"4096 draft rows" in L.dflash_last_error(), L.dflash_last_error()
    assert L.dflash_set_lm_head_mxfp4(h, None, None) == 0
    assert L.dflash_destroy(h) == 0


def test_mxfp4_setters_check_the_k_widths():
    """The MXFP4 attention and injection setters refuse, before anything is used, k widths that are
    not multiples of 128 (the streaming kernels read MXFP4 codes 128 k at a time): a drafter whose
    concatenated target width is 5 x 5184 = 25920 (a multiple of 64, as bf16 drafters need, but not
    of 128); the same setters succeed at 5 x 5120."""
    L = B.lib()
    fake = 0x5000
    for th, want in ((5184, -3), (5120, 0)):
        cfg = synth.WORKLOADS["b1_k16"].replace(target_hidden=th, name=f"b1_k16_t{th}")
        st, h, keep, kvb, wsb = _fake_handle(cfg)
        assert st == 0, L.dflash_last_error()
        assert L.dflash_set_inject_mxfp4(h, fake, fake, fake, fake) == want, L.dflash_last_error()
        assert L.dflash_set_attn_mxfp4(h, 0, fake, fake, fake, fake) == 0
        assert L.dflash_set_inject_mxfp4(h, None, None, None, None) == 0
        assert L.dflash_set_attn_mxfp4(h, 0, None, None, None, None) == 0
        assert L.dflash_destroy(h) == 0


def test_blocked_weight_entry_points_check_shapes_before_any_device_work():
    """dflash_block_weights refuses, before launching anything, a row count that is not a multiple
    of 16, a column count that is not a multiple of 32, NULL and src == dst.  dflash_set_blocked_weights
    refuses an fp32 drafter and a blocked lm_head whose vocabulary is not a multiple of 16 (leaving the
    handle as it was), takes NULL entries and clears with NULL."""
    L = B.lib()
    src, dst = 0x5000, 0x9000
    assert L.dflash_block_weights(src, 15, 64, dst, None) == -2
    assert L.dflash_block_weights(src, 16, 48, dst, None) == -2
    assert L.dflash_block_weights(src, 0, 64, dst, None) == -2
    assert L.dflash_block_weights(None, 16, 64, dst, None) == -1
    assert L.dflash_block_weights(src, 16, 64, src, None) == -1

    def table(cfg, lm=None, wq=None):
        bw = B.dflash_weights()
        bw.lm_head = lm
        flat = (ctypes.c_void_p * (cfg.n_layers * len(B.LAYER_TENSORS)))()
        if wq is not None:
            for l in range(cfg.n_layers):
                flat[l * len(B.LAYER_TENSORS) + B.LAYER_TENSORS.index("wq")] = wq
        bw.layers = ctypes.cast(flat, ctypes.POINTER(ctypes.c_void_p))
        return bw, flat

    cfg = synth.WORKLOADS["b1_k16"]
    st, h, keep, kvb, wsb = _fake_handle(cfg)
    assert st == 0, L.dflash_last_error()
    bw, flat = table(cfg, lm=0xA000, wq=0xB000)
    assert L.dflash_set_blocked_weights(h, ctypes.byref(bw)) == 0, L.dflash_last_error()
    bw, flat = table(cfg)          # every entry NULL: nothing blocked
    assert L.dflash_set_blocked_weights(h, ctypes.byref(bw)) == 0
    assert L.dflash_set_blocked_weights(h, None) == 0
    assert L.dflash_destroy(h) == 0

    ragged = cfg.replace(vocab=151930, mask_id=151929, name="b1_k16_v151930")
    st, h, keep, kvb, wsb = _fake_handle(ragged)
    assert st == 0, L.dflash_last_error()
    bw, flat = table(ragged, lm=0xA000)
    assert L.dflash_set_blocked_weights(h, ctypes.byref(bw)) == -2
    assert b"16" in L.dflash_last_error()
    bw, flat = table(ragged, wq=0xB000)   # the layer matrices can still be blocked
    assert L.dflash_set_blocked_weights(h, ctypes.byref(bw)) == 0
    assert L.dflash_destroy(h) == 0

    st, h, keep, kvb, wsb = _fake_handle(synth.WORKLOADS["tiny_fp32"])
    assert st == 0, L.dflash_last_error()
    bw, flat = table(synth.WORKLOADS["tiny_fp32"], wq=0xB000)
    assert L.dflash_set_blocked_weights(h, ctypes.byref(bw)) == -3
    assert L.dflash_set_blocked_weights(h, None) == 0
    assert L.dflash_destroy(h) == 0
