"""GPU parity: every libdflash entry point against the CPU oracle on the same seeded inputs.

Small drafters here span several GEMM tiles, ragged contexts, ring wrap-around, restarted
sequences, both GEMM paths (weight-streaming for <= 64 rows, LDS-tiled above) and both
selector modes."""
import numpy as np
import pytest

from block_diffusion_draft_inject_amd import binding as B
from block_diffusion_draft_inject_amd import synth
from oracle import dflash_oracle as O

pytestmark = pytest.mark.gpu

MID = synth.DraftConfig(name="mid_bf16", n_layers=2, hidden=512, n_heads=8, n_kv_heads=2, head_dim=128, ffn=1024,
                        vocab=8192, n_taps=2, target_hidden=512, block_size=16, sel_rank=16, mask_id=8191,
                        dtype="bf16", batch=8, window=64)


@pytest.fixture(scope="module")
def H():
    import parity_harness as H
    return H


def _prefill(case, seq_ids, spans):
    """spans: per sequence (first, L).  Injects in two calls (explicit start, then append)."""
    case.reset(seq_ids)
    first = [np.arange(f, f + (L - f) // 2 + 1) for f, L in spans]
    case.inject(seq_ids, first, start_pos=True)
    rest = [np.arange(f + (L - f) // 2 + 1, L) for f, L in spans]
    case.inject(seq_ids, rest, start_pos=False)


def _full_check(H, case, seq_ids, spans, anchors, mode_names=("viterbi", "greedy")):
    _prefill(case, seq_ids, spans)
    return _check(H, case, seq_ids, anchors, mode_names)


def _check(H, case, seq_ids, anchors, mode_names=("viterbi", "greedy")):
    cfg = case.cfg
    worst, same = H.check_kv(case, seq_ids)
    H.log(f"[kv] {cfg.name}: worst rel err {worst:.2e}, bit-equal {same:.4f}")
    assert worst <= 1.0
    if cfg.dtype == "bf16":
        assert same >= 0.99      # bf16 K/V: almost always the same rounding
    res = case.draft(seq_ids, anchors, logits=True)
    err, _ = H.check_draft(case, seq_ids, anchors, res)
    H.log(f"[draft] {cfg.name}: max |logit err| {err:.2e}")
    assert err <= H.LOGIT_TOL[cfg.dtype]
    for mode_name in mode_names:
        mode = B.SELECT_VITERBI if mode_name == "viterbi" else B.SELECT_GREEDY
        path, score, margin = case.select(anchors, res["_dev"], mode)
        n = H.check_select(case, anchors, res, path, score, margin, mode_name)
        H.log(f"[select] {cfg.name} {mode_name}: {n}/{len(anchors)} above the margin gate")
        match, alt, last = synth.match_draws(cfg.replace(batch=len(anchors)), 0)
        tgt = synth.stand_in_target(path, match, alt, last, cfg.vocab)
        nacc = H.check_verify(case, path.astype(np.int64), tgt)
        H.log(f"[verify] {cfg.name} {mode_name}: accepted {nacc.tolist()}")
    return res


def test_synth_target_matches_rule(H):
    import torch
    K, V, n = 8, 1000, 512
    d = torch.randint(0, V, (n, K - 1), dtype=torch.int32, device="cuda")
    ctr = torch.zeros(1, dtype=torch.int64, device="cuda")
    tgt = torch.empty((n, K), dtype=torch.int32, device="cuda")
    B.dflash_synth_target_argmax(n, K, V, d, 0.7, 123, ctr, tgt)
    torch.cuda.synchronize()
    dn, tn = d.cpu().numpy(), tgt.cpu().numpy()
    match = (tn[:, : K - 1] == dn)
    assert abs(match.mean() - 0.7) < 0.03
    assert tn.min() >= 0 and tn.max() < V
    assert ctr.item() == 1
    B.dflash_synth_target_argmax(n, K, V, d, 0.7, 123, ctr, tgt)
    torch.cuda.synchronize()
    assert ctr.item() == 2 and not np.array_equal(tgt.cpu().numpy(), tn)


def test_tiny_fp32_drafter(H):
    """2 layers, hidden 256, 4x64 heads, vocab 4096, 3x512 taps, context 128, K=8, batch 1."""
    cfg = synth.WORKLOADS["tiny_fp32"]
    case = H.Case(cfg, max_seqs=1, max_batch=1, max_inject_rows=128)
    anchors = synth.anchors(cfg).tolist()
    _full_check(H, case, [0], [(0, 128)], anchors)


def test_tiny_fp32_no_conv_and_empty_context(H):
    cfg = synth.WORKLOADS["tiny_fp32"].replace(use_conv=False)
    case = H.Case(cfg, max_seqs=2, max_batch=2, max_inject_rows=16)
    case.reset([0, 1])
    case.inject([0, 1], [np.arange(0, 5), np.arange(0, 0)], start_pos=True)
    res = case.draft([0, 1], [7, 9], logits=True)
    err, _ = H.check_draft(case, [0, 1], [7, 9], res)
    assert err <= H.LOGIT_TOL["f32"]


def test_device_error_word(H):
    case = H.Case(MID, max_seqs=2, max_batch=2, max_inject_rows=16)
    case.reset([0, 1])
    assert case.d.dflash_get_device_error() == 0
    import torch
    ids = torch.tensor([0, 7], dtype=torch.int32, device="cuda")          # 7 is out of range
    n_new = torch.tensor([2, 2], dtype=torch.int32, device="cuda")
    st = case.states_tensor([None, None], 2)
    case.d.dflash_inject_kv(ids, n_new, 2, st)
    assert case.d.dflash_get_device_error() & 1
    case.reset([0, 1])
    n_new = torch.tensor([5, 1], dtype=torch.int32, device="cuda")        # 5 > max_new
    case.d.dflash_inject_kv(torch.tensor([0, 1], dtype=torch.int32, device="cuda"), n_new, 2, st)
    assert case.d.dflash_get_device_error() & 2
    _, _, sl, _ = case.d.kv_views()
    assert sl[:2].cpu().tolist() == [2, 1]                                # clamped to max_new


def test_mid_bf16_weight_streaming_path(H):
    case = H.Case(MID, max_seqs=8, max_batch=8, max_inject_rows=48)
    seq_ids = [5, 0, 3]
    spans = [(0, 100), (0, 40), (1000, 1070)]     # ring wrap, short context, restarted at 1000
    _full_check(H, case, seq_ids, spans, anchors=[17, 8000, 4095])


def test_mid_bf16_tiled_path_and_ragged_batch(H):
    case = H.Case(MID, max_seqs=8, max_batch=8, max_inject_rows=256)
    seq_ids = list(range(8))
    rng = np.random.default_rng(1)
    Ls = rng.integers(1, 200, size=8)
    Ls[2] = 1      # a single context token
    spans = [(0, int(L)) for L in Ls]
    anchors = rng.integers(0, MID.vocab - 1, size=8).tolist()
    _full_check(H, case, seq_ids, spans, anchors)


def test_mid_bf16_selector_stress(H):
    """A, B ~ N(0,1): the pair term dominates, Viterbi != greedy != per-position argmax."""
    case = H.Case(MID, max_seqs=4, max_batch=4, max_inject_rows=64, selector_stress=True)
    _full_check(H, case, [0, 1, 2, 3], [(0, 70), (0, 20), (0, 64), (5, 90)], anchors=[1, 2, 3, 4])


def test_mid_bf16_single_block_16_rows(H):
    """One sequence at K=16: every draft GEMM has 16 rows (k-split kernels with the activation
    slice held in registers), and injections of at most 16 rows per call, ragged, so the
    injection GEMMs run with a device-side row count."""
    case = H.Case(MID, max_seqs=2, max_batch=1, max_inject_rows=16)
    case.reset([1])
    L = 0
    for n in (16, 5, 1, 16, 9, 16, 16):       # 79 rows: the 64-slot ring wraps
        case.inject([1], [np.arange(L, L + n)], start_pos=(L == 0))
        L += n
    _check(H, case, [1], anchors=[4242])


def test_mid_bf16_two_blocks_k8_ragged_inject(H):
    """K=8, two sequences (16 rows), injected together with ragged row counts per call."""
    cfg = MID.replace(block_size=8, name="mid_bf16_k8")
    case = H.Case(cfg, max_seqs=4, max_batch=2, max_inject_rows=16)
    seq_ids = [3, 1]
    case.reset(seq_ids)
    Ls = [0, 0]
    for n0, n1 in ((7, 1), (1, 8), (8, 0), (3, 5)):
        pos = [np.arange(Ls[0], Ls[0] + n0), np.arange(Ls[1], Ls[1] + n1)]
        case.inject(seq_ids, pos, start_pos=(Ls == [0, 0]))
        Ls = [Ls[0] + n0, Ls[1] + n1]
    _check(H, case, seq_ids, anchors=[12, 8190])


def _same_topk_without_logits(case, seq_ids, anchors, res):
    """The launch without full logits (a separate kernel instantiation) gives the same top-16."""
    plain = case.draft(seq_ids, anchors, logits=False)
    assert np.array_equal(plain["topk_ids"], res["topk_ids"])
    assert np.array_equal(plain["topk_logits"], res["topk_logits"])


def test_mid_bf16_big_tiles_ragged_vocab(H):
    """12 sequences at K=16 (192 rows: the 256 x 256 lm_head tiles, rows past 192 idle) and a
    vocabulary of 8000 (not a multiple of the 128- or 256-column tiles: the last tile reads
    clamped weight rows whose columns the epilogue must skip)."""
    cfg = MID.replace(vocab=8000, mask_id=7999, name="mid_bf16_v8000")
    case = H.Case(cfg, max_seqs=12, max_batch=12, max_inject_rows=160)
    seq_ids = list(range(12))
    rng = np.random.default_rng(3)
    spans = [(0, int(L)) for L in rng.integers(1, 150, size=12)]
    anchors = rng.integers(0, cfg.vocab - 1, size=12).tolist()
    res = _full_check(H, case, seq_ids, spans, anchors, mode_names=("viterbi",))
    _same_topk_without_logits(case, seq_ids, anchors, res)


def test_mid_bf16_lm_head_wave_kernel_without_logits(H):
    """Batch 1, K=16 (the independent-wave lm_head): top-16 with and without full logits."""
    case = H.Case(MID, max_seqs=2, max_batch=1, max_inject_rows=64)
    _prefill(case, [1], [(0, 50)])
    res = _check(H, case, [1], [123], mode_names=("viterbi",))
    _same_topk_without_logits(case, [1], [123], res)


@pytest.mark.parametrize("K,n_seq", [(16, 4), (32, 2)])
def test_mid_bf16_selector_rank_256(H, K, n_seq):
    """Selector rank 256, the width of the A/B token tables on the pages ("Architecture",
    "Problem 1"), with A, B ~ N(0,1) so that the pair term decides the path; K = 32 is the
    largest block the selector takes (with 2 query heads per KV head, so that the grouped
    attention rows of one KV head, 2 x 32, still fit one 64-row tile)."""
    cfg = MID.replace(sel_rank=256, block_size=K, n_kv_heads=8 // (64 // K), name=f"mid_bf16_r256_k{K}")
    case = H.Case(cfg, max_seqs=n_seq, max_batch=n_seq, max_inject_rows=64, selector_stress=True)
    seq_ids = list(range(n_seq))
    spans = [(0, 30 + 17 * i) for i in seq_ids]
    _full_check(H, case, seq_ids, spans, anchors=[11 + 1000 * i for i in seq_ids])


def test_mid_bf16_wide_tiles_192_rows(H):
    """12 sequences at K=16 (192 rows) with 16/4 heads and ffn 1536: the QKV (3072 columns) and
    gate/up (3072) GEMMs take the 256 x 128 tiles with paired k-steps, the 2048-column ones
    the 128 x 128 tiles; ragged contexts with ring wrap."""
    cfg = MID.replace(n_heads=16, n_kv_heads=4, ffn=1536, name="mid_bf16_wide")
    case = H.Case(cfg, max_seqs=12, max_batch=12, max_inject_rows=200)
    seq_ids = list(range(12))
    rng = np.random.default_rng(5)
    spans = [(0, int(L)) for L in rng.integers(1, 160, size=12)]
    anchors = rng.integers(0, cfg.vocab - 1, size=12).tolist()
    _full_check(H, case, seq_ids, spans, anchors, mode_names=("viterbi",))


@pytest.mark.parametrize("K", [2, 16, 64, 65, 130])
def test_verify_greedy_block_sizes(K):
    """Greedy verification alone (one wave per sequence, 64-slot chunks): 37 sequences (a
    partial last workgroup) with accepted prefixes of every length from 0 to K-1 (full
    acceptance included), against the oracle's longest-prefix rule; then an empty batch."""
    import torch
    rng = np.random.default_rng(K)
    n_seq, V = 37, 5000
    draft = rng.integers(0, V, size=(n_seq, K - 1))
    target = rng.integers(0, V, size=(n_seq, K))
    for b in range(n_seq):
        n = min(b * (K - 1) // (n_seq - 1), K - 1) if b < n_seq - 1 else K - 1
        target[b, :n] = draft[b, :n]
        if n < K - 1:
            target[b, n] = (draft[b, n] + 1 + rng.integers(0, V - 1)) % V   # a different token
    dev = lambda x: torch.tensor(x, dtype=torch.int32, device="cuda")
    d, t = dev(draft), dev(target)
    nacc = torch.empty(n_seq, dtype=torch.int32, device="cuda")
    ncom = torch.empty_like(nacc)
    nxt = torch.empty_like(nacc)
    com = torch.empty((n_seq, K), dtype=torch.int32, device="cuda")
    B.dflash_verify_greedy(n_seq, K, d, t, nacc, ncom, com, nxt)
    torch.cuda.synchronize()
    seen = set()
    for b in range(n_seq):
        n, c, a = O.verify_greedy(draft[b], target[b])
        seen.add(n)
        assert nacc[b].item() == n and ncom[b].item() == n + 1 and nxt[b].item() == a, b
        assert np.array_equal(com[b].cpu().numpy(), c), b
    assert 0 in seen and K - 1 in seen
    B.dflash_verify_greedy(0, K, d, t, nacc, ncom, com, nxt)   # empty batch: a no-op
    torch.cuda.synchronize()


def test_two_handles_share_kv_on_two_streams(H):
    """A second handle on the same KV cache (its own workspace) injects a new sequence's whole
    window on a second stream while the first handle injects accepted rows and drafts for two
    running sequences on its stream.  Outputs and the whole KV region equal those of the same
    calls run one after the other on one stream; the new sequence's K/V match the oracle."""
    import torch
    cfg = MID
    case = H.Case(cfg, max_seqs=4, max_batch=2, max_inject_rows=64)
    dB = B.Drafter(cfg, case.dev_w, max_seqs=4, max_batch=1, max_inject_rows=64, kv_from=case.d)
    case.reset([0, 1, 2])
    case.inject([0, 1], [np.arange(0, 50), np.arange(0, 30)])
    pos2 = np.arange(100, 100 + cfg.window)
    st2 = synth.target_states(cfg, 2, pos2)
    states2 = case.states_tensor([st2], len(pos2))
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    pool = torch.randn((2, 5, cfg.concat_width), generator=g, device="cuda").to(torch.bfloat16)
    ids01, nnew01 = case.tensor(np.array([0, 1], np.int32)), case.tensor(np.array([3, 5], np.int32))
    id2, nnew2 = case.tensor(np.array([2], np.int32)), case.tensor(np.array([len(pos2)], np.int32))
    sp2 = case.tensor(np.array([pos2[0]], np.int32))
    anchors = case.tensor(np.array([77, 4000], np.int32))
    torch.cuda.synchronize()
    snapshot = case.d.kv.clone()

    def run(two_streams):
        case.d.kv.copy_(snapshot)
        out = case.d.outputs(2, logits=True)
        torch.cuda.synchronize()
        sa = torch.cuda.Stream()
        sb = torch.cuda.Stream() if two_streams else sa
        dB.dflash_inject_kv(id2, nnew2, len(pos2), states2, start_pos=sp2, stream=sb.cuda_stream)
        case.d.dflash_inject_kv(ids01, nnew01, 5, pool, start_pos=None, stream=sa.cuda_stream)
        case.d.dflash_draft_block(ids01, anchors, out["topk_ids"], out["topk_logits"], out["h_final"],
                                  out["logits"], stream=sa.cuda_stream)
        torch.cuda.synchronize()
        return {k: v.clone() for k, v in out.items() if v is not None}, case.d.kv.clone()

    seq_out, seq_kv = run(False)
    par_out, par_kv = run(True)
    for k in seq_out:
        assert torch.equal(seq_out[k], par_out[k]), k
    assert torch.equal(seq_kv, par_kv)
    O.inject(cfg, case.W64, case.caches[2], pos2, st2.values, H.oracle_mode(cfg))
    worst, same = H.check_kv(case, [2])
    H.log(f"[two handles] new sequence K/V: worst rel err {worst:.2e}, bit-equal {same:.4f}")
    assert worst <= 1.0 and same >= 0.99
    # the two-stream drafts against the oracle: the running sequences took pool rows 0..2 (seq 0,
    # positions 50..52) and 0..4 (seq 1, positions 30..34) before drafting
    pool64 = pool.float().cpu().numpy().astype(np.float64)
    for i, (s, L0, n) in enumerate(((0, 50, 3), (1, 30, 5))):
        O.inject(cfg, case.W64, case.caches[s], np.arange(L0, L0 + n), pool64[i, :n], H.oracle_mode(cfg))
    worst, same = H.check_kv(case, [0, 1])
    assert worst <= 1.0 and same >= 0.99
    res = {k: v.cpu().numpy() for k, v in par_out.items()}
    err, _ = H.check_draft(case, [0, 1], [77, 4000], res)
    H.log(f"[two handles] two-stream drafts vs oracle: max |logit err| {err:.2e}")
    assert err <= H.LOGIT_TOL["bf16"]
    assert case.d.dflash_get_device_error() == 0


def test_mid_bf16_empty_context_mfma_attention(H):
    """Fresh sequences with no injected context (L = 0: the block attends to itself only, so every
    split-KV chunk past the first is empty) beside sequences with 1 and 63 context positions, on
    the MFMA attention of bf16 drafters, batch 1 (16 rows) and batch 3 (48 rows)."""
    case = H.Case(MID, max_seqs=4, max_batch=3, max_inject_rows=64)
    case.reset([0, 1, 2])
    case.inject([1, 2], [np.arange(0, 1), np.arange(0, 63)])
    res = case.draft([0], [5], logits=True)
    err, _ = H.check_draft(case, [0], [5], res)
    assert err <= H.LOGIT_TOL["bf16"]
    res = case.draft([1, 0, 2], [9, 4000, 123], logits=True)
    err, _ = H.check_draft(case, [1, 0, 2], [9, 4000, 123], res)
    H.log(f"[empty context] max |logit err| {err:.2e}")
    assert err <= H.LOGIT_TOL["bf16"]
    assert case.d.dflash_get_device_error() == 0


def _quantize_on_gpu(lm):
    import torch
    codes = torch.empty(lm.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty(lm.shape[0], dtype=torch.float32, device="cuda")
    B.dflash_quantize_fp8_rows(lm, codes, scales)
    torch.cuda.synchronize()
    return codes, scales


def test_fp8_quantizer_matches_oracle():
    """E4M3 codes and row scales, bit-exact against the oracle: ordinary rows, an all-zero row,
    a row of -0, a row below the zero-row threshold, a row of large values, a row of exact ties
    (midpoints between codes), a row with subnormal codes, alternating signs."""
    import torch
    rng = np.random.default_rng(21)
    W = rng.normal(0, 0.02, (300, 512))
    W[0] = 0.0
    W[1] = -0.0
    W[2] *= 1e-20
    W[3] *= 1e6
    vals = O.e4m3_value(np.arange(0, 0x7E, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    W[4] = np.resize(mids, 512) * 2.0 ** -10
    W[4, 0] = 448 * 2.0 ** -10                     # the row's scale is 2^-10, the midpoints stay ties
    W[5] = rng.normal(0, 1e-6, 512)
    W[5, 7] = 0.4                                  # everything else lands on subnormal codes
    W[6, ::2] = -W[6, ::2]
    Wb = O.bf16_round(W)
    dev = torch.tensor(Wb, dtype=torch.float32).to(torch.bfloat16).cuda()
    codes, scales = _quantize_on_gpu(dev)
    oc, osc = O.quantize_fp8_rows(Wb)
    assert np.array_equal(scales.cpu().numpy(), osc.astype(np.float32))
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.all(oc[0] == 0) and np.all(oc[1] == 0x80)


def test_mid_bf16_fp8_lm_head(H):
    """K=16 with the FP8 lm_head: codes as the oracle's, logits and top-16 against the oracle run
    with the dequantised lm_head, top-16 with and without full logits, at batch 1 (the
    independent-wave kernel) and batch 2 (32 rows: the skinny kernel); NULL codes restore the
    bf16 lm_head."""
    import torch
    case = H.Case(MID, max_seqs=2, max_batch=2, max_inject_rows=64)
    _prefill(case, [1, 0], [(0, 50), (0, 37)])
    codes, scales = _quantize_on_gpu(case.dev_w["lm_head"])
    oc, osc = O.quantize_fp8_rows(case.W64["lm_head"])
    assert np.array_equal(codes.cpu().numpy(), oc) and np.array_equal(scales.cpu().numpy(), osc.astype(np.float32))
    case.d.dflash_set_lm_head_fp8(codes, scales)
    bf16_lm = case.W64["lm_head"]
    case.W64["lm_head"] = O.dequantize_fp8_rows(oc, osc)
    try:
        res = _check(H, case, [1], [123], mode_names=("viterbi",))
        _same_topk_without_logits(case, [1], [123], res)
        res = _check(H, case, [1, 0], [123, 5], mode_names=("viterbi",))   # 32 rows
        _same_topk_without_logits(case, [1, 0], [123, 5], res)
    finally:
        case.W64["lm_head"] = bf16_lm
    case.d.dflash_set_lm_head_fp8(None, None)
    res = case.draft([1], [123], logits=True)
    err, _ = H.check_draft(case, [1], [123], res)
    assert err <= H.LOGIT_TOL["bf16"]


def _quantize_mxfp4_on_gpu(lm):
    import torch
    rows, cols = lm.shape
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")
    B.dflash_quantize_mxfp4_rows(lm, codes, scales)
    torch.cuda.synchronize()
    return codes, scales


def test_mxfp4_quantizer_matches_oracle():
    """MXFP4 codes and block scale bytes, bit-exact against the oracle: ordinary rows, rows spanning
    many binades, an all-zero row, a row of -0, a row below the zero-block threshold, a row of exact
    midpoints between E2M1 magnitudes (ties), a row of values that saturate, alternating signs."""
    import torch
    rng = np.random.default_rng(22)
    W = rng.normal(0, 0.02, (200, 512))
    W[:20] *= np.exp(rng.normal(0, 3, (20, 1)))
    W[20] = 0.0
    W[21] = -0.0
    W[22] *= 1e-22
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    W[23] = np.resize(np.concatenate([mids, -mids]), 512) * 2.0 ** -9
    W[23, ::32] = 4.0 * 2.0 ** -9                 # every block's exponent is -9: the midpoints stay ties
    W[24] = np.resize([7.9, 6.5, -7.0, 6.0], 512) * 2.0 ** -4
    W[25, ::2] = -W[25, ::2]
    Wb = O.bf16_round(W)
    dev = torch.tensor(Wb, dtype=torch.float32).to(torch.bfloat16).cuda()
    codes, scales = _quantize_mxfp4_on_gpu(dev)
    oc, osc = O.quantize_mxfp4_rows(Wb)
    assert np.array_equal(scales.cpu().numpy(), osc)
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.all(oc[20] == 0) and np.all(oc[21] == 0x88)


def test_mid_bf16_mxfp4_lm_head(H):
    """Batch 1, K=16 with the MXFP4 lm_head (the independent-wave kernel): codes as the oracle's,
    logits and top-16 against the oracle run with the dequantised lm_head, top-16 with and without
    full logits; NULL restores the bf16 lm_head.  (More rows: test_mxfp4_above_16_rows.)"""
    case = H.Case(MID, max_seqs=2, max_batch=2, max_inject_rows=64)
    _prefill(case, [1], [(0, 50)])
    codes, scales = _quantize_mxfp4_on_gpu(case.dev_w["lm_head"])
    oc, osc = O.quantize_mxfp4_rows(case.W64["lm_head"])
    assert np.array_equal(codes.cpu().numpy(), oc) and np.array_equal(scales.cpu().numpy(), osc)
    case.d.dflash_set_lm_head_mxfp4(codes, scales)
    bf16_lm = case.W64["lm_head"]
    case.W64["lm_head"] = O.dequantize_mxfp4_rows(oc, osc)
    try:
        res = _check(H, case, [1], [123], mode_names=("viterbi",))
        _same_topk_without_logits(case, [1], [123], res)
    finally:
        case.W64["lm_head"] = bf16_lm
    case.d.dflash_set_lm_head_mxfp4(None, None)
    res = case.draft([1], [123], logits=True)
    err, _ = H.check_draft(case, [1], [123], res)
    assert err <= H.LOGIT_TOL["bf16"]


def _fp8_stacked(case, W, mats, names_rows):
    """GPU codes of the row-stacked device matrices `mats`; each (layer or None, name, rows) block
    checked against the oracle's codes of that matrix and replaced in W by its dequantised form."""
    import torch
    codes, scales = _quantize_on_gpu(torch.cat(mats).contiguous() if len(mats) > 1 else mats[0])
    for layer, name, rows in names_rows:
        src = case.W64["layers"][layer][name] if layer is not None else case.W64[name]
        oc, osc = O.quantize_fp8_rows(src)
        assert np.array_equal(codes[rows].cpu().numpy(), oc), (layer, name)
        assert np.array_equal(scales[rows].cpu().numpy(), osc.astype(np.float32)), (layer, name)
        if layer is not None:
            W["layers"][layer][name] = O.dequantize_fp8_rows(oc, osc)
        else:
            W[name] = O.dequantize_fp8_rows(oc, osc)
    return codes, scales


def _fp8_drafter(case, mlp=True, lm_head=True, attn=False, inject=False):
    """Quantises the MLP matrices of every layer (stacked [gate; up], down), optionally the
    attention projections (stacked [wq; wk; wv], wo) and the injection matrices (fc, the stacked
    per-layer [wk; wv]), and the lm_head on the GPU, checks the codes against the oracle's,
    installs them, and returns float64 weights for the oracle with those matrices dequantised."""
    import copy
    import torch
    cfg = case.cfg
    W = copy.copy(case.W64)
    W["layers"] = [dict(lw) for lw in case.W64["layers"]]
    keep = []
    qw, kvw = cfg.q_width, cfg.kv_width
    if attn:
        for l, lw in enumerate(case.dev_w["layers"]):
            q8 = _fp8_stacked(case, W, [lw["wq"], lw["wk"], lw["wv"]],
                              [(l, "wq", slice(0, qw)), (l, "wk", slice(qw, qw + kvw)), (l, "wv", slice(qw + kvw, None))])
            o8 = _fp8_stacked(case, W, [lw["wo"]], [(l, "wo", slice(None))])
            case.d.dflash_set_attn_fp8(l, *q8, *o8)
    if inject:
        fc8 = _fp8_stacked(case, W, [case.dev_w["fc"]], [(None, "fc", slice(None))])
        mats, blocks = [], []
        for l, lw in enumerate(case.dev_w["layers"]):
            mats += [lw["wk"], lw["wv"]]
            blocks += [(l, "wk", slice(2 * l * kvw, (2 * l + 1) * kvw)), (l, "wv", slice((2 * l + 1) * kvw, (2 * l + 2) * kvw))]
        kv8 = _fp8_stacked(case, W, mats, blocks)
        case.d.dflash_set_inject_fp8(*fc8, *kv8)
    if mlp:
        for l, lw in enumerate(case.dev_w["layers"]):
            gu, gus = _quantize_on_gpu(torch.cat([lw["w_gate"], lw["w_up"]]).contiguous())
            dn, dns = _quantize_on_gpu(lw["w_down"])
            for name, codes, scales, rows in (("w_gate", gu, gus, slice(0, case.cfg.ffn)),
                                              ("w_up", gu, gus, slice(case.cfg.ffn, 2 * case.cfg.ffn)),
                                              ("w_down", dn, dns, slice(None))):
                oc, osc = O.quantize_fp8_rows(case.W64["layers"][l][name])
                assert np.array_equal(codes[rows].cpu().numpy(), oc), (l, name)
                assert np.array_equal(scales[rows].cpu().numpy(), osc.astype(np.float32)), (l, name)
                W["layers"][l][name] = O.dequantize_fp8_rows(oc, osc)
            case.d.dflash_set_mlp_fp8(l, gu, gus, dn, dns)
            keep += [gu, gus, dn, dns]
    if lm_head:
        codes, scales = _quantize_on_gpu(case.dev_w["lm_head"])
        oc, osc = O.quantize_fp8_rows(case.W64["lm_head"])
        assert np.array_equal(codes.cpu().numpy(), oc)
        case.d.dflash_set_lm_head_fp8(codes, scales)
        W["lm_head"] = O.dequantize_fp8_rows(oc, osc)
    return W


def test_mid_bf16_fp8_mlp_and_lm_head(H):
    """K=16 with FP8 MLP weights in both layers and the FP8 lm_head, against the oracle run with
    those matrices dequantised: batch 1 (stacked gate/up through the SwiGLU streaming kernel, down
    through the k-split one) and batch 2 (the skinny SwiGLU and k-split kernels); NULL restores
    bf16."""
    case = H.Case(MID, max_seqs=2, max_batch=2, max_inject_rows=64)
    _prefill(case, [1, 0], [(0, 50), (0, 61)])
    W8 = _fp8_drafter(case)
    W64 = case.W64
    case.W64 = W8
    try:
        res = _check(H, case, [1], [321], mode_names=("viterbi",))
        _same_topk_without_logits(case, [1], [321], res)
        _check(H, case, [1, 0], [321, 5], mode_names=("viterbi",))
    finally:
        case.W64 = W64
    for l in range(MID.n_layers):
        case.d.dflash_set_mlp_fp8(l, None, None, None, None)
    case.d.dflash_set_lm_head_fp8(None, None)
    res = case.draft([1], [321], logits=True)
    err, _ = H.check_draft(case, [1], [321], res)
    assert err <= H.LOGIT_TOL["bf16"]


def test_mid_bf16_fp8_every_gemm(H):
    """FP8 codes for every weight GEMM of a batch-1 cycle: injection (fc, stacked K/V), attention
    projections (stacked QKV, O), MLP and lm_head.  A prefill injected with the bf16 weights, then
    an injection of 5 rows with the FP8 ones (the streaming kernels), a draft, and an injection of
    20 rows (the skinny kernels), each against the oracle run with the same matrices (dequantised
    where FP8)."""
    case = H.Case(MID, max_seqs=2, max_batch=2, max_inject_rows=64)
    _prefill(case, [1], [(0, 50)])
    W64 = case.W64
    case.W64 = _fp8_drafter(case, mlp=True, lm_head=True, attn=True, inject=True)
    try:
        case.inject([1], [np.arange(50, 55)], start_pos=False)
        res = _check(H, case, [1], [77], mode_names=("viterbi",))
        _same_topk_without_logits(case, [1], [77], res)
        case.inject([1], [np.arange(55, 75)], start_pos=False)
        _check(H, case, [1], [78], mode_names=("viterbi",))
    finally:
        case.W64 = W64


@pytest.mark.parametrize("wide,n_seq", [(False, 5), (True, 10)], ids=["80_rows", "160_rows_wide_mlp"])
def test_fp8_every_gemm_tiles(H, wide, n_seq):
    """E4M3 codes for every weight GEMM at more than 64 rows (the LDS-DMA tile kernels, codes
    staged 16 rows x 64 k per 1 KiB block): 5 sequences at K=16 (80 rows: 128 x 128 layer tiles,
    the 128 x 128 lm_head tile) and 10 at hidden 1024 / ffn 4608 (160 rows: the 256 x 128 tile for
    gate/up, the 256 x 256 lm_head tile).  Ragged contexts injected with the bf16 weights, then one
    injection of up to 12 rows per sequence with the FP8 ones (tile kernels again), then a draft,
    against the oracle run with the same matrices (dequantised where FP8)."""
    cfg = MID_WIDE_MLP if wide else MID
    case = H.Case(cfg, max_seqs=n_seq, max_batch=n_seq, max_inject_rows=128)
    seq_ids = list(range(n_seq))
    rng = np.random.default_rng(40 + n_seq)
    lens = [int(L) for L in rng.integers(20, 90, size=n_seq)]
    _prefill(case, seq_ids, [(0, L) for L in lens])
    W64 = case.W64
    case.W64 = _fp8_drafter(case, mlp=True, lm_head=True, attn=True, inject=True)
    try:
        adds = [np.arange(L, L + int(a)) for L, a in zip(lens, rng.integers(1, 13, size=n_seq))]
        case.inject(seq_ids, adds, start_pos=False)
        anchors = rng.integers(0, cfg.vocab - 1, size=n_seq).tolist()
        res = _check(H, case, seq_ids, anchors, mode_names=("viterbi",))
        _same_topk_without_logits(case, seq_ids, anchors, res)
    finally:
        case.W64 = W64


# hidden 1024: the gate/up slices are two 64-k chunks (one 128-k MXFP4 super-chunk); ffn 4608:
# the down projection takes 5 k-splits of 1024, the last half past the end of K
MID_WIDE_MLP = synth.DraftConfig(name="mid_bf16_wide_mlp", n_layers=2, hidden=1024, n_heads=8, n_kv_heads=2,
                                 head_dim=128, ffn=4608, vocab=8192, n_taps=2, target_hidden=512, block_size=16,
                                 sel_rank=16, mask_id=8191, dtype="bf16", batch=8, window=64)


@pytest.mark.parametrize("cfg", [MID, MID_WIDE_MLP], ids=["one_chunk_slices", "super_chunks"])
def test_mid_bf16_mxfp4_mlp(H, cfg):
    """Batch 1, K=16 with MXFP4 MLP weights in both layers (stacked gate/up through the SwiGLU
    streaming kernel, down through the k-split one), with one-chunk slices (hidden 512, ffn 1024)
    and with 128-k super-chunks (hidden 1024, ffn 4608): codes and block scales as the oracle's,
    then a draft against the oracle run with those matrices dequantised; FP8 MLP weights set
    afterwards replace them; NULL restores bf16.  (More rows: test_mxfp4_above_16_rows.)"""
    import copy
    import torch
    case = H.Case(cfg, max_seqs=2, max_batch=2, max_inject_rows=64)
    _prefill(case, [1], [(0, 50)])
    W4 = copy.copy(case.W64)
    W4["layers"] = [dict(lw) for lw in case.W64["layers"]]
    keep = []
    for l, lw in enumerate(case.dev_w["layers"]):
        gu, gus = _quantize_mxfp4_on_gpu(torch.cat([lw["w_gate"], lw["w_up"]]).contiguous())
        dn, dns = _quantize_mxfp4_on_gpu(lw["w_down"])
        for name, codes, scales, rows in (("w_gate", gu, gus, slice(0, cfg.ffn)),
                                          ("w_up", gu, gus, slice(cfg.ffn, 2 * cfg.ffn)),
                                          ("w_down", dn, dns, slice(None))):
            oc, osc = O.quantize_mxfp4_rows(case.W64["layers"][l][name])
            assert np.array_equal(codes[rows].cpu().numpy(), oc), (l, name)
            assert np.array_equal(scales[rows].cpu().numpy(), osc), (l, name)
            W4["layers"][l][name] = O.dequantize_mxfp4_rows(oc, osc)
        case.d.dflash_set_mlp_mxfp4(l, gu, gus, dn, dns)
        keep += [gu, gus, dn, dns]
    W64 = case.W64
    case.W64 = W4
    try:
        res = _check(H, case, [1], [222], mode_names=("viterbi",))
        _same_topk_without_logits(case, [1], [222], res)
    finally:
        case.W64 = W64
    W8 = _fp8_drafter(case, mlp=True, lm_head=False)   # replaces the MXFP4 MLP weights
    case.W64 = W8
    try:
        _check(H, case, [1], [222], mode_names=("viterbi",))
    finally:
        case.W64 = W64
    for l in range(cfg.n_layers):
        case.d.dflash_set_mlp_mxfp4(l, None, None, None, None)
    res = case.draft([1], [222], logits=True)
    err, _ = H.check_draft(case, [1], [222], res)
    assert err <= H.LOGIT_TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_per_channel_conv(H, dtype):
    """The pages' per-channel two-tap conv (one correction per 16 channels): the fp32 tiny drafter
    (16 groups), and the mid bf16 drafter (32 groups) at batch 1 (16 rows: the streaming GEMMs for
    the corrections) and batch 12 (192 rows: the tile GEMMs), against the oracle."""
    if dtype == "f32":
        cfg = synth.WORKLOADS["tiny_fp32"].replace(conv_group=16, name="tiny_fp32_pc16")
        case = H.Case(cfg, max_seqs=1, max_batch=1, max_inject_rows=128)
        _full_check(H, case, [0], [(0, 128)], synth.anchors(cfg).tolist())
        return
    cfg = MID.replace(conv_group=16, name="mid_bf16_pc16")
    case = H.Case(cfg, max_seqs=12, max_batch=12, max_inject_rows=256)
    _full_check(H, case, [3], [(0, 50)], anchors=[77])
    rng = np.random.default_rng(9)
    seq_ids = list(range(12))
    spans = [(0, int(L)) for L in rng.integers(1, 120, size=12)]
    _full_check(H, case, seq_ids, spans, rng.integers(0, cfg.vocab - 1, size=12).tolist(), mode_names=("viterbi",))


def test_two_batch_pipeline_two_streams(H):
    """The two-batch pipeline: four sequences split into two halves, each half's whole cycle
    (inject its committed tokens -> draft -> select -> stand-in target -> verify, tau and the next
    anchor kept on the device) on its own handle (shared weights and KV cache) and stream, for two
    cycles.  Every output and the KV region equal those of the same calls on one stream, and both
    cycles' drafts of all four sequences match the oracle (fed the tau and anchors the GPU chose)."""
    import torch
    cfg = MID
    K = cfg.block_size
    case = H.Case(cfg, max_seqs=4, max_batch=4, max_inject_rows=64)
    halves = [(B.Drafter(cfg, case.dev_w, max_seqs=4, max_batch=2, max_inject_rows=64, kv_from=case.d), [0, 1]),
              (B.Drafter(cfg, case.dev_w, max_seqs=4, max_batch=2, max_inject_rows=64, kv_from=case.d), [2, 3])]
    case.reset([0, 1, 2, 3])
    case.inject([0, 1, 2, 3], [np.arange(0, 30 + 7 * i) for i in range(4)])
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    pool = torch.randn((4, K, cfg.concat_width), generator=g, device="cuda").to(torch.bfloat16)
    pools = [pool[:2].contiguous(), pool[2:].contiguous()]
    anchors0 = [[17, 4000], [123, 8000]]
    torch.cuda.synchronize()
    snapshot = case.d.kv.clone()

    def run(two_streams):
        case.d.kv.copy_(snapshot)
        st = [torch.cuda.Stream(), None]
        st[1] = torch.cuda.Stream() if two_streams else st[0]
        state = []
        for hidx, (d, ids) in enumerate(halves):
            t = lambda x, dt=torch.int32: torch.tensor(x, dtype=dt, device="cuda")
            state.append(dict(ids=t(ids), anchor=t(anchors0[hidx]), tau=t([0, 0]), out=None,
                              path=torch.empty((2, K - 1), dtype=torch.int32, device="cuda"),
                              score=torch.empty(2, device="cuda"), margin=torch.empty(2, device="cuda"),
                              target=torch.empty((2, K), dtype=torch.int32, device="cuda"),
                              nacc=t([0, 0]), com=torch.empty((2, K), dtype=torch.int32, device="cuda"),
                              ctr=torch.zeros(1, dtype=torch.int64, device="cuda")))
        records = []
        torch.cuda.synchronize()
        for step in range(2):
            rec = []
            for hidx, (d, ids) in enumerate(halves):
                s, x = st[hidx].cuda_stream, state[hidx]
                x["out"] = d.outputs(2, logits=True)
                anchor_in = x["anchor"].clone()
                d.dflash_inject_kv(x["ids"], x["tau"], K, pools[hidx], start_pos=None, stream=s)
                o = x["out"]
                d.dflash_draft_block(x["ids"], anchor_in, o["topk_ids"], o["topk_logits"], o["h_final"], o["logits"],
                                     stream=s)
                d.dflash_select_path(anchor_in, o["topk_ids"], o["topk_logits"], o["h_final"], B.SELECT_VITERBI,
                                     x["path"], x["score"], x["margin"], stream=s)
                B.dflash_synth_target_argmax(2, K, cfg.vocab, x["path"], 0.7, 99 + hidx, x["ctr"], x["target"],
                                             stream=s)
                B.dflash_verify_greedy(2, K, x["path"], x["target"], x["nacc"], x["tau"], x["com"], x["anchor"],
                                       stream=s)
                rec.append((anchor_in, x))
            torch.cuda.synchronize()
            records.append([dict(anchor=a.cpu().numpy(), tau=x["tau"].cpu().numpy(), path=x["path"].cpu().numpy(),
                                 **{k: v.cpu().numpy() for k, v in x["out"].items()}) for a, x in rec])
        return records, case.d.kv.clone()

    seq_rec, seq_kv = run(False)
    par_rec, par_kv = run(True)
    assert torch.equal(seq_kv, par_kv)
    for a, b in zip(seq_rec, par_rec):
        for ha, hb in zip(a, b):
            for k in ha:
                assert np.array_equal(ha[k], hb[k]), k
    # the oracle, teacher-forced with the GPU's tau and anchors
    pool64 = pool.float().cpu().numpy().astype(np.float64)
    for step, rec in enumerate(par_rec):
        if step == 1:
            for hidx, (_, ids) in enumerate(halves):
                tau0 = par_rec[0][hidx]["tau"]
                for i, sid in enumerate(ids):
                    L0 = case.caches[sid].length
                    O.inject(cfg, case.W64, case.caches[sid], np.arange(L0, L0 + int(tau0[i])),
                             pool64[sid, : int(tau0[i])], H.oracle_mode(cfg))
        for hidx, (_, ids) in enumerate(halves):
            r = rec[hidx]
            err, _ = H.check_draft(case, ids, r["anchor"].tolist(), r)
            assert err <= H.LOGIT_TOL["bf16"]
            H.log(f"[pipeline] step {step} half {hidx}: max |logit err| {err:.2e}, tau {r['tau'].tolist()}")
    assert case.d.dflash_get_device_error() == 0


def _mxfp4_stacked(case, W, mats, names_rows):
    """GPU MXFP4 codes and block scales of the row-stacked device matrices `mats`; each (layer or
    None, name, rows) block checked against the oracle's of that matrix and replaced in W by its
    dequantised form."""
    import torch
    codes, scales = _quantize_mxfp4_on_gpu(torch.cat(mats).contiguous() if len(mats) > 1 else mats[0])
    for layer, name, rows in names_rows:
        src = case.W64["layers"][layer][name] if layer is not None else case.W64[name]
        oc, osc = O.quantize_mxfp4_rows(src)
        assert np.array_equal(codes[rows].cpu().numpy(), oc), (layer, name)
        assert np.array_equal(scales[rows].cpu().numpy(), osc), (layer, name)
        if layer is not None:
            W["layers"][layer][name] = O.dequantize_mxfp4_rows(oc, osc)
        else:
            W[name] = O.dequantize_mxfp4_rows(oc, osc)
    return codes, scales


def _mxfp4_drafter(case, mlp=True, lm_head=True, attn=False, inject=False):
    """Quantises the MLP matrices of every layer (stacked [gate; up], down), the lm_head, and
    optionally the attention projections (stacked [wq; wk; wv], wo) and the injection matrices (fc,
    the stacked per-layer [wk; wv]) to MXFP4 on the GPU, checks codes and block scales against the
    oracle's, installs them, and returns float64 weights for the oracle with those matrices
    dequantised."""
    import copy
    import torch
    cfg = case.cfg
    W = copy.copy(case.W64)
    W["layers"] = [dict(lw) for lw in case.W64["layers"]]
    qw, kvw = cfg.q_width, cfg.kv_width
    if attn:
        for l, lw in enumerate(case.dev_w["layers"]):
            q4 = _mxfp4_stacked(case, W, [lw["wq"], lw["wk"], lw["wv"]],
                                [(l, "wq", slice(0, qw)), (l, "wk", slice(qw, qw + kvw)), (l, "wv", slice(qw + kvw, None))])
            o4 = _mxfp4_stacked(case, W, [lw["wo"]], [(l, "wo", slice(None))])
            case.d.dflash_set_attn_mxfp4(l, *q4, *o4)
    if inject:
        fc4 = _mxfp4_stacked(case, W, [case.dev_w["fc"]], [(None, "fc", slice(None))])
        mats, blocks = [], []
        for l, lw in enumerate(case.dev_w["layers"]):
            mats += [lw["wk"], lw["wv"]]
            blocks += [(l, "wk", slice(2 * l * kvw, (2 * l + 1) * kvw)), (l, "wv", slice((2 * l + 1) * kvw, (2 * l + 2) * kvw))]
        kv4 = _mxfp4_stacked(case, W, mats, blocks)
        case.d.dflash_set_inject_mxfp4(*fc4, *kv4)
    if mlp:
        for l, lw in enumerate(case.dev_w["layers"]):
            gu, gus = _quantize_mxfp4_on_gpu(torch.cat([lw["w_gate"], lw["w_up"]]).contiguous())
            dn, dns = _quantize_mxfp4_on_gpu(lw["w_down"])
            for name, codes, scales, rows in (("w_gate", gu, gus, slice(0, cfg.ffn)),
                                              ("w_up", gu, gus, slice(cfg.ffn, 2 * cfg.ffn)),
                                              ("w_down", dn, dns, slice(None))):
                oc, osc = O.quantize_mxfp4_rows(case.W64["layers"][l][name])
                assert np.array_equal(codes[rows].cpu().numpy(), oc), (l, name)
                assert np.array_equal(scales[rows].cpu().numpy(), osc), (l, name)
                W["layers"][l][name] = O.dequantize_mxfp4_rows(oc, osc)
            case.d.dflash_set_mlp_mxfp4(l, gu, gus, dn, dns)
    if lm_head:
        codes, scales = _quantize_mxfp4_on_gpu(case.dev_w["lm_head"])
        oc, osc = O.quantize_mxfp4_rows(case.W64["lm_head"])
        assert np.array_equal(codes.cpu().numpy(), oc) and np.array_equal(scales.cpu().numpy(), osc)
        case.d.dflash_set_lm_head_mxfp4(codes, scales)
        W["lm_head"] = O.dequantize_mxfp4_rows(oc, osc)
    return W


@pytest.mark.parametrize("wide,n_seq", [(False, 2), (False, 5), (True, 10)],
                         ids=["32_rows", "80_rows", "160_rows_wide"])
def test_mxfp4_above_16_rows(H, wide, n_seq):
    """MXFP4 lm_head and MLP weights above 16 draft rows: 2 sequences at K=16 (32 rows: the skinny
    kernels, codes streamed into registers), 5 (80 rows: the 128 x 128 LDS tiles, codes staged 32
    rows x 64 k per 1 KiB block, block scales in LDS) and 10 at hidden 1024 / ffn 4608 (160 rows:
    the 256 x 128 tile for gate/up, whose four code blocks come from waves 0-3, and the 256 x 256
    lm_head tile).  Ragged contexts, then a draft against the oracle run with the dequantised
    matrices, top-16 with and without full logits; NULL restores bf16."""
    cfg = MID_WIDE_MLP if wide else MID
    case = H.Case(cfg, max_seqs=n_seq, max_batch=n_seq, max_inject_rows=128)
    seq_ids = list(range(n_seq))
    rng = np.random.default_rng(70 + n_seq)
    lens = [int(L) for L in rng.integers(20, 90, size=n_seq)]
    _prefill(case, seq_ids, [(0, L) for L in lens])
    W64 = case.W64
    case.W64 = _mxfp4_drafter(case)
    anchors = rng.integers(0, cfg.vocab - 1, size=n_seq).tolist()
    try:
        res = _check(H, case, seq_ids, anchors, mode_names=("viterbi",))
        _same_topk_without_logits(case, seq_ids, anchors, res)
    finally:
        case.W64 = W64
    case.d.dflash_set_lm_head_mxfp4(None, None)
    for l in range(cfg.n_layers):
        case.d.dflash_set_mlp_mxfp4(l, None, None, None, None)
    res = case.draft(seq_ids, anchors, logits=True)
    err, _ = H.check_draft(case, seq_ids, anchors, res)
    assert err <= H.LOGIT_TOL["bf16"]


@pytest.mark.parametrize("wide,n_seq", [(False, 1), (False, 2), (False, 5), (True, 10)],
                         ids=["16_rows", "32_rows", "80_rows", "160_rows_wide"])
def test_mxfp4_every_gemm(H, wide, n_seq):
    """MXFP4 codes for every weight GEMM (injection fc and stacked K/V, QKV, O, gate/up, down,
    lm_head): 16 draft rows (the streaming kernels and the independent-wave lm_head), 32 (skinny),
    80 and 160 (LDS tiles; the 160-row case at hidden 1024 / ffn 4608).  Ragged contexts injected
    with the bf16 weights, then one injection of up to 12 rows per sequence with the MXFP4 ones,
    then a draft, against the oracle run with the same matrices (dequantised where MXFP4)."""
    cfg = MID_WIDE_MLP if wide else MID
    case = H.Case(cfg, max_seqs=n_seq, max_batch=n_seq, max_inject_rows=128)
    seq_ids = list(range(n_seq))
    rng = np.random.default_rng(90 + n_seq)
    lens = [int(L) for L in rng.integers(20, 90, size=n_seq)]
    _prefill(case, seq_ids, [(0, L) for L in lens])
    W64 = case.W64
    case.W64 = _mxfp4_drafter(case, mlp=True, lm_head=True, attn=True, inject=True)
    try:
        adds = [np.arange(L, L + int(a)) for L, a in zip(lens, rng.integers(1, 13, size=n_seq))]
        case.inject(seq_ids, adds, start_pos=False)
        anchors = rng.integers(0, cfg.vocab - 1, size=n_seq).tolist()
        res = _check(H, case, seq_ids, anchors, mode_names=("viterbi",))
        _same_topk_without_logits(case, seq_ids, anchors, res)
    finally:
        case.W64 = W64


def _blocked_copy(t):
    import torch
    out = torch.empty_like(t)
    B.dflash_block_weights(t, out)
    return out


@pytest.mark.gpu
def test_blocked_weights_layout_and_same_bits(H):
    """(1) dflash_block_weights lays a bf16 [48][96] matrix out as the header defines it (the
    definition written out here with NumPy).  (2) With blocked copies of the lm_head, W_fc and
    every layer matrix registered, injections of 40..64 rows for 12 sequences (fc and the stacked
    K/V on the MFMA tiles, passes of up to 200 rows) and a 192-row draft with full logits (QKV, O,
    gate/up, down and the lm_head on the tiles) leave the same KV cache bytes and give the same
    outputs, bit for bit, as the row-major weights.  (3) Registering the row-major matrices
    themselves as the "blocked" copies changes the draft (same bytes, other order), so the
    tiles did read the registered copies."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    src = torch.randn((48, 96), generator=g, device="cuda").to(torch.bfloat16)
    dst = _blocked_copy(src)
    torch.cuda.synchronize()
    s = src.view(torch.int16).cpu().numpy()
    got = dst.view(torch.int16).cpu().numpy().reshape(-1)
    want = np.empty_like(got)
    steps = s.shape[1] // 32
    for grp in range(s.shape[0] // 16):
        for c in range(steps):
            for lane in range(64):
                q = lane // 4
                k = 32 * c + 8 * ((lane % 4) ^ (((q >> 1) ^ (q >> 3)) & 3))
                off = ((grp * steps + c) * 64 + lane) * 8
                want[off:off + 8] = s[16 * grp + q, k:k + 8]
    assert np.array_equal(got, want)

    cfg = MID.replace(n_heads=16, n_kv_heads=4, ffn=1536, name="mid_bf16_wide")
    case = H.Case(cfg, max_seqs=12, max_batch=12, max_inject_rows=200)
    ids = list(range(12))
    lens = [40 + 2 * i for i in ids]
    names = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")
    blocked = {"lm_head": _blocked_copy(case.dev_w["lm_head"]), "fc": _blocked_copy(case.dev_w["fc"]),
               "layers": [{n: _blocked_copy(lw[n]) for n in names} for lw in case.dev_w["layers"]]}
    plain = {"lm_head": case.dev_w["lm_head"], "fc": case.dev_w["fc"],
             "layers": [{n: lw[n] for n in names} for lw in case.dev_w["layers"]]}
    case.reset(ids)
    torch.cuda.synchronize()
    snapshot = case.d.kv.clone()
    ids_t = case.tensor(np.array(ids, np.int32))
    anchors = case.tensor(np.array([17 + 600 * i for i in ids], np.int32))

    def run():
        case.d.kv.copy_(snapshot)
        case.inject(ids, [np.arange(0, n) for n in lens])
        out = case.d.outputs(12, logits=True)
        case.d.dflash_draft_block(ids_t, anchors, out["topk_ids"], out["topk_logits"], out["h_final"], out["logits"])
        torch.cuda.synchronize()
        assert case.d.dflash_get_device_error() == 0
        return {k: v.clone() for k, v in out.items() if v is not None}, case.d.kv.clone()

    ref_out, ref_kv = run()
    case.d.dflash_set_blocked_weights(blocked)
    blk_out, blk_kv = run()
    case.d.dflash_set_blocked_weights(plain)
    wrong_out, _ = run()
    case.d.dflash_set_blocked_weights(None)
    assert torch.equal(ref_kv, blk_kv)
    for k in ref_out:
        assert torch.equal(ref_out[k], blk_out[k]), k
    assert not torch.equal(ref_out["logits"], wrong_out["logits"])


def _splitmix64(x):
    """SplitMix64 (Steele, Lea and Flood; constants as published by Vigna), on Python integers."""
    m = (1 << 64) - 1
    z = (x + 0x9E3779B97F4A7C15) & m
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
    return z ^ (z >> 31)


@pytest.mark.parametrize("p", [0.7, -1.0])
def test_synth_target_exact_draws(H, p):
    """The stand-in target's tokens equal the rule written out from the generator's definition:
    per (sequence b, token i) the key seed ^ (counter << 24) ^ (b << 8); draft i is kept when
    u = (h1 >> 40) / 2^24 < p (h1 = splitmix64(key ^ 2i)), or, with p < 0, when i < tau =
    1 + splitmix64(key ^ 0xABCD) mod K; else it becomes (draft + 1 + h2 mod (V - 1)) mod V
    (h2 = splitmix64(key ^ (2i + 1))); the token after the block is splitmix64(key ^ 0xFFFF) mod V.
    130 sequences x K = 8 is more slots than the kernel's 1024 threads."""
    import torch
    K, V, n, seed = 8, 1000, 130, 123
    d = torch.randint(0, V, (n, K - 1), dtype=torch.int32, device="cuda")
    ctr = torch.full((1,), 5, dtype=torch.int64, device="cuda")
    tgt = torch.empty((n, K), dtype=torch.int32, device="cuda")
    B.dflash_synth_target_argmax(n, K, V, d, p, seed, ctr, tgt)
    torch.cuda.synchronize()
    dn, got = d.cpu().numpy(), tgt.cpu().numpy()
    want = np.empty_like(got)
    pf = np.float32(p)
    for b in range(n):
        key = seed ^ (5 << 24) ^ (b << 8)
        tau = 1 + _splitmix64(key ^ 0xABCD) % K
        for i in range(1, K):
            u = np.float32(_splitmix64(key ^ (2 * i)) >> 40) * np.float32(1.0 / 16777216.0)
            alt = 1 + _splitmix64(key ^ (2 * i + 1)) % (V - 1)
            match = (i < tau) if p < 0 else bool(u < pf)
            di = int(dn[b, i - 1])
            want[b, i - 1] = di if match else (di + alt) % V
        want[b, K - 1] = _splitmix64(key ^ 0xFFFF) % V
    assert np.array_equal(got, want)
    assert ctr.item() == 6
