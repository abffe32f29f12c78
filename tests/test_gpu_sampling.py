"""GPU parity of the sampling path: dflash_select_sample and dflash_verify_rejection against the
oracle's sample_walk and verify_rejection on the same seeded inputs.

The lattice, the uniforms and the target distributions come straight from the seeded input
module, not from another GPU stage.  The picks are integer decisions taken in fp32 on the GPU
and in fp64 by the oracle.  Each uniform is therefore moved, before either side runs, to a
point whose oracle decision is unchanged over +-1/4096 around it.  That is the largest
possible shift of a CDF boundary from fp32 rounding of 16 or V weights, with a wide margin.
Picks and token ids must then agree exactly, and probabilities to 1e-4."""
import numpy as np
import pytest

from block_diffusion_draft_inject_amd import binding as B
from block_diffusion_draft_inject_amd import synth
from oracle import dflash_oracle as O

pytestmark = pytest.mark.gpu

GRID = 4096          # uniforms are kept off every decision boundary by at least 1/GRID
Q_TOL = 1e-4

MID = synth.DraftConfig(name="mid_bf16", n_layers=2, hidden=512, n_heads=8, n_kv_heads=2, head_dim=128, ffn=1024,
                        vocab=8192, n_taps=2, target_hidden=512, block_size=16, sel_rank=16, mask_id=8191,
                        dtype="bf16", batch=8, window=64)


@pytest.fixture(scope="module")
def H():
    import parity_harness as H
    return H


def stable_uniform(decide, u):
    """The grid point nearest u (cell centres (k + 1/2) / GRID) whose decision equals that of
    both neighbouring cells."""
    k0 = min(GRID - 1, int(u * GRID))
    memo = {}

    def at(k):
        if k not in memo:
            memo[k] = decide((k + 0.5) / GRID)
        return memo[k]

    for dk in range(GRID):
        for k in ((k0 + dk, k0 - dk) if dk else (k0,)):
            if 1 <= k <= GRID - 2 and at(k - 1) == at(k) == at(k + 1):
                return np.float32((k + 0.5) / GRID)
    raise AssertionError("no stable uniform")


def guarded_walk_uniforms(S, u, temperature, top_p=1.0):
    u = np.asarray(u, dtype=np.float64).copy()
    for t in range(len(S)):
        def decide(x, t=t):
            v = u.copy()
            v[t] = x
            return int(O.sample_walk(S, v, temperature, top_p)[0][t])
        u[t] = stable_uniform(decide, float(u[t]))
    return u.astype(np.float32)


def nucleus_is_stable(S, u, temperature, top_p, eps=1e-4):
    """The oracle's walk keeps the same picks and the same cut when top_p moves by +-eps, so no
    candidate's preceding mass sits within fp32 rounding of top_p."""
    idx, _, qc = O.sample_walk(S, u, temperature, top_p)
    for tp in (top_p - eps, min(1.0, top_p + eps)):
        i2, _, q2 = O.sample_walk(S, u, temperature, tp)
        if not np.array_equal(idx, i2) or not np.array_equal(qc > 0, q2 > 0):
            return False
    return True


def guarded_inputs(S_all, u_raw, temperature, top_p):
    """Uniforms kept off the CDF boundaries, and a top_p within 2e-3 of the asked one that no
    walk's cut sits near."""
    if top_p >= 1.0:
        return np.stack([guarded_walk_uniforms(S, u, temperature) for S, u in zip(S_all, u_raw)]), 1.0
    for k in range(20):
        tp = top_p + (k + 1) // 2 * 1e-4 * (1 if k % 2 else -1)
        u = np.stack([guarded_walk_uniforms(S, v, temperature, tp) for S, v in zip(S_all, u_raw)])
        if all(nucleus_is_stable(S, v, temperature, tp) for S, v in zip(S_all, u)):
            return u, tp
    raise AssertionError("no stable top_p near the asked one")


def _lattice_case(H, cfg, n, tag):
    case = H.Case(cfg, max_seqs=n, max_batch=n, max_inject_rows=16)
    ids, logits, hf = synth.lattice(cfg, n, tag)
    anchors = synth.rng(cfg.seed, "sample_anchor", tag).integers(0, cfg.vocab - 1, size=n).astype(np.int32)
    return case, ids, logits, hf, anchors


def _sample_on_gpu(case, anchors, ids, logits, hf, temperature, u_walk, want_q_cand=True, top_p=1.0):
    torch = case.torch
    n, km1 = len(anchors), ids.shape[1]
    path = torch.full((n, km1), -7, dtype=torch.int32, device="cuda")
    qp = torch.full((n, km1), -1.0, dtype=torch.float32, device="cuda")
    qc = torch.full((n, km1, 16), -1.0, dtype=torch.float32, device="cuda") if want_q_cand else None
    case.d.dflash_select_sample(case.tensor(anchors), case.tensor(ids), case.tensor(logits), case.tensor(hf),
                                temperature, top_p, case.tensor(u_walk), path, qp, qc)
    torch.cuda.synchronize()
    return path.cpu().numpy(), qp.cpu().numpy(), (None if qc is None else qc.cpu().numpy())


@pytest.mark.parametrize("cfg,temperature,top_p",
                         [(MID, 1.0, 1.0), (MID, 0.6, 1.0), (synth.WORKLOADS["tiny_fp32"], 1.7, 1.0),
                          (MID, 1.0, 0.95), (MID, 0.7, 0.5), (synth.WORKLOADS["tiny_fp32"], 2.5, 0.8)],
                         ids=["mid_bf16_T1", "mid_bf16_T0.6", "tiny_fp32_T1.7", "mid_bf16_T1_p0.95",
                              "mid_bf16_T0.7_p0.5", "tiny_fp32_T2.5_p0.8"])
def test_sampling_walk_matches_oracle(H, cfg, temperature, top_p):
    n = 8
    case, ids, logits, hf, anchors = _lattice_case(H, cfg, n, tag=1)
    u_raw, _, _ = synth.sampling_uniforms(cfg, n, tag=1)
    S_all = [O.pair_scores(cfg, case.W64, int(anchors[b]), ids[b], logits[b], hf[b]) for b in range(n)]
    u, top_p = guarded_inputs(S_all, u_raw, temperature, top_p)
    path, qp, qc = _sample_on_gpu(case, anchors, ids, logits, hf, temperature, u, top_p=top_p)
    _, _, qc_none = _sample_on_gpu(case, anchors, ids, logits, hf, temperature, u, want_q_cand=False, top_p=top_p)
    assert qc_none is None
    n_cut = 0
    for b in range(n):
        idx, q_path, q_cand = O.sample_walk(S_all[b], u[b], temperature, top_p)
        n_cut += int(np.sum(q_cand == 0))
        want = ids[b][np.arange(cfg.block_size - 1), idx]
        assert np.array_equal(path[b], want), (b, path[b], want)
        np.testing.assert_allclose(qp[b], q_path, atol=Q_TOL, rtol=0)
        np.testing.assert_allclose(qc[b], q_cand, atol=Q_TOL, rtol=0)
    if top_p < 1.0:
        assert n_cut > 0            # the cut removed candidates somewhere
    want_qc = np.stack([O.sample_walk(S_all[b], u[b], temperature, top_p)[2] for b in range(n)])
    H.log(f"[sample] {cfg.name} T={temperature} top_p={top_p}: {n} walks equal, {n_cut} candidates cut, "
          f"max |q err| {np.max(np.abs(qc - want_qc)):.2e}")


def test_sampling_walk_cold_temperature_is_greedy(H):
    """T -> 0: the walk takes the greedy walk's picks whatever the uniforms (oracle pin: the
    sampling walk at small T reduces to the greedy walk)."""
    cfg, n = MID, 4
    case, ids, logits, hf, anchors = _lattice_case(H, cfg, n, tag=2)
    u, _, _ = synth.sampling_uniforms(cfg, n, tag=2)
    path, qp, _ = _sample_on_gpu(case, anchors, ids, logits, hf, 1e-4, u)
    for b in range(n):
        S = O.pair_scores(cfg, case.W64, int(anchors[b]), ids[b], logits[b], hf[b])
        g, _, margin = O.greedy_walk(S)
        if margin > 1e-2:
            assert np.array_equal(path[b], ids[b][np.arange(cfg.block_size - 1), g])
            assert np.all(qp[b] > 0.99)


def test_select_sample_rejects_bad_temperature_and_top_p(H):
    import torch
    cfg, n = MID, 1
    case, ids, logits, hf, anchors = _lattice_case(H, cfg, n, tag=3)
    u = np.zeros((n, cfg.block_size - 1), dtype=np.float32)
    for T in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(B.DflashError):
            _sample_on_gpu(case, anchors, ids, logits, hf, T, u)
    for p in (0.0, -0.5, 1.5, float("nan")):
        with pytest.raises(B.DflashError):
            _sample_on_gpu(case, anchors, ids, logits, hf, 1.0, u, top_p=p)


# ------------------------------------------------------------------------------ rejection verification

def _verify_on_gpu(case, draft, q_path, cand, q_cand, p, u_acc, u_res):
    torch = case.torch
    n, km1 = draft.shape
    K, V = km1 + 1, p.shape[-1]
    nacc = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    ncom = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    com = torch.full((n, K), -7, dtype=torch.int32, device="cuda")
    nxt = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    B.dflash_verify_rejection(n, K, V, case.tensor(draft.astype(np.int32)), case.tensor(q_path.astype(np.float32)),
                              case.tensor(cand.astype(np.int32)), case.tensor(q_cand.astype(np.float32)),
                              case.tensor(p), case.tensor(u_acc.astype(np.float32)),
                              case.tensor(u_res.astype(np.float32)), nacc, ncom, com, nxt)
    torch.cuda.synchronize()
    return nacc.cpu().numpy(), ncom.cpu().numpy(), com.cpu().numpy(), nxt.cpu().numpy()


def _guard_accept(u, q, pd):
    """Move u off the acceptance boundary u * q = p(d) by more than fp32 rounding of u * q."""
    u = np.float32(u)
    while abs(float(u) * float(q) - float(pd)) <= 1e-4 * (float(u) * float(q) + float(pd)):
        u = np.float32(min(0.999, float(u) + 0.01) if float(u) < 0.5 else float(u) - 0.01)
    return u


def _rejection_inputs(case, n, tag, temperature=1.0):
    """Draft, q and candidates from the oracle's own sampling walk on a seeded lattice."""
    cfg, W64 = case.cfg, case.W64
    ids, logits, hf = synth.lattice(cfg, n, tag)
    anchors = synth.rng(cfg.seed, "sample_anchor", tag).integers(0, cfg.vocab - 1, size=n)
    u_walk, u_acc, u_res = synth.sampling_uniforms(cfg, n, tag)
    draft = np.empty((n, cfg.block_size - 1), dtype=np.int64)
    q_path = np.empty((n, cfg.block_size - 1), dtype=np.float32)
    q_cand = np.empty((n, cfg.block_size - 1, 16), dtype=np.float32)
    for b in range(n):
        S = O.pair_scores(cfg, W64, int(anchors[b]), ids[b], logits[b], hf[b])
        idx, qp, qc = O.sample_walk(S, u_walk[b], temperature)
        draft[b] = ids[b][np.arange(cfg.block_size - 1), idx]
        q_path[b], q_cand[b] = qp, qc
    p = synth.target_probs(cfg, ids, tag)
    return draft, q_path, ids, q_cand, p, u_acc, u_res


def _guard_and_check(case, draft, q_path, cand, q_cand, p, u_acc, u_res):
    n, km1 = draft.shape
    u_acc = u_acc.copy()
    u_res = u_res.copy()
    p64, q64, qc64 = p.astype(np.float64), q_path.astype(np.float64), q_cand.astype(np.float64)
    for b in range(n):
        for i in range(km1):
            if 0 < u_acc[b, i] < 1:
                u_acc[b, i] = _guard_accept(u_acc[b, i], q_path[b, i], p[b, i, draft[b, i]])
        ua = u_acc[b].astype(np.float64)
        decide = lambda x, b=b, ua=ua: O.verify_rejection(draft[b], q64[b], cand[b], qc64[b], p64[b], ua, x)[2]
        u_res[b] = stable_uniform(decide, float(u_res[b]))
    nacc, ncom, com, nxt = _verify_on_gpu(case, draft, q_path, cand, q_cand, p, u_acc, u_res)
    for b in range(n):
        nn, c, tok = O.verify_rejection(draft[b], q64[b], cand[b], qc64[b], p64[b], u_acc[b].astype(np.float64),
                                        float(u_res[b]))
        assert (nacc[b], ncom[b], nxt[b]) == (nn, nn + 1, tok), (b, nacc[b], nn, nxt[b], tok)
        assert np.array_equal(com[b], c), (b, com[b], c)
    return nacc


@pytest.mark.parametrize("cfg", [MID, synth.WORKLOADS["tiny_fp32"]], ids=["mid_bf16", "tiny_fp32"])
def test_rejection_verification_matches_oracle(H, cfg):
    n = 16
    case = H.Case(cfg, max_seqs=1, max_batch=1, max_inject_rows=16)
    draft, q_path, cand, q_cand, p, u_acc, u_res = _rejection_inputs(case, n, tag=4)
    u_acc[0] = 0.0                     # every draft accepted: bonus draw from the last row
    u_acc[1, 0] = 0.999                # an early rejection where p(d) < 0.999 q(d) ...
    p[1, 0, draft[1, 0]] = 1e-6        # ... guaranteed by a tiny target probability
    nacc = _guard_and_check(case, draft, q_path, cand, q_cand, p, u_acc, u_res)
    assert nacc[0] == cfg.block_size - 1 and nacc[1] == 0
    assert 0 < np.mean(nacc[2:]) < cfg.block_size - 1     # mixed acceptance lengths
    H.log(f"[reject] {cfg.name}: accepted {nacc.tolist()}")


def test_rejection_verification_residual_without_mass(H):
    """Target rows that are not normalised: at the rejection the drafter's q covers p on every
    token, so max(0, p - q) has no mass and the token is drawn from p itself."""
    cfg = MID
    K, V = cfg.block_size, cfg.vocab
    case = H.Case(cfg, max_seqs=1, max_batch=1, max_inject_rows=16)
    n = 2
    rng = synth.rng(cfg.seed, "residual_without_mass")
    cand = np.stack([np.stack([rng.choice(V, 16, replace=False) for _ in range(K - 1)]) for _ in range(n)])
    draft = cand[:, :, 0].copy()
    q_cand = np.full((n, K - 1, 16), 1.0 / 16, dtype=np.float32)
    q_path = q_cand[:, :, 0].copy()
    p = np.zeros((n, K, V), dtype=np.float32)
    for b in range(n):
        for i in range(K - 1):
            p[b, i, cand[b, i]] = 1.0 / 16            # p == q on the candidates: every draft accepted ...
        p[b, 3, cand[b, 3]] = np.linspace(0.01, 0.05, 16, dtype=np.float32)   # ... until slot 4 (p <= q)
        p[b, K - 1, :] = 1.0 / V
    u_acc = np.full((n, K - 1), 0.5, dtype=np.float32)
    u_res = np.array([0.1, 0.8], dtype=np.float32)
    nacc = _guard_and_check(case, draft, q_path, cand, q_cand, p, u_acc, u_res)
    assert np.all(nacc == 3)


def test_rejection_verification_full_vocab_b32(H):
    """The bench's sampled workload size: 32 sequences, block 8, the large drafter's vocabulary."""
    big = synth.WORKLOADS["b32_k8_conv"]
    cfg = MID.replace(vocab=big.vocab, block_size=big.block_size, mask_id=big.vocab - 1)
    n = big.batch
    case = H.Case(MID, max_seqs=1, max_batch=1, max_inject_rows=16)     # only for the device helpers
    rng = synth.rng(cfg.seed, "full_vocab_verify")
    cand = np.stack([np.stack([rng.choice(cfg.vocab, 16, replace=False) for _ in range(cfg.block_size - 1)])
                     for _ in range(n)])
    q_cand = rng.dirichlet(np.ones(16), size=(n, cfg.block_size - 1)).astype(np.float32)
    pick = rng.integers(0, 16, size=(n, cfg.block_size - 1))
    draft = np.take_along_axis(cand, pick[..., None], axis=-1)[..., 0]
    q_path = np.take_along_axis(q_cand, pick[..., None], axis=-1)[..., 0]
    p = synth.target_probs(cfg, cand, tag=5)
    u_acc, _, u_res = synth.sampling_uniforms(cfg, n, tag=5)
    nacc = _guard_and_check(case, draft, q_path, cand, q_cand, p, u_acc, u_res)
    H.log(f"[reject] vocab {cfg.vocab} batch {n}: accepted {nacc.tolist()}")


def test_rejection_verification_empty_batch_and_bad_shapes(H):
    import torch
    z = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.dflash_verify_rejection(0, 8, 100, z, z, z, z, z, z, z, z, z, z, z)     # nothing to do
    for K, V in ((1, 100), (65, 100), (8, 1)):
        with pytest.raises(B.DflashError):
            B.dflash_verify_rejection(1, K, V, z, z, z, z, z, z, z, z, z, z, z)
