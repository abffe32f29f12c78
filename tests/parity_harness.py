"""Shared GPU-vs-oracle parity machinery (test infrastructure: imports the oracle).

Every comparison runs the oracle on the same seeded inputs as the HIP path; where a stage's
input is itself a GPU output (the selector's candidate lists, the verifier's draft), the
oracle stage is run on the GPU's own inputs (stage-wise parity)."""
from __future__ import annotations

import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from block_diffusion_draft_inject_amd import binding as B  # noqa: E402
from block_diffusion_draft_inject_amd import synth  # noqa: E402
from oracle import dflash_oracle as O  # noqa: E402

# Tolerances.  Logits: max-abs 3e-2 for bf16 drafters (the stated bound), 1e-4 for fp32.
LOGIT_TOL = {"bf16": 3e-2, "f32": 1e-4}
TIE_BAND = 1e-3          # top-16 ids may differ only between candidates this close in value
MARGIN_GATE = 1e-3       # paths must match exactly where the top-two margin exceeds this


def log(*a):
    print(*a, flush=True)


def weights64(w):
    out = {k: v.values.astype(np.float64) for k, v in w.items() if k != "layers"}
    out["layers"] = [{k: v.values.astype(np.float64) for k, v in lw.items()} for lw in w["layers"]]
    return out


def oracle_mode(cfg):
    return "bf16" if cfg.dtype == "bf16" else "exact"


def poison(drafter):
    """Fills the workspace and the K/V area of the cache with 0xFF bytes (NaN in bf16 and fp32),
    so that a kernel reading memory no earlier kernel wrote shows up as NaN in the results.
    The per-sequence length words stay zero."""
    drafter.ws.fill_(255)
    drafter.kv[: drafter.kv_layout.seq_len_offset].fill_(255)


class Case:
    """One drafter on the GPU plus its oracle twin."""

    def __init__(self, cfg, max_seqs, max_batch, max_inject_rows=1024, selector_stress=False, device="cuda"):
        import torch
        self.torch = torch
        self.cfg = cfg
        t0 = time.time()
        self.w = synth.make_weights(cfg, selector_stress=selector_stress)
        self.W64 = weights64(self.w)
        self.dev_w = B.upload_weights(self.w, cfg.dtype, device)
        self.d = B.Drafter(cfg, self.dev_w, max_seqs, max_batch, max_inject_rows, device)
        poison(self.d)
        self.caches = {}
        self.device = device
        log(f"[case] {cfg.name}: weights ready in {time.time() - t0:.1f}s")

    def tensor(self, a, dtype=None):
        t = self.torch.as_tensor(np.ascontiguousarray(a))
        if dtype is not None:
            t = t.to(dtype)
        return t.to(self.device)

    def states_tensor(self, per_seq_rows, max_new):
        """[n_seq][max_new][concat] device tensor from per-sequence Tensor rows (padded)."""
        cfg = self.cfg
        n = len(per_seq_rows)
        if cfg.dtype == "bf16":
            buf = np.zeros((n, max_new, cfg.concat_width), dtype=np.uint16)
        else:
            buf = np.zeros((n, max_new, cfg.concat_width), dtype=np.float32)
        for i, t in enumerate(per_seq_rows):
            if t is not None and t.storage.shape[0]:
                buf[i, : t.storage.shape[0]] = t.storage
        if cfg.dtype == "bf16":
            return self.torch.from_numpy(buf.view(np.int16)).to(self.device).view(self.torch.bfloat16)
        return self.torch.from_numpy(buf).to(self.device)

    def reset(self, seq_ids):
        self.d.dflash_reset_seqs(self.tensor(np.asarray(seq_ids, dtype=np.int32)))
        for s in seq_ids:
            self.caches[int(s)] = O.DraftCache(self.cfg.n_layers)

    def inject(self, seq_ids, positions_per_seq, start_pos=True, states_fn=None):
        """Injects states of the given absolute positions (contiguous per sequence) on both sides."""
        cfg = self.cfg
        rows = []
        for s, pos in zip(seq_ids, positions_per_seq):
            pos = np.asarray(pos, dtype=np.int64)
            st = (synth.target_states(cfg, int(s), pos) if states_fn is None else states_fn(int(s), pos))
            rows.append(st)
            if pos.size:
                O.inject(cfg, self.W64, self.caches[int(s)], pos, st.values, oracle_mode(cfg))
        n_new = np.array([len(p) for p in positions_per_seq], dtype=np.int32)
        max_new = int(max(1, n_new.max()))
        sp = np.array([int(p[0]) if len(p) else 0 for p in positions_per_seq], dtype=np.int32)
        self.d.dflash_inject_kv(self.tensor(np.asarray(seq_ids, dtype=np.int32)), self.tensor(n_new), max_new,
                                self.states_tensor(rows, max_new), start_pos=self.tensor(sp) if start_pos else None)

    def draft(self, seq_ids, anchors, logits=True):
        torch = self.torch
        n = len(seq_ids)
        out = self.d.outputs(n, logits=logits)
        self.d.dflash_draft_block(self.tensor(np.asarray(seq_ids, dtype=np.int32)),
                                  self.tensor(np.asarray(anchors, dtype=np.int32)),
                                  out["topk_ids"], out["topk_logits"], out["h_final"], out["logits"])
        torch.cuda.synchronize()
        res = {k: (None if v is None else (v.float().cpu().numpy() if v.dtype == torch.bfloat16 else v.cpu().numpy()))
               for k, v in out.items()}
        res["_dev"] = out
        return res

    def select(self, anchors, dev_out, mode):
        torch = self.torch
        n = len(anchors)
        K = self.cfg.block_size
        path = torch.empty((n, K - 1), dtype=torch.int32, device=self.device)
        score = torch.empty(n, dtype=torch.float32, device=self.device)
        margin = torch.empty(n, dtype=torch.float32, device=self.device)
        self.d.dflash_select_path(self.tensor(np.asarray(anchors, dtype=np.int32)), dev_out["topk_ids"],
                                  dev_out["topk_logits"], dev_out["h_final"], mode, path, score, margin)
        torch.cuda.synchronize()
        return path.cpu().numpy(), score.cpu().numpy(), margin.cpu().numpy()

    def verify(self, draft, target):
        torch = self.torch
        n, km1 = draft.shape
        K = km1 + 1
        nacc = torch.empty(n, dtype=torch.int32, device=self.device)
        ncom = torch.empty(n, dtype=torch.int32, device=self.device)
        com = torch.empty((n, K), dtype=torch.int32, device=self.device)
        nxt = torch.empty(n, dtype=torch.int32, device=self.device)
        B.dflash_verify_greedy(n, K, self.tensor(draft.astype(np.int32)), self.tensor(target.astype(np.int32)),
                               nacc, ncom, com, nxt)
        torch.cuda.synchronize()
        return nacc.cpu().numpy(), ncom.cpu().numpy(), com.cpu().numpy(), nxt.cpu().numpy()


# ------------------------------------------------------------------------------ checks

def check_kv(case, seq_ids, sample_layers=None, max_positions=64):
    """Cache contents vs the oracle for (a sample of) the positions each ring holds.

    Returns (worst error in units of the allowed bound, fraction of bit-identical elements).
    Allowed per element: bf16 drafters one bf16 ulp of the value (2^-7 |x|: the two sides
    round an fp32 vs an fp64 value, so a value next to a rounding boundary can land on either
    neighbour) plus 1e-2 rms for rounding flips upstream -- one flip of a large element of
    c = W_fc u_bar moves K/V by |w| * ulp(c), about 3e-3 rms with N(0, 0.02) weights;
    fp32 drafters 1e-5 rms."""
    cfg = case.cfg
    k, v, sl, sb = case.d.kv_views()
    torch = case.torch
    torch.cuda.synchronize()
    sl = sl.cpu().numpy()
    sb = sb.cpu().numpy()
    worst = 0.0
    same = tot = 0
    offenders = []
    layers = range(cfg.n_layers) if sample_layers is None else sample_layers
    for s in seq_ids:
        cache = case.caches[int(s)]
        assert sl[s] == cache.length, (s, sl[s], cache.length)
        held = [p for p in cache.positions() if p >= cache.length - cfg.window]
        if len(held) > max_positions:
            idx = np.linspace(0, len(held) - 1, max_positions).round().astype(int)
            held = [held[i] for i in idx]
        for l in layers:
            kc = k[l, s].float().cpu().numpy()
            vc = v[l, s].float().cpu().numpy()
            for p in held:
                slot = p % cfg.window
                for kind, got, ref in (("K", kc[:, slot], cache.k[l][p]), ("V", vc[:, slot], cache.v[l][p])):
                    rms = max(1e-30, float(np.sqrt(np.mean(ref * ref))))
                    if cfg.dtype == "bf16":
                        bound = 2.0 ** -7 * np.abs(ref) + 1e-2 * rms
                    else:
                        bound = np.full(ref.shape, 1e-5 * rms)
                    assert np.all(np.isfinite(got)), (s, l, kind, p)   # NaN would slip past max()
                    ratio = np.abs(got - ref) / bound
                    if float(np.max(ratio)) > 1.0:
                        i = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
                        offenders.append((float(ratio[i]), int(s), l, kind, p, tuple(int(x) for x in i),
                                          float(got[i]), float(ref[i]), rms))
                    worst = max(worst, float(np.max(ratio)))
                    same += int(np.sum(got == ref))
                    tot += got.size
    if offenders:
        offenders.sort(reverse=True)
        for o in offenders[:8]:
            log("[kv offender] ratio %.2f seq %d layer %d %s pos %d elem %s got %.6g ref %.6g rms %.3g" % o)
        log(f"[kv] {len(offenders)} (position, layer, K/V) entries exceed the bound")
    return worst, same / max(1, tot)


class SwapCount:
    """Top-16 set differences against the oracle, split by how far the candidate's oracle logit
    lies from the oracle's 16th value: within the 1e-3 tie band, or beyond it but within twice
    the row's measured logit error (two candidates closer than the logit error can swap)."""

    def __init__(self):
        self.rows = self.rows_swapped = self.tie = self.wide = self.wide_rows = 0
        self.max_gap = 0.0

    def add_row(self, gset, oset, o_logits, kth, row_err, band=TIE_BAND):
        self.rows += 1
        if gset == oset:
            return
        self.rows_swapped += 1
        wide = False
        for i in gset ^ oset:
            gap = abs(o_logits[i] - kth)
            assert gap <= band + 2 * row_err, ("top-16 set", i, gap, row_err)
            self.max_gap = max(self.max_gap, gap)
            if gap <= band:
                self.tie += 1
            else:
                self.wide += 1
                wide = True
        self.wide_rows += wide

    def __str__(self):
        return (f"{self.rows} rows, {self.rows_swapped} with a set difference: {self.tie} ids within the 1e-3 tie "
                f"band, {self.wide} beyond it in {self.wide_rows} rows (largest gap {self.max_gap:.2e})")

    def ok(self):
        return self.wide_rows <= max(2, WIDE_SWAP_ROWS * self.rows)


# Rows whose top-16 set differs from the oracle's by a candidate beyond the 1e-3 band (but within
# twice the row's logit error) are expected at this rate: near the 16th value of a 151936-word row
# of N(0, 0.9) logits neighbouring values lie ~0.02 apart, so a logit error of 2..7e-3 reorders a
# pair there in a few percent of rows.  The cap guards against a systematic drift.
WIDE_SWAP_ROWS = 0.15


def check_draft(case, seq_ids, anchors, res, band=TIE_BAND, oracles=None, swaps_out=None):
    """Logits, then top-16: bitwise equal to the exact top-16 of the GPU's own logits, and equal
    as a set to the oracle's up to near-ties.  A candidate may enter or leave the set only if its
    oracle logit is within `band` + 2 * (that row's max |GPU - oracle| logit error) of the
    oracle's 16th value: two candidates closer than the logit error can legitimately swap.  The
    differences beyond the 1e-3 band are counted and held to WIDE_SWAP_ROWS of the rows."""
    cfg = case.cfg
    errs = []
    o_all = []
    sc = SwapCount() if swaps_out is None else swaps_out
    for b, (s, a) in enumerate(zip(seq_ids, anchors)):
        o = oracles[b] if oracles is not None else O.draft_block(cfg, case.W64, case.caches[int(s)], int(a),
                                                                  oracle_mode(cfg))
        o_all.append(o)
        row_err = np.full(cfg.block_size - 1, np.inf)
        if res.get("logits") is not None:
            row_err = np.max(np.abs(res["logits"][b] - o["logits"]), axis=1)
            errs.append(float(row_err.max()))
            for t in range(cfg.block_size - 1):
                lg = res["logits"][b, t].astype(np.float64)
                ref = np.argsort(-lg, kind="stable")[:16]
                assert np.array_equal(res["topk_ids"][b, t], ref), ("own-logit top-16", b, t)
                assert np.array_equal(res["topk_logits"][b, t], res["logits"][b, t][ref])
        else:
            # no full logits: the GPU's top-16 values vs the oracle's logits of the same ids
            for t in range(cfg.block_size - 1):
                ids = res["topk_ids"][b, t]
                row_err[t] = float(np.max(np.abs(res["topk_logits"][b, t] - o["logits"][t][ids])))
            errs.append(float(row_err.max()))
        for t in range(cfg.block_size - 1):
            gset, oset = set(res["topk_ids"][b, t].tolist()), set(o["topk_ids"][t].tolist())
            sc.add_row(gset, oset, o["logits"][t], o["topk_logits"][t][-1], row_err[t], band)
        slot_err = np.max(np.abs(res["h_final"][b] - o["h_final"]), axis=1)
        hf_err = float(slot_err.max())
        assert hf_err < 0.1, ("h_final", b, hf_err, "per slot", np.round(slot_err, 4).tolist())
    err = max(errs) if errs else 0.0
    log(f"[draft] {cfg.name}: max |logit err| {err:.3e}; top-16 vs oracle: {sc}")
    assert sc.ok(), str(sc)
    return err, o_all


def check_select(case, anchors, res, gpu_path, gpu_score, gpu_margin, mode_name):
    """Selector on the GPU's own lattice: exact where the oracle margin exceeds the gate;
    elsewhere the GPU path must be (near-)optimal under the oracle's scores."""
    cfg = case.cfg
    n_checked = 0
    for b, a in enumerate(anchors):
        ids = res["topk_ids"][b].astype(np.int64)
        lg = res["topk_logits"][b].astype(np.float64)
        hf = res["h_final"][b].astype(np.float64)
        o = O.select_path(cfg, case.W64, int(a), ids, lg, hf, mode_name)
        assert abs(o["score"] - gpu_score[b]) <= MARGIN_GATE, (b, o["score"], gpu_score[b])
        if o["margin"] > MARGIN_GATE:
            assert np.array_equal(o["path_ids"], gpu_path[b]), (b, o["path_ids"], gpu_path[b])
            assert abs(o["margin"] - gpu_margin[b]) <= MARGIN_GATE
            n_checked += 1
        else:
            # several paths are optimal within the band: the GPU's must score within it
            S = O.pair_scores(cfg, case.W64, int(a), ids, lg, hf)
            idx = [int(np.where(ids[t] == gpu_path[b][t])[0][0]) for t in range(cfg.block_size - 1)]
            sc = S[0][0, idx[0]] + sum(S[t][idx[t - 1], idx[t]] for t in range(1, len(idx)))
            assert sc >= o["score"] - 2 * MARGIN_GATE
    return n_checked


def check_verify(case, draft, target):
    nacc, ncom, com, nxt = case.verify(draft, target)
    for b in range(draft.shape[0]):
        n, c, a = O.verify_greedy(draft[b], target[b])
        assert nacc[b] == n and ncom[b] == n + 1 and nxt[b] == a, b
        assert np.array_equal(com[b], c), b
    return nacc
