"""The allocation-free draft (dflash_draft_block_static: the pass's scratch in the library's static
device array) against the workspace draft (dflash_draft_block) through the C ABI: two calls in a
row on the same inputs, the second with fewer sequences, outputs bit-identical (the same kernels
on the same inputs in the same launch configuration), for a bf16 and an fp32 drafter; a call
too large for the static array is refused before anything is enqueued."""
import numpy as np
import pytest

from block_diffusion_draft_inject_amd import binding as B
from block_diffusion_draft_inject_amd import synth

pytestmark = pytest.mark.gpu

MID = synth.DraftConfig(name="mid_bf16", n_layers=2, hidden=512, n_heads=8, n_kv_heads=2, head_dim=128, ffn=1024,
                        vocab=8192, n_taps=2, target_hidden=512, block_size=16, sel_rank=16, mask_id=8191,
                        dtype="bf16", batch=8, window=64)


def _drafts(case, seq_ids, anchors):
    import torch
    outs = []
    for fn in (case.d.dflash_draft_block, case.d.dflash_draft_block_static):
        out = case.d.outputs(len(seq_ids), logits=True)
        for v in out.values():
            v.fill_(float("nan")) if v.dtype.is_floating_point else v.fill_(-7)
        fn(case.tensor(np.asarray(seq_ids, dtype=np.int32)), case.tensor(np.asarray(anchors, dtype=np.int32)),
           out["topk_ids"], out["topk_logits"], out["h_final"], out["logits"])
        torch.cuda.synchronize()
        outs.append({k: v.cpu() for k, v in out.items()})
    return outs


@pytest.mark.parametrize("name", ["mid_bf16", "tiny_fp32"])
def test_static_scratch_draft_matches_workspace_draft(name):
    import torch
    import parity_harness as H
    cfg = MID if name == "mid_bf16" else synth.WORKLOADS["tiny_fp32"]
    n = 3
    case = H.Case(cfg, max_seqs=n, max_batch=n, max_inject_rows=64)
    seq_ids = list(range(n))
    case.reset(seq_ids)
    case.inject(seq_ids, [np.arange(0, 40 + 9 * i) for i in seq_ids])
    anchors = [17, 4000, 123]
    for ids, anc in ((seq_ids, anchors), ([2], [77])):      # the second call smaller than the first
        ref, got = _drafts(case, ids, anc)
        for k in ref:
            assert torch.equal(ref[k], got[k]), (name, len(ids), k)
        assert not torch.isnan(got["logits"]).any()
        H.log(f"[static scratch] {name}: {len(ids)} sequences, outputs bit-identical to the workspace draft")
    # too many sequences for the 32 MiB array: refused with DFLASH_E_SHAPE
    big = int(np.ceil(33 * 2 ** 20 / max(1, B.dflash_workspace_bytes(cfg, 1, 1, 1))))
    while B.dflash_workspace_bytes(cfg, 1, big, 1) <= 32 * 2 ** 20:
        big *= 2
    ids = torch.zeros(big, dtype=torch.int32, device="cuda")
    out = case.d.outputs(1)
    with pytest.raises(B.DflashError) as e:
        case.d.dflash_draft_block_static(ids, ids, out["topk_ids"], out["topk_logits"], out["h_final"])
    assert e.value.status == -2 and b"static scratch" in B.lib().dflash_last_error()
    assert case.d.dflash_get_device_error() == 0
