"""dflash2_draft_select (steps 1-4 in one call, the candidate merge inside
the selector's kernel) against dflash2_draft_block followed by
dflash2_select_path on the same inputs: bit-identical candidate ids and
values, paths, draft tokens and path scores.  The two-call path is checked
against the oracle in test_gpu_draft.py, so this pins the fused one to the
oracle too.  Covered: candidate lists of the weight-streaming lm_head
(k <= 16 per 128-id group; 65-256 lists per row keep the separate merge
kernel, more than 256 are first folded 64 at a time) and of the
tiled one (16 per vocabulary run), 1..15 positions per sequence, a
transformed logit (multiplier and soft cap), and k > 16, where the merge
keeps its own kernel."""
import numpy as np
import pytest
import torch

import synth
from _gpu_common import DraftRun, log

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny_fp32", {}),
    ("small_bf16", {}),
    ("small_fp8", {}),
    ("small_bf16", dict(output_multiplier=0.5, final_logit_softcapping=30.0)),
    ("small_bf16", dict(top_k=20)),
    ("small_bf16", dict(block_size=2)),
    ("small_bf16", dict(vocab=8192)),    # 64 lists per row: the most the fused merge takes
    ("small_bf16", dict(vocab=8193)),    # 65 lists: the separate merge kernel
    ("small_bf16", dict(vocab=40000, top_k=8)),   # 313 lists of 8 keys: folded to 5 first
    ("medium_fp8", {}),
    ("medium_bf16", dict(block_size=16)),
    ("dense27b_bf16", {}),
    ("longblock_bf16", {}),
    ("fp8_b256", {}),
]


@pytest.mark.parametrize("name,over", CASES,
                         ids=[n + "".join(f"-{k}{v}" for k, v in o.items()) for n, o in CASES])
def test_draft_select_matches_two_calls(name, over):
    w = synth.get(name).replace(**over) if over else synth.get(name)
    g = DraftRun(w, debug=False)
    try:
        m = g.model
        log(f"{w.name} {over}: draft_select B={w.batch}")
        want_logits = name in ("small_bf16", "medium_fp8")
        out = m.draft_select(g.anchors, g.taps, g.offsets, g.ctx_lens, g.max_new, g.kc, g.vc,
                             debug_logits=want_logits)
        torch.cuda.synchronize()
        assert np.array_equal(out["topk_ids"].cpu().numpy(), g.topk_ids)
        assert np.array_equal(out["topk_vals"].cpu().numpy().view(np.uint32), g.topk_vals.view(np.uint32))
        assert np.array_equal(out["path"].cpu().numpy(), g.path)
        assert np.array_equal(out["drafts"].cpu().numpy(), g.drafts)
        assert np.array_equal(out["score"].cpu().numpy().view(np.uint32), g.score.view(np.uint32))
        if want_logits:
            # the top-k of the logits this call wrote is the call's own top-k
            z = out["debug_logits"].cpu().numpy().reshape(-1, w.vocab)
            ids = g.topk_ids.reshape(-1, w.top_k).astype(np.int64)
            raw = np.take_along_axis(z, ids, axis=1) + np.float32(0.0)
            top = -np.sort(-z, axis=1)[:, :w.top_k]
            assert np.array_equal(np.sort(raw, axis=1), np.sort(top, axis=1))
        log(f"{w.name}: identical to draft_block + select_path")
    finally:
        g.close()
