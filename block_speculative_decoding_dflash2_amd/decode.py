"""Multi-step speculative decoding around the draft step: draft -> select ->
verify rounds with the state carried over between rounds.

After a round that accepts `a` drafts, the target has verified the anchor and
those `a` drafts, so their a + 1 positions (L .. L + a) are appended to the
draft's context in the next round, the context grows to L + a + 1, and the
target's own next token (the bonus) becomes the new anchor (llama-cpp-python
wiki "DFlash2 Speculative Decoding", "Prerequisites" and "Complete Runnable
Code"; NVIDIA NIM for Alpamayo, "Observe Acceptance").  The block's own keys
and values only ever occupy cache rows past the context, which the next
append overwrites, so a rejected draft needs no rollback.

The target model is the caller's: `target_logits(step, drafts)` returns the
verifier's logits for the chosen drafts and `verified_taps(starts, counts)`
the target's hidden-state taps of newly verified positions.  Every step of
the draft path runs in the library's kernels; this module only carries state
between calls (one host synchronisation per round, for the accepted counts).
"""
from __future__ import annotations

from typing import Callable, Dict, List, Optional, Tuple

import numpy as np
import torch

from .metrics import speculative_metrics
from .runner import (DFlash2, to_device, verify_accept, verify_sample, verify_sample_workspace,
                     verify_workspace)


def decode_loop(model: DFlash2, k_cache: torch.Tensor, v_cache: torch.Tensor, anchors: np.ndarray,
                ctx_lens: np.ndarray, taps, new_offsets: np.ndarray, steps: int,
                target_logits: Callable[[int, np.ndarray], np.ndarray],
                verified_taps: Callable[[np.ndarray, np.ndarray], tuple],
                sampling: Optional[Tuple[float, int, float]] = None,
                uniforms: Optional[Callable[[int], np.ndarray]] = None,
                p_min: Optional[float] = None, n_min: int = 0, n_max: Optional[int] = None) -> Dict:
    """Run `steps` rounds.  `taps` (a Tensor with `.data`) and `new_offsets`
    are the first round's appended rows; `ctx_lens` the context lengths after
    that append.  sampling = (temperature, top_k, top_p) verifies by
    rejection sampling with the caller's uniforms(step) -> [B, bs] float32
    in [0, 1); p_min (with n_min / n_max) cuts each path with the selector
    confidence rule.  Returns per-round drafts / lens / accepted / bonus /
    ctx_lens (before the round) and the acceptance metrics."""
    cfg = model.cfg
    dev = model.device
    B, bs, V = len(anchors), cfg["block_size"], cfg["vocab"]
    P, k = bs - 1, cfg["selector_top_k"]
    if np.max(ctx_lens) + steps * bs + bs > cfg["max_context"]:
        raise ValueError("max_context too small for this many rounds")
    max_new = max(int(new_offsets[-1]), B * bs)
    ws = model.workspace(B, max_new)
    if sampling is None and p_min is None:
        vws = verify_workspace(B, bs, V, dev)
    else:
        vws = verify_sample_workspace(B, bs, V, dev)
    lens = torch.full((B,), P, dtype=torch.int32, device=dev)
    topk_ids = torch.empty((B, P, k), dtype=torch.int32, device=dev)
    topk_vals = torch.empty((B, P, k), dtype=torch.float32, device=dev)
    path = torch.empty((B, P), dtype=torch.int32, device=dev)
    drafts = torch.empty((B, P), dtype=torch.int32, device=dev)
    accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    bonus = torch.empty((B,), dtype=torch.int32, device=dev)
    anchors = np.asarray(anchors, dtype=np.int32).copy()
    ctx = np.asarray(ctx_lens, dtype=np.int64).copy()
    offsets = np.asarray(new_offsets, dtype=np.int32)
    rec: Dict[str, List[np.ndarray]] = {"drafts": [], "lens": [], "accepted": [], "bonus": [], "ctx_lens": []}
    for s in range(steps):
        d_anchors = torch.from_numpy(anchors).to(dev)
        d_ctx = torch.from_numpy(ctx.astype(np.int32)).to(dev)
        d_off = torch.from_numpy(offsets).to(dev)
        d_taps = to_device(taps.data.reshape(taps.data.shape[0], -1), dev)
        model.draft_block(d_anchors, d_taps, d_off, d_ctx, max_new, k_cache, v_cache, workspace=ws,
                          topk_ids=topk_ids, topk_vals=topk_vals)
        if p_min is None:
            model.select_path(d_anchors, topk_ids, topk_vals, path_idx=path, draft_tokens=drafts,
                              want_score=False)
        else:
            model.select_path_stop(d_anchors, topk_ids, topk_vals, p_min=p_min, n_min=n_min, n_max=n_max,
                                   path_idx=path, draft_tokens=drafts, draft_lens=lens)
        h_drafts = drafts.cpu().numpy()
        tl = torch.from_numpy(np.ascontiguousarray(target_logits(s, h_drafts))).to(dev)
        if sampling is None:
            if p_min is None:
                verify_accept(drafts, tl, workspace=vws, accepted=accepted, bonus=bonus)
            else:
                verify_sample(drafts, tl, None, 0.0, draft_lens=lens, workspace=vws, accepted=accepted,
                              bonus=bonus)
        else:
            u = torch.from_numpy(np.ascontiguousarray(uniforms(s), dtype=np.float32)).to(dev)
            verify_sample(drafts, tl, u, *sampling, draft_lens=lens, workspace=vws, accepted=accepted,
                          bonus=bonus)
        a = accepted.cpu().numpy()
        rec["drafts"].append(h_drafts)
        rec["lens"].append(lens.cpu().numpy())
        rec["accepted"].append(a)
        rec["bonus"].append(bonus.cpu().numpy())
        rec["ctx_lens"].append(ctx.copy())
        n_new = a.astype(np.int64) + 1
        taps, offsets = verified_taps(ctx, n_new)
        offsets = np.asarray(offsets, dtype=np.int32)
        ctx = ctx + n_new
        anchors = rec["bonus"][-1].astype(np.int32)
    per_step = np.stack(rec["accepted"]).reshape(-1)
    rec["metrics"] = speculative_metrics(per_step.tolist(), P)
    return rec
