"""Speculative-decoding acceptance metrics (NVIDIA NIM for Alpamayo,
"DFlash2 Speculative Decoding", section "Observe Acceptance", metrics
fields table): drafts proposed per step, steps, drafted and accepted
totals, acceptance rate = accepted / drafted, mean acceptance length =
1 + accepted / steps (the verified token counts), a histogram of accepted
drafts per step over 0..num_spec_tokens, and the acceptance rate by draft
position (the fraction of steps whose draft i was accepted)."""
from __future__ import annotations

from typing import Dict, Iterable, List


def speculative_metrics(per_step_accepted: Iterable[int], num_spec_tokens: int) -> Dict:
    acc: List[int] = [int(a) for a in per_step_accepted]
    steps = len(acc)
    drafted = steps * num_spec_tokens
    accepted = sum(acc)
    hist = [0] * (num_spec_tokens + 1)
    for a in acc:
        if not 0 <= a <= num_spec_tokens:
            raise ValueError(f"accepted count {a} outside 0..{num_spec_tokens}")
        hist[a] += 1
    return {
        "num_spec_tokens": num_spec_tokens,
        "num_spec_steps": steps,
        "num_draft_tokens": drafted,
        "num_accepted_draft_tokens": accepted,
        "draft_acceptance_rate": accepted / drafted if drafted else 0.0,
        "mean_acceptance_length": 1.0 + accepted / steps if steps else 0.0,
        "acceptance_histogram": hist,
        "acceptance_by_position": [sum(1 for a in acc if a > i) / steps if steps else 0.0
                                   for i in range(num_spec_tokens)],
    }
