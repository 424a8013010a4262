"""Pins of the multi-step decode loop (the steps either side of the path):
closed-form acceptance under a target that always / never agrees with the
drafts, context bookkeeping, and agreement of the loop's first round with
the single-step oracle."""
import numpy as np

import oracle as O
import synth
from block_speculative_decoding_dflash2_amd.metrics import speculative_metrics
from synth.configs import TINY_FP32

STEPS = 3


def _loop(w, steps=STEPS):
    W = synth.make_weights(w)
    inp = synth.make_step_inputs(w)
    rec = O.decode_loop(w, W, inp, steps,
                        lambda s, d: synth.make_target_logits(w, d, tag=1000 + s),
                        lambda starts, counts: synth.make_verified_taps(w, starts, counts))
    return W, inp, rec


def test_always_agreeing_target_accepts_every_draft():
    """Agreement 1: every round accepts all bs-1 drafts, the context grows
    by bs per round and the mean acceptance length is bs."""
    w = TINY_FP32.replace(batch=2, agree=("const", 1.0), spare_context=STEPS * 8)
    _, inp, rec = _loop(w)
    P = w.block_size - 1
    for s in range(STEPS):
        assert np.all(rec["accepted"][s] == P)
        assert np.array_equal(rec["ctx_lens"][s], inp.ctx_lens + s * w.block_size)
    m = speculative_metrics(np.concatenate(rec["accepted"]).tolist(), P)
    assert m["mean_acceptance_length"] == w.block_size
    assert m["acceptance_by_position"] == [1.0] * P


def test_never_agreeing_target_emits_one_token_per_round():
    """Agreement 0: no draft is accepted; the bonus (the target's own token)
    becomes the next anchor and the context grows by one per round."""
    w = TINY_FP32.replace(batch=2, agree=("const", 0.0), spare_context=STEPS * 8)
    _, inp, rec = _loop(w)
    for s in range(STEPS):
        assert np.all(rec["accepted"][s] == 0)
        assert np.array_equal(rec["ctx_lens"][s], inp.ctx_lens + s)
        assert np.all(rec["bonus"][s] != rec["drafts"][s][:, 0])


def test_first_round_is_the_single_step():
    w = TINY_FP32.replace(batch=2, spare_context=STEPS * 8)
    W, inp, rec = _loop(w, steps=1)
    one = O.step(w, W, inp, target_logits_fn=lambda d: synth.make_target_logits(w, d, tag=1000))
    assert np.array_equal(rec["drafts"][0], one["drafts"])
    assert np.array_equal(rec["accepted"][0], one["accepted"])
    assert np.array_equal(rec["bonus"][0], one["bonus"])


def test_acceptance_by_position_matches_histogram():
    m = speculative_metrics([0, 3, 7, 2, 7], 7)
    hist = m["acceptance_histogram"]
    for i, r in enumerate(m["acceptance_by_position"]):
        assert r == sum(hist[i + 1:]) / 5
