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


def test_sampled_loop_at_vanishing_temperature_is_the_greedy_loop():
    """Planted argmaxes stand a full logit above the rest, so at temperature
    1e-3 each row is a point mass on its argmax and the sampled loop must
    follow the greedy loop round for round."""
    w = TINY_FP32.replace(batch=2, agree=("const", 0.6), spare_context=STEPS * 8)
    W, inp, greedy = _loop(w)
    sampled = O.decode_loop(w, W, inp, STEPS,
                            lambda s, d: synth.make_target_logits(w, d, tag=1000 + s),
                            lambda starts, counts: synth.make_verified_taps(w, starts, counts),
                            sampling=(1e-3, 0, 1.0),
                            uniforms_fn=lambda s: synth.make_uniforms((w.batch, w.block_size), tag=s))
    for s in range(STEPS):
        for k in ("drafts", "accepted", "bonus", "ctx_lens"):
            assert np.array_equal(sampled[k][s], greedy[k][s]), (k, s)


def test_p_min_one_cuts_every_path_to_n_min():
    """p_min = 1 stops at the first position allowed (a confidence is below 1
    unless one candidate takes all the mass), so every round proposes n_min
    drafts and the context grows by at most n_min + 1."""
    w = TINY_FP32.replace(batch=2, agree=("const", 1.0), spare_context=STEPS * 8)
    W = synth.make_weights(w)
    inp = synth.make_step_inputs(w)
    rec = O.decode_loop(w, W, inp, STEPS,
                        lambda s, d: synth.make_target_logits(w, d, tag=1000 + s),
                        lambda starts, counts: synth.make_verified_taps(w, starts, counts),
                        p_min=1.0, n_min=2)
    for s in range(STEPS):
        assert np.all(rec["lens"][s] == 2)
        assert np.all(rec["accepted"][s] == 2)          # the target agrees with every draft
        if s + 1 < STEPS:
            assert np.array_equal(rec["ctx_lens"][s + 1], rec["ctx_lens"][s] + 3)
