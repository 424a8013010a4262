"""Pins for sampled (rejection) verification, the target's truncated
distribution, the selector's transition confidence and the draft-length
rule: hand-worked distributions, the lossless property measured by
integrating the oracle's decisions over a grid of uniforms, reductions to
the greedy rule (temperature 0, top-k 1, vanishing temperature) and
hand-worked confidence cases."""
import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _parse(tok: str) -> float:
    table = {"ln4": math.log(4.0), "ln3": math.log(3.0), "ln2": math.log(2.0), "inf": math.inf,
             "-inf": -math.inf, "nan": math.nan, "-0.0": -0.0}
    return table[tok] if tok in table else float(tok)


def _gold_cases():
    with open(os.path.join(GOLD, "sampled_hand.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _gold_cases(), ids=lambda c: c["note"][:40])
def test_target_distribution_hand_cases(case):
    z = np.array([_parse(t) for t in case["logits"]], dtype=np.float32)
    p = O.target_distribution(z, case["temperature"], case["top_k"], case["top_p"])
    np.testing.assert_allclose(p, case["p"], atol=1e-6, rtol=0)
    assert abs(p.sum() - 1.0) < 1e-12


def _rows(rng, V, n, spread=1.5):
    return (rng.standard_normal((n, V)) * spread).astype(np.float32)


SETTINGS = [(1.0, 0, 1.0), (1.0, 20, 0.95), (0.7, 3, 1.0), (1.3, 0, 0.8), (1.0, 4, 0.6)]


@pytest.mark.parametrize("T,top_k,top_p", SETTINGS)
def test_rejection_step_is_lossless(T, top_k, top_p):
    """For every draft token d and row, P(emit d by acceptance) + P(reject) *
    residual must equal the target's distribution.  Both measures come from
    the oracle's own decisions evaluated on a midpoint grid of uniforms (a
    wrong inequality, a residual that keeps d or forgets to renormalise, or a
    draw from the wrong row fails it)."""
    rng = np.random.default_rng(7)
    V, N = 7, 2000
    z = _rows(rng, V, 2)
    grid = (np.arange(N) + 0.5) / N
    for d in range(V):
        p0 = O.target_distribution(z[0], T, top_k, top_p)
        # acceptance measure over u_0 (v irrelevant)
        uni = np.stack([grid, np.full(N, 0.5)], axis=1).astype(np.float32)
        drafts = np.full((N, 1), d, dtype=np.int32)
        logits = np.broadcast_to(z[None], (N, 2, V))
        r = O.verify_sample(drafts, logits, uni, T, top_k, top_p)
        acc = r["accepted"].mean()
        assert abs(acc - p0[d]) <= 1.0 / N + 1e-12
        emitted = np.zeros(V)
        emitted[d] += acc
        if p0[d] < 1.0 - 1e-12:
            # residual measure over v, with u_0 forcing a rejection
            uni = np.stack([np.full(N, np.nextafter(np.float32(1), np.float32(0))), grid],
                           axis=1).astype(np.float32)
            r = O.verify_sample(drafts, logits, uni, T, top_k, top_p)
            assert np.all(r["accepted"] == 0)
            assert not np.any(r["bonus"] == d)
            hist = np.bincount(r["bonus"], minlength=V) / N
            emitted += (1.0 - acc) * hist
        np.testing.assert_allclose(emitted, p0, atol=(V + 2) / N)


@pytest.mark.parametrize("T,top_k,top_p", SETTINGS)
def test_all_accepted_bonus_follows_last_row(T, top_k, top_p):
    rng = np.random.default_rng(11)
    V, N, bs = 9, 3000, 3
    z = _rows(rng, V, bs)
    grid = (np.arange(N) + 0.5) / N
    # drafts = the target's most likely token, accepted for u = 0
    drafts = np.array([[int(np.argmax(z[0])), int(np.argmax(z[1]))]] * N, dtype=np.int32)
    uni = np.stack([np.zeros(N), np.zeros(N), grid], axis=1).astype(np.float32)
    r = O.verify_sample(drafts, np.broadcast_to(z[None], (N, bs, V)), uni, T, top_k, top_p)
    assert np.all(r["accepted"] == 2)
    hist = np.bincount(r["bonus"], minlength=V) / N
    np.testing.assert_allclose(hist, O.target_distribution(z[2], T, top_k, top_p), atol=(V + 1) / N)


def test_top_k_one_is_greedy():
    rng = np.random.default_rng(3)
    B, bs, V = 64, 6, 50
    z = _rows(rng, B * bs, V).reshape(B, bs, V)
    g = np.argmax(z, axis=2)
    drafts = np.where(rng.random((B, bs - 1)) < 0.8, g[:, :-1], rng.integers(0, V, (B, bs - 1))).astype(np.int32)
    uni = rng.random((B, bs)).astype(np.float32)
    for top_p in (1.0, 0.3):
        r = O.verify_sample(drafts, z, uni, 1.0, 1, top_p)
        want = O.verify_accept(drafts, z)
        np.testing.assert_array_equal(r["accepted"], want["accepted"])
        np.testing.assert_array_equal(r["bonus"], want["bonus"])


def test_temperature_zero_and_its_limit_are_greedy():
    rng = np.random.default_rng(4)
    B, bs, V = 48, 5, 40
    # well separated values: gaps of at least 0.25
    z = np.stack([rng.permutation(V) for _ in range(B * bs)]).astype(np.float32).reshape(B, bs, V) * 0.25
    g = np.argmax(z, axis=2)
    drafts = np.where(rng.random((B, bs - 1)) < 0.7, g[:, :-1], rng.integers(0, V, (B, bs - 1))).astype(np.int32)
    uni = (1e-4 + (1 - 2e-4) * rng.random((B, bs))).astype(np.float32)
    want = O.verify_accept(drafts, z)
    for T in (0.0, 1e-3):
        r = O.verify_sample(drafts, z, uni, T, 0, 1.0)
        np.testing.assert_array_equal(r["accepted"], want["accepted"])
        np.testing.assert_array_equal(r["bonus"], want["bonus"])


def test_draft_lens_cut_the_path():
    rng = np.random.default_rng(5)
    B, bs, V = 32, 6, 30
    z = _rows(rng, B * bs, V).reshape(B, bs, V)
    g = np.argmax(z, axis=2)
    drafts = g[:, :-1].astype(np.int32)                       # all agree greedily
    lens = rng.integers(0, bs, B).astype(np.int32)
    w = O.verify_accept_len(drafts, z, lens)
    np.testing.assert_array_equal(w["accepted"], lens)
    np.testing.assert_array_equal(w["bonus"], g[np.arange(B), lens])
    full = O.verify_accept_len(drafts, z, np.full(B, bs - 1))
    np.testing.assert_array_equal(full["accepted"], O.verify_accept(drafts, z)["accepted"])
    # sampled: a length-0 path draws the bonus from row 0's full distribution
    uni = rng.random((B, bs)).astype(np.float32)
    r = O.verify_sample(drafts, z, uni, 1.0, 0, 1.0, draft_lens=np.zeros(B, dtype=np.int32))
    assert np.all(r["accepted"] == 0)
    for b in range(B):
        assert r["bonus"][b] == O.inverse_cdf(O.target_distribution(z[b, 0], 1.0), uni[b, bs - 1])
    r = O.verify_sample(drafts, z, uni, 1.0, 0, 1.0, draft_lens=lens)
    assert np.all(r["accepted"] <= lens)
    assert np.all(r["draft_prob"][np.arange(bs - 1)[None, :] >= lens[:, None]] == 0)


def test_inverse_cdf_hand_cases():
    p = np.array([0.0, 0.25, 0.0, 0.5, 0.25])
    assert O.inverse_cdf(p, 0.0) == 1
    assert O.inverse_cdf(p, 0.2499) == 1
    assert O.inverse_cdf(p, 0.25) == 3      # strict: cum 0.25 is not > 0.25
    assert O.inverse_cdf(p, 0.7499) == 3
    assert O.inverse_cdf(p, 0.75) == 4
    assert O.inverse_cdf(p, 1.0) == 3       # out of range: the most likely id


# ------------------------------------------------- selector confidence

def test_path_confidence_hand_cases():
    k, r, V = 3, 4, 10
    tl = np.zeros((V, r), dtype=np.float32)
    tr = np.zeros((V, r), dtype=np.float32)
    ids = np.array([[[1, 2, 3], [4, 5, 6]]], dtype=np.int32)
    # zero tables: scores are the candidate values; weights 3:1:1 -> 3/5
    vals = np.array([[[math.log(3.0), 0.0, 0.0], [0.0, 0.0, 0.0]]], dtype=np.float32)
    sel = O.select_path([0], ids, vals, tl, tr)
    assert sel["path"].tolist() == [[0, 0]]
    conf = O.path_confidence([0], ids, vals, sel["path"], tl, tr)
    np.testing.assert_allclose(conf, [[0.6, 1.0 / 3.0]], rtol=1e-6)
    # the pair term counts: Tl[anchor] . Tr[c] = ln 2 for candidate 2 only
    tl[0, 0] = 1.0
    tr[2, 0] = math.log(2.0)
    vals = np.zeros((1, 2, 3), dtype=np.float32)
    sel = O.select_path([0], ids, vals, tl, tr)
    assert sel["path"][0, 0] == 1                       # candidate id 2 has rank 1
    conf = O.path_confidence([0], ids, vals, sel["path"], tl, tr)
    np.testing.assert_allclose(conf[0, 0], 0.5, rtol=1e-6)   # weights 1:2:1
    # position 1 is scored from the predecessor the path took (id 2):
    # Tl[2] . Tr[5] = ln 3 gives weights 1:3:1 over ids 4, 5, 6
    tl[2, 1] = 1.0
    tr[5, 1] = math.log(3.0)
    sel = O.select_path([0], ids, vals, tl, tr)
    assert sel["path"].tolist() == [[1, 1]]
    conf = O.path_confidence([0], ids, vals, sel["path"], tl, tr)
    np.testing.assert_allclose(conf[0], [0.5, 0.6], rtol=1e-6)


def test_draft_length_rule():
    conf = np.array([[0.9, 0.5, 0.2, 0.9],
                     [0.1, 0.9, 0.9, 0.9],
                     [0.9, 0.9, 0.9, 0.9]])
    assert O.draft_lengths(conf, 0.0).tolist() == [4, 4, 4]
    assert O.draft_lengths(conf, 0.3).tolist() == [2, 0, 4]
    assert O.draft_lengths(conf, 0.6).tolist() == [1, 0, 4]
    assert O.draft_lengths(conf, 0.3, n_min=1).tolist() == [2, 4, 4]
    assert O.draft_lengths(conf, 0.3, n_min=3).tolist() == [4, 4, 4]
    assert O.draft_lengths(conf, 0.3, n_max=1).tolist() == [1, 0, 1]
    assert O.draft_lengths(conf, 0.0, n_max=9).tolist() == [4, 4, 4]
    assert O.draft_lengths(conf, 0.3, n_min=5, n_max=2).tolist() == [2, 2, 2]
    assert O.draft_lengths(conf, 1.0).tolist() == [0, 0, 0]
    # a confidence equal to p_min does not stop the path
    assert O.draft_lengths(np.array([[0.5, 0.25]]), 0.5).tolist() == [1]


def test_distributions_near_the_top_p_bound():
    z = np.array([math.log(4.0), math.log(2.0), 0.0, 0.0, -math.inf], dtype=np.float32)
    assert len(O.target_distributions_near(z, 1.0, 0, 0.7, 0.0)) == 1
    assert len(O.target_distributions_near(z, 1.0, 0, 0.7, 0.01)) == 1      # no group within 0.01
    near = O.target_distributions_near(z, 1.0, 0, 0.751, 0.01)              # the tied pair sits at 0.75
    assert len(near) == 2
    np.testing.assert_allclose(near[0], O.target_distribution(z, 1.0, 0, 0.751), atol=1e-12)
    kept = sorted(int(np.count_nonzero(q)) for q in near)
    assert kept == [2, 4]
    near = O.target_distributions_near(z, 1.0, 0, 0.5, 0.01)                # token 1 sits at 0.5
    assert sorted(int(np.count_nonzero(q)) for q in near) == [1, 2]
    assert len(O.target_distributions_near(z, 0.0, 0, 0.5, 0.5)) == 1         # temperature 0: one answer
