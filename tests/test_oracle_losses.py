"""Pins for the training-side forward losses (position-decayed block
cross-entropy, selector cross-entropy against the true predecessor,
candidate_recall): closed forms on hand-made logits, torch's
cross_entropy on random rows, hand-worked selector cases and the handling
of unsupervised positions."""
import math

import numpy as np
import pytest
import torch

import oracle as O


def _zero_tables(V, r=4):
    return np.zeros((V, r), dtype=np.float32), np.zeros((V, r), dtype=np.float32)


def test_position_weights_closed_form():
    np.testing.assert_allclose(O.position_weights(4, 1.0), [1.0, math.exp(-1), math.exp(-2)], rtol=1e-15)
    np.testing.assert_allclose(O.position_weights(8, 4.0)[3], math.exp(-0.75), rtol=1e-15)
    assert np.all(O.position_weights(6, math.inf) == 1.0)


def test_uniform_logits_give_log_vocab():
    B, P, V, k = 2, 3, 50, 4
    tl, tr = _zero_tables(V)
    ids = np.tile(np.arange(k, dtype=np.int32), (B, P, 1))
    r = O.block_losses(np.zeros(B, np.int32), np.full((B, P), 7), np.zeros((B, P, V), np.float32), ids,
                       np.zeros((B, P, k), np.float32), tl, tr, 4.0, 0.5)
    np.testing.assert_allclose(r["block_ce"], math.log(V), rtol=1e-14)
    assert abs(r["block"] - math.log(V)) < 1e-14
    assert r["recall"] == 0.0 and r["selector"] == 0.0 and r["total"] == r["block"]


def test_weighted_block_loss_hand_case():
    V = 2
    tl, tr = _zero_tables(V)
    z = np.array([[[0.0, 0.0], [math.log(3.0), 0.0]]], dtype=np.float32)
    ids = np.array([[[0, 1], [0, 1]]], dtype=np.int32)
    r = O.block_losses([0], [[1, 0]], z, ids, np.zeros((1, 2, 2), np.float32), tl, tr, 1.0, 0.0)
    ce1 = math.log(4.0) - float(np.float32(math.log(3.0)))
    np.testing.assert_allclose(r["block_ce"][0], [math.log(2.0), ce1], rtol=1e-7)
    want = (math.log(2.0) + math.exp(-1) * ce1) / (1 + math.exp(-1))
    assert abs(r["block"] - want) < 1e-7


def test_block_ce_matches_torch_cross_entropy():
    rng = np.random.default_rng(2)
    B, P, V = 3, 5, 777
    z = (rng.standard_normal((B, P, V)) * 3).astype(np.float32)
    lab = rng.integers(0, V, (B, P))
    tl, tr = _zero_tables(V)
    ids = np.tile(np.arange(4, dtype=np.int32), (B, P, 1))
    r = O.block_losses(np.zeros(B, np.int32), lab, z, ids, np.zeros((B, P, 4), np.float32), tl, tr, 3.0, 0.0)
    ref = torch.nn.functional.cross_entropy(torch.from_numpy(z).double().reshape(-1, V),
                                            torch.from_numpy(lab).reshape(-1), reduction="none")
    np.testing.assert_allclose(r["block_ce"].reshape(-1), ref.numpy(), rtol=1e-12)
    w = O.position_weights(P + 1, 3.0)
    ref_loss = float((ref.reshape(B, P).numpy() * w).sum() / (B * w.sum()))
    assert abs(r["block"] - ref_loss) < 1e-12


def test_softcap_transform_enters_the_loss():
    V = 3
    tl, tr = _zero_tables(V)
    z = np.array([[[0.0, 100.0, -100.0]]], dtype=np.float32)
    ids = np.array([[[1, 0]]], dtype=np.int32)
    r = O.block_losses([0], [[0]], z, ids, np.zeros((1, 1, 2), np.float32), tl, tr, 1.0, 0.0,
                       multiplier=0.5, softcap=2.0)
    t = [0.0, 2.0 * math.tanh(25.0), 2.0 * math.tanh(-25.0)]
    lse = math.log(sum(math.exp(x) for x in t))
    assert abs(r["block_ce"][0, 0] - (lse - t[0])) < 1e-12


def test_selector_ce_hand_cases():
    V = 10
    tl, tr = _zero_tables(V)
    ids = np.array([[[1, 2, 3], [4, 5, 6]]], dtype=np.int32)
    vals = np.array([[[math.log(3.0), 0.0, 0.0], [0.0, 0.0, 0.0]]], dtype=np.float32)
    z = np.zeros((1, 2, V), np.float32)
    r = O.block_losses([0], [[1, 5]], z, ids, vals, tl, tr, 4.0, 0.25)
    # slot 1: weights 3:1:1, the label is the first candidate
    np.testing.assert_allclose(r["selector_ce"][0], [-math.log(0.6), math.log(3.0)], rtol=1e-6)
    # the pair term is scored from the TRUE predecessor (label 1 at slot 1,
    # not the first-ranked candidate): Tl[1] . Tr[5] = ln 2
    tl[1, 0] = 1.0
    tr[5, 0] = math.log(2.0)
    r2 = O.block_losses([0], [[2, 5]], z, ids, vals, tl, tr, 4.0, 0.25)
    assert abs(r2["selector_ce"][0, 1] - math.log(3.0)) < 1e-6           # predecessor 2: no pair term
    r3 = O.block_losses([0], [[1, 5]], z, ids, vals, tl, tr, 4.0, 0.25)
    assert abs(r3["selector_ce"][0, 1] - math.log(2.0)) < 1e-6           # weights 1:2:1 -> 2/4
    assert abs(r3["selector"] - (-math.log(0.6) + math.log(2.0)) / 2) < 1e-6
    assert abs(r3["total"] - (r3["block"] + 0.25 * r3["selector"])) < 1e-15


def test_recall_and_unsupervised_positions():
    V = 10
    tl, tr = _zero_tables(V)
    ids = np.array([[[1, 2], [3, 4], [5, 6]], [[1, 2], [3, 4], [5, 6]]], dtype=np.int32)
    vals = np.zeros((2, 3, 2), np.float32)
    z = np.zeros((2, 3, V), np.float32)
    labels = np.array([[1, 9, 6], [-1, 3, V]])
    r = O.block_losses([0, 0], labels, z, ids, vals, tl, tr, 2.0, 1.0)
    # supervised: (0,0) hit, (0,1) miss, (0,2) hit, (1,1) hit -> recall 3/4
    assert r["recall"] == 0.75
    assert r["in_cands"].tolist() == [[True, False, True], [False, True, False]]
    # selector signals: (0,0) (anchor), (0,2) (predecessor label 9 is known);
    # (1,1) has an unsupervised predecessor -> no signal
    sig = ~np.isnan(r["selector_ce"])
    assert sig.tolist() == [[True, False, True], [False, False, False]]
    assert np.isnan(r["block_ce"][1, 0]) and np.isnan(r["block_ce"][1, 2])
    np.testing.assert_allclose(r["block"], math.log(V), rtol=1e-14)
    np.testing.assert_allclose(r["selector"], math.log(2.0), rtol=1e-6)
