"""Pins for ranking, the path selector and verification: brute force on
small inputs (full sorts, exhaustive path enumeration in independent
pure-Python float32 arithmetic), the DFlash v1 special case, hand-worked
verification cases and the closed-form expected acceptance length."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle as O
import synth
from synth.configs import TINY_FP32, DENSE27B_BF16, BATCHED_BF16, LONGBLOCK_BF16, FP8_B256

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def f32(x: float) -> float:
    """Round a Python float (binary64) to the nearest binary32 value."""
    return float(np.float32(x))


# ---------------------------------------------------------------- top-k

@pytest.mark.parametrize("seed", range(4))
def test_topk_matches_full_sort(seed):
    rng = np.random.default_rng(seed)
    R, V, k = 5, 300, 16
    x = rng.integers(-4, 5, size=(R, V)).astype(np.float32) * np.float32(0.5)   # many ties
    x[0, :40] = -0.0
    x[0, 40:80] = 0.0
    x[1] = rng.standard_normal(V).astype(np.float32)
    ids, vals = O.topk(x, k)
    for r in range(R):
        keyed = [(0.0 if x[r, i] == 0 else float(x[r, i]), i) for i in range(V)]
        best = sorted(keyed, key=lambda t: (-t[0], t[1]))[:k]
        assert [i for _, i in best] == ids[r].tolist()
        assert [v for v, _ in best] == vals[r].tolist()


def test_topk_minus_zero_ties_like_plus_zero():
    x = np.zeros((1, 10), dtype=np.float32)
    x[0, 2] = -0.0
    x[0, 0] = -1.0
    ids, vals = O.topk(x, 3)
    assert ids[0].tolist() == [1, 2, 3]
    assert not np.signbit(vals).any()


# ---------------------------------------------------------------- selector

def _pair_py(tl, tr, a, b):
    acc = 0.0
    for m in range(tl.shape[1]):
        acc = f32(acc + f32(float(tl[a, m]) * float(tr[b, m])))
    return acc


def _brute_force(anchor, ids, vals, tl, tr):
    """All k^P paths, left-fold float32 sums in the dynamic program's order:
    acc = pi(c0, c1) + z1; then acc = (acc + pi(c_{t-1}, c_t)) + z_t."""
    P, k = ids.shape
    pi0 = [_pair_py(tl, tr, anchor, int(ids[0, j])) for j in range(k)]
    pit = [[[_pair_py(tl, tr, int(ids[t - 1, i]), int(ids[t, j])) for j in range(k)]
            for i in range(k)] for t in range(1, P)]
    best, best_paths = None, []
    for path in itertools.product(range(k), repeat=P):
        acc = f32(pi0[path[0]] + float(vals[0, path[0]]))
        for t in range(1, P):
            acc = f32(f32(acc + pit[t - 1][path[t - 1]][path[t]]) + float(vals[t, path[t]]))
        if best is None or acc > best:
            best, best_paths = acc, [path]
        elif acc == best:
            best_paths.append(path)
    return best, best_paths


def _left_fold(anchor, ids, vals, tl, tr, path):
    acc = f32(_pair_py(tl, tr, anchor, int(ids[0, path[0]])) + float(vals[0, path[0]]))
    for t in range(1, len(path)):
        acc = f32(f32(acc + _pair_py(tl, tr, int(ids[t - 1, path[t - 1]]), int(ids[t, path[t]])))
                  + float(vals[t, path[t]]))
    return acc


@pytest.mark.parametrize("tag", range(3))
def test_selector_equals_exhaustive_search_tiny(tag):
    """C1 shapes: k = 4, 7 positions -> 4^7 = 16384 paths (selector-active tables)."""
    w = TINY_FP32.replace(selector_active=True)
    W = synth.make_weights(w)
    inp = synth.make_selector_inputs(w, tag=tag)
    tl, tr = W.sel_tl.data, W.sel_tr.data
    out = O.select_path(inp["anchors"], inp["ids"], inp["vals"], tl, tr)
    best, paths = _brute_force(int(inp["anchors"][0]), inp["ids"][0], inp["vals"][0], tl, tr)
    assert float(out["score"][0]) == best
    got = tuple(out["path"][0].tolist())
    assert got in paths
    assert _left_fold(int(inp["anchors"][0]), inp["ids"][0], inp["vals"][0], tl, tr, got) == best
    assert out["drafts"][0].tolist() == [int(inp["ids"][0, t, j]) for t, j in enumerate(got)]


@pytest.mark.parametrize("tag", range(4))
def test_selector_tie_rule_integer_lattice(tag):
    """Exact integer arithmetic with many equal-score paths: the dynamic
    program returns the optimal path that is smallest when compared from the
    last position backwards (Q26)."""
    w = TINY_FP32.replace(batch=1)
    inp = synth.make_selector_inputs(w, tag=tag, integer_lattice=True)
    tl, tr = synth.make_integer_tables(w, tag=tag)
    out = O.select_path(inp["anchors"], inp["ids"], inp["vals"], tl, tr)
    best, paths = _brute_force(int(inp["anchors"][0]), inp["ids"][0], inp["vals"][0], tl, tr)
    assert len(paths) > 1                      # the case really has ties
    want = min(paths, key=lambda p: tuple(reversed(p)))
    assert float(out["score"][0]) == best
    assert tuple(out["path"][0].tolist()) == want


def test_selector_v1_special_cases():
    """Without a pair term (zero tables) or with one candidate per position,
    the path is the per-position top-1: DFlash v1 (AutoModel page, Variants
    table: DFlash is the same backbone without the selector)."""
    w = TINY_FP32.replace(batch=3, top_k=6)
    inp = synth.make_selector_inputs(w, tag=9)
    zero = np.zeros((w.vocab, w.rank), dtype=np.float32)
    out = O.select_path(inp["anchors"], inp["ids"], inp["vals"], zero, zero)
    assert np.array_equal(out["path"], np.zeros_like(out["path"]))
    assert np.array_equal(out["drafts"], inp["ids"][:, :, 0])
    W = synth.make_weights(w.replace(selector_active=True))
    out1 = O.select_path(inp["anchors"], inp["ids"][:, :, :1], inp["vals"][:, :, :1],
                         W.sel_tl.data, W.sel_tr.data)
    assert np.array_equal(out1["drafts"], inp["ids"][:, :, 0])


def test_pair_scores_reference_loop():
    rng = np.random.default_rng(11)
    tl = rng.standard_normal((20, 13)).astype(np.float32)
    tr = rng.standard_normal((20, 13)).astype(np.float32)
    a, b = [3, 4, 19], [0, 7]
    p = O.pair_scores(tl, tr, a, b)
    for i, ai in enumerate(a):
        for j, bj in enumerate(b):
            assert float(p[i, j]) == _pair_py(tl, tr, ai, bj)


# ---------------------------------------------------------------- verify

def _logits_with_argmax(g, V, rng):
    B, bs = g.shape
    z = rng.standard_normal((B, bs, V)).astype(np.float32)
    for b in range(B):
        for i in range(bs):
            z[b, i, g[b, i]] = z[b, i].max() + 1
    return z


def test_verify_hand_worked():
    gold = json.load(open(os.path.join(GOLD, "verify_hand.json")))
    rng = np.random.default_rng(12)
    for c in gold["cases"]:
        g = np.array([c["target_argmax"]])
        out = O.verify_accept(np.array([c["drafts"]]), _logits_with_argmax(g, 16, rng))
        assert out["accepted"][0] == c["accepted"] and out["bonus"][0] == c["bonus"]


def test_verify_ties_and_signed_zero():
    z = np.zeros((1, 2, 8), dtype=np.float32)
    z[0, 0, :] = -1
    z[0, 0, 5] = 2.0
    z[0, 0, 3] = 2.0          # tie -> smallest id 3
    z[0, 1, :] = -0.0         # all equal: id 0
    out = O.verify_accept(np.array([[3]]), z)
    assert out["argmax"][0].tolist() == [3, 0] and out["accepted"][0] == 1 and out["bonus"][0] == 0


def test_verify_lossless_property():
    """Emitted tokens (accepted drafts then the bonus) are exactly the
    target's greedy tokens for the first accepted + 1 rows."""
    rng = np.random.default_rng(13)
    B, bs, V = 50, 8, 40
    g = rng.integers(0, V, size=(B, bs))
    drafts = np.where(rng.random((B, bs - 1)) < 0.7, g[:, :-1], rng.integers(0, V, size=(B, bs - 1)))
    out = O.verify_accept(drafts, _logits_with_argmax(g, V, rng))
    for b in range(B):
        n = out["accepted"][b]
        emitted = list(drafts[b, :n]) + [out["bonus"][b]]
        assert emitted == list(g[b, :n + 1])
        assert n == bs - 1 or drafts[b, n] != g[b, n]


@pytest.mark.parametrize("w,expected", [
    (TINY_FP32, 2.141), (DENSE27B_BF16, 3.161), (BATCHED_BF16, 2.466),
    (LONGBLOCK_BF16, 2.594), (FP8_B256, 3.161)])
def test_expected_acceptance_closed_form(w, expected):
    """E[accepted] = sum_m prod_{i<=m} p_i for the synthetic verifier; checked
    by drawing many blocks through the planted-argmax generator and the
    oracle's verification."""
    bs = w.block_size
    p = [w.agreement(m) for m in range(1, bs)]
    closed = sum(np.prod(p[:m]) for m in range(1, bs))
    assert abs(closed - expected) < 1e-3
    small = w.replace(batch=4000, vocab=64)
    rng = np.random.default_rng(14)
    drafts = rng.integers(0, small.vocab, size=(small.batch, bs - 1))
    z = synth.make_target_logits(small, drafts)
    acc = O.verify_accept(drafts, z)["accepted"]
    se = acc.std() / np.sqrt(len(acc))
    assert abs(acc.mean() - closed) < 5 * se + 0.02
