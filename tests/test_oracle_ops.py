"""Pins for the oracle's building blocks: closed forms, hand-worked cases
from tests/golden, and special cases that reduce to library routines."""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_conv_hand_worked():
    g = json.load(open(os.path.join(GOLD, "conv_hand.json")))
    x = np.array(g["x"])[:, None]
    taps = np.array(g["taps"])[:, None]
    assert np.array_equal(O.block_conv(x, taps)[:, 0], np.array(g["expected"]))


def test_conv_matches_numpy_convolve_and_boundaries():
    rng = np.random.default_rng(2)
    bs, H, K = 9, 5, 3
    x = rng.standard_normal((bs, H))
    c = rng.standard_normal((K, H))
    y = O.block_conv(x, c)
    for ch in range(H):
        kern = c[:, ch].copy()
        kern[0] += 1.0                                  # correction form == plain conv with 1 + c0
        ref = np.convolve(x[:, ch], kern)[:bs]
        assert np.allclose(y[:, ch], ref, rtol=0, atol=1e-12)
    assert np.array_equal(O.block_conv(x, np.zeros((K, H))), x)
    x2 = x.copy()
    x2[1:] += 7.0                                       # later slots never reach slot 0
    assert np.array_equal(O.block_conv(x2, c)[0], y[0])


def test_rmsnorm_closed_form_and_torch():
    g = np.array([1.0, 2.0, -0.5, 3.0])
    x = np.full(4, 3.0)
    eps = 1e-6
    assert np.allclose(O.rmsnorm(x, g, eps), g * 3.0 / math.sqrt(9.0 + eps), rtol=1e-15)
    rng = np.random.default_rng(3)
    X = rng.standard_normal((6, 33))
    G = rng.standard_normal(33)
    ref = F.rms_norm(torch.from_numpy(X), (33,), torch.from_numpy(G), eps=eps).numpy()
    assert np.allclose(O.rmsnorm(X, G, eps), ref, rtol=1e-13, atol=1e-13)


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 1001)
    assert np.allclose(O.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-13, atol=1e-300)


def test_rope_identities():
    rng = np.random.default_rng(4)
    d, theta = 16, 1e6
    x = rng.standard_normal((5, 3, d))
    assert np.allclose(O.rope(x, np.zeros(5), theta), x, rtol=0, atol=0)
    p = np.array([0, 1, 7, 4095, 8200])
    y = O.rope(x, p, theta)
    h = d // 2
    assert np.allclose(x[..., :h] ** 2 + x[..., h:] ** 2, y[..., :h] ** 2 + y[..., h:] ** 2, rtol=1e-12)
    p2 = np.array([3, 5, 11, 2, 9])
    assert np.allclose(O.rope(O.rope(x, p, theta), p2, theta), O.rope(x, p + p2, theta), atol=1e-9)
    # frequency of pair i is theta^(-2i/d); pair 0 turns by exactly p radians
    e = np.zeros((1, 1, d))
    e[0, 0, 0] = 1.0
    r = O.rope(e, np.array([2]), theta)
    assert np.isclose(r[0, 0, 0], math.cos(2)) and np.isclose(r[0, 0, h], math.sin(2))
    e2 = np.zeros((1, 1, d))
    e2[0, 0, 3] = 1.0
    ang = 2 * theta ** (-6.0 / d)
    r2 = O.rope(e2, np.array([2]), theta)
    assert np.isclose(r2[0, 0, 3], math.cos(ang)) and np.isclose(r2[0, 0, 3 + h], math.sin(ang))


def test_attention_matches_torch_sdpa_gqa():
    rng = np.random.default_rng(5)
    T, S, nq, nkv, d = 7, 23, 8, 2, 16
    q = rng.standard_normal((T, nq, d))
    k = rng.standard_normal((S, nkv, d))
    v = rng.standard_normal((S, nkv, d))
    out = O.attention(q, k, v)
    tq = torch.from_numpy(q).permute(1, 0, 2)                      # [nq, T, d]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(nq // nkv, dim=0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(nq // nkv, dim=0)
    ref = F.scaled_dot_product_attention(tq, tk, tv).permute(1, 0, 2).numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_attention_single_key_returns_value():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 4, 8))
    k = rng.standard_normal((1, 2, 8))
    v = rng.standard_normal((1, 2, 8))
    out = O.attention(q, k, v)
    assert np.allclose(out[0, 0], v[0, 0]) and np.allclose(out[0, 3], v[0, 1])


def test_linear_chunking_is_exact():
    from synth.generate import encode
    rng = np.random.default_rng(7)
    w = encode(rng.standard_normal((37, 19)).astype(np.float32), "bf16")
    x = rng.standard_normal((3, 19))
    a = O.linear(x, w, chunk_elems=19 * 5)
    b = O.linear(x, w)
    ref = x @ O.bf16_bits_to_f64(w.data).T
    assert np.allclose(a, ref, rtol=1e-14) and np.allclose(b, ref, rtol=1e-14)
    assert np.allclose(O.linear(x, w, rows=(4, 11)), ref[:, 4:11], rtol=1e-14)


def test_logit_transform():
    x = np.linspace(-50, 50, 101)
    assert np.array_equal(O.logit_transform(x, 1.0, 0.0), x)
    y = O.logit_transform(x, 0.5, 10.0)
    assert np.all(np.abs(y) < 10.0) and np.allclose(y, -O.logit_transform(-x, 0.5, 10.0))
    assert np.all(np.diff(y) > 0)
    assert np.isclose(O.logit_transform(np.array([1e-4]), 0.5, 10.0)[0], 0.5e-4, rtol=1e-8)
    # multiplier first, then the cap: 0.5 * 20 = 10 -> 10 tanh(1); large inputs
    # saturate at the cap itself, not at multiplier * cap
    assert np.isclose(O.logit_transform(np.array([20.0]), 0.5, 10.0)[0], 10.0 * math.tanh(1.0), rtol=1e-14)
    assert np.isclose(O.logit_transform(np.array([1e4]), 0.5, 10.0)[0], 10.0, rtol=1e-14)


# ------------------------------------------------- dynamic convolution

def _fp32_tensor(a):
    return synth.Tensor(np.asarray(a, dtype=np.float32), "fp32")


def test_dynamic_conv_hand_case():
    """H = 2, one channel per group, two taps: row g*K + j of W is tap j of
    group g.  W picks x_t[0] as group 0's own-slot tap and x_t[1] as group
    1's previous-slot tap."""
    x = np.array([[1.0, 2.0], [3.0, 4.0]])
    W = _fp32_tensor([[1, 0], [0, 0], [0, 0], [0, 1]])
    y = O.dynamic_block_conv(x, W, kernel=2, group=1)
    np.testing.assert_array_equal(y, [[2.0, 2.0], [12.0, 12.0]])


def test_dynamic_conv_taps_are_shared_by_a_group():
    x = np.array([[1.0, 1.0, 2.0, 3.0]])
    W = np.zeros((4, 4), dtype=np.float32)
    W[2, 2] = 1.0                        # group 1 (channels 2, 3), tap 0 = x_t[2]
    y = O.dynamic_block_conv(x, _fp32_tensor(W), kernel=2, group=2)
    np.testing.assert_array_equal(y, [[1.0, 1.0, 6.0, 9.0]])


def test_dynamic_conv_identity_and_causality():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 8))
    assert np.array_equal(O.dynamic_block_conv(x, _fp32_tensor(np.zeros((12, 8))), 3, 2), x)
    W = _fp32_tensor(rng.standard_normal((12, 8)) * 0.1)
    y = O.dynamic_block_conv(x, W, 3, 2)
    x2 = x.copy()
    x2[3] += 1.0                          # a later slot never reaches back
    y2 = O.dynamic_block_conv(x2, W, 3, 2)
    np.testing.assert_array_equal(y[:3], y2[:3])
    assert not np.allclose(y[3:], y2[3:])
