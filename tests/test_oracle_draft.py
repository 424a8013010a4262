"""Special-case pins of the composed draft forward (context append + block
forward).  The pages print no worked example of a DFlash2 layer, so the
composition is pinned through cases with closed forms and through
invariants the method must have; everything else rests on the pinned
building blocks."""
import copy
import math

import numpy as np
import pytest

import oracle as O
import synth
from synth.configs import TINY_FP32
from synth.generate import encode

W0 = TINY_FP32.replace(batch=2, ctx=(20, 20), cold=False, gain_jitter=0.2)


def _setup(w, seqs=None):
    W = synth.make_weights(w)
    inp = synth.make_step_inputs(w, seqs)
    return W, inp


def _run(w, W, inp):
    B = len(inp.anchors)
    kc, vc = O.new_cache(w, B, inp.k_ctx, inp.v_ctx)
    O.append_context(w, W, kc, vc, inp.taps, inp.new_offsets, inp.ctx_lens)
    out = O.draft_block(w, W, kc, vc, inp.anchors, inp.ctx_lens)
    return out, kc, vc


def _conv2(x, c):
    """y[t] = (1 + c0) x[t] + c1 x[t-1] written out for two taps."""
    y = (1.0 + c[0]) * x
    y[1:] += c[1] * x[:-1]
    return y


def test_zero_sublayer_outputs_leave_conv_chain():
    """With W_o = 0 and W_down = 0 attention and FFN add nothing, so the
    residual stream is the embedding pushed through the 2 * nL block
    convolutions, and the logits are RMSNorm of rows 1.. times lm_head."""
    w = W0.replace(num_layers=2, input_embedding_scale=2.5)
    W, inp = _setup(w)
    for layer in W.layers:
        layer.wo = encode(np.zeros(layer.wo.shape, np.float32), "fp32")
        layer.w_down = encode(np.zeros(layer.w_down.shape, np.float32), "fp32")
    out, _, _ = _run(w, W, inp)
    E = W.embed.data.astype(np.float64)
    for b in range(len(inp.anchors)):
        toks = [int(inp.anchors[b])] + [w.mask_token_id] * (w.block_size - 1)
        h = w.input_embedding_scale * E[toks]
        for layer in W.layers:
            h = _conv2(h, layer.conv_attn.data.astype(np.float64))
            h = _conv2(h, layer.conv_ffn.data.astype(np.float64))
        assert np.allclose(out["h_final"][b], h, rtol=1e-12, atol=1e-15)
        g = W.final_norm.data.astype(np.float64)
        r = h[1:]
        n = r / np.sqrt((r ** 2).mean(axis=1, keepdims=True) + w.rms_eps) * g
        assert np.allclose(out["zeta"][b], n @ W.lm_head.data.astype(np.float64).T, rtol=1e-10, atol=1e-13)


def test_swiglu_gate_half_takes_the_silu():
    """With W_o = 0 and an FFN whose gate row 0 reads 2 n_0, up row 0 reads
    n_0 and W_down writes act_0 back to channel 0 (all else zero), the layer
    adds SiLU(2 n_0) * n_0 to channel 0 and nothing elsewhere (SwiGLU: the
    SiLU acts on the gate half of W_gate_up, the first ffn rows)."""
    w = W0.replace(num_layers=1)
    W, inp = _setup(w)
    layer = W.layers[0]
    H, F = w.hidden, w.ffn
    layer.wo = encode(np.zeros(layer.wo.shape, np.float32), "fp32")
    gu = np.zeros((2 * F, H), np.float32)
    gu[0, 0], gu[F, 0] = 2.0, 1.0
    layer.w_gate_up = encode(gu, "fp32")
    down = np.zeros((H, F), np.float32)
    down[0, 0] = 1.0
    layer.w_down = encode(down, "fp32")
    out, _, _ = _run(w, W, inp)
    E = W.embed.data.astype(np.float64)
    for b in range(len(inp.anchors)):
        toks = [int(inp.anchors[b])] + [w.mask_token_id] * (w.block_size - 1)
        h = _conv2(_conv2(w.input_embedding_scale * E[toks], layer.conv_attn.data.astype(np.float64)),
                   layer.conv_ffn.data.astype(np.float64))
        g = layer.ffn_norm.data.astype(np.float64)
        n0 = (h / np.sqrt((h ** 2).mean(axis=1, keepdims=True) + w.rms_eps) * g)[:, 0]
        want = h.copy()
        want[:, 0] += (2 * n0) / (1 + np.exp(-2 * n0)) * n0
        assert np.allclose(out["h_final"][b], want, rtol=1e-12, atol=1e-14)


def test_only_relative_positions_matter():
    """RoPE makes every attention score depend on position differences only.
    Moving the context and the block 29 positions later (29 other rows are
    appended first and a sliding window of exactly the 12 real rows hides
    them) must leave the logits unchanged up to the float32 rounding of the
    stored keys."""
    L, delta = 12, 29
    w = TINY_FP32.replace(batch=1, ctx=(L, L), cold=True, sliding_window=L, spare_context=40)
    W, inp = _setup(w)
    assert w.max_context >= delta + L + w.block_size
    kc, vc = O.new_cache(w, 1)
    O.append_context(w, W, kc, vc, inp.taps, inp.new_offsets, inp.ctx_lens)
    a = O.draft_block(w, W, kc, vc, inp.anchors, inp.ctx_lens)["zeta"]
    kc2, vc2 = O.new_cache(w, 1)
    other = np.random.default_rng(21).standard_normal((delta, w.num_taps, w.tap_width)).astype(np.float32)
    O.append_context(w, W, kc2, vc2, encode(other, "fp32"), np.array([0, delta]), np.array([delta]))
    O.append_context(w, W, kc2, vc2, inp.taps, np.array([0, L]), np.array([delta + L]))
    b = O.draft_block(w, W, kc2, vc2, inp.anchors, np.array([delta + L]))["zeta"]
    assert np.allclose(a, b, rtol=0, atol=1e-6 * np.abs(a).max())


def test_uniform_attention_averages_all_values():
    """Zero query rows make every score 0, so each head returns the plain
    mean of its kv head's values over all L context rows and all bs block
    rows.  With H = nq*d, W_o = identity and W_down = 0, the residual after
    the layer is conv_ffn(conv_attn(h) + mean values)."""
    w = W0.replace(num_layers=1, hidden=64, num_q_heads=4, num_kv_heads=2, head_dim=16)
    W, inp = _setup(w)
    layer = W.layers[0]
    qkv = layer.wqkv.data.copy()
    qkv[:w.num_q_heads * w.head_dim] = 0.0
    layer.wqkv = encode(qkv, "fp32")
    layer.wo = encode(np.eye(w.hidden, dtype=np.float32), "fp32")
    layer.w_down = encode(np.zeros(layer.w_down.shape, np.float32), "fp32")
    out, kc, vc = _run(w, W, inp)
    nq, nkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
    E = W.embed.data.astype(np.float64)
    for b in range(len(inp.anchors)):
        L = int(inp.ctx_lens[b])
        toks = [int(inp.anchors[b])] + [w.mask_token_id] * (w.block_size - 1)
        h = _conv2(E[toks], layer.conv_attn.data.astype(np.float64))
        g = layer.attn_norm.data.astype(np.float64)
        n = h / np.sqrt((h ** 2).mean(axis=1, keepdims=True) + w.rms_eps) * g
        vrows = qkv[(nq + nkv) * d:].astype(np.float64)            # value projection rows
        vb = (n @ vrows.T).reshape(w.block_size, nkv, d)
        mean = np.zeros(nq * d)
        for i in range(nq):
            grp = i // (nq // nkv)
            allv = np.concatenate([vc[0, b, grp, :L, :], vb[:, grp, :]])
            mean[i * d:(i + 1) * d] = allv.mean(axis=0)
        want = _conv2(h + mean[None, :], layer.conv_ffn.data.astype(np.float64))
        assert np.allclose(out["h_final"][b], want, rtol=1e-10, atol=1e-12)


def test_sequences_are_independent():
    w = W0.replace(batch=3, ctx=(9, 25))
    W, full = _setup(w)
    out_full, _, _ = _run(w, W, full)
    for b in range(3):
        one = synth.make_step_inputs(w, seqs=[b])
        o1, _, _ = _run(w, W, one)
        assert np.allclose(o1["zeta"][0], out_full["zeta"][b], rtol=1e-12, atol=1e-14)


def test_context_order_does_not_matter():
    """No mask and keys carry their positions already: permuting the stored
    context rows (keys with their values) leaves the output unchanged."""
    w = W0.replace(batch=1)
    W, inp = _setup(w)
    B = 1
    kc, vc = O.new_cache(w, B, inp.k_ctx, inp.v_ctx)
    O.append_context(w, W, kc, vc, inp.taps, inp.new_offsets, inp.ctx_lens)
    a = O.draft_block(w, W, kc, vc, inp.anchors, inp.ctx_lens)["zeta"]
    L = int(inp.ctx_lens[0])
    perm = np.random.default_rng(3).permutation(L)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, :, :, :L] = kc[:, :, :, perm]
    vc2[:, :, :, :L] = vc[:, :, :, perm]
    b = O.draft_block(w, W, kc2, vc2, inp.anchors, inp.ctx_lens)["zeta"]
    assert np.allclose(a, b, rtol=1e-11, atol=1e-13)


def test_append_in_two_steps_equals_one():
    """Appending rows in two steps (advancing the context length) writes the
    same cache as appending them at once: the positions of new rows are
    L - n_new .. L - 1 each time."""
    w = W0.replace(batch=1, cold=True, ctx=(12, 12))
    W, inp = _setup(w)
    kc1, vc1 = O.new_cache(w, 1)
    O.append_context(w, W, kc1, vc1, inp.taps, np.array([0, 12]), np.array([12]))
    kc2, vc2 = O.new_cache(w, 1)
    t1 = synth.Tensor(inp.taps.data[:5], "fp32")
    t2 = synth.Tensor(inp.taps.data[5:], "fp32")
    O.append_context(w, W, kc2, vc2, t1, np.array([0, 5]), np.array([5]))
    O.append_context(w, W, kc2, vc2, t2, np.array([0, 7]), np.array([12]))
    assert np.array_equal(kc1, kc2) and np.array_equal(vc1, vc2)


def test_append_position_zero_is_unrotated():
    """At position 0 RoPE is the identity, so the first context key is the
    plain key projection of the normalised projected taps."""
    w = W0.replace(batch=1, cold=True, ctx=(3, 3))
    W, inp = _setup(w)
    kc, vc = O.new_cache(w, 1)
    f = O.append_context(w, W, kc, vc, inp.taps, inp.new_offsets, inp.ctx_lens)
    nq, nkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
    kr = W.layers[0].wqkv.data[nq * d:(nq + nkv) * d].astype(np.float64)
    want = (f[0] @ kr.T).reshape(nkv, d).astype(np.float32).astype(np.float64)
    assert np.array_equal(kc[0, 0, :, 0, :], want)
    u = inp.taps.data.astype(np.float64).reshape(3, -1)
    pre = u @ W.proj.data.astype(np.float64).T
    g = W.proj_norm.data.astype(np.float64)
    assert np.allclose(f, pre / np.sqrt((pre ** 2).mean(1, keepdims=True) + w.rms_eps) * g, rtol=1e-12)


def test_step_runs_tiny_and_is_consistent():
    w = TINY_FP32
    W, inp = _setup(w)
    res = O.step(w, W, inp, lambda d: synth.make_target_logits(w, d))
    P = w.block_size - 1
    assert res["topk_ids"].shape == (1, P, w.top_k)
    # reported values are the logits at the chosen ids, sorted
    z32 = res["zeta"].astype(np.float32)
    for t in range(P):
        ids = res["topk_ids"][0, t]
        assert np.array_equal(res["topk_vals"][0, t], z32[0, t, ids])
        assert np.all(np.diff(res["topk_vals"][0, t]) <= 0)
    assert 0 <= res["accepted"][0] <= P


def test_sliding_window_reaches_back_exactly_w_rows():
    """[AM §Key Config Fields, draft_sliding_window] with window W the block
    attends to context positions L - W .. L - 1 only: rewriting older cache
    rows leaves the logits unchanged, rewriting the oldest row inside the
    window changes them, and W >= L is the same as no window."""
    w = W0.replace(batch=1, ctx=(24, 24))
    W, inp = _setup(w)
    kc, vc = O.new_cache(w, 1, inp.k_ctx, inp.v_ctx)
    O.append_context(w, W, kc, vc, inp.taps, inp.new_offsets, inp.ctx_lens)
    L = int(inp.ctx_lens[0])
    full = O.draft_block(w, W, kc, vc, inp.anchors, inp.ctx_lens)["zeta"]
    assert np.array_equal(full, O.draft_block(w.replace(sliding_window=L), W, kc, vc, inp.anchors,
                                              inp.ctx_lens)["zeta"])
    wl = w.replace(sliding_window=10)
    a = O.draft_block(wl, W, kc, vc, inp.anchors, inp.ctx_lens)["zeta"]
    rng = np.random.default_rng(5)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, :, :, :L - 10] = rng.standard_normal(kc2[:, :, :, :L - 10].shape)
    vc2[:, :, :, :L - 10] = rng.standard_normal(vc2[:, :, :, :L - 10].shape)
    assert np.array_equal(a, O.draft_block(wl, W, kc2, vc2, inp.anchors, inp.ctx_lens)["zeta"])
    kc3 = kc.copy()
    kc3[:, :, :, L - 10] += 1.0
    assert not np.allclose(a, O.draft_block(wl, W, kc3, vc, inp.anchors, inp.ctx_lens)["zeta"])
    assert not np.allclose(a, full)
