"""GPU decode loop (block_speculative_decoding_dflash2_amd.decode) against
the oracle's loop on the same seeded target: several rounds with the
context, anchor and appended taps carried over."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from _gpu_common import log

pytestmark = pytest.mark.gpu

STEPS = 4


def _run(w, **kw):
    from block_speculative_decoding_dflash2_amd import DFlash2
    from block_speculative_decoding_dflash2_amd.decode import decode_loop
    W = synth.make_weights(w)
    inp = synth.make_step_inputs(w)
    tl = lambda s, d: synth.make_target_logits(w, d, tag=1000 + s)
    vt = lambda starts, counts: synth.make_verified_taps(w, starts, counts)
    model = DFlash2(w.abi_config(), W)
    uni = lambda s: synth.make_uniforms((w.batch, w.block_size), tag=500 + s)
    okw = dict(kw)
    if "sampling" in kw:
        kw = dict(kw, uniforms=uni)
        okw = dict(okw, uniforms_fn=uni)
    try:
        kc, vc = model.new_caches()
        model.load_context(kc, vc, inp.k_ctx, inp.v_ctx)
        g = decode_loop(model, kc, vc, inp.anchors, inp.ctx_lens, inp.taps, inp.new_offsets, STEPS, tl, vt, **kw)
        torch.cuda.synchronize()
    finally:
        model.close()
    o = O.decode_loop(w, W, inp, STEPS, tl, vt, **okw)
    return g, o, tl


@pytest.mark.parametrize("name", ["tiny_fp32", "small_fp32"])
def test_decode_loop_fp32_trajectory(name):
    """fp32 logits agree with the oracle to ~1e-6, so the whole trajectory
    (drafts, accepted counts, bonus tokens, context lengths) is identical."""
    w = synth.get(name).replace(spare_context=STEPS * 8)
    g, o, _ = _run(w)
    for s in range(STEPS):
        log(f"{name} round {s}: accepted {g['accepted'][s].tolist()} (oracle {o['accepted'][s].tolist()})")
        assert np.array_equal(g["ctx_lens"][s], o["ctx_lens"][s])
        assert np.array_equal(g["drafts"][s], o["drafts"][s])
        assert np.array_equal(g["accepted"][s], o["accepted"][s])
        assert np.array_equal(g["bonus"][s], o["bonus"][s])
    log(f"{name}: {g['metrics']}")


@pytest.mark.parametrize("name", ["small_bf16", "medium_fp8"])
def test_decode_loop_bookkeeping(name):
    """bf16/fp8 drafts may differ from the oracle's at near-ties, so each
    round is checked on its own terms: verification of the GPU's drafts
    against the same target logits matches the oracle's verification
    exactly, and the context advances by accepted + 1."""
    w = synth.get(name).replace(spare_context=STEPS * 8)
    g, o, tl = _run(w)
    for s in range(STEPS):
        want = O.verify_accept(g["drafts"][s], tl(s, g["drafts"][s]))
        assert np.array_equal(g["accepted"][s], want["accepted"])
        assert np.array_equal(g["bonus"][s], want["bonus"])
        if s + 1 < STEPS:
            assert np.array_equal(g["ctx_lens"][s + 1], g["ctx_lens"][s] + g["accepted"][s] + 1)
    agree = np.mean([np.mean(g["drafts"][s] == o["drafts"][s]) for s in range(STEPS)])
    log(f"{name}: draft agreement with the oracle's loop {agree:.3f}; {g['metrics']}")


@pytest.mark.parametrize("name", ["tiny_fp32", "small_fp32"])
@pytest.mark.parametrize("kw", [dict(sampling=(1.0, 20, 0.95)), dict(p_min=0.2),
                                dict(sampling=(0.8, 0, 0.9), p_min=0.1, n_min=1)],
                         ids=["sampled", "p_min", "sampled_p_min"])
def test_decode_loop_fp32_sampled_trajectory(name, kw):
    """With rejection sampling and / or the confidence stop the fp32
    trajectory still follows the oracle's round for round, until a round
    with a sampled decision within the rounding allowance of its threshold
    (the rest may then legitimately diverge)."""
    from test_gpu_sampled import band
    w = synth.get(name).replace(spare_context=STEPS * 8)
    g, o, _ = _run(w, **kw)
    for s in range(STEPS):
        log(f"{name} {kw} round {s}: lens {g['lens'][s].tolist()} accepted {g['accepted'][s].tolist()} "
            f"(oracle {o['lens'][s].tolist()} / {o['accepted'][s].tolist()})")
        assert np.array_equal(g["ctx_lens"][s], o["ctx_lens"][s])
        assert np.array_equal(g["drafts"][s], o["drafts"][s])
        assert np.array_equal(g["lens"][s], o["lens"][s])
        if np.min(o["margin"][s]) <= band(w.vocab):
            log("  a decision lies within the allowance: later rounds not compared")
            break
        assert np.array_equal(g["accepted"][s], o["accepted"][s])
        assert np.array_equal(g["bonus"][s], o["bonus"][s])
