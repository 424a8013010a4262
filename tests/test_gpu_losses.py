"""GPU parity of the forward training losses (dflash2_draft_losses) against
the oracle on the same seeded logits, labels and candidates: per-slot block
and selector cross-entropies (float32 logsumexp against float64), the
unsupervised / missing-candidate patterns (exact) and the four totals."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from _gpu_common import log

pytestmark = pytest.mark.gpu


def _inputs(w, tag):
    B, P, V, k = w.batch, w.block_size - 1, w.vocab, w.top_k
    sel = synth.make_selector_inputs(w, tag=tag)
    z = synth.normal((B, P, V), (w.index, 4000, tag), std=2.0)
    rng = np.random.default_rng([tag, B, P, V])
    pick = rng.integers(0, k, (B, P))
    labels = np.where(rng.random((B, P)) < 0.7, np.take_along_axis(sel["ids"], pick[..., None], 2)[..., 0],
                      rng.integers(0, V, (B, P))).astype(np.int32)
    labels[rng.random((B, P)) < 0.1] = -1            # unsupervised slots
    return sel, z, labels


CASES = [("tiny_fp32", {}), ("small_bf16", {}), ("small_fp8", {}),
         ("small_bf16", dict(output_multiplier=0.5, final_logit_softcapping=30.0)),
         ("dense27b_bf16", {}), ("batched_bf16", {}), ("fp8_b256", {}),
         # 70000 supervised rows: more row blocks than a grid's y or z axis holds
         ("tiny_fp32", dict(batch=70000, block_size=2, vocab=64))]
CASE_IDS = ["tiny_fp32", "small_bf16", "small_fp8", "small_bf16_softcap", "dense27b_bf16", "batched_bf16",
            "fp8_b256", "tiny_fp32_70000_rows"]


@pytest.mark.parametrize("name,over", CASES, ids=CASE_IDS)
def test_losses_match_oracle(name, over):
    from test_gpu_verify_select import _select_model
    w = synth.get(name).replace(selector_active=True, **over)
    log(f"losses {name} {over} B={w.batch} P={w.block_size - 1} V={w.vocab}")
    tl, tr = synth.make_selector_tables(w)
    sel, z, labels = _inputs(w, tag=31)
    gamma, wsel = 4.0, 0.3
    want = O.block_losses(sel["anchors"], labels, z, sel["ids"], sel["vals"], tl, tr, gamma, wsel,
                          w.output_multiplier, w.final_logit_softcapping)
    m = _select_model(w, tl, tr)
    try:
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        got = m.draft_losses(t(sel["anchors"]), t(labels), t(z), t(sel["ids"]), t(sel["vals"]), gamma, wsel,
                             want_per_slot=True)
        torch.cuda.synchronize()
        bce, sce = got["block_ce"].cpu().numpy(), got["selector_ce"].cpu().numpy()
        losses = got["losses"].cpu().numpy()
    finally:
        m.close()
    assert np.array_equal(np.isnan(bce), np.isnan(want["block_ce"]))
    assert np.array_equal(np.isnan(sce), np.isnan(want["selector_ce"]))
    ok = ~np.isnan(want["block_ce"])
    err = np.abs(bce[ok] - want["block_ce"][ok])
    assert np.all(err <= 2e-5 + 2e-6 * np.abs(want["block_ce"][ok])), err.max()
    ok = ~np.isnan(want["selector_ce"])
    err_s = np.abs(sce[ok] - want["selector_ce"][ok])
    assert np.all(err_s <= 2e-5 + 2e-6 * np.abs(want["selector_ce"][ok])), err_s.max()
    ref = np.array([want["total"], want["block"], want["selector"], want["recall"]])
    np.testing.assert_allclose(losses, ref, rtol=2e-6, atol=2e-6)
    log(f"  losses {losses.tolist()} (oracle {ref.tolist()}), max CE err {err.max():.2e}, "
        f"selector slots {int(ok.sum())}")


def test_losses_edge_cases():
    """No supervised slot, equal weights (gamma = inf), -inf logits and a
    candidate list missing every label."""
    from test_gpu_verify_select import _select_model
    w = synth.get("small_bf16").replace(selector_active=True)
    tl, tr = synth.make_selector_tables(w)
    sel, z, labels = _inputs(w, tag=32)
    z[0, 0, ::2] = -np.inf
    m = _select_model(w, tl, tr)
    try:
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        for lab, gamma in [(np.full_like(labels, -1), 4.0), (labels, float("inf")),
                           (np.where(labels >= 0, (labels + 1) % w.vocab, labels), 2.0)]:
            ids = sel["ids"] if lab is not labels else sel["ids"]
            want = O.block_losses(sel["anchors"], lab, z, ids, sel["vals"], tl, tr, gamma, 0.5)
            got = m.draft_losses(t(sel["anchors"]), t(lab.astype(np.int32)), t(z), t(ids), t(sel["vals"]),
                                 gamma, 0.5)
            torch.cuda.synchronize()
            ref = np.array([want["total"], want["block"], want["selector"], want["recall"]])
            np.testing.assert_allclose(got["losses"].cpu().numpy(), ref, rtol=2e-6, atol=2e-6)
    finally:
        m.close()
