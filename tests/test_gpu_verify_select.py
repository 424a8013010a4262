"""GPU parity of dflash2_verify_accept and dflash2_select_path against the
oracle on the same seeded inputs: bit-exact integers (accepted lengths,
bonus tokens, argmaxes, paths, drafts) and bit-exact float32 path scores
and pair scores."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from _gpu_common import log

pytestmark = pytest.mark.gpu

VERIFY_SHAPES = [
    # name, B, bs, V
    ("tiny", 1, 8, 512),
    ("dense27b", 1, 8, 151936),
    ("batched", 64, 7, 131072),
    ("longblock", 16, 16, 151936),
    ("fp8_b256", 256, 8, 151936),
    ("ragged_vocab", 5, 4, 3001),
    ("min_block", 3, 2, 7),
    ("many_rows", 33000, 2, 16),   # 66000 rows: more row blocks than a grid's y axis holds
]


@pytest.mark.parametrize("name,B,bs,V", VERIFY_SHAPES)
def test_verify_matches_oracle(name, B, bs, V):
    from block_speculative_decoding_dflash2_amd import verify_accept
    log(f"verify {name} B={B} bs={bs} V={V}")
    w = synth.TEST_WORKLOADS["small_bf16"].replace(batch=B, block_size=bs, vocab=V, agree=("const", 0.8))
    rng = np.random.default_rng([7, B, bs, V])
    drafts = rng.integers(0, V, size=(B, bs - 1)).astype(np.int32)
    z = synth.make_target_logits(w, drafts, tag=1)
    want = O.verify_accept(drafts, z)
    d = torch.from_numpy(drafts).cuda()
    zt = torch.from_numpy(z).cuda()
    got = verify_accept(d, zt, want_argmax=True)
    torch.cuda.synchronize()
    assert np.array_equal(got["argmax"].cpu().numpy(), want["argmax"])
    assert np.array_equal(got["accepted"].cpu().numpy(), want["accepted"])
    assert np.array_equal(got["bonus"].cpu().numpy(), want["bonus"])


def test_verify_ties_signed_zero_and_full_accept():
    from block_speculative_decoding_dflash2_amd import verify_accept
    B, bs, V = 4, 5, 4096 + 8
    z = np.full((B, bs, V), -1.0, dtype=np.float32)
    z[0, :, 17] = 3.0
    z[0, :, 5] = 3.0                         # ties: smallest id wins
    z[1] = 0.0
    z[1, :, :100] = -0.0                     # -0.0 ranks as +0.0: id 0
    z[2, :, V - 1] = 9.0                     # maximum in the last element
    drafts = np.array([[5, 5, 5, 5], [0, 0, 1, 0], [V - 1] * 4, [1, 2, 3, 4]], dtype=np.int32)
    want = O.verify_accept(drafts, z)
    assert want["accepted"].tolist()[:3] == [4, 2, 4]
    got = verify_accept(torch.from_numpy(drafts).cuda(), torch.from_numpy(z).cuda(), want_argmax=True)
    torch.cuda.synchronize()
    assert np.array_equal(got["argmax"].cpu().numpy(), want["argmax"])
    assert np.array_equal(got["accepted"].cpu().numpy(), want["accepted"])
    assert np.array_equal(got["bonus"].cpu().numpy(), want["bonus"])


SELECT_WORKLOADS = ["tiny_fp32", "dense27b_bf16", "batched_bf16", "longblock_bf16", "fp8_b256",
                    "small_bf16", "small_fp8"]


def _select_model(w, tl, tr):
    """A handle whose only meaningful weights are the selector tables."""
    from block_speculative_decoding_dflash2_amd import DFlash2
    small = w.replace(hidden=32, num_layers=1, num_q_heads=1, num_kv_heads=1, head_dim=32, ffn=32,
                      num_taps=1, tap_width=32, ctx=(8, 8), weight_dtype="bf16")
    W = synth.make_weights(small.replace(vocab=8))
    W.sel_tl = synth.Tensor(tl, "fp32")
    W.sel_tr = synth.Tensor(tr, "fp32")
    cfg = small.abi_config()
    cfg["mask_token_id"] = 0
    return DFlash2(cfg, W)


@pytest.mark.parametrize("name", SELECT_WORKLOADS)
@pytest.mark.parametrize("lattice", [False, True])
def test_select_matches_oracle(name, lattice):
    w = synth.get(name).replace(selector_active=True)
    log(f"select {name} lattice={lattice}")
    if lattice:
        tl, tr = synth.make_integer_tables(w, tag=3)
    else:
        tl, tr = synth.make_selector_tables(w)
    inp = synth.make_selector_inputs(w, tag=5, integer_lattice=lattice)
    want = O.select_path(inp["anchors"], inp["ids"], inp["vals"], tl, tr)
    m = _select_model(w, tl, tr)
    try:
        got = m.select_path(torch.from_numpy(inp["anchors"]).cuda(), torch.from_numpy(inp["ids"]).cuda(),
                            torch.from_numpy(inp["vals"]).cuda(), debug_pair=True)
        torch.cuda.synchronize()
        assert np.array_equal(got["path"].cpu().numpy(), want["path"])
        assert np.array_equal(got["drafts"].cpu().numpy(), want["drafts"])
        assert np.array_equal(got["score"].cpu().numpy().view(np.uint32), want["score"].view(np.uint32))
        assert np.array_equal(got["pair"].cpu().numpy().view(np.uint32), want["pair"].view(np.uint32))
    finally:
        m.close()


def test_select_largest_selector():
    """selector_top_k 64 and selector_rank 256 (the ABI's limits): one LDS
    window of ~152 KB; bit-exact paths, scores and pair scores, and the
    confidence stop."""
    w = synth.get("tiny_fp32").replace(top_k=64, rank=256, batch=3, selector_active=True)
    tl, tr = synth.make_selector_tables(w)
    inp = synth.make_selector_inputs(w, tag=9)
    want = O.select_path(inp["anchors"], inp["ids"], inp["vals"], tl, tr)
    conf = O.path_confidence(inp["anchors"], inp["ids"], inp["vals"], want["path"], tl, tr)
    m = _select_model(w, tl, tr)
    try:
        a, i, v = (torch.from_numpy(inp[k]).cuda() for k in ("anchors", "ids", "vals"))
        got = m.select_path(a, i, v, debug_pair=True)
        stop = m.select_path_stop(a, i, v, p_min=0.0, want_conf=True)
        torch.cuda.synchronize()
        assert np.array_equal(got["path"].cpu().numpy(), want["path"])
        assert np.array_equal(got["score"].cpu().numpy().view(np.uint32), want["score"].view(np.uint32))
        assert np.array_equal(got["pair"].cpu().numpy().view(np.uint32), want["pair"].view(np.uint32))
        assert np.array_equal(stop["drafts"].cpu().numpy(), want["drafts"])
        np.testing.assert_allclose(stop["conf"].cpu().numpy(), conf, rtol=0, atol=2e-6)
    finally:
        m.close()


@pytest.mark.parametrize("k,bs,r", [(1, 8, 8), (3, 8, 8), (5, 2, 6), (33, 6, 12), (17, 16, 5)])
def test_select_odd_and_degenerate(k, bs, r):
    """Odd candidate counts (the last row and column of the 2 x 2 pair
    blocks are half used), k past a multiple of 16 (a ragged last round of
    the recursion's column reads), k = 1, one draft position, and ranks that
    are not a multiple of 4 (scalar table staging): bit-exact paths, scores,
    pair scores and confidences."""
    w = synth.get("tiny_fp32").replace(top_k=k, block_size=bs, rank=r, batch=4, selector_active=True)
    tl, tr = synth.make_selector_tables(w)
    inp = synth.make_selector_inputs(w, tag=11)
    want = O.select_path(inp["anchors"], inp["ids"], inp["vals"], tl, tr)
    conf = O.path_confidence(inp["anchors"], inp["ids"], inp["vals"], want["path"], tl, tr)
    m = _select_model(w, tl, tr)
    try:
        a, i, v = (torch.from_numpy(inp[key]).cuda() for key in ("anchors", "ids", "vals"))
        got = m.select_path(a, i, v, debug_pair=True)
        stop = m.select_path_stop(a, i, v, p_min=0.0, want_conf=True)
        torch.cuda.synchronize()
        assert np.array_equal(got["path"].cpu().numpy(), want["path"])
        assert np.array_equal(got["drafts"].cpu().numpy(), want["drafts"])
        assert np.array_equal(got["score"].cpu().numpy().view(np.uint32), want["score"].view(np.uint32))
        assert np.array_equal(got["pair"].cpu().numpy().view(np.uint32), want["pair"].view(np.uint32))
        assert np.array_equal(stop["drafts"].cpu().numpy(), want["drafts"])
        np.testing.assert_allclose(stop["conf"].cpu().numpy(), conf, rtol=0, atol=2e-6)
    finally:
        m.close()
