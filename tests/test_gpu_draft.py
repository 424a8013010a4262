"""GPU parity of the whole draft step (dflash2_draft_block + select_path +
verify_accept) against the oracle on the same seeded inputs.

Checked per workload:
  * appended context rows (every layer), the final residual stream and the
    float32 logits: normwise error max|g-o|/max|o| within the tolerance of
    the arithmetic (fp32 1e-5, bf16 2e-2, fp8 6e-2);
  * the GPU's top-k is exactly the top-k of its own logits (ids, order,
    values);
  * where the oracle's top-k boundary gap exceeds twice the measured logit
    error delta, the GPU's candidate set equals the oracle's;
  * where additionally the oracle's max-sum decision margin at a position
    exceeds 2 (bs-1) delta, the GPU's draft token equals the oracle's
    (required for >= 99.5% of such positions);
  * verification on logits planted around the oracle's path: accepted
    length and bonus equal the oracle's wherever the drafts agree.
Small workloads run the oracle on the whole batch; the large ones on a
sample of sequences (the step is independent across sequences)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from _gpu_common import TOL, DraftRun, log, normwise, oracle_for, topk_consistent

pytestmark = pytest.mark.gpu


def _through_margins(pair, vals, path):
    """Max-sum forward/backward over the oracle's lattice (float64): margin
    between the best path through the chosen candidate at each position and
    the best path through any other candidate there."""
    B, P, k = vals.shape
    out = np.empty((B, P))
    for b in range(B):
        z = vals[b].astype(np.float64)
        pr = pair[b].astype(np.float64)
        fwd = np.empty((P, k))
        fwd[0] = pr[0, 0] + z[0]
        for t in range(1, P):
            fwd[t] = (fwd[t - 1][:, None] + pr[t]).max(axis=0) + z[t]
        bwd = np.zeros((P, k))
        for t in range(P - 2, -1, -1):
            bwd[t] = (pr[t + 1] + (z[t + 1] + bwd[t + 1])[None, :]).max(axis=1)
        thr = fwd + bwd
        for t in range(P):
            j = path[b, t]
            others = np.delete(thr[t], j)
            out[b, t] = thr[t, j] - (others.max() if len(others) else np.inf)
    return out


def check_step(g: DraftRun, res, seqs):
    w = g.w
    tol = TOL[w.weight_dtype]
    P, k = w.block_size - 1, w.top_k
    seqs = list(seqs)
    # 1. appended context rows
    errs = []
    for layer in range(w.num_layers):
        rows = g.cache_rows(seqs, layer)
        for i, b in enumerate(seqs):
            L = int(g.inp.ctx_lens[b])
            n = int(g.inp.new_offsets[b + 1] - g.inp.new_offsets[b])
            ok_ = res["k_cache"][layer, i, :, L - n:L, :].transpose(1, 0, 2)
            ov = res["v_cache"][layer, i, :, L - n:L, :].transpose(1, 0, 2)
            errs += [normwise(rows[i][0], ok_), normwise(rows[i][1], ov)]
    e_cache = max(errs)
    # 2. hidden states and logits
    e_hidden = normwise(g.hidden[seqs], res["h_final"])
    glog = g.logits[seqs]
    e_logit = normwise(glog, res["zeta"])
    delta = float(np.max(np.abs(glog.astype(np.float64) - res["zeta"])))
    log(f"{w.name}: err cache {e_cache:.2e} hidden {e_hidden:.2e} logits {e_logit:.2e} (delta {delta:.2e})")
    assert e_cache <= tol and e_hidden <= tol and e_logit <= tol
    # 3. the GPU's top-k is the top-k of its own logits; its values are the
    # transformed logits (output_multiplier, then the soft cap) at those ids
    ids = g.topk_ids[seqs].reshape(-1, k)
    vals = g.topk_vals[seqs].reshape(-1, k)
    z_own = glog.reshape(-1, w.vocab)
    raw = np.take_along_axis(z_own, ids.astype(np.int64), axis=1)
    assert topk_consistent(ids, raw, z_own, k)
    mult, cap = w.output_multiplier, w.final_logit_softcapping
    if mult == 1.0 and cap == 0.0:
        assert np.array_equal(vals, raw + np.float32(0.0))
    else:
        # float32 multiply and tanhf on the GPU against float64: a few ulp
        want_t = O.logit_transform(raw.astype(np.float64), mult, cap)
        e_t = float(np.max(np.abs(vals - want_t)))
        log(f"{w.name}: transformed top-k values off by {e_t:.2e} (multiplier {mult}, cap {cap})")
        assert e_t <= 8 * np.finfo(np.float32).eps * max(1.0, float(np.max(np.abs(want_t))))
    # 4. candidate sets where the oracle's boundary gap exceeds 2 delta
    z32 = res["zeta"].astype(np.float32).reshape(len(seqs), P, -1)
    srt = -np.sort(-z32.astype(np.float64), axis=-1)
    gap = srt[..., k - 1] - srt[..., k] if w.vocab > k else np.full(srt.shape[:2], np.inf)
    qual = gap > 2 * delta
    same_set = np.array([[set(g.topk_ids[b, t].tolist()) == set(res["topk_ids"][i, t].tolist())
                          for t in range(P)] for i, b in enumerate(seqs)])
    assert same_set[qual].all(), f"candidate sets differ at {np.argwhere(qual & ~same_set)}"
    # ... and there the (transformed) candidate values, the selector's unary
    # term, agree with the oracle's within the logit tolerance
    same_ids = np.array([[np.array_equal(g.topk_ids[b, t], res["topk_ids"][i, t]) for t in range(P)]
                         for i, b in enumerate(seqs)])
    if same_ids.any():
        gv = g.topk_vals[seqs][same_ids]
        ov = res["topk_vals"][same_ids]
        e_vals = normwise(gv, ov)
        log(f"{w.name}: top-k values error {e_vals:.2e} on {same_ids.mean():.3f} of the positions")
        assert e_vals <= tol
    # 5. drafts where the max-sum decision margin is clear
    margins = _through_margins(res["pair"], res["topk_vals"], res["path"])
    seq_ok = qual.all(axis=1)
    clear = (margins > 2 * P * delta) & seq_ok[:, None]
    agree = g.drafts[seqs] == res["drafts"]
    frac = agree[clear].mean() if clear.any() else 1.0
    log(f"{w.name}: qualifying positions {clear.mean():.3f}, draft agreement there {frac:.4f}, "
        f"overall {agree.mean():.4f}; path differs from top-1 at {np.mean(res['path'] != 0):.3f}")
    assert frac >= 0.995
    # 6. verification against logits planted around the oracle's drafts
    from block_speculative_decoding_dflash2_amd import verify_accept
    tz = synth.make_target_logits(w, res["drafts"], seqs=np.array(seqs), tag=2)
    want = O.verify_accept(res["drafts"], tz)
    got = verify_accept(torch.from_numpy(np.ascontiguousarray(g.drafts[seqs])).cuda(),
                        torch.from_numpy(tz).cuda(), want_argmax=True)
    torch.cuda.synchronize()
    same = (g.drafts[seqs] == res["drafts"]).all(axis=1)
    assert np.array_equal(got["argmax"].cpu().numpy(), want["argmax"])
    assert np.array_equal(got["accepted"].cpu().numpy()[same], want["accepted"][same])
    assert np.array_equal(got["bonus"].cpu().numpy()[same], want["bonus"][same])


@pytest.mark.parametrize("name", ["tiny_fp32", "small_fp32", "small_bf16", "small_fp8", "medium_bf16",
                                  "medium_fp8"])
def test_draft_small_workloads(name):
    w = synth.get(name)
    g = DraftRun(w)
    try:
        _, res = oracle_for(w, g.W)
        check_step(g, res, range(w.batch))
    finally:
        g.close()


@pytest.mark.parametrize("name", ["small_bf16", "medium_fp8", "small_fp32"])
def test_draft_embedding_scale_and_logit_transform(name):
    """input_embedding_scale = 2.5 on the embedded block, and the logit
    transform output_multiplier = 0.5 then final_logit_softcapping = 30 on
    the candidates (NeMo AutoModel page, Key Config Fields): small_bf16 and
    small_fp32 take the weight-streaming lm_head (at most 64 rows), medium_fp8
    the LDS-tiled one.  Hidden states, logits, appended rows and the
    transformed top-k values are checked against the oracle, the drafts where
    the decision margins are clear.  A transform applied in the other order
    (cap, then multiplier) moves the values by far more than the bound."""
    w = synth.get(name).replace(input_embedding_scale=2.5, output_multiplier=0.5,
                                final_logit_softcapping=30.0, name=f"{name}_transform")
    g = DraftRun(w)
    try:
        _, res = oracle_for(w, g.W)
        check_step(g, res, range(w.batch))
        # the swapped order gives values that differ from the stored ones
        raw = np.take_along_axis(g.logits.reshape(-1, w.vocab), g.topk_ids.reshape(-1, w.top_k).astype(np.int64),
                                 axis=1).astype(np.float64)
        swapped = 0.5 * (30.0 * np.tanh(raw / 30.0))
        assert np.max(np.abs(swapped - g.topk_vals.reshape(-1, w.top_k))) > 1e-4
    finally:
        g.close()


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_lmhead_tiled_beyond_4gib():
    """A bf16 lm_head of 270000 x 8192 (4.1 GiB, rows 262144 and up start
    past 2^32 bytes) on the tiled path (70 rows): the logits of ids past the
    4 GiB line, and a sample below it, equal the float64 product of the GPU's
    own final hidden states (RMSNorm, gain) with those lm_head rows, and the
    top-k is the top-k of the GPU's own logits."""
    w = synth.get("small_bf16").replace(
        name="wide_vocab_bf16", index=15, batch=10, block_size=8, hidden=8192, num_layers=1,
        num_q_heads=2, num_kv_heads=1, head_dim=64, ffn=64, vocab=270000, num_taps=1, tap_width=64,
        ctx=(16, 16), top_k=4, rank=8)
    assert w.vocab * w.hidden * 2 > (1 << 32) and w.batch * (w.block_size - 1) > 64
    g = DraftRun(w)
    try:
        V, H = w.vocab, w.hidden
        z = g.logits.reshape(-1, V)
        h = g.hidden[:, 1:, :].reshape(-1, H).astype(np.float64)
        nf = O.rmsnorm(h, O.decode(g.W.final_norm), w.rms_eps)
        rng = np.random.default_rng(0)
        cols = np.unique(np.concatenate([np.arange(262144 - 64, V), rng.integers(0, 262144, 512)]))
        want = nf @ O.bf16_bits_to_f64(g.W.lm_head.data[cols]).T
        err = normwise(z[:, cols], want)
        log(f"wide vocab: logits error {err:.2e} over {len(cols)} ids ({np.sum(cols >= 262144)} past 4 GiB)")
        assert err <= TOL["bf16"]
        assert topk_consistent(g.topk_ids.reshape(-1, w.top_k), g.topk_vals.reshape(-1, w.top_k), z, w.top_k)
    finally:
        g.close()


def test_draft_is_deterministic():
    w = synth.get("small_bf16")
    a = DraftRun(w)
    b = DraftRun(w, W=a.W)
    try:
        assert np.array_equal(a.logits.view(np.uint32), b.logits.view(np.uint32))
        assert np.array_equal(a.topk_ids, b.topk_ids) and np.array_equal(a.drafts, b.drafts)
    finally:
        a.close()
        b.close()


def test_draft_selector_literal_weights_small():
    """Literal N(0, 0.02) selector factors (pair term tiny): still exact."""
    w = synth.get("small_bf16").replace(selector_active=False, name="small_bf16_literal")
    g = DraftRun(w)
    try:
        _, res = oracle_for(w, g.W)
        check_step(g, res, range(w.batch))
    finally:
        g.close()


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_draft_dense27b_full():
    """The 27B-class single-sequence workload at full size, oracle on the whole step."""
    w = synth.get("dense27b_bf16")
    g = DraftRun(w)
    try:
        _, res = oracle_for(w, g.W)
        check_step(g, res, range(w.batch))
    finally:
        g.close()


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,seqs", [("batched_bf16", [0, 37, 63]), ("longblock_bf16", [0, 15]),
                                       ("fp8_b256", [0, 129, 255])])
def test_draft_large_sampled(name, seqs):
    """Full-size batched workloads on the GPU; the oracle recomputes a sample
    of the sequences."""
    w = synth.get(name)
    g = DraftRun(w)
    try:
        _, res = oracle_for(w, g.W, seqs)
        check_step(g, res, seqs)
    finally:
        g.close()


@pytest.mark.parametrize("name", ["small_bf16", "medium_bf16", "medium_fp8"])
def test_lmhead_topk_heavy_ties(name):
    """lm_head rows that repeat five base rows make each logit row five
    values repeated ~V/5 times: the top-k must still be exactly the (value
    desc, id asc) order of the GPU's own logits.  On the tiled lm_head far
    more than 32 values of a row reach the row's bound, so this runs its
    exact-ranking fallback on every vocabulary tile."""
    w = synth.get(name)
    W = synth.make_weights(w)
    rep = np.arange(w.vocab) % 5
    W.lm_head.data[:] = W.lm_head.data[rep]
    if W.lm_head.scale is not None:
        W.lm_head.scale[:] = W.lm_head.scale[rep]
    g = DraftRun(w, W=W)
    try:
        k = w.top_k
        z = g.logits.reshape(-1, w.vocab)
        ties = (z == z.max(axis=1, keepdims=True)).sum(axis=1)
        log(f"{name}: copies of each row's maximum: min {ties.min()}, max {ties.max()}")
        assert ties.min() > 32
        assert topk_consistent(g.topk_ids.reshape(-1, k), g.topk_vals.reshape(-1, k), z, k)
    finally:
        g.close()


@pytest.mark.parametrize("name", ["medium_bf16", "medium_fp8"])
def test_lmhead_vocabulary_sweeps(name, monkeypatch):
    """The tiled lm_head with each block sweeping three vocabulary tiles
    (later tiles filter against the row's running 16th key): same checks as
    the single-tile default, plus the heavy-tie lattice."""
    monkeypatch.setenv("DFLASH2_LMHEAD_TILES_PER_BLOCK", "3")
    w = synth.get(name)
    g = DraftRun(w)
    try:
        _, res = oracle_for(w, g.W)
        check_step(g, res, range(w.batch))
    finally:
        g.close()
    W = synth.make_weights(w)
    rep = np.arange(w.vocab) % 5
    W.lm_head.data[:] = W.lm_head.data[rep]
    if W.lm_head.scale is not None:
        W.lm_head.scale[:] = W.lm_head.scale[rep]
    g = DraftRun(w, W=W)
    try:
        k = w.top_k
        z = g.logits.reshape(-1, w.vocab)
        assert topk_consistent(g.topk_ids.reshape(-1, k), g.topk_vals.reshape(-1, k), z, k)
    finally:
        g.close()


@pytest.mark.parametrize("name", ["medium_bf16", "medium_fp8"])
@pytest.mark.parametrize("bm", ["192", "256"])
def test_lmhead_row_tiles(name, bm, monkeypatch):
    """The tiled lm_head on 192- and 256-row tiles (one ragged tile, or a
    full and a ragged one), three vocabulary tiles per block: same checks
    as the default 128-row tiles."""
    monkeypatch.setenv("DFLASH2_LMHEAD_BM", bm)
    monkeypatch.setenv("DFLASH2_LMHEAD_TILES_PER_BLOCK", "3")
    w = synth.get(name)
    g = DraftRun(w)
    try:
        _, res = oracle_for(w, g.W)
        check_step(g, res, range(w.batch))
    finally:
        g.close()


@pytest.mark.parametrize("name", ["medium_bf16", "medium_fp8"])
def test_draft_tiled_single_split(name, monkeypatch):
    """Tiled GEMMs with one K split, so gate/up and QKV apply SwiGLU and the
    RoPE / cache stores in their own epilogue: same checks as the default."""
    monkeypatch.setenv("DFLASH2_TILED_MAX_SPLITS", "1")
    w = synth.get(name)
    g = DraftRun(w)
    try:
        _, res = oracle_for(w, g.W)
        check_step(g, res, range(w.batch))
    finally:
        g.close()


@pytest.mark.parametrize("name", ["medium_bf16", "medium_fp8"])
@pytest.mark.parametrize("splits", ["1", "8"])
def test_draft_tiled_128_row_tiles(name, splits, monkeypatch):
    """Tiled GEMMs on 128-row block tiles (fp8: two blocks per CU with two
    stage buffers; bf16: three stage buffers), ragged last row tile, with
    one K split (SwiGLU and QKV epilogues) and with the planner's splits
    (partial sums): same checks as the default 256-row tiles."""
    monkeypatch.setenv("DFLASH2_TILED_BM", "128")
    monkeypatch.setenv("DFLASH2_TILED_MAX_SPLITS", splits)
    w = synth.get(name)
    g = DraftRun(w)
    try:
        _, res = oracle_for(w, g.W)
        check_step(g, res, range(w.batch))
    finally:
        g.close()


@pytest.mark.parametrize("name,batch", [("small_bf16", 5), ("small_bf16", 8), ("small_fp8", 9)])
def test_draft_tiled_few_rows(name, batch):
    """33-64 activation rows: the linears whose depth is a multiple of 64 take
    the LDS-tiled GEMM (one ragged row tile, split K; the FFN down projection
    of depth 736 stays on the weight-streaming kernel), the lm_head (at most
    64 rows) the weight-streaming kernel."""
    w = synth.get(name).replace(batch=batch)
    assert 32 < w.batch * w.block_size <= 64 or 32 < w.batch * (w.block_size - 1) <= 64
    g = DraftRun(w)
    try:
        _, res = oracle_for(w, g.W)
        check_step(g, res, range(w.batch))
    finally:
        g.close()


@pytest.mark.parametrize("name,batch", [("small_bf16", 1), ("small_bf16", 2), ("small_fp8", 1), ("small_fp8", 2)])
def test_draft_streaming_few_rows(name, batch):
    """At most 16 activation rows (7-16 here): the weight-streaming GEMMs copy
    each block's rows of the activations into LDS and read their operands
    from there; the lm_head streams its weights too."""
    w = synth.get(name).replace(batch=batch)
    assert w.batch * w.block_size <= 16
    g = DraftRun(w)
    try:
        _, res = oracle_for(w, g.W)
        check_step(g, res, range(w.batch))
    finally:
        g.close()


@pytest.mark.parametrize("name,changes,tpb", [
    ("small_bf16", dict(vocab=40000, top_k=8), None),   # 313 lists of 8 keys per row: folded to 5
    ("small_fp8", dict(vocab=32897), None),             # 258 lists: the last fold block takes 2
    ("medium_fp8", dict(vocab=17000), "1"),             # tiled lm_head: 67 runs of one tile
])
def test_draft_many_candidate_lists(name, changes, tpb, monkeypatch):
    """Many candidate lists per row: more than 64 go to the merge kernel's
    256-thread block, more than 256 are first folded 64 at a time (16 best
    keys of each run of lists).  Same checks as the default workloads."""
    if tpb:
        monkeypatch.setenv("DFLASH2_LMHEAD_TILES_PER_BLOCK", tpb)
    w = synth.get(name).replace(**changes)
    g = DraftRun(w)
    try:
        _, res = oracle_for(w, g.W)
        check_step(g, res, range(w.batch))
    finally:
        g.close()


@pytest.mark.parametrize("splits", ["1", "8"])
def test_draft_tiled_192_row_tiles(splits, monkeypatch):
    """fp8 tiled GEMMs on 192-row block tiles (three accumulator row blocks
    per wave, three stage buffers): 280 rows in a full and a ragged row
    tile, one K split (SwiGLU and QKV epilogues) and the planner's splits."""
    monkeypatch.setenv("DFLASH2_TILED_BM", "192")
    monkeypatch.setenv("DFLASH2_TILED_MAX_SPLITS", splits)
    w = synth.get("medium_fp8")
    g = DraftRun(w)
    try:
        _, res = oracle_for(w, g.W)
        check_step(g, res, range(w.batch))
    finally:
        g.close()


@pytest.mark.parametrize("name,window", [("small_bf16", 64), ("medium_fp8", 100), ("small_fp32", 33),
                                         ("tiny_fp32", 8)])
def test_draft_sliding_window(name, window):
    """draft_sliding_window: attention reaches back `window` context rows;
    sequences both shorter and longer than the window.  tiny_fp32 and
    small_fp32 plan one key chunk (a block takes at least three 64-key
    sub-chunks), so the attention kernel writes its output without the merge
    pass; the bf16 and fp8 cases merge several chunks."""
    w = synth.get(name).replace(sliding_window=window)
    g = DraftRun(w)
    try:
        _, res = oracle_for(w, g.W)
        check_step(g, res, range(w.batch))
    finally:
        g.close()


@pytest.mark.parametrize("name,group", [("tiny_fp32", 16), ("small_fp32", 32), ("small_bf16", 32),
                                        ("small_fp8", 64), ("medium_bf16", 16), ("medium_fp8", 320)])
def test_draft_dynamic_conv(name, group):
    """Dynamic grouped convolution (conv_group_size > 0): every conv site's
    taps come from a GEMM against W_dconv on the slot's input; appended
    cache rows, hidden states and logits within the dtype bound."""
    w = synth.get(name).replace(conv_group_size=group)
    g = DraftRun(w)
    try:
        _, res = oracle_for(w, g.W)
        check_step(g, res, range(w.batch))
    finally:
        g.close()


@pytest.mark.parametrize("name,overhead", [("small_bf16", "0"), ("small_fp32", "0"), ("small_fp8", "65536")])
def test_draft_stream_split_planner_extremes(name, overhead, monkeypatch):
    """Weight-streaming GEMMs (at most 64 rows) under the split planner's
    extremes: a zero per-block cost (as many K splits as allowed) and a huge
    one (the fewest waves): same checks as the default."""
    monkeypatch.setenv("DFLASH2_STREAM_BLOCK_OVERHEAD", overhead)
    w = synth.get(name)
    g = DraftRun(w)
    try:
        _, res = oracle_for(w, g.W)
        check_step(g, res, range(w.batch))
    finally:
        g.close()


@pytest.mark.parametrize("name,tag,changes", [
    ("tiny_fp32", "bs2", dict(block_size=2)),          # one draft position: the lattice is one transition
    ("small_bf16", "bs2", dict(block_size=2)),
    ("small_bf16", "k1", dict(top_k=1)),               # one candidate per position: the path is forced
    ("medium_fp8", "k1", dict(top_k=1)),               # ... on the tiled lm_head
    ("small_fp32", "ctx1", dict(cold=True, ctx=(1, 3))),  # contexts of 1-3 rows, all appended this step
    ("small_bf16", "ctx1", dict(cold=True, ctx=(1, 3))),
])
def test_draft_degenerate_shapes(name, tag, changes):
    """The method's degenerate cases: block size 2, top-k 1 and contexts of
    one to three rows (a 32-row cache shorter than one key sub-chunk).  Same
    checks as the default workloads."""
    w = synth.get(name).replace(name=f"{name}_{tag}", **changes)
    g = DraftRun(w)
    try:
        _, res = oracle_for(w, g.W)
        if w.top_k == 1:  # the path is forced on both sides: drafts are the top-1 ids
            assert (res["path"] == 0).all()
            assert (g.path == 0).all() and np.array_equal(g.drafts, g.topk_ids[..., 0])
        check_step(g, res, range(w.batch))
    finally:
        g.close()
