"""GPU parity of sampled (rejection) verification, dflash2_verify_sample,
and of the draft-length rule, dflash2_select_path_stop, against the oracle on
the same seeded inputs.

Accepted lengths and bonus tokens are integers decided by floating point:
the kernel takes the decisions on exact 64-bit fixed-point sums of float32
weights, the oracle in float64.  For each sequence the test enumerates every
outcome the rule can give when each comparison (u_i against p_i(d_i), v
against the cumulative mass, the kept mass against the top-p bound) may go
either way within the rounding allowance band(V).  Where that set holds one
outcome the GPU must give exactly the oracle's; elsewhere (rare, counted) it
must give one of the set.  Draft probabilities agree within band(V)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from _gpu_common import log

pytestmark = pytest.mark.gpu

def band(V: int) -> float:
    """Rounding allowance for decisions and probabilities: float32 exp and
    division (relative error a few 1e-7 of the mass) plus the fixed-point
    rounding bound V * 2^-(53 - ceil(log2 V))."""
    bits = max(0, int(V - 1).bit_length())
    return 3e-6 + V * 2.0 ** -(53 - bits)


def _gpu(drafts, z, uni, T, top_k, top_p, lens=None):
    from block_speculative_decoding_dflash2_amd import verify_sample
    d = torch.from_numpy(np.ascontiguousarray(drafts)).cuda()
    zt = torch.from_numpy(np.ascontiguousarray(z)).cuda()
    ut = torch.from_numpy(np.ascontiguousarray(uni)).cuda()
    lt = None if lens is None else torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).cuda()
    r = verify_sample(d, zt, ut, T, top_k, top_p, draft_lens=lt, want_prob=True)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in r.items()}


def _outcomes(drafts_b, z_b, uni_b, T, top_k, top_p, n_len, bd):
    """Every (accepted, bonus) the rejection rule can give for one sequence
    when each decision may go either way within bd of its threshold and the
    top-p bound may move by bd (oracle.target_distributions_near)."""
    P = len(drafts_b)
    v = float(uni_b[P])
    res = set()
    rows = {}

    def dists(i):
        if i not in rows:
            rows[i] = O.target_distributions_near(z_b[i], T, top_k, top_p, bd)
        return rows[i]

    def draws(p):
        c = np.cumsum(p)
        lo = c - p
        return np.nonzero((p > 0) & (lo - bd <= v) & (v < c + bd))[0]

    def walk(i):
        if len(res) > 64:
            return
        for p in dists(i):
            if i == n_len:
                res.update((i, int(j)) for j in draws(p))
                continue
            d = int(drafts_b[i])
            u = float(uni_b[i])
            if u < p[d] + bd:
                walk(i + 1)
            if u >= p[d] - bd:
                r = p.copy()
                r[d] = 0.0
                if r.sum() > 0:
                    res.update((i, int(j)) for j in draws(r / r.sum()))
    walk(0)
    return res


def _check(drafts, z, uni, T, top_k, top_p, lens=None, seqs=None, max_ambiguous=0.05):
    """Runs the GPU on every sequence and the oracle on `seqs` (all if None):
    exact agreement wherever the oracle's outcome is the only one within the
    rounding allowance, membership in the allowed set elsewhere."""
    B, bs, V = z.shape
    P = bs - 1
    bd = band(V) if T > 0 else 0.0
    got = _gpu(drafts, z, uni, T, top_k, top_p, lens)
    seqs = np.arange(B) if seqs is None else np.asarray(seqs)
    sl = None if lens is None else np.asarray(lens)[seqs]
    want = O.verify_sample(drafts[seqs], z[seqs], uni[seqs], T, top_k, top_p, draft_lens=sl)
    lens_all = np.full(B, P) if lens is None else np.clip(np.asarray(lens), 0, P)
    amb = 0
    for i, b in enumerate(seqs):
        a, g = int(got["accepted"][b]), int(got["bonus"][b])
        allowed = _outcomes(drafts[b], z[b], uni[b], T, top_k, top_p, int(lens_all[b]), bd)
        assert (int(want["accepted"][i]), int(want["bonus"][i])) in allowed
        if len(allowed) == 1:
            assert (a, g) == (int(want["accepted"][i]), int(want["bonus"][i])), \
                (b, a, g, want["accepted"][i], want["bonus"][i])
        else:
            amb += 1
            assert (a, g) in allowed, (b, a, g, allowed)
        for t in range(P):
            if t >= lens_all[b]:
                assert got["draft_prob"][b, t] == 0.0
                continue
            cands = [q[int(drafts[b, t])] for q in O.target_distributions_near(z[b, t], T, top_k, top_p, bd)]
            err = min(abs(float(got["draft_prob"][b, t]) - c) for c in cands)
            assert err <= bd + 1e-7 * max(cands), (b, t, got["draft_prob"][b, t], cands)
    log(f"  {len(seqs)} sequences checked, {amb} with more than one allowed outcome, "
        f"accepted mean {got['accepted'][seqs].mean():.2f}")
    assert amb <= max(1, max_ambiguous * len(seqs)), amb
    return got, want


SMALL_SHAPES = [(16, 8, 3001), (24, 7, 2500), (9, 5, 1000), (4, 16, 4099), (3, 2, 7)]
SETTINGS = [(1.0, 20, 0.95), (1.0, 0, 1.0), (0.7, 0, 0.9), (1.3, 64, 1.0), (1.0, 2600, 0.8),
            (0.5, 1, 1.0), (2.0, 0, 0.5)]


@pytest.mark.parametrize("B,bs,V", SMALL_SHAPES)
@pytest.mark.parametrize("T,top_k,top_p", SETTINGS)
def test_sampled_matches_oracle(B, bs, V, T, top_k, top_p):
    log(f"sampled B={B} bs={bs} V={V} T={T} top_k={top_k} top_p={top_p}")
    drafts, z = synth.make_sampling_inputs(B, bs, V, tag=1)
    uni = synth.make_uniforms((B, bs), tag=2)
    _check(drafts, z, uni, T, top_k, top_p)


@pytest.mark.parametrize("V,spread,quantum,T,top_k,top_p", [
    (3001, 1.0, 0.5, 1.0, 20, 0.95),     # tie group across the 20th value
    (3001, 1.0, 0.5, 1.0, 0, 0.5),       # top-p boundary inside a tie group
    (3001, 1.0, 0.5, 0.8, 1000, 0.9),
    (5000, 0.3, 1.0, 1.0, 100, 1.0),     # the k-th value tied ~240 ways
    (5000, 0.3, 1.0, 1.0, 1000, 0.9),    # the k-th value tied > 2048 ways
    (5000, 0.3, 1.0, 1.0, 0, 0.97),      # full-vocabulary top-p over large ties
    (8192, 0.0, 1.0, 1.0, 7, 0.5),       # every logit equal (planted drafts aside)
    (5000, 0.3, 1.0, 1.0, 20, 0.9),      # the 20th value tied many ways, top-p on top
])
def test_sampled_ties(V, spread, quantum, T, top_k, top_p):
    log(f"sampled ties V={V} spread={spread} q={quantum} T={T} top_k={top_k} top_p={top_p}")
    B, bs = 12, 6
    drafts, z = synth.make_sampling_inputs(B, bs, V, tag=3, spread=spread, boost=6.0, quantum=quantum)
    uni = synth.make_uniforms((B, bs), tag=4)
    _check(drafts, z, uni, T, top_k, top_p)


@pytest.mark.parametrize("T,top_k,top_p", [(1.0, 20, 0.95), (0.9, 0, 0.8)])
def test_sampled_draft_lens(T, top_k, top_p):
    B, bs, V = 32, 8, 3001
    drafts, z = synth.make_sampling_inputs(B, bs, V, tag=5, agree=0.9)
    uni = synth.make_uniforms((B, bs), tag=6)
    lens = np.random.default_rng(7).integers(-1, bs + 1, size=B).astype(np.int32)   # clamped to [0, 7]
    got, _ = _check(drafts, z, uni, T, top_k, top_p, lens=np.clip(lens, 0, bs - 1))
    got2 = _gpu(drafts, z, uni, T, top_k, top_p, lens)
    for k in got:
        assert np.array_equal(got[k], got2[k])
    zero = np.zeros(B, dtype=np.int32)
    _check(drafts, z, uni, T, top_k, top_p, lens=zero)


def test_sampled_temperature_zero_is_greedy():
    B, bs, V = 20, 8, 3001
    drafts, z = synth.make_sampling_inputs(B, bs, V, tag=8, agree=0.9)
    z[:, :, 10] = z.max(axis=2)            # ties with the planted maxima: smallest id wins
    uni = synth.make_uniforms((B, bs), tag=9)
    lens = np.random.default_rng(3).integers(0, bs, size=B).astype(np.int32)
    for ln in (None, lens):
        got = _gpu(drafts, z, uni, 0.0, 20, 0.9, ln)
        want = O.verify_accept_len(drafts, z, np.full(B, bs - 1) if ln is None else ln)
        assert np.array_equal(got["accepted"], want["accepted"])
        assert np.array_equal(got["bonus"], want["bonus"])
        L = np.full(B, bs - 1) if ln is None else ln
        for b in range(B):
            for t in range(bs - 1):
                exp = 1.0 if (t < L[b] and want["argmax"][b, t] == drafts[b, t]) else 0.0
                assert got["draft_prob"][b, t] == exp


def test_sampled_special_rows():
    B, bs, V = 6, 4, 1500
    drafts, z = synth.make_sampling_inputs(B, bs, V, tag=10)
    z[0] = -np.inf                                      # no finite logit: uniform
    z[1, :, ::3] = np.nan                               # NaN weighs 0
    z[2, :, 5] = np.inf                                 # +inf takes the mass
    z[2, :, 900] = np.inf
    z[3, :, :] = -0.0                                   # all equal (signed zeros)
    z[3, :, 1::2] = 0.0
    z[4, :, :V - 1] = -np.inf                           # one finite entry (the last)
    drafts[4, 0] = V - 1
    uni = synth.make_uniforms((B, bs), tag=11)
    for T, k, p in [(1.0, 0, 1.0), (1.0, 20, 0.95), (0.6, 0, 0.5), (1.0, 3000, 1.0)]:
        _check(drafts, z, uni, T, k, p, max_ambiguous=0.0)


def test_sampled_is_lossless_on_gpu():
    """The GPU's own draws reproduce the target distribution: many copies of
    one (row, draft) pair with independent uniforms; the emitted first token
    must follow p_0 (chi-square style bound, 6 sigma per cell)."""
    V, N = 40, 200000
    rng = np.random.default_rng(12)
    row = (rng.standard_normal((2, V)) * 1.5).astype(np.float32)
    for T, k, p, d in [(1.0, 0, 1.0, 3), (0.8, 10, 0.9, int(np.argmax(row[0]))), (1.2, 0, 0.7, 7)]:
        z = np.broadcast_to(row[None], (N, 2, V)).copy()
        drafts = np.full((N, 1), d, dtype=np.int32)
        uni = synth.make_uniforms((N, 2), tag=13 + d)
        got = _gpu(drafts, z, uni, T, k, p)
        first = np.where(got["accepted"] == 1, d, got["bonus"])
        freq = np.bincount(first, minlength=V) / N
        p0 = O.target_distribution(row[0], T, k, p)
        sd = np.sqrt(p0 * (1 - p0) / N)
        assert np.all(np.abs(freq - p0) <= 6 * sd + 1e-6), np.max(np.abs(freq - p0) / (sd + 1e-12))


@pytest.mark.parametrize("B,T,top_k,top_p,nseq", [
    (256, 1.0, 20, 0.95, 6),       # the batched fp8 shape, headline sampling settings
    (1, 1.0, 20, 0.95, 1),         # the 27B-class shape, headline sampling settings
    (1, 1.0, 0, 0.95, 1),          # the 27B-class shape, top-p over the whole vocabulary
    (4, 0.8, 0, 1.0, 2),
])
def test_sampled_full_vocab(B, T, top_k, top_p, nseq):
    bs, V = 8, 151936
    log(f"sampled full B={B} V={V} T={T} top_k={top_k} top_p={top_p}")
    drafts, z = synth.make_sampling_inputs(B, bs, V, tag=14, spread=2.0, boost=20.0)
    uni = synth.make_uniforms((B, bs), tag=15)
    seqs = np.linspace(0, B - 1, nseq).astype(int)
    _check(drafts, z, uni, T, top_k, top_p, seqs=seqs, max_ambiguous=0.0)


@pytest.mark.parametrize("top_k", [1, 20, 31])
def test_sampled_sorted_rows(top_k):
    """Rows whose largest values sit at the end of the row (ascending
    logits) or at its start (descending), so the first ids the top-k pass
    samples say nothing about the rest; plus a row with NaN, +inf and -inf
    entries."""
    B, bs, V = 4, 4, 30000
    log(f"sampled sorted rows V={V} top_k={top_k}")
    drafts, z = synth.make_sampling_inputs(B, bs, V, tag=21)
    ramp = np.linspace(-8.0, 8.0, V, dtype=np.float32)
    z[0] = ramp
    z[1] = ramp[::-1]
    z[2, :, ::7] = np.nan
    z[2, :, 5] = np.inf
    z[2, :, 11::13] = -np.inf
    uni = synth.make_uniforms((B, bs), tag=22)
    _check(drafts, z, uni, 1.0, top_k, 0.95)


def test_sampled_deterministic():
    B, bs, V = 64, 8, 32768
    drafts, z = synth.make_sampling_inputs(B, bs, V, tag=16, spread=1.0, quantum=0.25)
    uni = synth.make_uniforms((B, bs), tag=17)
    for T, k, p in [(1.0, 20, 0.95), (1.0, 0, 0.9)]:
        a = _gpu(drafts, z, uni, T, k, p)
        b = _gpu(drafts, z, uni, T, k, p)
        for key in a:
            assert np.array_equal(a[key].view(np.uint32), b[key].view(np.uint32))


# ------------------------------------------------- selector confidence stop

@pytest.mark.parametrize("name", ["tiny_fp32", "small_bf16", "small_fp8", "dense27b_bf16", "longblock_bf16"])
def test_select_stop_matches_oracle(name):
    from test_gpu_verify_select import _select_model
    w = synth.get(name).replace(selector_active=True)
    log(f"select_stop {name}")
    tl, tr = synth.make_selector_tables(w)
    inp = synth.make_selector_inputs(w, tag=21)
    sel = O.select_path(inp["anchors"], inp["ids"], inp["vals"], tl, tr)
    conf = O.path_confidence(inp["anchors"], inp["ids"], inp["vals"], sel["path"], tl, tr)
    P = w.block_size - 1
    m = _select_model(w, tl, tr)
    try:
        a, i, v = (torch.from_numpy(inp[k]).cuda() for k in ("anchors", "ids", "vals"))
        plain = m.select_path(a, i, v)
        qs = np.quantile(conf, [0.1, 0.3, 0.6]).tolist()
        for p_min, n_min, n_max in [(0.0, 0, P), (qs[0], 0, P), (qs[1], 1, P), (qs[2], 0, max(P - 2, 0)),
                                    (qs[1], P + 3, -2), (1.0, 0, P)]:
            got = m.select_path_stop(a, i, v, p_min=p_min, n_min=n_min, n_max=n_max, want_conf=True,
                                     want_score=True)
            torch.cuda.synchronize()
            assert np.array_equal(got["path"].cpu().numpy(), sel["path"])
            assert np.array_equal(got["drafts"].cpu().numpy(), sel["drafts"])
            assert np.array_equal(got["score"].cpu().numpy().view(np.uint32), sel["score"].view(np.uint32))
            assert np.array_equal(got["path"].cpu().numpy(), plain["path"].cpu().numpy())
            gc = got["conf"].cpu().numpy()
            np.testing.assert_allclose(gc, conf, rtol=0, atol=2e-6)
            want = O.draft_lengths(conf, p_min, n_min, n_max)
            gl = got["lens"].cpu().numpy()
            for b in range(w.batch):
                if np.min(np.abs(conf[b] - p_min)) > 1e-5:
                    assert gl[b] == want[b], (b, gl[b], want[b])
                else:
                    assert 0 <= gl[b] <= P
    finally:
        m.close()


def test_sampled_after_select_stop():
    """Lengths from the selector feed the sampled verification directly."""
    from block_speculative_decoding_dflash2_amd import verify_sample
    from test_gpu_verify_select import _select_model
    w = synth.get("small_bf16").replace(selector_active=True)
    tl, tr = synth.make_selector_tables(w)
    inp = synth.make_selector_inputs(w, tag=22)
    m = _select_model(w, tl, tr)
    try:
        a, i, v = (torch.from_numpy(inp[k]).cuda() for k in ("anchors", "ids", "vals"))
        got = m.select_path_stop(a, i, v, p_min=0.3, want_conf=True)
        drafts = got["drafts"].cpu().numpy()
        lens = got["lens"].cpu().numpy()
        B, bs, V = w.batch, w.block_size, w.vocab
        _, z = synth.make_sampling_inputs(B, bs, V, tag=23)
        uni = synth.make_uniforms((B, bs), tag=24)
        r = verify_sample(got["drafts"], torch.from_numpy(z).cuda(), torch.from_numpy(uni).cuda(), 1.0, 20, 0.95,
                          draft_lens=got["lens"])
        torch.cuda.synchronize()
        want = O.verify_sample(drafts, z, uni, 1.0, 20, 0.95, draft_lens=lens)
        ga, gb = r["accepted"].cpu().numpy(), r["bonus"].cpu().numpy()
        bd = band(V)
        for b in range(B):
            allowed = _outcomes(drafts[b], z[b], uni[b], 1.0, 20, 0.95, int(lens[b]), bd)
            if len(allowed) == 1:
                assert (int(ga[b]), int(gb[b])) == (int(want["accepted"][b]), int(want["bonus"][b]))
            else:
                assert (int(ga[b]), int(gb[b])) in allowed
    finally:
        m.close()
