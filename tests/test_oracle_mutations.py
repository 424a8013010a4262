"""The oracle's pins catch planted mistakes.

Each case swaps one oracle function for a plausible wrong version (a dropped
term, a wrong sign, index, operand order or tie rule) for the length of one
test, on the CPU, and requires at least one of the pins written for that
function to fail with an AssertionError.  The oracle's own source is never
changed; the wrong versions live only here."""
import math

import numpy as np
import pytest

import oracle as O
import oracle.dflash2_oracle as OD
import test_oracle_draft as TD
import test_oracle_ops as TO
import test_oracle_select_verify as TS


def _rope(x, pos, theta, *, sign=1.0, expo=2.0, interleaved=False):
    d = x.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * theta ** (-expo * i / d)[None, :]
    shape = (len(pos),) + (1,) * (x.ndim - 2) + (half,)
    c, s = np.cos(ang).reshape(shape), sign * np.sin(ang).reshape(shape)
    if interleaved:
        y = np.empty_like(x)
        a, b = x[..., 0::2], x[..., 1::2]
        y[..., 0::2], y[..., 1::2] = a * c - b * s, b * c + a * s
        return y
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def _conv(x, taps, *, ahead=False, residual=True, reverse=False):
    bs, K = x.shape[0], taps.shape[0]
    y = x.copy() if residual else np.zeros_like(x)
    for j in range(K):
        t = taps[K - 1 - j] if reverse else taps[j]
        if ahead:
            y[:bs - j] += t * x[j:]
        else:
            y[j:] += t * x[:bs - j]
    return y


def _attention(q, k, v, *, scale=True, causal=False, modulo=False):
    T, nq, d = q.shape
    S, nkv = k.shape[0], k.shape[1]
    out = np.empty_like(q)
    for i in range(nq):
        g = i % nkv if modulo else i // (nq // nkv)
        s = q[:, i, :] @ k[:, g, :].T / (math.sqrt(d) if scale else 1.0)
        if causal:
            s = np.where(np.arange(S)[None, :] > np.arange(T)[:, None] + (S - T), -np.inf, s)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        out[:, i, :] = (p / p.sum(axis=1, keepdims=True)) @ v[:, g, :]
    return out


def _topk_largest_id(keys32, k):
    x = O.canonical_f32(keys32).astype(np.float64)[:, ::-1]
    V = x.shape[1]
    ids = np.empty((x.shape[0], k), dtype=np.int32)
    vals = np.empty((x.shape[0], k), dtype=np.float32)
    rows = np.arange(x.shape[0])
    for j in range(k):
        a = np.argmax(x, axis=1)
        ids[:, j], vals[:, j] = V - 1 - a, x[rows, a]
        x[rows, a] = -np.inf
    return ids, vals


def _select(anchors, cand_ids, cand_vals, tl, tr, *, pick=np.argmax, swap=False, unary=True):
    cand_ids = np.asarray(cand_ids)
    cand_vals = np.asarray(cand_vals, dtype=np.float32) * (1.0 if unary else 0.0)
    B, P, k = cand_ids.shape

    def pair(a, b):
        return O.pair_scores(tl, tr, b, a).T if swap else O.pair_scores(tl, tr, a, b)

    path = np.empty((B, P), dtype=np.int32)
    drafts = np.empty((B, P), dtype=np.int32)
    score = np.empty(B, dtype=np.float32)
    pairs = np.empty((B, P, k, k), dtype=np.float32)
    for b in range(B):
        p0 = pair([int(anchors[b])], cand_ids[b, 0])[0]
        pairs[b, 0] = p0[None, :]
        S = (p0 + cand_vals[b, 0]).astype(np.float32)
        back = np.zeros((P, k), dtype=np.int64)
        for t in range(1, P):
            pt = pair(cand_ids[b, t - 1], cand_ids[b, t])
            pairs[b, t] = pt
            tot = (S[:, None] + pt).astype(np.float32)
            bi = pick(tot, axis=0)
            back[t] = bi
            S = (tot[bi, np.arange(k)] + cand_vals[b, t]).astype(np.float32)
        j = int(pick(S))
        score[b] = S[j]
        for t in range(P - 1, -1, -1):
            path[b, t], drafts[b, t] = j, cand_ids[b, t, j]
            j = int(back[t, j])
    return {"path": path, "drafts": drafts, "score": score, "pair": pairs}


def _last_argmax(a, axis=None):
    if axis is None:
        return a.size - 1 - int(np.argmax(a[::-1]))
    return a.shape[axis] - 1 - np.argmax(np.flip(a, axis=axis), axis=axis)


def _verify(drafts, target_logits, *, row_shift=0, bonus_shift=0, stop_early=False):
    drafts = np.asarray(drafts)
    z = O.canonical_f32(target_logits)
    B, bs, _ = z.shape
    g = np.argmax(z, axis=2).astype(np.int32)
    acc = np.zeros(B, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    lim = bs - 2 if stop_early else bs - 1
    for b in range(B):
        n = 0
        while n < lim and g[b, min(n + row_shift, bs - 1)] == drafts[b, n]:
            n += 1
        acc[b], bonus[b] = n, g[b, min(n + bonus_shift, bs - 1)]
    return {"accepted": acc, "bonus": bonus, "argmax": g}


_ORIG_PAIR = OD.pair_scores


def _pair_swapped_tables(tl, tr, a_ids, b_ids):
    return _ORIG_PAIR(tr, tl, a_ids, b_ids)


def _pair_f64(tl, tr, a_ids, b_ids):
    A = tl[np.asarray(a_ids)].astype(np.float64)
    Bm = tr[np.asarray(b_ids)].astype(np.float64)
    return (A @ Bm.T).astype(np.float32)


OPS = [TO.test_conv_hand_worked, TO.test_conv_matches_numpy_convolve_and_boundaries,
       TO.test_rmsnorm_closed_form_and_torch, TO.test_silu_matches_torch, TO.test_rope_identities,
       TO.test_attention_matches_torch_sdpa_gqa, TO.test_attention_single_key_returns_value,
       TO.test_logit_transform]
DRAFT = [TD.test_uniform_attention_averages_all_values, TD.test_append_position_zero_is_unrotated]
SELECT = ([lambda t=t: TS.test_selector_equals_exhaustive_search_tiny(t) for t in range(3)]
          + [lambda t=t: TS.test_selector_tie_rule_integer_lattice(t) for t in range(4)]
          + [TS.test_selector_v1_special_cases, TS.test_pair_scores_reference_loop])
TOPK = [lambda s=s: TS.test_topk_matches_full_sort(s) for s in range(4)] + [TS.test_topk_minus_zero_ties_like_plus_zero]
VERIFY = [TS.test_verify_hand_worked, TS.test_verify_ties_and_signed_zero, TS.test_verify_lossless_property]

MUTANTS = {
    # name: (oracle function, wrong version, pins that must notice)
    "rmsnorm_l1": ("rmsnorm", lambda x, g, eps: x / np.mean(np.abs(x), axis=-1, keepdims=True) * g, OPS),
    "rmsnorm_no_gain": ("rmsnorm", lambda x, g, eps: x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps), OPS),
    "rmsnorm_eps_outside": ("rmsnorm", lambda x, g, eps: x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * g,
                            OPS),
    "silu_sign": ("silu", lambda x: x / (1.0 + np.exp(x)), OPS),
    "rope_sign": ("rope", lambda x, p, th: _rope(x, p, th, sign=-1.0), OPS + DRAFT),
    "rope_frequency": ("rope", lambda x, p, th: _rope(x, p, th, expo=1.0), OPS + DRAFT),
    "rope_interleaved": ("rope", lambda x, p, th: _rope(x, p, th, interleaved=True), OPS + DRAFT),
    "conv_looks_ahead": ("block_conv", lambda x, c: _conv(x, c, ahead=True), OPS),
    "conv_no_residual": ("block_conv", lambda x, c: _conv(x, c, residual=False), OPS),
    "conv_taps_reversed": ("block_conv", lambda x, c: _conv(x, c, reverse=True), OPS),
    "attention_no_scale": ("attention", lambda q, k, v: _attention(q, k, v, scale=False), OPS + DRAFT),
    "attention_causal": ("attention", lambda q, k, v: _attention(q, k, v, causal=True), OPS + DRAFT),
    "attention_gqa_modulo": ("attention", lambda q, k, v: _attention(q, k, v, modulo=True), OPS + DRAFT),
    "softcap_before_multiplier": ("logit_transform",
                                  lambda x, m, cap: m * (cap * np.tanh(x / cap) if cap > 0 else x), OPS),
    "topk_ties_to_largest_id": ("topk", _topk_largest_id, TOPK),
    "select_min_not_max": ("select_path", lambda *a: _select(*a, pick=np.argmin), SELECT),
    "select_pair_transposed": ("select_path", lambda *a: _select(*a, swap=True), SELECT),
    "select_no_unary": ("select_path", lambda *a: _select(*a, unary=False), SELECT),
    "select_ties_to_last": ("select_path", lambda *a: _select(*a, pick=_last_argmax), SELECT),
    "pair_tables_swapped": ("pair_scores", _pair_swapped_tables, SELECT),
    "pair_float64_sum": ("pair_scores", _pair_f64, SELECT),
    "verify_row_shift": ("verify_accept", lambda d, z: _verify(d, z, row_shift=1), VERIFY),
    "verify_bonus_next_row": ("verify_accept", lambda d, z: _verify(d, z, bonus_shift=1), VERIFY),
    "verify_never_accepts_all": ("verify_accept", lambda d, z: _verify(d, z, stop_early=True), VERIFY),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_planted_mistake(mutant, monkeypatch):
    name, wrong, pins = MUTANTS[mutant]
    monkeypatch.setattr(O, name, wrong)
    monkeypatch.setattr(OD, name, wrong)
    failed = []
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed.append(getattr(pin, "__name__", "pin"))
            break
    assert failed, f"no pin noticed the planted mistake {mutant!r} in oracle.{name}"


def test_pins_pass_on_the_oracle_itself():
    """The same pin lists pass on the untouched oracle (so a failure above is
    the mutant's doing)."""
    for pins in (OPS, DRAFT, SELECT, TOPK, VERIFY):
        for pin in pins:
            pin()


# ------------------------------------------------------------------ composed forward
# Mistakes inside append_context / draft_block are planted in a copy of the
# oracle's source (one exact text replacement each), executed as a separate
# module; the invariant pins of the composed forward must notice.

import inspect
import types

_SRC = inspect.getsource(OD)
DRAFT_PINS = [f for n, f in sorted(vars(TD).items()) if n.startswith("test_") and callable(f)]

SOURCE_MUTANTS = {
    "no_embedding_scale": ("w.input_embedding_scale * decode_rows(E", "decode_rows(E"),
    "mask_slots_hold_anchor": ("tokens[:, 0] = anchors", "tokens[:, :] = np.asarray(anchors)[:, None]"),
    "block_positions_from_zero": ("pos = np.asarray(ctx_lens, dtype=np.int64)[:, None] + np.arange(bs)[None, :]",
                                  "pos = np.zeros((B, 1), dtype=np.int64) + np.arange(bs)[None, :]"),
    "context_not_attended": ("o[b] = attention(q, np.concatenate([kc, kb]), np.concatenate([vc, vb]))",
                             "o[b] = attention(q, kb, vb)"),
    "attention_residual_dropped": ("h = h + linear(o, layer.wo)", "h = linear(o, layer.wo)"),
    "ffn_residual_dropped": ("h = h + linear(act, layer.w_down)", "h = linear(act, layer.w_down)"),
    "ffn_conv_skipped": ("h = conv(h, layer.conv_ffn, layer.dconv_ffn)", "h = h"),
    "final_norm_skipped": ("nf = rmsnorm(h[:, 1:, :], decode(W.final_norm), w.rms_eps)", "nf = h[:, 1:, :]"),
    "logits_from_wrong_slots": ("nf = rmsnorm(h[:, 1:, :]", "nf = rmsnorm(h[:, :-1, :]"),
    "swiglu_halves_swapped": ("act = silu(gu[..., :w.ffn]) * gu[..., w.ffn:]",
                              "act = silu(gu[..., w.ffn:]) * gu[..., :w.ffn]"),
    "context_positions_shifted": ("pos[o0:o1] = int(ctx_lens[b]) - (o1 - o0) + np.arange(o1 - o0)",
                                  "pos[o0:o1] = int(ctx_lens[b]) - (o1 - o0) + 1 + np.arange(o1 - o0)"),
    "context_keys_unrotated": ("kk = rope(kv[:, :nkv * d].reshape(n_rows, nkv, d), pos, w.rope_theta)",
                               "kk = kv[:, :nkv * d].reshape(n_rows, nkv, d)"),
    "feature_norm_skipped": ("f = rmsnorm(linear(u, W.proj), decode(W.proj_norm), w.rms_eps)",
                             "f = linear(u, W.proj)"),
    "block_keys_unrotated": ("kb = rope(qkv[b, :, nq * d:(nq + nkv) * d].reshape(bs, nkv, d), pos[b], w.rope_theta)",
                             "kb = qkv[b, :, nq * d:(nq + nkv) * d].reshape(bs, nkv, d)"),
    "window_off_by_one": ("lo = max(0, L - w.sliding_window)", "lo = max(0, L - w.sliding_window + 1)"),
}


def _mutant_module(old, new):
    assert _SRC.count(old) == 1, f"mutation site not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(_SRC.replace(old, new), "<oracle mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("mutant", sorted(SOURCE_MUTANTS))
def test_composed_pins_catch_planted_mistake(mutant, monkeypatch):
    m = _mutant_module(*SOURCE_MUTANTS[mutant])
    for name in ("append_context", "draft_block", "step"):
        monkeypatch.setattr(O, name, getattr(m, name))
        monkeypatch.setattr(OD, name, getattr(m, name))
    for pin in DRAFT_PINS:
        try:
            pin()
        except AssertionError:
            return
    pytest.fail(f"no composed-forward pin noticed {mutant!r}")


def test_composed_pins_pass_on_an_unmutated_copy(monkeypatch):
    m = _mutant_module("def draft_block(", "def draft_block(")
    for name in ("append_context", "draft_block", "step"):
        monkeypatch.setattr(O, name, getattr(m, name))
        monkeypatch.setattr(OD, name, getattr(m, name))
    for pin in DRAFT_PINS:
        pin()
