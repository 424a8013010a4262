"""CPU oracle of the DFlash2 block draft -> select -> verify step.

TEST INFRASTRUCTURE.  This module is the plain, slow statement of what the
step computes.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import it; the GPU library never does, and nothing here is
shared with it (decoders, norms, RoPE, attention, ranking and the dynamic
program are all written out again below).

Sources (page title, section):
  [AM]  NeMo AutoModel, "Train a DFlash Drafter for Speculative Decoding":
        §What is DFlash?, §Variants (table, row "DFlash 2"), §Objective,
        §Data (note on mask_token_id), §Key Config Fields (table).
  [VL]  NeMo SpeechLM, "DFlash speculative decoding with vLLM":
        intro, §DFlash2 inference, §Validation.
  [LC]  llama-cpp-python wiki, "DFlash2 Speculative Decoding":
        §Prerequisites, §Configuration Notes.
  [NIM] NVIDIA NIM for Alpamayo, "DFlash2 Speculative Decoding":
        §Observe Acceptance (metrics fields table).

Precision: the network (context append, block forward, logits) runs in
float64 on the exact values of the stored inputs (bf16 and fp32 decode
exactly, fp8 decodes to code * scale).  Appended cache rows are rounded to
the cache dtype because the caller sees them.  Ranking (top-k), the selector
dynamic program and verification run in exact IEEE float32 with a fixed
operation order, so their integer outputs can be compared bit for bit.

Readings of points the pages leave open are labelled Q1..Q30 (the numbering
of the design notes); each function names the ones it takes.

Parity pins: every function except `draft_block`/`step` as a whole is pinned
by tests against brute force, closed forms or library special cases.  The
composition of the whole draft forward has no worked example on the pages:
parity unpinned for the composed network beyond its pinned parts and the
special-case invariants in tests/test_oracle_draft.py.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

# ----------------------------------------------------------------------------
# Decoding stored bytes into exact values (independent of the encoders).
# ----------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 is the top half of an IEEE binary32: widen and reinterpret."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u32.view(np.float32).astype(np.float64)


def fp8_e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3fn: sign, 4-bit exponent (bias 7), 3-bit mantissa; exponent 0
    is subnormal (m/8 * 2^-6); code 0x7F/0xFF is NaN; no infinities."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


def decode_rows(t, r0: int = 0, r1: Optional[int] = None) -> np.ndarray:
    """Exact float64 values of rows [r0, r1) of a stored tensor."""
    r1 = t.data.shape[0] if r1 is None else r1
    x = t.data[r0:r1]
    if t.dtype == "fp32":
        return x.astype(np.float64)
    if t.dtype == "bf16":
        return bf16_bits_to_f64(x)
    if t.dtype == "fp8":
        return fp8_e4m3fn_to_f64(x) * t.scale[r0:r1].astype(np.float64)[:, None]
    raise ValueError(t.dtype)


def decode(t) -> np.ndarray:
    return decode_rows(t)


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to what a cache of `dtype` stores (fp32 or bf16,
    nearest-even), returned as float64 values."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)  # IEEE RNE
    if dtype == "fp32":
        return x32.astype(np.float64)
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# Building blocks.
# ----------------------------------------------------------------------------


def linear(x: np.ndarray, w, rows: Optional[tuple] = None, chunk_elems: int = 1 << 26) -> np.ndarray:
    """y = x . W^T for a stored weight W[out, in] (row-major [out, in], as
    every linear of the draft is stored).  `rows` selects a contiguous block
    of output rows.  The weight is decoded a block of output rows at a time to
    bound memory; every output is a full-length dot product."""
    r0, r1 = (0, w.data.shape[0]) if rows is None else rows
    K = w.data.shape[1]
    step = max(1, chunk_elems // K)
    y = np.empty(x.shape[:-1] + (r1 - r0,), dtype=np.float64)
    x2 = x.reshape(-1, K)
    y2 = y.reshape(-1, r1 - r0)
    for a in range(r0, r1, step):
        b = min(r1, a + step)
        y2[:, a - r0:b - r0] = x2 @ decode_rows(w, a, b).T
    return y


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g.
    [AM §What is DFlash?: the draft trains its own norms; Q8: RMSNorm]."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding (Q14).  x [..., n, d] with one position
    per leading row n: for i < d/2 the pair (x_i, x_{i+d/2}) is rotated by the
    angle pos * theta^(-2i/d)."""
    d = x.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * theta ** (-2.0 * i / d)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    shape = (len(pos),) + (1,) * (x.ndim - 2) + (half,)
    c, s = c.reshape(shape), s.reshape(shape)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def block_conv(x: np.ndarray, taps: np.ndarray) -> np.ndarray:
    """In-block depthwise convolution in correction form (Q10-Q13):
    y[t] = x[t] + sum_{j<K} taps[j] * x[t-j], with x[t-j] = 0 before slot 0.
    [AM §Variants, DFlash 2: a two-tap in-block convolution around every
    sublayer; it never reaches outside the block]."""
    bs = x.shape[0]
    y = x.copy()
    for j in range(taps.shape[0]):
        y[j:] += taps[j] * x[:bs - j]
    return y


def dynamic_block_conv(x: np.ndarray, wc, kernel: int, group: int) -> np.ndarray:
    """In-block convolution with dynamic, group-shared taps (Readings D1-D3):
    slot t's taps c[t] = W x_t, reshaped [H / group, kernel] (row
    g * kernel + j of W is tap j of channel group g), and
    y[t, ch] = x[t, ch] + sum_{j<kernel} c[t, ch // group, j] * x[t-j, ch],
    with x[t-j] = 0 before slot 0.  [VL §DFlash2 inference: DFlash2 adds
    dynamic convolutions; AM §Key Config Fields: conv_kernel_size taps and
    conv_group_size channels per dynamic correction; AM §Variants: the
    convolution stays inside the block.]  x [bs, H] float64; wc a stored
    weight Tensor [(H / group) * kernel, H]."""
    bs, H = x.shape
    taps = linear(x, wc).reshape(bs, H // group, kernel)
    per_channel = np.repeat(taps, group, axis=1)          # [bs, H, kernel]
    y = x.copy()
    for j in range(kernel):
        y[j:] += per_channel[j:, :, j] * x[:bs - j]
    return y


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Unmasked (non-causal) softmax attention with grouped KV heads.
    q [T, nq, d], k/v [S, nkv, d] -> [T, nq, d].  q-head i reads kv head
    i // (nq / nkv).  [AM §What is DFlash?: the block is denoised in one
    non-causal pass]."""
    T, nq, d = q.shape
    nkv = k.shape[1]
    grp = nq // nkv
    out = np.empty_like(q)
    for i in range(nq):
        g = i // grp
        s = q[:, i, :] @ k[:, g, :].T / math.sqrt(d)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, i, :] = p @ v[:, g, :]
    return out


def logit_transform(x: np.ndarray, multiplier: float, softcap: float) -> np.ndarray:
    """The target's logit transform (Q16): m*x, then cap*tanh(x/cap) when a
    cap is set.  [AM §Key Config Fields: output_multiplier /
    final_logit_softcapping, identity unless set]."""
    y = multiplier * x
    if softcap > 0:
        y = softcap * np.tanh(y / softcap)
    return y


# ----------------------------------------------------------------------------
# O1: context append.
# ----------------------------------------------------------------------------


def new_cache(w, batch: int, k_init: Optional[np.ndarray] = None, v_init=None):
    """float64 K and V caches [nL, B, nkv, Lmax, d] (logical row order),
    optionally initialised from stored rows (fp32 values or bf16 bits)."""
    shape = (w.num_layers, batch, w.num_kv_heads, w.max_context, w.head_dim)

    def conv(a):
        if a is None:
            return np.zeros(shape)
        return a.astype(np.float64) if a.dtype == np.float32 else bf16_bits_to_f64(a)
    return conv(k_init), conv(v_init)


def append_context(w, W, k_cache, v_cache, taps, new_offsets, ctx_lens) -> np.ndarray:
    """Project the target hidden-state taps of the newly verified positions
    and write every layer's context keys/values.

    [AM §What is DFlash?: the draft is conditioned on hidden states taken
    from the frozen target at target_layer_ids and owns a feature
    projection; LC §Tips: the draft keeps its own context.]
    Readings: Q4 taps concatenated on the feature axis in target_layer_ids
    order; Q5 one bias-free projection then RMSNorm; Q6 each layer projects
    the same feature with its own K/V rows of W_qkv, K stored after RoPE;
    Q2 new rows sit at positions L - n_new .. L - 1.
    Returns the normalised features f [sum n_new, H]."""
    nq, nkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
    tv = decode(taps)
    n_rows = tv.shape[0]
    if n_rows == 0:
        return np.zeros((0, w.hidden))
    u = tv.reshape(n_rows, w.num_taps * w.tap_width)
    f = rmsnorm(linear(u, W.proj), decode(W.proj_norm), w.rms_eps)
    pos = np.empty(n_rows, dtype=np.int64)
    seq = np.empty(n_rows, dtype=np.int64)
    for b in range(len(ctx_lens)):
        o0, o1 = int(new_offsets[b]), int(new_offsets[b + 1])
        pos[o0:o1] = int(ctx_lens[b]) - (o1 - o0) + np.arange(o1 - o0)
        seq[o0:o1] = b
    for l, layer in enumerate(W.layers):
        kv = linear(f, layer.wqkv, rows=(nq * d, (nq + 2 * nkv) * d))
        kk = rope(kv[:, :nkv * d].reshape(n_rows, nkv, d), pos, w.rope_theta)
        vv = kv[:, nkv * d:].reshape(n_rows, nkv, d)
        kk = round_to_storage(kk, w.act_dtype)
        vv = round_to_storage(vv, w.act_dtype)
        for r in range(n_rows):
            k_cache[l, seq[r], :, pos[r], :] = kk[r]
            v_cache[l, seq[r], :, pos[r], :] = vv[r]
    return f


# ----------------------------------------------------------------------------
# O2-O4: block forward and logits.
# ----------------------------------------------------------------------------


def draft_block(w, W, k_cache, v_cache, anchors, ctx_lens) -> Dict[str, np.ndarray]:
    """One non-causal forward of the draft over a block per sequence.

    [AM §What is DFlash?: slot 0 is the real anchor token, the other slots
    hold MASK, the whole block is denoised in one non-causal pass using the
    target's frozen embed_tokens and lm_head; AM §Data: the mask id is a
    reserved token; AM §Variants: DFlash 2 adds a two-tap in-block
    convolution around every sublayer; AM §Key Config Fields:
    input_embedding_scale, output_multiplier / final_logit_softcapping,
    draft_sliding_window.]
    Readings: Q1 slot t predicts the token at slot t; Q2 slot t sits at
    position L + t; Q3 context = projected taps only; Q13 conv before each
    sublayer's pre-norm on the residual stream, none before the final norm;
    Q14 RoPE; Q15 SwiGLU; Q18 logits for slots 1..bs-1 only.

    Returns zeta [B, bs-1, V] (float64 logits before the transform) and
    h_final [B, bs, H] (residual stream after the last layer)."""
    B, bs, H = len(anchors), w.block_size, w.hidden
    nq, nkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
    tokens = np.full((B, bs), w.mask_token_id, dtype=np.int64)
    tokens[:, 0] = anchors
    E = W.embed
    h = np.stack([w.input_embedding_scale * decode_rows(E, int(t), int(t) + 1)[0]
                  for t in tokens.reshape(-1)]).reshape(B, bs, H)
    pos = np.asarray(ctx_lens, dtype=np.int64)[:, None] + np.arange(bs)[None, :]
    G = getattr(w, "conv_group_size", 0)

    def conv(x, static, dyn):
        if G > 0:
            return np.stack([dynamic_block_conv(x[b], dyn, w.conv_kernel_size, G) for b in range(B)])
        taps = decode(static)
        return np.stack([block_conv(x[b], taps) for b in range(B)])

    for l, layer in enumerate(W.layers):
        h = conv(h, layer.conv_attn, layer.dconv_attn)
        n = rmsnorm(h, decode(layer.attn_norm), w.rms_eps)
        qkv = linear(n, layer.wqkv)                       # [B, bs, (nq+2nkv)d]
        o = np.empty((B, bs, nq * d))
        for b in range(B):
            L = int(ctx_lens[b])
            q = rope(qkv[b, :, :nq * d].reshape(bs, nq, d), pos[b], w.rope_theta)
            kb = rope(qkv[b, :, nq * d:(nq + nkv) * d].reshape(bs, nkv, d), pos[b], w.rope_theta)
            vb = qkv[b, :, (nq + nkv) * d:].reshape(bs, nkv, d)
            lo = max(0, L - w.sliding_window) if w.sliding_window > 0 else 0
            kc = k_cache[l, b, :, lo:L, :].transpose(1, 0, 2)  # [S, nkv, d]
            vc = v_cache[l, b, :, lo:L, :].transpose(1, 0, 2)
            o[b] = attention(q, np.concatenate([kc, kb]), np.concatenate([vc, vb])).reshape(bs, nq * d)
        h = h + linear(o, layer.wo)
        h = conv(h, layer.conv_ffn, layer.dconv_ffn)
        n = rmsnorm(h, decode(layer.ffn_norm), w.rms_eps)
        gu = linear(n, layer.w_gate_up)
        act = silu(gu[..., :w.ffn]) * gu[..., w.ffn:]
        h = h + linear(act, layer.w_down)
    nf = rmsnorm(h[:, 1:, :], decode(W.final_norm), w.rms_eps)
    zeta = linear(nf, W.lm_head)
    return {"zeta": zeta, "h_final": h}


# ----------------------------------------------------------------------------
# O5: top-k candidates per block position.
# ----------------------------------------------------------------------------


def canonical_f32(x: np.ndarray) -> np.ndarray:
    """float32 keys with -0.0 turned into +0.0 (Q23)."""
    return np.asarray(x, dtype=np.float32) + np.float32(0.0)


def topk(keys32: np.ndarray, k: int):
    """The k largest entries of each row under (value desc, id asc), in that
    order, found by k rounds of "take the first maximum, then strike it out"
    (Q23).  keys32 [R, V] float32.  [AM §Variants: the selector walks each
    position's top-k candidates; LC §Configuration Notes: selector_top_k is
    fixed by the head]."""
    x = canonical_f32(keys32).astype(np.float64)
    R = x.shape[0]
    ids = np.empty((R, k), dtype=np.int32)
    vals = np.empty((R, k), dtype=np.float32)
    taken = np.zeros(x.shape, dtype=bool)
    rows = np.arange(R)
    for j in range(k):
        masked = np.where(taken, -np.inf, x)
        a = np.argmax(masked, axis=1)        # first occurrence: smallest id among equals
        ids[:, j] = a
        vals[:, j] = x[rows, a]
        taken[rows, a] = True
    return ids, vals


# ----------------------------------------------------------------------------
# O6: pairwise low-rank path selector.
# ----------------------------------------------------------------------------


def pair_scores(tl: np.ndarray, tr: np.ndarray, a_ids: np.ndarray, b_ids: np.ndarray) -> np.ndarray:
    """pi(a, b) = sum_m Tl[a, m] * Tr[b, m] in float32, multiply then add,
    m ascending from +0 (Q21, Q25).  Returns [len(a), len(b)] float32."""
    A = tl[np.asarray(a_ids)].astype(np.float32)      # [na, r]
    Bm = tr[np.asarray(b_ids)].astype(np.float32)     # [nb, r]
    acc = np.zeros((A.shape[0], Bm.shape[0]), dtype=np.float32)
    for m in range(A.shape[1]):
        prod = (A[:, m][:, None] * Bm[:, m][None, :]).astype(np.float32)
        acc = (acc + prod).astype(np.float32)
    return acc


def select_path(anchors, cand_ids, cand_vals, tl, tr) -> Dict[str, np.ndarray]:
    """Max-sum (Viterbi) path through the per-position candidate lattice.

    [AM §Variants: a pairwise path selector picks one coherent path through
    every position's top-k; AM §Objective: each position's candidates are
    scored against the ground-truth predecessor; LC §Complete Runnable Code: the selector
    lattice replaces vocabulary sampling.]
    Readings: Q19 first-order chain starting at the anchor; Q20 unary term =
    the candidate's logit; Q21 pair term = rank-r bilinear form through the
    factor tables; Q26 the smallest predecessor index wins a tie, and the
    smallest final index.  Arithmetic in float32:
        S_1[j] = pi(c0, c_1j) + z_1j
        S_t[j] = max_i (S_{t-1}[i] + pi(c_{t-1,i}, c_tj)) + z_tj
    cand_ids/cand_vals [B, P, k]; returns path [B, P] (candidate ranks),
    drafts [B, P] (token ids), score [B] float32 and pair [B, P, k, k]
    (row i of slab 0 repeats pi(c0, .))."""
    cand_ids = np.asarray(cand_ids)
    cand_vals = np.asarray(cand_vals, dtype=np.float32)
    B, P, k = cand_ids.shape
    path = np.empty((B, P), dtype=np.int32)
    drafts = np.empty((B, P), dtype=np.int32)
    score = np.empty(B, dtype=np.float32)
    pair = np.empty((B, P, k, k), dtype=np.float32)
    for b in range(B):
        p0 = pair_scores(tl, tr, [int(anchors[b])], cand_ids[b, 0])[0]
        pair[b, 0] = p0[None, :]
        S = (p0 + cand_vals[b, 0]).astype(np.float32)
        back = np.zeros((P, k), dtype=np.int64)
        for t in range(1, P):
            pt = pair_scores(tl, tr, cand_ids[b, t - 1], cand_ids[b, t])
            pair[b, t] = pt
            tot = (S[:, None] + pt).astype(np.float32)       # [i, j]
            bi = np.argmax(tot, axis=0)                      # first max over i
            back[t] = bi
            S = (tot[bi, np.arange(k)] + cand_vals[b, t]).astype(np.float32)
        j = int(np.argmax(S))
        score[b] = S[j]
        for t in range(P - 1, -1, -1):
            path[b, t] = j
            drafts[b, t] = cand_ids[b, t, j]
            j = int(back[t, j])
    return {"path": path, "drafts": drafts, "score": score, "pair": pair}


# ----------------------------------------------------------------------------
# O7: greedy verification.
# ----------------------------------------------------------------------------


def verify_accept(drafts, target_logits) -> Dict[str, np.ndarray]:
    """Longest accepted prefix under greedy verification.

    [VL intro and §Validation: the target checks the drafts and accepted
    output equals the target's greedy output; LC §Prerequisites: the target
    scores [last id, drafts...] in one batch; NIM §Observe Acceptance: the
    verified token counts towards each step's output.]
    Reading Q27: row i of the target logits is the target's prediction after
    block slot i; draft d_{i+1} (drafts[:, i]) is accepted while it equals
    that row's argmax; the bonus token is the argmax of the first row that
    disagrees (row bs-1 when every draft is accepted).  Argmax ties go to the
    smallest id after -0.0 -> +0.0."""
    drafts = np.asarray(drafts)
    z = canonical_f32(target_logits)
    B, bs, V = z.shape
    g = np.argmax(z, axis=2).astype(np.int32)
    accepted = np.zeros(B, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = 0
        while n < bs - 1 and g[b, n] == drafts[b, n]:
            n += 1
        accepted[b] = n
        bonus[b] = g[b, n]
    return {"accepted": accepted, "bonus": bonus, "argmax": g}


# ----------------------------------------------------------------------------
# O8: draft length from the selector's transition confidence.
# ----------------------------------------------------------------------------


def path_confidence(anchors, cand_ids, cand_vals, path, tl, tr) -> np.ndarray:
    """Confidence of each transition the chosen path takes.

    [LC §Configuration Notes: a positive draft_p_min stops a path before a
    low-confidence selector transition.]  Reading S6: at position t the
    selector's local choice among the k candidates, given the predecessor the
    path took (the anchor at t = 0), scores candidate j with the lattice's own
    float32 transition score s_j = pi(c_prev, c_tj) + z_tj; the confidence is
    the softmax of those k scores at the chosen candidate, evaluated here in
    float64 on the float32 scores.  Returns conf [B, P] float64."""
    cand_ids = np.asarray(cand_ids)
    cand_vals = np.asarray(cand_vals, dtype=np.float32)
    path = np.asarray(path)
    B, P, k = cand_ids.shape
    conf = np.empty((B, P), dtype=np.float64)
    for b in range(B):
        prev = int(anchors[b])
        for t in range(P):
            s = (pair_scores(tl, tr, [prev], cand_ids[b, t])[0] + cand_vals[b, t]).astype(np.float32)
            s = s.astype(np.float64)
            w = np.exp(s - s.max())
            j = int(path[b, t])
            conf[b, t] = w[j] / w.sum()
            prev = int(cand_ids[b, t, j])
    return conf


def draft_lengths(conf, p_min: float, n_min: int = 0, n_max: Optional[int] = None) -> np.ndarray:
    """Number of drafts proposed per sequence.

    [LC §Configuration Notes: draft_p_min stops the path before a transition
    whose confidence is below it; draft_n_max caps the draft length at
    block_size - 1; LC §Complete Runnable Code: SpecConfig also carries
    draft_n_min.]  Reading S7: n_max is clamped to [0, P] and n_min to
    [0, n_max]; the path stops at the first position t >= n_min whose
    confidence is below p_min (drafts 0..t-1 are proposed), else at P, and
    never runs past n_max.  p_min = 0 never stops a path."""
    conf = np.asarray(conf, dtype=np.float64)
    B, P = conf.shape
    hi = P if n_max is None else min(max(int(n_max), 0), P)
    lo = min(max(int(n_min), 0), hi)
    out = np.empty(B, dtype=np.int32)
    for b in range(B):
        n = P
        for t in range(lo, P):
            if conf[b, t] < p_min:
                n = t
                break
        out[b] = min(n, hi)
    return out


def verify_accept_len(drafts, target_logits, draft_lens) -> Dict[str, np.ndarray]:
    """Greedy verification of a path cut to draft_lens[b] drafts: the
    accepted prefix stops at the length, and the bonus is the argmax of the
    row after the last accepted draft (row draft_lens[b] when all are
    accepted).  Same tie and -0.0 rules as verify_accept (Q23, Q27)."""
    drafts = np.asarray(drafts)
    z = canonical_f32(target_logits)
    B, bs, V = z.shape
    g = np.argmax(z, axis=2).astype(np.int32)
    accepted = np.zeros(B, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = 0
        while n < int(draft_lens[b]) and g[b, n] == drafts[b, n]:
            n += 1
        accepted[b] = n
        bonus[b] = g[b, n]
    return {"accepted": accepted, "bonus": bonus, "argmax": g}


# ----------------------------------------------------------------------------
# O9: sampled (rejection) verification.
# ----------------------------------------------------------------------------

F32_MAX = float(np.finfo(np.float32).max)


def clean_logits(z) -> np.ndarray:
    """Reading S2: NaN -> -inf (probability 0), +inf -> the largest float32,
    -0.0 -> +0.0; float32 inputs widened exactly to float64."""
    x = np.asarray(z, dtype=np.float32).astype(np.float64)
    x = np.where(np.isnan(x), -np.inf, x)
    x = np.minimum(x, F32_MAX)
    return x + 0.0


def target_distribution(z_row, temperature: float, top_k: int = 0, top_p: float = 1.0) -> np.ndarray:
    """The target's sampling distribution for one row of its logits, float64.

    [AM §Key Config Fields, paragraph on spec_generate: temperature, top_p and
    top_k truncate the target's own distribution, the one the drafts are
    verified against; the DFlash 2 acceptance figures use temperature 1.0,
    top-p 0.95, top-k 20.]  Readings:
      S1  temperature 0 is greedy: a point mass on the row's argmax (ties to
          the smallest id), the rule of the greedy verification;
      S2  logits cleaned by clean_logits;
      S3  weights e_v = exp((z_v - m) / T) with m the row maximum, and
          e_v = 1 for every entry equal to m (so a row without a finite logit
          is uniform over its entries);
      S4  top-k (0 = off, >= V = off) keeps every entry whose value is at
          least the k-th largest value counted with multiplicity, so an entry
          tied with the k-th is kept;
      S5  top-p (>= 1 = off) is applied after top-k: a kept entry stays when
          the kept mass strictly above its value is below top_p times the
          kept mass (the smallest prefix by value reaching top_p, with a
          value group kept or dropped whole).
    Returns p [V] summing to 1."""
    z = clean_logits(z_row)
    V = z.size
    if temperature == 0:
        zc = canonical_f32(np.asarray(z_row, dtype=np.float32)).astype(np.float64)
        nan = np.isnan(zc)
        g = 0
        if not nan.all():
            zz = np.where(nan, -np.inf, zc)
            g = int(np.nonzero(~nan & (zz == zz[~nan].max()))[0][0])
        p = np.zeros(V)
        p[g] = 1.0
        return p
    e, keep = _weights_top_k(z, temperature, top_k)
    if top_p < 1.0:
        S = e[keep].sum()
        above = _mass_strictly_above(z, e, keep)
        keep &= above < top_p * S
    p = np.where(keep, e, 0.0)
    return p / p.sum()


def _weights_top_k(z, temperature, top_k):
    """Readings S3 and S4 on cleaned logits: weights and the top-k kept mask."""
    m = z.max()
    with np.errstate(invalid="ignore", over="ignore"):
        e = np.exp((z - m) / temperature)
    e[z == m] = 1.0
    keep = np.ones(z.size, dtype=bool)
    if 0 < top_k < z.size:
        kth = np.sort(z)[::-1][top_k - 1]
        keep &= z >= kth
    return e, keep


def target_distributions_near(z_row, temperature: float, top_k: int = 0, top_p: float = 1.0,
                              band: float = 0.0) -> list:
    """Every distribution target_distribution would give if the top-p bound
    were moved anywhere within [top_p - band, top_p + band] (a value group
    whose kept mass above lies that close to the bound may be kept or
    dropped by an evaluation with rounding error below band).  The first
    entry is target_distribution itself."""
    exact = target_distribution(z_row, temperature, top_k, top_p)
    if temperature == 0 or top_p >= 1.0 or band <= 0:
        return [exact]
    z = clean_logits(z_row)
    e, keep = _weights_top_k(z, temperature, top_k)
    S = e[keep].sum()
    frac = _mass_strictly_above(z, e, keep) / S
    out, seen = [exact], {int(np.count_nonzero(exact))}
    levels = np.unique(frac[keep])
    cuts = [top_p - band] + [float(np.nextafter(L, 2.0)) for L in levels if top_p - band < L <= top_p + band]
    for c in cuts:
        kp = keep & (frac < c)
        if not kp.any() or int(np.count_nonzero(kp)) in seen:
            continue
        seen.add(int(np.count_nonzero(kp)))
        q = np.where(kp, e, 0.0)
        out.append(q / q.sum())
    return out


def _mass_strictly_above(z, e, keep) -> np.ndarray:
    """For every kept entry, the kept mass of strictly larger values (value
    groups summed with np.unique, then accumulated from the top)."""
    vals, inv = np.unique(z[keep], return_inverse=True)       # ascending
    group_mass = np.bincount(inv, weights=e[keep], minlength=vals.size)
    above_group = np.cumsum(group_mass[::-1])[::-1] - group_mass   # larger values only
    above = np.zeros(z.size)
    above[keep] = above_group[inv]
    return above


def inverse_cdf(p: np.ndarray, v: float) -> int:
    """The smallest id j with sum_{i <= j} p_i > v, ids ascending (Reading
    S8); no such j (only for v >= 1) gives the id of the largest p, ties to
    the smallest id."""
    c = np.cumsum(p)
    hit = np.nonzero(c > v)[0]
    return int(hit[0]) if hit.size else int(np.argmax(p))


def verify_sample(drafts, target_logits, uniforms, temperature: float, top_k: int = 0,
                  top_p: float = 1.0, draft_lens=None) -> Dict[str, np.ndarray]:
    """Rejection-sampling verification of one deterministic draft path.

    [AM §Key Config Fields: drafts are verified by rejection sampling against
    the target's (truncated) distribution, so sampled decoding keeps the
    target's output distribution; LC §Configuration Notes: the DFlash2 path
    comes from the selector lattice, not from a vocabulary sampler.]  The
    rule is speculative sampling (Leviathan, Kalman and Matias 2023; Chen et
    al. 2023) with the draft distribution q_i a point mass on d_i
    (Reading S9): draft i is accepted when u_i < min(1, p_i(d_i) / q_i(d_i))
    = p_i(d_i); at the first rejection the bonus is drawn from max(p_i - q_i,
    0) normalised (p_i with d_i struck out); when every proposed draft is
    accepted the bonus is drawn from the next row's p.  Draws use
    inverse_cdf with v = uniforms[b, bs-1].

    uniforms [B, bs]: u_i for draft i in columns 0..bs-2, v in column bs-1.
    draft_lens [B] (None = bs-1) cuts each path.
    Returns accepted, bonus, draft_prob [B, bs-1] (p_i(d_i) for i below the
    length, 0 beyond) and margin [B]: the smallest distance of any uniform
    from the threshold it was compared with, for the decisions this sequence
    took (target_distributions_near covers the top-p bound)."""
    drafts = np.asarray(drafts)
    z = np.asarray(target_logits, dtype=np.float32)
    u = np.asarray(uniforms, dtype=np.float32).astype(np.float64)
    assert np.all((u >= 0) & (u < 1)), "uniforms lie in [0, 1)"
    exact = temperature == 0          # point masses: no rounding-sensitive decision
    B, bs, V = z.shape
    P = bs - 1
    lens = np.full(B, P) if draft_lens is None else np.asarray(draft_lens)
    accepted = np.zeros(B, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    draft_prob = np.zeros((B, P))
    margin = np.full(B, np.inf)
    for b in range(B):
        n_len = int(lens[b])
        n = 0
        dist = None
        while n <= n_len:
            p = target_distribution(z[b, n], temperature, top_k, top_p)
            if n == n_len:
                dist = p
                break
            d = int(drafts[b, n])
            q = np.zeros(V)
            q[d] = 1.0
            pd = p[d]
            draft_prob[b, n] = pd
            if not exact:
                margin[b] = min(margin[b], abs(u[b, n] - min(1.0, pd / q[d])))
            if u[b, n] < min(1.0, pd / q[d]):
                n += 1
                continue
            r = np.maximum(p - q, 0.0)
            dist = r / r.sum()
            break
        for i in range(n + 1, n_len):
            p = target_distribution(z[b, i], temperature, top_k, top_p)
            draft_prob[b, i] = p[int(drafts[b, i])]
        accepted[b] = n
        v = u[b, P]
        bonus[b] = inverse_cdf(dist, v)
        c = np.cumsum(dist)
        j = int(bonus[b])
        lo = c[j - 1] if j > 0 else 0.0
        if not exact:
            margin[b] = min(margin[b], abs(c[j] - v), abs(v - lo))
    return {"accepted": accepted, "bonus": bonus, "draft_prob": draft_prob, "margin": margin}


def top_p_margin(z_row, temperature, top_k, top_p) -> float:
    """Distance of the top-p decision nearest its bound, as a fraction of the
    kept mass (inf when top-p is off or the temperature is 0)."""
    if top_p >= 1.0 or temperature == 0:
        return np.inf
    z = clean_logits(z_row)
    e, keep = _weights_top_k(z, temperature, top_k)
    S = e[keep].sum()
    before = _mass_strictly_above(z, e, keep)[keep] / S
    return float(np.min(np.abs(before - top_p)))


# ----------------------------------------------------------------------------
# O10: training-side forward losses.
# ----------------------------------------------------------------------------


def position_weights(block_size: int, gamma: float) -> np.ndarray:
    """w_k = exp(-(k - 1) / gamma) for supervised slots k = 1 .. bs-1
    ([AM §Objective]); gamma = inf gives equal weights."""
    k = np.arange(1, block_size, dtype=np.float64)
    return np.exp(-(k - 1.0) / gamma)


def block_losses(anchors, labels, logits, cand_ids, cand_vals, tl, tr, gamma: float,
                 selector_loss_weight: float, multiplier: float = 1.0, softcap: float = 0.0) -> Dict:
    """The DFlash 2 training objective evaluated forward on given logits.

    [AM §Objective: slots 1..bs-1 are supervised, their cross-entropy
    weighted by exp(-(k-1)/loss_decay_gamma); DFlash 2 adds, weighted by
    selector_loss_weight, a cross-entropy over each position's top-k
    candidates scored against the ground-truth predecessor; positions whose
    true token missed the candidates carry no selector signal and are
    reported as candidate_recall.  AM §Key Config Fields: the logit
    transform applies in training too.]  Readings:
      L1  logits [B, bs-1, V] are the pre-transform float32 logits; CE uses
          the transformed ones (logit_transform), in float64;
      L2  labels [B, bs-1] are the true tokens of slots 1..bs-1; a label
          outside [0, V) marks a position as unsupervised (no terms, not
          counted anywhere);
      L3  block loss = sum_k w_k CE_k / sum_k w_k over supervised positions;
      L4  selector score of candidate j at slot k: the lattice's float32
          pi(true_{k-1}, c_kj) + z_kj, with true_0 = the anchor and true_{k-1}
          = label_{k-1}; CE_sel = logsumexp_j s - s_true (float64 on the
          float32 scores); a position has a selector signal when its label is
          among its candidates and its predecessor is known (anchor, or a
          supervised label);
      L5  selector loss = mean CE_sel over positions with a signal (0 when
          none); candidate_recall = supervised positions whose label is among
          the candidates / supervised positions; total = block loss +
          selector_loss_weight * selector loss.
    Returns block_ce [B, P], selector_ce [B, P] (NaN without a signal),
    in_cands [B, P] bool and the scalars total, block, selector, recall."""
    labels = np.asarray(labels)
    z = np.asarray(logits, dtype=np.float32)
    cand_ids = np.asarray(cand_ids)
    cand_vals = np.asarray(cand_vals, dtype=np.float32)
    B, P, V = z.shape
    zt = logit_transform(z.astype(np.float64), multiplier, softcap)
    w = position_weights(P + 1, gamma)
    block_ce = np.full((B, P), np.nan)
    sel_ce = np.full((B, P), np.nan)
    in_c = np.zeros((B, P), dtype=bool)
    num = den = 0.0
    sel_sum, sel_n, sup_n, hit_n = 0.0, 0, 0, 0
    for b in range(B):
        for k in range(P):
            lab = int(labels[b, k])
            if not 0 <= lab < V:
                continue
            row = zt[b, k]
            m = row.max()
            lse = m + np.log(np.exp(row - m).sum())
            block_ce[b, k] = lse - row[lab]
            num += w[k] * block_ce[b, k]
            den += w[k]
            sup_n += 1
            hit = np.nonzero(cand_ids[b, k] == lab)[0]
            if hit.size == 0:
                continue
            in_c[b, k] = True
            hit_n += 1
            prev = int(anchors[b]) if k == 0 else int(labels[b, k - 1])
            if not 0 <= prev < V:
                continue
            s = (pair_scores(tl, tr, [prev], cand_ids[b, k])[0] + cand_vals[b, k]).astype(np.float32)
            s = s.astype(np.float64)
            ms = s.max()
            sel_ce[b, k] = ms + np.log(np.exp(s - ms).sum()) - s[int(hit[0])]
            sel_sum += sel_ce[b, k]
            sel_n += 1
    block = num / den if den > 0 else 0.0
    selector = sel_sum / sel_n if sel_n else 0.0
    recall = hit_n / sup_n if sup_n else 0.0
    return {"block_ce": block_ce, "selector_ce": sel_ce, "in_cands": in_c, "block": block,
            "selector": selector, "recall": recall, "total": block + selector_loss_weight * selector}


# ----------------------------------------------------------------------------
# The whole step.
# ----------------------------------------------------------------------------


def step(w, W, inp, target_logits_fn=None) -> Dict[str, np.ndarray]:
    """O1..O7 for the sequences in `inp`.  `target_logits_fn(drafts)`
    supplies the verifier's logits for the chosen drafts (None skips
    verification)."""
    B = len(inp.anchors)
    k_cache, v_cache = new_cache(w, B, inp.k_ctx, inp.v_ctx)
    f = append_context(w, W, k_cache, v_cache, inp.taps, inp.new_offsets, inp.ctx_lens)
    fwd = draft_block(w, W, k_cache, v_cache, inp.anchors, inp.ctx_lens)
    zeta = fwd["zeta"]
    keys32 = zeta.astype(np.float32).reshape(-1, w.vocab)
    ids, _ = topk(keys32, w.top_k)
    z = logit_transform(zeta, w.output_multiplier, w.final_logit_softcapping).astype(np.float32)
    z = z.reshape(-1, w.vocab)
    vals = np.take_along_axis(z, ids.astype(np.int64), axis=1)
    P = w.block_size - 1
    ids = ids.reshape(B, P, w.top_k)
    vals = vals.reshape(B, P, w.top_k)
    sel = select_path(inp.anchors, ids, vals, W.sel_tl.data, W.sel_tr.data)
    out = {"f": f, "k_cache": k_cache, "v_cache": v_cache, "zeta": zeta,
           "h_final": fwd["h_final"], "topk_ids": ids, "topk_vals": vals, **sel}
    if target_logits_fn is not None:
        tl = target_logits_fn(sel["drafts"])
        out.update(verify_accept(sel["drafts"], tl))
        out["target_logits"] = tl
    return out


# ----------------------------------------------------------------------------
# The steps either side of the path: a multi-step decode loop.
# ----------------------------------------------------------------------------


def decode_loop(w, W, inp, steps: int, target_logits_fn, verified_taps_fn, sampling=None,
                uniforms_fn=None, p_min=None, n_min: int = 0, n_max=None) -> Dict[str, list]:
    """`steps` draft -> select -> verify rounds with the state carried over.

    [LC §Prerequisites and §Complete Runnable Code: the target scores the
    last verified token plus the drafts in one batch, the accepted prefix
    and the target's own next token are emitted; NIM §Observe Acceptance:
    per-step accepted counts and the verified token; AM §What is DFlash?:
    the draft is conditioned on the target's hidden states of verified
    positions.]  Reading Q2: after a step that accepts a drafts, the
    target has verified the anchor and those a drafts, so their a + 1
    positions (L .. L + a) are appended next step, the context grows to
    L + a + 1 and the target's next token (the bonus) is the new anchor.
    The block's own keys are never kept (no draft-side rollback).

    target_logits_fn(step, drafts) -> [B, bs, V] float32 verifier logits;
    verified_taps_fn(starts, counts) -> (taps Tensor, offsets) for positions
    starts[b] .. starts[b] + counts[b] - 1.  sampling = (temperature, top_k,
    top_p) verifies by rejection sampling (O9) with uniforms_fn(step) ->
    [B, bs]; p_min cuts each path with the confidence rule (O8).  Returns
    per-step lists of drafts, lens, accepted, bonus, ctx_lens (before the
    step) and margin (sampled decisions' distance from their thresholds)."""
    B = len(inp.anchors)
    k_cache, v_cache = new_cache(w, B, inp.k_ctx, inp.v_ctx)
    anchors = np.asarray(inp.anchors).copy()
    ctx = np.asarray(inp.ctx_lens).astype(np.int64).copy()
    taps, offsets = inp.taps, np.asarray(inp.new_offsets)
    P = w.block_size - 1
    rec = {"drafts": [], "lens": [], "accepted": [], "bonus": [], "ctx_lens": [], "margin": []}
    for s in range(steps):
        append_context(w, W, k_cache, v_cache, taps, offsets, ctx)
        fwd = draft_block(w, W, k_cache, v_cache, anchors, ctx)
        zeta = fwd["zeta"]
        ids, _ = topk(zeta.astype(np.float32).reshape(-1, w.vocab), w.top_k)
        z = logit_transform(zeta, w.output_multiplier, w.final_logit_softcapping).astype(np.float32)
        vals = np.take_along_axis(z.reshape(-1, w.vocab), ids.astype(np.int64), axis=1)
        ids3, vals3 = ids.reshape(B, P, w.top_k), vals.reshape(B, P, w.top_k)
        sel = select_path(anchors, ids3, vals3, W.sel_tl.data, W.sel_tr.data)
        lens = np.full(B, P, dtype=np.int32)
        if p_min is not None:
            conf = path_confidence(anchors, ids3, vals3, sel["path"], W.sel_tl.data, W.sel_tr.data)
            lens = draft_lengths(conf, p_min, n_min, n_max)
        tz = target_logits_fn(s, sel["drafts"])
        if sampling is None:
            ver = verify_accept_len(sel["drafts"], tz, lens)
            ver["margin"] = np.full(B, np.inf)
        else:
            ver = verify_sample(sel["drafts"], tz, uniforms_fn(s), *sampling, draft_lens=lens)
        rec["drafts"].append(sel["drafts"])
        rec["lens"].append(lens)
        rec["margin"].append(ver["margin"])
        rec["accepted"].append(ver["accepted"])
        rec["bonus"].append(ver["bonus"])
        rec["ctx_lens"].append(ctx.copy())
        n_new = ver["accepted"].astype(np.int64) + 1
        taps, offsets = verified_taps_fn(ctx, n_new)
        ctx = ctx + n_new
        anchors = ver["bonus"].astype(np.int32)
    return rec

