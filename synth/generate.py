"""Seeded synthetic inputs for the DFlash2 draft -> select -> verify step.

Every tensor is drawn from its own numpy stream
``default_rng([20261202, workload.index, tensor_id, chunk])`` in fixed-size
chunks, so the bytes do not depend on thread count or machine.  Weights are
N(0, 0.02^2) (stored as fp32, bf16 or fp8 e4m3fn + per-row scale), tap
activations and pre-existing cache rows N(0, 1), anchors uniform over the
vocabulary minus the reserved mask id, and verifier logits N(0, 1) with a
planted argmax that agrees with a given draft path with the workload's
per-position probability.

Nothing here computes any step of the method; it only makes inputs.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional

import numpy as np

from .codecs import f32_to_bf16_bits, f32_to_fp8_rowwise
from .configs import Workload

SEED = 20261202
CHUNK = 1 << 22

# tensor ids (seed components)
T_EMBED, T_LMHEAD, T_PROJ, T_PROJ_NORM, T_FINAL_NORM, T_SEL_L, T_SEL_R = range(7)
L_CONV_ATTN, L_ATTN_NORM, L_WQKV, L_WO, L_CONV_FFN, L_FFN_NORM, L_WGU, L_WDOWN, L_DCONV_ATTN, L_DCONV_FFN = range(10)
S_ANCHOR, S_CTXLEN, S_ACCEPT, S_TAPS, S_KCACHE, S_VCACHE = range(1000, 1006)
S_VERIFIED_TAPS = 1006
V_LOGITS, V_PLANT = 2000, 2001
V_SAMPLE_LOGITS, V_SAMPLE_PLANT, V_UNIFORM = 2002, 2003, 2004
X_SEL_IDS, X_SEL_VALS, X_SEL_ANCH = 3000, 3001, 3002


def _layer_tid(layer: int, which: int) -> int:
    return 100 + 10 * layer + which


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal(shape, seed_key, std: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2) of the given shape, chunked over the flat index."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(c):
        s, e = c * CHUNK, min(n, (c + 1) * CHUNK)
        rng = np.random.default_rng([SEED, *seed_key, c])
        rng.standard_normal(e - s, dtype=np.float32, out=out[s:e])
        if std != 1.0:
            out[s:e] *= np.float32(std)

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


def _bf16_threaded(x: np.ndarray) -> np.ndarray:
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    n = flat.size
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(c):
        s, e = c * CHUNK, min(n, (c + 1) * CHUNK)
        out[s:e] = f32_to_bf16_bits(flat[s:e])

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(nchunks)))
    return out.reshape(x.shape)


def _fp8_threaded(x: np.ndarray):
    n_rows = x.shape[0]
    rows = max(1, CHUNK // max(1, x.shape[1]))
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(n_rows, dtype=np.float32)

    def work(r0):
        r1 = min(n_rows, r0 + rows)
        codes[r0:r1], scales[r0:r1] = f32_to_fp8_rowwise(x[r0:r1])

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(0, n_rows, rows)))
    return codes, scales


@dataclasses.dataclass
class Tensor:
    """Stored bytes of one tensor: fp32 values, bf16 bits (uint16) or fp8
    e4m3fn bits (uint8) with a float32 scale per leading-axis row."""
    data: np.ndarray
    dtype: str
    scale: Optional[np.ndarray] = None

    @property
    def shape(self):
        return self.data.shape


def encode(x: np.ndarray, dtype: str) -> Tensor:
    if dtype == "fp32":
        return Tensor(np.ascontiguousarray(x, dtype=np.float32), "fp32")
    if dtype == "bf16":
        return Tensor(_bf16_threaded(x), "bf16")
    if dtype == "fp8":
        codes, scales = _fp8_threaded(x)
        return Tensor(codes, "fp8", scales)
    raise ValueError(dtype)


@dataclasses.dataclass
class Layer:
    conv_attn: Tensor   # [K, H]   param dtype
    attn_norm: Tensor   # [H]      param dtype
    wqkv: Tensor        # [(nq + 2 nkv) d, H]  rows: q heads, k heads, v heads
    wo: Tensor          # [H, nq d]
    conv_ffn: Tensor    # [K, H]
    ffn_norm: Tensor    # [H]
    w_gate_up: Tensor   # [2F, H]  rows 0..F-1 gate, F..2F-1 up
    w_down: Tensor      # [H, F]
    dconv_attn: Optional[Tensor] = None   # [(H / G) K, H] weight dtype (dynamic taps, G = conv_group_size)
    dconv_ffn: Optional[Tensor] = None


@dataclasses.dataclass
class Weights:
    embed: Tensor       # [V, H] param dtype
    lm_head: Tensor     # [V, H] weight dtype (+ scale for fp8)
    proj: Tensor        # [H, nT * Ht]
    proj_norm: Tensor   # [H]
    final_norm: Tensor  # [H]
    sel_tl: Tensor      # [V, r] fp32
    sel_tr: Tensor      # [V, r] fp32
    layers: List[Layer]


def _gain(w: Workload, tid, n) -> Tensor:
    if w.gain_jitter > 0:
        g = 1.0 + normal((n,), (w.index, tid), w.gain_jitter)
    else:
        g = np.ones(n, dtype=np.float32)
    return encode(g, w.param_dtype)


def make_weights(w: Workload) -> Weights:
    H, V, sd = w.hidden, w.vocab, w.weight_std
    pd, wd = w.param_dtype, w.weight_dtype
    layers = []
    for l in range(w.num_layers):
        t = lambda which: (w.index, _layer_tid(l, which))
        layers.append(Layer(
            conv_attn=encode(normal((w.conv_kernel_size, H), t(L_CONV_ATTN), sd), pd),
            attn_norm=_gain(w, _layer_tid(l, L_ATTN_NORM), H),
            wqkv=encode(normal((w.qkv_rows, H), t(L_WQKV), sd), wd),
            wo=encode(normal((H, w.num_q_heads * w.head_dim), t(L_WO), sd), wd),
            conv_ffn=encode(normal((w.conv_kernel_size, H), t(L_CONV_FFN), sd), pd),
            ffn_norm=_gain(w, _layer_tid(l, L_FFN_NORM), H),
            w_gate_up=encode(normal((2 * w.ffn, H), t(L_WGU), sd), wd),
            w_down=encode(normal((H, w.ffn), t(L_WDOWN), sd), wd),
        ))
        if w.conv_group_size > 0:
            gk = H // w.conv_group_size * w.conv_kernel_size
            layers[-1].dconv_attn = encode(normal((gk, H), t(L_DCONV_ATTN), sd), wd)
            layers[-1].dconv_ffn = encode(normal((gk, H), t(L_DCONV_FFN), sd), wd)
    tl, tr = make_selector_tables(w)
    return Weights(
        embed=encode(normal((V, H), (w.index, T_EMBED), sd), pd),
        lm_head=encode(normal((V, H), (w.index, T_LMHEAD), sd), wd),
        proj=encode(normal((H, w.num_taps * w.tap_width), (w.index, T_PROJ), sd), wd),
        proj_norm=_gain(w, T_PROJ_NORM, H),
        final_norm=_gain(w, T_FINAL_NORM, H),
        sel_tl=encode(tl, "fp32"),
        sel_tr=encode(tr, "fp32"),
        layers=layers,
    )


def make_selector_tables(w: Workload):
    """Left and right selector factor tables [V, r] float32."""
    tstd = w.selector_table_std()
    return (normal((w.vocab, w.rank), (w.index, T_SEL_L), tstd),
            normal((w.vocab, w.rank), (w.index, T_SEL_R), tstd))


def accepted_draws(w: Workload, n: int, seed_key) -> np.ndarray:
    """Number of leading drafts a verifier agreeing at position m with
    probability agreement(m) accepts, for n independent blocks."""
    rng = np.random.default_rng([SEED, *seed_key])
    u = rng.random((n, w.block_size - 1))
    p = np.array([w.agreement(m) for m in range(1, w.block_size)])
    ok = u < p[None, :]
    acc = np.zeros(n, dtype=np.int64)
    alive = np.ones(n, dtype=bool)
    for m in range(w.block_size - 1):
        alive &= ok[:, m]
        acc += alive
    return acc


@dataclasses.dataclass
class StepInputs:
    anchors: np.ndarray       # [B] int32
    ctx_lens: np.ndarray      # [B] int32 -- context length L_b after the append
    new_offsets: np.ndarray   # [B+1] int32 prefix sums of n_new
    taps: Tensor              # [sum n_new, nT, Ht] act dtype
    k_ctx: np.ndarray         # [nL, B, nkv, Lmax, d] act-dtype bits/values; rows < L_b - n_new_b valid
    v_ctx: np.ndarray         # same layout as k_ctx (logical [row, d] order)

    @property
    def n_new(self) -> np.ndarray:
        return np.diff(self.new_offsets)


def make_step_inputs(w: Workload, seqs: Optional[np.ndarray] = None) -> StepInputs:
    """Inputs of one draft step.  With `seqs`, only those sequences of the
    batch are materialised (same values as in the full batch)."""
    B = w.batch
    rng = np.random.default_rng([SEED, w.index, S_ANCHOR])
    anchors = rng.integers(0, w.vocab - 1, size=B).astype(np.int32)
    lo, hi = w.ctx
    if lo == hi:
        ctx = np.full(B, lo, dtype=np.int64)
    else:
        ctx = np.random.default_rng([SEED, w.index, S_CTXLEN]).integers(lo, hi + 1, size=B)
    if w.cold:
        n_new = ctx.copy()
    else:
        n_new = 1 + accepted_draws(w, B, (w.index, S_ACCEPT))
    if seqs is None:
        seqs = np.arange(B)
    seqs = np.asarray(seqs)
    nb = len(seqs)
    offsets = np.zeros(nb + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(n_new[seqs])
    # taps: one stream per sequence so a subset reproduces the full batch
    taps = np.empty((int(offsets[-1]), w.num_taps, w.tap_width), dtype=np.float32)
    for i, b in enumerate(seqs):
        taps[offsets[i]:offsets[i + 1]] = normal((int(n_new[b]), w.num_taps, w.tap_width),
                                                 (w.index, S_TAPS, int(b)))
    # pre-existing cache rows [0, L - n_new), per (layer, sequence)
    nL, nkv, d, Lmax = w.num_layers, w.num_kv_heads, w.head_dim, w.max_context
    cdt = np.float32 if w.act_dtype == "fp32" else np.uint16
    k_ctx = np.zeros((nL, nb, nkv, Lmax, d), dtype=cdt)
    v_ctx = np.zeros((nL, nb, nkv, Lmax, d), dtype=cdt)
    for l in range(nL):
        for i, b in enumerate(seqs):
            old = int(ctx[b] - n_new[b])
            if old <= 0:
                continue
            for arr, tid in ((k_ctx, S_KCACHE), (v_ctx, S_VCACHE)):
                x = normal((nkv, old, d), (w.index, tid, l, int(b)))
                arr[l, i, :, :old, :] = x if cdt == np.float32 else _bf16_threaded(x)
    return StepInputs(
        anchors=anchors[seqs].astype(np.int32),
        ctx_lens=ctx[seqs].astype(np.int32),
        new_offsets=offsets.astype(np.int32),
        taps=encode(taps, w.act_dtype),
        k_ctx=k_ctx, v_ctx=v_ctx,
    )


def make_verified_taps(w: Workload, starts: np.ndarray, counts: np.ndarray,
                       seqs: Optional[np.ndarray] = None):
    """Target hidden-state taps of newly verified positions, for a decode
    loop: sequence seqs[i] gets rows for positions starts[i] ..
    starts[i] + counts[i] - 1, each row N(0, 1) seeded by (sequence,
    position), so a position's taps do not depend on which step verified it.
    Returns (taps Tensor [sum(counts), num_taps, tap_width], offsets [B+1])."""
    starts = np.asarray(starts, dtype=np.int64)
    counts = np.asarray(counts, dtype=np.int64)
    seqs = np.arange(len(starts)) if seqs is None else np.asarray(seqs)
    offsets = np.zeros(len(starts) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    taps = np.empty((int(offsets[-1]), w.num_taps, w.tap_width), dtype=np.float32)
    for i, b in enumerate(seqs):
        for j in range(int(counts[i])):
            taps[offsets[i] + j] = normal((w.num_taps, w.tap_width),
                                          (w.index, S_VERIFIED_TAPS, int(b), int(starts[i]) + j))
    return encode(taps, w.act_dtype), offsets.astype(np.int32)


def make_target_logits(w: Workload, drafts: np.ndarray, seqs: Optional[np.ndarray] = None,
                       tag: int = 0) -> np.ndarray:
    """Verifier logits [B, bs, V] float32: N(0, 1) with a planted argmax.

    Row i (i < bs-1) is the target's prediction after block slot i; its argmax
    is drafts[b, i] with probability agreement(i + 1), otherwise uniform over
    the other V - 1 ids.  Row bs-1 has a uniform argmax.  The planted entry is
    set to the row maximum + 1.  `drafts` is [len(seqs), bs-1].
    """
    B, bs, V = w.batch, w.block_size, w.vocab
    if seqs is None:
        seqs = np.arange(B)
    seqs = np.asarray(seqs)
    drafts = np.asarray(drafts).reshape(len(seqs), bs - 1)
    out = np.empty((len(seqs), bs, V), dtype=np.float32)
    p = np.array([w.agreement(m) for m in range(1, bs)] + [0.0])

    def work(i):
        b = int(seqs[i])
        rows = normal((bs, V), (w.index, V_LOGITS, tag, b))
        rng = np.random.default_rng([SEED, w.index, V_PLANT, tag, b])
        u = rng.random(bs)
        other = rng.integers(0, V - 1, size=bs)
        for r in range(bs):
            if r < bs - 1:
                dr = int(drafts[i, r])
                tau = dr if u[r] < p[r] else (int(other[r]) + (1 if other[r] >= dr else 0))
            else:
                tau = int(rng.integers(0, V))
            rows[r, tau] = rows[r].max() + np.float32(1.0)
        out[i] = rows

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(len(seqs))))
    return out


def make_sampling_inputs(B: int, bs: int, V: int, tag: int = 0, spread: float = 2.0, boost: float = 16.0,
                         agree: float = 0.8, quantum: float = 0.0):
    """Inputs of sampled verification: drafts [B, bs-1] uniform over the
    vocabulary and target logits [B, bs, V] float32 N(0, spread^2), where the
    draft's logit in row i < bs-1 is raised with probability `agree` by
    boost * U(0.3, 1) (from an unlikely to an almost certain token of the
    target).  quantum > 0 rounds every logit to a multiple of it, so equal
    values are common."""
    drng = np.random.default_rng([SEED, V_SAMPLE_PLANT, tag, B, bs, V])
    drafts = drng.integers(0, V, size=(B, bs - 1)).astype(np.int32)
    raise_it = drng.random((B, bs - 1)) < agree
    amount = (boost * drng.uniform(0.3, 1.0, size=(B, bs - 1))).astype(np.float32)
    out = np.empty((B, bs, V), dtype=np.float32)

    def work(b):
        rows = normal((bs, V), (V_SAMPLE_LOGITS, tag, b, V), std=spread)
        for r in range(bs - 1):
            if raise_it[b, r]:
                rows[r, drafts[b, r]] += amount[b, r]
        if quantum > 0:
            rows = (np.round(rows / np.float32(quantum)) * np.float32(quantum)).astype(np.float32)
        out[b] = rows

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(B)))
    return drafts, out


def make_uniforms(shape, tag: int = 0) -> np.ndarray:
    """float32 uniforms k / 2^24, k uniform on 0 .. 2^24 - 1: exact in
    float32 and strictly below 1."""
    rng = np.random.default_rng([SEED, V_UNIFORM, tag, *[int(x) for x in shape]])
    return (rng.integers(0, 1 << 24, size=shape) / float(1 << 24)).astype(np.float32)


def make_selector_inputs(w: Workload, tag: int = 0, integer_lattice: bool = False) -> Dict[str, np.ndarray]:
    """Stand-alone selector inputs: anchors [B], candidate ids [B, bs-1, k]
    (distinct per position) and candidate values [B, bs-1, k] float32 sorted
    descending.  With integer_lattice=True the values are small integers and
    ties are common; pair tables for that case come from
    make_integer_tables."""
    B, P, k, V = w.batch, w.block_size - 1, w.top_k, w.vocab
    rng = np.random.default_rng([SEED, w.index, X_SEL_IDS, tag])
    ids = np.empty((B, P, k), dtype=np.int32)
    for b in range(B):
        for t in range(P):
            ids[b, t] = rng.choice(V, size=k, replace=False)
    vrng = np.random.default_rng([SEED, w.index, X_SEL_VALS, tag])
    if integer_lattice:
        vals = vrng.integers(0, 2, size=(B, P, k)).astype(np.float32)
    else:
        vals = (vrng.standard_normal((B, P, k)) * 1.5 + 8.0).astype(np.float32)
    vals = -np.sort(-vals, axis=-1)
    anchors = np.random.default_rng([SEED, w.index, X_SEL_ANCH, tag]).integers(0, V - 1, size=B).astype(np.int32)
    return {"anchors": anchors, "ids": ids, "vals": vals}


def make_integer_tables(w: Workload, tag: int = 0):
    """Sparse selector factor tables with entries in {0, 1} (float32): every
    pair score is a small integer, so equal-score paths are frequent."""
    rng = np.random.default_rng([SEED, w.index, T_SEL_L, 77, tag])
    tl = (rng.random((w.vocab, w.rank)) < 0.15).astype(np.float32)
    tr = (rng.random((w.vocab, w.rank)) < 0.15).astype(np.float32)
    return tl, tr
