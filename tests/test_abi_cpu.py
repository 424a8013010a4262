"""CPU checks of the C ABI: the library loads, exports every entry point
include/dflash2.h declares, and rejects bad arguments before any HIP call
(every case here runs without a GPU).  Also the acceptance-metrics record
against the hand-worked fixture."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import block_speculative_decoding_dflash2_amd as pkg
from block_speculative_decoding_dflash2_amd import _lib as L
from block_speculative_decoding_dflash2_amd.runner import config_struct
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash2.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash2_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(L.EXPORTED)
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def _fake_weights(nl=1, fp8=False):
    """Non-null placeholder addresses: create() only validates the table."""
    lw = (L.dflash2_layer_weights * nl)()
    for i in range(nl):
        for f, _ in L.dflash2_layer_weights._fields_:
            if f.endswith("_scale") and not fp8:
                continue
            setattr(lw[i], f, 0x1000)
    w = L.dflash2_weights()
    for f, _ in L.dflash2_weights._fields_:
        if f == "layers":
            continue
        if f.endswith("_scale") and not fp8:
            continue
        setattr(w, f, 0x1000)
    w.layers = ctypes.cast(lw, ctypes.POINTER(L.dflash2_layer_weights))
    return w, lw


def _status_create(cfg):
    w, keep = _fake_weights(cfg["num_layers"], cfg["weight_dtype"] == "fp8")
    h = ctypes.c_void_p()
    st = L.lib.dflash2_create(ctypes.byref(config_struct(cfg)), ctypes.byref(w), ctypes.byref(h))
    if st == 0:
        L.lib.dflash2_destroy(h)
    return st


BASE = synth.get("tiny_fp32").abi_config()


@pytest.mark.parametrize("change,status", [
    ({}, L.DFLASH2_OK),
    ({"block_size": 1}, L.DFLASH2_ERR_SHAPE),
    ({"num_q_heads": 6, "num_kv_heads": 4}, L.DFLASH2_ERR_SHAPE),
    ({"conv_kernel_size": 9}, L.DFLASH2_ERR_SHAPE),
    ({"conv_kernel_size": 0}, L.DFLASH2_ERR_SHAPE),
    ({"selector_top_k": 0}, L.DFLASH2_ERR_SHAPE),
    ({"selector_top_k": 65}, L.DFLASH2_ERR_SHAPE),
    ({"selector_rank": 0}, L.DFLASH2_ERR_SHAPE),
    ({"selector_rank": 257}, L.DFLASH2_ERR_SHAPE),
    ({"mask_token_id": 512}, L.DFLASH2_ERR_SHAPE),
    ({"weight_dtype": 7}, L.DFLASH2_ERR_INVALID_ARG),
    ({"hidden": 0}, L.DFLASH2_ERR_INVALID_ARG),
    ({"head_dim": 24}, L.DFLASH2_ERR_UNSUPPORTED),
    ({"hidden": 80}, L.DFLASH2_ERR_UNSUPPORTED),
    ({"max_context": 36}, L.DFLASH2_ERR_UNSUPPORTED),
    ({"max_context": 4}, L.DFLASH2_ERR_SHAPE),
    ({"selector_top_k": 64, "selector_rank": 256}, L.DFLASH2_OK),   # the largest selector fits LDS
    # the logit transform must be strictly increasing (top-k ranks the raw logits)
    ({"output_multiplier": 0.0}, L.DFLASH2_ERR_INVALID_ARG),
    ({"output_multiplier": -0.5}, L.DFLASH2_ERR_INVALID_ARG),
    ({"output_multiplier": float("nan")}, L.DFLASH2_ERR_INVALID_ARG),
    ({"output_multiplier": float("inf")}, L.DFLASH2_ERR_INVALID_ARG),
    ({"output_multiplier": 0.5, "final_logit_softcapping": 30.0, "input_embedding_scale": 2.5}, L.DFLASH2_OK),
    ({"input_embedding_scale": float("nan")}, L.DFLASH2_ERR_INVALID_ARG),
    ({"input_embedding_scale": float("-inf")}, L.DFLASH2_ERR_INVALID_ARG),
    ({"input_embedding_scale": -1.0}, L.DFLASH2_OK),
    ({"final_logit_softcapping": float("inf")}, L.DFLASH2_ERR_INVALID_ARG),
    ({"final_logit_softcapping": -1.0}, L.DFLASH2_ERR_INVALID_ARG),
    ({"rms_eps": float("nan")}, L.DFLASH2_ERR_INVALID_ARG),
    ({"rope_theta": float("inf")}, L.DFLASH2_ERR_INVALID_ARG),
    # contraction lengths: the GEMM tiles address at most 128 rows of 2^20
    # elements with 32-bit offsets from a 64-bit tile base
    ({"ffn": 1 << 20}, L.DFLASH2_OK),
    ({"ffn": (1 << 20) + 32}, L.DFLASH2_ERR_UNSUPPORTED),
    ({"num_taps": 33, "tap_width": 1 << 15}, L.DFLASH2_ERR_UNSUPPORTED),
    ({"num_taps": 32, "tap_width": 1 << 15}, L.DFLASH2_OK),
    ({"num_q_heads": 8193, "num_kv_heads": 1, "head_dim": 128}, L.DFLASH2_ERR_UNSUPPORTED),
    ({"num_taps": 1 << 16, "tap_width": 1 << 16}, L.DFLASH2_ERR_UNSUPPORTED),  # product overflows int32
])
def test_create_validation(change, status):
    cfg = dict(BASE, **change)
    assert _status_create(cfg) == status
    if status != L.DFLASH2_OK:
        assert L.dflash2_last_error() != ""


def test_create_rejects_null_weights_and_missing_fp8_scales():
    cfg = dict(BASE)
    w, keep = _fake_weights(1)
    w.embed = None
    h = ctypes.c_void_p()
    assert L.lib.dflash2_create(ctypes.byref(config_struct(cfg)), ctypes.byref(w), ctypes.byref(h)) \
        == L.DFLASH2_ERR_INVALID_ARG
    cfg8 = dict(BASE, weight_dtype="fp8")
    w8, keep8 = _fake_weights(1, fp8=False)
    assert L.lib.dflash2_create(ctypes.byref(config_struct(cfg8)), ctypes.byref(w8), ctypes.byref(h)) \
        == L.DFLASH2_ERR_INVALID_ARG
    assert "scale" in L.dflash2_last_error()


def _handle(cfg):
    w, keep = _fake_weights(cfg["num_layers"], cfg["weight_dtype"] == "fp8")
    h = L.dflash2_create(config_struct(cfg), w)
    return h, (w, keep)


def test_create_rejects_misaligned_weights():
    """Weight and scale pointers must be 16-byte aligned."""
    cfg = dict(BASE)
    for field in ("lm_head", "embed", "proj_norm"):
        w, lw = _fake_weights(cfg["num_layers"])
        setattr(w, field, 0x1008)
        h = ctypes.c_void_p()
        assert L.lib.dflash2_create(ctypes.byref(config_struct(cfg)), ctypes.byref(w), ctypes.byref(h)) \
            == L.DFLASH2_ERR_INVALID_ARG, field
        assert "16-byte aligned" in L.dflash2_last_error()
    w, lw = _fake_weights(cfg["num_layers"])
    lw[0].w_down = 0x1004
    h = ctypes.c_void_p()
    assert L.lib.dflash2_create(ctypes.byref(config_struct(cfg)), ctypes.byref(w), ctypes.byref(h)) \
        == L.DFLASH2_ERR_INVALID_ARG
    assert "16-byte aligned" in L.dflash2_last_error()
    cfg8 = dict(BASE, weight_dtype="fp8")
    w8, lw8 = _fake_weights(cfg8["num_layers"], fp8=True)
    assert L.lib.dflash2_create(ctypes.byref(config_struct(cfg8)), ctypes.byref(w8), ctypes.byref(h)) == 0
    L.lib.dflash2_destroy(h)
    w8.lm_head_scale = 0x1004
    assert L.lib.dflash2_create(ctypes.byref(config_struct(cfg8)), ctypes.byref(w8), ctypes.byref(h)) \
        == L.DFLASH2_ERR_INVALID_ARG
    assert "16-byte aligned" in L.dflash2_last_error()


def test_workspace_size_and_draft_argument_errors():
    h, keep = _handle(BASE)
    try:
        n1 = L.dflash2_workspace_size(h, 1, 32)
        n0 = L.dflash2_workspace_size(h, 1, 0)
        assert n1 > n0 > 0 and n1 % 256 == 0
        with pytest.raises(L.DFlash2Error) as e:
            L.dflash2_workspace_size(h, 2, 8)          # batch > max_batch
        assert e.value.status == L.DFLASH2_ERR_SHAPE
        p = 0x1000
        # null anchor pointer
        with pytest.raises(L.DFlash2Error) as e:
            L.dflash2_draft_block(h, None, 1, None, p, p, p, 8, p, p, p, p, None, None, p, n1)
        assert e.value.status == L.DFLASH2_ERR_INVALID_ARG
        # workspace too small / misaligned
        with pytest.raises(L.DFlash2Error) as e:
            L.dflash2_draft_block(h, None, 1, p, p, p, p, 32, p, p, p, p, None, None, p, n1 - 1)
        assert e.value.status == L.DFLASH2_ERR_WORKSPACE
        with pytest.raises(L.DFlash2Error) as e:
            L.dflash2_draft_block(h, None, 1, p, p, p, p, 32, p, p, p, p, None, None, p + 8, n1)
        assert e.value.status == L.DFLASH2_ERR_WORKSPACE
        with pytest.raises(L.DFlash2Error) as e:
            L.dflash2_draft_block(h, None, 0, p, p, p, p, 32, p, p, p, p, None, None, p, n1)
        assert e.value.status == L.DFLASH2_ERR_SHAPE
        # misaligned taps, cache or debug output
        for args in ((p, p + 2, p, p, 32, p, p), (p, p, p, p, 32, p + 8, p), (p, p, p, p, 32, p, p + 4)):
            with pytest.raises(L.DFlash2Error) as e:
                L.dflash2_draft_block(h, None, 1, *args, p, p, None, None, p, n1)
            assert e.value.status == L.DFLASH2_ERR_INVALID_ARG
            assert "16-byte aligned" in L.dflash2_last_error()
        with pytest.raises(L.DFlash2Error) as e:
            L.dflash2_draft_block(h, None, 1, p, p, p, p, 32, p, p, p, p, p + 4, None, p, n1)
        assert e.value.status == L.DFLASH2_ERR_INVALID_ARG
        with pytest.raises(L.DFlash2Error) as e:
            L.dflash2_select_path(h, None, 1, p, None, p, p, p, None, None)
        assert e.value.status == L.DFLASH2_ERR_INVALID_ARG
        with pytest.raises(L.DFlash2Error) as e:
            L.dflash2_select_path(h, None, 3, p, p, p, p, p, None, None)
        assert e.value.status == L.DFLASH2_ERR_SHAPE
        # the stop variant: lengths are required, p_min lies in [0, 1]
        with pytest.raises(L.DFlash2Error) as e:
            L.dflash2_select_path_stop(h, None, 1, p, p, p, 0.1, 0, 7, p, p, None, None, None)
        assert e.value.status == L.DFLASH2_ERR_INVALID_ARG
        for bad in (-0.1, 1.5, float("nan")):
            with pytest.raises(L.DFlash2Error) as e:
                L.dflash2_select_path_stop(h, None, 1, p, p, p, bad, 0, 7, p, p, p, None, None)
            assert e.value.status == L.DFLASH2_ERR_INVALID_ARG
        with pytest.raises(L.DFlash2Error) as e:
            L.dflash2_select_path_stop(h, None, 3, p, p, p, 0.1, 0, 7, p, p, p, None, None)
        assert e.value.status == L.DFLASH2_ERR_SHAPE
        # draft_select: the draft_block checks, plus path and draft outputs required
        for path, drafts in ((None, p), (p, None)):
            with pytest.raises(L.DFlash2Error) as e:
                L.dflash2_draft_select(h, None, 1, p, p, p, p, 32, p, p, p, p, path, drafts, None, None, p, n1)
            assert e.value.status == L.DFLASH2_ERR_INVALID_ARG
        with pytest.raises(L.DFlash2Error) as e:
            L.dflash2_draft_select(h, None, 1, p, p, p, p, 32, p, p, p, p, p, p, None, None, p, n1 - 1)
        assert e.value.status == L.DFLASH2_ERR_WORKSPACE
        with pytest.raises(L.DFlash2Error) as e:
            L.dflash2_draft_select(h, None, 2, p, p, p, p, 32, p, p, p, p, p, p, None, None, p, n1)
        assert e.value.status == L.DFLASH2_ERR_SHAPE
    finally:
        L.dflash2_destroy(h)


def test_verify_argument_errors():
    n = L.dflash2_verify_workspace_size(4, 8, 1000)
    assert n > 0 and n % 256 == 0
    p = 0x1000
    with pytest.raises(L.DFlash2Error) as e:
        L.dflash2_verify_accept(None, 4, 1, 1000, p, p, p, p, None, p, n)
    assert e.value.status == L.DFLASH2_ERR_SHAPE
    with pytest.raises(L.DFlash2Error) as e:
        L.dflash2_verify_accept(None, 4, 8, 1000, p, None, p, p, None, p, n)
    assert e.value.status == L.DFLASH2_ERR_INVALID_ARG
    with pytest.raises(L.DFlash2Error) as e:
        L.dflash2_verify_accept(None, 4, 8, 1000, p, p, p, p, None, p, n - 8)
    assert e.value.status == L.DFLASH2_ERR_WORKSPACE


@pytest.mark.parametrize("vocab,hidden,dtype", [(262144, 8192, "bf16"), (151936, 16384, "bf16"),
                                                (270000, 8192, "bf16"), (262144, 16384, "fp8")])
def test_create_accepts_lm_head_beyond_4gib(vocab, hidden, dtype):
    """lm_head weights of 4 GiB and more (V * H * bytes >= 2^32) are valid:
    the tiled GEMMs form 64-bit tile bases, so no offset wraps inside the
    weight (the GPU side is checked by test_lmhead_tiled_beyond_4gib)."""
    cfg = dict(BASE, vocab=vocab, hidden=hidden, mask_token_id=vocab - 1, weight_dtype=dtype)
    assert vocab * hidden * (1 if dtype == "fp8" else 2) >= 1 << 32
    assert _status_create(cfg) == L.DFLASH2_OK, L.dflash2_last_error()


def test_verify_noalloc_argument_errors():
    """The allocation-free verifier rejects bad sizes, null pointers and
    batches whose scratch exceeds its fixed 1 MiB (batch * block_size >
    131072) before any device work."""
    p = 0x1000
    with pytest.raises(L.DFlash2Error) as e:
        L.dflash2_verify_accept_noalloc(None, 4, 1, 1000, p, p, p, p, None)
    assert e.value.status == L.DFLASH2_ERR_SHAPE
    with pytest.raises(L.DFlash2Error) as e:
        L.dflash2_verify_accept_noalloc(None, 4, 8, 1000, p, p, None, p, None)
    assert e.value.status == L.DFLASH2_ERR_INVALID_ARG
    with pytest.raises(L.DFlash2Error) as e:
        L.dflash2_verify_accept_noalloc(None, 16385, 8, 1000, p, p, p, p, None)
    assert e.value.status == L.DFLASH2_ERR_WORKSPACE
    assert "131072" in L.dflash2_last_error()
    # the largest accepted batch needs exactly the built-in 1 MiB
    assert L.dflash2_verify_workspace_size(16384, 8, 151936) == 1 << 20


def test_full_workload_configs_validate():
    for name in synth.WORKLOADS:
        cfg = synth.get(name).abi_config()
        assert _status_create(cfg) == L.DFLASH2_OK, (name, L.dflash2_last_error())
    for name in synth.TEST_WORKLOADS:
        cfg = synth.get(name).abi_config()
        assert _status_create(cfg) == L.DFLASH2_OK, (name, L.dflash2_last_error())


def test_speculative_metrics_fixture():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "metrics_hand.json")))
    m = pkg.metrics.speculative_metrics(g["per_step_accepted"], g["num_spec_tokens"])
    for k, v in g["expected"].items():
        assert m[k] == pytest.approx(v) if isinstance(v, float) else m[k] == v, k


def test_verify_sample_argument_errors():
    n = L.dflash2_verify_sample_workspace_size(4, 8, 1000)
    assert n >= L.dflash2_verify_workspace_size(4, 8, 1000) and n % 256 == 0
    assert n >= 4 * 8 * 24
    p = 0x1000

    def call(**kw):
        a = dict(batch=4, bs=8, V=1000, drafts=p, lens=None, logits=p, uni=p, T=1.0, top_k=20, top_p=0.95,
                 acc=p, bonus=p, prob=None, ws=p, nbytes=n)
        a.update(kw)
        L.dflash2_verify_sample(None, a["batch"], a["bs"], a["V"], a["drafts"], a["lens"], a["logits"], a["uni"],
                                a["T"], a["top_k"], a["top_p"], a["acc"], a["bonus"], a["prob"], a["ws"],
                                a["nbytes"])

    cases = [(dict(bs=1), L.DFLASH2_ERR_SHAPE), (dict(batch=0), L.DFLASH2_ERR_SHAPE),
             (dict(logits=None), L.DFLASH2_ERR_INVALID_ARG), (dict(bonus=None), L.DFLASH2_ERR_INVALID_ARG),
             (dict(T=-1.0), L.DFLASH2_ERR_INVALID_ARG), (dict(T=float("nan")), L.DFLASH2_ERR_INVALID_ARG),
             (dict(T=float("inf")), L.DFLASH2_ERR_INVALID_ARG), (dict(top_k=-1), L.DFLASH2_ERR_INVALID_ARG),
             (dict(top_p=0.0), L.DFLASH2_ERR_INVALID_ARG), (dict(top_p=float("nan")), L.DFLASH2_ERR_INVALID_ARG),
             (dict(uni=None), L.DFLASH2_ERR_INVALID_ARG), (dict(nbytes=n - 8), L.DFLASH2_ERR_WORKSPACE),
             (dict(ws=p + 16), L.DFLASH2_ERR_WORKSPACE)]
    for kw, status in cases:
        with pytest.raises(L.DFlash2Error) as e:
            call(**kw)
        assert e.value.status == status, kw


def test_draft_losses_argument_errors():
    n = L.dflash2_draft_losses_workspace_size(4, 8, 1000)
    assert n > 0 and n % 256 == 0
    w = synth.get("small_bf16")
    cfg = w.abi_config()
    wts, keep = _fake_weights(cfg["num_layers"], False)
    h = L.dflash2_create(config_struct(cfg), wts)
    try:
        p = 0x1000
        nb = L.dflash2_draft_losses_workspace_size(1, cfg["block_size"], cfg["vocab"])

        def call(**kw):
            a = dict(batch=1, anchors=p, labels=p, logits=p, ids=p, vals=p, gamma=4.0, wsel=0.5, losses=p,
                     ws=p, nbytes=nb)
            a.update(kw)
            L.dflash2_draft_losses(h, None, a["batch"], a["anchors"], a["labels"], a["logits"], a["ids"],
                                   a["vals"], a["gamma"], a["wsel"], None, None, a["losses"], a["ws"],
                                   a["nbytes"])

        cases = [(dict(batch=0), L.DFLASH2_ERR_SHAPE), (dict(batch=cfg["max_batch"] + 1), L.DFLASH2_ERR_SHAPE),
                 (dict(labels=None), L.DFLASH2_ERR_INVALID_ARG), (dict(losses=None), L.DFLASH2_ERR_INVALID_ARG),
                 (dict(gamma=0.0), L.DFLASH2_ERR_INVALID_ARG), (dict(gamma=float("nan")), L.DFLASH2_ERR_INVALID_ARG),
                 (dict(wsel=float("inf")), L.DFLASH2_ERR_INVALID_ARG), (dict(nbytes=nb - 8), L.DFLASH2_ERR_WORKSPACE),
                 (dict(ws=p + 8), L.DFLASH2_ERR_WORKSPACE)]
        for kw, status in cases:
            with pytest.raises(L.DFlash2Error) as e:
                call(**kw)
            assert e.value.status == status, kw
    finally:
        L.dflash2_destroy(h)


def test_one_hip_runtime_per_process():
    """Loading the binding before anything else must not bring in a second
    HIP runtime beside PyTorch's: the library receives PyTorch's device
    pointers and streams."""
    import subprocess
    import sys
    code = ("from block_speculative_decoding_dflash2_amd import _lib\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "print(len({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"
