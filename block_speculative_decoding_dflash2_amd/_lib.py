"""ctypes binding of libdflash2.so (include/dflash2.h): same names, argument
marshalling only.  Every step of the computation runs in the library's HIP
kernels; there is no Python or CPU fallback, and importing this module fails
loudly when the built library is missing."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_void_p

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("DFLASH2_LIB", os.path.join(_PKG, "libdflash2.so"))

DFLASH2_OK, DFLASH2_ERR_INVALID_ARG, DFLASH2_ERR_SHAPE, DFLASH2_ERR_UNSUPPORTED, \
    DFLASH2_ERR_WORKSPACE, DFLASH2_ERR_HIP = range(6)
DFLASH2_FP32, DFLASH2_BF16, DFLASH2_FP8_E4M3 = range(3)
DTYPE_CODE = {"fp32": DFLASH2_FP32, "bf16": DFLASH2_BF16, "fp8": DFLASH2_FP8_E4M3}

_INT_FIELDS = ("hidden", "num_layers", "num_q_heads", "num_kv_heads", "head_dim", "ffn", "vocab",
               "num_taps", "tap_width", "block_size", "conv_kernel_size", "selector_top_k",
               "selector_rank", "max_batch", "max_context", "sliding_window", "mask_token_id",
               "weight_dtype", "conv_group_size")
_FLOAT_FIELDS = ("rms_eps", "rope_theta", "input_embedding_scale", "output_multiplier",
                 "final_logit_softcapping")


class dflash2_config(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in _INT_FIELDS] + [(n, c_float) for n in _FLOAT_FIELDS]


class dflash2_layer_weights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in (
        "conv_attn", "attn_norm", "wqkv", "wqkv_scale", "wo", "wo_scale", "conv_ffn", "ffn_norm",
        "w_gate_up", "w_gate_up_scale", "w_down", "w_down_scale", "dconv_attn", "dconv_attn_scale",
        "dconv_ffn", "dconv_ffn_scale")]


class dflash2_weights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in (
        "embed", "lm_head", "lm_head_scale", "proj", "proj_scale", "proj_norm", "final_norm",
        "sel_tl", "sel_tr")] + [("layers", POINTER(dflash2_layer_weights))]


KERNEL_KINDS = ("gemm", "lmhead_topk", "topk_merge", "norm", "qkv_epilogue", "kv_append", "swiglu",
                "attention", "attn_combine", "select", "verify_partial", "verify_final", "sample_rows",
                "sample_pick", "loss_rows", "loss_seq", "merge_select")


class dflash2_trace_entry(ctypes.Structure):
    _fields_ = [("start", c_void_p), ("stop", c_void_p), ("kind", c_int32), ("reserved", c_int32),
                ("bytes", c_int64), ("flops", c_int64)]


class DFlash2Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"dflash2 status {status}: {message}")
        self.status = status


def _load():
    # One HIP runtime per process: the library takes device pointers and
    # streams from PyTorch, so its libamdhip64 dependency must resolve to the
    # runtime PyTorch loads.  Importing torch first makes the loader reuse it;
    # loading the library first would bring in a second, separate runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m block_speculative_decoding_dflash2_amd.build` (there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32p, f32p = c_void_p, c_void_p, c_void_p
    sig = {
        "dflash2_create": ([POINTER(dflash2_config), POINTER(dflash2_weights), POINTER(c_void_p)], c_int32),
        "dflash2_destroy": ([vp], None),
        "dflash2_workspace_size": ([vp, c_int32, c_int64, POINTER(c_size_t)], c_int32),
        "dflash2_draft_block": ([vp, vp, c_int32, i32p, vp, i32p, i32p, c_int64, vp, vp, i32p, f32p,
                                 f32p, f32p, vp, c_size_t], c_int32),
        "dflash2_draft_select": ([vp, vp, c_int32, i32p, vp, i32p, i32p, c_int64, vp, vp, i32p, f32p, i32p,
                                  i32p, f32p, f32p, vp, c_size_t], c_int32),
        "dflash2_select_path": ([vp, vp, c_int32, i32p, i32p, f32p, i32p, i32p, f32p, f32p], c_int32),
        "dflash2_select_path_stop": ([vp, vp, c_int32, i32p, i32p, f32p, c_float, c_int32, c_int32, i32p, i32p,
                                      i32p, f32p, f32p], c_int32),
        "dflash2_verify_workspace_size": ([c_int32, c_int32, c_int32, POINTER(c_size_t)], c_int32),
        "dflash2_verify_sample_workspace_size": ([c_int32, c_int32, c_int32, POINTER(c_size_t)], c_int32),
        "dflash2_verify_sample": ([vp, c_int32, c_int32, c_int32, i32p, i32p, f32p, f32p, c_float, c_int32,
                                   c_float, i32p, i32p, f32p, vp, c_size_t], c_int32),
        "dflash2_verify_accept": ([vp, c_int32, c_int32, c_int32, i32p, f32p, i32p, i32p, i32p, vp,
                                   c_size_t], c_int32),
        "dflash2_verify_accept_noalloc": ([vp, c_int32, c_int32, c_int32, i32p, f32p, i32p, i32p, i32p],
                                          c_int32),
        "dflash2_draft_losses_workspace_size": ([c_int32, c_int32, c_int32, POINTER(c_size_t)], c_int32),
        "dflash2_draft_losses": ([vp, vp, c_int32, i32p, i32p, f32p, i32p, f32p, c_float, c_float, f32p, f32p,
                                  f32p, vp, c_size_t], c_int32),
        "dflash2_peak_mfma": ([vp, c_int32, c_int32, c_int32, f32p], c_int32),
        "dflash2_peak_read": ([vp, vp, c_size_t, c_int32, vp], c_int32),
        "dflash2_trace_attach": ([POINTER(dflash2_trace_entry), c_int32], c_int32),
        "dflash2_trace_detach": ([], c_int32),
        "dflash2_last_error": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()
EXPORTED = ("dflash2_create", "dflash2_destroy", "dflash2_workspace_size", "dflash2_draft_block",
            "dflash2_draft_select",
            "dflash2_select_path", "dflash2_select_path_stop", "dflash2_verify_workspace_size",
            "dflash2_verify_accept", "dflash2_verify_accept_noalloc", "dflash2_verify_sample_workspace_size",
            "dflash2_verify_sample",
            "dflash2_draft_losses_workspace_size", "dflash2_draft_losses",
            "dflash2_trace_attach", "dflash2_trace_detach", "dflash2_last_error", "dflash2_peak_mfma",
            "dflash2_peak_read")


def dflash2_peak_mfma(stream, blocks, iters, zero_operands, out) -> None:
    _check(lib.dflash2_peak_mfma(stream, blocks, iters, zero_operands, out))


def dflash2_peak_read(stream, src, nbytes, blocks, out) -> None:
    _check(lib.dflash2_peak_read(stream, src, nbytes, blocks, out))


def dflash2_trace_attach(entries, capacity: int) -> None:
    _check(lib.dflash2_trace_attach(entries, capacity))


def dflash2_trace_detach() -> int:
    return lib.dflash2_trace_detach()


def _check(status: int):
    if status != DFLASH2_OK:
        raise DFlash2Error(status, lib.dflash2_last_error().decode())


def dflash2_last_error() -> str:
    return lib.dflash2_last_error().decode()


def dflash2_create(config: dflash2_config, weights: dflash2_weights) -> int:
    h = c_void_p()
    _check(lib.dflash2_create(ctypes.byref(config), ctypes.byref(weights), ctypes.byref(h)))
    return h.value


def dflash2_destroy(handle: int) -> None:
    lib.dflash2_destroy(handle)


def dflash2_workspace_size(handle: int, batch: int, max_new_rows: int) -> int:
    n = c_size_t()
    _check(lib.dflash2_workspace_size(handle, batch, max_new_rows, ctypes.byref(n)))
    return n.value


def dflash2_draft_block(handle, stream, batch, anchor_ids, new_taps, new_offsets, ctx_lens,
                        max_new_rows, k_cache, v_cache, topk_ids, topk_vals, debug_logits,
                        debug_hidden, workspace, workspace_bytes) -> None:
    _check(lib.dflash2_draft_block(handle, stream, batch, anchor_ids, new_taps, new_offsets, ctx_lens,
                                   max_new_rows, k_cache, v_cache, topk_ids, topk_vals, debug_logits,
                                   debug_hidden, workspace, workspace_bytes))


def dflash2_draft_select(handle, stream, batch, anchor_ids, new_taps, new_offsets, ctx_lens,
                         max_new_rows, k_cache, v_cache, topk_ids, topk_vals, path_idx, draft_tokens,
                         path_score, debug_logits, workspace, workspace_bytes) -> None:
    _check(lib.dflash2_draft_select(handle, stream, batch, anchor_ids, new_taps, new_offsets, ctx_lens,
                                    max_new_rows, k_cache, v_cache, topk_ids, topk_vals, path_idx, draft_tokens,
                                    path_score, debug_logits, workspace, workspace_bytes))


def dflash2_select_path(handle, stream, batch, anchor_ids, topk_ids, topk_vals, path_idx,
                        draft_tokens, path_score, debug_pair) -> None:
    _check(lib.dflash2_select_path(handle, stream, batch, anchor_ids, topk_ids, topk_vals, path_idx,
                                   draft_tokens, path_score, debug_pair))


def dflash2_verify_workspace_size(batch: int, block_size: int, vocab: int) -> int:
    n = c_size_t()
    _check(lib.dflash2_verify_workspace_size(batch, block_size, vocab, ctypes.byref(n)))
    return n.value


def dflash2_verify_accept(stream, batch, block_size, vocab, draft_tokens, target_logits, accepted,
                          bonus, target_argmax, workspace, workspace_bytes) -> None:
    _check(lib.dflash2_verify_accept(stream, batch, block_size, vocab, draft_tokens, target_logits,
                                     accepted, bonus, target_argmax, workspace, workspace_bytes))


def dflash2_verify_accept_noalloc(stream, batch, block_size, vocab, draft_tokens, target_logits, accepted,
                                  bonus, target_argmax) -> None:
    _check(lib.dflash2_verify_accept_noalloc(stream, batch, block_size, vocab, draft_tokens, target_logits,
                                             accepted, bonus, target_argmax))


def dflash2_select_path_stop(handle, stream, batch, anchor_ids, topk_ids, topk_vals, p_min, n_min, n_max,
                             path_idx, draft_tokens, draft_lens, path_conf, path_score) -> None:
    _check(lib.dflash2_select_path_stop(handle, stream, batch, anchor_ids, topk_ids, topk_vals, float(p_min),
                                        int(n_min), int(n_max), path_idx, draft_tokens, draft_lens, path_conf,
                                        path_score))


def dflash2_verify_sample_workspace_size(batch: int, block_size: int, vocab: int) -> int:
    n = c_size_t()
    _check(lib.dflash2_verify_sample_workspace_size(batch, block_size, vocab, ctypes.byref(n)))
    return n.value


def dflash2_verify_sample(stream, batch, block_size, vocab, draft_tokens, draft_lens, target_logits, uniforms,
                          temperature, top_k, top_p, accepted, bonus, draft_prob, workspace,
                          workspace_bytes) -> None:
    _check(lib.dflash2_verify_sample(stream, batch, block_size, vocab, draft_tokens, draft_lens, target_logits,
                                     uniforms, float(temperature), int(top_k), float(top_p), accepted, bonus,
                                     draft_prob, workspace, workspace_bytes))


def dflash2_draft_losses_workspace_size(batch: int, block_size: int, vocab: int) -> int:
    n = c_size_t()
    _check(lib.dflash2_draft_losses_workspace_size(batch, block_size, vocab, ctypes.byref(n)))
    return n.value


def dflash2_draft_losses(handle, stream, batch, anchor_ids, labels, logits, topk_ids, topk_vals, gamma,
                         selector_loss_weight, block_ce, selector_ce, losses, workspace, workspace_bytes) -> None:
    _check(lib.dflash2_draft_losses(handle, stream, batch, anchor_ids, labels, logits, topk_ids, topk_vals,
                                    float(gamma), float(selector_loss_weight), block_ce, selector_ce, losses,
                                    workspace, workspace_bytes))
