"""Convenience layer over the C ABI: owns the device copies of the weights
(PyTorch is used for device memory and streams only), builds the handle, and
calls dflash2_draft_block / dflash2_select_path / dflash2_verify_accept with
raw device pointers on the current stream."""
from __future__ import annotations

import ctypes
from typing import Dict, Optional

import numpy as np
import torch

from . import _lib as L


def config_struct(cfg: Dict) -> L.dflash2_config:
    c = L.dflash2_config()
    for name in L._INT_FIELDS:
        v = cfg.get(name, 0) if name == "conv_group_size" else cfg[name]
        if name == "weight_dtype" and isinstance(v, str):
            v = L.DTYPE_CODE[v]
        setattr(c, name, int(v))
    for name in L._FLOAT_FIELDS:
        setattr(c, name, float(cfg[name]))
    return c


def to_device(arr: np.ndarray, device="cuda") -> torch.Tensor:
    """Host array -> device tensor with the same bytes (bf16 bits travel as int16)."""
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        arr = arr.view(np.int16)
    return torch.from_numpy(arr).to(device)


def ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def current_stream() -> int:
    return torch.cuda.current_stream().cuda_stream


class DFlash2:
    """One draft head on one device.  `weights` is any object with the
    attributes embed, lm_head, proj, proj_norm, final_norm, sel_tl, sel_tr
    and layers[i].{conv_attn, attn_norm, wqkv, wo, conv_ffn, ffn_norm,
    w_gate_up, w_down}, each holding `.data` (stored bytes as a numpy array)
    and `.scale` (float32 per-row scales for fp8, else None)."""

    def __init__(self, cfg: Dict, weights, device="cuda"):
        self.cfg = dict(cfg)
        self.device = torch.device(device)
        self._keep = []
        self.fp32 = self.cfg["weight_dtype"] in ("fp32", L.DFLASH2_FP32)

        def up(t):
            if t is None:
                return None
            d = to_device(t, self.device)
            self._keep.append(d)
            return d.data_ptr()

        nl = len(weights.layers)
        self._layers = (L.dflash2_layer_weights * nl)()
        for i, lw in enumerate(weights.layers):
            x = self._layers[i]
            for name in ("conv_attn", "attn_norm", "wqkv", "wo", "conv_ffn", "ffn_norm", "w_gate_up", "w_down",
                         "dconv_attn", "dconv_ffn"):
                t = getattr(lw, name, None)
                if t is None:
                    continue
                setattr(x, name, up(t.data))
                if name in ("wqkv", "wo", "w_gate_up", "w_down", "dconv_attn", "dconv_ffn"):
                    setattr(x, name + "_scale", up(t.scale))
        w = L.dflash2_weights()
        for name in ("embed", "proj_norm", "final_norm", "sel_tl", "sel_tr"):
            setattr(w, name, up(getattr(weights, name).data))
        w.lm_head = up(weights.lm_head.data)
        w.lm_head_scale = up(weights.lm_head.scale)
        w.proj = up(weights.proj.data)
        w.proj_scale = up(weights.proj.scale)
        w.layers = ctypes.cast(self._layers, ctypes.POINTER(L.dflash2_layer_weights))
        self._w = w
        self._c = config_struct(self.cfg)
        self.handle = L.dflash2_create(self._c, self._w)

    def close(self):
        if getattr(self, "handle", None):
            L.dflash2_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- buffers -----------------------------------------------------------
    @property
    def act_torch_dtype(self):
        return torch.float32 if self.fp32 else torch.int16

    def new_caches(self, fill=None):
        c = self.cfg
        shape_k = (c["num_layers"], c["max_batch"], c["num_kv_heads"], c["max_context"], c["head_dim"])
        shape_v = (c["num_layers"], c["max_batch"], c["num_kv_heads"], c["head_dim"], c["max_context"])
        k = torch.zeros(shape_k, dtype=self.act_torch_dtype, device=self.device)
        v = torch.zeros(shape_v, dtype=self.act_torch_dtype, device=self.device)
        return k, v

    def load_context(self, k_cache, v_cache, k_rows: np.ndarray, v_rows: np.ndarray, seqs=None):
        """Copy host context rows (logical layout [nL, B, nkv, Lmax, d]) into
        the device caches (V stored transposed)."""
        nb = k_rows.shape[1]
        seqs = range(nb) if seqs is None else seqs
        kd = to_device(k_rows, self.device)
        vd = to_device(v_rows, self.device).transpose(-1, -2)
        for i, b in enumerate(seqs):
            k_cache[:, b].copy_(kd[:, i])
            v_cache[:, b].copy_(vd[:, i])

    def workspace(self, batch: int, max_new_rows: int) -> torch.Tensor:
        n = L.dflash2_workspace_size(self.handle, batch, max_new_rows)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=self.device)
        assert ws.data_ptr() % 256 == 0
        return ws

    # ---- the three calls -----------------------------------------------------
    def draft_block(self, anchors, taps, offsets, ctx_lens, max_new_rows, k_cache, v_cache,
                    workspace=None, topk_ids=None, topk_vals=None, debug_logits=False,
                    debug_hidden=False, stream=None):
        c = self.cfg
        B = anchors.numel()
        P, k = c["block_size"] - 1, c["selector_top_k"]
        dev = self.device
        if topk_ids is None:
            topk_ids = torch.empty((B, P, k), dtype=torch.int32, device=dev)
        if topk_vals is None:
            topk_vals = torch.empty((B, P, k), dtype=torch.float32, device=dev)
        if isinstance(debug_logits, torch.Tensor):
            dl = debug_logits
        else:
            dl = torch.empty((B, P, c["vocab"]), dtype=torch.float32, device=dev) if debug_logits else None
        dh = torch.empty((B, P + 1, c["hidden"]), dtype=torch.float32, device=dev) if debug_hidden else None
        if workspace is None:
            workspace = self.workspace(B, max_new_rows)
        L.dflash2_draft_block(self.handle, current_stream() if stream is None else stream, B,
                              ptr(anchors), ptr(taps), ptr(offsets), ptr(ctx_lens), int(max_new_rows),
                              ptr(k_cache), ptr(v_cache), ptr(topk_ids), ptr(topk_vals), ptr(dl),
                              ptr(dh), ptr(workspace), workspace.numel())
        return {"topk_ids": topk_ids, "topk_vals": topk_vals, "debug_logits": dl, "debug_hidden": dh}

    def draft_select(self, anchors, taps, offsets, ctx_lens, max_new_rows, k_cache, v_cache,
                     workspace=None, topk_ids=None, topk_vals=None, path_idx=None, draft_tokens=None,
                     want_score=True, debug_logits=False, stream=None):
        """draft_block followed by select_path in one call (the candidate
        merge runs inside the selector's kernel)."""
        c = self.cfg
        B = anchors.numel()
        P, k = c["block_size"] - 1, c["selector_top_k"]
        dev = self.device
        if topk_ids is None:
            topk_ids = torch.empty((B, P, k), dtype=torch.int32, device=dev)
        if topk_vals is None:
            topk_vals = torch.empty((B, P, k), dtype=torch.float32, device=dev)
        if path_idx is None:
            path_idx = torch.empty((B, P), dtype=torch.int32, device=dev)
        if draft_tokens is None:
            draft_tokens = torch.empty((B, P), dtype=torch.int32, device=dev)
        score = torch.empty((B,), dtype=torch.float32, device=dev) if want_score else None
        if isinstance(debug_logits, torch.Tensor):
            dl = debug_logits
        else:
            dl = torch.empty((B, P, c["vocab"]), dtype=torch.float32, device=dev) if debug_logits else None
        if workspace is None:
            workspace = self.workspace(B, max_new_rows)
        L.dflash2_draft_select(self.handle, current_stream() if stream is None else stream, B,
                               ptr(anchors), ptr(taps), ptr(offsets), ptr(ctx_lens), int(max_new_rows),
                               ptr(k_cache), ptr(v_cache), ptr(topk_ids), ptr(topk_vals), ptr(path_idx),
                               ptr(draft_tokens), ptr(score), ptr(dl), ptr(workspace), workspace.numel())
        return {"topk_ids": topk_ids, "topk_vals": topk_vals, "path": path_idx, "drafts": draft_tokens,
                "score": score, "debug_logits": dl}

    def select_path(self, anchors, topk_ids, topk_vals, debug_pair=False, want_score=True,
                    path_idx=None, draft_tokens=None, stream=None):
        c = self.cfg
        B = anchors.numel()
        P, k = c["block_size"] - 1, c["selector_top_k"]
        dev = self.device
        if path_idx is None:
            path_idx = torch.empty((B, P), dtype=torch.int32, device=dev)
        if draft_tokens is None:
            draft_tokens = torch.empty((B, P), dtype=torch.int32, device=dev)
        score = torch.empty((B,), dtype=torch.float32, device=dev) if want_score else None
        pair = torch.empty((B, P, k, k), dtype=torch.float32, device=dev) if debug_pair else None
        L.dflash2_select_path(self.handle, current_stream() if stream is None else stream, B,
                              ptr(anchors), ptr(topk_ids), ptr(topk_vals), ptr(path_idx),
                              ptr(draft_tokens), ptr(score), ptr(pair))
        return {"path": path_idx, "drafts": draft_tokens, "score": score, "pair": pair}

    def draft_losses(self, anchors, labels, logits, topk_ids, topk_vals, gamma, selector_loss_weight,
                     want_per_slot=False, workspace=None, losses=None, stream=None):
        """Forward training losses (dflash2_draft_losses).  Returns losses [4]
        (total, block, selector, candidate_recall) and, if asked, the
        per-slot block and selector cross-entropies."""
        c = self.cfg
        B = anchors.numel()
        P = c["block_size"] - 1
        dev = self.device
        if workspace is None:
            n = L.dflash2_draft_losses_workspace_size(B, c["block_size"], c["vocab"])
            workspace = torch.empty(n, dtype=torch.uint8, device=dev)
        if losses is None:
            losses = torch.empty((4,), dtype=torch.float32, device=dev)
        bce = torch.empty((B, P), dtype=torch.float32, device=dev) if want_per_slot else None
        sce = torch.empty((B, P), dtype=torch.float32, device=dev) if want_per_slot else None
        L.dflash2_draft_losses(self.handle, current_stream() if stream is None else stream, B, ptr(anchors),
                               ptr(labels), ptr(logits), ptr(topk_ids), ptr(topk_vals), gamma,
                               selector_loss_weight, ptr(bce), ptr(sce), ptr(losses), ptr(workspace),
                               workspace.numel())
        return {"losses": losses, "block_ce": bce, "selector_ce": sce}

    def select_path_stop(self, anchors, topk_ids, topk_vals, p_min=0.0, n_min=0, n_max=None,
                         want_conf=False, want_score=False, path_idx=None, draft_tokens=None,
                         draft_lens=None, stream=None):
        """select_path plus the draft-length rule (draft_p_min / n_min / n_max)."""
        c = self.cfg
        B = anchors.numel()
        P = c["block_size"] - 1
        dev = self.device
        if path_idx is None:
            path_idx = torch.empty((B, P), dtype=torch.int32, device=dev)
        if draft_tokens is None:
            draft_tokens = torch.empty((B, P), dtype=torch.int32, device=dev)
        if draft_lens is None:
            draft_lens = torch.empty((B,), dtype=torch.int32, device=dev)
        conf = torch.empty((B, P), dtype=torch.float32, device=dev) if want_conf else None
        score = torch.empty((B,), dtype=torch.float32, device=dev) if want_score else None
        L.dflash2_select_path_stop(self.handle, current_stream() if stream is None else stream, B,
                                   ptr(anchors), ptr(topk_ids), ptr(topk_vals), p_min, n_min,
                                   P if n_max is None else n_max, ptr(path_idx), ptr(draft_tokens),
                                   ptr(draft_lens), ptr(conf), ptr(score))
        return {"path": path_idx, "drafts": draft_tokens, "lens": draft_lens, "conf": conf, "score": score}


class KernelTrace:
    """Per-kernel HIP-event timing of every library launch made on this
    thread while the context is active (dflash2_trace_attach)."""

    def __init__(self, capacity: int):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                  ctypes.c_void_p]
        self.capacity = capacity
        self.entries = (L.dflash2_trace_entry * capacity)()
        for e in self.entries:
            for f in ("start", "stop"):
                h = ctypes.c_void_p()
                if self._hip.hipEventCreate(ctypes.byref(h)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                setattr(e, f, h.value)
        self.count = 0

    def __enter__(self):
        L.dflash2_trace_attach(self.entries, self.capacity)
        return self

    def __exit__(self, *exc):
        self.count = L.dflash2_trace_detach()
        return False

    def records(self):
        """[(kind name, bytes, flops, milliseconds)] -- call after synchronising."""
        out = []
        ms = ctypes.c_float()
        for e in self.entries[:self.count]:
            if self._hip.hipEventElapsedTime(ctypes.byref(ms), e.start, e.stop) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append((L.KERNEL_KINDS[e.kind], int(e.bytes), int(e.flops), float(ms.value)))
        return out

    def close(self):
        for e in self.entries:
            for f in ("start", "stop"):
                h = getattr(e, f)
                if h:
                    self._hip.hipEventDestroy(h)
                    setattr(e, f, None)


def verify_workspace(batch: int, block_size: int, vocab: int, device="cuda") -> torch.Tensor:
    n = L.dflash2_verify_workspace_size(batch, block_size, vocab)
    return torch.empty(n, dtype=torch.uint8, device=device)


def verify_accept(draft_tokens, target_logits, want_argmax=False, workspace=None, accepted=None,
                  bonus=None, stream=None):
    B, bs, V = target_logits.shape
    dev = target_logits.device
    if accepted is None:
        accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if bonus is None:
        bonus = torch.empty((B,), dtype=torch.int32, device=dev)
    am = torch.empty((B, bs), dtype=torch.int32, device=dev) if want_argmax else None
    if workspace is None:
        workspace = verify_workspace(B, bs, V, dev)
    L.dflash2_verify_accept(current_stream() if stream is None else stream, B, bs, V,
                            ptr(draft_tokens), ptr(target_logits), ptr(accepted), ptr(bonus), ptr(am),
                            ptr(workspace), workspace.numel())
    return {"accepted": accepted, "bonus": bonus, "argmax": am}


def verify_sample_workspace(batch: int, block_size: int, vocab: int, device="cuda") -> torch.Tensor:
    n = L.dflash2_verify_sample_workspace_size(batch, block_size, vocab)
    return torch.empty(n, dtype=torch.uint8, device=device)


def verify_sample(draft_tokens, target_logits, uniforms, temperature, top_k=0, top_p=1.0, draft_lens=None,
                  want_prob=False, workspace=None, accepted=None, bonus=None, stream=None):
    """Rejection-sampling verification (dflash2_verify_sample).  uniforms
    [B, bs] float32 on the device: u_i in columns 0..bs-2, the draw's v last."""
    B, bs, V = target_logits.shape
    dev = target_logits.device
    if accepted is None:
        accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    if bonus is None:
        bonus = torch.empty((B,), dtype=torch.int32, device=dev)
    prob = torch.empty((B, bs - 1), dtype=torch.float32, device=dev) if want_prob else None
    if workspace is None:
        workspace = verify_sample_workspace(B, bs, V, dev)
    L.dflash2_verify_sample(current_stream() if stream is None else stream, B, bs, V, ptr(draft_tokens),
                            ptr(draft_lens), ptr(target_logits), ptr(uniforms), temperature, top_k, top_p,
                            ptr(accepted), ptr(bonus), ptr(prob), ptr(workspace), workspace.numel())
    return {"accepted": accepted, "bonus": bonus, "draft_prob": prob}
