"""Shared helpers of the GPU parity tests: run one draft step of a workload
through the C ABI and the same step through the oracle, on the same seeded
inputs."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle as O
import synth

TOL = {"fp32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}


def log(msg: str):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def normwise(g, o) -> float:
    """max |g - o| / max |o| over the whole tensor."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    return float(np.max(np.abs(g - o)) / max(np.max(np.abs(o)), 1e-300))


def act_to_f64(t: torch.Tensor, dtype: str) -> np.ndarray:
    a = t.cpu().numpy()
    if dtype == "fp32":
        return a.astype(np.float64)
    return O.bf16_bits_to_f64(a.view(np.uint16))


class DraftRun:
    """GPU outputs of one draft step (draft_block + select_path) of workload w."""

    def __init__(self, w, W=None, inp=None, debug=True):
        from block_speculative_decoding_dflash2_amd import DFlash2, to_device
        self.w = w
        self.W = synth.make_weights(w) if W is None else W
        self.inp = synth.make_step_inputs(w) if inp is None else inp
        inp = self.inp
        log(f"{w.name}: uploading")
        self.model = DFlash2(w.abi_config(), self.W)
        m = self.model
        self.kc, self.vc = m.new_caches()
        m.load_context(self.kc, self.vc, inp.k_ctx, inp.v_ctx)
        dev = m.device
        self.anchors = torch.from_numpy(inp.anchors).to(dev)
        self.offsets = torch.from_numpy(inp.new_offsets).to(dev)
        self.ctx_lens = torch.from_numpy(inp.ctx_lens).to(dev)
        self.taps = to_device(inp.taps.data.reshape(inp.taps.data.shape[0], -1), dev)
        self.max_new = int(inp.new_offsets[-1])
        log(f"{w.name}: draft_block B={w.batch} new_rows={self.max_new}")
        out = m.draft_block(self.anchors, self.taps, self.offsets, self.ctx_lens, self.max_new,
                            self.kc, self.vc, debug_logits=debug, debug_hidden=debug)
        sel = m.select_path(self.anchors, out["topk_ids"], out["topk_vals"], debug_pair=debug)
        torch.cuda.synchronize()
        log(f"{w.name}: GPU step done")
        self.topk_ids = out["topk_ids"].cpu().numpy()
        self.topk_vals = out["topk_vals"].cpu().numpy()
        self.logits = out["debug_logits"].cpu().numpy() if debug else None
        self.hidden = out["debug_hidden"].cpu().numpy() if debug else None
        self.path = sel["path"].cpu().numpy()
        self.drafts = sel["drafts"].cpu().numpy()
        self.score = sel["score"].cpu().numpy()
        self.drafts_dev = sel["drafts"]

    def cache_rows(self, seqs, layer):
        """Appended rows of (layer, seq) as float64 [n_new, nkv, d] for K and V."""
        w, inp = self.w, self.inp
        out = []
        for b in seqs:
            L = int(inp.ctx_lens[b])
            n = int(inp.new_offsets[b + 1] - inp.new_offsets[b])
            k = act_to_f64(self.kc[layer, b, :, L - n:L, :], w.act_dtype).transpose(1, 0, 2)
            v = act_to_f64(self.vc[layer, b, :, :, L - n:L], w.act_dtype).transpose(2, 0, 1)
            out.append((k, v))
        return out

    def close(self):
        self.model.close()
        del self.kc, self.vc
        torch.cuda.empty_cache()


def oracle_for(w, W, seqs=None):
    """Oracle step on the sequences `seqs` (all when None)."""
    inp = synth.make_step_inputs(w, seqs)
    t0 = time.time()
    res = O.step(w, W, inp)
    log(f"{w.name}: oracle done in {time.time() - t0:.1f}s")
    return inp, res


def topk_consistent(ids, vals, logits, k):
    """The GPU's own top-k agrees with its own debug logits: values are the
    logits at the ids, sorted by (value desc, id asc), and no other logit
    outranks the k-th."""
    R = ids.shape[0]
    z = logits.reshape(R, -1).astype(np.float32) + np.float32(0.0)
    for r in range(R):
        ii = ids[r].astype(np.int64)
        vv = z[r, ii]
        if not np.array_equal(vv, vals[r] + np.float32(0.0)):
            return False
        keys = list(zip((-vv).tolist(), ii.tolist()))
        if keys != sorted(keys):
            return False
        kth_v, kth_i = float(vv[-1]), int(ii[-1])
        mask = np.ones(z.shape[1], dtype=bool)
        mask[ii] = False
        rest = z[r, mask]
        rest_ids = np.nonzero(mask)[0]
        if np.any(rest > kth_v) or np.any((rest == kth_v) & (rest_ids < kth_i)):
            return False
    return True
