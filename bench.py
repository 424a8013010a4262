"""Throughput of the DFlash2 draft -> select -> verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--extra NAMES]

One step = dflash2_draft_select (context append, block forward, lm_head +
top-k, and the path selector, whose kernel also merges the candidates;
the same results as dflash2_draft_block + dflash2_select_path) +
dflash2_verify_accept over one batch of seeded synthetic inputs already
resident in HBM.  Consecutive steps rotate
over three sets of input and cache buffers (taps, K/V caches, verifier
logits), so the 256 MB Infinity Cache cannot serve one step's inputs from
the previous step.  Default workload: the 27B-class single-sequence draft
(batch 1, block 8, hidden 5120, 5 layers, vocab 151936, bf16); the fp8
high-batch draft+verify workload (batch 256, block 8, W8A16) is measured in
the same run and reported under "extra_workloads".  Prints one JSON line:
drafted blocks/s (value) and draft tokens/s, the roofline of the dominant
kernel measured with HIP events over a traced repeat of the timed steps,
and the CPU oracle's throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 2500.0, "fp32": 157.3}  # fp8 weights run as bf16 MFMA (W8A16)
ROTATE = 3


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


# Sources that define each traced kernel kind (its kernel code, device
# helpers and argument structs).
KERNEL_SOURCES = {
    "gemm": ["gemm.hip", "gemm_tiled.hip", "dma_tile.h", "common.h", "kernels.h"],
    "lmhead_topk": ["gemm.hip", "lmhead_tiled.hip", "dma_tile.h", "common.h", "kernels.h"],
    "attention": ["attention.hip", "common.h", "kernels.h"],
}


def kernel_source_hash(kernel: str = "gemm") -> str:
    """sha256 over the sources of one kernel kind; a traffic measurement is
    only used while that kernel is unchanged since it was taken."""
    import hashlib
    csrc = os.path.join(ROOT, "block_speculative_decoding_dflash2_amd", "csrc")
    names = KERNEL_SOURCES.get(kernel) or sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".h")))
    h = hashlib.sha256()
    for f in sorted(names):
        h.update(f.encode())
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (rocprofv3 FETCH_SIZE + WRITE_SIZE, each scaled by the counter's reading
    for a 1 GiB copy), or None if absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != kernel_source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def attention_kv_bytes(w, ctx_lens) -> int:
    """Algorithmic K/V bytes of one attention launch (one layer): every
    sequence reads its own context rows (the sliding window's, if set) plus
    the block's rows, once, for K and for V."""
    ab = 4 if w.act_dtype == "fp32" else 2
    rows = 0
    for L in np.asarray(ctx_lens, dtype=np.int64):
        lo = max(0, int(L) - w.sliding_window) if w.sliding_window > 0 else 0
        rows += int(L) - lo + w.block_size
    return rows * w.num_kv_heads * w.head_dim * 2 * ab


def measure_peaks():
    """The rates this chip sustains (library kernels dflash2_peak_mfma and
    dflash2_peak_read): bf16 MFMA on register-resident random and all-zero
    operands, and a non-temporal streaming read of 2 GiB (the best of
    several grid sizes)."""
    import torch
    from block_speculative_decoding_dflash2_amd import _lib as L
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    blocks, iters = 1024, 4000
    buf = torch.empty(blocks * 4, dtype=torch.float32, device=dev)
    for zero, key in ((0, "mfma_bf16_random_tflops"), (1, "mfma_bf16_zero_tflops")):
        L.dflash2_peak_mfma(stream, blocks, 50, zero, buf.data_ptr())
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best = 0.0
        for _ in range(3):
            e0.record()
            L.dflash2_peak_mfma(stream, blocks, iters, zero, buf.data_ptr())
            e1.record()
            torch.cuda.synchronize()
            flops = blocks * 4 * iters * 16 * 32768
            best = max(best, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        out[key] = round(best, 1)
    nbytes = 2 << 30
    src = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(1)
    # the best over grid sizes (two to sixteen blocks of 256 threads per CU)
    rout = torch.empty(4096 * 256, dtype=torch.int32, device=dev)
    best = 0.0
    for rblocks in (512, 1024, 2048, 4096):
        L.dflash2_peak_read(stream, src.data_ptr(), nbytes, rblocks, rout.data_ptr())
        torch.cuda.synchronize()
        for _ in range(3):
            e0.record()
            L.dflash2_peak_read(stream, src.data_ptr(), nbytes, rblocks, rout.data_ptr())
            e1.record()
            torch.cuda.synchronize()
            best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    out["hbm_read_gbs"] = round(best, 1)
    del src, rout, buf
    torch.cuda.empty_cache()
    log(f"measured peaks: {out}")
    return out


def add_measured_fraction(roofline, peaks):
    if not roofline or not peaks:
        return
    ref = peaks["hbm_read_gbs"] if roofline["bound"] == "hbm" else peaks["mfma_bf16_random_tflops"]
    roofline["peak_measured"] = ref
    roofline["frac_of_measured"] = round(roofline["achieved"] / ref, 4)


def run_workload(name, args, primary: bool):
    import torch
    import synth
    from block_speculative_decoding_dflash2_amd import (DFlash2, to_device, verify_accept, verify_workspace,
                                                        verify_sample, verify_sample_workspace)
    from block_speculative_decoding_dflash2_amd.runner import KernelTrace
    from block_speculative_decoding_dflash2_amd.metrics import speculative_metrics

    w = synth.get(name)
    if args.conv_group_size:
        w = w.replace(conv_group_size=args.conv_group_size)
    t0 = time.time()
    W = synth.make_weights(w)
    inp = synth.make_step_inputs(w)
    log(f"generated {w.name} inputs in {time.time() - t0:.1f}s")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    model = DFlash2(w.abi_config(), W, device=dev)
    B, bs, V, k = w.batch, w.block_size, w.vocab, w.top_k
    max_new = int(inp.new_offsets[-1])
    anchors = torch.from_numpy(inp.anchors).to(dev)
    offsets = torch.from_numpy(inp.new_offsets).to(dev)
    ctx_lens = torch.from_numpy(inp.ctx_lens).to(dev)
    # ROTATE independent copies of every per-step input and cache buffer
    sets = []
    for j in range(ROTATE):
        kc, vc = model.new_caches()
        model.load_context(kc, vc, inp.k_ctx, inp.v_ctx)
        taps = to_device(inp.taps.data.reshape(inp.taps.data.shape[0], -1), dev)
        sets.append({"kc": kc, "vc": vc, "taps": taps})
    ws = model.workspace(B, max_new)
    topk_ids = torch.empty((B, bs - 1, k), dtype=torch.int32, device=dev)
    topk_vals = torch.empty((B, bs - 1, k), dtype=torch.float32, device=dev)
    path = torch.empty((B, bs - 1), dtype=torch.int32, device=dev)
    drafts = torch.empty((B, bs - 1), dtype=torch.int32, device=dev)
    accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    bonus = torch.empty((B,), dtype=torch.int32, device=dev)
    sampling = None
    if args.sampling:
        T_, k_, p_ = args.sampling.split(",")
        sampling = (float(T_), int(k_), float(p_))
        vws = verify_sample_workspace(B, bs, V, dev)
        uniforms = torch.from_numpy(synth.make_uniforms((B, bs), tag=1)).to(dev)
    else:
        vws = verify_workspace(B, bs, V, dev)
    lens = torch.empty((B,), dtype=torch.int32, device=dev) if args.p_min is not None else None
    dlogits = labels = None
    if args.losses:
        gamma, wsel = (float(x) for x in args.losses.split(","))
        dlogits = torch.empty((B, bs - 1, V), dtype=torch.float32, device=dev)
        rng = np.random.default_rng(5)
        labels = torch.from_numpy(rng.integers(0, V, (B, bs - 1)).astype(np.int32)).to(dev)
        loss_out = torch.empty((4,), dtype=torch.float32, device=dev)

    # verifier logits planted around the drafts of a first (untimed) step,
    # one independent draw per buffer set
    s0 = sets[0]
    model.draft_block(anchors, s0["taps"], offsets, ctx_lens, max_new, s0["kc"], s0["vc"], workspace=ws,
                      topk_ids=topk_ids, topk_vals=topk_vals)
    model.select_path(anchors, topk_ids, topk_vals, path_idx=path, draft_tokens=drafts, want_score=False)
    torch.cuda.synchronize()
    d_host = drafts.cpu().numpy()
    for j, s in enumerate(sets):
        s["target"] = torch.from_numpy(synth.make_target_logits(w, d_host, tag=j)).to(dev)
    log(f"{w.name}: {ROTATE} buffer sets resident")

    it = [0]

    def step():
        s = sets[it[0] % ROTATE]
        it[0] += 1
        if dlogits is None and lens is None:
            # steps 1-4 in one call: the candidate merge runs in the selector's kernel
            model.draft_select(anchors, s["taps"], offsets, ctx_lens, max_new, s["kc"], s["vc"], workspace=ws,
                               topk_ids=topk_ids, topk_vals=topk_vals, path_idx=path, draft_tokens=drafts,
                               want_score=False)
        else:
            model.draft_block(anchors, s["taps"], offsets, ctx_lens, max_new, s["kc"], s["vc"], workspace=ws,
                              topk_ids=topk_ids, topk_vals=topk_vals, debug_logits=dlogits)
        if dlogits is not None:
            model.draft_losses(anchors, labels, dlogits, topk_ids, topk_vals, gamma, wsel, losses=loss_out)
        if lens is None:
            if dlogits is not None:
                model.select_path(anchors, topk_ids, topk_vals, path_idx=path, draft_tokens=drafts,
                                  want_score=False)
        else:
            model.select_path_stop(anchors, topk_ids, topk_vals, p_min=args.p_min, path_idx=path,
                                   draft_tokens=drafts, draft_lens=lens)
        if sampling is None:
            verify_accept(drafts, s["target"], workspace=vws, accepted=accepted, bonus=bonus)
        else:
            verify_sample(drafts, s["target"], uniforms, *sampling, draft_lens=lens, workspace=vws,
                          accepted=accepted, bonus=bonus)

    if args.copy_calibration and primary:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("calibration copy: 1 GiB read + 1 GiB written")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    s_step = elapsed / args.steps
    log(f"{w.name}: {args.steps} steps in {elapsed * 1e3:.2f} ms -> {s_step * 1e6:.1f} us/step")

    roofline = None
    per_kind = {}
    if not args.no_trace:
        # the library traces K/V bytes at the host-side bound max_context;
        # the algorithmic bytes count each sequence's actual rows
        ab = 4 if w.act_dtype == "fp32" else 2
        lib_kv = B * w.num_kv_heads * w.max_context * w.head_dim * 2 * ab
        real_kv = attention_kv_bytes(w, inp.ctx_lens)
        tr = KernelTrace(capacity=args.steps * 128 + 64)
        with tr:
            for _ in range(args.steps):
                step()
        torch.cuda.synchronize()
        recs = tr.records()
        tr.close()
        for kind, by, fl, ms in recs:
            if kind == "attention":
                by = by - lib_kv + real_kv
            d = per_kind.setdefault(kind, {"launches": 0, "ms": 0.0, "bytes": 0, "flops": 0})
            d["launches"] += 1
            d["ms"] += ms
            d["bytes"] += by
            d["flops"] += fl
        traced_total = sum(d["ms"] for d in per_kind.values())
        dom = max(per_kind, key=lambda kk: per_kind[kk]["ms"])
        d = per_kind[dom]
        secs = d["ms"] / 1e3
        ai = d["flops"] / max(d["bytes"], 1)
        mfma_peak = MFMA_PEAK_TFLOPS[w.weight_dtype]
        ridge = mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
        if ai < ridge:
            achieved = d["bytes"] / secs / 1e9
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
        else:
            achieved = d["flops"] / secs / 1e12
            roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": mfma_peak, "unit": "TFLOP/s",
                        "frac": round(achieved / mfma_peak, 4), "traffic": None}
        roofline.update({"kernel": dom, "launches_per_step": d["launches"] // args.steps,
                         "avg_launch_us": round(d["ms"] * 1e3 / d["launches"], 2),
                         "bytes_per_launch": d["bytes"] // d["launches"],
                         "flops_per_launch": d["flops"] // d["launches"],
                         "share_of_kernel_time": round(d["ms"] / traced_total, 3)})
        roofline["traffic"] = measured_traffic(w.name, dom)
        for kind, dd in sorted(per_kind.items(), key=lambda kv: -kv[1]["ms"]):
            log(f"  {kind:15s} {dd['launches'] // args.steps:3d}/step {dd['ms'] * 1e3 / args.steps:9.1f} us/step "
                f"{dd['bytes'] / max(dd['ms'], 1e-9) / 1e6:8.1f} GB/s "
                f"{dd['flops'] / max(dd['ms'], 1e-9) / 1e9:8.1f} TFLOP/s")
        log(f"  kernel time {traced_total * 1e3 / args.steps:.1f} us/step (wall {s_step * 1e6:.1f})")

    # acceptance of the planted verifier: the timed steps verify one planted
    # draw per sequence; with few sequences that is too few samples, so more
    # independent planted draws (untimed) are verified until at least 64
    # sequence-steps are counted
    acc = accepted.cpu().numpy().tolist()
    if sampling is None:
        for tag in range(ROTATE, ROTATE - 1 + -(-64 // B)):
            t_extra = torch.from_numpy(synth.make_target_logits(w, drafts.cpu().numpy(), tag=tag)).to(dev)
            verify_accept(drafts, t_extra, workspace=vws, accepted=accepted, bonus=bonus)
            acc += accepted.cpu().numpy().tolist()
            del t_extra
    spec = speculative_metrics(acc, bs - 1)
    model.close()
    del sets, ws, model
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, W, inp, primary)

    return {
        "w": w, "s_step": s_step, "roofline": roofline, "per_kind": per_kind, "cpu": cpu, "spec": spec,
        "sampling": sampling,
    }


def cpu_baseline(w, W, inp, whole: bool):
    """The oracle timed on this host's cores on a bounded sample of the same
    workload: whole steps (batch 1) repeated to ~10 s, or for a batched
    workload its first sequences, one at a time, until ~10 s (at most ~30 s)."""
    import oracle as O
    import synth
    from threadpoolctl import threadpool_info
    nthreads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    t_all, reps, seqs = 0.0, 0, 0
    while reps < 1 or (t_all < 10.0 and t_all + t_all / reps < 30.0):
        if whole:
            sub = inp
            n = w.batch
        else:
            sub = synth.make_step_inputs(w, np.array([reps]))
            n = 1
        t1 = time.time()
        O.step(w, W, sub)
        t_all += time.time() - t1
        reps += 1
        seqs += n
    what = (f"{reps} full steps of {w.name} ({w.batch} block(s) each)" if whole else
            f"sequences 0..{reps - 1} of {w.name} (of {w.batch}), one oracle step each")
    log(f"oracle on {w.name}: {seqs} blocks in {t_all:.1f}s, {nthreads} BLAS threads")
    return {"value": round(seqs / t_all, 6), "unit": "blocks/s", "cores": int(nthreads), "kind": "oracle",
            "sample": f"{what}, float64 NumPy oracle, {t_all:.1f}s in total",
            "cpu_model": cpu_model()}


def record(r, args):
    w, s_step = r["w"], r["s_step"]
    B, bs = w.batch, w.block_size
    spec = r["spec"]
    return {
        "value": round(B / s_step, 2),
        "unit": "blocks/s",
        "ms_per_step": round(s_step * 1e3, 4),
        "dtype": w.weight_dtype,
        "config": {"workload": w.name, "batch": B, "block_size": bs, "hidden": w.hidden,
                   "draft_layers": w.num_layers, "heads": f"{w.num_q_heads}/{w.num_kv_heads}x{w.head_dim}",
                   "ffn": w.ffn, "taps": f"{w.num_taps}x{w.tap_width}", "context": list(w.ctx),
                   "vocab": w.vocab, "top_k": w.top_k, "selector_rank": w.rank, "parallelism": "none (1 GPU)",
                   "verification": ("greedy" if r["sampling"] is None else
                                    "rejection sampling T=%g top_k=%d top_p=%g" % r["sampling"]),
                   "draft_p_min": args.p_min, "forward_losses": args.losses,
                   "conv": (f"dynamic, {w.conv_group_size} channels per group" if w.conv_group_size
                            else "static per-channel taps"),
                   "buffer_sets_rotated": ROTATE},
        "draft_tokens_per_s": round(B * (bs - 1) / s_step, 1),
        "roofline": r["roofline"],
        "cpu_baseline": r["cpu"],
        "acceptance": dict({kk: spec[kk] for kk in ("draft_acceptance_rate", "mean_acceptance_length")},
                           sequence_steps=spec["num_spec_steps"]),
        "kernels_us_per_step": {kk: round(dd["ms"] * 1e3 / args.steps, 2) for kk, dd in r["per_kind"].items()},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dense27b_bf16")
    ap.add_argument("--extra", default="fp8_b256",
                    help="comma-separated workloads also measured in this run ('none': only --workload)")
    ap.add_argument("--sampling", default=None, metavar="T,TOP_K,TOP_P",
                    help="verify by rejection sampling at this temperature / top-k / top-p "
                         "(default: greedy verification)")
    ap.add_argument("--p-min", type=float, default=None,
                    help="cut each draft path with the selector confidence rule (draft_p_min)")
    ap.add_argument("--losses", default=None, metavar="GAMMA,WEIGHT",
                    help="also evaluate the forward training losses on the step's logits (the draft "
                         "then writes its float32 logits) with synthetic labels")
    ap.add_argument("--conv-group-size", type=int, default=None,
                    help="run the workload with dynamic grouped convolution (channels per group)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-trace", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured MFMA / HBM read ceilings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the step shards by sequence with no exchange, so "
              f"--gpus {args.gpus} is not supported (run one process per GPU).", file=sys.stderr)
        sys.exit(2)

    peaks = None if args.no_peaks else measure_peaks()
    main_r = run_workload(args.workload, args, primary=True)
    add_measured_fraction(main_r["roofline"], peaks)
    w = main_r["w"]
    rec = record(main_r, args)
    out = {
        "metric": "drafted blocks/s per MI355X",
        "value": rec.pop("value"),
        "unit": rec.pop("unit"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": rec.pop("dtype"),
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) taps and context, planted-argmax verifier logits)",
    }
    out.update(rec)
    extras = [x for x in (args.extra or "").split(",") if x and x != "none" and x != args.workload]
    if extras:
        out["extra_workloads"] = []
        for name in extras:
            r = run_workload(name, args, primary=False)
            add_measured_fraction(r["roofline"], peaks)
            out["extra_workloads"].append(record(r, args))
    if peaks:
        out["measured_peaks"] = peaks
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
