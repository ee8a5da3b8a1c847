"""Throughput of the streamed LoRA training step (forward + recompute backward) at the
Llama-3.1-8B shape on one MI355X, through the C ABI.

Workload: 32 decoder layers, hidden 4096, 32/8 heads x 128, SwiGLU 14336; base
weights ~ N(0, 0.02) in bf16, NF4-packed (block 64) with double-quantised absmax
(8-bit, block 256) in pinned host RAM; LoRA r 16 / alpha 32 on all seven
projections; batch 8 x seq 512 bf16 X ~ N(0, 1), dY ~ N(0, 1); every layer streamed
through a two-slot device pool for the forward and again for the recompute
backward.  Synthetic data, random weights (no checkpoints or datasets).

One step = ls_forward + ls_backward + ls_sync; inputs are resident in HBM when the
timed region starts.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def h2d_probe(torch, nbytes=256 << 20, reps=6):
    """Best-of-N pinned host -> device copy rate (GB/s) on a side stream."""
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    s = torch.cuda.Stream()
    best = float("inf")
    with torch.cuda.stream(s):
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            dst.copy_(src, non_blocking=True)
            e1.record(s)
            e1.synchronize()
            best = min(best, e0.elapsed_time(e1))
    return nbytes / (best * 1e-3) / 1e9


def host_cpu():
    """Model name, logical CPUs and physical cores of this host (/proc/cpuinfo)."""
    model, cores, phys = None, set(), None
    try:
        for line in open("/proc/cpuinfo"):
            k, _, v = line.partition(":")
            k, v = k.strip(), v.strip()
            if k == "model name" and model is None:
                model = v
            elif k == "physical id":
                phys = v
            elif k == "core id":
                cores.add((phys, v))
    except OSError:
        pass
    return {"model": model, "logical_cpus": os.cpu_count(), "physical_cores": len(cores) or None}


def blas_threads():
    from threadpoolctl import threadpool_info
    n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
    return max(n) if n else 1


def oracle_layers(w, n_layers):
    """(seconds spent in the oracle's packer, dequantised layers) for layers 0 .. n_layers-1."""
    from layer_streamed_qlora_amd import synth
    from oracle import stack
    src = [synth.layer_weights(w, l) for l in range(n_layers)]
    t0 = time.perf_counter()
    enc = [stack.quantize_layer(s, w.quant, w.double_quant) for s in src]
    t_pack = time.perf_counter() - t0
    nbytes = sum(v.size * 2 for s in src for v in s.values())
    return t_pack, nbytes, [stack.dequant_layer(e) for e in enc]


def oracle_step_time(w, layers, batch, seq, threads=None):
    """Seconds of one oracle forward + recompute backward over `layers` at batch x seq,
    with the BLAS thread pool limited to `threads` if given."""
    from threadpoolctl import threadpool_limits
    from layer_streamed_qlora_amd import synth
    from oracle import model, stack
    nl = len(layers)
    sub = w.with_(n_layers=nl, batch=batch, seq=seq)
    loras = [synth.layer_lora(w, l) for l in range(nl)]
    x, dy = synth.activations(sub)
    shp = model.LayerShape(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.intermediate, w.rms_eps,
                           w.rope_theta, w.lora_r, w.lora_alpha)
    with threadpool_limits(threads):
        t0 = time.perf_counter()
        stack.train_step(x, dy, layers, loras, shp, batch, seq, parity=True, with_reference=w.dpo)
        return time.perf_counter() - t0


def cpu_baseline(w, full=False):
    """The oracle, untuned, on bounded samples, scaled to the stack's depth.

    The reported value: 1 of the stack's layers at batch 1 x seq 512, one forward +
    recompute backward with every BLAS thread.  Beside it: the same layer at 1 x 128 on
    one thread, the whole two-layer toy stack, the oracle's packer rate, and (full=True)
    one Qwen2.5-32B-shaped layer at 1 x 256."""
    from layer_streamed_qlora_amd import synth
    threads = blas_threads()
    t_pack, nbytes, layers = oracle_layers(w, 1)
    dt = oracle_step_time(w, layers, 1, 512)
    out = {"value": 512 / (dt * w.n_layers), "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"1 of {w.n_layers} layers at batch 1 x seq 512, one forward + recompute backward in "
                     f"{dt:.2f} s, scaled by depth ({w.n_layers}/1)"}
    dt1 = oracle_step_time(w, layers, 1, 128, threads=1)
    toy = synth.WORKLOADS["toy"]
    _, _, toy_layers = oracle_layers(toy, toy.n_layers)
    dtt = oracle_step_time(toy, toy_layers, toy.batch, toy.seq)
    dtt1 = oracle_step_time(toy, toy_layers, toy.batch, toy.seq, threads=1)
    more = {
        "host": host_cpu(),
        "one_thread": {"value": 128 / (dt1 * w.n_layers), "unit": "tokens/s",
                       "sample": f"1 of {w.n_layers} layers at batch 1 x seq 128 on 1 thread in {dt1:.2f} s, "
                                 "scaled by depth"},
        "toy_step": {"seconds": round(dtt, 4), "seconds_one_thread": round(dtt1, 4),
                     "sample": f"the whole {toy.n_layers}-layer toy stack at batch {toy.batch} x seq {toy.seq}"},
        "packer": {"MB_per_s": round(nbytes / t_pack / 1e6, 1),
                   "sample": f"NF4{' + double-quant' if w.double_quant else ''} encoding of one layer, "
                             f"{nbytes / 1e6:.0f} MB of bf16 weights in {t_pack:.2f} s"},
    }
    if full:
        q = synth.WORKLOADS["qwen32b"]
        _, _, ql = oracle_layers(q, 1)
        dq = oracle_step_time(q, ql, 1, 256)
        more["qwen32b"] = {"value": 256 / (dq * q.n_layers), "unit": "tokens/s",
                           "sample": f"1 of {q.n_layers} Qwen2.5-32B-shaped layers at batch 1 x seq 256 in "
                                     f"{dq:.2f} s, scaled by depth"}
    out["more"] = more
    return out


def profile_record(name):
    """The machine-readable line of a committed counter summary under profiles/, or None
    when the kernel source changed since the counters were taken."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    try:
        lines = open(os.path.join(here, "profiles", name)).read().splitlines()
    except OSError:
        return None
    for line in lines:
        if line.startswith("machine-readable: "):
            rec = json.loads(line[len("machine-readable: "):])
            src = os.path.join(here, rec["kernel_source"])
            if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["kernel_source_sha256"]:
                return None
            return rec
    return None


def measured_traffic(kernel_class):
    """HBM bytes per launch of the kernel class on the forward pass's launches, the ones
    the timed region times (FETCH_SIZE + WRITE_SIZE counters)."""
    rec = profile_record("llama8b_gemm_traffic.md")
    if rec is None or rec.get("class") != kernel_class or "traffic_bytes_per_launch_forward_pass" not in rec:
        return None
    return float(rec["traffic_bytes_per_launch_forward_pass"])


def measured_mfma_busy():
    """MFMA busy share of cycles per dequant-GEMM kernel (SQ_VALU_MFMA_BUSY_CYCLES)."""
    rec = profile_record("llama8b_gemm_mfma_counters.md")
    if rec is None:
        return None
    return {"mfma_busy": rec["mfma_busy"], "shader_clock_GHz": rec["shader_clock_GHz"],
            "source": "profiles/llama8b_gemm_mfma_counters.md"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama8b")
    ap.add_argument("--layers", type=int, default=0, help="override depth (0 = the workload's)")
    ap.add_argument("--batch", type=int, default=0, help="override the batch (0 = the workload's)")
    ap.add_argument("--seq", type=int, default=0, help="override the sequence length (0 = the workload's)")
    ap.add_argument("--buffers", type=int, default=2,
                    help="device slots of the streaming pool (0 = as deep as half the free memory allows)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline-full", action="store_true",
                    help="also time one Qwen2.5-32B-shaped layer on the oracle (about a minute more)")
    ap.add_argument("--no-profile", action="store_true")
    ap.add_argument("--vocab", type=int, default=128256, help="output-head rows for the head+loss measurement (0 = none)")
    ap.add_argument("--store-file", default="", help="keep the frozen base in this file instead of pinned RAM")
    ap.add_argument("--profile-stride", type=int, default=4,
                    help="time the forward GEMMs of every k-th layer in the timed region (1 = every layer)")
    ap.add_argument("--copy-split", type=int, default=0, choices=(0, 1),
                    help="1 = copy each layer as four separately fenced pieces (q|k|v, o, gate|up, down)")
    ap.add_argument("--resident", action="store_true",
                    help="keep every layer on the device (no streaming): the reference point of the streamed run")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from layer_streamed_qlora_amd import binding as B
    from layer_streamed_qlora_amd import synth

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    w = synth.WORKLOADS[args.workload]
    if args.layers:
        w = w.with_(n_layers=args.layers)
    if args.batch or args.seq:
        w = w.with_(batch=args.batch or w.batch, seq=args.seq or w.seq)
    T = w.tokens
    profile = 0 if args.no_profile else 1
    # the timed region records events around the forward pass's dequant GEMMs of every
    # profile_stride-th layer only (the roofline kernel; every layer has the same shapes);
    # every event is a packet in the stream and widens the gap before the next kernel, so
    # the full per-class breakdown comes from extra steps afterwards
    cfg = B.make_config(w, n_buffers=args.buffers, profile=B.LS_PROFILE_GEMM if profile else 0, adamw=1,
                        profile_stride=args.profile_stride,
                        resident=1 if args.resident else 0,
                        vocab=args.vocab,
                        store_path=args.store_file or None, copy_split=args.copy_split)
    t0 = time.time()
    ctx = B.Context(cfg)
    t_stage, staged_bytes = 0.0, 0
    for l in range(w.n_layers):
        dw = synth.device_layer_weights(w, l)
        host = {k: v.view(torch.int16).cpu().numpy().view(np.uint16) for k, v in dw.items()}
        ts = time.perf_counter()
        ctx.stage_layer(l, host)
        t_stage += time.perf_counter() - ts
        staged_bytes += sum(v.nbytes for v in host.values())
        del dw, host
        if (l + 1) % 8 == 0 and l + 1 < w.n_layers:
            log(f"staged {l + 1} of {w.n_layers} layers ({time.time() - t0:.0f} s)")
    loras = [synth.device_lora(w, l) for l in range(w.n_layers)]
    grads = []
    for l in range(w.n_layers):
        gl = {}
        for i, p in enumerate(synth.PROJS):
            a, b = loras[l][p]
            da, db = torch.zeros_like(a), torch.zeros_like(b)
            gl[p] = (da, db)
            ctx.set_lora(l, i, a.data_ptr(), b.data_ptr(), da.data_ptr(), db.data_ptr())
        grads.append(gl)
    g = torch.Generator(device="cuda:0")
    g.manual_seed(7)
    X = torch.randn((T, w.hidden), generator=g, device="cuda:0").to(torch.bfloat16)
    g.manual_seed(8)
    dY = torch.randn((T, w.hidden), generator=g, device="cuda:0").to(torch.bfloat16)
    Y = torch.empty_like(X)
    dX = torch.empty_like(X)
    # a DPO workload runs each layer's adapters-off reference pass on the same slot
    Yr = torch.empty_like(X) if w.dpo else None
    torch.cuda.synchronize()
    log(f"setup {time.time() - t0:.1f} s: {w.n_layers} layers staged, blob {ctx.stats().blob_bytes / 1e6:.2f} MB")
    probe = h2d_probe(torch)
    log(f"host-link probe {probe:.2f} GB/s")

    def step():
        ctx.forward(X.data_ptr(), w.batch, w.seq, 1, Y.data_ptr(), Yr.data_ptr() if Yr is not None else 0)
        ctx.backward(dY.data_ptr(), dX.data_ptr(), 0)
        ctx.sync()

    for i in range(args.warmup):
        step()
        log(f"warmup step {i} done")
    torch.cuda.synchronize()
    s0 = ctx.stats()
    kacc = {k: [0, 0.0, 0.0, 0.0] for k in B.KERNEL_CLASSES}

    def add_kernels(st, into):
        for j, k in enumerate(B.KERNEL_CLASSES):
            into[k][0] += st.k_launches[j]
            into[k][1] += st.k_ms[j]
            into[k][2] += st.k_flop[j]
            into[k][3] += st.k_bytes[j]

    t_start = time.perf_counter()
    for i in range(args.steps):
        step()
        add_kernels(ctx.stats(), kacc)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    s1 = ctx.stats()
    log(f"timed {args.steps} steps in {elapsed:.3f} s")
    # per-class breakdown and copy / compute overlap: fully profiled steps after the timed region
    n_b = 2
    acc = {"copy": 0.0, "compute": 0.0, "overlap": 0.0, "span": 0.0}
    kfull = {k: [0, 0.0, 0.0, 0.0] for k in B.KERNEL_CLASSES}
    if profile:
        ctx.set_profile(B.LS_PROFILE_ALL)
        for i in range(n_b):
            step()
            st = ctx.stats()
            acc["copy"] += st.last_copy_ms
            acc["compute"] += st.last_compute_ms
            acc["overlap"] += st.last_overlap_ms
            acc["span"] += st.last_span_ms
            add_kernels(st, kfull)
    ms_per_step = elapsed / args.steps * 1e3
    value = T * args.steps / elapsed
    assert torch.isfinite(Y.float()).all() and torch.isfinite(dX.float()).all(), "non-finite output"

    copies = (s1.h2d_copies - s0.h2d_copies) / args.steps
    h2d_bytes = (s1.h2d_bytes - s0.h2d_bytes) / args.steps
    shape = {"llama8b": "Llama-3.1-8B", "qwen3b": "Qwen2.5-3B", "qwen32b": "Qwen2.5-32B",
             "qwen72b": "Qwen2.5-72B", "toy": "toy"}.get(args.workload, args.workload)
    base = ("NF4 block 64 + double-quant absmax" if w.double_quant else "NF4 block 64, fp32 absmax") \
        if w.quant == "nf4" else "bf16"
    metric = ("train tokens/s (fwd+bwd, streamed NF4 base) @Llama-3.1-8B shape"
              if args.workload == "llama8b" and not args.resident else
              f"train tokens/s (fwd+bwd{' + reference pass' if w.dpo else ''}, "
              f"{'resident' if args.resident else 'streamed'} {w.quant.upper()} base) "
              f"@{shape} shape")
    out = {
        "metric": metric,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {shape}-shaped decoder stack, {w.n_layers} layers, "
                               f"hidden {w.hidden}, {w.n_heads}/{w.n_kv_heads} heads x {w.head_dim}, "
                               f"SwiGLU {w.intermediate}, {base} base, "
                               f"LoRA r {w.lora_r} alpha {int(w.lora_alpha)} on 7 projections, "
                               + ("every layer resident on the device" if args.resident else
                                  f"streamed through {s1.n_slots} device slots"
                                  + (" (depth chosen by the library)" if args.buffers == 0 else ""))
                               + (", adapters-off reference pass per layer (DPO)" if w.dpo else ""),
                   "batch": w.batch, "seq": w.seq, "tokens_per_step": T, "parallelism": "none (1 GPU)",
                   "store": "file (page cache dropped after each read)" if args.store_file else "pinned host RAM",
                   "copies": ("each layer as four separately fenced pieces (q|k|v, o, gate|up, down)"
                              if args.copy_split else "one per layer")},
        # the library's one device allocation (its plan), the caller's tensors (inputs,
        # outputs, adapters and their gradients, allocated through torch), the pinned store
        "memory": {"library_device_bytes": s1.device_bytes, "caller_device_bytes_peak": torch.cuda.max_memory_allocated(),
                   "pinned_store_bytes": s1.store_bytes, "blob_bytes": s1.blob_bytes},
        # the library's host packer (ls_stage_layer: NF4 encoding into the pinned store)
        "staging": {"bf16_MB_per_s": round(staged_bytes / t_stage / 1e6, 1) if t_stage else None,
                    "layers": w.n_layers, "seconds": round(t_stage, 2)},
    }
    if profile:
        kern = {k: {"launches_per_step": v[0] / n_b, "ms_per_step": v[1] / n_b,
                    "tflops": (v[2] / (v[1] * 1e-3) / 1e12) if v[1] > 0 else None,
                    "avg_launch_ms": v[1] / v[0] if v[0] else None} for k, v in kfull.items()}
        dom = "gemm_fwd"    # the dominant class (largest summed time in the breakdown below)
        kl, kms, kfl, kby = kacc[dom]
        achieved = kfl / (kms * 1e-3) / 1e12
        # the class is timed on the forward pass's launches (4 per layer, of every
        # profile_stride-th layer), where it runs alone; the recompute's launches share the
        # GPU with the previous layer's backward
        out["roofline"] = {"bound": "mfma", "kernel": f"fused dequant GEMM ({dom}, forward-pass launches"
                                                      + (f" of every {args.profile_stride}th layer" if args.profile_stride > 1 else "") + ")",
                           "launches_per_step": kl / args.steps, "achieved": round(achieved, 1),
                           "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                           "traffic": measured_traffic(dom), "avg_launch_ms": round(kms / kl, 4),
                           "flop_per_launch": kfl / kl, "algorithmic_bytes_per_launch": kby / kl}
        gemm_ms = kfull["gemm_fwd"][1] + kfull["gemm_bwd"][1]
        gemm_fl = kfull["gemm_fwd"][2] + kfull["gemm_bwd"][2]
        out["mfma"] = {"dequant_gemm_tflops": round(gemm_fl / (gemm_ms * 1e-3) / 1e12, 1),
                       "frac_of_peak": round(gemm_fl / (gemm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                       "kernels": kern,
                       "counters": measured_mfma_busy(),
                       "breakdown_from": f"{n_b} fully profiled steps after the timed region (events around "
                                         "every launch); the timed region times the forward dequant GEMMs only"}
        copy_ms = acc["copy"] / n_b
        out["h2d"] = {"bytes_per_step": h2d_bytes, "copies_per_step": copies,
                      "achieved_GBps": round(h2d_bytes / (copy_ms * 1e-3) / 1e9, 2) if copy_ms else None,
                      "probe_GBps": round(probe, 2),
                      "frac_of_probe": round(h2d_bytes / (copy_ms * 1e-3) / 1e9 / probe, 4) if copy_ms else None,
                      "copy_ms_per_step": round(copy_ms, 3),
                      "overlap_ms_per_step": round(acc["overlap"] / n_b, 3),
                      "copy_hidden_frac": round(acc["overlap"] / acc["copy"], 4) if acc["copy"] else None}
    if profile:
        # the optimizer step that closes the training loop, after the timed region (it is
        # not part of the fwd+bwd metric): AdamW over every adapter from the last gradients
        n_opt = 10
        oms, obytes = [], 0.0
        for t in range(1, n_opt + 1):
            ctx.adamw_step(t, 2e-4)
            ctx.sync()
            st = ctx.stats()
            oms.append(st.k_ms[B.KERNEL_CLASSES.index("optim")])
            obytes = st.k_bytes[B.KERNEL_CLASSES.index("optim")]
        o_ms = sorted(oms)[len(oms) // 2]
        out["optimizer"] = {"kernel": "k_adamw (AdamW over every adapter, one launch)",
                            "params": int(obytes / 28), "algorithmic_bytes_per_launch": obytes,
                            "median_launch_ms": round(o_ms, 4), "bound": "hbm",
                            "achieved": round(obytes / (o_ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(obytes / (o_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    if profile and args.vocab:
        # the training step with the output head and SFT loss (outside the fwd+bwd metric):
        # forward, head + loss over the streamed vocabulary slices, backward from its dY
        g.manual_seed(9)
        Wh = (torch.randn((args.vocab, w.hidden), generator=g, device="cuda:0") * 0.02).to(torch.bfloat16)
        gf = torch.ones(w.hidden, dtype=torch.bfloat16, device="cuda:0")
        ctx.stage_head(Wh.view(torch.int16).cpu().numpy().view(np.uint16), gf.view(torch.int16).cpu().numpy().view(np.uint16))
        del Wh
        labels = torch.from_numpy(synth.labels(w, args.vocab, T)).to("cuda:0")
        hout = torch.zeros(2 + 2 * w.batch, device="cuda:0")
        dYh = torch.empty_like(X)

        def head_step():
            ctx.forward(X.data_ptr(), w.batch, w.seq, 1, Y.data_ptr())
            ctx.head_loss(Y.data_ptr(), 0, labels.data_ptr(), B.LS_LOSS_SFT, 0.0, hout.data_ptr(), dYh.data_ptr())
            ctx.backward(dYh.data_ptr(), dX.data_ptr(), 0)
            ctx.sync()

        head_step()
        n_h = 3
        hk = [0.0, 0.0]
        c0 = ctx.stats().h2d_copies
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n_h):
            head_step()
            st = ctx.stats()
            j = B.KERNEL_CLASSES.index("head")
            hk[0] += st.k_ms[j]; hk[1] += st.k_flop[j]
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / n_h
        loss = float(hout[0].item())
        assert np.isfinite(loss) and torch.isfinite(dYh.float()).all(), "non-finite head loss or gradient"
        out["with_head"] = {"vocab": args.vocab, "loss": "SFT cross entropy, 25% of tokens unlabelled",
                            "head_slices": -(-args.vocab // (ctx.stats().blob_bytes // (2 * w.hidden) // 256 * 256)),
                            "ms_per_step": round(dt * 1e3, 3), "tokens_per_s": round(T / dt, 1),
                            "head_kernel_ms_per_step": round(hk[0] / n_h, 3),
                            "head_tflops": round(hk[1] / (hk[0] * 1e-3) / 1e12, 1) if hk[0] else None,
                            "copies_per_step": (ctx.stats().h2d_copies - c0) / n_h, "sft_loss": round(loss, 4)}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(w, full=args.cpu_baseline_full)
    ctx.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
