"""Shared helpers for the tests: run the HIP path through the C ABI on seeded inputs,
and run the oracle on the same inputs.  The two sides share only ``synth``."""
from __future__ import annotations

import numpy as np

from layer_streamed_qlora_amd import binding as B
from layer_streamed_qlora_amd import synth
from oracle import model as omodel
from oracle import nf4 as onf4
from oracle import stack as ostack

PROJS = synth.PROJS


def rel_l2(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    n = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (n if n > 0 else 1.0))


def layer_bits(w, layer_seed):
    lw = synth.layer_weights(w, layer_seed)
    return lw, {k: synth.bf16_bits(v) for k, v in lw.items()}


def oracle_shape(w):
    return omodel.LayerShape(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.intermediate,
                             w.rms_eps, w.rope_theta, w.lora_r, w.lora_alpha)


class GpuRun:
    """One context with staged layers and torch-owned adapters on cuda:0."""

    def __init__(self, w, layer_seeds, resident=0, n_buffers=2, profile=0, zero_b=False, max_tokens=None,
                 max_seq=None, lora_mask=0x7F, weights=None, adamw=0, vocab=0, store_path=None, layer_bits=None,
                 copy_split=0, profile_stride=0):
        """weights: per-layer float32 dicts of bf16 values (default: drawn from the
        seeds); layer_bits: per-layer dicts of bf16 bit patterns, staged as they are
        (then ``src`` is None)."""
        import torch
        self.torch = torch
        self.w = w
        self.layer_seeds = list(layer_seeds)
        L = len(self.layer_seeds)
        cfg = B.make_config(w, n_buffers=n_buffers, resident=resident, profile=profile, n_layers=L,
                            max_tokens=max_tokens, max_seq=max_seq, lora_mask=lora_mask, adamw=adamw,
                            vocab=vocab, store_path=store_path, copy_split=copy_split,
                            profile_stride=profile_stride)
        self.ctx = B.Context(cfg)
        self.src = [] if layer_bits is None else None
        for i, seed in enumerate(self.layer_seeds):
            if layer_bits is not None:
                self.ctx.stage_layer(i, layer_bits[i])
                continue
            lw = weights[i] if weights is not None else synth.layer_weights(w, seed)
            self.src.append(lw)
            self.ctx.stage_layer(i, {k: synth.bf16_bits(v) for k, v in lw.items()})
        self.lora_np = []
        self.A, self.Bm, self.dA, self.dB = [], [], [], []
        dev = torch.device("cuda:0")
        for i, seed in enumerate(self.layer_seeds):
            lo = synth.layer_lora(w, seed)
            if zero_b:
                lo = {p: (a, np.zeros_like(b)) for p, (a, b) in lo.items()}
            self.lora_np.append(lo)
            A, Bm, dA, dB = {}, {}, {}, {}
            for pi, p in enumerate(PROJS):
                a, b = lo[p]
                A[p] = torch.from_numpy(a).to(dev)
                Bm[p] = torch.from_numpy(b).to(dev)
                dA[p] = torch.zeros_like(A[p])
                dB[p] = torch.zeros_like(Bm[p])
                if (lora_mask >> pi) & 1:
                    self.ctx.set_lora(i, pi, A[p].data_ptr(), Bm[p].data_ptr(), dA[p].data_ptr(), dB[p].data_ptr())
            self.A.append(A); self.Bm.append(Bm); self.dA.append(dA); self.dB.append(dB)

    def to_dev_bf16(self, x32):
        t = self.torch.from_numpy(synth.bf16_bits(x32).view(np.int16)).to("cuda:0")
        return t.view(self.torch.bfloat16)

    def from_dev_bf16(self, t):
        return (t.view(self.torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)

    def step(self, x32, dy32, batch, seq, with_ref=False, backward=True, lora_on=True, accumulate=0):
        torch = self.torch
        T = batch * seq
        X = self.to_dev_bf16(x32)
        Y = torch.empty((T, self.w.hidden), dtype=torch.bfloat16, device="cuda:0")
        Yr = torch.empty_like(Y) if with_ref else None
        self.ctx.forward(X.data_ptr(), batch, seq, lora_on, Y.data_ptr(), Yr.data_ptr() if with_ref else 0)
        out = {}
        if backward:
            dY = self.to_dev_bf16(dy32)
            dX = torch.empty_like(Y)
            self.ctx.backward(dY.data_ptr(), dX.data_ptr(), accumulate)
        self.ctx.sync()
        torch.cuda.synchronize()
        out["Y"] = self.from_dev_bf16(Y)
        if with_ref:
            out["Y_ref"] = self.from_dev_bf16(Yr)
        if backward:
            out["dX"] = self.from_dev_bf16(dX)
            out["dA"] = [{p: self.dA[l][p].cpu().numpy().copy() for p in PROJS} for l in range(len(self.layer_seeds))]
            out["dB"] = [{p: self.dB[l][p].cpu().numpy().copy() for p in PROJS} for l in range(len(self.layer_seeds))]
        return out

    def read_weight(self, layer, proj):
        torch = self.torch
        n_out, n_in = self.w.proj_shape(PROJS[proj])
        out = torch.empty((n_out, n_in), dtype=torch.bfloat16, device="cuda:0")
        self.ctx.read_weight(layer, proj, out.data_ptr())
        torch.cuda.synchronize()
        return out.view(torch.int16).cpu().numpy().view(np.uint16)

    def close(self):
        self.ctx.close()


def oracle_layers(w, src_layers):
    """Encode and dequantise every layer on the oracle side, the seven projections of a
    layer on a thread pool (numpy releases the interpreter lock in the heavy calls)."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=7) as ex:
        enc = [ostack.quantize_layer(lw, w.quant, w.double_quant, map_fn=ex.map) for lw in src_layers]
        deq = [ostack.dequant_layer(e, map_fn=ex.map) for e in enc]
    return enc, deq


def oracle_step(w, src_layers, loras, x32, dy32, batch, seq, with_ref=False, parity=True):
    _, lw = oracle_layers(w, src_layers)
    return ostack.train_step(x32, dy32, lw, loras, oracle_shape(w), batch, seq, parity=parity,
                             with_reference=with_ref)


def compare(gpu, ora, tol_act=1e-2, tol_grad=2e-2, layers=None):
    """Per-tensor relative L2 errors; returns (worst dict, failures list)."""
    errs = {"Y": rel_l2(gpu["Y"], ora["Y"])}
    if "dX" in gpu:
        errs["dX"] = rel_l2(gpu["dX"], ora["dX"])
        L = len(ora["grads"])
        for l in range(L) if layers is None else layers:
            for p in PROJS:
                da, db = ora["grads"][l][p]
                errs[f"dA[{l}].{p}"] = rel_l2(gpu["dA"][l][p], da)
                errs[f"dB[{l}].{p}"] = rel_l2(gpu["dB"][l][p], db)
    fails = [(k, v) for k, v in errs.items() if v > (tol_act if k == "Y" else tol_grad) or not np.isfinite(v)]
    return errs, fails
