"""Workload shapes and seeded synthetic inputs.

This module holds no arithmetic of the method: it only defines the shapes of the
measured workloads and draws the random base weights, adapters, inputs and upstream
gradients that both the HIP path and the CPU oracle consume.  Neither side imports
the other; both take what this module produces.

Workloads (vocab-free decoder stacks; the pages measure Llama-3.1-8B with an NF4 base
and Qwen2.5-3B with a bf16 base: "Soup: Fine-Tuning an 8B Model on a 4 GB Laptop GPU,
One Layer at a Time", first paragraph; the >165 MB-per-layer NF4 case at 32B/72B: same
page, third paragraph; the DPO reference pass: "Soup CLI fine-tunes Llama-3.1-8B on a
4 GB laptop GPU ...", third paragraph):

* ``toy``      2 layers, hidden 256, 4/4 heads x 64, SwiGLU 688, NF4 (fp32 absmax),
               LoRA r 8 / alpha 16, batch 1 x seq 128.
* ``llama8b``  32 layers, hidden 4096, 32/8 heads x 128, SwiGLU 14336, NF4 + double
               quantised absmax, LoRA r 16 / alpha 32, batch 8 x seq 512.
* ``qwen3b``   36 layers, hidden 2048, 16/2 heads x 128, SwiGLU 11008, bf16 base,
               batch 4 x seq 1024.
* ``qwen32b``  64 layers, hidden 5120, 40/8 heads x 128, SwiGLU 27648, NF4 + DQ
               (> 165 MB per layer), batch 2 x seq 1024.
* ``qwen72b``  80 layers, hidden 8192, 64/8 heads x 128, SwiGLU 29568, NF4 + DQ, DPO:
               2 chosen/rejected pairs x seq 512 = 4 sequences of 512.

Distributions: base W ~ N(0, 0.02) (second argument = standard deviation), rounded to
bf16; RMSNorm weights = 1; A ~ N(0, 1/r); B ~ N(0, 0.01) (float32); X, dY ~ N(0, 1)
rounded to bf16.

Seeds: every tensor gets its own ``numpy`` PCG64 stream seeded with
SeedSequence([workload id, layer, tensor id]); X uses tensor id 100, dY 101.  The big
stacks can also be drawn on the GPU with a seeded ``torch.Generator``
(``device_layer_weights``); those values differ from the numpy ones and are used only
where nothing is compared against the oracle (timing).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

PROJS = ("q", "k", "v", "o", "gate", "up", "down")
TENSOR_ID = {p: i for i, p in enumerate(PROJS)}      # base weights 0..6
LORA_A_ID = {p: 10 + i for i, p in enumerate(PROJS)}  # 10..16
LORA_B_ID = {p: 20 + i for i, p in enumerate(PROJS)}  # 20..26
X_ID, DY_ID = 100, 101


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    quant: str            # "nf4" | "bf16"
    double_quant: bool
    lora_r: int
    lora_alpha: float
    batch: int
    seq: int
    dpo: bool = False
    rms_eps: float = 1e-5
    rope_theta: float = 1e4

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    def proj_shape(self, p):
        h, q, kv, i = self.hidden, self.n_heads * self.head_dim, self.n_kv_heads * self.head_dim, self.intermediate
        return {"q": (q, h), "k": (kv, h), "v": (kv, h), "o": (h, q),
                "gate": (i, h), "up": (i, h), "down": (h, i)}[p]

    def params_per_layer(self) -> int:
        return sum(a * b for a, b in (self.proj_shape(p) for p in PROJS))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "toy": Workload("toy", 0, 2, 256, 4, 4, 64, 688, "nf4", False, 8, 16.0, 1, 128),
    "llama8b": Workload("llama8b", 1, 32, 4096, 32, 8, 128, 14336, "nf4", True, 16, 32.0, 8, 512),
    "qwen3b": Workload("qwen3b", 2, 36, 2048, 16, 2, 128, 11008, "bf16", False, 16, 32.0, 4, 1024),
    "qwen32b": Workload("qwen32b", 3, 64, 5120, 40, 8, 128, 27648, "nf4", True, 16, 32.0, 2, 1024),
    "qwen72b": Workload("qwen72b", 4, 80, 8192, 64, 8, 128, 29568, "nf4", True, 16, 32.0, 4, 512, dpo=True),
}


def _rng(wid: int, layer: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([wid, layer, tensor])))


def _to_bf16_values(x32: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) via torch's own conversion and
    return the values as float32 (input plumbing, not part of the method)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def bf16_bits(values32: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of bf16-representable float32 values."""
    v = np.ascontiguousarray(values32, dtype=np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def layer_weight(w: Workload, layer: int, p: str) -> np.ndarray:
    """Base weight p of one layer: float32 array of bf16 values [out, in]."""
    x = _rng(w.wid, layer, TENSOR_ID[p]).standard_normal(w.proj_shape(p), dtype=np.float32) * np.float32(0.02)
    return _to_bf16_values(x)


def layer_weights(w: Workload, layer: int) -> dict:
    """Base weights of one layer: proj -> float32 array of bf16 values [out, in];
    'g1', 'g2' -> ones [hidden].  The seven tensors have independent streams, so they
    are drawn on a thread pool (the values do not depend on it)."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=len(PROJS)) as ex:
        out = dict(zip(PROJS, ex.map(lambda p: layer_weight(w, layer, p), PROJS)))
    out["g1"] = np.ones(w.hidden, np.float32)
    out["g2"] = np.ones(w.hidden, np.float32)
    return out


def layer_lora(w: Workload, layer: int) -> dict:
    """Adapters of one layer: proj -> (A [r, in], B [out, r]) float32."""
    out = {}
    r = w.lora_r
    for p in PROJS:
        n_out, n_in = w.proj_shape(p)
        a = _rng(w.wid, layer, LORA_A_ID[p]).standard_normal((r, n_in), dtype=np.float32) * np.float32(1.0 / r)
        b = _rng(w.wid, layer, LORA_B_ID[p]).standard_normal((n_out, r), dtype=np.float32) * np.float32(0.01)
        out[p] = (a, b)
    return out


def activations(w: Workload, tokens: int | None = None):
    """(X, dY), each [tokens, hidden] float32 arrays of bf16 values."""
    t = w.tokens if tokens is None else tokens
    x = _rng(w.wid, 0, X_ID).standard_normal((t, w.hidden), dtype=np.float32)
    dy = _rng(w.wid, 0, DY_ID).standard_normal((t, w.hidden), dtype=np.float32)
    return _to_bf16_values(x), _to_bf16_values(dy)


def device_layer_weights(w: Workload, layer: int, device="cuda"):
    """Fast on-device draw of one layer's bf16 base weights (torch tensors), seeded per
    (workload, layer, tensor).  Used for timing runs of the large stacks."""
    import torch
    out = {}
    for p in PROJS:
        g = torch.Generator(device=device)
        g.manual_seed(1_000_000 * w.wid + 1000 * layer + TENSOR_ID[p])
        t = torch.randn(w.proj_shape(p), generator=g, device=device, dtype=torch.float32)
        out[p] = (t * 0.02).to(torch.bfloat16)
    out["g1"] = torch.ones(w.hidden, device=device, dtype=torch.bfloat16)
    out["g2"] = torch.ones(w.hidden, device=device, dtype=torch.bfloat16)
    return out


def device_lora(w: Workload, layer: int, device="cuda"):
    import torch
    out = {}
    r = w.lora_r
    for p in PROJS:
        n_out, n_in = w.proj_shape(p)
        g = torch.Generator(device=device)
        g.manual_seed(1_000_000 * w.wid + 1000 * layer + LORA_A_ID[p])
        a = torch.randn((r, n_in), generator=g, device=device) * (1.0 / r)
        g.manual_seed(1_000_000 * w.wid + 1000 * layer + LORA_B_ID[p])
        b = torch.randn((n_out, r), generator=g, device=device) * 0.01
        out[p] = (a.contiguous(), b.contiguous())
    return out


HEAD_W_ID, HEAD_G_ID, LABEL_ID = 90, 91, 92


def head_weights(w: Workload, vocab: int):
    """Frozen output head: (W [vocab, hidden] float32 of bf16 values ~ N(0, 0.02),
    g_final [hidden] float32 of bf16 values near 1)."""
    W = _rng(w.wid, 0, HEAD_W_ID).standard_normal((vocab, w.hidden), dtype=np.float32) * np.float32(0.02)
    g = 1.0 + 0.1 * _rng(w.wid, 0, HEAD_G_ID).standard_normal(w.hidden, dtype=np.float32)
    return _to_bf16_values(W), _to_bf16_values(g.astype(np.float32))


def labels(w: Workload, vocab: int, tokens: int, ignore_frac: float = 0.25, seed: int = 0):
    """int32 target ids in [0, vocab), a fraction of them -100 (no loss), like the
    prompt tokens of instruction records."""
    g = _rng(w.wid, seed, LABEL_ID)
    lab = g.integers(0, vocab, tokens).astype(np.int32)
    lab[g.random(tokens) < ignore_frac] = -100
    return lab
