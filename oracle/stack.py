"""The layer stack, its recompute backward, the adapters-off reference pass and a
simulated two-slot streaming pool (TEST INFRASTRUCTURE ONLY).

What the pages fix:

* the frozen base lives outside the GPU and each decoder layer is brought in one at a
  time through a two-buffer pool, the next layer loading while the current one
  computes; during backward every layer is read again for the checkpoint
  recomputation (the lachieslifestyle.com how-to, section "What Soup layer streaming
  changes"; "Soup: Fine-Tuning an 8B Model on a 4 GB Laptop GPU, One Layer at a Time",
  first paragraph);
* streaming changes where the weights come from, not the arithmetic: the forward is
  bit-exact against a resident run (same toknow.ai page, second paragraph);
* the DPO reference model is the same streamed base with its adapters switched off
  ("Soup CLI fine-tunes Llama-3.1-8B on a 4 GB laptop GPU ...", third paragraph).

So the stack is the plain composition of ``model.layer_forward`` over the layers; the
backward recomputes each layer from its saved input (its checkpoint) and applies
``model.layer_backward`` in reverse order.

Parity mode rounds to bf16 (round-to-nearest-even) at: the input X and the upstream
gradient dY, every layer output (= next layer's input and checkpoint), every
inter-layer dX, and the operands of every matrix product inside a layer (bf16 compute
dtype, see ``model``).  The dequantised weights are bf16 by construction.  All
accumulation is float64.  Exact mode rounds nowhere.
"""
from __future__ import annotations

import numpy as np

from . import nf4
from .model import PROJS, LayerShape, layer_backward, layer_forward


def _round(x, parity):
    return nf4.bf16_round(x).astype(np.float64) if parity else np.asarray(x, dtype=np.float64)


def _bf16(x):
    return nf4.bf16_round(x).astype(np.float64)


def _rnd(parity):
    return _bf16 if parity else (lambda x: x)


# ----------------------------------------------------------------- base weights
def quantize_layer(src: dict, quant: str, double_quant: bool, map_fn=map) -> dict:
    """Encode one layer's bf16 source weights the way the store holds them.
    Returns dict proj -> NF4Tensor (quant 'nf4') or float32 bf16 values (quant 'bf16'),
    plus 'g1', 'g2' (bf16 values, kept as is).  The projections are independent;
    ``map_fn`` (e.g. a thread pool's map) only decides how they are visited."""
    if quant not in ("nf4", "bf16"):
        raise ValueError(quant)

    def enc(p):
        return nf4.NF4Tensor(src[p], double_quant) if quant == "nf4" else np.asarray(src[p], np.float32)

    out = {"g1": np.asarray(src["g1"], np.float32), "g2": np.asarray(src["g2"], np.float32)}
    out.update(zip(PROJS, map_fn(enc, PROJS)))
    return out


def dequant_layer(enc: dict, map_fn=map) -> dict:
    """float64 weights the arithmetic uses (dequantised NF4 or the bf16 values)."""
    def deq(p):
        t = enc[p]
        return (t.dequant() if isinstance(t, nf4.NF4Tensor) else t).astype(np.float64)

    w = {"g1": enc["g1"].astype(np.float64), "g2": enc["g2"].astype(np.float64)}
    w.update(zip(PROJS, map_fn(deq, PROJS)))
    return w


def _lora64(lora_l):
    return {p: (np.asarray(a, np.float64), np.asarray(b, np.float64)) for p, (a, b) in lora_l.items()}


# ------------------------------------------------------------------------ stack
def stack_forward(x, layer_weights, loras, shp: LayerShape, batch, seq, lora_on=True,
                  parity=True, weight_source=None):
    """Forward through all layers.  ``layer_weights[l]`` are float64 weight dicts, or,
    if ``weight_source`` is given, it is called as weight_source(l) to fetch them (the
    streamed case).  Returns (Y, checkpoints) with checkpoints[l] = input of layer l."""
    get = weight_source or (lambda l: layer_weights[l])
    n_layers = len(loras)
    x = _round(x, parity)
    ckpts = []
    for l in range(n_layers):
        ckpts.append(x)
        y, _ = layer_forward(x, get(l), _lora64(loras[l]), shp, batch, seq, lora_on, _rnd(parity))
        x = _round(y, parity)
    return x, ckpts


def stack_backward(dy, ckpts, layer_weights, loras, shp: LayerShape, batch, seq,
                   parity=True, weight_source=None):
    """Recompute backward, last layer first.  Returns (dX, grads) with grads[l] a dict
    proj -> (dA, dB)."""
    get = weight_source or (lambda l: layer_weights[l])
    n_layers = len(loras)
    dy = _round(dy, parity)
    grads = [None] * n_layers
    for l in reversed(range(n_layers)):
        w = get(l)
        lo = _lora64(loras[l])
        _, cache = layer_forward(ckpts[l], w, lo, shp, batch, seq, True, _rnd(parity))   # recompute
        dx, grads[l] = layer_backward(dy, cache, w, lo, shp, batch, seq, _rnd(parity))
        dy = _round(dx, parity)
    return dy, grads


def train_step(x, dy, layer_weights, loras, shp, batch, seq, parity=True, with_reference=False):
    """Policy forward (+ optional adapters-off reference forward) and policy backward.
    Returns dict with Y, dX, grads and, if requested, Y_ref."""
    y, ckpts = stack_forward(x, layer_weights, loras, shp, batch, seq, True, parity)
    out = {"Y": y}
    if with_reference:
        out["Y_ref"], _ = stack_forward(x, layer_weights, loras, shp, batch, seq, False, parity)
    out["dX"], out["grads"] = stack_backward(dy, ckpts, layer_weights, loras, shp, batch, seq, parity)
    return out


# ------------------------------------------------- simulated streaming (two slots)
class HostStore:
    """Each layer's encoded tensors serialised into one byte blob; an offset table with
    64-bit offsets says where each piece starts.  Stands in for pinned host RAM."""

    ALIGN = 256

    def __init__(self, encoded_layers):
        self.layout = []          # per piece: (name, offset, nbytes, dtype, shape)
        self.meta = {}            # non-array facts (shapes, numel, double_quant, mean)
        first = encoded_layers[0]
        off = 0
        pieces = []
        for name in ("g1", "g2") + PROJS:
            t = first[name]
            if isinstance(t, nf4.NF4Tensor):
                self.meta[name] = ("nf4", t.shape, t.numel, t.double_quant)
                parts = [("packed", t.packed)]
                if t.double_quant:
                    parts += [("qabs", t.qabs), ("scale2", t.scale2),
                              ("mean", np.array([t.mean], np.float32))]
                else:
                    parts += [("absmax", t.absmax)]
            else:
                self.meta[name] = ("raw", t.shape)
                parts = [("raw", t)]
            for part, arr in parts:
                off = -(-off // self.ALIGN) * self.ALIGN
                pieces.append((name, part, np.int64(off), arr.nbytes, arr.dtype, arr.shape))
                off += arr.nbytes
        self.blob_bytes = int(-(-off // self.ALIGN) * self.ALIGN)
        self.layout = pieces
        self.blobs = [self._serialise(enc) for enc in encoded_layers]

    def _piece(self, enc, name, part):
        t = enc[name]
        if part == "raw":
            return np.asarray(t)
        if part == "mean":
            return np.array([t.mean], np.float32)
        return getattr(t, part)

    def _serialise(self, enc):
        blob = np.zeros(self.blob_bytes, dtype=np.uint8)
        for name, part, off, nbytes, dtype, shape in self.layout:
            arr = np.ascontiguousarray(self._piece(enc, name, part))
            assert arr.nbytes == nbytes and arr.dtype == dtype
            blob[int(off):int(off) + nbytes] = arr.view(np.uint8).reshape(-1)
        return blob

    def decode(self, buf) -> dict:
        """float64 weights read back out of a blob-shaped buffer (a device slot)."""
        got = {}
        for name, part, off, nbytes, dtype, shape in self.layout:
            got.setdefault(name, {})[part] = buf[int(off):int(off) + nbytes].view(dtype).reshape(shape)
        w = {}
        for name, parts in got.items():
            m = self.meta[name]
            if m[0] == "raw":
                w[name] = parts["raw"].astype(np.float64)
                continue
            _, shape, numel, dq = m
            codes = nf4.unpack_nibbles(parts["packed"], numel)
            absmax = (nf4.dq_decode(parts["qabs"], parts["scale2"], parts["mean"][0])
                      if dq else parts["absmax"])
            w[name] = nf4.dequant_codes(codes, absmax).reshape(shape).astype(np.float64)
        return w


class TwoSlotPool:
    """Copies blob l into slot l % n_slots before layer l runs and poisons the slot
    (0xFF bytes: NF4 code 15 and NaN scales) when the layer is done with it."""

    def __init__(self, store: HostStore, n_slots: int = 2):
        self.store = store
        self.slots = [np.full(store.blob_bytes, 0xFF, dtype=np.uint8) for _ in range(n_slots)]
        self.copies = 0

    def fetch(self, l):
        slot = self.slots[l % len(self.slots)]
        slot[:] = self.store.blobs[l]
        self.copies += 1
        w = self.store.decode(slot)
        slot[:] = 0xFF          # release: anything read after this sees poison
        return w


def streamed_train_step(x, dy, store: HostStore, loras, shp, batch, seq, parity=True, n_slots=2):
    """``train_step`` with every layer pulled through the pool: forward reads layers
    0..L-1, the recompute backward reads L-1..0 again."""
    pool = TwoSlotPool(store, n_slots)
    y, ckpts = stack_forward(x, None, loras, shp, batch, seq, True, parity, weight_source=pool.fetch)
    dx, grads = stack_backward(dy, ckpts, None, loras, shp, batch, seq, parity, weight_source=pool.fetch)
    return {"Y": y, "dX": dx, "grads": grads, "copies": pool.copies}
