"""Write the oracle's results for the whole Llama-3.1-8B-shaped stack (32 layers,
NF4 + double quantisation, LoRA r 16 / alpha 32 on all seven projections) at batch 1 x
seq 128, for the full-depth GPU parity test.  Calls only ``oracle/`` (and the seeded
input generators of ``synth``); nothing here comes from the HIP path.

The stack computed is the plain composition of the decoder layer over 32 layers with a
recompute backward, parity mode (bf16 operands); streaming changes where the weights
come from, not the arithmetic ("Soup: Fine-Tuning an 8B Model on a 4 GB Laptop GPU,
One Layer at a Time", second paragraph).

Stored (float32 values of the float64 results, plus float64 norms):
  Y, dX       rows ROWS of the [128, 4096] outputs, and each tensor's full norm;
  dA, dB      for every (layer, projection), the values at N_SAMPLE flat indices drawn
              by ``sample_indices`` (seeded), and each tensor's full norm.

A second pass runs the same oracle functions, with the same bf16 rounding points, on
float32 arrays: every product then accumulates in float32, as on the GPU.  Its samples
are stored under the same keys with the suffix ``_f32``.  Their distance from the
float64 results is the floor any float32-accumulating implementation sits at: a
difference far below one bf16 unit before a rounding point flips some roundings, and
the stack carries those flips through every later layer.

Run: python tests/golden/make_llama8b_depth32.py   (about 15 minutes on 8 cores)
"""
from __future__ import annotations

import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from layer_streamed_qlora_amd import synth  # noqa: E402
from oracle import model as omodel  # noqa: E402
from oracle import nf4 as onf4  # noqa: E402
from oracle import stack as ostack  # noqa: E402

OUT = os.path.join(HERE, "llama8b_depth32_1x128.npz")
BATCH, SEQ = 1, 128
ROWS = np.array([0, 1, 2, 3, 7, 8, 17, 31, 32, 63, 64, 90, 100, 125, 126, 127])
N_SAMPLE = 512


def workload():
    return synth.WORKLOADS["llama8b"].with_(batch=BATCH, seq=SEQ)


def sample_indices(layer: int, proj: int, numel: int) -> np.ndarray:
    """The flat indices of the stored gradient entries of (layer, proj): the first and
    last element, then distinct seeded draws, sorted."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([77, layer, proj])))
    idx = np.unique(np.concatenate([[0, numel - 1], g.choice(numel, N_SAMPLE - 2, replace=False)]))
    while idx.size < N_SAMPLE:
        idx = np.unique(np.concatenate([idx, g.choice(numel, N_SAMPLE - idx.size, replace=False)]))
    return idx


def main():
    w = workload()
    shp = omodel.LayerShape(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.intermediate, w.rms_eps, w.rope_theta,
                            w.lora_r, w.lora_alpha)
    x, dy = synth.activations(w)
    loras = [synth.layer_lora(w, l) for l in range(w.n_layers)]
    enc = {}
    t0 = time.time()

    def encoded(l):
        if l not in enc:
            src = synth.layer_weights(w, l)
            with ThreadPoolExecutor(max_workers=7) as ex:
                enc[l] = ostack.quantize_layer(src, w.quant, w.double_quant, map_fn=ex.map)
        return enc[l]

    def weights(l):
        with ThreadPoolExecutor(max_workers=7) as ex:
            d = ostack.dequant_layer(encoded(l), map_fn=ex.map)
        print(f"layer {l} ready ({time.time() - t0:.0f} s)", flush=True)
        return d

    y, ckpts = ostack.stack_forward(x, None, loras, shp, BATCH, SEQ, True, True, weight_source=weights)
    dx, grads = ostack.stack_backward(dy, ckpts, None, loras, shp, BATCH, SEQ, True, weight_source=weights)
    rec = {"rows": ROWS}

    def store(suffix, y, dx, grads, norms):
        rec["Y_rows" + suffix] = np.asarray(y)[ROWS].astype(np.float32)
        rec["dX_rows" + suffix] = np.asarray(dx)[ROWS].astype(np.float32)
        if norms:
            rec["Y_norm"] = np.float64(np.linalg.norm(y))
            rec["dX_norm"] = np.float64(np.linalg.norm(dx))
        for l in range(w.n_layers):
            for pi, p in enumerate(synth.PROJS):
                for which, g in (("dA", grads[l][p][0]), ("dB", grads[l][p][1])):
                    flat = np.asarray(g, np.float64).reshape(-1)
                    idx = sample_indices(l, 2 * pi + (which == "dB"), flat.size)
                    rec[f"{which}_{l}_{p}{suffix}"] = flat[idx].astype(np.float32)
                    if norms:
                        rec[f"{which}_{l}_{p}_norm"] = np.float64(np.linalg.norm(flat))

    store("", y, dx, grads, True)
    del ckpts, grads
    # the float32-accumulation pass: same functions, same rounding points, float32 arrays
    f32 = np.float32
    rnd32 = lambda a: onf4.bf16_round(a).astype(f32)

    def weights32(l):
        return {k: v.astype(f32) for k, v in weights(l).items()}

    lo32 = [{p: (a.astype(f32), b.astype(f32)) for p, (a, b) in lo.items()} for lo in loras]
    h = rnd32(x)
    ck32 = []
    for l in range(w.n_layers):
        ck32.append(h)
        yl, _ = omodel.layer_forward(h, weights32(l), lo32[l], shp, BATCH, SEQ, True, rnd32)
        h = rnd32(yl)
    y32, g = h, rnd32(dy)
    grads32 = [None] * w.n_layers
    for l in reversed(range(w.n_layers)):
        wl = weights32(l)
        _, cache = omodel.layer_forward(ck32[l], wl, lo32[l], shp, BATCH, SEQ, True, rnd32)
        dxl, grads32[l] = omodel.layer_backward(g, cache, wl, lo32[l], shp, BATCH, SEQ, rnd32)
        g = rnd32(dxl)
    store("_f32", y32, g, grads32, False)
    np.savez(OUT, **rec)
    print(f"wrote {OUT} ({os.path.getsize(OUT)} bytes) in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main()
