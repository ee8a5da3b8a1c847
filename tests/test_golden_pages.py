"""Pins of the stored NF4 format and of the library's per-layer blob sizes against the
sizes the pages print (tests/golden/page_sizes.txt, each figure with its source).

Bytes per weight are measured on what the oracle's encoder actually produces (packed
codes, float32 block absmax; with double quantisation the 8-bit codes, the per-group
float32 scales and the mean), not retyped from a formula, and scaled to the
Llama-3.1-8B parameter count.  A wrong block size, nibble packing or scale width moves
these sizes out of the pages' ranges."""
import os

import numpy as np
import pytest

from layer_streamed_qlora_amd import binding as B
from layer_streamed_qlora_amd import synth
from oracle import nf4

HERE = os.path.dirname(os.path.abspath(__file__))


def figures():
    ranges, groups = {}, {}
    for line in open(os.path.join(HERE, "golden", "page_sizes.txt")):
        line = line.split("#", 1)[0].strip() if line.lstrip().startswith("#") else line.strip()
        if not line:
            continue
        parts = [p.strip() for p in line.split("|")]
        if len(parts) == 2:
            groups[parts[0]] = parts[1].split()
        else:
            ranges[parts[0]] = (float(parts[1]), float(parts[2]))
    return ranges, groups


# Llama-3.1-8B: 32 decoder layers, hidden 4096, 32 query / 8 key-value heads of 128,
# SwiGLU 14336, vocabulary 128256 with separate input and output embeddings
LLAMA = synth.WORKLOADS["llama8b"]
VOCAB = 128256
LLAMA_PARAMS = (LLAMA.n_layers * (LLAMA.params_per_layer() + 2 * LLAMA.hidden)
                + 2 * VOCAB * LLAMA.hidden + LLAMA.hidden)

# the shapes of the pages' size classes (Qwen2.5 family from its published configs)
SHAPES = {
    "llama-3.1-8b": LLAMA,
    "qwen2.5-14b": synth.Workload("qwen14b", 0, 48, 5120, 40, 8, 128, 13824, "nf4", True, 16, 32.0, 1, 128),
    "qwen2.5-32b": synth.WORKLOADS["qwen32b"],
    "qwen2.5-72b": synth.WORKLOADS["qwen72b"],
}


@pytest.fixture(scope="module")
def encoded_bytes_per_weight():
    """(NF4 bytes per weight, NF4 + double-quantisation bytes per weight) measured on
    the oracle's encoding of 1 M weights (whole blocks and whole absmax groups).  The
    second level's one float32 mean per tensor is left out here (4 bytes per tensor)."""
    n = nf4.NF4_BLOCK * nf4.DQ_GROUP * 64
    w = nf4.bf16_round(np.random.default_rng(0).standard_normal(n).astype(np.float32) * 0.02)
    codes, absmax = nf4.quantize_nf4(w)
    packed = nf4.pack_nibbles(codes)
    q, scale, mean = nf4.double_quantize(absmax)
    plain = packed.nbytes + np.asarray(absmax, np.float32).nbytes
    assert np.asarray(mean, np.float32).size == 1
    dq = packed.nbytes + q.nbytes + np.asarray(scale, np.float32).nbytes
    return plain / n, dq / n


def test_llama_parameter_count_is_8b():
    assert 8.0e9 < LLAMA_PARAMS < 8.1e9


def test_full_and_half_precision_sizes():
    r, _ = figures()
    lo, hi = r["fp32_8b"]
    assert lo < LLAMA_PARAMS * 4 / 1e9 < hi
    lo, hi = r["half_8b"]
    assert lo < LLAMA_PARAMS * 2 / 1e9 < hi


def test_nf4_size_double_quant_saving_and_ratio(encoded_bytes_per_weight):
    r, _ = figures()
    plain, dq = encoded_bytes_per_weight
    nf4_gb, dq_gb = LLAMA_PARAMS * plain / 1e9, LLAMA_PARAMS * dq / 1e9
    lo, hi = r["nf4_8b"]
    assert lo < nf4_gb < hi and lo < dq_gb < hi, (nf4_gb, dq_gb)
    lo, hi = r["dq_saving_8b"]
    assert lo < nf4_gb - dq_gb < hi, nf4_gb - dq_gb
    lo, hi = r["half_over_nf4"]
    assert lo < 2.0 / plain < hi and lo < 2.0 / dq < hi, (2.0 / plain, 2.0 / dq)


def test_layer_blobs_fall_on_the_pages_side_of_the_threshold(encoded_bytes_per_weight):
    """The library's planned blob per layer (NF4 + double quantisation) and the oracle's
    encoded bytes per layer put 8B and 14B below the pages' ~165 MB threshold and 32B
    and 72B above it."""
    r, g = figures()
    lo, hi = r["nf4_bug_layer"]
    _, dq = encoded_bytes_per_weight
    for side, names in (("below", g["below_threshold"]), ("above", g["above_threshold"])):
        for name in names:
            w = SHAPES[name]
            _, _, blob = B.ls_plan_bytes(B.make_config(w, n_layers=1))
            oracle_mb = w.params_per_layer() * dq / 1e6
            if side == "below":
                assert blob / 1e6 < lo and oracle_mb < lo, (name, blob, oracle_mb)
            else:
                assert blob / 1e6 > hi and oracle_mb > hi, (name, blob, oracle_mb)
            # the library's blob holds the oracle's encoded bytes of the seven
            # projections (with one float32 mean each), the two bf16 norm weights and
            # alignment padding
            assert 0 <= blob - (w.params_per_layer() * dq + 7 * 4 + 4 * w.hidden) < 64 * 1024, (name, blob)
