"""The library's host NF4 packer against the oracle's encoder, byte for byte, on whole
tensors of the measured shapes (CPU only).

Packing is one of the two results the GPU path must reproduce exactly (with the
dequantised weights).  The encoding is the NF4 block quantisation with double
quantisation of the absmax values ("Fine-Tuning an 8B Parameter Model on a 4 GB Laptop
GPU", section "Quantization: Shrink the Weights"); the large case is the 251.5 MB
Qwen2.5-32B-shaped layer, above the ~165 MB per layer where the pages report streamed
NF4 runs going wrong ("Soup: Fine-Tuning an 8B Model on a 4 GB Laptop GPU, One Layer at
a Time", third paragraph).  Compared: codes, first-level absmax, 8-bit codes, group
scales and the tensor mean, all as raw bits.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from layer_streamed_qlora_amd import binding as B
from layer_streamed_qlora_amd import synth
from oracle import nf4

pytestmark = pytest.mark.slow


def compare_tensor(values32, dq):
    bits = synth.bf16_bits(values32)
    packed, am, qabs, s2, mean = B.ls_pack_nf4(bits, dq)
    t = nf4.NF4Tensor(values32, dq)
    assert np.array_equal(packed, t.packed)
    assert np.array_equal(am.view(np.uint32), t.absmax.view(np.uint32))
    if dq:
        assert np.array_equal(qabs, t.qabs)
        assert np.array_equal(s2.view(np.uint32), t.scale2.view(np.uint32))
        assert np.float32(mean).view(np.uint32) == np.float32(t.mean).view(np.uint32)
    return values32.size


def run_layer(name, layer, projs):
    w = synth.WORKLOADS[name]
    src = synth.layer_weights(w, layer)
    with ThreadPoolExecutor(max_workers=4) as ex:
        sizes = list(ex.map(lambda p: compare_tensor(src[p], w.double_quant), projs))
    return sum(sizes)


def test_llama8b_whole_layer_double_quant():
    n = run_layer("llama8b", 0, synth.PROJS)
    assert n == synth.WORKLOADS["llama8b"].params_per_layer()


def test_qwen32b_mlp_tensors_of_the_251mb_layer():
    n = run_layer("qwen32b", 0, ("gate", "up", "down"))
    assert n == 3 * 27648 * 5120
