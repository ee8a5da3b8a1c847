"""CPU checks of the C-ABI library: it loads, exports every symbol include/ls.h
declares, its host encoder is bit-exact with the oracle, and the pre-flight checks
refuse bad configs and over-budget plans before touching the GPU."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from layer_streamed_qlora_amd import binding as B
from layer_streamed_qlora_amd import synth
from oracle import nf4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    txt = open(os.path.join(ROOT, "include", "ls.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(ls_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    syms = header_symbols()
    assert len(syms) >= 12
    for s in syms:
        assert hasattr(lib, s), s
    assert set(syms) == set(B.SIGNATURES), set(syms) ^ set(B.SIGNATURES)


def test_codebook_bitwise_equals_oracle():
    assert np.array_equal(B.ls_nf4_codebook().view(np.uint32), nf4.nf4_codebook().view(np.uint32))


def _oracle_encode(values32, dq):
    t = nf4.NF4Tensor(values32, dq)
    return t


@pytest.mark.parametrize("dq", [False, True])
@pytest.mark.parametrize("shape", [(256, 688), (688, 256), (3, 40), (1, 1000)])
def test_packer_bit_exact(dq, shape):
    rng = np.random.default_rng(sum(shape) + dq)
    x = nf4.bf16_round(rng.standard_normal(shape).astype(np.float32) * 0.02)
    x.reshape(-1)[:64] = 0.0                      # an all-zero block
    x.reshape(-1)[64] = -x.reshape(-1)[65]        # mixed signs of the same magnitude
    bits = synth.bf16_bits(x)
    packed, am, qabs, s2, mean = B.ls_pack_nf4(bits, dq)
    t = _oracle_encode(x, dq)
    assert np.array_equal(packed, t.packed)
    assert np.array_equal(am.view(np.uint32), t.absmax.view(np.uint32))
    if dq:
        assert np.array_equal(qabs, t.qabs)
        assert np.array_equal(s2.view(np.uint32), t.scale2.view(np.uint32))
        assert np.float32(mean).view(np.uint32) == np.float32(t.mean).view(np.uint32)


def test_packer_ties_and_level_multiples():
    """Values exactly at level multiples and at midpoints (ties go to the higher code)."""
    lv = nf4.nf4_codebook()
    am = np.float32(1.0)
    vals = []
    for i in range(15):
        vals += [lv[i], (np.float64(lv[i]) + np.float64(lv[i + 1])) / 2]
    vals.append(1.0)
    x = nf4.bf16_round(np.array(vals + [0.0] * (64 - len(vals)), np.float32) * am)
    packed, amx, *_ = B.ls_pack_nf4(synth.bf16_bits(x), False)
    t = _oracle_encode(x, False)
    assert np.array_equal(packed, t.packed) and amx[0] == t.absmax[0]


def test_packer_thread_count_does_not_matter():
    rng = np.random.default_rng(9)
    x = nf4.bf16_round(rng.standard_normal(300_000).astype(np.float32) * 0.02)
    bits = synth.bf16_bits(x)
    a = B.ls_pack_nf4(bits, True, n_threads=1)
    b = B.ls_pack_nf4(bits, True, n_threads=7)
    for u, v in zip(a, b):
        assert np.array_equal(np.asarray(u), np.asarray(v))


def test_plan_sizes():
    """Blob per layer: 4 bits per weight + block scales + norm weights, 256-B pieces."""
    for name, lo, hi in [("llama8b", 112.4e6, 112.7e6), ("qwen3b", 154.0e6, 154.3e6),
                         ("qwen32b", 251.4e6, 251.7e6), ("qwen72b", 452.6e6, 453.0e6)]:
        w = synth.WORKLOADS[name]
        dev, host, blob = B.ls_plan_bytes(B.make_config(w))
        assert lo < blob < hi, (name, blob)
        assert host == blob * w.n_layers
    # the >165 MB-per-layer case of the pages
    _, _, blob = B.ls_plan_bytes(B.make_config(synth.WORKLOADS["qwen32b"]))
    assert blob > 165e6


def test_budget_refusal_allocates_nothing():
    cfg = B.make_config(synth.WORKLOADS["toy"], vram_budget=1 << 20)
    h = C.c_void_p()
    st = B.lib().ls_create(C.byref(cfg), None, None, C.byref(h))
    assert st == B.LS_ERR_BUDGET and not h.value
    assert b"exceeds budget" in B.lib().ls_last_error(None)


@pytest.mark.parametrize("field,value", [("nf4_block", 32), ("lora_r", 0), ("n_buffers", 1), ("head_dim", 96),
                                         ("n_kv_heads", 3), ("hidden", 100), ("lora_mask", 0x80),
                                         ("max_seq", 0), ("double_quant", 2), ("copy_split", 2),
                                         ("profile_stride", -1)])
def test_invalid_config(field, value):
    cfg = B.make_config(synth.WORKLOADS["toy"], vram_budget=1 << 40)
    setattr(cfg, field, value)
    h = C.c_void_p()
    assert B.lib().ls_create(C.byref(cfg), None, None, C.byref(h)) == B.LS_ERR_INVALID
    assert not h.value


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        B.lib()


def test_plan_holds_streamed_head():
    """A 2000-row bf16 head on the toy stack: slices of as many whole 256-row groups as
    fit one layer slot, each stored as one more blob of the pinned store."""
    w = synth.WORKLOADS["toy"]
    d0, h0, blob = B.ls_plan_bytes(B.make_config(w))
    d1, h1, _ = B.ls_plan_bytes(B.make_config(w, vocab=2000))
    rows = blob // (2 * w.hidden) // 256 * 256
    slices = -(-2000 // rows)
    assert h0 == blob * w.n_layers and h1 == blob * (w.n_layers + slices)
    assert d1 - d0 >= 4 * w.tokens * rows + 2 * w.tokens * rows + 4 * w.tokens * w.hidden
    bad = B.make_config(w, vocab=-1)
    with pytest.raises(B.LsError):
        B.ls_plan_bytes(bad)


def test_file_store_plan_and_validation(tmp_path):
    """With the base in a file, pinned host memory is one 4096-aligned staging blob per
    slot instead of the whole store; a file store without a path is refused."""
    w = synth.WORKLOADS["toy"]
    _, h_ram, blob = B.ls_plan_bytes(B.make_config(w, n_buffers=3))
    _, h_file, _ = B.ls_plan_bytes(B.make_config(w, n_buffers=3, store_path=str(tmp_path / "s.bin")))
    assert h_ram == blob * w.n_layers
    assert h_file == -(-blob // 4096) * 4096 * 3
    bad = B.make_config(w)
    bad.store = B.LS_STORE_FILE
    with pytest.raises(B.LsError):
        B.ls_plan_bytes(bad)


def test_automatic_pool_depth_plan():
    """n_buffers = 0 plans the deepest pool that fits vram_budget: one slot per layer (at
    most 64) without a budget, the deepest fitting depth with one, and two slots (which
    ls_create then refuses) when even that does not fit."""
    w = synth.WORKLOADS["llama8b"]
    plan = lambda **kw: B.ls_plan_bytes(B.make_config(w, **kw))[0]
    assert plan(n_buffers=0) == plan(n_buffers=32)
    assert plan(n_buffers=0, vram_budget=plan(n_buffers=5)) == plan(n_buffers=5)
    assert plan(n_buffers=0, vram_budget=plan(n_buffers=5) - 1) == plan(n_buffers=4)
    assert plan(n_buffers=0, vram_budget=1 << 20) == plan(n_buffers=2)
    deep = synth.WORKLOADS["qwen72b"]
    assert B.ls_plan_bytes(B.make_config(deep, n_buffers=0))[0] == B.ls_plan_bytes(B.make_config(deep, n_buffers=64))[0]
    for bad in (1, 65):
        with pytest.raises(B.LsError):
            B.ls_plan_bytes(B.make_config(w, n_buffers=bad))
