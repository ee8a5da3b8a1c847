"""Pins of the oracle's layer math and stack against facts that do not come from it:
library routines on special cases, closed forms, invariants, brute force on tiny
inputs, finite differences, and the identities the pages state."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import model, nf4, stack
from layer_streamed_qlora_amd import synth

TINY = synth.Workload("tiny", 9, 2, 32, 2, 1, 16, 48, "nf4", False, 4, 8.0, 2, 6)


def tiny_shape(w=TINY):
    return model.LayerShape(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.intermediate,
                            w.rms_eps, w.rope_theta, w.lora_r, w.lora_alpha)


def tiny_weights(w=TINY, seed=0, exact=True):
    """float64 weights (random, not quantised) and adapters for the tiny stack."""
    rng = np.random.default_rng(seed)
    layers, loras = [], []
    for _ in range(w.n_layers):
        lw = {p: rng.standard_normal(w.proj_shape(p)) * 0.2 for p in model.PROJS}
        lw["g1"] = 1.0 + 0.1 * rng.standard_normal(w.hidden)
        lw["g2"] = 1.0 + 0.1 * rng.standard_normal(w.hidden)
        lo = {}
        for p in model.PROJS:
            o, i = w.proj_shape(p)
            lo[p] = (rng.standard_normal((w.lora_r, i)) * 0.3, rng.standard_normal((o, w.lora_r)) * 0.3)
        layers.append(lw)
        loras.append(lo)
    return layers, loras


# -------------------------------------------------------------- component pins
def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 33))
    g = rng.standard_normal(33)
    got, _ = model.rmsnorm_fwd(x, g, 1e-5)
    want = F.rms_norm(torch.from_numpy(x), (33,), torch.from_numpy(g), eps=1e-5).numpy()
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_attention_matches_torch_sdpa_gqa():
    rng = np.random.default_rng(1)
    b, s, hq, hkv, hd = 2, 9, 4, 2, 8
    q = rng.standard_normal((b, s, hq, hd))
    k = rng.standard_normal((b, s, hkv, hd))
    v = rng.standard_normal((b, s, hkv, hd))
    got, _ = model.attention_fwd(q, k, v, hq // hkv)
    tq = torch.from_numpy(q).transpose(1, 2)
    tk = torch.from_numpy(np.repeat(k, 2, axis=2)).transpose(1, 2)
    tv = torch.from_numpy(np.repeat(v, 2, axis=2)).transpose(1, 2)
    want = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True).transpose(1, 2).numpy()
    assert np.allclose(got, want, rtol=1e-10, atol=1e-12)


def test_attention_brute_force_loops():
    rng = np.random.default_rng(2)
    b, s, hq, hkv, hd = 1, 5, 2, 1, 3
    q, k, v = (rng.standard_normal((b, s, h, hd)) for h in (hq, hkv, hkv))
    got, _ = model.attention_fwd(q, k, v, 2)
    for h in range(hq):
        for i in range(s):
            sc = [sum(q[0, i, h, d] * k[0, j, 0, d] for d in range(hd)) / math.sqrt(hd) for j in range(i + 1)]
            m = max(sc)
            e = [math.exp(x - m) for x in sc]
            z = sum(e)
            for d in range(hd):
                want = sum(e[j] / z * v[0, j, 0, d] for j in range(i + 1))
                assert abs(got[0, i, h, d] - want) < 1e-12


def test_attention_first_token_is_its_value():
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((1, 4, 2, 8)) for _ in range(3))
    out, _ = model.attention_fwd(q, k, v, 1)
    assert np.allclose(out[0, 0], v[0, 0], rtol=0, atol=1e-15)


def test_rope_closed_forms():
    # head_dim 2: pair (x1, x2) at position p rotates by angle p (inv_freq = 1)
    cos, sin = model.rope_tables(3, 2, 1e4)
    x = np.zeros((1, 3, 1, 2))
    x[..., 0] = 1.0
    y = model.rope_fwd(x, cos, sin)
    for p in range(3):
        assert np.allclose(y[0, p, 0], [math.cos(p), math.sin(p)], atol=1e-15)
    # frequencies theta^(-2i/hd)
    cos, sin = model.rope_tables(2, 8, 1e4)
    ang = np.arccos(np.clip(cos[1], -1, 1))
    assert np.allclose(ang, [1.0, 1e4 ** (-0.25), 1e4 ** (-0.5), 1e4 ** (-0.75)], rtol=1e-12)


def test_rope_relative_position_invariant():
    rng = np.random.default_rng(4)
    hd = 16
    cos, sin = model.rope_tables(40, hd, 1e4)
    q = rng.standard_normal(hd)
    k = rng.standard_normal(hd)
    big = np.zeros((1, 40, 1, hd))
    big[0, :, 0] = q
    rq = model.rope_fwd(big, cos, sin)[0, :, 0]
    big[0, :, 0] = k
    rk = model.rope_fwd(big, cos, sin)[0, :, 0]
    d1 = rq[10] @ rk[7]
    d2 = rq[33] @ rk[30]
    assert abs(d1 - d2) < 1e-10
    assert np.allclose(np.linalg.norm(rq, axis=1), np.linalg.norm(q))


def test_silu_matches_torch():
    z = np.linspace(-20, 20, 1001)
    assert np.allclose(model.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-14, atol=1e-300)


def test_lora_only_projection_textbook():
    """P6: with W = 0, Y = s X A^T B^T, checked with explicit loops."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 5))
    a = rng.standard_normal((2, 5))
    b = rng.standard_normal((4, 2))
    y, _ = model.lora_proj_fwd(x, np.zeros((4, 5)), a, b, 1.5)
    for m in range(3):
        for n in range(4):
            want = 1.5 * sum(b[n, r] * sum(x[m, k] * a[r, k] for k in range(5)) for r in range(2))
            assert abs(y[m, n] - want) < 1e-12


# ------------------------------------------------------ finite differences (P4)
def _loss(w, layers, loras, x, dy):
    shp = tiny_shape(w)
    y, _ = stack.stack_forward(x, layers, loras, shp, w.batch, w.seq, True, parity=False)
    return float(np.sum(y * dy))


@pytest.mark.parametrize("what", ["X", "A", "B"])
def test_finite_differences(what):
    w = TINY
    layers, loras = tiny_weights(w)
    rng = np.random.default_rng(7)
    x = rng.standard_normal((w.tokens, w.hidden))
    dy = rng.standard_normal((w.tokens, w.hidden))
    shp = tiny_shape(w)
    _, ck = stack.stack_forward(x, layers, loras, shp, w.batch, w.seq, True, parity=False)
    dx, grads = stack.stack_backward(dy, ck, layers, loras, shp, w.batch, w.seq, parity=False)
    eps = 1e-6
    targets = []
    if what == "X":
        targets.append((x, dx))
    else:
        j = 0 if what == "A" else 1
        for l in range(w.n_layers):
            for p in model.PROJS:
                targets.append((loras[l][p][j], grads[l][p][j]))
    worst = 0.0
    for arr, g in targets:
        flat = arr.reshape(-1)
        gflat = g.reshape(-1)
        idx = np.arange(flat.size) if flat.size <= 64 else np.random.default_rng(8).choice(flat.size, 64, replace=False)
        for i in idx:
            keep = flat[i]
            flat[i] = keep + eps
            lp = _loss(w, layers, loras, x, dy)
            flat[i] = keep - eps
            lm = _loss(w, layers, loras, x, dy)
            flat[i] = keep
            fd = (lp - lm) / (2 * eps)
            worst = max(worst, abs(fd - gflat[i]) / max(1.0, abs(gflat[i])))
    assert worst < 1e-6, worst


# --------------------------------------------------------------- identities
def _toy_encoded(w):
    return [stack.quantize_layer(synth.layer_weights(w, l), w.quant, w.double_quant) for l in range(w.n_layers)]


def _shape_of(w):
    return model.LayerShape(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.intermediate,
                            w.rms_eps, w.rope_theta, w.lora_r, w.lora_alpha)


def test_b_zero_is_base_only_and_lora_off_is_reference():
    """P2/P3: B = 0 gives the base-only output bitwise and dA = 0 exactly; the
    adapters-off reference pass equals the B = 0 policy pass bitwise."""
    w = synth.WORKLOADS["toy"].with_(seq=32)
    enc = _toy_encoded(w)
    lw = [stack.dequant_layer(e) for e in enc]
    loras = [synth.layer_lora(w, l) for l in range(w.n_layers)]
    zero_b = [{p: (a, np.zeros_like(b)) for p, (a, b) in lo.items()} for lo in loras]
    x, dy = synth.activations(w)
    shp = _shape_of(w)
    out0 = stack.train_step(x, dy, lw, zero_b, shp, w.batch, w.seq, with_reference=True)
    ref_on, _ = stack.stack_forward(x, lw, loras, shp, w.batch, w.seq, lora_on=False)
    assert np.array_equal(out0["Y"], out0["Y_ref"])
    assert np.array_equal(out0["Y"], ref_on)
    for g in out0["grads"]:
        for p in model.PROJS:
            assert np.all(g[p][0] == 0)
    # and LoRA does change things when B != 0
    out1 = stack.train_step(x, dy, lw, loras, shp, w.batch, w.seq)
    assert not np.array_equal(out1["Y"], out0["Y"])


@pytest.mark.parametrize("n_layers,dq", [(2, False), (5, True)])
def test_simulated_streaming_equals_resident(n_layers, dq):
    """P5: pulling every layer through a two-slot pool (poisoned on release), twice per
    step, gives bitwise the resident result."""
    w = synth.WORKLOADS["toy"].with_(seq=16, n_layers=n_layers, double_quant=dq)
    enc = _toy_encoded(w)
    lw = [stack.dequant_layer(e) for e in enc]
    loras = [synth.layer_lora(w, l) for l in range(w.n_layers)]
    x, dy = synth.activations(w)
    shp = _shape_of(w)
    res = stack.train_step(x, dy, lw, loras, shp, w.batch, w.seq)
    store = stack.HostStore(enc)
    st = stack.streamed_train_step(x, dy, store, loras, shp, w.batch, w.seq)
    assert st["copies"] == 2 * n_layers
    assert np.array_equal(res["Y"], st["Y"]) and np.array_equal(res["dX"], st["dX"])
    for l in range(n_layers):
        for p in model.PROJS:
            for j in range(2):
                assert np.array_equal(res["grads"][l][p][j], st["grads"][l][p][j])


def test_poisoned_slot_would_be_seen():
    """The pool's poison is visible if a layer were read after release."""
    w = synth.WORKLOADS["toy"].with_(seq=16)
    store = stack.HostStore(_toy_encoded(w))
    pool = stack.TwoSlotPool(store)
    pool.fetch(0)
    dec = store.decode(pool.slots[0])
    assert np.isnan(dec["q"]).all() or not np.isfinite(dec["q"]).all()


def test_parity_mode_rounds_layer_outputs():
    w = synth.WORKLOADS["toy"].with_(seq=16)
    lw = [stack.dequant_layer(e) for e in _toy_encoded(w)]
    loras = [synth.layer_lora(w, l) for l in range(w.n_layers)]
    x, dy = synth.activations(w)
    shp = _shape_of(w)
    y, ck = stack.stack_forward(x, lw, loras, shp, w.batch, w.seq)
    for t in [y] + ck:
        assert np.array_equal(nf4.bf16_round(t).astype(np.float64), t)
    ye, _ = stack.stack_forward(x, lw, loras, shp, w.batch, w.seq, parity=False)
    rel = np.linalg.norm(ye - y) / np.linalg.norm(ye)
    assert 0 < rel < 1e-2
