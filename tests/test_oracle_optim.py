"""Pins of the oracle's AdamW update and adapter-file checker against facts that do
not come from them: a library implementation of the same published update, closed
forms, the CRC-32 check value, an independent reader of the container, and planted
corruptions."""
import json
import math
import struct

import numpy as np
import pytest
import torch

from oracle import adapters, optim


HPS = [optim.AdamW(), optim.AdamW(lr=3e-4, beta1=0.0, beta2=0.95, eps=1e-6, weight_decay=0.0),
       optim.AdamW(lr=2e-2, beta1=0.5, beta2=0.9, eps=1e-3, weight_decay=0.3)]


@pytest.mark.parametrize("hp", HPS)
def test_adamw_matches_torch_adamw_float64(hp):
    """torch.optim.AdamW is the same decoupled-decay update (lr-scaled decay); in float64
    on the CPU the two agree to rounding over several steps with changing gradients."""
    rng = np.random.default_rng(3)
    theta0 = rng.standard_normal((5, 7))
    grads = [rng.standard_normal((5, 7)) * 10.0 ** rng.uniform(-4, 1) for _ in range(6)]
    p = torch.tensor(theta0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([p], lr=hp.lr, betas=(hp.beta1, hp.beta2), eps=hp.eps, weight_decay=hp.weight_decay,
                            foreach=False)
    th, m, v = theta0, np.zeros_like(theta0), np.zeros_like(theta0)
    for t, g in enumerate(grads, start=1):
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        th, m, v = optim.adamw_step(th, g, m, v, t, hp)
        st = opt.state[p]
        np.testing.assert_allclose(th, p.detach().numpy(), rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-13, atol=1e-300)
        np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-13, atol=1e-300)


def test_first_step_closed_form():
    hp = optim.AdamW(lr=1e-2, weight_decay=0.05, eps=1e-6)
    rng = np.random.default_rng(4)
    th, g = rng.standard_normal(50), rng.standard_normal(50) * 1e-3
    got, m, v = optim.adamw_step(th, g, np.zeros(50), np.zeros(50), 1, hp)
    want = th * (1 - hp.lr * hp.weight_decay) - hp.lr * g / (np.abs(g) + hp.eps)
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(m, (1 - hp.beta1) * g, rtol=1e-15)
    np.testing.assert_allclose(v, (1 - hp.beta2) * g * g, rtol=1e-15)


def test_constant_gradient_moves_by_lr_every_step():
    """Same g every step: bias correction makes every move lr g / (|g| + eps), so after
    t steps (no decay) theta = theta0 - t lr g / (|g| + eps).  A missing bias correction
    or a wrong power of beta breaks this."""
    hp = optim.AdamW(lr=1e-3, weight_decay=0.0)
    g = np.array([2.0, -0.5, 1e-3, -7.0])
    th, m, v = np.zeros(4), np.zeros(4), np.zeros(4)
    for t in range(1, 21):
        th, m, v = optim.adamw_step(th, g, m, v, t, hp)
    np.testing.assert_allclose(th, -20 * hp.lr * g / (np.abs(g) + hp.eps), rtol=1e-12)


def test_zero_gradient_is_pure_decay():
    hp = optim.AdamW(lr=0.1, weight_decay=0.2)
    th0 = np.array([1.0, -3.0, 0.25])
    th, m, v = th0, np.zeros(3), np.zeros(3)
    for t in range(1, 6):
        th, m, v = optim.adamw_step(th, np.zeros(3), m, v, t, hp)
    np.testing.assert_allclose(th, th0 * (1 - 0.02) ** 5, rtol=1e-15)
    assert not m.any() and not v.any()


def test_step_count_starts_at_one():
    with pytest.raises(ValueError):
        optim.adamw_step(np.zeros(1), np.zeros(1), np.zeros(1), np.zeros(1), 0, optim.AdamW())


# ----------------------------------------------------------------- adapter files
DIMS = [(32, 32), (16, 32), (16, 32), (32, 32), (48, 32), (48, 32), (32, 48)]   # (out, in) per projection


def _tensors(n_layers=2, mask=0x7F, r=4, seed=0):
    rng = np.random.default_rng(seed)
    return {k: rng.standard_normal(s).astype(np.float32) for k, s in adapters.expected(n_layers, mask, r, DIMS).items()}


def test_crc32_check_value():
    """CRC-32 (ISO-HDLC) of the ASCII digits 1..9 is 0xCBF43926 (the catalogued check value)."""
    assert adapters.crc32_hex(np.frombuffer(b"123456789", np.uint8)) == "cbf43926"


def test_peft_names():
    assert adapters.peft_key(0, 0, "A") == "base_model.model.model.layers.0.self_attn.q_proj.lora_A.weight"
    assert adapters.peft_key(31, 6, "B") == "base_model.model.model.layers.31.mlp.down_proj.lora_B.weight"
    assert len(adapters.expected(3, 0b1000101, 8, DIMS)) == 3 * 3 * 2


def test_written_file_is_valid_and_reads_back(tmp_path):
    t = _tensors()
    f = str(tmp_path / "a.safetensors")
    adapters.write(f, t, 2, 4, 8.0, 0x7F)
    assert adapters.check(f, 2, 0x7F, 4, DIMS) == []
    got = adapters.load(f)                       # the safetensors package
    header, data = adapters.read_raw(f)          # the published layout, by hand
    for k, a in t.items():
        assert got[k].tobytes() == a.tobytes()
        b, e = header[k]["data_offsets"]
        assert data[b:e] == a.tobytes()


def _rewrite(f, edit_header=None, edit_data=None):
    header, data = adapters.read_raw(f)
    if edit_header:
        edit_header(header)
    data = bytearray(data)
    if edit_data:
        edit_data(header, data)
    hb = json.dumps(header).encode()
    hb += b" " * (-len(hb) % 8)
    with open(f, "wb") as fh:
        fh.write(struct.pack("<Q", len(hb)) + hb + bytes(data))


def test_checker_catches_planted_corruptions(tmp_path):
    t = _tensors()
    k0 = adapters.peft_key(1, 4, "A")

    def fresh(name):
        f = str(tmp_path / name)
        adapters.write(f, t, 2, 4, 8.0, 0x7F)
        return f

    # the no-op failure mode: keys renamed so that a loader keyed on the expected names finds nothing
    f = fresh("renamed.safetensors")
    _rewrite(f, lambda h: h.update({k.replace("base_model.model.", ""): h.pop(k)
                                    for k in [k for k in h if k != "__metadata__"]}))
    probs = adapters.check(f, 2, 0x7F, 4, DIMS)
    assert any(p.startswith("missing") for p in probs) and any(p.startswith("unexpected") for p in probs)
    # one flipped bit in one tensor's data
    f = fresh("flip.safetensors")
    _rewrite(f, edit_data=lambda h, d: d.__setitem__(h[k0]["data_offsets"][0] + 5, d[h[k0]["data_offsets"][0] + 5] ^ 1))
    assert adapters.check(f, 2, 0x7F, 4, DIMS) == [f"crc mismatch for {k0}"]
    # a dropped tensor, a wrong shape, a wrong rank in the metadata
    f = fresh("drop.safetensors")
    _rewrite(f, lambda h: h.pop(k0))
    assert f"missing {k0}" in adapters.check(f, 2, 0x7F, 4, DIMS)
    f = fresh("shape.safetensors")
    _rewrite(f, lambda h: h[k0].update(shape=[32, 4]))
    assert f"bad dtype/shape for {k0}" in adapters.check(f, 2, 0x7F, 4, DIMS)
    f = fresh("rank.safetensors")
    _rewrite(f, lambda h: h["__metadata__"].update({"lsq.r": "8"}))
    assert any("lsq.r" in p for p in adapters.check(f, 2, 0x7F, 4, DIMS))
    # a stack with a different mask or depth rejects the file
    f = fresh("ok.safetensors")
    assert adapters.check(f, 3, 0x7F, 4, DIMS) and adapters.check(f, 2, 0x3F, 4, DIMS)
