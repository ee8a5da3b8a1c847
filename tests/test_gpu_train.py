"""GPU checks of the training-loop closure through the C ABI: the AdamW update of the
adapters against the oracle's AdamW, adapter files written and loaded by the library
against the oracle's reader and checker, and a short training loop whose every update
is the oracle's AdamW applied to the GPU's own gradients."""
import os

import numpy as np
import pytest

from layer_streamed_qlora_amd import binding as B
from layer_streamed_qlora_amd import synth
from oracle import adapters as oad
from oracle import optim as oopt
import lsq_harness as H

pytestmark = pytest.mark.gpu

TOY = synth.WORKLOADS["toy"]
PROJS = H.PROJS


def say(*a):
    print(*a, flush=True)


def dims(w):
    return [w.proj_shape(p) for p in PROJS]


def snapshot(run):
    """float32 copies of every registered A, B."""
    return [{p: (run.A[l][p].cpu().numpy().copy(), run.Bm[l][p].cpu().numpy().copy()) for p in PROJS}
            for l in range(len(run.layer_seeds))]


def fill_grads(run, rng, scale=1e-2, zero=()):
    torch = run.torch
    g = []
    for l in range(len(run.layer_seeds)):
        gl = {}
        for p in PROJS:
            ga = (rng.standard_normal(run.dA[l][p].shape) * scale).astype(np.float32)
            gb = (rng.standard_normal(run.dB[l][p].shape) * scale).astype(np.float32)
            if (l, p) in zero:
                ga[:] = 0
                gb[:] = 0
            run.dA[l][p].copy_(torch.from_numpy(ga))
            run.dB[l][p].copy_(torch.from_numpy(gb))
            gl[p] = (ga, gb)
        g.append(gl)
    torch.cuda.synchronize()
    return g


# fp32 update vs the float64 oracle: each step rounds p once (<= 1 ulp of p), and the
# step lr * m_hat / (sqrt(v_hat) + eps), whose size is at most ~lr, carries a relative
# error of a few float32 ulps from the moments and the arithmetic (bounded here by
# 1e-5), so after S steps |dp| <= (S + 2) ulp(|p|) + S * 1e-5 * lr
def assert_close_f32(got, want, steps, lr):
    want = np.asarray(want, np.float64)
    tol = (steps + 2) * np.spacing(np.abs(want).astype(np.float32)).astype(np.float64) + steps * 1e-5 * lr
    bad = np.abs(np.asarray(got, np.float64) - want) > tol
    assert not bad.any(), (int(bad.sum()), float(np.max(np.abs(got - want))))


@pytest.mark.parametrize("rank,hp", [
    (8, oopt.AdamW()),
    (64, oopt.AdamW(lr=2e-3, beta1=0.0, beta2=0.95, eps=1e-6, weight_decay=0.0)),
    (16, oopt.AdamW(lr=5e-3, beta1=0.8, beta2=0.99, eps=1e-4, weight_decay=0.1)),
])
def test_adamw_matches_oracle(rank, hp):
    """Several steps with changing gradients; rank 64 gives tensors of several 8192-element
    chunks with a ragged last chunk; one projection has all-zero gradients."""
    w = TOY.with_(lora_r=rank, lora_alpha=2.0 * rank)
    say("case: adamw rank", rank, hp)
    run = H.GpuRun(w, [0, 1], adamw=1)
    rng = np.random.default_rng(rank)
    state = {(l, p, k): (v.astype(np.float64), np.zeros(v.shape), np.zeros(v.shape))
             for l, d in enumerate(snapshot(run)) for p, ab in d.items() for k, v in zip("AB", ab)}
    S = 3
    for t in range(1, S + 1):
        g = fill_grads(run, rng, scale=10.0 ** rng.uniform(-4, -1), zero={(1, "o")})
        run.ctx.adamw_step(t, hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay)
        run.ctx.sync()
        for (l, p, k), (th, m, v) in state.items():
            gg = g[l][p][0 if k == "A" else 1].astype(np.float64)
            state[(l, p, k)] = oopt.adamw_step(th, gg, m, v, t, hp)
    got = snapshot(run)
    run.close()
    for (l, p, k), (th, _, _) in state.items():
        assert_close_f32(got[l][p][0 if k == "A" else 1], th, S, hp.lr)


def test_adamw_skips_unregistered_gradients_and_refuses_bad_input():
    w = TOY
    run = H.GpuRun(w, [0, 1], adamw=1)
    before = snapshot(run)
    # layer 0 / down: registered without gradient buffers, so it must not move
    run.ctx.set_lora(0, 6, run.A[0]["down"].data_ptr(), run.Bm[0]["down"].data_ptr(), 0, 0)
    fill_grads(run, np.random.default_rng(2))
    run.ctx.adamw_step(1, 1e-2)
    run.ctx.sync()
    after = snapshot(run)
    assert np.array_equal(after[0]["down"][0], before[0]["down"][0])
    assert np.array_equal(after[0]["down"][1], before[0]["down"][1])
    assert not np.array_equal(after[1]["down"][0], before[1]["down"][0])
    for kw in (dict(step=0, lr=1e-3), dict(step=1, lr=-1.0), dict(step=1, lr=1e-3, beta1=1.0),
               dict(step=1, lr=1e-3, eps=0.0), dict(step=1, lr=float("nan"))):
        with pytest.raises(B.LsError) as e:
            run.ctx.adamw_step(**kw)
        assert e.value.status == B.LS_ERR_INVALID
    run.close()
    run = H.GpuRun(w, [0], adamw=0)
    with pytest.raises(B.LsError) as e:
        run.ctx.adamw_step(1, 1e-3)
    assert e.value.status == B.LS_ERR_STATE
    run.close()


def test_adamw_unaligned_view_and_reset():
    """A registration at a 4-byte offset takes the scalar path; after a reset the moments
    are zero again, so the first step repeats exactly."""
    torch = pytest.importorskip("torch")
    w = TOY
    run = H.GpuRun(w, [0], adamw=1, lora_mask=1 << 3)   # only o
    n_out, n_in = w.proj_shape("o")
    big = torch.zeros(w.lora_r * n_in + 1, device="cuda:0")
    big[1:] = run.A[0]["o"].reshape(-1)
    A = big[1:].view(w.lora_r, n_in)
    dA = torch.full_like(A, 1e-3)
    run.dB[0]["o"].fill_(-2e-3)
    run.ctx.set_lora(0, 3, A.data_ptr(), run.Bm[0]["o"].data_ptr(), dA.data_ptr(), run.dB[0]["o"].data_ptr())
    a0, b0 = A.cpu().numpy().copy(), run.Bm[0]["o"].cpu().numpy().copy()
    hp = oopt.AdamW(lr=1e-2, weight_decay=0.0)
    run.ctx.adamw_step(1, hp.lr, weight_decay=0.0)
    run.ctx.sync()
    a1 = A.cpu().numpy().copy()
    want = oopt.first_step_closed_form(a0, np.full_like(a0, 1e-3), hp)
    assert_close_f32(a1, want, 1, hp.lr)
    # reset, restore the parameters, step again: bitwise the same as the first step
    run.ctx.adamw_reset()
    A.copy_(torch.from_numpy(a0))
    run.Bm[0]["o"].copy_(torch.from_numpy(b0))
    run.ctx.adamw_step(1, hp.lr, weight_decay=0.0)
    run.ctx.sync()
    assert np.array_equal(A.cpu().numpy(), a1)
    run.close()


def test_save_load_roundtrip_and_refusal(tmp_path):
    w = TOY
    x, dy = synth.activations(w)
    run = H.GpuRun(w, [0, 1])
    y0 = run.step(x, dy, w.batch, w.seq, backward=False)["Y"]
    snap = snapshot(run)
    f = str(tmp_path / "adapters.safetensors")
    run.ctx.save_adapters(f)
    # the oracle's checker accepts the file and its reader sees the device values bitwise
    assert oad.check(f, 2, 0x7F, w.lora_r, dims(w)) == []
    tensors = oad.load(f)
    assert len(tensors) == 2 * 7 * 2
    for l in range(2):
        for pi, p in enumerate(PROJS):
            assert tensors[oad.peft_key(l, pi, "A")].tobytes() == snap[l][p][0].tobytes()
            assert tensors[oad.peft_key(l, pi, "B")].tobytes() == snap[l][p][1].tobytes()
    # wipe the adapters, load: restored bitwise, and the forward is the same again
    for l in range(2):
        for p in PROJS:
            run.A[l][p].zero_()
            run.Bm[l][p].zero_()
    run.ctx.load_adapters(f)
    assert all(np.array_equal(a, b) for s0, s1 in zip(snap, snapshot(run)) for p in PROJS
               for a, b in zip(s0[p], s1[p]))
    y1 = run.step(x, dy, w.batch, w.seq, backward=False)["Y"]
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
    # a file whose names were changed (the silent no-op failure) is refused and nothing changes
    header, data = oad.read_raw(f)
    bad = str(tmp_path / "renamed.safetensors")
    oad.write(bad, {k.replace("self_attn", "attn"): tensors[k] for k in tensors}, 2, w.lora_r, w.lora_alpha, 0x7F)
    for l in range(2):
        for p in PROJS:
            run.A[l][p].mul_(2.0)
    doubled = snapshot(run)
    with pytest.raises(B.LsError) as e:
        run.ctx.load_adapters(bad)
    assert e.value.status == B.LS_ERR_INVALID and "tensor" in str(e.value)
    assert all(np.array_equal(a, b) for s0, s1 in zip(doubled, snapshot(run)) for p in PROJS
               for a, b in zip(s0[p], s1[p]))
    run.close()


def test_training_loop_each_update_is_adamw_of_own_gradients():
    """forward -> loss 0.5 |Y - target|^2 -> backward -> AdamW, five steps: the loss falls,
    and every step's new adapters equal the oracle's AdamW applied to the adapters and
    gradients the GPU held before that step."""
    torch = pytest.importorskip("torch")
    w = TOY
    run = H.GpuRun(w, [0, 1], adamw=1)
    x, _ = synth.activations(w)
    rng = np.random.default_rng(11)
    target = (rng.standard_normal((w.tokens, w.hidden)) * 0.5).astype(np.float32)
    hp = oopt.AdamW(lr=3e-3)
    state = None
    losses = []
    for t in range(1, 6):
        y = run.step(x, np.zeros_like(x), w.batch, w.seq, backward=False)["Y"]
        diff = (y.astype(np.float64) - target)
        losses.append(0.5 * float(np.sum(diff * diff)) / w.tokens)
        out = run.step(x, (diff / w.tokens).astype(np.float32), w.batch, w.seq)
        before = snapshot(run)
        if state is None:
            state = {(l, p, k): (np.zeros(v.shape), np.zeros(v.shape))
                     for l, d in enumerate(before) for p, ab in d.items() for k, v in zip("AB", ab)}
        run.ctx.adamw_step(t, hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay)
        run.ctx.sync()
        after = snapshot(run)
        for (l, p, k), (m, v) in list(state.items()):
            i = 0 if k == "A" else 1
            g = (out["dA"] if k == "A" else out["dB"])[l][p].astype(np.float64)
            th, m, v = oopt.adamw_step(before[l][p][i].astype(np.float64), g, m, v, t, hp)
            state[(l, p, k)] = (m, v)
            assert_close_f32(after[l][p][i], th, 1, hp.lr)
    say("losses", [f"{v:.5f}" for v in losses])
    assert losses[-1] < losses[0]
    run.close()
