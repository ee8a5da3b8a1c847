"""GPU checks of the output head and loss through the C ABI (ls_stage_head,
ls_head_loss) against the oracle: SFT cross entropy and DPO on the toy stack with a
2000-row head streamed in three slices (768, 768, 464 rows), the full chain into
ls_backward, bit-for-bit agreement of streamed and resident runs, and the error paths."""
import numpy as np
import pytest

from layer_streamed_qlora_amd import binding as B
from layer_streamed_qlora_amd import synth
from oracle import head as ohead
from oracle import nf4 as onf4
from oracle import stack as ostack
import lsq_harness as H

pytestmark = pytest.mark.gpu

TOY = synth.WORKLOADS["toy"]
V = 2000
BATCH, SEQ = 2, 64
T = BATCH * SEQ


def say(*a):
    print(*a, flush=True)


def bf16(x):
    return onf4.bf16_round(x).astype(np.float64)


def toy_labels():
    lab = synth.labels(TOY, V, T)
    lab[0], lab[1], lab[2] = 767, 768, 1999          # both sides of a slice boundary, the ragged last slice
    lab[3], lab[4] = V, -5                            # out of range: no loss
    lab[SEQ] = 1535                                  # last row of the second slice
    return lab


def oracle_labels(lab):
    return np.where((lab >= 0) & (lab < V), lab, ohead.IGNORE)


class HeadRun:
    def __init__(self, resident=0, n_buffers=2, zero_b=False, store_path=None, vocab=V):
        import torch
        self.torch = torch
        self.run = H.GpuRun(TOY, [0, 1], resident=resident, n_buffers=n_buffers, zero_b=zero_b, vocab=vocab,
                            store_path=store_path)
        self.Wh, self.gf = synth.head_weights(TOY, vocab)
        self.run.ctx.stage_head(synth.bf16_bits(self.Wh), synth.bf16_bits(self.gf))

    def step(self, kind, lab, beta=0.1, backward=True):
        torch, run = self.torch, self.run
        x, _ = synth.activations(TOY)
        X = run.to_dev_bf16(x)
        Y = torch.empty((T, TOY.hidden), dtype=torch.bfloat16, device="cuda:0")
        Yr = torch.empty_like(Y)
        dY = torch.empty_like(Y)
        dX = torch.empty_like(Y)
        L = torch.from_numpy(lab.astype(np.int32)).to("cuda:0")
        out = torch.zeros(2 + 2 * BATCH, dtype=torch.float32, device="cuda:0")
        dpo = kind == B.LS_LOSS_DPO
        run.ctx.forward(X.data_ptr(), BATCH, SEQ, 1, Y.data_ptr(), Yr.data_ptr() if dpo else 0)
        run.ctx.head_loss(Y.data_ptr(), Yr.data_ptr() if dpo else 0, L.data_ptr(), kind, beta, out.data_ptr(),
                          dY.data_ptr())
        if backward:
            run.ctx.backward(dY.data_ptr(), dX.data_ptr(), 0)
        run.ctx.sync()
        torch.cuda.synchronize()
        res = {"x": x, "Y": run.from_dev_bf16(Y), "dY": run.from_dev_bf16(dY), "out": out.cpu().numpy().copy()}
        if dpo:
            res["Y_ref"] = run.from_dev_bf16(Yr)
        if backward:
            res["dX"] = run.from_dev_bf16(dX)
            res["dA"] = [{p: run.dA[l][p].cpu().numpy().copy() for p in H.PROJS} for l in range(2)]
            res["dB"] = [{p: run.dB[l][p].cpu().numpy().copy() for p in H.PROJS} for l in range(2)]
        return res

    def close(self):
        self.run.close()


def rel(a, b):
    return abs(float(a) - float(b)) / max(abs(float(b)), 1e-30)


def test_sft_head_parity_and_full_chain():
    lab = toy_labels()
    hr = HeadRun()
    say("case: toy SFT head, vocab", V, "slices of", hr.run.ctx.stats().blob_bytes // (2 * TOY.hidden))
    g = hr.step(B.LS_LOSS_SFT, lab)
    src = hr.run.src
    hr.close()
    lo = oracle_labels(lab)
    # the head alone, on the GPU's own hidden states
    yn, r, z = ohead.head_forward(g["Y"], hr.gf, hr.Wh, TOY.rms_eps, rnd=bf16)
    loss, seqsum, n, dz = ohead.sft_loss(z, lo, SEQ)
    dy = ohead.head_backward(dz, hr.Wh, g["Y"], hr.gf, r, rnd=bf16)
    say("loss gpu", g["out"][0], "oracle", loss, "| dY rel L2", H.rel_l2(g["dY"], dy))
    assert g["out"][1] == n == int(((lab >= 0) & (lab < V)).sum())
    assert rel(g["out"][0], loss) < 1e-4
    np.testing.assert_allclose(g["out"][2:2 + BATCH], seqsum, rtol=1e-4)
    assert np.all(g["out"][2 + BATCH:] == 0)
    assert H.rel_l2(g["dY"], dy) < 2e-2
    # the whole chain: oracle stack -> head -> loss -> dY -> recompute backward
    _, lw = H.oracle_layers(TOY, src)
    loras = [synth.layer_lora(TOY, l) for l in range(2)]
    shp = H.oracle_shape(TOY)
    y_o, ck = ostack.stack_forward(g["x"], lw, loras, shp, BATCH, SEQ, True, True)
    yn, r, z = ohead.head_forward(y_o, hr.gf, hr.Wh, TOY.rms_eps, rnd=bf16)
    loss_o, _, _, dz = ohead.sft_loss(z, lo, SEQ)
    dy_o = ohead.head_backward(dz, hr.Wh, y_o, hr.gf, r, rnd=bf16)
    dx_o, grads = ostack.stack_backward(dy_o, ck, lw, loras, shp, BATCH, SEQ, True)
    errs, fails = H.compare({"Y": g["Y"], "dX": g["dX"], "dA": g["dA"], "dB": g["dB"]},
                            {"Y": y_o, "dX": dx_o, "grads": grads})
    say({k: f"{v:.2e}" for k, v in errs.items() if k in ("Y", "dX")}, "loss", loss_o)
    assert rel(g["out"][0], loss_o) < 1e-2
    assert not fails, fails


def test_sft_head_odd_vocabulary():
    """1999 rows: the last slice has 463 rows, not a multiple of four, so the last
    column quad of the head product is partial; loss and dY still match the oracle."""
    v = 1999
    lab = synth.labels(TOY, v, T)
    lab[0], lab[1], lab[2] = v - 1, 1535, 1536       # the ragged slice's last row, a slice boundary
    hr = HeadRun(vocab=v)
    say("case: toy SFT head, vocab", v)
    g = hr.step(B.LS_LOSS_SFT, lab, backward=False)
    hr.close()
    lo = np.where((lab >= 0) & (lab < v), lab, ohead.IGNORE)
    yn, r, z = ohead.head_forward(g["Y"], hr.gf, hr.Wh, TOY.rms_eps, rnd=bf16)
    loss, seqsum, n, dz = ohead.sft_loss(z, lo, SEQ)
    dy = ohead.head_backward(dz, hr.Wh, g["Y"], hr.gf, r, rnd=bf16)
    say("loss gpu", g["out"][0], "oracle", loss, "| dY rel L2", H.rel_l2(g["dY"], dy))
    assert g["out"][1] == n
    assert rel(g["out"][0], loss) < 1e-4
    np.testing.assert_allclose(g["out"][2:2 + BATCH], seqsum, rtol=1e-4)
    assert H.rel_l2(g["dY"], dy) < 2e-2


def test_dpo_equal_policy_is_log2():
    """B = 0: the adapters add nothing, policy and reference outputs are equal bit for bit,
    every margin is exactly 0, the loss is log 2 and each token's gradient carries
    -/+ beta / (2P)."""
    lab = toy_labels()
    hr = HeadRun(zero_b=True)
    beta = 0.5
    g = hr.step(B.LS_LOSS_DPO, lab, beta=beta, backward=False)
    hr.close()
    assert np.array_equal(g["Y"].view(np.uint32), g["Y_ref"].view(np.uint32))
    assert g["out"][0] == np.float32(np.log(2.0))
    assert np.array_equal(g["out"][2:2 + BATCH], g["out"][2 + BATCH:])
    lo = oracle_labels(lab)
    yn, r, z = ohead.head_forward(g["Y"], hr.gf, hr.Wh, TOY.rms_eps, rnd=bf16)
    _, _, _, _, dz = ohead.dpo_loss(z, z, lo, SEQ, beta)
    dy = ohead.head_backward(dz, hr.Wh, g["Y"], hr.gf, r, rnd=bf16)
    assert H.rel_l2(g["dY"], dy) < 2e-2


def test_dpo_parity_and_full_chain():
    lab = toy_labels()
    hr = HeadRun()
    beta = 2.0
    g = hr.step(B.LS_LOSS_DPO, lab, beta=beta)
    src = hr.run.src
    hr.close()
    lo = oracle_labels(lab)
    _, r, zp = ohead.head_forward(g["Y"], hr.gf, hr.Wh, TOY.rms_eps, rnd=bf16)
    _, _, zr = ohead.head_forward(g["Y_ref"], hr.gf, hr.Wh, TOY.rms_eps, rnd=bf16)
    loss, pol, ref, margin, dz = ohead.dpo_loss(zp, zr, lo, SEQ, beta)
    dy = ohead.head_backward(dz, hr.Wh, g["Y"], hr.gf, r, rnd=bf16)
    say("dpo loss gpu", g["out"][0], "oracle", loss, "margin", margin, "| dY rel L2", H.rel_l2(g["dY"], dy))
    assert rel(g["out"][0], loss) < 1e-3
    np.testing.assert_allclose(g["out"][2:2 + BATCH], pol, rtol=1e-4)
    np.testing.assert_allclose(g["out"][2 + BATCH:], ref, rtol=1e-4)
    assert H.rel_l2(g["dY"], dy) < 2e-2
    # whole chain with the reference pass
    _, lw = H.oracle_layers(TOY, src)
    loras = [synth.layer_lora(TOY, l) for l in range(2)]
    shp = H.oracle_shape(TOY)
    y_o, ck = ostack.stack_forward(g["x"], lw, loras, shp, BATCH, SEQ, True, True)
    yr_o, _ = ostack.stack_forward(g["x"], lw, loras, shp, BATCH, SEQ, False, True)
    _, r, zp = ohead.head_forward(y_o, hr.gf, hr.Wh, TOY.rms_eps, rnd=bf16)
    _, _, zr = ohead.head_forward(yr_o, hr.gf, hr.Wh, TOY.rms_eps, rnd=bf16)
    loss_o, _, _, _, dz = ohead.dpo_loss(zp, zr, lo, SEQ, beta)
    dy_o = ohead.head_backward(dz, hr.Wh, y_o, hr.gf, r, rnd=bf16)
    dx_o, grads = ostack.stack_backward(dy_o, ck, lw, loras, shp, BATCH, SEQ, True)
    errs, fails = H.compare({"Y": g["Y"], "dX": g["dX"], "dA": g["dA"], "dB": g["dB"]},
                            {"Y": y_o, "dX": dx_o, "grads": grads})
    say({k: f"{v:.2e}" for k, v in errs.items() if k in ("Y", "dX")}, "loss", loss_o)
    assert rel(g["out"][0], loss_o) < 1e-2
    assert not fails, fails


@pytest.mark.parametrize("kind", [B.LS_LOSS_SFT, B.LS_LOSS_DPO])
def test_head_streamed_equals_resident_bitwise(kind, tmp_path):
    lab = toy_labels()
    outs = []
    for resident, nb, path in ((1, 2, None), (0, 2, None), (0, 3, None), (0, 2, str(tmp_path / "store.bin"))):
        say("case: head kind", kind, "resident", resident, "slots", nb, "file store" if path else "")
        hr = HeadRun(resident=resident, n_buffers=nb, store_path=path)
        outs.append(hr.step(kind, lab, beta=0.3))
        hr.close()
    a = outs[0]
    for b in outs[1:]:
        assert np.array_equal(a["out"].view(np.uint32), b["out"].view(np.uint32))
        for k in ("dY", "dX"):
            assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k


def test_head_errors():
    torch = pytest.importorskip("torch")
    hr = HeadRun()
    ctx = hr.run.ctx
    buf = torch.zeros((T, TOY.hidden), dtype=torch.bfloat16, device="cuda:0")
    lab = torch.zeros(T, dtype=torch.int32, device="cuda:0")
    out = torch.zeros(2 + 2 * BATCH, device="cuda:0")
    p = buf.data_ptr()
    with pytest.raises(B.LsError) as e:        # no forward yet
        ctx.head_loss(p, 0, lab.data_ptr(), B.LS_LOSS_SFT, 0, out.data_ptr(), p)
    assert e.value.status == B.LS_ERR_STATE
    ctx.forward(p, BATCH, SEQ, 1, p)           # no reference pass
    with pytest.raises(B.LsError) as e:
        ctx.head_loss(p, p, lab.data_ptr(), B.LS_LOSS_DPO, 0.1, out.data_ptr(), p)
    assert e.value.status == B.LS_ERR_STATE
    for kw in (dict(kind=7, beta=0.1), dict(kind=B.LS_LOSS_DPO, beta=0.0)):
        with pytest.raises(B.LsError) as e:
            ctx.head_loss(p, p, lab.data_ptr(), kw["kind"], kw["beta"], out.data_ptr(), p)
        assert e.value.status in (B.LS_ERR_INVALID, B.LS_ERR_STATE)
    ctx.sync()
    hr.close()
    run = H.GpuRun(TOY, [0])
    with pytest.raises(B.LsError) as e:
        run.ctx.stage_head(np.zeros((4, TOY.hidden), np.uint16), np.zeros(TOY.hidden, np.uint16))
    assert e.value.status == B.LS_ERR_STATE
    run.close()
