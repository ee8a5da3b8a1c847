"""Calls out of order are refused, and a HIP failure is sticky.

The library refuses rather than run wrong (the lachieslifestyle.com how-to, "Step 7:
Train and keep the log": a run that cannot be right is stopped with its reason): a
backward needs a forward over the current weights and adapters; a forward needs every
layer staged; the store cannot change under work in flight.  Once an asynchronous
failure is seen (here a read from the file store that comes up short, forced from the
host by truncating the file), every later call returns LS_ERR_HIP with its message.
Every GPU kernel involved still runs normally: nothing here faults the device.
"""
import os

import numpy as np
import pytest

from layer_streamed_qlora_amd import binding as B
from layer_streamed_qlora_amd import synth
import lsq_harness as H

pytestmark = pytest.mark.gpu

TOY = synth.WORKLOADS["toy"]


def status_of(fn, *a):
    try:
        fn(*a)
    except B.LsError as e:
        return e.status
    return B.LS_OK


def buffers(run):
    torch = run.torch
    T, h = TOY.tokens, TOY.hidden
    x, dy = synth.activations(TOY)
    X = run.to_dev_bf16(x)
    dY = run.to_dev_bf16(dy)
    Y = torch.empty((T, h), dtype=torch.bfloat16, device="cuda:0")
    dX = torch.empty_like(Y)
    return X, dY, Y, dX


def test_backward_needs_a_valid_forward():
    run = H.GpuRun(TOY, [0, 1])
    X, dY, Y, dX = buffers(run)
    c = run.ctx
    # backward before any forward
    assert status_of(c.backward, dY.data_ptr(), dX.data_ptr()) == B.LS_ERR_STATE
    # a forward with the adapters off cannot be differentiated
    c.forward(X.data_ptr(), 1, 128, 0, Y.data_ptr())
    c.sync()
    assert status_of(c.backward, dY.data_ptr(), dX.data_ptr()) == B.LS_ERR_STATE
    # a valid forward, then a re-staged layer: the forward's products are stale
    c.forward(X.data_ptr(), 1, 128, 1, Y.data_ptr())
    c.sync()
    c.stage_layer(1, {k: synth.bf16_bits(v) for k, v in synth.layer_weights(TOY, 1).items()})
    assert status_of(c.backward, dY.data_ptr(), dX.data_ptr()) == B.LS_ERR_STATE
    # ... and a re-registered adapter
    c.forward(X.data_ptr(), 1, 128, 1, Y.data_ptr())
    c.sync()
    c.set_lora(0, 2, run.A[0]["v"].data_ptr(), run.Bm[0]["v"].data_ptr(), run.dA[0]["v"].data_ptr(),
               run.dB[0]["v"].data_ptr())
    assert status_of(c.backward, dY.data_ptr(), dX.data_ptr()) == B.LS_ERR_STATE
    # a fresh forward makes it valid again
    c.forward(X.data_ptr(), 1, 128, 1, Y.data_ptr())
    c.backward(dY.data_ptr(), dX.data_ptr())
    c.sync()
    assert np.isfinite(run.from_dev_bf16(dX)).all()
    run.close()


def test_forward_needs_every_layer_staged():
    cfg = B.make_config(TOY, n_layers=2)
    ctx = B.Context(cfg)
    run_like = H.GpuRun(TOY, [0])           # only for its buffers
    X, dY, Y, dX = buffers(run_like)
    ctx.stage_layer(0, {k: synth.bf16_bits(v) for k, v in synth.layer_weights(TOY, 0).items()})
    assert status_of(ctx.forward, X.data_ptr(), 1, 128, 1, Y.data_ptr()) == B.LS_ERR_STATE
    assert "not staged" in B.lib().ls_last_error(ctx.h).decode()
    ctx.close()
    run_like.close()


def test_store_cannot_change_under_work_in_flight():
    run = H.GpuRun(TOY, [0, 1])
    X, dY, Y, dX = buffers(run)
    c = run.ctx
    src = {k: synth.bf16_bits(v) for k, v in synth.layer_weights(TOY, 0).items()}
    c.forward(X.data_ptr(), 1, 128, 1, Y.data_ptr())
    assert status_of(c.stage_layer, 0, src) == B.LS_ERR_STATE
    c.backward(dY.data_ptr(), dX.data_ptr())
    assert status_of(c.stage_layer, 0, src) == B.LS_ERR_STATE
    c.sync()
    c.stage_layer(0, src)                   # allowed once the streams are drained
    run.close()


def test_a_failed_store_read_is_sticky(tmp_path):
    path = str(tmp_path / "store.bin")
    run = H.GpuRun(TOY, [0, 1, 2], store_path=path)   # 3 layers, 2 slots: copies every step
    X, dY, Y, dX = buffers(run)
    c = run.ctx
    c.forward(X.data_ptr(), 1, 128, 1, Y.data_ptr())
    c.backward(dY.data_ptr(), dX.data_ptr())
    c.sync()
    os.truncate(path, 0)                    # every later read of a blob comes up short
    c.forward(X.data_ptr(), 1, 128, 1, Y.data_ptr())
    assert status_of(c.sync) == B.LS_ERR_HIP
    msg = B.lib().ls_last_error(c.h).decode()
    assert "store file" in msg
    src = {k: synth.bf16_bits(v) for k, v in synth.layer_weights(TOY, 0).items()}
    for call, args in ((c.forward, (X.data_ptr(), 1, 128, 1, Y.data_ptr())), (c.backward, (dY.data_ptr(), dX.data_ptr())),
                       (c.stage_layer, (0, src)), (c.set_lora, (0, 0, run.A[0]["q"].data_ptr(), run.Bm[0]["q"].data_ptr())),
                       (c.sync, ()), (c.adamw_reset, ())):
        assert status_of(call, *args) == B.LS_ERR_HIP, call.__name__
    st = c.stats()                          # statistics still readable
    assert st.h2d_copies > 0
    run.close()
    assert not os.path.exists(path)
