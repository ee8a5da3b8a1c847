"""GPU parity of the HIP path against the oracle on the toy stack (2 layers, hidden
256, 4/4 heads x 64, SwiGLU 688, NF4 block 64, LoRA r 8 / alpha 16, 1 x 128), plus the
identities the pages state, all through the C ABI."""
import numpy as np
import pytest

from layer_streamed_qlora_amd import synth
import lsq_harness as H

pytestmark = pytest.mark.gpu

TOY = synth.WORKLOADS["toy"]


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def toy_oracle():
    w = TOY
    x, dy = synth.activations(w)
    src = [synth.layer_weights(w, l) for l in range(w.n_layers)]
    loras = [synth.layer_lora(w, l) for l in range(w.n_layers)]
    ora = H.oracle_step(w, src, loras, x, dy, w.batch, w.seq, with_ref=True)
    return x, dy, ora


@pytest.mark.parametrize("dq", [False, True])
def test_dequant_bitwise(dq):
    w = TOY.with_(double_quant=dq)
    say("case: dequant bitwise toy dq=", dq)
    run = H.GpuRun(w, [0, 1])
    enc, _ = H.oracle_layers(w, run.src)
    for l in range(2):
        for pi, p in enumerate(H.PROJS):
            got = run.read_weight(l, pi)
            want = H.onf4.bf16_bits(enc[l][p].dequant())
            assert np.array_equal(got, want), (l, p, int(np.sum(got != want)))
    run.close()


def test_toy_stack_parity(toy_oracle):
    x, dy, ora = toy_oracle
    say("case: toy stack parity, streamed, 2 slots")
    run = H.GpuRun(TOY, [0, 1])
    gpu = run.step(x, dy, TOY.batch, TOY.seq, with_ref=True)
    run.close()
    errs, fails = H.compare(gpu, ora)
    errs["Y_ref"] = H.rel_l2(gpu["Y_ref"], ora["Y_ref"])
    say({k: f"{v:.2e}" for k, v in errs.items()})
    assert not fails, fails
    assert errs["Y_ref"] <= 1e-2


def test_toy_streamed_equals_resident_bitwise():
    w = TOY
    x, dy = synth.activations(w)
    outs = []
    for resident in (0, 1):
        say("case: toy streamed vs resident, resident =", resident)
        run = H.GpuRun(w, [0, 1], resident=resident)
        outs.append(run.step(x, dy, w.batch, w.seq, with_ref=True))
        run.close()
    a, b = outs
    for k in ("Y", "Y_ref", "dX"):
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k
    for l in range(2):
        for p in H.PROJS:
            assert np.array_equal(a["dA"][l][p].view(np.uint32), b["dA"][l][p].view(np.uint32)), (l, p)
            assert np.array_equal(a["dB"][l][p].view(np.uint32), b["dB"][l][p].view(np.uint32)), (l, p)


@pytest.mark.parametrize("n_buffers,split", [(3, 0), (5, 0), (0, 0), (2, 1), (3, 1)])
def test_deeper_pool_equals_resident_and_reuses_slots(n_buffers, split):
    """A pool of two or more slots on a 6-layer stack, with the DPO reference pass: two
    consecutive steps are bit for bit the resident run, and in the second step every
    slot still holding the layer the other direction needs first is reused, so it copies
    2 (L - n_buffers) blobs.  With n_buffers = 0 the library picks the depth: one slot
    per layer here, so the second step copies nothing.  split = 1 copies every layer as
    four pieces, each fenced on its own (copy_split)."""
    w = TOY
    L = 6
    x, dy = synth.activations(w)
    say("case: toy pool depth", n_buffers, "split copies" if split else "")
    res = H.GpuRun(w, range(L), resident=1)
    want = res.step(x, dy, w.batch, w.seq, with_ref=True)
    res.close()
    run = H.GpuRun(w, range(L), n_buffers=n_buffers, copy_split=split)
    if n_buffers == 0:
        n_buffers = run.ctx.stats().n_slots
        assert n_buffers == L, n_buffers
    for s in range(2):
        c0 = run.ctx.stats().h2d_copies
        got = run.step(x, dy, w.batch, w.seq, with_ref=True)
        copies = run.ctx.stats().h2d_copies - c0
        for k in ("Y", "Y_ref", "dX"):
            assert np.array_equal(got[k].view(np.uint32), want[k].view(np.uint32)), (s, k)
        for l in range(L):
            for p in H.PROJS:
                assert np.array_equal(got["dA"][l][p].view(np.uint32), want["dA"][l][p].view(np.uint32)), (s, l, p)
                assert np.array_equal(got["dB"][l][p].view(np.uint32), want["dB"][l][p].view(np.uint32)), (s, l, p)
    assert copies == 2 * (L - n_buffers), copies
    run.close()


def test_b_zero_is_base_only_and_reference_is_lora_off():
    w = TOY
    x, dy = synth.activations(w)
    say("case: toy B = 0")
    run = H.GpuRun(w, [0, 1], zero_b=True)
    g0 = run.step(x, dy, w.batch, w.seq, with_ref=True)
    off = run.step(x, dy, w.batch, w.seq, backward=False, lora_on=False)
    run.close()
    assert np.array_equal(g0["Y"], off["Y"])
    assert np.array_equal(g0["Y"], g0["Y_ref"])
    for l in range(2):
        for p in H.PROJS:
            assert np.all(g0["dA"][l][p] == 0), (l, p)


def test_accumulate_adds():
    w = TOY
    x, dy = synth.activations(w)
    say("case: toy accumulate")
    run = H.GpuRun(w, [0, 1])
    a = run.step(x, dy, w.batch, w.seq)
    b = run.step(x, dy, w.batch, w.seq, accumulate=1)
    run.close()
    for l in range(2):
        for p in H.PROJS:
            assert np.array_equal(b["dA"][l][p], a["dA"][l][p] * 2), (l, p)
            assert np.array_equal(b["dB"][l][p], a["dB"][l][p] * 2), (l, p)


@pytest.mark.parametrize("n_layers", [1, 2])
def test_outputs_may_alias_inputs(n_layers):
    """Y written over X (with the reference pass on) and dX written over dY give the same
    bits as separate buffers, dA and dB included: the down projection's dB reads dY on the
    side stream, which must finish before the last layer writes dX over it."""
    torch = pytest.importorskip("torch")
    w = TOY
    x, dy = synth.activations(w)
    say("case: toy aliasing, layers", n_layers)
    run = H.GpuRun(w, list(range(n_layers)))
    sep = run.step(x, dy, w.batch, w.seq, with_ref=True)
    X = run.to_dev_bf16(x)
    Yr = torch.empty_like(X)
    run.ctx.forward(X.data_ptr(), w.batch, w.seq, 1, X.data_ptr(), Yr.data_ptr())   # Y over X
    D = run.to_dev_bf16(dy)
    run.ctx.backward(D.data_ptr(), D.data_ptr(), 0)                                   # dX over dY
    run.ctx.sync()
    torch.cuda.synchronize()
    got = {"Y": run.from_dev_bf16(X), "Y_ref": run.from_dev_bf16(Yr), "dX": run.from_dev_bf16(D)}
    dA = [{p: run.dA[l][p].cpu().numpy() for p in H.PROJS} for l in range(n_layers)]
    dB = [{p: run.dB[l][p].cpu().numpy() for p in H.PROJS} for l in range(n_layers)]
    run.close()
    for k in ("Y", "Y_ref", "dX"):
        assert np.array_equal(got[k].view(np.uint32), sep[k].view(np.uint32)), k
    for l in range(n_layers):
        for p in H.PROJS:
            assert np.array_equal(dA[l][p].view(np.uint32), sep["dA"][l][p].view(np.uint32)), (l, p)
            assert np.array_equal(dB[l][p].view(np.uint32), sep["dB"][l][p].view(np.uint32)), (l, p)


@pytest.mark.parametrize("batch,seq", [(3, 40), (2, 8)])
def test_ragged_shapes(batch, seq):
    """Token counts and sequence lengths that leave partial tiles everywhere."""
    w = TOY.with_(batch=batch, seq=seq)
    x, dy = synth.activations(w)
    say("case: toy ragged", batch, seq)
    run = H.GpuRun(w, [0, 1], max_tokens=128, max_seq=128)
    gpu = run.step(x, dy, batch, seq)
    src = run.src
    run.close()
    ora = H.oracle_step(w, src, [synth.layer_lora(w, l) for l in range(2)], x, dy, batch, seq)
    errs, fails = H.compare(gpu, ora)
    say({k: f"{v:.2e}" for k, v in errs.items() if k in ("Y", "dX")})
    assert not fails, fails


def test_empty_batch():
    w = TOY
    say("case: toy empty batch")
    run = H.GpuRun(w, [0, 1])
    for l in range(2):
        for p in H.PROJS:
            run.dA[l][p].fill_(7.0)
            run.dB[l][p].fill_(7.0)
    out = run.step(np.zeros((0, w.hidden), np.float32), np.zeros((0, w.hidden), np.float32), 0, 128)
    run.close()
    assert out["Y"].shape == (0, w.hidden)
    for l in range(2):
        for p in H.PROJS:
            assert np.all(out["dA"][l][p] == 0) and np.all(out["dB"][l][p] == 0)


@pytest.mark.parametrize("rank", [3, 32, 64])
def test_lora_ranks(rank):
    """A rank padded up to 16, and ranks whose stacked low-rank terms in the backward
    (3 r columns for q|k|v, 2 r for gate|up) are wider than one 64-column K tile."""
    w = TOY.with_(lora_r=rank, lora_alpha=2.0 * rank)
    x, dy = synth.activations(w)
    say("case: toy lora rank", rank)
    run = H.GpuRun(w, [0, 1])
    gpu = run.step(x, dy, w.batch, w.seq)
    src = run.src
    run.close()
    ora = H.oracle_step(w, src, [synth.layer_lora(w, l) for l in range(2)], x, dy, w.batch, w.seq)
    errs, fails = H.compare(gpu, ora)
    say({k: f"{v:.2e}" for k, v in errs.items() if k in ("Y", "dX")})
    assert not fails, fails


@pytest.mark.parametrize("split", [0, 1])
def test_file_store_equals_host_store_bitwise(tmp_path, split):
    """The base kept in a file and read through pinned staging buffers gives the same bits
    as the pinned-RAM store, over two steps; every copy is one file read (split = 1: one
    read per layer, copied to the slot in four pieces), and the file is gone after
    ls_destroy."""
    import os
    w = TOY
    L = 4
    x, dy = synth.activations(w)
    outs = []
    for path in (None, str(tmp_path / "store.bin")):
        say("case: toy store", "file" if path else "host", "split copies" if split and path else "")
        run = H.GpuRun(w, range(L), store_path=path, copy_split=split if path else 0)
        outs.append([run.step(x, dy, w.batch, w.seq, with_ref=True) for _ in range(2)])
        st = run.ctx.stats()
        if path is not None:
            say("store reads", st.store_reads, "copies", st.h2d_copies, "uncached", st.store_uncached)
            assert st.store_reads == st.h2d_copies > 0
        run.close()
        if path is not None:
            assert not os.path.exists(path)
    for a, b in zip(*outs):
        for k in ("Y", "Y_ref", "dX"):
            assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k
        for l in range(L):
            for p in H.PROJS:
                assert np.array_equal(a["dA"][l][p].view(np.uint32), b["dA"][l][p].view(np.uint32)), (l, p)
                assert np.array_equal(a["dB"][l][p].view(np.uint32), b["dB"][l][p].view(np.uint32)), (l, p)


def test_file_store_bad_path_is_refused():
    from layer_streamed_qlora_amd import binding as B
    cfg = B.make_config(TOY, store_path="/nonexistent-dir/for/sure/store.bin")
    with pytest.raises(B.LsError) as e:
        B.Context(cfg)
    assert e.value.status == B.LS_ERR_INVALID


def test_profiling_levels():
    """LS_PROFILE_GEMM times only the forward pass's dequant GEMMs (4 per layer; the
    recompute's are not timed), of every profile_stride-th layer if that is set;
    LS_PROFILE_ALL every class and the copy intervals; the results do not depend on the
    level."""
    from layer_streamed_qlora_amd import binding as B
    w = TOY
    x, dy = synth.activations(w)
    run = H.GpuRun(w, [0, 1, 2], profile=B.LS_PROFILE_GEMM)   # 3 layers, 2 slots: every step copies
    a = run.step(x, dy, w.batch, w.seq)
    st = run.ctx.stats()
    assert st.k_launches[0] == 4 * 3 and all(st.k_launches[j] == 0 for j in range(1, B.LS_KC_N))
    assert st.last_copy_ms == 0.0
    sampled = H.GpuRun(w, [0, 1, 2], profile=B.LS_PROFILE_GEMM, profile_stride=2)   # layers 0 and 2
    c = sampled.step(x, dy, w.batch, w.seq)
    assert sampled.ctx.stats().k_launches[0] == 4 * 2
    sampled.close()
    for k in ("Y", "dX"):
        assert np.array_equal(a[k].view(np.uint32), c[k].view(np.uint32)), k
    run.ctx.set_profile(B.LS_PROFILE_ALL)
    b = run.step(x, dy, w.batch, w.seq)
    st = run.ctx.stats()
    assert all(st.k_launches[j] > 0 for j in range(0, 5)) and st.last_copy_ms > 0.0
    for k in ("Y", "dX"):
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k
    with pytest.raises(B.LsError) as e:
        run.ctx.set_profile(7)
    assert e.value.status == B.LS_ERR_INVALID
    run.close()
