"""ls_lora_linear_noalloc (the projection for callers that cannot allocate: graph
capture, serving loops) against ls_lora_linear on the same inputs, bit for bit, over
two calls in a row, the second with a smaller input, so that whatever the first call
left in the fixed scratch must not leak into the second; then a call whose sizes do not
fit the fixed scratch is refused."""
import numpy as np
import pytest

from layer_streamed_qlora_amd import binding as B
from layer_streamed_qlora_amd import synth
from oracle import nf4 as onf4

pytestmark = pytest.mark.gpu


def make_case(torch, n_out, n_in, M, r, dq, seed):
    rng = np.random.default_rng(seed)
    dev = "cuda:0"
    w32 = onf4.bf16_round(rng.standard_normal((n_out, n_in)).astype(np.float32) * 0.02)
    packed, am, qabs, s2, mean = B.ls_pack_nf4(synth.bf16_bits(w32), dq)
    keep = []
    put = lambda a: keep.append(torch.from_numpy(np.ascontiguousarray(a)).to(dev)) or keep[-1].data_ptr()
    desc = B.ls_weight(quant=B.LS_QUANT_NF4, double_quant=int(dq), n_out=n_out, n_in=n_in)
    desc.w = put(packed)
    if dq:
        desc.qabs, desc.scale2, desc.mean = put(qabs), put(s2), put(np.array([mean], np.float32))
    else:
        desc.absmax = put(am)
    x = onf4.bf16_round(rng.standard_normal((M, n_in)).astype(np.float32))
    X = put(synth.bf16_bits(x).view(np.int16))
    A = put(rng.standard_normal((r, n_in)).astype(np.float32) / r)
    Bm = put(rng.standard_normal((n_out, r)).astype(np.float32) * 0.01)
    return desc, X, A, Bm, keep


def run_both(torch, n_out, n_in, M, r, dq, seed):
    desc, X, A, Bm, keep = make_case(torch, n_out, n_in, M, r, dq, seed)
    y_ws = torch.empty((M, n_out), dtype=torch.int16, device="cuda:0")
    y_na = torch.full((M, n_out), -1, dtype=torch.int16, device="cuda:0")
    nbytes = B.ls_lora_linear_workspace_bytes(M, n_in, n_out, r)
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda:0")
    ws_ptr = (ws.data_ptr() + 255) // 256 * 256
    B.ls_lora_linear(desc, X, M, A, Bm, r, 2.0 * r, y_ws.data_ptr(), ws_ptr, nbytes)
    B.ls_lora_linear_noalloc(desc, X, M, A, Bm, r, 2.0 * r, y_na.data_ptr())
    torch.cuda.synchronize()
    return y_ws.cpu().numpy(), y_na.cpu().numpy()


def test_noalloc_equals_workspace_call_twice_then_smaller():
    torch = pytest.importorskip("torch")
    # first call: larger rank and shapes; second: smaller rank (the A rows past r must
    # read as zero again), fewer tokens, narrower weight
    for n_out, n_in, M, r, dq, seed in ((2048, 4096, 512, 32, True, 1), (512, 1024, 96, 8, False, 2)):
        a, b = run_both(torch, n_out, n_in, M, r, dq, seed)
        assert np.array_equal(a, b), (n_out, n_in, M, r, int(np.sum(a != b)))
        assert np.any(a != 0)


def test_noalloc_refuses_sizes_beyond_its_scratch():
    torch = pytest.importorskip("torch")
    desc, X, A, Bm, keep = make_case(torch, 64, 64, 8, 16, False, 3)
    # A and B in bf16 alone would take 8 MiB each: refused on the host, before any launch
    desc.n_out, desc.n_in = 65536, 65536
    y = torch.empty((8, 64), dtype=torch.int16, device="cuda:0")
    big = B.ls_lora_linear_workspace_bytes(16384, 65536, 65536, 64)
    assert big > 12 << 20
    with pytest.raises(B.LsError) as e:
        B.ls_lora_linear_noalloc(desc, X, 16384, A, Bm, 64, 128.0, y.data_ptr())
    assert e.value.status == B.LS_ERR_INVALID and "fixed scratch" in str(e.value)
