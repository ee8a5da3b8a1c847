"""ls_lora_linear: one LoRA projection outside any context, Y = X deq(W)^T +
(alpha / r) (X A^T) B^T ("Fine-Tuning an 8B Parameter Model on a 4 GB Laptop GPU",
section "LoRA and QLoRA: Train a Fraction of the Parameters"), against the oracle's
projection in parity mode, for NF4 with and without double quantisation and a bf16
base, on a 64-aligned shape (512-thread GEMM) and a 688-wide one (256-thread GEMM),
with a ragged token count; rank 0 is the base term alone."""
import numpy as np
import pytest

from layer_streamed_qlora_amd import binding as B
from layer_streamed_qlora_amd import synth
from oracle import model as omodel
from oracle import nf4 as onf4

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


class DevWeight:
    """A weight packed by the library's host encoder and copied to the device."""

    def __init__(self, torch, w32, quant, dq):
        self.keep = []
        dev = "cuda:0"
        n_out, n_in = w32.shape
        self.desc = B.ls_weight(quant=B.LS_QUANT_NF4 if quant == "nf4" else B.LS_QUANT_BF16, double_quant=int(dq),
                                n_out=n_out, n_in=n_in)
        bits = synth.bf16_bits(w32)
        if quant == "bf16":
            t = torch.from_numpy(bits.view(np.int16)).to(dev)
            self.keep.append(t)
            self.desc.w = t.data_ptr()
            return
        packed, am, qabs, s2, mean = B.ls_pack_nf4(bits, dq)
        put = lambda a: self.keep.append(torch.from_numpy(np.ascontiguousarray(a)).to(dev)) or self.keep[-1].data_ptr()
        self.desc.w = put(packed)
        if dq:
            self.desc.qabs = put(qabs)
            self.desc.scale2 = put(s2)
            self.desc.mean = put(np.array([mean], np.float32))
        else:
            self.desc.absmax = put(am)


def case(torch, n_out, n_in, M, r, quant, dq, seed):
    rng = np.random.default_rng(seed)
    w32 = onf4.bf16_round(rng.standard_normal((n_out, n_in)).astype(np.float32) * 0.02)
    x32 = onf4.bf16_round(rng.standard_normal((M, n_in)).astype(np.float32))
    a = rng.standard_normal((max(r, 1), n_in)).astype(np.float32) / max(r, 1)
    b = rng.standard_normal((n_out, max(r, 1))).astype(np.float32) * 0.01
    W = DevWeight(torch, w32, quant, dq)
    X = torch.from_numpy(synth.bf16_bits(x32).view(np.int16)).to("cuda:0")
    A = torch.from_numpy(a[:r]).to("cuda:0").contiguous()
    Bt = torch.from_numpy(b[:, :r]).to("cuda:0").contiguous()
    Y = torch.empty((M, n_out), dtype=torch.int16, device="cuda:0")
    nbytes = B.ls_lora_linear_workspace_bytes(M, n_in, n_out, r)
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda:0")
    ws_ptr = (ws.data_ptr() + 255) // 256 * 256
    B.ls_lora_linear(W.desc, X.data_ptr(), M, A.data_ptr() if r else 0, Bt.data_ptr() if r else 0, r, 2.0 * r,
                     Y.data_ptr(), ws_ptr, nbytes)
    torch.cuda.synchronize()
    got = onf4.bf16_from_bits(Y.cpu().numpy().view(np.uint16))
    deq = onf4.NF4Tensor(w32, dq).dequant() if quant == "nf4" else w32
    rnd = lambda v: onf4.bf16_round(v).astype(np.float64)
    want, _ = omodel.lora_proj_fwd(x32.astype(np.float64), deq.astype(np.float64), a[:r].astype(np.float64),
                                   b[:, :r].astype(np.float64), 2.0, r > 0, rnd)
    err = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    # against the oracle's output rounded to bf16 the distance is what is left once the
    # output rounding itself (about 1.6e-3 of relative L2 on any such data) is taken out
    want16 = onf4.bf16_round(want).astype(np.float64)
    err16 = float(np.linalg.norm(got - want16) / np.linalg.norm(want16))
    return got, want, err, err16


@pytest.mark.parametrize("n_out,n_in,M,r,quant,dq", [
    (1024, 4096, 300, 16, "nf4", True),
    (256, 688, 130, 8, "nf4", False),
    (512, 1024, 64, 32, "bf16", False),
    (1024, 4096, 257, 0, "nf4", True),
])
def test_against_the_oracle(n_out, n_in, M, r, quant, dq):
    torch = pytest.importorskip("torch")
    got, want, err, err16 = case(torch, n_out, n_in, M, r, quant, dq, n_out + n_in + M + r)
    say(f"ls_lora_linear {n_out}x{n_in} M={M} r={r} {quant}{' dq' if dq else ''}: rel L2 {err:.2e}, "
        f"against the rounded oracle {err16:.2e}")
    assert err <= 1e-2
    assert err16 <= 1e-3


def test_refusals():
    torch = pytest.importorskip("torch")
    w = B.ls_weight(quant=B.LS_QUANT_BF16, double_quant=0, n_out=64, n_in=40)   # n_in not a multiple of 16
    x = torch.zeros((4, 64), dtype=torch.int16, device="cuda:0")
    with pytest.raises(B.LsError) as e:
        B.ls_lora_linear(w, x.data_ptr(), 4, 0, 0, 0, 1.0, x.data_ptr(), x.data_ptr(), 1 << 20)
    assert e.value.status == B.LS_ERR_INVALID and "multiple of 16" in str(e.value)
    w.n_in = 64
    w.w = x.data_ptr()
    with pytest.raises(B.LsError) as e:   # workspace too small
        B.ls_lora_linear(w, x.data_ptr(), 4, 0, 0, 0, 1.0, x.data_ptr(), x.data_ptr(), 16)
    assert e.value.status == B.LS_ERR_INVALID and "workspace" in str(e.value)
