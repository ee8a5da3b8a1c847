"""Bit-exact dequantisation on the path the GEMMs take.

ls_base_gemm runs the fused dequant-GEMM kernels that the forward and the backward
launch for a projection group (q|k|v stacked, o, gate|up paired, down), with the
adapter term off.  Rows of X holding a single 1.0 make every output a float32 sum of
one product 1.0 * w and zeros, so the output is the dequantised weight itself; it must
equal the oracle's bf16_rne(fp32(level[code] * absmax)) exactly (the dequantisation
the pages name: "Fine-Tuning an 8B Parameter Model on a 4 GB Laptop GPU", section
"Quantization: Shrink the Weights"; the NF4 base that went wrong above about 165 MB
per layer: "Soup: Fine-Tuning an 8B Model on a 4 GB Laptop GPU, One Layer at a Time",
third paragraph).

Both orientations are read over every element: the forward orientation (X deq(W)^T)
returns columns of deq(W), the backward's W^T orientation (dY deq(W)) returns rows.
Cases: the toy layer (NF4 with float32 absmax; its 688-wide projections take the
256-thread kernels), a Llama-3.1-8B-shaped layer (NF4 + double quantisation), a
Qwen2.5-3B-shaped layer (bf16 base) and a Qwen2.5-32B-shaped layer (NF4 + double
quantisation, a 251.5 MB blob).  Values compare as floats, so +0 and -0 count equal;
every non-zero weight matches bit for bit.
"""
import numpy as np
import pytest

from layer_streamed_qlora_amd import synth
from oracle import stack as ostack
import lsq_harness as H

pytestmark = pytest.mark.gpu

GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
M_MAX = 4096


def say(*a):
    print(*a, flush=True)


def oracle_dequant(w, src):
    """float32 dequantised weights of one layer, from the oracle's own encoding."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=7) as ex:
        enc = ostack.quantize_layer(src, w.quant, w.double_quant, map_fn=ex.map)

        def deq(p):
            t = enc[p]
            return t.dequant() if hasattr(t, "dequant") else np.asarray(t, np.float32)

        return dict(zip(H.PROJS, ex.map(deq, H.PROJS)))


def one_hot(torch, m, width, first):
    x = torch.zeros((m, width), dtype=torch.bfloat16, device="cuda:0")
    idx = torch.arange(m, device="cuda:0")
    x[idx, first + idx] = 1.0
    return x


def readback_case(name, layer):
    torch = pytest.importorskip("torch")
    w = synth.WORKLOADS[name].with_(batch=1, seq=128)
    say(f"case: dequant through the fused GEMMs, {name} layer {layer}")
    run = H.GpuRun(w, [layer], max_tokens=M_MAX, max_seq=128)
    deq = oracle_dequant(w, run.src[0])
    run.src = None
    checked = 0
    for gi, projs in enumerate(GROUPS):
        want = np.concatenate([deq[p] for p in projs], axis=0)     # [sum n_out, n_in]
        n_out, n_in = want.shape
        # forward orientation: X = rows e_c, c in [c0, c0 + m): out = deq(W)[:, c].T
        for c0 in range(0, n_in, M_MAX):
            m = min(M_MAX, n_in - c0)
            x = one_hot(torch, m, n_in, c0)
            out = torch.empty((m, n_out), dtype=torch.float32, device="cuda:0")
            run.ctx.base_gemm(0, gi, 0, x.data_ptr(), m, out.data_ptr())
            got = out.cpu().numpy()
            exp = want[:, c0:c0 + m].T
            bad = got != exp
            assert not bad.any(), (name, projs, "W", c0, int(bad.sum()), np.argwhere(bad)[:4].tolist())
            checked += got.size
            del x, out
        # backward orientation: dY = rows e_r over the stacked outputs: out = deq(W)[r, :]
        for r0 in range(0, n_out, M_MAX):
            m = min(M_MAX, n_out - r0)
            x = one_hot(torch, m, n_out, r0)
            out = torch.empty((m, n_in), dtype=torch.float32, device="cuda:0")
            run.ctx.base_gemm(0, gi, 1, x.data_ptr(), m, out.data_ptr())
            got = out.cpu().numpy()
            bad = got != want[r0:r0 + m]
            assert not bad.any(), (name, projs, "W^T", r0, int(bad.sum()), np.argwhere(bad)[:4].tolist())
            checked += got.size
            del x, out
    run.close()
    total = sum(np.prod(w.proj_shape(p)) for p in H.PROJS)
    assert checked == 2 * total
    say(f"{name}: {checked} dequantised weights equal the oracle's")


def test_toy_layer_both_kernels():
    readback_case("toy", 0)


def test_llama8b_layer_nf4_double_quant():
    readback_case("llama8b", 31)


def test_qwen3b_layer_bf16_base():
    readback_case("qwen3b", 5)


def test_qwen32b_layer_251mb_blob():
    readback_case("qwen32b", 0)


def test_llama8b_split_tiles_random_activations():
    """The tail-split launches (the tiles past the last full round of compute units cut
    into K ranges whose float32 sums the piece that finishes last adds in piece order),
    with random activations on the Llama-3.1-8B shapes: the q|k|v forward at 4096 rows
    (384 tiles of 256 x 256: two pieces per tail tile), the down projection's W^T
    orientation at 4096 rows (896 tiles: two pieces), the down forward at 1024 rows (64
    tiles: four pieces; again at 1000 rows, a ragged last row block) and the q|k|v W^T
    orientation at 512 rows (32 tiles: eight pieces).  Every sampled output row must match the float64 product of the same bf16
    activations and the oracle's dequantised weights within the float32 accumulation
    bound K 2^-23 sum |x w|, and a second call must give the same bits."""
    torch = pytest.importorskip("torch")
    w = synth.WORKLOADS["llama8b"].with_(batch=1, seq=128)
    say("case: split-tile dequant GEMMs, llama8b layer 7, random activations")
    run = H.GpuRun(w, [7], max_tokens=M_MAX, max_seq=128)
    deq = oracle_dequant(w, run.src[0])
    run.src = None
    g = torch.Generator(device="cpu").manual_seed(1234)
    for gi, transposed, m in ((0, 0, 4096), (3, 1, 4096), (3, 0, 1024), (0, 1, 512), (3, 0, 1000)):
        projs = GROUPS[gi]
        wmat = np.concatenate([deq[p] for p in projs], axis=0).astype(np.float64)   # [sum n_out, n_in]
        b = wmat if transposed else wmat.T                                          # [K, N]
        k_dim, n_dim = b.shape
        x = torch.randn((m, k_dim), generator=g).to(torch.bfloat16)
        xd = x.to("cuda:0")
        outs = []
        for _ in range(2):
            out = torch.empty((m, n_dim), dtype=torch.float32, device="cuda:0")
            run.ctx.base_gemm(0, gi, transposed, xd.data_ptr(), m, out.data_ptr())
            outs.append(out.cpu().numpy())
            del out
        assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32)), (projs, "not deterministic")
        rows = np.concatenate([np.arange(mt * 256, min(m, mt * 256 + 256), 37) for mt in range((m + 255) // 256)])
        xs = x.float().numpy().astype(np.float64)[rows]
        exp = xs @ b
        bound = k_dim * 2.0 ** -23 * (np.abs(xs) @ np.abs(b)) + 1e-30
        err = np.abs(outs[0][rows].astype(np.float64) - exp)
        worst = float((err / bound).max())
        say(f"{'+'.join(projs)} {'W^T' if transposed else 'W'} at {m} rows: {len(rows)} rows x {n_dim}, "
            f"worst error / bound {worst:.3g}")
        assert worst <= 1.0, (projs, transposed, m, worst)
        del xd
    run.close()
