"""NF4 encoding of the frozen base (TEST INFRASTRUCTURE ONLY; see ``oracle/__init__``).

The pages name the encoding but print none of its numbers: "Fine-Tuning an 8B
Parameter Model on a 4 GB Laptop GPU" (codeinktechnologies.com), section
"Quantization: Shrink the Weights", says the base is stored as 4-bit NormalFloat
(NF4) as introduced by the QLoRA paper, and that nested (double) quantisation of the
quantisation constants saves a further ~0.4 GB at 8B.  The lachieslifestyle.com
how-to, section "Step 5: Enable 4-bit layer streaming", sets ``quantization: 4bit``.
Block size 64 and the 8-bit / block-256 second level come from the workload
definitions this repository is measured on.

Readings taken where the pages are silent:

* codebook: the NormalFloat construction of the QLoRA paper (section 3): 8 positive
  levels at standard-normal quantiles of equally spaced probabilities from delta down
  to 1/2 (exclusive), 7 negative levels likewise, exact zero, normalised by the
  largest magnitude; delta = ((1 - 1/30) + (1 - 1/32)) / 2 exactly; all in float64,
  rounded once to float32.
* blocks run over the row-major flattened tensor (a block may straddle rows);
* absmax is the float32 max |x| of the bf16 weights in the block; n = fp32(x/absmax);
  the code is the nearest level, ties to the higher index; an all-zero block gets
  code 7 (the exact 0 level);
* nibble order: byte k holds element 2k in its high nibble, 2k+1 in its low nibble;
* double quantisation: one float32 mean per tensor (float64 sum in index order,
  divided by the count, rounded to float32), per group of 256 absmax values a
  float32 scale = max |fp32(a - mean)|; code = round-half-even(clamp(127 (a-mean)/scale,
  -127, 127)) evaluated in float64; decode fp32(fp32(fp32(c/127) * scale) + mean),
  two separate roundings;
* dequantisation: w = bf16_rne(fp32(level[code] * absmax)).
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import ndtri

NF4_BLOCK = 64
DQ_GROUP = 256
# delta of the NormalFloat construction, kept exact (QLoRA paper, section 3).
NF4_DELTA = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))


# --------------------------------------------------------------------------- bf16
def bf16_round(x) -> np.ndarray:
    """Round float64/float32 values to the nearest bfloat16 value, ties to even.

    Plain definition: bfloat16 keeps 8 significant bits and float32's exponent range
    (subnormal spacing 2**-133).  Returned as float32 (exactly representable).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    finite = np.isfinite(x) & (x != 0.0)
    m, e = np.frexp(x[finite])            # x = m * 2**e, 0.5 <= |m| < 1
    q = np.exp2(np.maximum(e - 8, -133).astype(np.float64))   # spacing of bf16 near x
    r = np.rint(x[finite] / q) * q        # x/q is exact (power-of-two scaling); rint = RNE
    out[finite] = r
    out[~finite] = x[~finite]
    max_bf16 = float(np.float32(np.frombuffer(np.uint32(0x7F7F0000).tobytes(), np.float32)[0]))
    out = np.where(np.abs(out) > max_bf16, np.copysign(np.inf, out), out)
    return out.astype(np.float32)


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-representable."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value is not bf16-representable"
    return (u >> 16).astype(np.uint16)


def bf16_from_bits(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------- codebook
def nf4_codebook() -> np.ndarray:
    """The 16 NF4 levels (float32, ascending): index 0 = -1, 7 = 0, 15 = +1."""
    d = NF4_DELTA
    pos_p = d + np.arange(8, dtype=np.float64) * (0.5 - d) / 8.0   # delta .. 1/2 (excl.)
    neg_p = d + np.arange(7, dtype=np.float64) * (0.5 - d) / 7.0
    pos = ndtri(pos_p)
    neg = -ndtri(neg_p)
    levels = np.sort(np.concatenate([neg, [0.0], pos]))
    levels = levels / np.max(np.abs(levels))
    return levels.astype(np.float32)


# ------------------------------------------------------------------- quantisation
def nearest_level(n: np.ndarray, levels: np.ndarray) -> np.ndarray:
    """Index of the nearest level to each float32 n; ties go to the higher index.

    The midpoints of adjacent levels are exact in float64; the nearest level is the
    number of midpoints <= n (a tie sits exactly on a midpoint and counts it, so it
    goes up).  The tests pin this against a brute-force argmin of |n - level|.
    """
    lv = levels.astype(np.float64)
    mids = (lv[:-1] + lv[1:]) / 2.0
    return np.searchsorted(mids, np.asarray(n, dtype=np.float64), side="right").astype(np.uint8)


def quantize_nf4(w_bf16: np.ndarray, block: int = NF4_BLOCK, chunk: int = 1 << 20):
    """Blockwise NF4 quantisation of a bf16-valued tensor.

    Returns (codes uint8 [numel], absmax float32 [ceil(numel/block)]).  Blocks run over
    the row-major flattening; a short final block uses the elements present.
    """
    x = np.ascontiguousarray(w_bf16, dtype=np.float32).reshape(-1)
    numel = x.size
    nblocks = -(-numel // block)
    levels = nf4_codebook()
    codes = np.empty(numel, dtype=np.uint8)
    absmax = np.empty(nblocks, dtype=np.float32)
    blocks_per_chunk = max(1, chunk // block)
    for b0 in range(0, nblocks, blocks_per_chunk):
        b1 = min(nblocks, b0 + blocks_per_chunk)
        e0, e1 = b0 * block, min(numel, b1 * block)
        seg = x[e0:e1]
        full = (e1 - e0) // block
        am = np.empty(b1 - b0, dtype=np.float32)
        if full:
            am[:full] = np.max(np.abs(seg[: full * block].reshape(full, block)), axis=1)
        if full < b1 - b0:
            am[full] = np.max(np.abs(seg[full * block:]))
        absmax[b0:b1] = am
        per_elem = np.repeat(am, block)[: e1 - e0]
        zero = per_elem == 0
        with np.errstate(divide="ignore", invalid="ignore"):
            n = (seg / np.where(zero, np.float32(1), per_elem)).astype(np.float32)
        c = nearest_level(n, levels)
        c[zero] = 7
        codes[e0:e1] = c
    return codes, absmax


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte: element 2k in the high nibble, 2k+1 in the low nibble.
    An odd final element is padded with code 7."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    if c.size % 2:
        c = np.concatenate([c, np.array([7], dtype=np.uint8)])
    return ((c[0::2] << 4) | c[1::2]).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray, numel: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p >> 4
    out[1::2] = p & 0x0F
    return out[:numel]


# ------------------------------------------------------------ double quantisation
def double_quantize(absmax: np.ndarray, group: int = DQ_GROUP):
    """Second-level quantisation of the absmax constants.

    Returns (qcodes uint8 [n], scale float32 [ceil(n/group)], mean float32 scalar).
    qcodes hold the int8 code in two's complement.
    """
    a = np.asarray(absmax, dtype=np.float32).reshape(-1)
    n = a.size
    # mean: float64 sum taken left to right in index order, divided by n, rounded to
    # float32 (cumsum accumulates sequentially, unlike numpy's pairwise sum).
    mean = np.float32(np.cumsum(a.astype(np.float64))[-1] / np.float64(n)) if n else np.float32(0)
    ngroups = -(-n // group)
    scale = np.empty(ngroups, dtype=np.float32)
    q = np.empty(n, dtype=np.int64)
    for g in range(ngroups):
        seg = a[g * group:(g + 1) * group]
        centred32 = (seg - mean).astype(np.float32)           # float32 subtraction
        s = np.float32(np.max(np.abs(centred32)))
        scale[g] = s
        if s == 0:
            q[g * group:(g + 1) * group] = 0
            continue
        t = (seg.astype(np.float64) - np.float64(mean)) / np.float64(s) * 127.0
        q[g * group:(g + 1) * group] = np.rint(np.clip(t, -127.0, 127.0))
    return (q & 0xFF).astype(np.uint8), scale, mean


def dq_decode(qcodes: np.ndarray, scale: np.ndarray, mean, group: int = DQ_GROUP) -> np.ndarray:
    """Decode double-quantised absmax: fp32(fp32(fp32(c/127) * scale) + mean)."""
    c = np.asarray(qcodes, dtype=np.uint8).astype(np.int8).astype(np.float32)
    frac = (c / np.float32(127.0)).astype(np.float32)
    s = np.repeat(np.asarray(scale, dtype=np.float32), group)[: c.size]
    prod = (frac * s).astype(np.float32)
    return (prod + np.float32(mean)).astype(np.float32)


# ------------------------------------------------------------------ dequantisation
def dequant_codes(codes: np.ndarray, absmax: np.ndarray, block: int = NF4_BLOCK) -> np.ndarray:
    """w = bf16_rne(fp32(level[code] * absmax[block of element])), float32 array."""
    levels = nf4_codebook()
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    am = np.repeat(np.asarray(absmax, dtype=np.float32), block)[: c.size]
    prod = (levels[c] * am).astype(np.float32)
    return bf16_round(prod)


class NF4Tensor:
    """A quantised [out, in] weight: packed codes plus first- or second-level scales."""

    def __init__(self, w_bf16: np.ndarray, double_quant: bool):
        w = np.asarray(w_bf16, dtype=np.float32)
        self.shape = w.shape
        self.numel = w.size
        codes, absmax = quantize_nf4(w)
        self.packed = pack_nibbles(codes)
        self.absmax = absmax
        self.double_quant = double_quant
        if double_quant:
            self.qabs, self.scale2, self.mean = double_quantize(absmax)
        else:
            self.qabs = self.scale2 = self.mean = None

    def effective_absmax(self) -> np.ndarray:
        if self.double_quant:
            return dq_decode(self.qabs, self.scale2, self.mean)
        return self.absmax

    def dequant(self) -> np.ndarray:
        codes = unpack_nibbles(self.packed, self.numel)
        return dequant_codes(codes, self.effective_absmax()).reshape(self.shape)

    def nbytes(self) -> int:
        n = self.packed.nbytes
        if self.double_quant:
            return n + self.qabs.nbytes + self.scale2.nbytes + 4
        return n + self.absmax.nbytes

