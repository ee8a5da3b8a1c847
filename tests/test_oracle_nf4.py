"""Pins of the oracle's NF4 encoding against facts that do not come from the oracle.

Each check is built so that a plausible slip in ``oracle/nf4.py`` (wrong delta, wrong
level count, a transposed nibble, a tie sent the wrong way, a dropped rounding step)
fails at least one of them.
"""
import math

import numpy as np
import pytest

from oracle import nf4


# ------------------------------------------------------------------ codebook pins
def _phi(x):
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def _phi_inv_bisect(p):
    """Standard-normal quantile by bisection on erfc (independent of scipy.ndtri)."""
    lo, hi = -40.0, 40.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if _phi(mid) < p:
            lo = mid
        else:
            hi = mid
        if hi - lo <= 0:
            break
    return 0.5 * (lo + hi)


def test_codebook_structure():
    lv = nf4.nf4_codebook()
    assert lv.dtype == np.float32 and lv.shape == (16,)
    assert np.all(np.diff(lv) > 0)
    assert lv[0] == -1.0 and lv[7] == 0.0 and lv[15] == 1.0
    # approximate values of three levels (from the normal quantile construction)
    assert abs(lv[14] - 0.7230) < 1e-4
    assert abs(lv[8] - 0.0796) < 1e-4
    assert abs(lv[1] - (-0.6962)) < 1e-4
    # asymmetric: 7 negative, 8 positive levels
    assert np.sum(lv < 0) == 7 and np.sum(lv > 0) == 8


def test_codebook_matches_bisection_quantiles():
    """Rebuild every level from erfc-bisected quantiles; must agree bitwise in float32."""
    d = (29.0 / 30.0 + 31.0 / 32.0) / 2.0
    c = _phi_inv_bisect(d)
    pos = [_phi_inv_bisect(d + i * (0.5 - d) / 8) / c for i in range(8)]
    neg = [-_phi_inv_bisect(d + i * (0.5 - d) / 7) / c for i in range(7)]
    ref = np.sort(np.array(pos + neg + [0.0], dtype=np.float64)).astype(np.float32)
    lv = nf4.nf4_codebook()
    # bisection is accurate to ~1e-15 absolute; float32 rounding hides that unless a
    # value sits on a rounding boundary, which the assert would reveal.
    assert np.array_equal(ref.view(np.uint32), lv.view(np.uint32))


def test_codebook_probabilities_equally_spaced():
    """Phi(level * Phi^-1(delta)) of the positive levels are equally spaced from delta
    toward 1/2 (step (1/2-delta)/8); the negative levels likewise with 7 steps."""
    lv = nf4.nf4_codebook().astype(np.float64)
    d = nf4.NF4_DELTA
    c = _phi_inv_bisect(d)
    pos = sorted(lv[lv > 0], reverse=True)
    p = np.array([_phi(v * c) for v in pos])
    assert np.allclose(np.diff(p), (0.5 - d) / 8, atol=2e-7)
    neg = sorted(-lv[lv < 0], reverse=True)
    p = np.array([_phi(v * c) for v in neg])
    assert np.allclose(np.diff(p), (0.5 - d) / 7, atol=2e-7)


def test_delta_is_exact():
    assert nf4.NF4_DELTA == 0.5 * (29.0 / 30.0 + 31.0 / 32.0)
    # a rounded delta (0.9677) would move levels by >1e-5: make sure the table is
    # sensitive to it, so the bisection test above really pins delta.
    c = _phi_inv_bisect(0.9677)
    alt = _phi_inv_bisect(0.9677 - 7 * (0.9677 - 0.5) / 8) / c
    assert abs(alt - nf4.nf4_codebook()[8]) > 1e-6


# ----------------------------------------------------------------------- bf16 pins
def _bf16_bits_trick(x32):
    """RNE float32 -> bf16 by the integer carry trick (finite inputs)."""
    u = x32.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (r << 16).astype(np.uint32).view(np.float32)


def test_bf16_round_float32_inputs():
    rng = np.random.default_rng(0)
    u = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    u[::3] = (u[::3] & 0xFFFF0000) | 0x8000          # exact ties
    x = u.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 3.0e38)]
    got = nf4.bf16_round(x)
    want = _bf16_bits_trick(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_bf16_round_float64_brute_force():
    """Between the two bf16 neighbours of x, pick the nearer (tie: even mantissa)."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal(20_000) * 10.0 ** rng.integers(-30, 30, size=20_000)
    got = nf4.bf16_round(x).astype(np.float64)
    x32 = x.astype(np.float32)
    for xi, gi, fi in zip(x, got, x32):
        # bf16 neighbours of |xi|: truncate float32 bits, then step one ulp either way
        u = int(np.array([abs(fi)], np.float32).view(np.uint32)[0]) & 0xFFFF0000
        cands = []
        for k in (-1, 0, 1):
            b = u + k * 0x10000
            if 0 <= b < 0x7F800000:
                cands.append(float(np.array([b], np.uint32).view(np.float32)[0]))
        mag = min(cands, key=lambda c: (abs(c - abs(xi)),
                                         (int(np.array([c], np.float32).view(np.uint32)[0]) >> 16) & 1))
        best = math.copysign(mag, xi)
        assert gi == best, (xi, gi, best)


# ------------------------------------------------------------------ quantiser pins
def _nearest_brute(n, lv):
    """argmin over the 16 levels of |n - level| in float64 (exact for float32 n),
    scanning from the top so that ties pick the higher index."""
    dist = np.abs(np.asarray(n, np.float64)[:, None] - lv.astype(np.float64)[None, :])
    return (15 - np.argmin(dist[:, ::-1], axis=1)).astype(np.uint8)


def test_nearest_level_equals_brute_force():
    lv = nf4.nf4_codebook()
    mids = (lv[:-1].astype(np.float64) + lv[1:].astype(np.float64)) / 2.0
    rng = np.random.default_rng(2)
    n = rng.uniform(-1, 1, size=1_000_000).astype(np.float32)
    # every float32 within a few ulps of each midpoint (covers exact ties)
    near = []
    for m in mids:
        f = np.float32(m)
        for k in range(-3, 4):
            f2 = f
            for _ in range(abs(k)):
                f2 = np.nextafter(f2, np.float32(np.sign(k) * 2))
            near.append(f2)
    n = np.concatenate([n, np.array(near, np.float32), lv, -lv])
    assert np.array_equal(nf4.nearest_level(n, lv), _nearest_brute(n, lv))


def test_exact_tie_goes_to_higher_index():
    lv = np.arange(16, dtype=np.float32) / 8 - 1          # midpoints exactly representable
    n = np.array([(lv[3] + lv[4]) / 2], np.float32)
    assert nf4.nearest_level(n, lv)[0] == 4
    assert _nearest_brute(n, lv)[0] == 4


def test_nibble_order():
    packed = nf4.pack_nibbles(np.array([1, 2, 3, 4, 15, 0], np.uint8))
    assert list(packed) == [0x12, 0x34, 0xF0]
    assert list(nf4.unpack_nibbles(packed, 6)) == [1, 2, 3, 4, 15, 0]
    assert list(nf4.pack_nibbles(np.array([5], np.uint8))) == [0x57]   # pad nibble 7


def test_block_absmax_and_codes_small_example():
    """Hand-worked block: values are bf16-exact multiples of the levels."""
    lv = nf4.nf4_codebook()
    am = np.float32(0.5)
    idx = np.arange(64) % 16
    x = nf4.bf16_round(lv[idx] * am)
    x[5] = am                                   # make the absmax element explicit
    codes, absmax = nf4.quantize_nf4(x)
    assert absmax[0] == am
    assert codes[5] == 15
    assert codes[0] == 0 and codes[7] == 7 and codes[15] == 15


def test_quantise_round_trip_and_error_bound():
    rng = np.random.default_rng(3)
    w = nf4.bf16_round(rng.standard_normal((96, 320)).astype(np.float32) * 0.02)
    codes, absmax = nf4.quantize_nf4(w)
    deq = nf4.dequant_codes(codes, absmax)
    codes2, absmax2 = nf4.quantize_nf4(deq)
    assert np.array_equal(absmax2, absmax)
    assert np.array_equal(codes2, codes)
    lv = nf4.nf4_codebook().astype(np.float64)
    half_gap = np.max(np.diff(lv)) / 2
    err = np.abs(w.reshape(-1).astype(np.float64) - deq.astype(np.float64))
    bound = np.repeat(absmax.astype(np.float64), 64) * (half_gap + 2.0 ** -8)
    assert np.all(err <= bound)


def test_blocks_straddle_rows_and_zero_block():
    rng = np.random.default_rng(4)
    w = nf4.bf16_round(rng.standard_normal((3, 40)).astype(np.float32))   # 120 = 64 + 56
    w[0, :] = w[0, :]
    codes, absmax = nf4.quantize_nf4(w)
    flat = w.reshape(-1)
    assert absmax.shape == (2,)
    assert absmax[0] == np.max(np.abs(flat[:64])) and absmax[1] == np.max(np.abs(flat[64:]))
    z = np.zeros((2, 64), np.float32)
    codes, absmax = nf4.quantize_nf4(z)
    assert np.all(codes == 7) and np.all(absmax == 0)
    assert np.all(nf4.dequant_codes(codes, absmax) == 0)


def test_dequant_definition_on_all_codes():
    """Every (code, absmax) pair: one float32 multiply, then RNE to bf16."""
    lv = nf4.nf4_codebook()
    rng = np.random.default_rng(5)
    am = rng.uniform(1e-3, 1.0, size=64).astype(np.float32)
    for c in range(16):
        got = nf4.dequant_codes(np.full(64 * 64, c, np.uint8), np.repeat(am, 64)[::64].copy())
        prod = np.float32(lv[c]) * am            # float32 multiply
        want = _bf16_bits_trick(prod.astype(np.float32))
        assert np.array_equal(got.reshape(64, 64)[:, 0].view(np.uint32), want.view(np.uint32))


# ------------------------------------------------------------ double quantisation
def test_double_quant_round_trip_bound():
    rng = np.random.default_rng(6)
    a = (np.abs(rng.standard_normal(1000)) * 0.03 + 0.02).astype(np.float32)
    q, s, mean = nf4.double_quantize(a)
    assert q.dtype == np.uint8 and s.shape == (4,)
    assert abs(float(mean) - math.fsum(map(float, a)) / a.size) <= abs(float(mean)) * 2 ** -23
    ahat = nf4.dq_decode(q, s, mean)
    sc = np.repeat(s.astype(np.float64), 256)[:1000]
    ulp = np.spacing(np.abs(ahat).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(a.astype(np.float64) - ahat) <= sc / 254 + 2 * ulp)
    # codes are in [-127, 127] and the group extreme maps to +-127
    c = q.astype(np.int8)
    assert c.min() >= -127 and c.max() <= 127
    assert np.all(np.max(np.abs(c[:256].astype(int))) == 127)


def test_double_quant_constant_group():
    a = np.full(300, 0.25, np.float32)
    q, s, mean = nf4.double_quantize(a)
    assert mean == np.float32(0.25) and np.all(s == 0) and np.all(q == 0)
    assert np.all(nf4.dq_decode(q, s, mean) == np.float32(0.25))


def test_dq_decode_two_roundings():
    """decode = fp32(fp32(fp32(c/127) * s) + mean); check one value by hand in fp32."""
    c = np.array([np.uint8(np.int8(-45).view(np.uint8))])
    s = np.array([0.0123], np.float32)
    mean = np.float32(0.0457)
    f = np.float32(np.float32(-45.0) / np.float32(127.0))
    want = np.float32(np.float32(f * s[0]) + mean)
    assert nf4.dq_decode(c, s, mean)[0] == want


def test_nf4_tensor_sizes():
    """Stored size: 4 bits per weight + 4 bytes per block (fp32 absmax), or with double
    quantisation 1 byte per block + 4 bytes per group of 256 blocks + 4 bytes mean."""
    w = np.zeros((128, 512), np.float32)
    t = nf4.NF4Tensor(w, double_quant=False)
    assert t.nbytes() == 128 * 512 // 2 + 4 * (128 * 512 // 64)
    t = nf4.NF4Tensor(w, double_quant=True)
    nb = 128 * 512 // 64
    assert t.nbytes() == 128 * 512 // 2 + nb + 4 * (-(-nb // 256)) + 4
