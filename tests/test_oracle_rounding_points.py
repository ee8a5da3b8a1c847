"""Where the oracle's parity mode rounds to bf16, pinned by a second, independently
written implementation of one decoder layer (forward and backward) in scalar loops.

The reading being pinned: every matrix product takes bf16 operands and accumulates
exactly, nothing else is rounded (the pages fix a 16-bit compute dtype for the 4-bit
base, "Fine-Tuning an 8B Parameter Model on a 4 GB Laptop GPU", section "Quantization:
Shrink the Weights", and recommend bf16, section "Practical Advice Before You Start").
The operands, named as below:

  in   the input of each projection (n1, the attention output, n2, silu(g) u)
  A, B the adapters;  Hs = s X A^T (forward) and Gs = s dY B (backward)
  qk   q and k after the rotary embedding;  v
  P    the softmax probabilities (the normalised softmax is the operand of P V)
  dy   each projection's output gradient (dgate, dup, dh, dq, dk, dv, the layer's dY)
  dO   the attention output gradient
  cdS  the gradient of the product Q K^T, c dS with c = 1/sqrt(hd): the scores are
       S = c (Q K^T), so the backward products dQ = (c dS) K and dK = (c dS)^T Q take
       the gradient of that product as their operand

This module shares no code with ``oracle.model``: it rounds with its own float64 ->
bf16 routine and computes every sum as an explicit loop.  The test asserts that the
oracle equals this implementation with exactly the set above, that it differs from it
when any one of those roundings is dropped, and that it differs when any plausible
extra rounding is added (scores, residual, gate/up outputs, dP, d(act), the summed
input gradients, dq/dk before the inverse rotation) or a rounding is moved (dS rounded
before the scale c; the unnormalised exp(S - max) rounded instead of P).
"""
import math

import numpy as np
import pytest

from oracle import model as omodel
from oracle import nf4 as onf4

R7 = frozenset({"in", "A", "B", "Hs", "qk", "v", "P", "dy", "Gs", "dO", "cdS"})
EXTRA = ("S", "h", "gu", "dP", "dact", "dn", "dqk")
MOVED = ("dS_then_c", "P_unnorm")


def bf16(x: float) -> float:
    """Nearest bfloat16 value (8 significant bits, ties to even) of a float64."""
    if x == 0.0 or not math.isfinite(x):
        return x
    m, e = math.frexp(x)                  # x = m 2^e, 0.5 <= |m| < 1
    q = math.ldexp(1.0, max(e - 8, -133))
    return round(x / q) * q               # x / q is exact; round() is half-to-even


class Shape:
    # head_dim 6: c = 1/sqrt(6) is not a power of two, so rounding c dS and rounding dS
    # before the scale give different operands
    hidden, n_heads, n_kv_heads, head_dim, intermediate = 8, 2, 1, 6, 12
    eps, theta, r, alpha = 1e-5, 1e4, 2, 4.0


def loop_layer(x, W, lora, sh, batch, seq, dy, rounds):
    """Forward and backward of one layer.  x, dy: [T][h] lists; W[p]: [out][in];
    lora[p] = (A [r][in], B [out][r]).  ``rounds`` names the rounded tensors."""
    T, H, hq, hkv, hd, I = batch * seq, sh.hidden, sh.n_heads, sh.n_kv_heads, sh.head_dim, sh.intermediate
    s = sh.alpha / sh.r
    R = lambda name, v: bf16(v) if name in rounds else v

    def rms(rows, g):
        out, rs = [], []
        for row in rows:
            r = 1.0 / math.sqrt(sum(v * v for v in row) / len(row) + sh.eps)
            rs.append(r)
            out.append([row[i] * r * g[i] for i in range(len(row))])
        return out, rs

    def rms_back(dn, rows, g, rs):
        # n_i = g_i x_i r(x), dr/dx_j = -r^3 x_j / D
        out = []
        for t, row in enumerate(rows):
            r, D = rs[t], len(row)
            dot = sum(dn[t][i] * g[i] * row[i] for i in range(D))
            out.append([r * g[j] * dn[t][j] - r ** 3 / D * row[j] * dot for j in range(D)])
        return out

    def proj(X, p):
        w, (a, b) = W[p], lora[p]
        n_out, n_in = len(w), len(w[0])
        Xr = [[R("in", v) for v in row] for row in X]
        hs = [[R("Hs", s * sum(Xr[t][i] * R("A", a[j][i]) for i in range(n_in))) for j in range(sh.r)] for t in range(T)]
        y = [[sum(Xr[t][i] * w[o][i] for i in range(n_in)) + sum(hs[t][j] * R("B", b[o][j]) for j in range(sh.r))
              for o in range(n_out)] for t in range(T)]
        return y, (Xr, hs)

    def proj_back(dY, p, saved):
        w, (a, b) = W[p], lora[p]
        Xr, hs = saved
        n_out, n_in = len(w), len(w[0])
        D = [[R("dy", v) for v in row] for row in dY]
        G = [[R("Gs", s * sum(D[t][o] * R("B", b[o][j]) for o in range(n_out))) for j in range(sh.r)] for t in range(T)]
        dX = [[sum(D[t][o] * w[o][i] for o in range(n_out)) + sum(G[t][j] * R("A", a[j][i]) for j in range(sh.r))
               for i in range(n_in)] for t in range(T)]
        dB = [[sum(D[t][o] * hs[t][j] for t in range(T)) for j in range(sh.r)] for o in range(n_out)]
        dA = [[sum(G[t][j] * Xr[t][i] for t in range(T)) for i in range(n_in)] for j in range(sh.r)]
        return dX, dA, dB

    def angle(pos, i):
        return pos * sh.theta ** (-2.0 * i / hd)

    def rotate(vec, pos, inverse=False):
        half, out = hd // 2, list(vec)
        for i in range(half):
            c, sn = math.cos(angle(pos, i)), math.sin(angle(pos, i))
            if inverse:   # transpose of the rotation
                out[i], out[i + half] = vec[i] * c + vec[i + half] * sn, vec[i + half] * c - vec[i] * sn
            else:
                out[i], out[i + half] = vec[i] * c - vec[i + half] * sn, vec[i + half] * c + vec[i] * sn
        return out

    g1, g2 = W["g1"], W["g2"]
    n1, r1 = rms(x, g1)
    qf, sq = proj(n1, "q")
    kf, sk = proj(n1, "k")
    vf, sv = proj(n1, "v")
    pos = [t % seq for t in range(T)]
    Q = [[[R("qk", v) for v in rotate(qf[t][h * hd:(h + 1) * hd], pos[t])] for h in range(hq)] for t in range(T)]
    K = [[[R("qk", v) for v in rotate(kf[t][h * hd:(h + 1) * hd], pos[t])] for h in range(hkv)] for t in range(T)]
    V = [[[R("v", vf[t][h * hd + d]) for d in range(hd)] for h in range(hkv)] for t in range(T)]
    c = 1.0 / math.sqrt(hd)
    grp = hq // hkv
    P = {}           # (h, t) -> {u: P}
    att = [[0.0] * (hq * hd) for _ in range(T)]
    for t in range(T):
        b0 = t - pos[t]
        for h in range(hq):
            kh = h // grp
            keys = range(b0, t + 1)
            S = {u: R("S", c * sum(Q[t][h][d] * K[u][kh][d] for d in range(hd))) for u in keys}
            mx = max(S.values())
            e = {u: math.exp(S[u] - mx) for u in keys}
            z = sum(e.values())
            if "P_unnorm" in rounds:
                pr = {u: R("P", e[u]) for u in keys}
                P[(h, t)] = {u: e[u] / z for u in keys}
                for d in range(hd):
                    att[t][h * hd + d] = sum(pr[u] * V[u][kh][d] for u in keys) / z
            else:
                P[(h, t)] = {u: R("P", e[u] / z) for u in keys}
                for d in range(hd):
                    att[t][h * hd + d] = sum(P[(h, t)][u] * V[u][kh][d] for u in keys)
    of, so = proj(att, "o")
    hres = [[R("h", x[t][i] + of[t][i]) for i in range(H)] for t in range(T)]
    n2, r2 = rms(hres, g2)
    gf, sg = proj(n2, "gate")
    uf, su = proj(n2, "up")
    gf = [[R("gu", v) for v in row] for row in gf]
    uf = [[R("gu", v) for v in row] for row in uf]
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))
    act = [[gf[t][j] * sig(gf[t][j]) * uf[t][j] for j in range(I)] for t in range(T)]
    df, sd = proj(act, "down")
    y = [[hres[t][i] + df[t][i] for i in range(H)] for t in range(T)]

    grads = {}
    dact, *gd = proj_back(dy, "down", sd)
    grads["down"] = tuple(gd)
    dact = [[R("dact", v) for v in row] for row in dact]
    dg = [[dact[t][j] * uf[t][j] * sig(gf[t][j]) * (1.0 + gf[t][j] * (1.0 - sig(gf[t][j]))) for j in range(I)]
          for t in range(T)]
    du = [[dact[t][j] * gf[t][j] * sig(gf[t][j]) for j in range(I)] for t in range(T)]
    dng, *gg = proj_back(dg, "gate", sg)
    dnu, *gu = proj_back(du, "up", su)
    grads["gate"], grads["up"] = tuple(gg), tuple(gu)
    dn2 = [[R("dn", dng[t][i] + dnu[t][i]) for i in range(H)] for t in range(T)]
    back2 = rms_back(dn2, hres, g2, r2)
    dh = [[dy[t][i] + back2[t][i] for i in range(H)] for t in range(T)]
    datt, *go = proj_back(dh, "o", so)
    grads["o"] = tuple(go)
    dO = [[R("dO", v) for v in row] for row in datt]
    dQ = [[[0.0] * hd for _ in range(hq)] for _ in range(T)]
    dK = [[[0.0] * hd for _ in range(hkv)] for _ in range(T)]
    dV = [[[0.0] * hd for _ in range(hkv)] for _ in range(T)]
    for t in range(T):
        b0 = t - pos[t]
        for h in range(hq):
            kh = h // grp
            keys = range(b0, t + 1)
            pr = P[(h, t)]
            dP = {u: R("dP", sum(dO[t][h * hd + d] * V[u][kh][d] for d in range(hd))) for u in keys}
            rowdot = sum(pr[u] * dP[u] for u in keys)
            for u in keys:
                ds = pr[u] * (dP[u] - rowdot)
                cds = c * R("dS_then_c", ds) if "dS_then_c" in rounds else R("cdS", c * ds)
                for d in range(hd):
                    dQ[t][h][d] += cds * K[u][kh][d]
                    dK[u][kh][d] += cds * Q[t][h][d]
                    dV[u][kh][d] += pr[u] * dO[t][h * hd + d]
    dq = [sum(([R("dqk", v) for v in dQ[t][h]] for h in range(hq)), []) for t in range(T)]
    dk = [sum(([R("dqk", v) for v in dK[t][h]] for h in range(hkv)), []) for t in range(T)]
    dq = [sum((rotate(dq[t][h * hd:(h + 1) * hd], pos[t], True) for h in range(hq)), []) for t in range(T)]
    dk = [sum((rotate(dk[t][h * hd:(h + 1) * hd], pos[t], True) for h in range(hkv)), []) for t in range(T)]
    dv = [sum((dV[t][h] for h in range(hkv)), []) for t in range(T)]
    dn1 = [[0.0] * H for _ in range(T)]
    for p, dp, saved in (("q", dq, sq), ("k", dk, sk), ("v", dv, sv)):
        dxp, *gp = proj_back(dp, p, saved)
        grads[p] = tuple(gp)
        dn1 = [[dn1[t][i] + dxp[t][i] for i in range(H)] for t in range(T)]
    dn1 = [[R("dn", v) for v in row] for row in dn1]
    back1 = rms_back(dn1, x, g1, r1)
    dx = [[dh[t][i] + back1[t][i] for i in range(H)] for t in range(T)]
    return y, dx, grads


@pytest.fixture(scope="module")
def case():
    sh = Shape()
    batch, seq = 2, 3
    rng = np.random.default_rng(123)
    T = batch * seq
    H, qd, kvd, I = sh.hidden, sh.n_heads * sh.head_dim, sh.n_kv_heads * sh.head_dim, sh.intermediate
    dims = {"q": (qd, H), "k": (kvd, H), "v": (kvd, H), "o": (H, qd), "gate": (I, H), "up": (I, H), "down": (H, I)}
    # inputs and base weights are bf16 values (as the stack hands them in); the adapters
    # are float32 values that bf16 rounding changes
    W = {p: onf4.bf16_round(rng.standard_normal(d) * 0.5).astype(np.float64) for p, d in dims.items()}
    W["g1"] = np.ones(H)
    W["g2"] = np.ones(H)
    lora = {p: (rng.standard_normal((sh.r, d[1])).astype(np.float32).astype(np.float64) * 0.7,
                rng.standard_normal((d[0], sh.r)).astype(np.float32).astype(np.float64) * 0.7) for p, d in dims.items()}
    x = onf4.bf16_round(rng.standard_normal((T, H))).astype(np.float64)
    dy = onf4.bf16_round(rng.standard_normal((T, H))).astype(np.float64)
    shp = omodel.LayerShape(H, sh.n_heads, sh.n_kv_heads, sh.head_dim, I, sh.eps, sh.theta, sh.r, sh.alpha)
    rnd = lambda a: onf4.bf16_round(a).astype(np.float64)
    y, cache = omodel.layer_forward(x, W, lora, shp, batch, seq, True, rnd)
    dx, grads = omodel.layer_backward(dy, cache, W, lora, shp, batch, seq, rnd)
    ora = flatten(y, dx, grads)
    lists = dict(x=x.tolist(), W={k: v.tolist() for k, v in W.items()},
                 lora={p: (a.tolist(), b.tolist()) for p, (a, b) in lora.items()}, dy=dy.tolist())
    return sh, batch, seq, lists, ora


def flatten(y, dx, grads):
    """The layer's results as a list of float64 tensors: Y, dX, then dA, dB per projection."""
    parts = [np.asarray(y, np.float64), np.asarray(dx, np.float64)]
    for p in omodel.PROJS:
        parts += [np.asarray(grads[p][0], np.float64), np.asarray(grads[p][1], np.float64)]
    return parts


def run_loops(case, rounds):
    sh, batch, seq, L, _ = case
    y, dx, grads = loop_layer(L["x"], L["W"], L["lora"], sh, batch, seq, L["dy"], rounds)
    return flatten(y, dx, grads)


def max_rel(a, b):
    """Largest per-tensor difference, relative to that tensor's largest magnitude."""
    return max(float(np.max(np.abs(u - v)) / np.max(np.abs(v))) for u, v in zip(a, b))


def test_oracle_rounds_exactly_the_product_operands(case):
    got = run_loops(case, R7)
    assert max_rel(got, case[4]) < 1e-12


@pytest.mark.parametrize("name", sorted(R7))
def test_dropping_any_operand_rounding_is_seen(case, name):
    assert max_rel(run_loops(case, R7 - {name}), case[4]) > 1e-5, name


@pytest.mark.parametrize("name", EXTRA)
def test_an_extra_rounding_is_seen(case, name):
    assert max_rel(run_loops(case, R7 | {name}), case[4]) > 1e-5, name


def test_moved_roundings_are_seen(case):
    assert max_rel(run_loops(case, (R7 - {"cdS"}) | {"dS_then_c"}), case[4]) > 1e-5
    assert max_rel(run_loops(case, R7 | {"P_unnorm"}), case[4]) > 1e-5


def test_exact_mode_equals_loops_without_rounding(case):
    """The oracle's exact mode (no rounding) against the loops with an empty set: the
    same layer, only the summation order differs."""
    sh, batch, seq, L, _ = case
    W = {k: np.asarray(v) for k, v in L["W"].items()}
    lora = {p: (np.asarray(a), np.asarray(b)) for p, (a, b) in L["lora"].items()}
    shp = omodel.LayerShape(sh.hidden, sh.n_heads, sh.n_kv_heads, sh.head_dim, sh.intermediate, sh.eps, sh.theta,
                            sh.r, sh.alpha)
    x, dy = np.asarray(L["x"]), np.asarray(L["dy"])
    y, cache = omodel.layer_forward(x, W, lora, shp, batch, seq, True)
    dx, grads = omodel.layer_backward(dy, cache, W, lora, shp, batch, seq)
    assert max_rel(run_loops(case, frozenset()), flatten(y, dx, grads)) < 1e-12
