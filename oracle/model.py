"""LoRA projection and Llama-style decoder layer in float64 (TEST INFRASTRUCTURE ONLY).

What is computed, and where the pages fix it:

* Every projection is Y = X W^T + s (X A^T) B^T with s = alpha / r: the frozen base W
  plus a trainable low-rank adapter (A [r, in], B [out, r]) kept in full precision
  ("Fine-Tuning an 8B Parameter Model on a 4 GB Laptop GPU", section "LoRA and QLoRA:
  Train a Fraction of the Parameters"; r and alpha from the lachieslifestyle.com
  how-to, section "Step 5: Enable 4-bit layer streaming").  Adapters sit on all seven
  projections q, k, v, o, gate, up, down.
* The layer is the pre-norm decoder of the Llama / Qwen families the pages list
  (same how-to, "Step 5"): RMSNorm, q/k/v, rotary embedding, causal grouped-query
  attention, o projection + residual, RMSNorm, SwiGLU MLP + residual.
* The base and the norm weights are frozen: backward returns dX and, for each
  projection, dA and dB only (same QLoRA section).

Readings where the pages are silent: no biases, no dropout; RMSNorm y = x g /
sqrt(mean(x^2) + eps); rotary embedding in the non-interleaved (rotate-half) form with
positions 0..S-1 inside each sequence and frequencies theta^(-2i/hd) (float64 here);
attention scale 1/sqrt(hd), causal mask only, GQA by sharing each kv head between
n_heads / n_kv_heads consecutive q heads; silu(z) = z / (1 + exp(-z)).

Layout: activations are token-major [T, features] with T = batch * seq and token
t = b * seq + s.  All arithmetic is float64.  The backward is derived by hand (chain
rule written out below); tests pin it against central finite differences.

Operand precision.  The pages give the compute dtype as bf16 (the QLoRA loading
example in "Fine-Tuning an 8B Parameter Model on a 4 GB Laptop GPU" sets a 16-bit
compute dtype for the 4-bit weights; its "Practical Advice" section recommends bf16),
and the LoRA adapters are kept in full precision.  The reading taken: every matrix
product takes bf16 operands (its inputs are rounded to bf16, nearest-even) and is
accumulated exactly; nothing else is rounded.  The functions below take ``rnd``:
the identity for exact arithmetic, or bf16 rounding for that reading.  The operands
are: the input of each projection, the adapters A and B, s*H (forward) and s*G
(backward), q and k after the rotary embedding, v, the probabilities P, and in the
backward the output gradient of each projection, dO and dS of the attention.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

PROJS = ("q", "k", "v", "o", "gate", "up", "down")


def _ident(x):
    return x


@dataclass(frozen=True)
class LayerShape:
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    rms_eps: float = 1e-5
    rope_theta: float = 1e4
    lora_r: int = 16
    lora_alpha: float = 32.0

    @property
    def scale(self) -> float:
        return float(self.lora_alpha) / float(self.lora_r)

    def proj_shape(self, p: str):
        """(out_features, in_features) of projection p."""
        h, q, kv, i = self.hidden, self.n_heads * self.head_dim, self.n_kv_heads * self.head_dim, self.intermediate
        return {"q": (q, h), "k": (kv, h), "v": (kv, h), "o": (h, q),
                "gate": (i, h), "up": (i, h), "down": (h, i)}[p]


# ------------------------------------------------------------------- primitives
def rmsnorm_fwd(x, g, eps):
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r * g, r


def rmsnorm_bwd(dn, x, g, r):
    """n_j = g_j x_j r with r = (sum x^2 / D + eps)^-1/2, so
    dx_j = r g_j dn_j - (r^3 / D) x_j sum_i dn_i g_i x_i."""
    d = x.shape[-1]
    gdn = dn * g
    return r * gdn - (r ** 3 / d) * x * np.sum(gdn * x, axis=-1, keepdims=True)


def rope_tables(seq, head_dim, theta):
    half = head_dim // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / head_dim)
    ang = np.arange(seq, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang), np.sin(ang)


def rope_fwd(x, cos, sin):
    """x [B, S, H, hd]; out1 = x1 cos - x2 sin, out2 = x2 cos + x1 sin."""
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    c, s = cos[None, :, None, :], sin[None, :, None, :]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_bwd(dy, cos, sin):
    """Transpose of the rotation: dx1 = d1 cos + d2 sin, dx2 = d2 cos - d1 sin."""
    half = dy.shape[-1] // 2
    d1, d2 = dy[..., :half], dy[..., half:]
    c, s = cos[None, :, None, :], sin[None, :, None, :]
    return np.concatenate([d1 * c + d2 * s, d2 * c - d1 * s], axis=-1)


def attention_fwd(q, k, v, n_rep, rnd=_ident):
    """q [B, S, Hq, hd], k/v [B, S, Hkv, hd] -> out [B, S, Hq, hd], probabilities P
    (P is the operand of the second product, so it is returned after ``rnd``)."""
    b, s, hq, hd = q.shape
    kk = np.repeat(k, n_rep, axis=2)
    vv = np.repeat(v, n_rep, axis=2)
    scores = np.einsum("bihd,bjhd->bhij", q, kk) / np.sqrt(hd)
    mask = np.triu(np.ones((s, s), dtype=bool), k=1)
    scores = np.where(mask[None, None], -np.inf, scores)
    scores = scores - np.max(scores, axis=-1, keepdims=True)
    p = np.exp(scores)
    p = rnd(p / np.sum(p, axis=-1, keepdims=True))
    out = np.einsum("bhij,bjhd->bihd", p, vv)
    return out, p


def attention_bwd(dout, q, k, v, p, n_rep, rnd=_ident):
    """dV = P^T dO; dP = dO V^T; dS = P (dP - rowsum(dP P)); dQ = c dS K; dK = c dS^T Q,
    with dK, dV summed over the q heads that share a kv head.  dO and c dS are the
    operands of the products (``rnd``)."""
    b, s, hq, hd = q.shape
    c = 1.0 / np.sqrt(hd)
    dout = rnd(dout)
    kk = np.repeat(k, n_rep, axis=2)
    vv = np.repeat(v, n_rep, axis=2)
    dvv = np.einsum("bhij,bihd->bjhd", p, dout)
    dp = np.einsum("bihd,bjhd->bhij", dout, vv)
    ds = rnd(c * (p * (dp - np.sum(dp * p, axis=-1, keepdims=True))))
    dq = np.einsum("bhij,bjhd->bihd", ds, kk)
    dkk = np.einsum("bhij,bihd->bjhd", ds, q)
    hkv = hq // n_rep
    dk = dkk.reshape(b, s, hkv, n_rep, hd).sum(axis=3)
    dv = dvv.reshape(b, s, hkv, n_rep, hd).sum(axis=3)
    return dq, dk, dv


def silu(z):
    return z / (1.0 + np.exp(-z))


def silu_grad(z):
    sg = 1.0 / (1.0 + np.exp(-z))
    return sg * (1.0 + z * (1.0 - sg))


# ------------------------------------------------------------------ projections
def lora_proj_fwd(x, w, a, b, s, lora_on=True, rnd=_ident):
    """Y = X W^T + (s X A^T) B^T with operands X, A, B and s X A^T passed through
    ``rnd``.  Returns (Y, Hs = s X A^T after ``rnd``, or None)."""
    x = rnd(x)
    y = x @ w.T
    if not lora_on:
        return y, None
    hs = rnd(s * (x @ rnd(a).T))
    return y + hs @ rnd(b).T, hs


def lora_proj_bwd(dy, x, w, a, b, hs, s, rnd=_ident):
    """Given dY for Y = X W^T + Hs B^T, Hs = s X A^T (W frozen), with G = dY B:
    dX = dY W + (s G) A; dB = dY^T Hs; dA = (s G)^T X.  dY, A, B, X and s G are
    operands (``rnd``)."""
    dy = rnd(dy)
    x = rnd(x)
    a = rnd(a)
    gs = rnd(s * (dy @ rnd(b)))
    dx = dy @ w + gs @ a
    db = dy.T @ hs
    da = gs.T @ x
    return dx, da, db


# ----------------------------------------------------------------------- layer
def layer_forward(x, weights, lora, shp: LayerShape, batch, seq, lora_on=True, rnd=_ident):
    """One decoder layer.  x [T, h] float64; weights: dict proj -> W [out, in] plus
    'g1', 'g2' [h]; lora: dict proj -> (A [r, in], B [out, r]).  ``rnd`` is applied
    to the operands of the matrix products.
    Returns (y, cache) where cache holds what the backward needs."""
    s = shp.scale
    hq, hkv, hd = shp.n_heads, shp.n_kv_heads, shp.head_dim
    t = batch * seq
    c = {"x": x}
    n1, r1 = rmsnorm_fwd(x, weights["g1"], shp.rms_eps)
    c["n1"], c["r1"] = n1, r1
    hs = {}
    outs = {}
    for p in ("q", "k", "v"):
        a, b = lora[p]
        outs[p], hs[p] = lora_proj_fwd(n1, weights[p], a, b, s, lora_on, rnd)
    cos, sin = rope_tables(seq, hd, shp.rope_theta)
    q = rnd(rope_fwd(outs["q"].reshape(batch, seq, hq, hd), cos, sin))
    k = rnd(rope_fwd(outs["k"].reshape(batch, seq, hkv, hd), cos, sin))
    v = rnd(outs["v"].reshape(batch, seq, hkv, hd))
    att, prob = attention_fwd(q, k, v, hq // hkv, rnd)
    att = att.reshape(t, hq * hd)
    c.update(q=q, k=k, v=v, prob=prob, att=att, cos=cos, sin=sin)
    a, b = lora["o"]
    o, hs["o"] = lora_proj_fwd(att, weights["o"], a, b, s, lora_on, rnd)
    h = x + o
    n2, r2 = rmsnorm_fwd(h, weights["g2"], shp.rms_eps)
    c.update(h=h, n2=n2, r2=r2)
    a, b = lora["gate"]
    gt, hs["gate"] = lora_proj_fwd(n2, weights["gate"], a, b, s, lora_on, rnd)
    a, b = lora["up"]
    up, hs["up"] = lora_proj_fwd(n2, weights["up"], a, b, s, lora_on, rnd)
    act = silu(gt) * up
    c.update(gt=gt, up=up, act=act)
    a, b = lora["down"]
    d, hs["down"] = lora_proj_fwd(act, weights["down"], a, b, s, lora_on, rnd)
    y = h + d
    c["hs"] = hs
    return y, c


def layer_backward(dy, cache, weights, lora, shp: LayerShape, batch, seq, rnd=_ident):
    """Backward of ``layer_forward`` (LoRA on).  Returns (dx, grads) with grads a dict
    proj -> (dA [r, in], dB [out, r])."""
    s = shp.scale
    hq, hkv, hd = shp.n_heads, shp.n_kv_heads, shp.head_dim
    t = batch * seq
    hs = cache["hs"]
    grads = {}
    # y = h + down(act)
    a, b = lora["down"]
    dact, da_, db_ = lora_proj_bwd(dy, cache["act"], weights["down"], a, b, hs["down"], s, rnd)
    grads["down"] = (da_, db_)
    dh = dy.copy()
    # act = silu(gt) * up
    gt, up = cache["gt"], cache["up"]
    dgt = dact * up * silu_grad(gt)
    dup = dact * silu(gt)
    a, b = lora["gate"]
    dn2_g, da_, db_ = lora_proj_bwd(dgt, cache["n2"], weights["gate"], a, b, hs["gate"], s, rnd)
    grads["gate"] = (da_, db_)
    a, b = lora["up"]
    dn2_u, da_, db_ = lora_proj_bwd(dup, cache["n2"], weights["up"], a, b, hs["up"], s, rnd)
    grads["up"] = (da_, db_)
    dh = dh + rmsnorm_bwd(dn2_g + dn2_u, cache["h"], weights["g2"], cache["r2"])
    # h = x + o(att)
    dx = dh.copy()
    a, b = lora["o"]
    datt, da_, db_ = lora_proj_bwd(dh, cache["att"], weights["o"], a, b, hs["o"], s, rnd)
    grads["o"] = (da_, db_)
    dq, dk, dv = attention_bwd(datt.reshape(batch, seq, hq, hd), cache["q"], cache["k"],
                               cache["v"], cache["prob"], hq // hkv, rnd)
    dq = rope_bwd(dq, cache["cos"], cache["sin"]).reshape(t, hq * hd)
    dk = rope_bwd(dk, cache["cos"], cache["sin"]).reshape(t, hkv * hd)
    dv = dv.reshape(t, hkv * hd)
    dn1 = np.zeros_like(cache["n1"])
    for p, dp in (("q", dq), ("k", dk), ("v", dv)):
        a, b = lora[p]
        dxp, da_, db_ = lora_proj_bwd(dp, cache["n1"], weights[p], a, b, hs[p], s, rnd)
        grads[p] = (da_, db_)
        dn1 = dn1 + dxp
    dx = dx + rmsnorm_bwd(dn1, cache["x"], weights["g1"], cache["r1"])
    return dx, grads
