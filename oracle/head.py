"""Output head and training losses (TEST INFRASTRUCTURE ONLY; see ``oracle/__init__``).

What the pages fix:

* streaming bounds the weights, not the logits: the tool the pages describe keeps the
  whole logits tensor resident, 8.71 GB at batch 8 on a 152k-token vocabulary ("Soup
  CLI fine-tunes Llama-3.1-8B on a 4 GB laptop GPU ...", third and fifth paragraphs).
  The chunked head therefore computes exactly the full softmax, without ever holding
  [T, V];
* supervised fine-tuning on instruction / response records (the lachieslifestyle.com
  how-to, "Step 3: Prepare a small training dataset");
* preference training with DPO over the streamed base, whose reference model is the
  same base with the adapters switched off (the tesserapress piece, third paragraph).

Readings taken where the pages are silent:

* head = a final RMSNorm with frozen weight g_f, then logits = yn W^T with a frozen
  16-bit W [V, h] and no bias (QLoRA keeps the output layer in 16 bits);
* labels: one target id per token, or -100 for a token that carries no loss; the
  caller aligns targets with positions (the usual next-token shift);
* SFT loss = mean over labelled tokens of -log softmax(logits)[label];
* DPO (Rafailov et al., "Direct Preference Optimization", the DPO objective): sequences
  come in pairs, 2i chosen and 2i+1 rejected; a sequence's log-probability is the sum
  over its labelled tokens; loss = mean over pairs of
  -log sigmoid(beta [(pi_c - ref_c) - (pi_r - ref_r)]), with pi from the policy
  (adapters on) and ref from the reference pass (adapters off);
* precision (parity mode): yn and the logit gradient are rounded to bf16 as the operands
  of the two head products, the head is bf16 by construction; logits, the log-sum-exp and
  every sum are float64.

Gradients are written out by hand: with logp_t = z_t[label_t] - logsumexp(z_t) and
g_t = dL/dlogp_t, dz_t = g_t (onehot(label_t) - softmax(z_t)); SFT g_t = -1/N on
labelled tokens; DPO g_t = -beta sigmoid(-m_i) / P on the chosen sequence of pair i and
+beta sigmoid(-m_i) / P on the rejected one (m_i the pair's margin, P pairs).
"""
from __future__ import annotations

import numpy as np

from . import model

IGNORE = -100


def head_forward(y, g, w, eps, rnd=lambda x: x):
    """(yn as used by the product, rstd, logits) for hidden states y [T, h]."""
    yn, r = model.rmsnorm_fwd(np.asarray(y, np.float64), np.asarray(g, np.float64), eps)
    ynr = rnd(yn)
    return ynr, r, ynr @ np.asarray(w, np.float64).T


def log_softmax(z):
    z = np.asarray(z, np.float64)
    m = z.max(axis=-1, keepdims=True)
    return z - (m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True)))


def token_logp(logits, labels):
    """(logp per token, 0 where unlabelled; mask of labelled tokens)."""
    labels = np.asarray(labels)
    mask = labels != IGNORE
    lp = log_softmax(logits)
    idx = np.where(mask, labels, 0)
    return np.where(mask, lp[np.arange(len(labels)), idx], 0.0), mask


def seq_sums(tok, seq):
    return np.asarray(tok, np.float64).reshape(-1, seq).sum(axis=1)


def _dlogits(logits, labels, g_tok):
    p = np.exp(log_softmax(logits))
    d = -p * g_tok[:, None]
    rows = np.nonzero(np.asarray(labels) != IGNORE)[0]
    d[rows, np.asarray(labels)[rows]] += g_tok[rows]
    return d


def sft_loss(logits, labels, seq):
    """(loss, per-sequence logp sums, number of labelled tokens, dlogits)."""
    tok, mask = token_logp(logits, labels)
    n = int(mask.sum())
    loss = -tok.sum() / n
    g_tok = np.where(mask, -1.0 / n, 0.0)
    return loss, seq_sums(tok, seq), n, _dlogits(logits, labels, g_tok)


def dpo_loss(logits_pol, logits_ref, labels, seq, beta):
    """(loss, policy and reference per-sequence logp sums, pair margins, dlogits of the
    policy)."""
    tok_p, mask = token_logp(logits_pol, labels)
    tok_r, _ = token_logp(logits_ref, labels)
    pol, ref = seq_sums(tok_p, seq), seq_sums(tok_r, seq)
    if len(pol) % 2:
        raise ValueError("DPO needs an even number of sequences (chosen, rejected pairs)")
    margin = beta * ((pol[0::2] - ref[0::2]) - (pol[1::2] - ref[1::2]))
    P = len(margin)
    loss = np.mean(np.logaddexp(0.0, -margin))          # -log sigmoid(m)
    sig = 1.0 / (1.0 + np.exp(margin))                   # sigmoid(-m)
    coef = np.empty(2 * P)
    coef[0::2] = -beta * sig / P
    coef[1::2] = beta * sig / P
    g_tok = np.where(mask, np.repeat(coef, seq), 0.0)
    return loss, pol, ref, margin, _dlogits(logits_pol, labels, g_tok)


def head_backward(dlogits, w, y, g, r, rnd=lambda x: x):
    """dL/dy through the head product and the final RMSNorm (g frozen)."""
    dyn = rnd(dlogits) @ np.asarray(w, np.float64)
    return model.rmsnorm_bwd(dyn, np.asarray(y, np.float64), np.asarray(g, np.float64), r)
