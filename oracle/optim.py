"""AdamW update of the trainable adapters (TEST INFRASTRUCTURE ONLY; see ``oracle/__init__``).

What the pages fix: only the adapters train, the base stays frozen ("Fine-Tuning an
8B Parameter Model on a 4 GB Laptop GPU" (codeinktechnologies.com), section "LoRA and
QLoRA: Train a Fraction of the Parameters"), and Adam keeps two extra tensors per
trained parameter (same page, the list of what makes training memory-hungry, item
"Optimizer states").  The pages print no update rule or hyperparameters.

Reading taken: Adam with decoupled weight decay (AdamW,
Loshchilov & Hutter, "Decoupled Weight Decay Regularization", Algorithm 2), with the
decay scaled by the learning rate as in the widely used PyTorch parametrisation:

    theta <- theta * (1 - lr * wd)
    m <- beta1 * m + (1 - beta1) * g
    v <- beta2 * v + (1 - beta2) * g^2
    m_hat = m / (1 - beta1^t),  v_hat = v / (1 - beta2^t)
    theta <- theta - lr * m_hat / (sqrt(v_hat) + eps)

t is the 1-based step count; m and v start at zero.  Everything here is float64; the
moments are returned so that several steps can be chained.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class AdamW:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01


def adamw_step(theta, grad, m, v, t: int, hp: AdamW):
    """One AdamW step (t >= 1).  Returns (theta, m, v) as new float64 arrays."""
    if t < 1:
        raise ValueError("the step count starts at 1")
    theta = np.asarray(theta, np.float64) * (1.0 - hp.lr * hp.weight_decay)
    g = np.asarray(grad, np.float64)
    m = hp.beta1 * np.asarray(m, np.float64) + (1.0 - hp.beta1) * g
    v = hp.beta2 * np.asarray(v, np.float64) + (1.0 - hp.beta2) * g * g
    m_hat = m / (1.0 - hp.beta1 ** t)
    v_hat = v / (1.0 - hp.beta2 ** t)
    theta = theta - hp.lr * m_hat / (np.sqrt(v_hat) + hp.eps)
    return theta, m, v


def first_step_closed_form(theta, grad, hp: AdamW):
    """t = 1 from zero moments: m_hat = g and v_hat = g^2 exactly, so the step is
    theta (1 - lr wd) - lr g / (|g| + eps)."""
    theta = np.asarray(theta, np.float64)
    g = np.asarray(grad, np.float64)
    return theta * (1.0 - hp.lr * hp.weight_decay) - hp.lr * g / (np.abs(g) + hp.eps)


def steady_gradient_limit(grad, hp: AdamW, t: int):
    """With the same gradient g at every step from zero moments, m = (1 - beta1^t) g and
    v = (1 - beta2^t) g^2, so every bias-corrected step is lr g / (|g| + eps) (plus the
    decay term).  Returns that per-step move, independent of t."""
    g = np.asarray(grad, np.float64)
    assert t >= 1 and math.isfinite(hp.lr)
    return hp.lr * g / (np.abs(g) + hp.eps)
