"""Pins of the oracle's output head and losses against facts that do not come from it:
the library's cross entropy and its autograd, closed forms of the DPO objective,
an exact identity of the softplus, and central finite differences."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import head

T, V, H, SEQ = 12, 37, 16, 6


def _case(seed=0, ignore=(2, 7)):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, V)) * 2.0
    labels = rng.integers(0, V, T)
    labels[list(ignore)] = head.IGNORE
    return logits, labels


def test_sft_loss_and_gradient_match_torch_cross_entropy():
    logits, labels = _case()
    loss, seqsum, n, dz = head.sft_loss(logits, labels, SEQ)
    z = torch.tensor(logits, dtype=torch.float64, requires_grad=True)
    ref = F.cross_entropy(z, torch.tensor(labels), ignore_index=head.IGNORE, reduction="mean")
    ref.backward()
    assert n == T - 2
    assert abs(loss - ref.item()) < 1e-13
    np.testing.assert_allclose(dz, z.grad.numpy(), rtol=1e-12, atol=1e-15)
    per_tok = -F.cross_entropy(z.detach(), torch.tensor(labels), ignore_index=head.IGNORE, reduction="none").numpy()
    np.testing.assert_allclose(seqsum, per_tok.reshape(-1, SEQ).sum(1), rtol=1e-13)


def test_log_softmax_matches_torch_on_large_logits():
    z = np.array([[1000.0, 999.0, -1000.0], [-5.0, -5.0, -5.0]])
    np.testing.assert_allclose(head.log_softmax(z), F.log_softmax(torch.tensor(z), -1).numpy(), rtol=1e-13)


def test_dpo_equal_policy_and_reference_is_log2():
    """margin 0 => loss log 2, and every coefficient is -/+ beta sigmoid(0) / P = -/+ beta / (2P)."""
    logits, labels = _case(1)
    beta = 0.3
    loss, pol, ref, margin, dz = head.dpo_loss(logits, logits, labels, SEQ, beta)
    assert abs(loss - np.log(2.0)) < 1e-15 and np.all(margin == 0)
    # dz of a chosen token = -beta/(2P) (onehot - p); P = 1 pair here
    p = np.exp(head.log_softmax(logits))
    t = 0
    want = -beta / 2 * (np.eye(V)[labels[t]] - p[t])
    np.testing.assert_allclose(dz[t], want, rtol=1e-13, atol=1e-16)
    t = SEQ + 0   # first token of the rejected sequence
    np.testing.assert_allclose(dz[t], beta / 2 * (np.eye(V)[labels[t]] - p[t]), rtol=1e-13, atol=1e-16)


def test_dpo_swap_identity():
    """Swapping chosen and rejected negates every margin; softplus(m) - softplus(-m) = m,
    so the loss rises by exactly the mean margin."""
    rng = np.random.default_rng(2)
    lp, lr_ = rng.standard_normal((T, V)), rng.standard_normal((T, V))
    labels = rng.integers(0, V, T)
    beta = 0.7
    l1, _, _, m1, _ = head.dpo_loss(lp, lr_, labels, SEQ, beta)
    sw = np.concatenate([np.arange(SEQ, 2 * SEQ), np.arange(SEQ)])
    l2, _, _, m2, _ = head.dpo_loss(lp[sw], lr_[sw], labels[sw], SEQ, beta)
    np.testing.assert_allclose(m2, -m1, rtol=1e-14)
    assert abs((l2 - l1) - np.mean(m1)) < 1e-13


@pytest.mark.parametrize("beta", [0.1, 2.0])
def test_dpo_gradient_finite_differences(beta):
    rng = np.random.default_rng(3)
    lp, lr_ = rng.standard_normal((2 * SEQ, V)), rng.standard_normal((2 * SEQ, V))
    labels = rng.integers(0, V, 2 * SEQ)
    labels[4] = head.IGNORE
    _, _, _, _, dz = head.dpo_loss(lp, lr_, labels, SEQ, beta)
    eps = 1e-6
    for (t, j) in [(0, 3), (4, 5), (SEQ + 1, labels[SEQ + 1]), (2 * SEQ - 1, 0), (1, labels[1])]:
        a, b = lp.copy(), lp.copy()
        a[t, j] += eps
        b[t, j] -= eps
        fd = (head.dpo_loss(a, lr_, labels, SEQ, beta)[0] - head.dpo_loss(b, lr_, labels, SEQ, beta)[0]) / (2 * eps)
        assert abs(fd - dz[t, j]) < 1e-8, (t, j, fd, dz[t, j])


def test_head_backward_finite_differences():
    """SFT loss of head_forward(y) differentiated through the head product and the final
    RMSNorm, exact arithmetic."""
    rng = np.random.default_rng(4)
    y = rng.standard_normal((T, H))
    g = 1.0 + 0.1 * rng.standard_normal(H)
    w = rng.standard_normal((V, H)) * 0.3
    labels = rng.integers(0, V, T)
    eps_n = 1e-5

    def loss_of(yy):
        _, _, z = head.head_forward(yy, g, w, eps_n)
        return head.sft_loss(z, labels, SEQ)[0]

    yn, r, z = head.head_forward(y, g, w, eps_n)
    dz = head.sft_loss(z, labels, SEQ)[3]
    dy = head.head_backward(dz, w, y, g, r)
    h = 1e-6
    for (t, k) in [(0, 0), (3, 7), (11, 15), (6, 2)]:
        a, b = y.copy(), y.copy()
        a[t, k] += h
        b[t, k] -= h
        fd = (loss_of(a) - loss_of(b)) / (2 * h)
        assert abs(fd - dy[t, k]) < 1e-8, (t, k, fd, dy[t, k])


def test_dpo_needs_pairs():
    logits, labels = _case(5)
    with pytest.raises(ValueError):
        head.dpo_loss(logits[:SEQ * 1], logits[:SEQ * 1], labels[:SEQ], SEQ, 0.1)
