"""Pins of the generic chunked-loss oracle (CPU only).

The oracle (``oracle/chunked_oracle.py``) forms the full logits and applies a
row-additive loss; the pins check it against a closed form (zero weight),
torch CPU float64 autograd of the composite loss, central finite differences,
row-block independence, and, with a cross-entropy loss function, the separate
cross-entropy oracle.  A transposed contraction (G.T @ W, or G @ X), a dropped
factor 2 or a swapped weight in the weighted squared error fails one of them.
"""
import numpy as np
import pytest

import oracle


def _problem(n, h, v, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, h))
    w = rng.standard_normal((v, h)) * 0.4
    y = rng.standard_normal((n, v))
    r = rng.uniform(0.5, 1.5, n)
    f = rng.uniform(0.5, 1.5, v)
    return x, w, y, r, f


def test_zero_weight_closed_form():
    n, h, v = 4, 3, 5
    x, _, y, r, f = _problem(n, h, v)
    w = np.zeros((v, h))
    loss, gi, gw = oracle.weighted_mse(x, w, y, r, f)
    exp_loss = 0.0
    exp_gw = np.zeros((v, h))
    for i in range(n):
        for j in range(v):
            exp_loss += y[i, j] ** 2 * r[i] * f[j]
            for k in range(h):
                exp_gw[j, k] += -2.0 * y[i, j] * r[i] * f[j] * x[i, k]
    assert loss == pytest.approx(exp_loss, rel=1e-12)
    assert not gi.any()
    np.testing.assert_allclose(gw, exp_gw, rtol=1e-12, atol=1e-14)


def test_matches_torch_autograd_fp64():
    torch = pytest.importorskip("torch")
    x, w, y, r, f = _problem(7, 5, 11, seed=3)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    z = torch.nn.functional.linear(xt, wt)
    loss = (((z - torch.tensor(y)) ** 2) * torch.tensor(r)[:, None] * torch.tensor(f)[None, :]).sum()
    loss.backward()
    o_loss, gi, gw = oracle.weighted_mse(x, w, y, r, f)
    assert o_loss == pytest.approx(loss.item(), rel=1e-12)
    np.testing.assert_allclose(gi, xt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(gw, wt.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_finite_differences():
    x, w, y, r, f = _problem(3, 4, 5, seed=5)
    _, gi, gw = oracle.weighted_mse(x, w, y, r, f)
    eps = 1e-6
    for arr, grad in ((x, gi), (w, gw)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            fp = oracle.weighted_mse(x, w, y, r, f)[0]
            arr[idx] = old - eps
            fm = oracle.weighted_mse(x, w, y, r, f)[0]
            arr[idx] = old
            num[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


def test_row_blocks_do_not_matter():
    x, w, y, r, f = _problem(10, 3, 6, seed=7)
    a = oracle.weighted_mse(x, w, y, r, f, row_block=3)
    b = oracle.weighted_mse(x, w, y, r, f, row_block=1000)
    assert a[0] == pytest.approx(b[0], rel=1e-13)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-13)
    np.testing.assert_allclose(a[2], b[2], rtol=1e-12, atol=1e-14)


def test_cross_entropy_through_the_generic_path():
    """The generic path with a sum cross-entropy loss function equals the
    cross-entropy oracle (reduction sum, no bias, no cap)."""
    from scipy.special import logsumexp
    rng = np.random.default_rng(11)
    n, h, v = 9, 4, 13
    x = rng.standard_normal((n, h))
    w = rng.standard_normal((v, h)) * 0.5
    t = rng.integers(0, v, size=n).astype(np.int64)

    def ce(z, tt):
        lse = logsumexp(z, axis=1)
        loss = float(np.sum(lse - z[np.arange(len(tt)), tt]))
        g = np.exp(z - lse[:, None])
        g[np.arange(len(tt)), tt] -= 1.0
        return loss, g

    loss, gi, gw = oracle.chunked_linear_loss(x, w, ce, t, row_block=4)
    fwd, gh_ref, gw_ref, _ = oracle.forward_backward(x, w, None, t, np.array(1.0), reduction="sum")
    assert loss == pytest.approx(float(fwd.loss), rel=1e-12)
    np.testing.assert_allclose(gi, gh_ref, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(gw, gw_ref, rtol=1e-11, atol=1e-13)
