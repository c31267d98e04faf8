"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test checks the oracle against something it does not share code with:
closed forms, the torch CPU float64 library definition the quack page uses as
its reference (``linear_cross_entropy_func_ref``), central finite
differences, and invariants of the mathematics.  The list is chosen so that a
dropped term, a wrong sign, index or operand order anywhere in the oracle
fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle

IGN = -100


def _problem(n, h, v, *, seed=0, bias=True, ignore=(), wstd=0.3, bstd=0.5):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, h))
    w = rng.standard_normal((v, h)) * wstd
    b = rng.standard_normal(v) * bstd if bias else None
    t = rng.integers(0, v, size=n).astype(np.int64)
    for i in ignore:
        t[i] = IGN
    return x, w, b, t


def _grad_loss(reduction, n, seed=1):
    if reduction == "none":
        return np.random.default_rng(seed).standard_normal(n)
    return np.array(1.7)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
@pytest.mark.parametrize("z_loss", [0.0, 0.01])
@pytest.mark.parametrize("scale,cap", [(1.0, None), (0.5, 3.0)])
def test_zero_weights_closed_form(reduction, z_loss, scale, cap):
    """W = 0, b = 0: every logit is 0, so p = 1/V on every row."""
    n, h, v = 7, 5, 11
    x, _, _, t = _problem(n, h, v, ignore=(2, 5))
    w = np.zeros((v, h))
    b = np.zeros(v)
    g = _grad_loss(reduction, n)
    fwd, gh, gw, gb = oracle.forward_backward(x, w, b, t, g, logit_scale=scale, softcap=cap,
                                              z_loss=z_loss, reduction=reduction)
    lnv = math.log(v)
    valid = t != IGN
    nv = int(valid.sum())
    row = lnv + z_loss * lnv * lnv
    np.testing.assert_allclose(fwd.lse, lnv, rtol=1e-14)
    np.testing.assert_allclose(fwd.entropy, lnv, rtol=1e-12)
    np.testing.assert_allclose(fwd.row_loss, np.where(valid, row, 0.0), rtol=1e-14)
    assert (fwd.argmax == 0).all()                       # ties -> lowest index
    assert fwd.num_correct == int((t[valid] == 0).sum())
    assert fwd.entropy_sum == pytest.approx(nv * lnv, rel=1e-12)
    if reduction == "sum":
        assert float(fwd.loss) == pytest.approx(nv * row, rel=1e-13)
    elif reduction == "mean":
        assert float(fwd.loss) == pytest.approx(row, rel=1e-13)
    # gradients, written out with loops from dLoss/du_ij = s * c_i * ((1+2 lam lnV)/V - [j = t_i])
    c = np.zeros(n)
    for i in range(n):
        if valid[i]:
            if reduction == "none":
                c[i] = g[i]
            elif reduction == "sum":
                c[i] = float(g)
            else:
                c[i] = float(g) / nv
    exp_gw = np.zeros((v, h))
    exp_gb = np.zeros(v)
    for i in range(n):
        for j in range(v):
            d = scale * c[i] * ((1 + 2 * z_loss * lnv) / v - (1.0 if t[i] == j else 0.0))
            exp_gb[j] += d
            exp_gw[j] += d * x[i]
    np.testing.assert_allclose(gh, 0.0, atol=0)
    np.testing.assert_allclose(gw, exp_gw, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gb, exp_gb, rtol=1e-12, atol=1e-14)


def test_transform_order_and_softcap_closed_form():
    """Bias, then scale, then cap*tanh(./cap).  W = 0 so z_j = cap*tanh(s*b_j/cap).

    With s = 0.5, cap = 2 and b_1 = -b_2 = 4*atanh(1/2) the logits are exactly
    (0, 1, -1), so LSE = ln(1 + 2 cosh 1) and the row loss for target 0 is LSE.
    Scaling after the cap, or adding the bias after the scale, gives other numbers.
    """
    s, cap = 0.5, 2.0
    a = 4.0 * math.atanh(0.5)
    b = np.array([0.0, a, -a])
    x = np.ones((2, 4))
    w = np.zeros((3, 4))
    t = np.array([0, 1], dtype=np.int64)
    fwd = oracle.forward(x, w, b, t, logit_scale=s, softcap=cap, reduction="none")
    lse = math.log(1.0 + 2.0 * math.cosh(1.0))
    np.testing.assert_allclose(fwd.lse, [lse, lse], rtol=1e-14)
    np.testing.assert_allclose(fwd.row_loss, [lse, lse - 1.0], rtol=1e-14)
    np.testing.assert_allclose(fwd.target_logit, [0.0, 1.0], atol=1e-15)
    assert list(fwd.argmax) == [1, 1]
    # entropy of softmax(0, 1, -1): LSE - (e - 1/e)/(1 + e + 1/e)
    e = math.e
    ent = lse - (e - 1 / e) / (1 + e + 1 / e)
    np.testing.assert_allclose(fwd.entropy, [ent, ent], rtol=1e-13)


@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
def test_single_vocabulary_row_closed_form(reduction):
    """V = 1: p = 1 on every row, so LSE = z, the row loss is lam z^2, the entropy 0,
    the argmax 0, and dLoss/dz = 2 lam c z (the one-hot and p cancel).  Everything
    below is written out per row with math.tanh, not through the oracle's arrays."""
    n, h = 6, 4
    s, cap, lam = 0.8, 4.0, 0.05
    x, w, b, _ = _problem(n, h, 1, seed=3)
    t = np.zeros(n, dtype=np.int64)
    t[3] = IGN
    g = _grad_loss(reduction, n)
    fwd, gh, gw, gb = oracle.forward_backward(x, w, b, t, g, logit_scale=s, softcap=cap, z_loss=lam,
                                              reduction=reduction)
    valid = t != IGN
    nv = int(valid.sum())
    exp_gh = np.zeros((n, h))
    exp_gw = np.zeros((1, h))
    exp_gb = np.zeros(1)
    total = 0.0
    for i in range(n):
        u = sum(x[i, k] * w[0, k] for k in range(h)) + b[0]
        z = cap * math.tanh(s * u / cap)
        assert fwd.lse[i] == pytest.approx(z, rel=1e-13, abs=1e-15)
        assert fwd.entropy[i] == pytest.approx(0.0, abs=1e-14)
        assert fwd.argmax[i] == 0
        assert fwd.top2_gap[i] == math.inf
        if not valid[i]:
            assert fwd.row_loss[i] == 0.0
            continue
        assert fwd.row_loss[i] == pytest.approx(lam * z * z, rel=1e-12)
        total += lam * z * z
        c = float(g[i]) if reduction == "none" else (float(g) if reduction == "sum" else float(g) / nv)
        du = s * (1.0 - (z / cap) ** 2) * 2.0 * lam * c * z
        exp_gh[i] = du * w[0]
        exp_gw[0] += du * x[i]
        exp_gb[0] += du
    assert fwd.num_correct == nv
    if reduction == "sum":
        assert float(fwd.loss) == pytest.approx(total, rel=1e-12)
    elif reduction == "mean":
        assert float(fwd.loss) == pytest.approx(total / nv, rel=1e-12)
    np.testing.assert_allclose(gh, exp_gh, rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(gw, exp_gw, rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(gb, exp_gb, rtol=1e-11, atol=1e-15)


def test_z_loss_closed_form_uniform_logits():
    """With all logits equal to k the row loss is ln V + lam (k + ln V)^2."""
    v, k, lam = 6, 0.75, 0.1
    x = np.zeros((3, 2))
    w = np.zeros((v, 2))
    b = np.full(v, k)
    t = np.array([0, 3, IGN], dtype=np.int64)
    fwd = oracle.forward(x, w, b, t, z_loss=lam, reduction="sum")
    lse = k + math.log(v)
    assert float(fwd.loss) == pytest.approx(2 * (lse - k + lam * lse * lse), rel=1e-14)


def test_argmax_ties_lowest_index():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 3))
    w = rng.standard_normal((5, 3))
    w[3] = w[1]          # rows 1 and 3 always tie
    w[4] = w[1]
    fwd = oracle.forward(x, w, None, np.zeros(4, dtype=np.int64), reduction="sum")
    z = x @ w.T
    for i in range(4):
        best = max(range(5), key=lambda j: (z[i, j], -j))
        assert fwd.argmax[i] == best


def _identity_problem(rows):
    """Logits equal to the given rows: H = V, W = I, x = rows (so x.W^T = x exactly)."""
    x = np.asarray(rows, dtype=np.float64)
    v = x.shape[1]
    return x, np.eye(v), np.zeros(x.shape[0], dtype=np.int64)


@pytest.mark.parametrize("fn", ["forward", "full_pass_with_bias_grad"])
def test_top2_gap_and_row_max_closed_forms(fn):
    """top2_gap is the largest minus the second-largest logit of the row (0 on a
    tie), row_max the largest; rows chosen so both are exact binary fractions."""
    x, w, t = _identity_problem([[3.0, 1.0, 2.0],        # gap 1 (not 2: the runner-up is 2)
                                 [1.0, 3.0, 3.0],        # tie at the top: gap 0, argmax 1
                                 [-5.0, 2.0, 1.75],      # gap 0.25
                                 [0.5, 0.5, 0.5],        # all equal: gap 0, argmax 0
                                 [-1.0, -4.0, -0.5]])    # negative logits: gap 0.5
    if fn == "forward":
        fwd = oracle.forward(x, w, None, t, reduction="sum")
    else:
        fwd, _ = oracle.full_pass_with_bias_grad(x, w, None, t, np.array(1.0), reduction="sum")
    assert list(fwd.top2_gap) == [1.0, 0.0, 0.25, 0.0, 0.5]
    assert list(fwd.row_max) == [3.0, 3.0, 2.0, 0.5, -0.5]
    assert list(fwd.argmax) == [0, 1, 1, 0, 2]


def test_top2_gap_single_column_is_inf():
    x, w, t = _identity_problem([[0.25], [-7.0]])
    fwd = oracle.forward(x, w, None, t, reduction="sum")
    assert np.isinf(fwd.top2_gap).all() and (fwd.top2_gap > 0).all()
    assert list(fwd.row_max) == [0.25, -7.0]


def test_top2_gap_and_row_max_follow_the_transformed_logits():
    """Scale and cap apply before the metrics: with s = 2, cap = 3 the row
    u = (1, 0.5, -1) has z = 3 tanh(2u/3); with s = -1 the order reverses."""
    x, w, t = _identity_problem([[1.0, 0.5, -1.0]])
    fwd = oracle.forward(x, w, None, t, logit_scale=2.0, softcap=3.0, reduction="sum")
    assert fwd.row_max[0] == pytest.approx(3 * math.tanh(2 / 3), rel=1e-15)
    assert fwd.top2_gap[0] == pytest.approx(3 * (math.tanh(2 / 3) - math.tanh(1 / 3)), rel=1e-14)
    x, w, t = _identity_problem([[3.0, 1.0, 2.0]])
    fwd = oracle.forward(x, w, None, t, logit_scale=-1.0, reduction="sum")
    assert fwd.argmax[0] == 1 and fwd.row_max[0] == -1.0 and fwd.top2_gap[0] == 1.0


def test_row_max_against_brute_force():
    """Random rows: row_max and top2_gap equal a sort of the row's z, argmax its first maximum."""
    x, w, b, t = _problem(9, 4, 13, seed=8)
    fwd = oracle.forward(x, w, b, t, logit_scale=0.7, softcap=2.0, reduction="sum")
    for i in range(9):
        z = [2.0 * math.tanh(0.7 * (sum(x[i, k] * w[j, k] for k in range(4)) + b[j]) / 2.0)
             for j in range(13)]
        zs = sorted(z)
        assert fwd.row_max[i] == pytest.approx(zs[-1], rel=1e-13)
        assert fwd.top2_gap[i] == pytest.approx(zs[-1] - zs[-2], abs=1e-13)
        assert fwd.argmax[i] == z.index(zs[-1])


# ---------------------------------------------------------------- library special case

@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
@pytest.mark.parametrize("with_bias", [False, True])
def test_matches_torch_cross_entropy_fp64(reduction, with_bias):
    """scale 1, no cap, no z-loss: F.cross_entropy(F.linear(x, W, b)) in float64."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    n, h, v = 9, 6, 13
    x, w, b, t = _problem(n, h, v, bias=with_bias, ignore=(0, 4))
    g = _grad_loss(reduction, n)
    fwd, gh, gw, gb = oracle.forward_backward(x, w, b, t, g, reduction=reduction)
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True) if with_bias else None
    logits = F.linear(xt, wt, bt)
    ref = F.cross_entropy(logits, torch.tensor(t), ignore_index=IGN, reduction=reduction)
    ref.backward(torch.tensor(g) if reduction == "none" else torch.tensor(float(g), dtype=torch.float64))
    np.testing.assert_allclose(fwd.loss, ref.detach().numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(fwd.lse, torch.logsumexp(logits, 1).detach().numpy(), rtol=1e-13)
    np.testing.assert_allclose(gh, xt.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gw, wt.grad.numpy(), rtol=1e-12, atol=1e-14)
    if with_bias:
        np.testing.assert_allclose(gb, bt.grad.numpy(), rtol=1e-12, atol=1e-14)
    valid = t != IGN
    amax = logits.argmax(1).numpy()
    assert fwd.num_correct == int((valid & (amax == t)).sum())
    p = torch.softmax(logits, 1)
    ent = -(p * torch.log_softmax(logits, 1)).sum(1).detach().numpy()
    assert fwd.entropy_sum == pytest.approx(float(ent[valid].sum()), rel=1e-12)


def test_mean_with_no_valid_row():
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    x, w, b, t = _problem(3, 4, 5, ignore=(0, 1, 2))
    fwd, gh, gw, gb = oracle.forward_backward(x, w, b, t, np.array(1.0), reduction="mean")
    ref = F.cross_entropy(F.linear(torch.tensor(x), torch.tensor(w), torch.tensor(b)),
                          torch.tensor(t), ignore_index=IGN, reduction="mean")
    assert math.isnan(float(fwd.loss)) and math.isnan(float(ref))
    assert not gh.any() and not gw.any() and not gb.any()
    assert fwd.num_correct == 0 and fwd.entropy_sum == 0.0


# ---------------------------------------------------------------- finite differences

@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
def test_finite_differences(reduction):
    """Central differences of the scalar objective with every option switched on."""
    n, h, v = 5, 3, 7
    x, w, b, t = _problem(n, h, v, ignore=(3,), wstd=0.8, bstd=0.7)
    opts = dict(logit_scale=0.7, softcap=1.5, z_loss=0.05, reduction=reduction)
    g = _grad_loss(reduction, n)

    def objective(xx, ww, bb):
        loss = oracle.forward(xx, ww, bb, t, **opts).loss
        return float(np.sum(loss * g)) if reduction == "none" else float(loss) * float(g)

    _, gh, gw, gb = oracle.forward_backward(x, w, b, t, g, **opts)
    eps = 1e-6
    for arr, grad in ((x, gh), (w, gw), (b, gb)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            fp = objective(x, w, b)
            arr[idx] = old - eps
            fm = objective(x, w, b)
            arr[idx] = old
            num[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


# ---------------------------------------------------------------- invariants

def test_row_gradient_sums():
    """sum_j dLoss/dz_ij = 0 without z-loss and 2 lam c_i LSE_i with it."""
    n, h, v = 8, 5, 17
    x, w, b, t = _problem(n, h, v, ignore=(1,))
    g = np.array(2.5)
    for lam in (0.0, 0.02):
        fwd, _, _, gb = oracle.forward_backward(x, w, b, t, g, z_loss=lam, reduction="sum")
        coef = oracle.row_coefficients(t, g, reduction="sum")
        z = x @ w.T + b
        dz = oracle.logit_grad_block(z, fwd.lse, t, coef, z_loss=lam)
        np.testing.assert_allclose(dz.sum(1), 2 * lam * coef * fwd.lse, atol=1e-13)
        np.testing.assert_allclose(gb.sum(), (2 * lam * coef * fwd.lse).sum(), atol=1e-12)


def test_ignored_rows_contribute_nothing():
    n, h, v = 10, 4, 9
    x, w, b, t = _problem(n, h, v, ignore=(2, 3, 7))
    opts = dict(logit_scale=0.8, softcap=4.0, z_loss=0.01, reduction="sum")
    fwd, gh, gw, gb = oracle.forward_backward(x, w, b, t, np.array(1.0), **opts)
    keep = t != IGN
    sub, sgh, sgw, sgb = oracle.forward_backward(x[keep], w, b, t[keep], np.array(1.0), **opts)
    assert not gh[~keep].any()
    np.testing.assert_allclose(gh[keep], sgh, rtol=1e-13)
    np.testing.assert_allclose(gw, sgw, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(gb, sgb, rtol=1e-12, atol=1e-15)
    assert float(fwd.loss) == pytest.approx(float(sub.loss), rel=1e-14)
    assert fwd.num_correct == sub.num_correct
    assert fwd.entropy_sum == pytest.approx(sub.entropy_sum, rel=1e-14)
    np.testing.assert_array_equal(fwd.row_loss[~keep], 0.0)


def test_scale_folds_into_weight_and_bias():
    """Without a cap, scale s on (x.W^T + b) equals scale 1 on (x.(sW)^T + s b)."""
    n, h, v = 6, 5, 8
    x, w, b, t = _problem(n, h, v, ignore=(0,))
    s = 0.37
    g = np.array(1.3)
    f1, gh1, gw1, gb1 = oracle.forward_backward(x, w, b, t, g, logit_scale=s, z_loss=0.03)
    f2, gh2, gw2, gb2 = oracle.forward_backward(x, s * w, s * b, t, g, logit_scale=1.0, z_loss=0.03)
    np.testing.assert_allclose(f1.loss, f2.loss, rtol=1e-13)
    np.testing.assert_allclose(f1.lse, f2.lse, rtol=1e-13)
    np.testing.assert_allclose(gh1, gh2, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(gw1, s * gw2, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(gb1, s * gb2, rtol=1e-12, atol=1e-15)


def test_bias_shift_invariance():
    n, h, v = 6, 4, 10
    x, w, b, t = _problem(n, h, v, ignore=(5,))
    s, shift = 0.9, 3.25
    g = np.array(1.0)
    f1, gh1, gw1, gb1 = oracle.forward_backward(x, w, b, t, g, logit_scale=s)
    f2, gh2, gw2, gb2 = oracle.forward_backward(x, w, b + shift, t, g, logit_scale=s)
    np.testing.assert_allclose(f1.loss, f2.loss, rtol=1e-12)
    np.testing.assert_allclose(f2.lse, f1.lse + s * shift, rtol=1e-13)
    np.testing.assert_allclose(gh1, gh2, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(gw1, gw2, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(gb1, gb2, rtol=1e-10, atol=1e-13)


def test_huge_cap_is_no_cap():
    x, w, b, t = _problem(5, 4, 9)
    g = np.array(1.0)
    f1, gh1, gw1, _ = oracle.forward_backward(x, w, b, t, g, softcap=1e7)
    f2, gh2, gw2, _ = oracle.forward_backward(x, w, b, t, g, softcap=None)
    np.testing.assert_allclose(f1.loss, f2.loss, rtol=1e-12)
    np.testing.assert_allclose(gh1, gh2, rtol=1e-10)
    np.testing.assert_allclose(gw1, gw2, rtol=1e-10)


def test_reductions_agree():
    n, h, v = 12, 5, 7
    x, w, b, t = _problem(n, h, v, ignore=(1, 2, 9))
    none = oracle.forward(x, w, b, t, reduction="none")
    s = oracle.forward(x, w, b, t, reduction="sum")
    m = oracle.forward(x, w, b, t, reduction="mean")
    assert float(s.loss) == pytest.approx(none.loss.sum(), rel=1e-14)
    assert float(m.loss) == pytest.approx(none.loss.sum() / 9, rel=1e-14)
    # gradients: "none" with g_i = 1 equals "sum"; mean is sum / n_valid
    _, ghn, gwn, gbn = oracle.forward_backward(x, w, b, t, np.ones(n), reduction="none")
    _, ghs, gws, gbs = oracle.forward_backward(x, w, b, t, np.array(1.0), reduction="sum")
    _, ghm, gwm, gbm = oracle.forward_backward(x, w, b, t, np.array(1.0), reduction="mean")
    np.testing.assert_allclose(ghn, ghs, rtol=1e-14)
    np.testing.assert_allclose(gws / 9, gwm, rtol=1e-13)
    np.testing.assert_allclose(gbs / 9, gbm, rtol=1e-13, atol=1e-16)


def test_entropy_bounds():
    x, w, b, t = _problem(20, 6, 31, wstd=2.0)
    f = oracle.forward(x, w, b, t, softcap=5.0, reduction="sum")
    assert (f.entropy >= -1e-12).all() and (f.entropy <= math.log(31) + 1e-12).all()


def test_out_of_range_target_raises():
    x, w, b, t = _problem(3, 2, 4)
    t[1] = 4
    with pytest.raises(ValueError):
        oracle.forward(x, w, b, t)


# ---------------------------------------------------------------- sampled helpers

def test_sampled_and_full_pass_agree_with_full_gradients():
    n, h, v = 40, 8, 50
    x, w, b, t = _problem(n, h, v, ignore=(3, 11, 12))
    opts = dict(logit_scale=0.6, softcap=3.0, z_loss=0.02, reduction="none")
    g = _grad_loss("none", n)
    fwd, gh, gw, gb = oracle.forward_backward(x, w, b, t, g, **opts)
    rows = np.array([0, 3, 17, 39])
    vids = np.array([1, 5, 49, int(t[0])])
    sgh, sgw = oracle.sampled_gradients(x, w, b, t, g, fwd.lse, rows, vids, **opts)
    np.testing.assert_allclose(sgh, gh[rows], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(sgw, gw[vids], rtol=1e-12, atol=1e-15)
    f2, gb2 = oracle.full_pass_with_bias_grad(x, w, b, t, g, row_block=7, **opts)
    np.testing.assert_allclose(gb2, gb, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(f2.lse, fwd.lse, rtol=1e-14)
    np.testing.assert_allclose(f2.loss, fwd.loss, rtol=1e-14)
