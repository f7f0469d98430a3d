"""Pins of the float64 oracle against facts that do not come from the oracle:
values the pages print, closed forms, a library routine for the special case
p = 1, brute force, finite differences and invariances.  CPU only."""

import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _problem(N=6, H=4, V=9, seed=0, n_ignored=2, p_const=None):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) * 0.7
    y = rng.integers(0, V, N)
    y[:n_ignored] = -100
    rng.shuffle(y)
    p = rng.uniform(0.05, 1.0, N) if p_const is None else np.full(N, p_const)
    return h, W, y, p


def _loss(h, W, y, p, **kw):
    return O.forward_backward(h, W, y, p, need_grads=False, **kw)["loss"]


# --------------------------------------------------------------- P1: W = 0
@pytest.mark.parametrize("V", [7, 1000])
def test_zero_weight_gives_log_V(V):
    h, _, y, _ = _problem(N=8, H=5, V=V, seed=1)
    W = np.zeros((V, 5))
    r = O.forward_backward(h, W, y, np.ones(8), reduction="mean")
    assert abs(r["loss"] - math.log(V)) < 4e-16 * math.log(V) * 4


@pytest.mark.parametrize("eps,s,red", [(0.0, 1.0, "mean"), (0.1, 0.5, "sum"), (0.3, 2.0, "mean")])
def test_zero_weight_closed_form(eps, s, red):
    N, H, V = 10, 3, 11
    h, _, y, p = _problem(N=N, H=H, V=V, seed=2, n_ignored=3)
    W = np.zeros((V, H))
    r = O.forward_backward(h, W, y, p, label_smoothing=eps, logit_scale=s, reduction=red)
    valid = y != -100
    D = valid.sum() if red == "mean" else 1.0
    assert r["loss"] == pytest.approx(math.log(V) * np.sum(1.0 / p[valid]) / D, rel=1e-14)
    # g_ij = s/(p_i D) ((1-eps)/V - (1-eps)[j=y_i]) -> dH = g W = 0, dW = g^T h
    g = np.zeros((N, V))
    for i in np.nonzero(valid)[0]:
        g[i, :] = s / (p[i] * D) * (1.0 - eps) / V
        g[i, y[i]] -= s / (p[i] * D) * (1.0 - eps)
    np.testing.assert_allclose(r["dW"], g.T @ h, rtol=1e-13, atol=1e-15)
    assert np.all(r["dH"] == 0.0)


# ------------------------------------------------------- P2: row sums of g
@pytest.mark.parametrize("eps", [0.0, 0.1, 0.7])
def test_dlogit_rows_sum_to_zero(eps):
    h, W, y, p = _problem(N=12, H=6, V=40, seed=3, n_ignored=4)
    z = O.scaled_logits(h, W, 0.7)
    lse = O.row_logsumexp(z)
    valid = y != -100
    g = O.dlogits(z, lse, np.where(valid, y, -1), p, valid, 5.0, eps, 0.7, 40)
    assert np.max(np.abs(g.sum(axis=1))) < 1e-14
    # and the target entry is the only negative one-hot contribution
    assert np.all(g[~valid] == 0.0)


# ------------------------------------------------------ P3: ignore semantics
def test_ignored_rows_are_inert():
    h, W, y, p = _problem(N=9, H=5, V=13, seed=4, n_ignored=3)
    kw = dict(label_smoothing=0.2, logit_scale=0.8, reduction="mean")
    a = O.forward_backward(h, W, y, p, **kw)
    ig = np.nonzero(y == -100)[0]
    h2, p2 = h.copy(), p.copy()
    h2[ig] = 1e3 * np.arange(1, 6)      # huge hidden rows
    p2[ig[0]] = 0.0                      # p = 0 on an ignored row must not matter
    p2[ig[1]] = np.nan
    b = O.forward_backward(h2, W, y, p2, **kw)
    assert a["loss"] == b["loss"]
    assert np.all(b["dH"][ig] == 0.0)
    assert np.all(b["row_loss"][ig] == 0.0)
    np.testing.assert_allclose(a["dW"], b["dW"], rtol=1e-14, atol=0)


def test_all_ignored_batch():
    h, W, y, p = _problem(N=4, H=3, V=5, seed=5, n_ignored=4)
    r = O.forward_backward(h, W, y, p)
    assert r["loss"] == 0.0 and np.all(r["dH"] == 0) and np.all(r["dW"] == 0)


# --------------------------------------------------- P4: finite differences
@pytest.mark.parametrize("eps,s,red", [(0.0, 1.0, "mean"), (0.1, 0.5, "mean"),
                                        (0.1, 0.5, "sum"), (0.25, 1.7, "sum")])
def test_finite_differences(eps, s, red):
    h, W, y, p = _problem(N=5, H=3, V=7, seed=6, n_ignored=1)
    kw = dict(label_smoothing=eps, logit_scale=s, reduction=red)
    r = O.forward_backward(h, W, y, p, **kw)
    d = 1e-6
    for arr, grad in ((h, r["dH"]), (W, r["dW"])):
        num = np.zeros_like(arr)
        for idx in np.ndindex(*arr.shape):
            old = arr[idx]
            arr[idx] = old + d
            lp = _loss(h, W, y, p, **kw)
            arr[idx] = old - d
            lm = _loss(h, W, y, p, **kw)
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * d)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


def test_literal_loss_reading_is_not_the_gradients_loss():
    """With eps > 0 and p != 1, the page's literal loss (smoothing term not
    divided by p) is not the function whose gradient the page computes; the
    reading taken (divide the whole smoothed CE) is.  With p = 1 they agree."""
    h, W, y, p = _problem(N=5, H=3, V=7, seed=7, n_ignored=1)
    kw = dict(label_smoothing=0.1, logit_scale=0.5, reduction="sum")
    r = O.forward_backward(h, W, y, p, **kw)
    assert abs(r["loss"] - r["loss_literal"]) > 1e-3
    r1 = O.forward_backward(h, W, y, np.ones(5), **kw)
    assert r1["loss"] == pytest.approx(r1["loss_literal"], rel=1e-15)

    d = 1e-6

    def lit(Wm):
        return O.forward_backward(h, Wm, y, p, need_grads=False, **kw)["loss_literal"]
    num = np.zeros_like(W)
    for idx in np.ndindex(*W.shape):
        Wp, Wm = W.copy(), W.copy()
        Wp[idx] += d
        Wm[idx] -= d
        num[idx] = (lit(Wp) - lit(Wm)) / (2 * d)
    assert np.max(np.abs(num - r["dW"])) > 1e-3


# ------------------------------------ P5: library special case (p = 1)
@pytest.mark.parametrize("eps,s,red", [(0.0, 1.0, "mean"), (0.1, 0.5, "mean"),
                                        (0.3, 1.5, "sum"), (0.0, 2.0, "sum")])
def test_matches_torch_cross_entropy_when_p_is_one(eps, s, red):
    torch = pytest.importorskip("torch")
    h, W, y, _ = _problem(N=16, H=8, V=50, seed=8, n_ignored=5)
    r = O.forward_backward(h, W, y, np.ones(16), label_smoothing=eps,
                           logit_scale=s, reduction=red)
    ht = torch.tensor(h, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    logits = s * (ht @ Wt.T)
    lt = torch.nn.functional.cross_entropy(logits, torch.tensor(y), ignore_index=-100,
                                           label_smoothing=eps, reduction=red)
    lt.backward()
    assert r["loss"] == pytest.approx(lt.item(), rel=1e-13)
    np.testing.assert_allclose(r["dH"], ht.grad.numpy(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(r["dW"], Wt.grad.numpy(), rtol=1e-11, atol=1e-14)


# ------------------------------------------------ P6: vocabulary shards
def test_page3_split_softmax_example():
    rows = {}
    with open(os.path.join(GOLDEN, "page3_split_softmax.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, *v = line.split()
                rows.setdefault(k, []).append([float(x) for x in v])
    pred = np.array(rows["predict"])
    table = np.array(rows["table"])
    n0, n1 = (int(x) for x in rows["shard_rows"][0])
    want = np.array(rows["row0_prob"][0])
    dec = int(rows["printed_decimals"][0][0])
    # the page's cosine normalisation of both operands (preprocessing, as printed)
    h = pred / np.linalg.norm(pred, axis=1, keepdims=True)
    Wn = table / np.linalg.norm(table, axis=1, keepdims=True)
    y = np.array([0, 3])
    parts = [O.shard_partials(h, Wn[:n0], y, 0, 1.0),
             O.shard_partials(h, Wn[n0:n0 + n1], y, n0, 1.0)]
    lse, _, _ = O.combine_shard_partials(parts)
    z = O.scaled_logits(h, Wn, 1.0)
    prob0 = np.exp(z[0] - lse[0])
    assert np.max(np.abs(prob0 - want)) <= 0.5 * 10.0 ** (-dec) + 1e-15
    # and the split result equals the single-device softmax
    assert np.max(np.abs(lse - O.row_logsumexp(z))) < 1e-15


@pytest.mark.parametrize("cuts", [[300, 750], [1, 2, 999], [500]])
def test_shard_combine_reproduces_full_vocab(cuts):
    N, H, V = 20, 6, 1000
    h, W, y, p = _problem(N=N, H=H, V=V, seed=9, n_ignored=6)
    eps, s = 0.1, 0.5
    full = O.forward_backward(h, W, y, p, label_smoothing=eps, logit_scale=s, reduction="sum")
    bounds = [0] + cuts + [V]
    parts = [O.shard_partials(h, W[a:b], y, a, s) for a, b in zip(bounds[:-1], bounds[1:])]
    lse, zt, zs = O.combine_shard_partials(parts)
    np.testing.assert_allclose(lse, full["lse"], rtol=1e-14)
    valid = y != -100
    rl = O.row_losses(lse, zt, zs, V, p, valid, eps)
    np.testing.assert_allclose(rl, full["row_loss"], rtol=1e-12, atol=1e-14)
    dH = np.zeros((N, H))
    dWs = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        dh, dw = O.shard_backward(h, W[a:b], y, p, lse, a, V, 1.0, eps, s)
        dH += dh
        dWs.append(dw)
    np.testing.assert_allclose(dH, full["dH"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(np.concatenate(dWs), full["dW"], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------- P7: invariances
def test_logit_scale_folds_into_weight():
    h, W, y, p = _problem(N=7, H=4, V=11, seed=10, n_ignored=2)
    s = 0.37
    a = O.forward_backward(h, W, y, p, logit_scale=s, label_smoothing=0.1)
    b = O.forward_backward(h, s * W, y, p, logit_scale=1.0, label_smoothing=0.1)
    assert a["loss"] == pytest.approx(b["loss"], rel=1e-14)
    np.testing.assert_allclose(a["dH"], b["dH"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(a["dW"], s * b["dW"], rtol=1e-12, atol=1e-15)


def test_vocab_and_row_permutations():
    h, W, y, p = _problem(N=8, H=5, V=12, seed=11, n_ignored=2)
    kw = dict(logit_scale=0.9, label_smoothing=0.05)
    a = O.forward_backward(h, W, y, p, **kw)
    perm = np.random.default_rng(0).permutation(12)          # new row k = old perm[k]
    inv = np.argsort(perm)
    y2 = np.where(y >= 0, inv[np.maximum(y, 0)], y)
    b = O.forward_backward(h, W[perm], y2, p, **kw)
    assert a["loss"] == pytest.approx(b["loss"], rel=1e-14)
    np.testing.assert_allclose(b["dW"], a["dW"][perm], rtol=1e-12, atol=1e-15)
    rp = np.random.default_rng(1).permutation(8)
    c = O.forward_backward(h[rp], W, y[rp], p[rp], **kw)
    assert a["loss"] == pytest.approx(c["loss"], rel=1e-14)
    np.testing.assert_allclose(c["dH"], a["dH"][rp], rtol=1e-12, atol=1e-15)


def test_row_blocking_does_not_change_results():
    h, W, y, p = _problem(N=23, H=5, V=17, seed=12, n_ignored=5)
    a = O.forward_backward(h, W, y, p, label_smoothing=0.1, row_block=1024)
    b = O.forward_backward(h, W, y, p, label_smoothing=0.1, row_block=4)
    assert a["loss"] == pytest.approx(b["loss"], rel=1e-14)
    np.testing.assert_allclose(a["dW"], b["dW"], rtol=1e-12, atol=1e-15)
    np.testing.assert_array_equal(a["dH"], b["dH"])


# ------------------------------------------------------------ P8: reduction
def test_mean_is_sum_over_divisor():
    h, W, y, p = _problem(N=10, H=4, V=9, seed=13, n_ignored=3)
    s_ = O.forward_backward(h, W, y, p, reduction="sum")
    m_ = O.forward_backward(h, W, y, p, reduction="mean")
    t_ = O.forward_backward(h, W, y, p, reduction="mean", total=10)
    assert m_["loss"] == pytest.approx(s_["loss"] / 7, rel=1e-14)
    assert t_["loss"] == pytest.approx(s_["loss"] / 10, rel=1e-14)
    np.testing.assert_allclose(m_["dW"], s_["dW"] / 7, rtol=1e-13)
    np.testing.assert_allclose(t_["dH"], s_["dH"] / 10, rtol=1e-13)
    with pytest.raises(ValueError):
        O.divisor(np.ones(3, bool), "none")


# ------------------------------------------------------ P9: brute force
def test_two_class_closed_form():
    h = np.array([[0.3, -1.2, 2.0]])
    W = np.array([[0.5, 0.1, -0.4], [-0.2, 0.8, 0.3]])
    for yv, p in ((0, 0.4), (1, 0.9)):
        r = O.forward_backward(h, W, np.array([yv]), np.array([p]), reduction="sum")
        z = h @ W.T
        other = 1 - yv
        want = math.log1p(math.exp(z[0, other] - z[0, yv])) / p
        assert r["loss"] == pytest.approx(want, rel=1e-14)
        # dlogit of the other class = sigmoid(z_o - z_y) / p, target = minus that
        sg = 1.0 / (1.0 + math.exp(-(z[0, other] - z[0, yv])))
        g = np.zeros(2)
        g[other], g[yv] = sg / p, -sg / p
        np.testing.assert_allclose(r["dW"], np.outer(g, h[0]), rtol=1e-13)


# ------------------------------------------- sampled helpers = full problem
def test_sampled_helpers_match_full():
    N, H, V = 30, 6, 50
    h, W, y, p = _problem(N=N, H=H, V=V, seed=14, n_ignored=9)
    kw = dict(label_smoothing=0.1, logit_scale=0.5)
    full = O.forward_backward(h, W, y, p, reduction="mean", total=N, **kw)
    rows = [0, 3, 17, 29]
    lse, zt, zs = O.row_stats(h, W, y, rows, 0.5)
    np.testing.assert_allclose(lse, full["lse"][rows], rtol=1e-14)
    np.testing.assert_allclose(O.dH_rows(h, W, y, p, lse, rows, N, 0.1, 0.5),
                               full["dH"][rows], rtol=1e-12, atol=1e-15)
    vr = [0, 7, 49] + [int(v) for v in y[y >= 0][:2]]
    np.testing.assert_allclose(O.dW_rows(h, W, y, p, full["lse"], vr, N, 0.1, 0.5),
                               full["dW"][vr], rtol=1e-12, atol=1e-15)
    # shard variants of dH_rows and dW_rows
    dh, dw = O.shard_backward(h, W[20:40], y, p, full["lse"], 20, V, N, 0.1, 0.5)
    np.testing.assert_allclose(
        O.dH_rows(h, W[20:40], y, p, full["lse"][rows], rows, N, 0.1, 0.5, V_global=V,
                  vocab_start=20), dh[rows], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(
        O.dW_rows(h, W[20:40], y, p, full["lse"], [0, 5, 19], N, 0.1, 0.5,
                  V_global=V, vocab_start=20),
        dw[[0, 5, 19]], rtol=1e-12, atol=1e-15)


def test_out_of_range_target_rejected():
    h, W, y, p = _problem(N=4, H=3, V=5, seed=15, n_ignored=0)
    y[1] = 5
    with pytest.raises(ValueError):
        O.forward_backward(h, W, y, p)


# ------------------------- page 1's bias, EOB weight and upstream gradient
def test_bias_is_an_extra_input_column():
    """h W^T + b equals [h, 1] [W, b]^T, so the bias path must reproduce the
    bias-free oracle on augmented inputs, and db must be the gradient of the
    appended weight column (g^T 1 = column sums of g)."""
    h, W, y, p = _problem(N=9, H=5, V=13, seed=21, n_ignored=3)
    b = np.random.default_rng(22).standard_normal(13)
    kw = dict(label_smoothing=0.2, logit_scale=0.7, reduction="mean")
    r = O.forward_backward(h, W, y, p, bias=b, **kw)
    ha = np.concatenate([h, np.ones((9, 1))], axis=1)
    Wa = np.concatenate([W, b[:, None]], axis=1)
    ra = O.forward_backward(ha, Wa, y, p, **kw)
    assert r["loss"] == pytest.approx(ra["loss"], rel=1e-14)
    np.testing.assert_allclose(r["dH"], ra["dH"][:, :5], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r["dW"], ra["dW"][:, :5], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r["db"], ra["dW"][:, 5], rtol=1e-12, atol=1e-15)
    assert O.forward_backward(h, W, y, p, **kw)["db"] is None


@pytest.mark.parametrize("eps,s,red", [(0.0, 1.0, "mean"), (0.1, 0.5, "sum")])
def test_bias_finite_differences(eps, s, red):
    h, W, y, p = _problem(N=5, H=3, V=7, seed=23, n_ignored=1)
    b = np.random.default_rng(24).standard_normal(7) * 0.5
    kw = dict(label_smoothing=eps, logit_scale=s, reduction=red)
    r = O.forward_backward(h, W, y, p, bias=b, **kw)
    d = 1e-6
    num = np.zeros(7)
    for j in range(7):
        bp, bm = b.copy(), b.copy()
        bp[j] += d
        bm[j] -= d
        num[j] = (_loss(h, W, y, p, bias=bp, **kw) - _loss(h, W, y, p, bias=bm, **kw)) / (2 * d)
    np.testing.assert_allclose(r["db"], num, rtol=1e-6, atol=1e-8)


def test_bias_matches_torch_linear_cross_entropy():
    torch = pytest.importorskip("torch")
    h, W, y, _ = _problem(N=12, H=6, V=40, seed=25, n_ignored=4)
    b = np.random.default_rng(26).standard_normal(40)
    r = O.forward_backward(h, W, y, np.ones(12), bias=b, label_smoothing=0.1,
                           logit_scale=0.5, reduction="mean")
    ht = torch.tensor(h, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True)
    lt = torch.nn.functional.cross_entropy(0.5 * torch.nn.functional.linear(ht, Wt, bt),
                                           torch.tensor(y), ignore_index=-100,
                                           label_smoothing=0.1, reduction="mean")
    lt.backward()
    assert r["loss"] == pytest.approx(lt.item(), rel=1e-13)
    np.testing.assert_allclose(r["dH"], ht.grad.numpy(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(r["dW"], Wt.grad.numpy(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(r["db"], bt.grad.numpy(), rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("w", [2.5, 0.0])
def test_eob_weight_scales_eob_rows(w):
    """EOB rows' loss is multiplied by the weight: with p = 1 it is torch's
    unreduced CE weighted per row, summed and divided by the non-ignored
    count; the divisor still counts the EOB rows."""
    torch = pytest.importorskip("torch")
    h, W, y, _ = _problem(N=14, H=6, V=20, seed=27, n_ignored=3)
    eob = 5
    y[[1, 4, 9]] = np.where(y[[1, 4, 9]] == -100, -100, eob)
    y[[2, 11]] = eob
    kw = dict(label_smoothing=0.1, logit_scale=0.8, reduction="mean")
    r = O.forward_backward(h, W, y, np.ones(14), eob_token_id=eob, eob_weight=w, **kw)
    ht = torch.tensor(h, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    ce = torch.nn.functional.cross_entropy(0.8 * (ht @ Wt.T), torch.tensor(y), ignore_index=-100,
                                           label_smoothing=0.1, reduction="none")
    wt = torch.tensor(np.where(y == eob, w, 1.0))
    lt = (ce * wt).sum() / float(np.count_nonzero(y != -100))
    lt.backward()
    assert r["loss"] == pytest.approx(lt.item(), rel=1e-13)
    np.testing.assert_allclose(r["dH"], ht.grad.numpy(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(r["dW"], Wt.grad.numpy(), rtol=1e-11, atol=1e-14)


def test_eob_weight_one_or_absent_changes_nothing():
    h, W, y, p = _problem(N=8, H=4, V=9, seed=28, n_ignored=2)
    y[3] = 4
    base = O.forward_backward(h, W, y, p)
    for kw in (dict(eob_token_id=4, eob_weight=1.0), dict(eob_token_id=None, eob_weight=3.0)):
        r = O.forward_backward(h, W, y, p, **kw)
        assert r["loss"] == base["loss"]
        assert np.array_equal(r["dH"], base["dH"]) and np.array_equal(r["dW"], base["dW"])


def test_scale_grads_follows_the_chain_rule():
    """Gradients of do * loss by central differences equal scale_grads(do, ...)
    of the unit-upstream gradients; do = 1 returns them untouched."""
    h, W, y, p = _problem(N=4, H=3, V=6, seed=29, n_ignored=1)
    b = np.random.default_rng(30).standard_normal(6)
    r = O.forward_backward(h, W, y, p, bias=b)
    same = O.scale_grads(1.0, r["dH"], r["dW"], r["db"])
    assert all(a is c for a, c in zip(same, (r["dH"], r["dW"], r["db"])))
    do = -1.75
    dH, dW, db = O.scale_grads(do, r["dH"], r["dW"], r["db"])
    d = 1e-6
    num = np.zeros_like(W)
    for idx in np.ndindex(*W.shape):
        Wp, Wm = W.copy(), W.copy()
        Wp[idx] += d
        Wm[idx] -= d
        num[idx] = do * (_loss(h, Wp, y, p, bias=b) - _loss(h, Wm, y, p, bias=b)) / (2 * d)
    np.testing.assert_allclose(dW, num, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dH, do * r["dH"], rtol=1e-15)
    np.testing.assert_allclose(db, do * r["db"], rtol=1e-15)
    assert O.scale_grads(2.0, None)[0] is None


def test_forward_only_closed_form_and_library():
    """The forward-only entry: W = 0 closed form (lse = log V, loss = log V
    sum(1/p)/D) and torch's cross-entropy for p = 1."""
    torch = pytest.importorskip("torch")
    h, W, y, p = _problem(N=10, H=5, V=11, seed=31, n_ignored=3)
    r0 = O.forward(h, np.zeros_like(W), y, p, reduction="sum")
    np.testing.assert_allclose(r0["lse"], math.log(11), rtol=1e-15)
    valid = y != -100
    assert r0["loss"] == pytest.approx(math.log(11) * np.sum(1 / p[valid]), rel=1e-14)
    r = O.forward(h, W, y, np.ones(10), label_smoothing=0.05, logit_scale=1.3, reduction="mean")
    lt = torch.nn.functional.cross_entropy(1.3 * torch.tensor(h @ W.T), torch.tensor(y),
                                           ignore_index=-100, label_smoothing=0.05)
    assert r["loss"] == pytest.approx(lt.item(), rel=1e-13)
    np.testing.assert_allclose(r["lse"], torch.logsumexp(1.3 * torch.tensor(h @ W.T), 1).numpy(),
                               rtol=1e-14)


def test_sampled_helpers_with_bias():
    N, H, V = 20, 5, 30
    h, W, y, p = _problem(N=N, H=H, V=V, seed=32, n_ignored=6)
    b = np.random.default_rng(33).standard_normal(V)
    full = O.forward_backward(h, W, y, p, bias=b, label_smoothing=0.1, logit_scale=0.5,
                              reduction="sum")
    rows = [1, 8, 19]
    lse, _, _ = O.row_stats(h, W, y, rows, 0.5, bias=b)
    np.testing.assert_allclose(lse, full["lse"][rows], rtol=1e-14)
    np.testing.assert_allclose(O.dH_rows(h, W, y, p, lse, rows, 1.0, 0.1, 0.5, bias=b),
                               full["dH"][rows], rtol=1e-12, atol=1e-15)
    vr = [0, 13, 29]
    dw, db = O.dW_rows(h, W, y, p, full["lse"], vr, 1.0, 0.1, 0.5, bias=b, with_db=True)
    np.testing.assert_allclose(dw, full["dW"][vr], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(db, full["db"][vr], rtol=1e-12, atol=1e-15)
