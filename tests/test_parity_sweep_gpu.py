"""Seeded sweep of small configurations, HIP path against the float64 oracle.

Thirty configurations drawn once from a fixed seed: sizes (N, H a multiple of
64 for bf16, V anywhere from 1 to 3000), dtype, label smoothing (0 to 1),
logit scale, reduction and divisor, chunk sizes that are and are not
multiples of 64, bias with db, the end-of-block weight, and ignore patterns
from none to all rows.  Each goes through fldce_fwd_bwd_ex (which
fldce_fwd_bwd equals bit for bit when no option is set) and is compared
element by element: loss, dH, dW, db, per-row lse; ignored rows exactly +0."""

import numpy as np
import pytest

import oracle as O
from lm_head_linear_bf16_amd import synth
from _helpers import GRAD_RTOL, LOSS_RTOL, grad_err, host, say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


def _draw_cases(n=30, seed=20251203):
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        dtype = "bf16" if rng.random() < 0.75 else "f32"
        B = int(rng.integers(1, 5))
        L = int(rng.integers(1, 200))
        H = int(rng.choice([64, 128, 192, 320])) if dtype == "bf16" else int(rng.integers(1, 200))
        V = int(rng.choice([1, 2, 63, 257, 1000, 2047, 3000]))
        cfg = dict(
            dtype=dtype, B=B, L=L, H=H, V=V,
            eps=float(rng.choice([0.0, 0.1, 0.37, 1.0])),
            s=float(rng.choice([0.5, 1.0, 1.7])),
            reduction=str(rng.choice(["mean", "sum"])),
            total_is_N=bool(rng.random() < 0.5),
            chunk=int(rng.choice([0, 0, 64, 100, 256, 333])),
            bias=bool(rng.random() < 0.4),
            eob_w=(None if rng.random() < 0.6 else float(rng.choice([0.0, 0.5, 3.0]))),
            ignore=str(rng.choice(["recipe", "recipe", "none", "all", "most"])),
            index=1000 + k,
        )
        cases.append(cfg)
    return cases


CASES = _draw_cases()


def _targets(w, mode, V):
    target, p_mask = synth.targets(w)
    target = target.copy()
    rng = np.random.default_rng([w.index, 77])
    if mode == "none":      # every row has a target
        ig = target == -100
        target[ig] = rng.integers(0, V, int(ig.sum()))
    elif mode == "all":
        target[:] = -100
    elif mode == "most":    # all but a handful
        keep = rng.choice(len(target), size=min(3, len(target)), replace=False)
        t = np.full_like(target, -100)
        t[keep] = rng.integers(0, V, len(keep))
        target = t
    return target, p_mask


@pytest.mark.parametrize("cfg", CASES, ids=[f"sweep{k:02d}" for k in range(len(CASES))])
def test_sweep(cfg):
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    w = synth.custom(f"sweep{cfg['index']}", cfg["B"], cfg["L"], cfg["H"], cfg["V"],
                     dtype=cfg["dtype"], index=cfg["index"], label_smoothing=cfg["eps"],
                     logit_scale=cfg["s"], reduction=cfg["reduction"],
                     total_is_N=cfg["total_is_N"])
    target, p_mask = _targets(w, cfg["ignore"], w.V)
    eob = None
    if cfg["eob_w"] is not None:
        eob = int(w.V // 2)
        valid = np.nonzero(target != -100)[0]
        target[valid[::3]] = eob
    h, W = synth.hidden(w), synth.weight(w)
    b = synth.bias(w) if cfg["bias"] else None
    say(f"case {cfg}")
    r = fldce.fldce_fwd_bwd_ex(to_dev(h, dev), to_dev(W, dev), torch.from_numpy(target).to(dev),
                               torch.from_numpy(p_mask).to(dev),
                               None if b is None else to_dev(b, dev),
                               label_smoothing=w.label_smoothing, logit_scale=w.logit_scale,
                               reduction=w.reduction, total=w.total, eob_token_id=eob,
                               eob_weight=1.0 if cfg["eob_w"] is None else cfg["eob_w"],
                               want_db=b is not None, chunk_rows=cfg["chunk"], row_stats=True)
    torch.cuda.synchronize()
    o = O.forward_backward(h.values, W.values, target, p_mask, label_smoothing=w.label_smoothing,
                           logit_scale=w.logit_scale, reduction=w.reduction,
                           total=w.total or None, bias=None if b is None else b.values,
                           eob_token_id=eob, eob_weight=1.0 if cfg["eob_w"] is None else cfg["eob_w"])
    got = float(r["loss"].item())
    if w.V == 1:
        # one class: every row's loss is lse - z_y = 0 up to rounding, and the
        # GPU's z_y (a dot product) and lse (the GEMM) round differently
        assert abs(got) <= 1e-5, got
    elif o["loss"] == 0.0:
        assert got == 0.0
    else:
        assert abs(got - o["loss"]) <= LOSS_RTOL[w.dtype] * abs(o["loss"]), (got, o["loss"])
    ig = target == -100
    assert np.all(host(r["dH"])[ig] == 0.0)
    assert np.all(host(r["row_loss"])[ig] == 0.0) and np.all(host(r["row_lse"])[ig] == 0.0)
    tol = GRAD_RTOL[w.dtype]
    errs = {"dH": grad_err(host(r["dH"]), o["dH"]), "dW": grad_err(host(r["dW"]), o["dW"])}
    if b is not None:
        errs["db"] = grad_err(host(r["db"]), o["db"])
    say(f"  loss {got:.7g} oracle {o['loss']:.7g}  errs {errs}")
    if w.V == 1:
        # one class: every gradient is 0 mathematically and only rounding is
        # left (the stored logit and lse differ in the last bits), so bound it
        # by the tolerance times the gradients' natural scale: c_i |W| for dH
        # rows, sum_i c_i |h_i| for dW, c_i = w_i s / (p_i D)
        valid = target != -100
        D = O.divisor(valid, w.reduction, w.total or None)
        wt = np.where((target == eob) if eob is not None else False, cfg["eob_w"] or 0.0, 1.0)
        c = np.where(valid, wt * w.logit_scale / (p_mask * D), 0.0)
        assert np.abs(host(r["dH"])).max() <= tol * c.max() * np.abs(W.values).max()
        assert np.abs(host(r["dW"])).max() <= tol * (c[:, None] * np.abs(h.values)).sum(axis=0).max()
    else:
        assert max(errs.values()) <= tol, errs
    valid = ~ig
    np.testing.assert_allclose(host(r["row_lse"])[valid], o["lse"][valid], rtol=0,
                               atol=2e-3 if w.dtype == "bf16" else 2e-5)
