"""The rest of page 1's interface on the HIP path, against the float64 oracle
through the C ABI: the bias and db, the end-of-block weight, the forward-only
loss, the upstream-gradient scaling and the autograd wrapper.  Sizes span
several 256-wide tiles with ragged tails; a full-size 4b case with a bias
uses the stored full-vocabulary row statistics."""

import os

import numpy as np
import pytest

import oracle as O
from lm_head_linear_bf16_amd import synth
from _helpers import GOLDEN, GRAD_RTOL, LOSS_RTOL, grad_err, host, say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


def _eob_targets(target, eob, frac=0.2, seed=5):
    """Turn about `frac` of the non-ignored targets into the EOB token."""
    t = target.copy()
    v = np.nonzero(t != -100)[0]
    pick = np.random.default_rng(seed).choice(v, max(1, int(frac * len(v))), replace=False)
    t[pick] = eob
    return t


def _inputs(w, with_bias, dev):
    torch = torch_cuda()
    target, p_mask = synth.targets(w)
    h, W = synth.hidden(w), synth.weight(w)
    b = synth.bias(w) if with_bias else None
    return (target, p_mask, h, W, b, to_dev(h, dev), to_dev(W, dev),
            None if b is None else to_dev(b, dev))


def _check_loss(w, got, want):
    if want == 0.0:
        assert got == 0.0
    else:
        assert abs(got - want) <= LOSS_RTOL[w.dtype] * abs(want), (got, want)


EXT_CASES = [
    # name, workload, bias, db, eob weight (None = no EOB), chunk rows
    ("bias_bf16", synth.custom("bias_bf16", 3, 171, 192, 2053, label_smoothing=0.1,
                               logit_scale=0.5), True, True, None, 0),
    ("bias_eob_bf16", synth.custom("bias_eob_bf16", 2, 320, 256, 4099, label_smoothing=0.3,
                                   logit_scale=1.7, total_is_N=False), True, True, 2.5, 0),
    ("bias_chunked_bf16", synth.custom("bias_chunked_bf16", 7, 100, 128, 1500,
                                       label_smoothing=0.1, logit_scale=0.5), True, True, None, 256),
    ("db_no_bias_bf16", synth.custom("db_no_bias_bf16", 3, 100, 128, 1000), False, True, None, 0),
    ("eob_zero_bf16", synth.custom("eob_zero_bf16", 3, 100, 128, 1000, reduction="sum"),
     False, False, 0.0, 0),
    ("bias_eob_f32", synth.custom("bias_eob_f32", 2, 64, 64, 1000, dtype="f32",
                                  label_smoothing=0.1, logit_scale=0.5), True, True, 3.0, 0),
    ("bias_chunked_f32", synth.custom("bias_chunked_f32", 5, 70, 80, 777, dtype="f32",
                                      label_smoothing=0.2), True, True, None, 64),
]


@pytest.mark.parametrize("case", EXT_CASES, ids=lambda c: c[0])
def test_fwd_bwd_ex(case):
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    name, w, with_bias, want_db, eob_w, chunk = case
    dev = torch.device("cuda:0")
    target, p_mask, h, W, b, hd, Wd, bd = _inputs(w, with_bias, dev)
    eob = None
    if eob_w is not None:
        eob = 17
        target = _eob_targets(target, eob)
    say(f"case {name}: N={w.N} H={w.H} V={w.V} {w.dtype} bias={with_bias} db={want_db} "
        f"eob_w={eob_w} chunk={chunk}")
    r = fldce.fldce_fwd_bwd_ex(hd, Wd, torch.from_numpy(target).to(dev),
                               torch.from_numpy(p_mask).to(dev), bd,
                               label_smoothing=w.label_smoothing, logit_scale=w.logit_scale,
                               reduction=w.reduction, total=w.total, eob_token_id=eob,
                               eob_weight=1.0 if eob_w is None else eob_w, want_db=want_db,
                               chunk_rows=chunk, row_stats=True)
    torch.cuda.synchronize()
    o = O.forward_backward(h.values, W.values, target, p_mask, label_smoothing=w.label_smoothing,
                           logit_scale=w.logit_scale, reduction=w.reduction,
                           total=w.total or None, bias=None if b is None else b.values,
                           eob_token_id=eob, eob_weight=1.0 if eob_w is None else eob_w)
    _check_loss(w, float(r["loss"].item()), o["loss"])
    ig = target == -100
    assert np.all(host(r["dH"])[ig] == 0.0)
    tol = GRAD_RTOL[w.dtype]
    e = [grad_err(host(r["dH"]), o["dH"]), grad_err(host(r["dW"]), o["dW"])]
    if want_db:
        # oracle db for a bias-free call is the same column sum of g
        db_want = o["db"] if o["db"] is not None else O.forward_backward(
            h.values, W.values, target, p_mask, label_smoothing=w.label_smoothing,
            logit_scale=w.logit_scale, reduction=w.reduction, total=w.total or None,
            bias=np.zeros(w.V), eob_token_id=eob,
            eob_weight=1.0 if eob_w is None else eob_w)["db"]
        e.append(grad_err(host(r["db"]), db_want))
    else:
        assert r["db"] is None
    say(f"  loss {float(r['loss'].item()):.7g} oracle {o['loss']:.7g}  grad errs {e}")
    assert max(e) <= tol
    valid = ~ig
    np.testing.assert_allclose(host(r["row_lse"])[valid], o["lse"][valid], rtol=0,
                               atol=2e-3 if w.dtype == "bf16" else 2e-5)
    if eob_w == 0.0:
        rows = target == eob
        assert np.all(host(r["dH"])[rows] == 0.0) and np.all(host(r["row_loss"])[rows] == 0.0)


def test_fwd_bwd_plain_equals_ex_without_options():
    """fldce_fwd_bwd is fldce_fwd_bwd_ex with no bias, no db, no EOB: bitwise."""
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    w = synth.custom("plain_vs_ex", 3, 100, 128, 1000, label_smoothing=0.1)
    target, p_mask, _, _, _, hd, Wd, _ = _inputs(w, False, dev)
    t, p = torch.from_numpy(target).to(dev), torch.from_numpy(p_mask).to(dev)
    say("case plain_vs_ex")
    a = fldce.fldce_fwd_bwd(hd, Wd, t, p, label_smoothing=0.1, total=w.total)
    b = fldce.fldce_fwd_bwd_ex(hd, Wd, t, p, None, label_smoothing=0.1, total=w.total)
    torch.cuda.synchronize()
    assert torch.equal(a["loss"], b["loss"])
    assert torch.equal(a["dH"], b["dH"]) and torch.equal(a["dW"], b["dW"])


FWD_CASES = [
    ("fwd_bf16", synth.custom("fwd_bf16", 3, 171, 192, 2053, label_smoothing=0.1,
                              logit_scale=0.5), False, None),
    ("fwd_bias_eob_bf16", synth.custom("fwd_bias_eob_bf16", 2, 320, 256, 4099,
                                       label_smoothing=0.3, total_is_N=False), True, 2.0),
    ("fwd_f32", synth.custom("fwd_f32", 2, 64, 64, 1000, dtype="f32"), False, None),
    ("fwd_bias_f32", synth.custom("fwd_bias_f32", 3, 50, 96, 555, dtype="f32",
                                  label_smoothing=0.2, logit_scale=0.7), True, 0.5),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: c[0])
def test_forward_only(case):
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    name, w, with_bias, eob_w = case
    dev = torch.device("cuda:0")
    target, p_mask, h, W, b, hd, Wd, bd = _inputs(w, with_bias, dev)
    eob = None
    if eob_w is not None:
        eob = 3
        target = _eob_targets(target, eob)
    say(f"case {name}: N={w.N} H={w.H} V={w.V} {w.dtype} bias={with_bias} eob_w={eob_w}")
    r = fldce.fldce_fwd(hd, Wd, torch.from_numpy(target).to(dev),
                        torch.from_numpy(p_mask).to(dev), bd, label_smoothing=w.label_smoothing,
                        logit_scale=w.logit_scale, reduction=w.reduction, total=w.total,
                        eob_token_id=eob, eob_weight=1.0 if eob_w is None else eob_w,
                        row_stats=True)
    torch.cuda.synchronize()
    o = O.forward(h.values, W.values, target, p_mask, label_smoothing=w.label_smoothing,
                  logit_scale=w.logit_scale, reduction=w.reduction, total=w.total or None,
                  bias=None if b is None else b.values, eob_token_id=eob,
                  eob_weight=1.0 if eob_w is None else eob_w)
    _check_loss(w, float(r["loss"].item()), o["loss"])
    valid = target != -100
    atol = 2e-3 if w.dtype == "bf16" else 2e-5
    np.testing.assert_allclose(host(r["row_lse"])[valid], o["lse"][valid], rtol=0, atol=atol)
    assert np.all(host(r["row_lse"])[~valid] == 0.0) and np.all(host(r["row_loss"])[~valid] == 0.0)
    rl = host(r["row_loss"])
    np.testing.assert_allclose(rl, o["row_loss"], rtol=5e-3 if w.dtype == "bf16" else 1e-5,
                               atol=atol)


def test_forward_only_matches_fwd_bwd_loss():
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    w = synth.custom("fwd_vs_fwdbwd", 4, 96, 128, 777, label_smoothing=0.1, logit_scale=0.5)
    target, p_mask, _, _, _, hd, Wd, _ = _inputs(w, False, dev)
    t, p = torch.from_numpy(target).to(dev), torch.from_numpy(p_mask).to(dev)
    say("case fwd_vs_fwdbwd")
    a = fldce.fldce_fwd(hd, Wd, t, p, label_smoothing=0.1, logit_scale=0.5, total=w.total,
                        row_stats=True)
    b = fldce.fldce_fwd_bwd(hd, Wd, t, p, label_smoothing=0.1, logit_scale=0.5, total=w.total,
                            row_stats=True)
    torch.cuda.synchronize()
    # same kernels up to the z store: per-row lse and losses agree bit for bit
    assert torch.equal(a["row_lse"], b["row_lse"]) and torch.equal(a["row_loss"], b["row_loss"])
    assert torch.equal(a["loss"], b["loss"])


def test_forward_only_edges():
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    say("case fwd edges: N = 0, all ignored")
    W = torch.zeros(300, 128, dtype=torch.bfloat16, device=dev)
    h = torch.zeros(0, 128, dtype=torch.bfloat16, device=dev)
    r = fldce.fldce_fwd(h, W, torch.zeros(0, dtype=torch.int64, device=dev))
    torch.cuda.synchronize()
    assert float(r["loss"].item()) == 0.0
    h = torch.randn(70, 128, device=dev).to(torch.bfloat16)
    t = torch.full((70,), -100, dtype=torch.int64, device=dev)
    r = fldce.fldce_fwd(h, W, t, row_stats=True)
    torch.cuda.synchronize()
    assert float(r["loss"].item()) == 0.0
    assert float(r["row_lse"].abs().max()) == 0.0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_scale_grads(dtype):
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(3)
    xs = [torch.randn(n, generator=g).to(td) for n in (1003, 64 * 33, 7)]
    say(f"case scale_grads {dtype}")
    dev_xs = [x.to(dev) for x in xs]
    one = torch.ones(1, dtype=torch.float32, device=dev)
    fldce.fldce_scale_grads(one, *dev_xs)
    torch.cuda.synchronize()
    for a, b in zip(dev_xs, xs):
        assert torch.equal(a.cpu(), b), "do == 1 must leave the gradients untouched"
    do = -0.3125
    fldce.fldce_scale_grads(torch.full((1,), do, device=dev), *dev_xs)
    torch.cuda.synchronize()
    for a, b in zip(dev_xs, xs):
        want = O.scale_grads(do, b.double().numpy())[0]
        # one rounding of the float32 product to the gradient dtype
        np.testing.assert_allclose(a.cpu().double().numpy(), want,
                                   rtol=2.0 ** -8 if dtype == "bf16" else 2.0 ** -23, atol=0)


def test_autograd_module():
    """loss.backward() through the module: gradients equal the oracle's times
    the upstream gradient; bias and EOB on; [B, L, H] input."""
    torch = torch_cuda()
    from lm_head_linear_bf16_amd.autograd import FusedLinearDiffusionCrossEntropyLoss
    dev = torch.device("cuda:0")
    w = synth.custom("autograd", 2, 160, 128, 1100, label_smoothing=0.1, logit_scale=0.5)
    target, p_mask, h, W, b, hd, Wd, bd = _inputs(w, True, dev)
    eob = 11
    target = _eob_targets(target, eob)
    say("case autograd module")
    x = hd.view(w.B, w.L, w.H).clone().requires_grad_(True)
    Wp = Wd.clone().requires_grad_(True)
    bp = bd.clone().requires_grad_(True)
    mod = FusedLinearDiffusionCrossEntropyLoss(label_smoothing=0.1, logit_scale=0.5)
    loss = mod(x, torch.from_numpy(target).to(dev).view(w.B, w.L), Wp, bp,
               torch.from_numpy(p_mask).to(dev).view(w.B, w.L), eob_token_id=eob, eob_weight=1.5)
    (2.5 * loss).backward(retain_graph=True)
    torch.cuda.synchronize()
    with pytest.raises(RuntimeError, match="second backward"):  # it would scale them twice
        loss.backward()
    o = O.forward_backward(h.values, W.values, target, p_mask, label_smoothing=0.1,
                           logit_scale=0.5, reduction="mean", bias=b.values, eob_token_id=eob,
                           eob_weight=1.5)
    _check_loss(w, float(loss.item()), o["loss"])
    dH, dW, db = O.scale_grads(2.5, o["dH"], o["dW"], o["db"])
    e = [grad_err(host(x.grad.view(w.N, w.H)), dH), grad_err(host(Wp.grad), dW),
         grad_err(host(bp.grad), db)]
    say(f"  grad errs {e}")
    assert max(e) <= GRAD_RTOL["bf16"]


def test_full_size_4b_with_bias_and_eob():
    """4b workload (N=2048, H=2560, V=151936) with the seeded bias and an EOB
    weight, in the benchmark's launch configuration: loss from the stored
    full-vocabulary statistics, sampled dH rows, dW rows and db entries."""
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS["4b"]
    g = np.load(os.path.join(GOLDEN, "rowstats_4b_bias.npz"))
    if str(g["fingerprint"]) != synth.fingerprint(w):
        pytest.fail("rowstats_4b_bias.npz is stale: rerun tests/golden/make_golden.py 4b_bias")
    target, p_mask = synth.targets(w)
    h, W, b = synth.hidden(w), synth.weight(w), synth.bias(w)
    valid = target != -100
    eob = int(target[valid][0])
    say(f"case full 4b bias + eob {eob}: N={w.N} H={w.H} V={w.V}")
    r = fldce.fldce_fwd_bwd_ex(to_dev(h, dev), to_dev(W, dev), torch.from_numpy(target).to(dev),
                               torch.from_numpy(p_mask).to(dev), to_dev(b, dev),
                               reduction=w.reduction, total=w.total, eob_token_id=eob,
                               eob_weight=2.0, row_stats=True)
    torch.cuda.synchronize()
    p_eff = O.eob_p_mask(target, p_mask, eob, 2.0)
    D = O.divisor(valid, w.reduction, w.total)
    rl = O.row_losses(g["lse"], g["z_target"], g["z_sum"], w.V, p_eff, valid, 0.0)
    want = O.loss_from_row_losses(rl, D)
    got = float(r["loss"].item())
    say(f"  loss {got:.7g} oracle {want:.7g}")
    assert abs(got - want) <= LOSS_RTOL["bf16"] * abs(want)
    rows = np.unique(np.concatenate([np.nonzero(target == eob)[0],
                                     np.random.default_rng(0).choice(np.nonzero(valid)[0], 30,
                                                                     replace=False)]))
    dH_want = O.dH_rows(h.values, W.values, target, p_eff, g["lse"][rows], rows, D, 0.0, 1.0,
                        bias=b.values)
    eh = grad_err(host(r["dH"][torch.from_numpy(rows).to(dev)]), dH_want)
    vr = np.unique(np.concatenate([[eob, 0, w.V - 1],
                                   np.random.default_rng(1).choice(w.V, 12, replace=False)]))
    dW_want, db_want = O.dW_rows(h.values, W.values, target, p_eff, g["lse"], vr, D, 0.0, 1.0,
                                 bias=b.values, with_db=True)
    vt = torch.from_numpy(vr).to(dev)
    ew = grad_err(host(r["dW"][vt]), dW_want)
    eb = grad_err(host(r["db"][vt]), db_want)
    say(f"  dH rows err {eh:.2e}  dW rows err {ew:.2e}  db err {eb:.2e}")
    assert max(eh, ew, eb) <= GRAD_RTOL["bf16"]


def test_deterministic_repeat_ex_and_forward():
    """Bias, db, EOB and the forward-only entry repeat bit for bit (fixed-order
    reductions everywhere, including the db column sums and the split-K dH)."""
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    w = synth.custom("repeat_ex", 4, 200, 256, 3000, label_smoothing=0.1, logit_scale=0.5)
    target, p_mask, _, _, _, hd, Wd, bd = _inputs(w, True, dev)
    t, p = torch.from_numpy(_eob_targets(target, 7)).to(dev), torch.from_numpy(p_mask).to(dev)
    say("case repeat ex / forward")
    kw = dict(label_smoothing=0.1, logit_scale=0.5, total=w.N, eob_token_id=7, eob_weight=1.5)
    a = fldce.fldce_fwd_bwd_ex(hd, Wd, t, p, bd, row_stats=True, **kw)
    b = fldce.fldce_fwd_bwd_ex(hd, Wd, t, p, bd, row_stats=True, **kw)
    f1 = fldce.fldce_fwd(hd, Wd, t, p, bd, row_stats=True, **kw)
    f2 = fldce.fldce_fwd(hd, Wd, t, p, bd, row_stats=True, **kw)
    torch.cuda.synchronize()
    for k in ("loss", "dH", "dW", "db", "row_lse", "row_loss"):
        assert torch.equal(a[k], b[k]), k
    for k in ("loss", "row_lse", "row_loss"):
        assert torch.equal(f1[k], f2[k]), k
        assert torch.equal(f1[k], a[k]), k  # the forward half of fwd_bwd_ex, bit for bit


def test_binding_checks_caller_outputs():
    """Caller-given outputs must hold exactly the elements the kernels write
    (checked before any launch); correct ones are written in place."""
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    h, W = torch.zeros(4, 64, dtype=bf, device=dev), torch.zeros(10, 64, dtype=bf, device=dev)
    t = torch.zeros(4, dtype=torch.int64, device=dev)
    say("case caller outputs")
    with pytest.raises(ValueError, match="dH must hold 256"):
        fldce.fldce_fwd_bwd(h, W, t, out={"dH": torch.zeros(4, 63, dtype=bf, device=dev)})
    with pytest.raises(ValueError, match="db must hold 10"):
        fldce.fldce_fwd_bwd_ex(h, W, t, want_db=True,
                               out={"db": torch.zeros(11, dtype=bf, device=dev)})
    with pytest.raises(ValueError, match="dW_local must hold 640"):
        fldce.fldce_shard_bwd(h, W, t, None, torch.zeros(4, device=dev), 0, 10,
                              out={"dW_local": torch.zeros(10, 63, dtype=bf, device=dev)})
    with pytest.raises(TypeError):
        fldce.fldce_fwd(h, W, t, out={"loss": torch.zeros(1, dtype=torch.float64, device=dev)})
    o = {k: torch.full(s, float("nan"), dtype=d, device=dev)
         for k, s, d in (("loss", (1,), torch.float32), ("dH", (4, 64), bf), ("dW", (10, 64), bf),
                         ("db", (10,), bf), ("row_lse", (4,), torch.float32),
                         ("row_loss", (4,), torch.float32))}
    r = fldce.fldce_fwd_bwd_ex(h, W, t, want_db=True, row_stats=True, out=o)
    torch.cuda.synchronize()
    for k in o:
        assert r[k].data_ptr() == o[k].data_ptr(), k
        assert torch.isfinite(o[k].float()).all(), k
    # all-zero inputs: uniform softmax over 10 classes, loss = log 10
    assert abs(float(o["loss"].item()) - float(np.log(10.0))) < 1e-5


def test_autograd_module_without_grad_runs_forward_only():
    """Evaluation through the module (torch.no_grad, or inputs that need no
    gradient) runs fldce_fwd: the loss is bitwise the one the training path
    computes, and nothing is attached to the autograd graph."""
    torch = torch_cuda()
    from lm_head_linear_bf16_amd.autograd import FusedLinearDiffusionCrossEntropyLoss
    dev = torch.device("cuda:0")
    w = synth.custom("autograd_eval", 2, 100, 128, 1100, label_smoothing=0.1, logit_scale=0.5)
    target, p_mask, _, _, _, hd, Wd, bd = _inputs(w, True, dev)
    t = torch.from_numpy(target).to(dev)
    pm = torch.from_numpy(p_mask).to(dev)
    mod = FusedLinearDiffusionCrossEntropyLoss(label_smoothing=0.1, logit_scale=0.5)
    say("case autograd module without grad")
    x = hd.clone().requires_grad_(True)
    train = mod(x, t, Wd, bd, pm)
    with torch.no_grad():
        ev1 = mod(x, t, Wd, bd, pm)
    ev2 = mod(hd, t, Wd, bd, pm)            # nothing requires grad
    torch.cuda.synchronize()
    assert train.requires_grad and not ev1.requires_grad and not ev2.requires_grad
    assert ev1.grad_fn is None and ev2.grad_fn is None
    assert torch.equal(train.detach(), ev1) and torch.equal(ev1, ev2)


PARTIAL_CASES = [
    ("single_bf16", synth.custom("partial_bf16", 3, 150, 128, 2053, label_smoothing=0.1,
                                 logit_scale=0.5), 0),
    ("chunked_bf16", synth.custom("partial_chunked_bf16", 3, 150, 128, 2053,
                                  label_smoothing=0.1, logit_scale=0.5), 128),
    ("f32", synth.custom("partial_f32", 2, 64, 72, 777, dtype="f32", label_smoothing=0.1), 0),
]


@pytest.mark.parametrize("case", PARTIAL_CASES, ids=lambda c: c[0])
def test_fwd_bwd_ex_some_gradients(case):
    """dH, dW and db are each optional in fldce_fwd_bwd_ex: whatever is
    computed equals the full call bit for bit (loss and row statistics too),
    the rest is not touched; with none, only the loss."""
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    name, w, chunk = case
    dev = torch.device("cuda:0")
    target, p_mask, _, _, _, hd, Wd, bd = _inputs(w, True, dev)
    t, p = torch.from_numpy(target).to(dev), torch.from_numpy(p_mask).to(dev)
    kw = dict(label_smoothing=w.label_smoothing, logit_scale=w.logit_scale, reduction=w.reduction,
              total=w.total, eob_token_id=5, eob_weight=2.0, chunk_rows=chunk, row_stats=True)
    say(f"case partial gradients {name}")
    full = fldce.fldce_fwd_bwd_ex(hd, Wd, t, p, bd, want_db=True, **kw)
    for want in [(True, False, False), (False, True, False), (False, False, True),
                 (True, False, True), (False, False, False)]:
        r = fldce.fldce_fwd_bwd_ex(hd, Wd, t, p, bd, want_dH=want[0], want_dW=want[1],
                                   want_db=want[2], **kw)
        torch.cuda.synchronize()
        for key in ("loss", "row_lse", "row_loss"):
            assert torch.equal(r[key], full[key]), (want, key)
        for key, on in zip(("dH", "dW", "db"), want):
            if on:
                assert torch.equal(r[key], full[key]), (want, key)
            else:
                assert r[key] is None, (want, key)


def test_autograd_frozen_weight():
    """A weight that needs no gradient: only dH (and db) are computed, equal
    to the full backward's bit for bit; weight.grad stays None."""
    torch = torch_cuda()
    from lm_head_linear_bf16_amd.autograd import FusedLinearDiffusionCrossEntropyLoss
    dev = torch.device("cuda:0")
    w = synth.custom("autograd_frozen", 2, 120, 128, 1100, label_smoothing=0.1, logit_scale=0.5)
    target, p_mask, _, _, _, hd, Wd, bd = _inputs(w, True, dev)
    t, pm = torch.from_numpy(target).to(dev), torch.from_numpy(p_mask).to(dev)
    mod = FusedLinearDiffusionCrossEntropyLoss(label_smoothing=0.1, logit_scale=0.5)
    say("case autograd frozen weight")
    xa, Wa, ba = (hd.clone().requires_grad_(True), Wd.clone().requires_grad_(True),
                  bd.clone().requires_grad_(True))
    (1.5 * mod(xa, t, Wa, ba, pm)).backward()
    xb, Wb, bb = hd.clone().requires_grad_(True), Wd.clone(), bd.clone().requires_grad_(True)
    (1.5 * mod(xb, t, Wb, bb, pm)).backward()
    torch.cuda.synchronize()
    assert Wb.grad is None
    assert torch.equal(xa.grad, xb.grad) and torch.equal(ba.grad, bb.grad)
