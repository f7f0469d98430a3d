"""Parity at the full workload sizes, in the launch configuration the
benchmark times (default chunking), on outputs the oracle computes row by row:

* the loss, from the oracle's stored per-row float64 statistics (full-vocab
  lse, target logit, row sum of logits; tests/golden/make_golden.py) and the
  oracle's row-loss and reduction steps;
* per-row lse of sampled rows;
* dH of sampled token rows (oracle: that row's softmax over the vocabulary);
* dW of sampled vocabulary rows (oracle: that column of g over all rows);
* ignored rows exactly zero in dH.

For the vocabulary shard: the shard's partials on sampled rows, their combine
with the other shards' (oracle) partials against the full-vocabulary lse, and
the shard backward from the stored global lse."""

import os

import numpy as np
import pytest

import oracle as O
from lm_head_linear_bf16_amd import synth
from _helpers import GOLDEN, GRAD_RTOL, LOSS_RTOL, grad_err, host, say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


def _golden(w):
    path = os.path.join(GOLDEN, f"rowstats_{w.name}.npz")
    g = np.load(path)
    if str(g["fingerprint"]) != synth.fingerprint(w):
        pytest.fail(f"{path} is stale: rerun tests/golden/make_golden.py {w.name}")
    return g


def _sample_rows(target, n_valid=40, n_ign=6, seed=0):
    rng = np.random.default_rng(seed)
    v = np.nonzero(target != -100)[0]
    ig = np.nonzero(target == -100)[0]
    rows = list(rng.choice(v, n_valid, replace=False)) + list(rng.choice(ig, n_ign, replace=False))
    rows += [int(v[0]), int(v[-1])] if n_ign == 0 else [0, len(target) - 1]
    return np.unique(np.array(rows, dtype=np.int64))


def _sample_vocab(target, V, seed=1):
    rng = np.random.default_rng(seed)
    t = target[target != -100]
    counts = np.bincount(t, minlength=V)
    most = np.argsort(-counts, kind="stable")[:8]
    untargeted = np.nonzero(counts == 0)[0]
    rows = list(most) + list(rng.choice(V, 12, replace=False)) + [0, V - 1, V - 2, V - 129]
    if len(untargeted):
        rows += list(rng.choice(untargeted, min(4, len(untargeted)), replace=False))
    return np.unique(np.array(rows, dtype=np.int64))


@pytest.mark.parametrize("name", ["4b", "headline", "block"])
def test_full_size_fwd_bwd(name):
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[name]
    g = _golden(w)
    t, p = synth.targets(w)
    h, W = synth.hidden(w), synth.weight(w)
    say(f"case full {name}: N={w.N} H={w.H} V={w.V} (default chunking)")
    r = fldce.fldce_fwd_bwd(to_dev(h, dev), to_dev(W, dev), torch.from_numpy(t).to(dev),
                            torch.from_numpy(p).to(dev), label_smoothing=w.label_smoothing,
                            logit_scale=w.logit_scale, reduction=w.reduction, total=w.total,
                            row_stats=True)
    torch.cuda.synchronize()
    valid = t != -100
    D = O.divisor(valid, w.reduction, w.total or None)
    rl = O.row_losses(g["lse"], g["z_target"], g["z_sum"], w.V, p, valid, w.label_smoothing)
    want = O.loss_from_row_losses(rl, D)
    got = float(r["loss"].item())
    say(f"  loss {got:.7g} oracle {want:.7g}")
    assert abs(got - want) <= LOSS_RTOL["bf16"] * abs(want)
    ig = torch.from_numpy(~valid).to(dev)
    assert float(r["dH"][ig].float().abs().max()) == 0.0
    assert float(r["row_loss"][ig].abs().max()) == 0.0
    rows = _sample_rows(t)
    np.testing.assert_allclose(host(r["row_lse"][torch.from_numpy(rows).to(dev)])[valid[rows]],
                               g["lse"][rows][valid[rows]], atol=2e-3, rtol=0)
    dH_want = O.dH_rows(h.values, W.values, t, p, g["lse"][rows], rows, D, w.label_smoothing,
                        w.logit_scale)
    eh = grad_err(host(r["dH"][torch.from_numpy(rows).to(dev)]), dH_want)
    vr = _sample_vocab(t, w.V)
    dW_want = O.dW_rows(h.values, W.values, t, p, g["lse"], vr, D, w.label_smoothing, w.logit_scale)
    ew = grad_err(host(r["dW"][torch.from_numpy(vr).to(dev)]), dW_want)
    say(f"  dH rows err {eh:.2e}  dW rows err {ew:.2e}")
    assert eh <= GRAD_RTOL["bf16"] and ew <= GRAD_RTOL["bf16"]


def test_full_size_vocab_shard():
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS["shard"]
    g = _golden(w)
    t, p = synth.targets(w)
    h = synth.hidden(w)
    k, v0, Vl = w.shard_k, w.vocab_start, w.V_local
    Wk = synth.weight(w, shard=k)
    hd, td = to_dev(h, dev), torch.from_numpy(t).to(dev)
    Wd = to_dev(Wk, dev)
    say(f"case full shard partials: N={w.N} H={w.H} V_local={Vl} shard {k}")
    r = fldce.fldce_shard_partials(hd, Wd, td, v0, logit_scale=w.logit_scale)
    torch.cuda.synchronize()
    rows = _sample_rows(t, n_ign=0)
    ign = np.nonzero(t == -100)[0]
    for x, want in (("row_max", -np.inf), ("row_sumexp", 0.0), ("target_logit", 0.0),
                    ("row_sumlogit", 0.0)):
        assert np.all(host(r[x])[ign] == want), x  # skipped rows
    m, S, tl, rs = (host(r[x])[rows] for x in ("row_max", "row_sumexp", "target_logit",
                                               "row_sumlogit"))
    om, oS, ot, orr = O.shard_partials(h.values[rows], Wk.values, t[rows], v0, w.logit_scale)
    np.testing.assert_allclose(m, om, atol=5e-3, rtol=0)
    np.testing.assert_allclose(np.log(S) + m, np.log(oS) + om, atol=2e-3, rtol=0)
    np.testing.assert_allclose(tl, ot, atol=5e-3, rtol=0)
    np.testing.assert_allclose(rs, orr, atol=5e-2, rtol=2e-3)
    # combine with the other seven shards (oracle partials) = full-vocabulary lse
    parts = []
    for j in range(w.shards):
        if j == k:
            parts.append((m, S, tl, rs))
        else:
            parts.append(O.shard_partials(h.values[rows], synth.weight(w, shard=j).values, t[rows],
                                          j * Vl, w.logit_scale))
    lse, zt, _ = O.combine_shard_partials(parts)
    np.testing.assert_allclose(lse, g["lse"][rows], atol=2e-3, rtol=0)
    np.testing.assert_allclose(zt, g["z_target"][rows], atol=5e-3, rtol=0)

    say(f"case full shard backward: N={w.N} H={w.H} V_local={Vl}")
    lse_d = torch.from_numpy(g["lse"].astype(np.float32)).to(dev)
    b = fldce.fldce_shard_bwd(hd, Wd, td, torch.from_numpy(p).to(dev), lse_d, v0, w.V,
                              label_smoothing=w.label_smoothing, logit_scale=w.logit_scale,
                              reduction=w.reduction, total=w.total)
    torch.cuda.synchronize()
    valid = t != -100
    D = O.divisor(valid, w.reduction, w.total or None)
    ig = torch.from_numpy(~valid).to(dev)
    assert float(b["dH_partial"][ig].abs().max()) == 0.0
    dh_want = O.dH_rows(h.values, Wk.values, t, p, g["lse"][rows], rows, D, w.label_smoothing,
                        w.logit_scale, V_global=w.V, vocab_start=v0)
    eh = grad_err(host(b["dH_partial"][torch.from_numpy(rows).to(dev)]), dh_want)
    tin = t[valid & (t >= v0) & (t < v0 + Vl)] - v0
    vr = _sample_vocab(np.concatenate([tin, np.full(1, -100)]), Vl)
    dw_want = O.dW_rows(h.values, Wk.values, t, p, g["lse"], vr, D, w.label_smoothing,
                        w.logit_scale, V_global=w.V, vocab_start=v0)
    ew = grad_err(host(b["dW_local"][torch.from_numpy(vr).to(dev)]), dw_want)
    say(f"  dH_partial rows err {eh:.2e}  dW_local rows err {ew:.2e}")
    assert eh <= GRAD_RTOL["bf16"] and ew <= GRAD_RTOL["bf16"]


def test_full_size_headline_chunked():
    """The headline workload in chunks of 2048 compacted rows: the fp32 dW
    accumulator carries over chunks (first, middle and last chunk modes) at
    the full vocabulary."""
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS["headline"]
    g = _golden(w)
    t, p = synth.targets(w)
    h, W = synth.hidden(w), synth.weight(w)
    say(f"case full headline, chunk_rows=2048: N={w.N} H={w.H} V={w.V}")
    r = fldce.fldce_fwd_bwd(to_dev(h, dev), to_dev(W, dev), torch.from_numpy(t).to(dev),
                            torch.from_numpy(p).to(dev), label_smoothing=w.label_smoothing,
                            logit_scale=w.logit_scale, reduction=w.reduction, total=w.total,
                            chunk_rows=2048)
    torch.cuda.synchronize()
    valid = t != -100
    D = O.divisor(valid, w.reduction, w.total or None)
    rl = O.row_losses(g["lse"], g["z_target"], g["z_sum"], w.V, p, valid, w.label_smoothing)
    want = O.loss_from_row_losses(rl, D)
    got = float(r["loss"].item())
    say(f"  loss {got:.7g} oracle {want:.7g}")
    assert abs(got - want) <= LOSS_RTOL["bf16"] * abs(want)
    rows = _sample_rows(t, seed=3)
    dH_want = O.dH_rows(h.values, W.values, t, p, g["lse"][rows], rows, D, w.label_smoothing,
                        w.logit_scale)
    eh = grad_err(host(r["dH"][torch.from_numpy(rows).to(dev)]), dH_want)
    vr = _sample_vocab(t, w.V, seed=4)
    dW_want = O.dW_rows(h.values, W.values, t, p, g["lse"], vr, D, w.label_smoothing, w.logit_scale)
    ew = grad_err(host(r["dW"][torch.from_numpy(vr).to(dev)]), dW_want)
    say(f"  dH rows err {eh:.2e}  dW rows err {ew:.2e}")
    assert eh <= GRAD_RTOL["bf16"] and ew <= GRAD_RTOL["bf16"]
