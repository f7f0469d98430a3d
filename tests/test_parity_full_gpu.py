"""Parity at the full workload sizes, in the launch configuration the
benchmark times (default chunking), element by element:

* ``4b`` and ``headline`` (also in 2048-row chunks): the whole dH [N, H] and
  dW [V, H] against the float64 oracle (page 1, fused_linear_cross_entropy_-
  forward: every row of ``dx`` and ``dw`` from the chunk loop's products),
  the loss, every row's lse and loss, ignored rows exactly zero;
* ``block``: every row's lse and loss against the stored full-vocabulary
  statistics, the loss, and dH / dW on 512 sampled token / vocabulary rows
  (the oracle computes those rows exactly; the whole tensors would need
  about 30 TFLOP of float64 GEMMs);
* ``shard`` (one GPU's vocabulary shard): every row's partials (max, sum of
  exp, target logit, sum of logits) against the oracle's, and combined with
  the other seven shards' partials (stored, written by the oracle) against
  the full-vocabulary lse, target logit and row sum, for the rows with a
  target and, with an ignore_index no target has, for every row (page 3
  section 4); the whole dH_partial and dW_local of the shard backward.

The oracle runs on the rows whose target is not ignore_index: ignored rows
add nothing to the loss, dW or the divisor's count (pinned on the CPU), and
their dH rows are checked to be exactly zero here."""

import functools
import os

import numpy as np
import pytest

import oracle as O
from lm_head_linear_bf16_amd import synth
from _helpers import GOLDEN, GRAD_RTOL, LOSS_RTOL, grad_err, host, say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu

LSE_ATOL = 2e-3          # per-row lse (about 12 at V = 151936), fp32 from bf16 inputs
ROW_LOSS_RTOL = 2e-3     # per-row loss, as the bf16 loss tolerance
NO_TARGET_IGNORE = -(2 ** 63)  # an ignore_index no target equals: every row counts


def _golden(w):
    path = os.path.join(GOLDEN, f"rowstats_{w.name}.npz")
    g = np.load(path)
    if str(g["fingerprint"]) != synth.fingerprint(w):
        pytest.fail(f"{path} is stale: rerun tests/golden/make_golden.py {w.name}")
    return g


@functools.lru_cache(maxsize=1)
def _oracle_valid(name: str) -> dict:
    """The oracle's loss, per-row lse / loss, dH and dW over the valid rows of
    a workload (cached: the plain and chunked tests share it)."""
    w = synth.WORKLOADS[name]
    t, p = synth.targets(w)
    h, W = synth.hidden(w).values, synth.weight(w).values
    v = t != synth.IGNORE_INDEX
    say(f"  oracle: {int(v.sum())} valid rows of {w.name}")
    o = O.forward_backward(h[v], W, t[v], p[v], label_smoothing=w.label_smoothing,
                           logit_scale=w.logit_scale, reduction=w.reduction,
                           total=w.total or None, row_block=512)
    return dict(valid=v, loss=o["loss"], lse=o["lse"], row_loss=o["row_loss"], dH=o["dH"],
                dW=o["dW"], D=o["D"])


def _check_rows(r, w, t, p, g, valid):
    """Every row's lse and loss against the stored statistics; the loss."""
    D = O.divisor(valid, w.reduction, w.total or None)
    rl_want = O.row_losses(g["lse"], g["z_target"], g["z_sum"], w.V, p, valid, w.label_smoothing)
    want = O.loss_from_row_losses(rl_want, D)
    got = float(r["loss"].item())
    say(f"  loss {got:.7g} oracle {want:.7g}")
    assert abs(got - want) <= LOSS_RTOL["bf16"] * abs(want)
    lse, rl = host(r["row_lse"]), host(r["row_loss"])
    assert np.all(lse[~valid] == 0.0) and np.all(rl[~valid] == 0.0)
    e_lse = np.abs(lse[valid] - g["lse"][valid]).max()
    e_rl = (np.abs(rl[valid] - rl_want[valid]) / np.abs(rl_want[valid])).max()
    say(f"  every row: lse max err {e_lse:.2e}, row loss max rel err {e_rl:.2e}")
    assert e_lse <= LSE_ATOL and e_rl <= ROW_LOSS_RTOL
    return D


def _check_full_grads(r, name, valid, torch, dev):
    o = _oracle_valid(name)
    assert np.array_equal(o["valid"], valid)
    ig = torch.from_numpy(~valid).to(dev)
    assert float(r["dH"][ig].float().abs().max()) == 0.0   # ignored rows: exactly +0
    vd = torch.from_numpy(valid).to(dev)
    eh = grad_err(host(r["dH"][vd]), o["dH"])
    ew = grad_err(host(r["dW"]), o["dW"])
    say(f"  full dH err {eh:.2e}  full dW err {ew:.2e} (bound {GRAD_RTOL['bf16']:.0e})")
    assert eh <= GRAD_RTOL["bf16"] and ew <= GRAD_RTOL["bf16"]
    lrel = abs(float(r["loss"].item()) - o["loss"]) / abs(o["loss"])
    assert lrel <= LOSS_RTOL["bf16"]


def _run_fwd_bwd(w, chunk_rows=0):
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    t, p = synth.targets(w)
    h, W = synth.hidden(w), synth.weight(w)
    say(f"case full {w.name}: N={w.N} H={w.H} V={w.V} chunk_rows={chunk_rows or 'default'}")
    r = fldce.fldce_fwd_bwd(to_dev(h, dev), to_dev(W, dev), torch.from_numpy(t).to(dev),
                            torch.from_numpy(p).to(dev), label_smoothing=w.label_smoothing,
                            logit_scale=w.logit_scale, reduction=w.reduction, total=w.total,
                            row_stats=True, chunk_rows=chunk_rows)
    torch.cuda.synchronize()
    return torch, dev, t, p, h, W, r


@pytest.mark.parametrize("name", ["4b", "headline"])
def test_full_size_fwd_bwd_every_element(name):
    w = synth.WORKLOADS[name]
    torch, dev, t, p, h, W, r = _run_fwd_bwd(w)
    valid = t != synth.IGNORE_INDEX
    _check_rows(r, w, t, p, _golden(w), valid)
    _check_full_grads(r, name, valid, torch, dev)


def test_full_size_headline_chunked_every_element():
    """The headline workload in chunks of 2048 compacted rows: the fp32 dW
    accumulator carries over chunks (first, middle and last chunk modes)."""
    w = synth.WORKLOADS["headline"]
    torch, dev, t, p, h, W, r = _run_fwd_bwd(w, chunk_rows=2048)
    valid = t != synth.IGNORE_INDEX
    _check_rows(r, w, t, p, _golden(w), valid)
    _check_full_grads(r, "headline", valid, torch, dev)


def _sample_rows(target, n_valid, n_ign, seed):
    rng = np.random.default_rng(seed)
    v = np.nonzero(target != synth.IGNORE_INDEX)[0]
    ig = np.nonzero(target == synth.IGNORE_INDEX)[0]
    rows = list(rng.choice(v, n_valid, replace=False)) + list(rng.choice(ig, n_ign, replace=False))
    rows += [int(v[0]), int(v[-1]), 0, len(target) - 1]
    return np.unique(np.array(rows, dtype=np.int64))


def _sample_vocab(target, V, n, seed):
    """The most targeted rows, untargeted rows, the first and last rows and
    the rows at the edges of the last 256-row tile, plus random rows."""
    rng = np.random.default_rng(seed)
    tv = target[target != synth.IGNORE_INDEX]
    counts = np.bincount(tv, minlength=V)
    most = np.argsort(-counts, kind="stable")[:32]
    untargeted = np.nonzero(counts == 0)[0]
    edge = [0, V - 1, V - 2, V - 129, (V // 256) * 256, (V // 256) * 256 - 1]
    rows = list(most) + edge + list(rng.choice(untargeted, min(32, len(untargeted)), replace=False))
    rows += list(rng.choice(V, n - len(rows), replace=False))
    return np.unique(np.array(rows, dtype=np.int64))


def test_full_size_block_rows_and_samples():
    """Block diffusion (N = 16384, H = 4096, 15% padding, counted mean): every
    row's lse and loss; dH and dW on 512 sampled rows each."""
    w = synth.WORKLOADS["block"]
    torch, dev, t, p, h, W, r = _run_fwd_bwd(w)
    valid = t != synth.IGNORE_INDEX
    g = _golden(w)
    D = _check_rows(r, w, t, p, g, valid)
    ig = torch.from_numpy(~valid).to(dev)
    assert float(r["dH"][ig].float().abs().max()) == 0.0
    rows = _sample_rows(t, 480, 24, seed=5)
    dH_want = O.dH_rows(h.values, W.values, t, p, g["lse"][rows], rows, D, w.label_smoothing,
                        w.logit_scale)
    eh = grad_err(host(r["dH"][torch.from_numpy(rows).to(dev)]), dH_want)
    vr = _sample_vocab(t, w.V, 512, seed=6)
    dW_want = O.dW_rows(h.values, W.values, t, p, g["lse"], vr, D, w.label_smoothing, w.logit_scale)
    ew = grad_err(host(r["dW"][torch.from_numpy(vr).to(dev)]), dW_want)
    say(f"  {len(rows)} dH rows err {eh:.2e}  {len(vr)} dW rows err {ew:.2e}")
    assert eh <= GRAD_RTOL["bf16"] and ew <= GRAD_RTOL["bf16"]


def _combine_with_rest(m, S, tl, rs, g):
    """Combine this shard's partials with the stored combine of the other
    shards (oracle's own combine step) -> (lse, target logit, row sum)."""
    rest = (g["rest_lse"], np.ones_like(g["rest_lse"]), g["rest_target"], g["rest_sum"])
    return O.combine_shard_partials([(m, S, tl, rs), rest])


def test_full_size_vocab_shard_every_element():
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
    valid = t != synth.IGNORE_INDEX
    say(f"case full shard partials: N={w.N} H={w.H} V_local={Vl} shard {k}")
    r = fldce.fldce_shard_partials(hd, Wd, td, v0, logit_scale=w.logit_scale)
    torch.cuda.synchronize()
    m, S, tl, rs = (host(r[x]) for x in ("row_max", "row_sumexp", "target_logit",
                                         "row_sumlogit"))
    for x, want in ((m, -np.inf), (S, 0.0), (tl, 0.0), (rs, 0.0)):
        assert np.all(x[~valid] == want)  # rows with ignore_index are skipped
    om, oS, ot, orr = O.shard_partials(h.values[valid], Wk.values, t[valid], v0, w.logit_scale)
    em = np.abs(m[valid] - om).max()
    el = np.abs(np.log(S[valid]) + m[valid] - (np.log(oS) + om)).max()
    et = np.abs(tl[valid] - ot).max()
    er = (np.abs(rs[valid] - orr) / np.maximum(np.abs(orr), 1.0)).max()
    say(f"  every valid row: max err {em:.2e}, shard lse err {el:.2e}, target err {et:.2e}, "
        f"row-sum rel err {er:.2e}")
    assert em <= 5e-3 and el <= LSE_ATOL and et <= 5e-3 and er <= 2e-3
    lse, zt, zs = _combine_with_rest(m[valid], S[valid], tl[valid], rs[valid],
                                     {x: g[x][valid] for x in ("rest_lse", "rest_target",
                                                               "rest_sum")})
    e1 = np.abs(lse - g["lse"][valid]).max()
    e2 = np.abs(zt - g["z_target"][valid]).max()
    say(f"  combined with the other 7 shards: lse err {e1:.2e}, target logit err {e2:.2e}")
    assert e1 <= LSE_ATOL and e2 <= 5e-3

    say("case full shard partials of every row (an ignore_index no target has)")
    ra = fldce.fldce_shard_partials(hd, Wd, td, v0, ignore_index=NO_TARGET_IGNORE,
                                    logit_scale=w.logit_scale)
    torch.cuda.synchronize()
    ma, Sa, ta, rsa = (host(ra[x]) for x in ("row_max", "row_sumexp", "target_logit",
                                             "row_sumlogit"))
    assert np.array_equal(ma[valid], m[valid]) and np.array_equal(Sa[valid], S[valid])
    assert np.all(ta[~valid] == 0.0)  # a target outside every shard: no target logit
    lse, zt, zs = _combine_with_rest(ma, Sa, ta, rsa, g)
    e1 = np.abs(lse - g["lse"]).max()
    e3 = (np.abs(zs - g["z_sum"]) / np.maximum(np.abs(g["z_sum"]), 1.0)).max()
    say(f"  every row combined: lse err {e1:.2e}, row-sum rel err {e3:.2e}")
    assert e1 <= LSE_ATOL and e3 <= 2e-3

    say(f"case full shard backward: N={w.N} H={w.H} V_local={Vl}")
    lse_d = torch.from_numpy(g["lse"].astype(np.float32)).to(dev)
    b = fldce.fldce_shard_bwd(hd, Wd, td, torch.from_numpy(p).to(dev), lse_d, v0, w.V,
                              label_smoothing=w.label_smoothing, logit_scale=w.logit_scale,
                              reduction=w.reduction, total=w.total)
    torch.cuda.synchronize()
    D = O.divisor(valid, w.reduction, w.total or None)
    ig = torch.from_numpy(~valid).to(dev)
    assert float(b["dH_partial"][ig].abs().max()) == 0.0
    dh_want, dw_want = O.shard_backward(h.values[valid], Wk.values, t[valid], p[valid],
                                        g["lse"][valid], v0, w.V, D, w.label_smoothing,
                                        w.logit_scale, row_block=512)
    eh = grad_err(host(b["dH_partial"][torch.from_numpy(valid).to(dev)]), dh_want)
    ew = grad_err(host(b["dW_local"]), dw_want)
    say(f"  full dH_partial err {eh:.2e}  full dW_local err {ew:.2e}")
    assert eh <= GRAD_RTOL["bf16"] and ew <= GRAD_RTOL["bf16"]
