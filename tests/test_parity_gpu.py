"""HIP path vs the float64 oracle, element by element, at sizes the oracle
finishes in seconds (several 256-wide tiles and ragged tails), through the C
ABI.  Edge cases: vocabulary not a multiple of 64/128/256, token count not a
multiple of the tile, several row chunks, all rows ignored, no rows, no
p_mask, fp32 inputs with any H, vocabulary shards."""

import numpy as np
import pytest

import oracle as O
from lm_head_linear_bf16_amd import synth
from _helpers import GRAD_RTOL, LOSS_RTOL, grad_err, host, say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


def _run(w, chunk_rows=0, p_none=False, target=None, p_mask=None, h=None, W=None):
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    if target is None:
        target, p_mask = synth.targets(w)
    h = h or synth.hidden(w)
    W = W or synth.weight(w)
    say(f"case {w.name}: N={w.N} H={w.H} V={w.V} {w.dtype} eps={w.label_smoothing} "
        f"s={w.logit_scale} {w.reduction} total={w.total} chunk={chunk_rows}")
    r = fldce.fldce_fwd_bwd(to_dev(h, dev), to_dev(W, dev), torch.from_numpy(target).to(dev),
                            None if p_none else torch.from_numpy(p_mask).to(dev),
                            label_smoothing=w.label_smoothing, logit_scale=w.logit_scale,
                            reduction=w.reduction, total=w.total, chunk_rows=chunk_rows,
                            row_stats=True)
    torch.cuda.synchronize()
    o = O.forward_backward(h.values, W.values, target, None if p_none else p_mask,
                           label_smoothing=w.label_smoothing, logit_scale=w.logit_scale,
                           reduction=w.reduction, total=w.total or None)
    return r, o, target


def _compare(w, r, o, target):
    loss = float(r["loss"].item())
    if o["loss"] == 0.0:
        assert loss == 0.0
    else:
        assert abs(loss - o["loss"]) <= LOSS_RTOL[w.dtype] * abs(o["loss"]), (loss, o["loss"])
    ig = target == -100
    dH = host(r["dH"])
    assert np.all(dH[ig] == 0.0), "ignored rows must have exactly zero dH"
    assert not np.any(np.signbit(r["dH"].float().cpu().numpy()[ig])), "ignored dH rows are +0"
    assert np.all(host(r["row_loss"])[ig] == 0.0)
    if o["loss"] != 0.0:
        assert grad_err(dH, o["dH"]) <= GRAD_RTOL[w.dtype]
        assert grad_err(host(r["dW"]), o["dW"]) <= GRAD_RTOL[w.dtype]
        valid = ~ig
        np.testing.assert_allclose(host(r["row_lse"])[valid], o["lse"][valid], rtol=0,
                                   atol=2e-3 if w.dtype == "bf16" else 2e-5)
    else:
        assert np.all(host(r["dW"]) == 0.0)


CASES = [
    synth.custom("ragged_bf16", 3, 100, 128, 1000),
    synth.custom("smooth_sum_bf16", 3, 171, 192, 2053, label_smoothing=0.1, logit_scale=0.5,
                 reduction="sum"),
    synth.custom("count_mean_bf16", 2, 320, 256, 4099, label_smoothing=0.3, logit_scale=1.7,
                 total_is_N=False),
    synth.custom("block_pad_bf16", 4, 96, 128, 777, p_block=4, pad_tail=17, total_is_N=False),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_bf16_small(w):
    r, o, t = _run(w)
    _compare(w, r, o, t)


@pytest.mark.parametrize("chunk", [64, 256, 300])
def test_bf16_chunked(chunk):
    """316 of 700 rows have a target: a first chunk, later ones carried in
    fp32, a final one that holds the last row and writes dW, and empty
    chunks after it (chunks cover the compacted rows in order)."""
    w = synth.custom("chunked_bf16", 7, 100, 128, 1500, label_smoothing=0.1, logit_scale=0.5)
    r, o, t = _run(w, chunk_rows=chunk)
    _compare(w, r, o, t)


@pytest.mark.parametrize("n_valid", [64, 128, 129])
def test_bf16_chunked_rows_fill_whole_chunks(n_valid):
    """The valid rows end exactly at a chunk boundary (64, 128) or one row
    past it (129): the chunk holding the last row is final although a full
    chunk, and every chunk after it is empty."""
    w = synth.custom("chunked_fill_bf16", 3, 100, 128, 1001, label_smoothing=0.2, logit_scale=0.7)
    target, p_mask = synth.targets(w)
    rng = np.random.default_rng(n_valid)
    target = np.full(w.N, -100, dtype=np.int64)
    keep = np.sort(rng.choice(w.N, n_valid, replace=False))
    target[keep] = rng.integers(0, w.V, n_valid)
    r, o, t = _run(w, chunk_rows=64, target=target, p_mask=p_mask)
    _compare(w, r, o, t)


def test_bf16_largest_vocabulary():
    """The largest bf16 vocabulary, V = 2^23 - 64 (the last multiple of 64
    below the 2^23 limit): a lane's byte offset into the stored exponentials
    (row < 256 of a 256-row tile, times 2 Vp) reaches just under 2^32, and
    targets sit in the last vocabulary columns.  Every row's lse, the loss,
    the whole dH, and dW on the first and last 256 vocabulary rows and the
    targets' rows, against the oracle."""
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    V = (1 << 23) - 64
    w = synth.custom("largest_vocab_bf16", 1, 16, 64, V, label_smoothing=0.1, logit_scale=0.5,
                     reduction="sum", index=420)
    _, p = synth.targets(w)
    rng = np.random.default_rng(420)
    t = rng.integers(0, V, w.N)
    t[:4] = [V - 1, V - 64, V - 65, 0]
    h, W = synth.hidden(w), synth.weight(w)
    say(f"case largest vocabulary: N={w.N} H={w.H} V={V}")
    r = fldce.fldce_fwd_bwd(to_dev(h, dev), to_dev(W, dev), torch.from_numpy(t).to(dev),
                            torch.from_numpy(p).to(dev), label_smoothing=0.1, logit_scale=0.5,
                            reduction="sum", row_stats=True)
    torch.cuda.synchronize()
    rows = np.arange(w.N)
    lse, zt, zs = O.row_stats(h.values, W.values, t, rows, 0.5)
    np.testing.assert_allclose(host(r["row_lse"]), lse, rtol=0, atol=2e-3)
    valid = np.ones(w.N, dtype=bool)
    loss = O.loss_from_row_losses(O.row_losses(lse, zt, zs, V, p, valid, 0.1), 1.0)
    assert abs(float(r["loss"].item()) - loss) <= LOSS_RTOL["bf16"] * abs(loss)
    dH = O.dH_rows(h.values, W.values, t, p, lse, rows, 1.0, 0.1, 0.5)
    assert grad_err(host(r["dH"]), dH) <= GRAD_RTOL["bf16"]
    vr = np.unique(np.concatenate([np.arange(256), np.arange(V - 256, V), t]))
    dW = O.dW_rows(h.values, W.values, t, p, lse, vr, 1.0, 0.1, 0.5)
    assert grad_err(host(r["dW"][torch.from_numpy(vr).to(dev)]), dW) <= GRAD_RTOL["bf16"]


def test_fp32_tiny_workload():
    w = synth.WORKLOADS["tiny"]
    r, o, t = _run(w)
    _compare(w, r, o, t)


@pytest.mark.parametrize("chunk", [0, 32])
def test_fp32_any_H(chunk):
    w = synth.custom("fp32_odd", 1, 77, 50, 333, dtype="f32", label_smoothing=0.2,
                     logit_scale=0.7, reduction="sum")
    r, o, t = _run(w, chunk_rows=chunk)
    _compare(w, r, o, t)


def test_p_mask_none_is_ones():
    w = synth.custom("nopmask_bf16", 2, 128, 128, 600)
    r, o, t = _run(w, p_none=True)
    _compare(w, r, o, t)


def test_no_ignored_rows():
    w = synth.custom("all_valid_bf16", 2, 150, 128, 900, label_smoothing=0.1, logit_scale=0.5)
    t = np.random.default_rng(7).integers(0, w.V, w.N).astype(np.int64)
    _, p = synth.targets(w)
    r, o, _ = _run(w, target=t, p_mask=p)
    _compare(w, r, o, t)


def _far_target_inputs(w, seed):
    """N(0, 1) raw logits times a large logit scale on the second half of the
    rows (spreads of about a hundred nats between a row's best logit and a
    random target), raw logits 50 times smaller on the first half."""
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((w.N, w.H)).astype(np.float32)
    h[: w.N // 2] *= 0.02
    W = (rng.standard_normal((w.V, w.H)) / np.sqrt(w.H)).astype(np.float32)
    return synth._as_dtype(h, w.dtype), synth._as_dtype(W, w.dtype)


@pytest.mark.parametrize("chunk", [0, 128])
def test_targets_far_below_the_row_maximum(chunk):
    """Rows whose best logit lies more than 30 nats above the target logit
    are recomputed relative to their logsumexp (the stored exponentials of
    the other rows are relative to the target logit): loss, lse, dH and dW
    against the oracle with both kinds of rows in one batch, and the
    forward-only loss equal bit for bit."""
    w = synth.custom("far_targets_bf16", 2, 150, 128, 3001, label_smoothing=0.1,
                     logit_scale=20.0, w_std=1.0 / np.sqrt(128), total_is_N=False)
    h, W = _far_target_inputs(w, seed=21)
    t, p = synth.targets(w)
    r, o, _ = _run(w, chunk_rows=chunk, target=t, p_mask=p, h=h, W=W)
    z = O.scaled_logits(h.values, W.values, w.logit_scale)
    v = t != -100
    gap = z.max(axis=1) - z[np.arange(w.N), np.where(v, t, 0)]
    assert np.any(v & (gap > 35.0)) and np.any(v & (gap < 25.0))  # both kinds of rows
    _compare(w, r, o, t)
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    f = fldce.fldce_fwd(to_dev(h, dev), to_dev(W, dev), torch.from_numpy(t).to(dev),
                        torch.from_numpy(p).to(dev), label_smoothing=w.label_smoothing,
                        logit_scale=w.logit_scale, reduction=w.reduction, total=w.total,
                        row_stats=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(f["row_lse"]), host(r["row_lse"]))
    assert float(f["loss"].item()) == float(r["loss"].item())


@pytest.mark.parametrize("eps", [0.5, 0.75, 1.0])
@pytest.mark.parametrize("chunk", [0, 100])
def test_large_label_smoothing_flat_softmax(eps, chunk):
    """Label smoothing up to 1 on nearly flat softmax rows (tiny logits), where
    the smoothing share eps / V is most of every gradient entry: up to 1/2 the
    exponentials are the backward operand and the share is added to the
    products; above it the gradient is formed from the stored logits before
    its one rounding.  fwd_bwd (one chunk and chunked) and a vocabulary
    shard's backward against the oracle."""
    w = synth.custom(f"flat_eps_bf16", 1, 160, 128, 2000, label_smoothing=eps, logit_scale=0.5,
                     reduction="sum", index=410)
    r, o, t = _run(w, chunk_rows=chunk)
    _compare(w, r, o, t)
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    h, W = synth.hidden(w), synth.weight(w)
    tt, p = synth.targets(w)
    v0, Vl = 500, 777
    say(f"case shard bwd eps={eps}")
    b = fldce.fldce_shard_bwd(to_dev(h, dev), to_dev(W, dev)[v0:v0 + Vl].contiguous(),
                              torch.from_numpy(tt).to(dev), torch.from_numpy(p).to(dev),
                              torch.from_numpy(o["lse"].astype(np.float32)).to(dev), v0, w.V,
                              label_smoothing=eps, logit_scale=0.5, reduction="sum",
                              chunk_rows=chunk)
    torch.cuda.synchronize()
    odh, odw = O.shard_backward(h.values, W.values[v0:v0 + Vl], tt, p, o["lse"], v0, w.V, 1.0,
                                eps, 0.5)
    assert grad_err(host(b["dH_partial"]), odh) <= GRAD_RTOL["bf16"]
    assert grad_err(host(b["dW_local"]), odw) <= GRAD_RTOL["bf16"]


def test_all_ignored():
    w = synth.custom("all_ignored_bf16", 1, 200, 128, 500, total_is_N=False)
    t = np.full(w.N, -100, dtype=np.int64)
    p = np.zeros(w.N, dtype=np.float32)      # never read on ignored rows
    r, o, _ = _run(w, target=t, p_mask=p)
    assert o["loss"] == 0.0
    _compare(w, r, o, t)


def test_empty_batch():
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    say("case empty: N=0")
    W = torch.randn(300, 128, device=dev).to(torch.bfloat16)
    h = torch.empty(0, 128, device=dev, dtype=torch.bfloat16)
    t = torch.empty(0, dtype=torch.int64, device=dev)
    dW = torch.full_like(W, 7.0)
    r = fldce.fldce_fwd_bwd(h, W, t, out={"dW": dW})
    torch.cuda.synchronize()
    assert r["loss"].item() == 0.0 and torch.all(r["dW"] == 0)


def test_ignored_rows_do_not_leak():
    """Changing h and p_mask of ignored rows leaves loss and dW bit-identical."""
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    w = synth.custom("leak_bf16", 2, 150, 128, 900, label_smoothing=0.1)
    t, p = synth.targets(w)
    h, W = synth.hidden(w), synth.weight(w)
    say("case ignored-leak")
    hd, Wd = to_dev(h, dev), to_dev(W, dev)
    td, pd = torch.from_numpy(t).to(dev), torch.from_numpy(p).to(dev)
    a = fldce.fldce_fwd_bwd(hd, Wd, td, pd, label_smoothing=0.1, total=w.N)
    ig = torch.from_numpy(t == -100).to(dev)
    h2 = hd.clone()
    h2[ig] = 3.0
    p2 = pd.clone()
    p2[ig] = 0.0
    b = fldce.fldce_fwd_bwd(h2, Wd, td, p2, label_smoothing=0.1, total=w.N)
    torch.cuda.synchronize()
    assert torch.equal(a["loss"], b["loss"])
    assert torch.equal(a["dW"], b["dW"])
    assert torch.equal(a["dH"], b["dH"])


def test_deterministic_repeat():
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    w = synth.custom("repeat_bf16", 4, 200, 256, 3000, label_smoothing=0.1, logit_scale=0.5)
    t, p = synth.targets(w)
    args = (to_dev(synth.hidden(w), dev), to_dev(synth.weight(w), dev),
            torch.from_numpy(t).to(dev), torch.from_numpy(p).to(dev))
    say("case repeat")
    a = fldce.fldce_fwd_bwd(*args, label_smoothing=0.1, logit_scale=0.5, total=w.N)
    b = fldce.fldce_fwd_bwd(*args, label_smoothing=0.1, logit_scale=0.5, total=w.N)
    torch.cuda.synchronize()
    for k in ("loss", "dH", "dW"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_vocab_shards_match_full_vocab(dtype):
    """Three shards of a 1200-row vocabulary: partials vs the oracle's, host
    combine vs the full-vocabulary oracle, shard backward vs the oracle's, and
    the shard gradients reassemble the full dH and dW."""
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    w = synth.custom("shards_" + dtype, 3, 110, 128, 1200, dtype=dtype, shards=3,
                     label_smoothing=0.1, logit_scale=0.5)
    t, p = synth.targets(w)
    h = synth.hidden(w)
    Wfull = synth.weight(w)
    hd, td, pd = to_dev(h, dev), torch.from_numpy(t).to(dev), torch.from_numpy(p).to(dev)
    full = O.forward_backward(h.values, Wfull.values, t, p, label_smoothing=0.1, logit_scale=0.5,
                              total=w.N)
    parts = []
    tol = 1e-5 if dtype == "f32" else 2e-3
    for k in range(3):
        Wk = synth.weight(w, shard=k)
        v0 = k * w.V_local
        say(f"case shard partials k={k} {dtype}")
        r = fldce.fldce_shard_partials(hd, to_dev(Wk, dev), td, v0, logit_scale=0.5)
        torch.cuda.synchronize()
        m, S, tl, rs = (host(r[x]) for x in ("row_max", "row_sumexp", "target_logit", "row_sumlogit"))
        om, oS, ot, orr = O.shard_partials(h.values, Wk.values, t, v0, 0.5)
        valid = t != -100
        # rows whose target is ignore_index are skipped: (-inf, 0, 0, 0)
        assert np.all(np.isneginf(m[~valid])) and np.all(S[~valid] == 0)
        assert np.all(tl[~valid] == 0) and np.all(rs[~valid] == 0)
        np.testing.assert_allclose(m[valid], om[valid], atol=tol * 4, rtol=0)
        np.testing.assert_allclose(np.log(S[valid]) + m[valid], np.log(oS[valid]) + om[valid],
                                   atol=tol * 4, rtol=0)
        np.testing.assert_allclose(tl, ot, atol=tol * 4, rtol=0)
        np.testing.assert_allclose(rs[valid], orr[valid], atol=tol * 40, rtol=tol)
        assert np.all(tl[(t < v0) | (t >= v0 + w.V_local)] == 0.0)
        parts.append((m, S, tl, rs))
    valid = t != -100
    with np.errstate(invalid="ignore", divide="ignore"):
        lse, zt, zs = O.combine_shard_partials(parts)
    np.testing.assert_allclose(lse[valid], full["lse"][valid], atol=tol * 4, rtol=0)
    rl = O.row_losses(np.where(valid, lse, 0.0), zt, zs, w.V, p, valid, 0.1)
    loss = O.loss_from_row_losses(rl, float(w.N))
    assert abs(loss - full["loss"]) <= LOSS_RTOL[dtype] * abs(full["loss"])
    # shard backward from the oracle's global lse
    lse_d = torch.from_numpy(full["lse"].astype(np.float32)).to(dev)
    dH = np.zeros_like(full["dH"])
    dWs = []
    for k in range(3):
        Wk = synth.weight(w, shard=k)
        v0 = k * w.V_local
        say(f"case shard bwd k={k} {dtype}")
        r = fldce.fldce_shard_bwd(hd, to_dev(Wk, dev), td, pd, lse_d, v0, w.V,
                                  label_smoothing=0.1, logit_scale=0.5, total=w.N)
        torch.cuda.synchronize()
        odh, odw = O.shard_backward(h.values, Wk.values, t, p, full["lse"], v0, w.V, float(w.N),
                                    0.1, 0.5)
        gh, gw = host(r["dH_partial"]), host(r["dW_local"])
        assert grad_err(gh, odh) <= GRAD_RTOL[dtype]
        assert grad_err(gw, odw) <= GRAD_RTOL[dtype]
        assert np.all(gh[~valid] == 0.0)
        dH += gh
        dWs.append(gw)
    assert grad_err(dH, full["dH"]) <= GRAD_RTOL[dtype]
    assert grad_err(np.concatenate(dWs), full["dW"]) <= GRAD_RTOL[dtype]


# Edge shapes: a single token, V smaller than one 128-wide slab, one vocabulary
# row, H = 64 (one K step), token counts one past a tile and one short of a
# 64-row block, vocabularies one past / short of 256 and 1024, and the
# counted mean; each against the oracle element by element.
EDGE_CASES = [
    synth.custom("one_token", 1, 1, 64, 300),
    synth.custom("v_lt_slab", 2, 40, 128, 100, label_smoothing=0.1),
    synth.custom("v_one", 1, 30, 64, 1),
    synth.custom("h64_v257", 1, 257, 64, 257, logit_scale=0.3, total_is_N=False),
    synth.custom("n63_v1023", 1, 63, 192, 1023, label_smoothing=0.2, reduction="sum"),
    synth.custom("n513_v1025", 1, 513, 128, 1025, label_smoothing=0.05, logit_scale=2.0),
    synth.custom("n1_f32", 1, 1, 33, 77, dtype="f32", label_smoothing=0.3),
    synth.custom("v_one_f32", 1, 9, 16, 1, dtype="f32"),
]


@pytest.mark.parametrize("w", EDGE_CASES, ids=lambda w: w.name)
def test_edge_shapes(w):
    r, o, t = _run(w)
    if w.V > 1:
        _compare(w, r, o, t)
        return
    # one class: the loss and every gradient are exactly 0 mathematically; the
    # kernels leave only rounding (lse and the stored logit differ in the last
    # bits), bounded by 1e-2 of the gradients' natural scale c_i |W|, sum c_i |h|
    valid = t != -100
    _, p = synth.targets(w)
    c = np.where(valid, w.logit_scale / (p * O.divisor(valid, w.reduction, w.total or None)), 0.0)
    h, W = synth.hidden(w).values, synth.weight(w).values
    assert abs(float(r["loss"].item())) <= 1e-4
    assert np.abs(host(r["dH"])).max() <= 1e-2 * c.max() * np.abs(W).max()
    assert np.abs(host(r["dW"])).max() <= 1e-2 * (c[:, None] * np.abs(h)).sum(axis=0).max()
    assert np.all(host(r["dH"])[~valid] == 0.0)
