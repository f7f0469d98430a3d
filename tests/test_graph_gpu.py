"""HIP graph capture of the entry points.

Each entry point only enqueues kernel launches on the caller's stream: no
allocation, memset, copy or synchronisation happens inside a call, and the
row count, the divisor and every data-dependent choice are taken on the
device.  So a call captured into a graph (torch.cuda.graph, which captures
the current HIP stream) and replayed must reproduce, bit for bit, what an
eager call gives on the same input values, also when other input values
(another ignore pattern, hence another number of rows that reach the GEMMs)
are copied into the captured buffers between replays, and with unrelated
eager work and synchronisations between the replays."""

import dataclasses

import numpy as np
import pytest

from lm_head_linear_bf16_amd import synth
from _helpers import say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


def _sets(w, n_sets=2, shard=None):
    """Input value sets of one shape: the recipe under seeds index, index + 1."""
    out = []
    for k in range(n_sets):
        wk = dataclasses.replace(w, index=w.index + k)
        target, p_mask = synth.targets(wk)
        Wt = synth.weight(wk) if shard is None else synth.weight(wk, shard=shard)
        out.append(dict(h=synth.hidden(wk), W=Wt, b=synth.bias(wk), target=target,
                        p_mask=p_mask))
    return out


def _load(static, s, dev):
    """Copy one value set into the captured input buffers."""
    torch = torch_cuda()
    static["h"].copy_(to_dev(s["h"], dev))
    static["W"].copy_(to_dev(s["W"], dev))
    static["b"].copy_(to_dev(s["b"], dev))
    static["target"].copy_(torch.from_numpy(s["target"]).to(dev))
    static["p_mask"].copy_(torch.from_numpy(s["p_mask"]).to(dev))


def _snapshot(r):
    return {k: v.clone() for k, v in r.items() if v is not None}


def _run_graph_case(name, w, call, shard=None):
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    sets = _sets(w, shard=shard)
    n_valid = [int(np.count_nonzero(s["target"] != -100)) for s in sets]
    assert n_valid[0] != n_valid[1], "the two value sets should differ in rows that reach the GEMMs"
    s0 = sets[0]
    static = dict(h=to_dev(s0["h"], dev), W=to_dev(s0["W"], dev), b=to_dev(s0["b"], dev),
                  target=torch.from_numpy(s0["target"]).to(dev),
                  p_mask=torch.from_numpy(s0["p_mask"]).to(dev))
    say(f"case {name}: eager references, N={w.N} H={w.H} V={w.V} {w.dtype} rows {n_valid}")
    want = []
    for s in sets:
        _load(static, s, dev)
        want.append(_snapshot(call(static)))
        torch.cuda.synchronize()
    _load(static, sets[0], dev)
    # warm up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say(f"case {name}: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        got = call(static)
    torch.cuda.synchronize()
    noise = torch.randn(1 << 20, device=dev)
    for rep, k in enumerate([0, 1, 0, 1]):
        _load(static, sets[k], dev)
        for v in got.values():
            if v is not None:
                v.fill_(float("nan"))
        float((noise * rep).sum())   # unrelated eager work and a synchronisation
        say(f"case {name}: replay {rep} on value set {k}")
        g.replay()
        torch.cuda.synchronize()
        for key, ref in want[k].items():
            assert torch.equal(got[key], ref), f"{name}: replay {rep}: {key} differs from eager"
    del g


def _static_out(static):
    torch = torch_cuda()
    h, W = static["h"], static["W"]
    return dict(loss=torch.empty(1, dtype=torch.float32, device=h.device),
                dH=torch.empty_like(h), dW=torch.empty_like(W))


def test_graph_fwd_bwd_chunked_bf16():
    """Chunks of 64 rows (167 of the 684 rows have a target in the first value
    set): the first chunk, later ones carried in fp32, the final one found on
    the device, empty chunks after it; split-K dH with its reduction, and the
    device-side row count."""
    from lm_head_linear_bf16_amd import fldce
    torch = torch_cuda()
    w = synth.custom("graph_chunked_bf16", 4, 171, 192, 3001, label_smoothing=0.1,
                     logit_scale=0.5, total_is_N=False, index=300)
    dev = torch.device("cuda:0")
    ws = torch.empty(fldce.fldce_workspace_size(w.N, w.H, w.V, torch.bfloat16, 64),
                     dtype=torch.uint8, device=dev)
    box = {}

    def call(st):
        if "out" not in box:
            box["out"] = _static_out(st)
        r = fldce.fldce_fwd_bwd(st["h"], st["W"], st["target"], st["p_mask"],
                                label_smoothing=w.label_smoothing, logit_scale=w.logit_scale,
                                reduction=w.reduction, total=w.total, chunk_rows=64,
                                row_stats=True, workspace=ws, out=box["out"])
        return r
    _run_graph_case("fwd_bwd_chunked_bf16", w, call)


def test_graph_fwd_bwd_ex_bias_eob_bf16():
    from lm_head_linear_bf16_amd import fldce
    torch = torch_cuda()
    w = synth.custom("graph_ex_bf16", 3, 111, 128, 2053, label_smoothing=0.2, logit_scale=1.3,
                     index=310)
    dev = torch.device("cuda:0")
    ws = torch.empty(fldce.fldce_workspace_size(w.N, w.H, w.V, torch.bfloat16),
                     dtype=torch.uint8, device=dev)

    def call(st):
        return fldce.fldce_fwd_bwd_ex(st["h"], st["W"], st["target"], st["p_mask"], st["b"],
                                      label_smoothing=w.label_smoothing,
                                      logit_scale=w.logit_scale, reduction=w.reduction,
                                      total=w.total, eob_token_id=7, eob_weight=2.5,
                                      want_db=True, row_stats=True, workspace=ws)
    _run_graph_case("fwd_bwd_ex_bias_eob_bf16", w, call)


def test_graph_fwd_f32():
    from lm_head_linear_bf16_amd import fldce
    torch = torch_cuda()
    w = synth.custom("graph_fwd_f32", 2, 90, 80, 777, dtype="f32", label_smoothing=0.1,
                     index=320, total_is_N=False)
    dev = torch.device("cuda:0")
    ws = torch.empty(fldce.fldce_fwd_workspace_size(w.N, w.H, w.V, torch.float32),
                     dtype=torch.uint8, device=dev)

    def call(st):
        return fldce.fldce_fwd(st["h"], st["W"], st["target"], st["p_mask"], st["b"],
                               label_smoothing=w.label_smoothing, logit_scale=w.logit_scale,
                               reduction=w.reduction, total=w.total, row_stats=True,
                               workspace=ws)
    _run_graph_case("fwd_f32", w, call)


def test_graph_shard_partials_and_bwd_bf16():
    """One vocabulary shard: partials, then the backward from an lse that the
    graph itself derives from the partials (a torch op between the two calls)."""
    from lm_head_linear_bf16_amd import fldce
    torch = torch_cuda()
    w = synth.custom("graph_shard_bf16", 3, 120, 128, 1500, shards=3, label_smoothing=0.1,
                     index=330)
    k, v0 = 1, 500
    Vl = 500
    dev = torch.device("cuda:0")
    ws_p = torch.empty(fldce.fldce_shard_partials_workspace_size(w.N, w.H, Vl, torch.bfloat16),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(fldce.fldce_shard_bwd_workspace_size(w.N, w.H, Vl, torch.bfloat16),
                       dtype=torch.uint8, device=dev)

    def call(st):
        p = fldce.fldce_shard_partials(st["h"], st["W"], st["target"], v0, logit_scale=1.0,
                                       workspace=ws_p)
        lse = (p["row_max"] + torch.log(p["row_sumexp"])).nan_to_num(0.0, 0.0, 0.0)
        b = fldce.fldce_shard_bwd(st["h"], st["W"], st["target"], st["p_mask"], lse, v0, w.V,
                                  label_smoothing=w.label_smoothing, reduction=w.reduction,
                                  total=w.total, workspace=ws_b)
        return {**{"p_" + key: v for key, v in p.items()}, **{"b_" + key: v for key, v in b.items()}}
    _run_graph_case("shard_bf16", w, call, shard=k)
