"""The allocation-free forward (fldce_fwd_noalloc: the library's own device
array instead of a workspace) against fldce_fwd with a workspace, through the
C ABI: two calls in a row on one device, the second with a smaller input (the
array keeps the first call's contents), bf16 and fp32, with and without bias,
label smoothing and an end-of-block weight.  Both run the same kernels, so
the results must agree bit for bit."""

import numpy as np
import pytest

from lm_head_linear_bf16_amd import synth
from _helpers import say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


def _case(w, dev, with_bias):
    import torch
    t, p = synth.targets(w)
    h, W = to_dev(synth.hidden(w), dev), to_dev(synth.weight(w), dev)
    b = to_dev(synth.bias(w), dev) if with_bias else None
    return h, W, b, torch.from_numpy(t).to(dev), torch.from_numpy(p).to(dev)


def _compare(fldce, torch, dev, w, with_bias, eob):
    h, W, b, t, p = _case(w, dev, with_bias)
    kw = dict(label_smoothing=w.label_smoothing, logit_scale=w.logit_scale,
              reduction=w.reduction, total=w.total, row_stats=True)
    if eob is not None:
        kw.update(eob_token_id=eob, eob_weight=2.5)
    N = w.N
    # outputs allocated before the call: the entry point itself allocates nothing
    out = dict(loss=torch.full((1,), float("nan"), device=dev),
               row_lse=torch.full((N,), float("nan"), device=dev),
               row_loss=torch.full((N,), float("nan"), device=dev))
    say(f"case noalloc {w.name}: N={N} H={w.H} V={w.V} {w.dtype} bias={with_bias} eob={eob}")
    na = fldce.fldce_fwd_noalloc(h, W, t, p, b, out=out, **kw)
    ref = fldce.fldce_fwd(h, W, t, p, b, **kw)
    torch.cuda.synchronize()
    for k in ("loss", "row_lse", "row_loss"):
        got, want = na[k].cpu().numpy(), ref[k].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), k
    say(f"  loss {float(na['loss'].item()):.7g} (bitwise equal to fldce_fwd)")


def test_noalloc_two_calls_second_smaller():
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    big = synth.custom("noalloc_big", 2, 1024, 2560, 151936, label_smoothing=0.1, logit_scale=0.5,
                       index=301)
    small = synth.custom("noalloc_small", 1, 300, 1024, 50000, index=302)
    assert fldce.fldce_fwd_workspace_size(big.N, big.H, big.V, 1) <= fldce.NOALLOC_SCRATCH_BYTES
    _compare(fldce, torch, dev, big, with_bias=False, eob=None)
    _compare(fldce, torch, dev, small, with_bias=True, eob=7)


def test_noalloc_fp32_then_smaller_bf16():
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    _compare(fldce, torch, dev, synth.WORKLOADS["tiny"], with_bias=True, eob=None)
    w = synth.custom("noalloc_b16", 1, 100, 128, 3001, label_smoothing=0.2, logit_scale=2.0,
                     index=303)
    _compare(fldce, torch, dev, w, with_bias=False, eob=11)


def test_noalloc_rejects_oversized_calls_before_launching():
    torch = torch_cuda()
    from lm_head_linear_bf16_amd import fldce
    dev = torch.device("cuda:0")
    N, H, V = 3379, 2560, 151936
    h = torch.zeros(N, H, dtype=torch.bfloat16, device=dev)
    W = torch.zeros(V, H, dtype=torch.bfloat16, device=dev)
    t = torch.zeros(N, dtype=torch.int64, device=dev)
    loss = torch.full((1,), 7.0, device=dev)
    with pytest.raises(fldce.FldceError) as e:
        fldce.fldce_fwd_noalloc(h, W, t, out=dict(loss=loss))
    assert e.value.status == -9
    torch.cuda.synchronize()
    assert float(loss.item()) == 7.0   # nothing was enqueued
