"""The C-ABI library loads, exports every symbol include/fldce.h declares, and
rejects invalid arguments before touching the GPU.  CPU only: no compute call
reaches a kernel here (every call below fails host-side validation)."""

import ctypes
import os
import re

import pytest

from lm_head_linear_bf16_amd import fldce

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fldce.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fldce_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fldce.LIB_PATH):
        pytest.skip("libfldce.so not built")
    return fldce.lib()


def test_every_declared_symbol_is_exported_and_bound(L):
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
        assert n in fldce._SIGNATURES, f"binding lacks {n}"
        assert hasattr(fldce, n) or n in ("fldce_status_string",), f"python name {n}"


def test_header_is_a_c_abi(L, tmp_path):
    """The header compiles as strict C99, and a C program that takes the
    address of every declared entry point links against libfldce.so and
    calls the two host-only ones (no GPU needed)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    names = _declared()
    src = tmp_path / "abi.c"
    src.write_text(
        '#include "fldce.h"\n#include <stdio.h>\n'
        "typedef void (*fn_t)(void);\n"
        "int main(void) {\n"
        "  static const fn_t all[] = {" + ", ".join(f"(fn_t){n}" for n in names) + "};\n"
        '  printf("%d %s %d\\n", fldce_version(), fldce_status_string(0),\n'
        "         (int)(sizeof(all) / sizeof(all[0])));\n"
        "  return 0;\n}\n")
    exe = tmp_path / "abi"
    libdir = os.path.dirname(fldce.LIB_PATH)
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-Wno-cast-function-type", "-I", os.path.join(ROOT, "include"), str(src),
                    "-o", str(exe), "-L", libdir, "-l:" + os.path.basename(fldce.LIB_PATH),
                    "-Wl,-rpath," + libdir], check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    assert out[0] == str(fldce.fldce_version()) and out[1] == "ok" and int(out[2]) == len(names)


def test_status_strings(L):
    assert fldce.status_string(0) == "ok"
    for s in range(-9, 0):
        assert fldce.status_string(s) != "unknown status"
    assert fldce.status_string(-99) == "unknown status"
    assert fldce.fldce_version() == 2


def test_workspace_queries(L):
    a = fldce.fldce_workspace_size(8192, 2560, 151936, 1)
    b = fldce.fldce_workspace_size(8192, 2560, 151936, 1, 1024)
    assert a > b > 0
    assert fldce.fldce_workspace_size(0, 64, 10, 1) > 0
    assert fldce.fldce_workspace_size(-1, 64, 10, 1) == 0
    assert fldce.fldce_workspace_size(10, 64, 10, 7) == 0
    assert fldce.fldce_workspace_size(1 << 28, 64, 10, 1) == 0
    assert fldce.fldce_fwd_workspace_size(10, 64, 1 << 31, 1) == 0
    assert fldce.fldce_shard_bwd_workspace_size(10, (1 << 20) + 64, 10, 1) == 0
    assert fldce.fldce_shard_partials_workspace_size(32768, 5120, 18992, 1) > 0
    assert fldce.fldce_shard_bwd_workspace_size(32768, 5120, 18992, 1) > 0
    assert fldce.fldce_default_chunk_rows(8192, 2560, 151936) == 8192
    # a vocabulary too large for one chunk of all rows gets a multiple of 256
    c = fldce.fldce_default_chunk_rows(1 << 20, 4096, 151936)
    assert 0 < c < (1 << 20) and c % 256 == 0


P = 0x10000          # fake, aligned "device" addresses: validation fails first
BAD = 0x10001        # misaligned


def _fwd(L, **kw):
    a = dict(h=P, W=P, target=P, p_mask=None, N=16, H=64, V=100, dtype=1, ignore=-100, eps=0.0,
             s=1.0, red=1, total=0, loss=P, dH=P, dW=P, lse=None, rl=None, chunk=0, ws=P,
             wsb=1 << 40, stream=None)
    a.update(kw)
    return L.fldce_fwd_bwd(a["h"], a["W"], a["target"], a["p_mask"], a["N"], a["H"], a["V"],
                           a["dtype"], a["ignore"], a["eps"], a["s"], a["red"], a["total"],
                           a["loss"], a["dH"], a["dW"], a["lse"], a["rl"], a["chunk"], a["ws"],
                           a["wsb"], a["stream"])


def test_fwd_bwd_argument_checks(L):
    assert _fwd(L, W=None) == -1
    assert _fwd(L, h=None) == -1
    assert _fwd(L, loss=None) == -1
    assert _fwd(L, dH=None) == -1            # both gradients are required outputs here
    assert _fwd(L, dW=None) == -1
    assert _fwd(L, dtype=3) == -3
    assert _fwd(L, N=-1) == -2
    assert _fwd(L, V=0) == -2
    assert _fwd(L, H=0) == -2
    assert _fwd(L, N=1 << 28) == -2          # documented range: N < 2^28, V < 2^31, H <= 2^20
    assert _fwd(L, V=1 << 31) == -2
    assert _fwd(L, H=(1 << 20) + 64) == -2
    assert _fwd(L, red=2) == -4
    assert _fwd(L, eps=-0.1) == -4
    assert _fwd(L, eps=1.5) == -4
    assert _fwd(L, eps=float("nan")) == -4
    assert _fwd(L, s=0.0) == -4
    assert _fwd(L, s=-1.0) == -4
    assert _fwd(L, s=float("inf")) == -4
    assert _fwd(L, chunk=-5) == -4
    assert _fwd(L, h=BAD) == -6
    assert _fwd(L, dW=BAD) == -6
    assert _fwd(L, wsb=16) == -5
    assert _fwd(L, ws=None) == -5
    assert _fwd(L, H=100) == -8          # bf16 needs H % 64 == 0
    assert _fwd(L, V=(1 << 31) - 1, N=1 << 20) == -8   # logits grid past 2^32 work-items
    assert _fwd(L, H=100, dtype=0, wsb=16) == -5   # fp32 takes any H (fails later on workspace)
    assert _fwd(L, V=1 << 30, dtype=0) == -8    # fp32 grids hold 4 work-items per vocabulary row


def test_shard_argument_checks(L):
    f = L.fldce_shard_partials
    assert f(P, P, P, 16, 64, 100, -1, 1, -100, 1.0, P, P, P, None, P, 1 << 40, None) == -2
    assert f(P, P, P, 16, 64, 100, 0, 1, -100, 1.0, None, P, P, None, P, 1 << 40, None) == -1
    assert f(P, P, P, 16, 64, 100, 0, 1, -100, 0.0, P, P, P, None, P, 1 << 40, None) == -4
    assert f(P, P, P, 16, 64, 100, 0, 1, -100, 1.0, P, P, P, None, P, 8, None) == -5
    b = L.fldce_shard_bwd
    base = [P, P, P, None, P, 16, 64, 100, 0, 1000, 1, -100, 0.0, 1.0, 1, 0, P, P, 0, P, 1 << 40, None]

    def call(**over):
        a = list(base)
        idx = dict(vocab_start=8, V_global=9, red=14, eps=12, lse=4, ws_bytes=20, dHp=16)
        for k, v in over.items():
            a[idx[k]] = v
        return b(*a)
    assert call(V_global=50) == -2        # shard [0, 100) outside a 50-row vocabulary
    assert call(vocab_start=950) == -2
    assert call(red=5) == -4
    assert call(eps=2.0) == -4
    assert call(lse=None) == -1
    assert call(dHp=BAD) == -6
    assert call(ws_bytes=1) == -5


def _ex(L, **kw):
    a = dict(h=P, W=P, bias=None, target=P, p_mask=None, N=16, H=64, V=100, dtype=1, ignore=-100,
             eps=0.0, s=1.0, red=1, total=0, eob=-1, eob_w=1.0, loss=P, dH=P, dW=P, db=None,
             lse=None, rl=None, chunk=0, ws=P, wsb=1 << 40, stream=None)
    a.update(kw)
    return L.fldce_fwd_bwd_ex(*a.values())


def _fwd_only(L, **kw):
    a = dict(h=P, W=P, bias=None, target=P, p_mask=None, N=16, H=64, V=100, dtype=1, ignore=-100,
             eps=0.0, s=1.0, red=1, total=0, eob=-1, eob_w=1.0, loss=P, lse=None, rl=None, ws=P,
             wsb=1 << 40, stream=None)
    a.update(kw)
    return L.fldce_fwd(*a.values())


def _fwd_noalloc(L, **kw):
    a = dict(h=P, W=P, bias=None, target=P, p_mask=None, N=16, H=64, V=100, dtype=1, ignore=-100,
             eps=0.0, s=1.0, red=1, total=0, eob=-1, eob_w=1.0, loss=P, lse=None, rl=None,
             stream=None)
    a.update(kw)
    return L.fldce_fwd_noalloc(*a.values())


def test_noalloc_argument_checks(L):
    """The allocation-free forward rejects what fldce_fwd rejects, and any
    call whose intermediates exceed its fixed device array, before it looks
    at a device."""
    f = _fwd_noalloc
    assert f(L, W=None) == -1
    assert f(L, loss=None) == -1
    assert f(L, dtype=2) == -3
    assert f(L, N=-1) == -2
    assert f(L, red=3) == -4
    assert f(L, s=0.0) == -4
    assert f(L, eob=5, eob_w=-1.0) == -4
    assert f(L, bias=BAD) == -6
    assert f(L, H=96) == -8
    lim = fldce.NOALLOC_SCRATCH_BYTES
    assert fldce.fldce_fwd_workspace_size(3378, 2560, 151936, 1) <= lim
    assert fldce.fldce_fwd_workspace_size(3379, 2560, 151936, 1) > lim
    assert f(L, N=3379, H=2560, V=151936) == -9
    assert f(L, N=8192, H=2560, V=151936) == -9
    assert "FLDCE_NOALLOC_SCRATCH_BYTES" in fldce.status_string(-9)
    assert f"((size_t){lim >> 20} << 20)" in open(HEADER).read()


@pytest.mark.parametrize("f", [_ex, _fwd_only])
def test_extended_argument_checks(L, f):
    assert f(L, W=None) == -1
    assert f(L, loss=None) == -1
    assert f(L, dtype=2) == -3
    assert f(L, red=3) == -4
    assert f(L, eps=2.0) == -4
    assert f(L, eob=5, eob_w=-1.0) == -4          # weight must be >= 0
    assert f(L, eob=5, eob_w=float("nan")) == -4
    assert f(L, eob=5, eob_w=float("inf")) == -4
    assert f(L, eob=-1, eob_w=-1.0, wsb=8) == -5  # no EOB: the weight is not checked
    assert f(L, bias=BAD) == -6
    assert f(L, H=96) == -8
    assert f(L, V=1 << 23) == -8                  # bf16 reads its operands through buffers
    assert f(L, V=(1 << 23) - 1, wsb=8) == -5     # just below: fails on the workspace only
    assert f(L, wsb=8) == -5
    if f is _ex:
        assert f(L, db=BAD) == -6
        assert f(L, dH=None, wsb=8) == -5         # dH / dW optional here: fails on the workspace
        assert f(L, dW=None, wsb=8) == -5
        assert f(L, dH=None, dW=None, wsb=8) == -5
        assert f(L, dW=BAD) == -6
        assert f(L, chunk=-1) == -4


def test_fwd_workspace_query(L):
    a = fldce.fldce_fwd_workspace_size(8192, 2560, 151936, 1)
    assert 0 < a < fldce.fldce_workspace_size(8192, 2560, 151936, 1)
    assert fldce.fldce_fwd_workspace_size(-1, 64, 10, 1) == 0
    assert fldce.fldce_fwd_workspace_size(4, 64, 10, 5) == 0


def test_scale_grads_argument_checks(L):
    f = L.fldce_scale_grads
    assert f(None, 1, P, 16, None, 0, None, 0, None) == -1
    assert f(P, 4, P, 16, None, 0, None, 0, None) == -3
    assert f(P, 1, P, -1, None, 0, None, 0, None) == -2
    assert f(P, 1, None, 16, None, 0, None, 0, None) == -1
    assert f(P, 1, P, 16, BAD, 8, None, 0, None) == -6
    assert f(BAD, 1, P, 16, None, 0, None, 0, None) == -6


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    h = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fldce.fldce_fwd_bwd(h, h, torch.zeros(4, dtype=torch.int64))


def test_binding_checks_sizes_before_any_call():
    """Every input size a kernel relies on is checked in the binding (sizes
    first, so the checks run here on host tensors): W's columns, target /
    p_mask / lse / bias lengths.  Caller-given outputs: tests/test_parity_ext_gpu.py."""
    torch = pytest.importorskip("torch")
    bf = torch.bfloat16
    h, W = torch.zeros(4, 64, dtype=bf), torch.zeros(10, 64, dtype=bf)
    t = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(ValueError, match="columns"):
        fldce.fldce_fwd_bwd(h, torch.zeros(10, 128, dtype=bf), t)
    with pytest.raises(ValueError, match="target must hold 4"):
        fldce.fldce_fwd_bwd(h, W, torch.zeros(3, dtype=torch.int64))
    with pytest.raises(ValueError, match="p_mask must hold 4"):
        fldce.fldce_fwd(h, W, t, torch.ones(5))
    with pytest.raises(ValueError, match="bias must hold 10"):
        fldce.fldce_fwd_bwd_ex(h, W, t, None, torch.zeros(9, dtype=bf))
    with pytest.raises(ValueError, match="lse must hold 4"):
        fldce.fldce_shard_bwd(h, W, t, None, torch.zeros(2), 0, 10)
    with pytest.raises(ValueError, match="2-D"):
        fldce.fldce_shard_partials(h.view(-1), W, t, 0)
