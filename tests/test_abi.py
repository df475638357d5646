"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments with the documented status codes
before launching anything (so these run without a GPU)."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn97.h")

from exact_attention_97_amd import _lib as L  # noqa: E402

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libattn97.so not built")

OK, NULL, SHAPE, UNSUP, ALIGN, WS, HIP, VALUE, SCRATCH = range(9)
P = 0x10000  # a fake, 256-byte aligned device address: never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(attn_[a-z0-9_]+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = L.load()
    names = declared_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in attn97.h but not exported"
    assert set(names) == set(L.EXPORTS)


def test_version_and_strerror():
    lib = L.load()
    assert b"gfx950" in lib.attn_version()
    texts = {lib.attn_strerror(c) for c in range(9)}
    assert len(texts) == 9
    assert lib.attn_strerror(99) == b"unknown status"


def test_default_opts():
    lib = L.load()
    o = L.AttnOpts()
    o.exp_mode, o.poly_fraction, o.rescale_tau, o.bwd_mode = 7, 3.0, -1.0, 7
    lib.attn_default_opts(ctypes.byref(o))
    assert (o.exp_mode, o.poly_fraction, o.rescale_tau, o.bwd_mode) == (0, 0.5, 8.0, 1)
    # the struct layout of include/attn97.h: int, float, float, int
    assert [f[0] for f in L.AttnOpts._fields_] == ["exp_mode", "poly_fraction", "rescale_tau", "bwd_mode"]
    assert ctypes.sizeof(L.AttnOpts) == 16


def fwd(**kw):
    a = dict(Q=P, K=P, V=P, O=P, LSE=P, B=1, H=1, S=16, D=64, scale=0.125, causal=0, opts=None, stream=None)
    a.update(kw)
    opts = ctypes.byref(a["opts"]) if a["opts"] is not None else None
    return L.load().attn_fwd(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["H"], a["S"], a["D"],
                             a["scale"], a["causal"], opts, a["stream"])


def bwd(**kw):
    a = dict(Q=P, K=P, V=P, O=P, dO=P, LSE=P, dQ=P, dK=P, dV=P, ws=P, wsb=1 << 40, B=1, H=1, S=16, D=64,
             scale=0.125, causal=0, opts=None, stream=None)
    a.update(kw)
    opts = ctypes.byref(a["opts"]) if a["opts"] is not None else None
    return L.load().attn_bwd(a["Q"], a["K"], a["V"], a["O"], a["dO"], a["LSE"], a["dQ"], a["dK"], a["dV"],
                             a["ws"], a["wsb"], a["B"], a["H"], a["S"], a["D"], a["scale"], a["causal"],
                             opts, a["stream"])


@pytest.mark.parametrize("name", ["Q", "K", "V", "O", "LSE"])
def test_fwd_null(name):
    assert fwd(**{name: None}) == NULL


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), SHAPE), (dict(H=0), SHAPE), (dict(S=0), SHAPE), (dict(S=-3), SHAPE),
    (dict(D=32), UNSUP), (dict(D=96), UNSUP), (dict(D=512), UNSUP),
    (dict(B=1 << 10, H=1 << 10, S=1 << 10, D=64), SHAPE),
    (dict(Q=P + 8), ALIGN), (dict(V=P + 2), ALIGN), (dict(LSE=P + 4), ALIGN),
    (dict(scale=float("nan")), VALUE), (dict(scale=float("inf")), VALUE),
])
def test_fwd_rejects(kw, code):
    assert fwd(**kw) == code


def test_fwd_bad_options():
    assert fwd(opts=L.make_opts(exp_mode=3)) == UNSUP
    assert fwd(opts=L.make_opts(exp_mode=-1)) == UNSUP
    assert fwd(opts=L.make_opts(rescale_tau=-1.0)) == VALUE
    assert fwd(opts=L.make_opts(rescale_tau=float("nan"))) == VALUE
    assert fwd(opts=L.make_opts(rescale_tau=float("inf"))) == VALUE
    # tau above 64 could let 2^tau times S probabilities approach the fp32 range
    assert fwd(opts=L.make_opts(rescale_tau=64.5)) == VALUE
    assert fwd(opts=L.make_opts(rescale_tau=200.0)) == VALUE
    for frac in (-0.1, 1.01, float("nan"), float("inf")):
        assert fwd(opts=L.make_opts(exp_mode="mixed", poly_fraction=frac)) == VALUE
        assert fwd(opts=L.make_opts(exp_mode="native", poly_fraction=frac)) == VALUE


@pytest.mark.parametrize("name", ["Q", "K", "V", "O", "dO", "LSE", "dQ", "dK", "dV"])
def test_bwd_null(name):
    assert bwd(**{name: None}) == NULL


@pytest.mark.parametrize("kw,code", [
    (dict(S=0), SHAPE), (dict(D=48), UNSUP), (dict(dO=P + 8), ALIGN), (dict(dK=P + 2), ALIGN),
    (dict(scale=float("nan")), VALUE), (dict(ws=None), WS), (dict(wsb=16), WS), (dict(ws=P + 16), WS),
])
def test_bwd_rejects(kw, code):
    assert bwd(**kw) == code


def test_bwd_bad_options():
    assert bwd(opts=L.make_opts(bwd_mode=2)) == UNSUP


def test_bwd_d256_modes():
    # D = 256 runs in the split mode only; validation reaches the workspace check
    assert bwd(D=256, opts=L.make_opts(bwd_mode="atomic")) == UNSUP
    assert bwd(D=256, wsb=16, opts=L.make_opts(bwd_mode="split")) == WS


def test_workspace_bytes():
    lib = L.load()
    o = L.make_opts(bwd_mode="atomic")
    B, H, S, D = 2, 3, 100, 128
    delta = 2 * ((B * H * S * 4 + 255) // 256 * 256)  # Delta and -LSE log2e
    assert lib.attn_bwd_workspace_bytes(B, H, S, D, 0, ctypes.byref(o)) == delta + B * H * S * D * 4
    assert lib.attn_bwd_workspace_bytes(B, H, S, D, 1, ctypes.byref(o)) == delta + B * H * S * D * 4
    o.bwd_mode = 1
    assert lib.attn_bwd_workspace_bytes(B, H, S, D, 0, ctypes.byref(o)) == delta
    assert lib.attn_bwd_workspace_bytes(B, H, S, D, 1, None) == delta
    assert lib.attn_bwd_workspace_bytes(0, H, S, D, 0, None) == 0
    assert lib.attn_bwd_workspace_bytes(B, H, S, 80, 0, None) == 0


def test_exp2_eval_rejects():
    lib = L.load()
    assert lib.attn_exp2_eval(None, None, 0, 0, None) == OK  # empty: nothing launched
    assert lib.attn_exp2_eval(None, P, 4, 0, None) == NULL
    assert lib.attn_exp2_eval(P, P, -1, 0, None) == SHAPE
    assert lib.attn_exp2_eval(P, P, 4, 2, None) == UNSUP
    assert lib.attn_exp2_eval(P + 2, P, 4, 0, None) == ALIGN


def test_prof_hooks_without_launches():
    lib = L.load()
    assert lib.attn_prof_reset() == OK
    n, ms = ctypes.c_int(-1), ctypes.c_double(-1.0)
    assert lib.attn_prof_collect(b"fwd", ctypes.byref(n), ctypes.byref(ms)) == OK
    assert (n.value, ms.value) == (0, 0.0)
    assert lib.attn_prof_collect(b"nope", ctypes.byref(n), ctypes.byref(ms)) == UNSUP
    assert lib.attn_prof_collect(None, ctypes.byref(n), ctypes.byref(ms)) == NULL


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros((1, 1, 4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        L.attn_fwd(q, q, q)


def test_product_path_does_not_import_oracle():
    """The package and its sources never reference the oracle."""
    pkg = os.path.join(ROOT, "exact_attention_97_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in text and "from oracle" not in text, f


def test_splitkv_workspace_and_rejects():
    lib = L.load()
    # Sq=10, Sk=1000, D=128: 64-key tiles -> 16 tiles; 3 splits -> 6 tiles (384 keys) per split -> 3 splits
    B, H, Sq, Sk, D = 2, 3, 10, 1000, 128
    per = B * H * Sq
    want = ((3 * per * D * 4 + 255) // 256 * 256) + ((3 * per * 4 + 255) // 256 * 256)
    assert lib.attn_fwd_splitkv_workspace_bytes(B, H, Sq, Sk, D, 0, 3) == want
    # more splits than key tiles are clamped to one split per tile (16)
    want16 = ((16 * per * D * 4 + 255) // 256 * 256) + ((16 * per * 4 + 255) // 256 * 256)
    assert lib.attn_fwd_splitkv_workspace_bytes(B, H, Sq, Sk, D, 0, 1000) == want16
    assert lib.attn_fwd_splitkv_workspace_bytes(B, H, Sq, Sk, D, 0, 0) > 0
    assert lib.attn_fwd_splitkv_workspace_bytes(B, H, 20, 10, D, 1, 0) == 0  # causal, Sk < Sq
    assert lib.attn_fwd_splitkv_workspace_bytes(B, H, Sq, Sk, 80, 0, 0) == 0
    assert lib.attn_fwd_splitkv_workspace_bytes(B, H, Sq, Sk, D, 0, -1) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(Sq=0), SHAPE), (dict(D=48), UNSUP), (dict(O=P + 8), ALIGN), (dict(scale=float("nan")), VALUE),
    (dict(splits=-2), VALUE), (dict(causal=1, Sq=50, Sk=40), SHAPE), (dict(ws=None), WS), (dict(wsb=16), WS),
])
def test_splitkv_rejects(kw, code):
    lib = L.load()
    a = dict(Q=P, K=P, V=P, O=P, LSE=P, ws=P, wsb=1 << 40, B=1, H=1, Sq=4, Sk=40, D=64, scale=0.1, causal=0, splits=0)
    a.update(kw)
    assert lib.attn_fwd_splitkv(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["ws"], a["wsb"], a["B"], a["H"], a["Sq"],
                                a["Sk"], a["D"], a["scale"], a["causal"], a["splits"], None, None) == code


def bwd_noalloc(**kw):
    a = dict(Q=P, K=P, V=P, O=P, dO=P, LSE=P, dQ=P, dK=P, dV=P, B=1, H=1, S=16, D=64, scale=0.125, causal=0,
             opts=None, stream=None)
    a.update(kw)
    opts = ctypes.byref(a["opts"]) if a["opts"] is not None else None
    return L.load().attn_bwd_noalloc(a["Q"], a["K"], a["V"], a["O"], a["dO"], a["LSE"], a["dQ"], a["dK"], a["dV"],
                                     a["B"], a["H"], a["S"], a["D"], a["scale"], a["causal"], opts, a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), NULL), (dict(dV=None), NULL), (dict(S=0), SHAPE), (dict(D=96), UNSUP), (dict(dK=P + 2), ALIGN),
    (dict(scale=float("nan")), VALUE), (dict(D=256, opts=L.make_opts(bwd_mode="atomic")), UNSUP),
    # beyond the fixed scratch: split needs 2 * 4 bytes per row, atomic also 4 * D per row
    (dict(B=1, H=65, S=65536, D=64), SCRATCH),
    (dict(B=1, H=16, S=8192, D=128, opts=L.make_opts(bwd_mode="atomic")), SCRATCH),
])
def test_bwd_noalloc_rejects(kw, code):
    """Argument errors and the scratch limit are reported before any device call."""
    assert bwd_noalloc(**kw) == code


def test_noalloc_limit_matches_workspace_rule():
    lib = L.load()
    split = L.make_opts(bwd_mode="split")
    assert lib.attn_bwd_workspace_bytes(1, 65, 65536, 64, 0, ctypes.byref(split)) > L.NOALLOC_SCRATCH_BYTES
    assert lib.attn_bwd_workspace_bytes(1, 64, 65536, 64, 0, ctypes.byref(split)) == L.NOALLOC_SCRATCH_BYTES
    assert lib.attn_bwd_workspace_bytes(2, 16, 8192, 128, 0, ctypes.byref(split)) <= L.NOALLOC_SCRATCH_BYTES
    assert lib.attn_bwd_workspace_bytes(1, 32, 32768, 128, 0, ctypes.byref(split)) <= L.NOALLOC_SCRATCH_BYTES


def test_fp8_dot_eval_rejects():
    lib = L.load()
    assert lib.attn_fp8_dot_eval(P, P, P, 0, None) == OK  # nothing to do, nothing launched
    assert lib.attn_fp8_dot_eval(P, P, P, -1, None) == SHAPE
    assert lib.attn_fp8_dot_eval(None, P, P, 1, None) == NULL
    assert lib.attn_fp8_dot_eval(P, None, P, 1, None) == NULL
    assert lib.attn_fp8_dot_eval(P, P, None, 1, None) == NULL
    assert lib.attn_fp8_dot_eval(P + 8, P, P, 1, None) == ALIGN
    assert lib.attn_fp8_dot_eval(P, P, P + 4, 1, None) == ALIGN


def test_fp8_buffer_layout():
    lib = L.load()
    B, H, S, D = 2, 3, 200, 128
    Sp, BH = 256, 6
    r = lambda n: (n + 255) // 256 * 256
    # q8, k8, v8t, qs (per row), ks (per head), vs (per column), scratch (V column maxima, K head maxima)
    sizes = [r(BH * Sp * D), r(BH * Sp * D), r(BH * D * Sp), r(BH * Sp * 4), r(BH * 4), r(BH * D * 4),
             r(BH * D * 4) + r(BH * 8)]
    assert lib.attn_fp8_buffer_bytes(B, H, S, D) == sum(sizes)
    offs = (ctypes.c_size_t * 7)()
    assert lib.attn_fp8_buffer_offsets(B, H, S, D, offs) == OK
    assert list(offs) == [sum(sizes[:i]) for i in range(7)]
    assert lib.attn_fp8_buffer_bytes(B, H, S, 64) == 0
    assert lib.attn_fp8_buffer_offsets(B, H, S, 64, offs) == UNSUP
    assert lib.attn_fp8_buffer_offsets(B, H, S, D, None) == NULL


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), NULL), (dict(S=0), SHAPE), (dict(D=64), UNSUP), (dict(K=P + 4), ALIGN), (dict(signs=P + 2), ALIGN),
    (dict(buf=None), WS), (dict(bufb=1024), WS), (dict(buf=P + 16), WS),
])
def test_fp8_quantize_rejects(kw, code):
    lib = L.load()
    a = dict(Q=P, K=P, V=P, signs=None, buf=P, bufb=1 << 40, B=1, H=2, S=100, D=128)
    a.update(kw)
    assert lib.attn_fp8_quantize(a["Q"], a["K"], a["V"], a["signs"], a["buf"], a["bufb"], a["B"], a["H"], a["S"], a["D"],
                                 None) == code


@pytest.mark.parametrize("kw,code", [
    (dict(O=None), NULL), (dict(B=0), SHAPE), (dict(D=256), UNSUP), (dict(LSE=P + 4), ALIGN),
    (dict(scale=float("inf")), VALUE), (dict(buf=None), WS), (dict(bufb=100), WS),
])
def test_fwd_fp8_rejects(kw, code):
    lib = L.load()
    a = dict(buf=P, bufb=1 << 40, O=P, LSE=P, B=1, H=2, S=100, D=128, scale=0.1, causal=0)
    a.update(kw)
    assert lib.attn_fwd_fp8(a["buf"], a["bufb"], a["O"], a["LSE"], a["B"], a["H"], a["S"], a["D"], a["scale"],
                            a["causal"], None, None) == code


def test_set_variant():
    lib = L.load()
    assert lib.attn_set_variant(b"fwd", 1) == OK
    assert lib.attn_set_variant(b"fwd", 2) == OK
    assert lib.attn_set_variant(b"fwd", 3) == VALUE
    assert lib.attn_set_variant(b"fwd", -1) == OK
    assert lib.attn_set_variant(b"bwd_dq", 1) == OK
    assert lib.attn_set_variant(b"bwd_dq", 2) == OK
    assert lib.attn_set_variant(b"bwd_dq", 3) == VALUE
    assert lib.attn_set_variant(b"bwd_dq", -2) == VALUE
    assert lib.attn_set_variant(b"bwd_dkdv", 1) == OK
    assert lib.attn_set_variant(b"bwd_dkdv", 2) == VALUE
    # the measured losers are no longer built
    assert lib.attn_set_variant(b"fwd_fp8", 0) == UNSUP
    assert lib.attn_set_variant(b"bwd_main", 0) == UNSUP
    assert lib.attn_set_variant(b"nope", 0) == UNSUP
    assert lib.attn_set_variant(None, 0) == NULL
    for k in (b"fwd", b"bwd_dq", b"bwd_dkdv"):
        assert lib.attn_set_variant(k, -1) == OK
