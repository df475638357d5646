"""GPU parity of the FP8 forward pass (quantizer and attention) against the FP8 oracle.

Both sides take the same steps (transform, E4M3 rounding with the same
scales, tiled online softmax with P rounded to E4M3), so they differ only by
where float32 on the GPU rounds differently from float64 in the oracle:
the transform's sums, the scale quotients and the exponentials.  Each such
difference can move a value across an E4M3 rounding boundary and change
one code by one step; the rounding boundaries are 2^-4 relative apart and
the float32 differences about 1e-6 relative, so a few codes in 10^5 flip.
Hence:

* quantizer: at least 99.9% of the codes equal, every other one an adjacent
  code; scales equal to float32 rounding (relative 1e-6);
* attention at tau = 0 (the running max moves with every row, as in the
  oracle): the tolerances of the bf16 path, O max 2e-2 and mean 2e-3, LSE
  max 1e-3 (a flipped P code changes O by at most 2^-4 p |v| / l), plus
  the error of the FP8 matrix instruction itself: it does not accumulate
  exactly in float32; measured on the device (random E4M3 operands, 1024
  outputs), each 64-product instruction is off by at most 2^-12 times its
  largest single product.  A score takes two instructions, so row i's scores
  may move by 2^-11 scale max_d|q_id| max|k| (dequantized operands); row
  i's LSE by at most that much (its derivative in each score is P <= 1) and
  its O by at most twice that times max|v|.  The tests allow twice this
  (2^-10 ...) on top of the tolerances above;
* attention at the default tau = 8: P is rounded relative to a running max
  that may lag, a different but equally fine grid, so it is held to the
  accuracy of the method instead: its error against the exact oracle is at
  most 1.25 times the FP8 oracle's own error plus 1e-3.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

from exact_attention_97_amd import _lib as L
from exact_attention_97_amd.inputs import hadamard_signs, make_qkvdo
from oracle import attention as A
from oracle import fp8 as F

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3


def _np(t):
    import torch

    return t.detach().to("cpu", torch.float64).numpy()


def _same_code(a, b):
    a = np.asarray(a, dtype=np.int64)
    b = np.asarray(b, dtype=np.int64)
    return (a == b) | (((a & 0x7F) == 0) & ((b & 0x7F) == 0))


def _adjacent(a, b):
    # codes of neighbouring E4M3 values (same sign, magnitude codes one apart)
    a = np.asarray(a, dtype=np.int64)
    b = np.asarray(b, dtype=np.int64)
    return ((a & 0x80) == (b & 0x80)) & (np.abs((a & 0x7F) - (b & 0x7F)) == 1)


def _check_codes(name, got, want, min_equal=0.999):
    eq = _same_code(got, want)
    frac = float(eq.mean())
    ok_other = bool(np.all(_adjacent(got[~eq], want[~eq])))
    print(f"    {name}: {frac * 100:.4f}% codes equal, {int((~eq).sum())} adjacent", flush=True)
    assert frac >= min_equal and ok_other, f"{name}: {frac:.6f} equal, non-adjacent differences: {not ok_other}"


def _v_codes_from_gpu(v8t, S):
    """Undo the key permutation of the transposed V codes: [D, Sp] -> [S, D]."""
    key = np.arange(S)
    k = key % 64
    pos = 32 * ((k >> 2) & 1) + 16 * ((k >> 5) & 1) + 4 * ((k >> 3) & 3) + (k & 3)
    return v8t[:, (key - k) + pos].T


def _signs(D, seed=11):
    return hadamard_signs(D, seed)


def _mfma_slack(q, k, v, scale, signs, rows=None):
    """Per-row allowance for the FP8 matrix instruction's own error (see the module docstring):
    LSE slack 2^-10 scale max_d|q_id| max|k| and O slack twice that times max|v|."""
    d = F.quantize_head(q, k, v, signs)
    qh = d["qh"] if rows is None else d["qh"][np.asarray(rows)]
    ls = 2.0 ** -10 * scale * np.abs(qh).max(axis=1) * np.abs(d["kh"]).max()
    return ls, 2.0 * ls * np.abs(d["vh"]).max()


@pytest.mark.parametrize("S,rotate", [(200, True), (64, False), (333, True)])
def test_quantizer_matches_oracle(S, rotate):
    import torch

    B, H, D = 1, 2, 128
    print(f"[fp8 quantize] S={S} rotate={rotate}", flush=True)
    q, k, v, _ = make_qkvdo(B, H, S, D, seed=31, outlier_frac=0.01)
    sg = _signs(D)
    buf = L.fp8_quantize(q.cuda(), k.cuda(), v.cuda(), sg.cuda() if rotate else None)
    torch.cuda.synchronize()
    views = {n: t.cpu().numpy() for n, t in L.fp8_buffer_views(buf, B, H, S, D).items()}
    Sp = views["qs"].shape[1]
    for h in range(H):
        ref = F.quantize_head(_np(q[0, h]), _np(k[0, h]), _np(v[0, h]), sg.numpy() if rotate else None)
        _check_codes(f"h{h} q8", views["q8"][h, :S], ref["q8"])
        _check_codes(f"h{h} k8", views["k8"][h, :S], ref["k8"])
        _check_codes(f"h{h} v8", _v_codes_from_gpu(views["v8t"][h], S), ref["v8"])
        assert np.allclose(views["qs"][h, :S], ref["qs"], rtol=1e-6, atol=0)
        assert np.allclose(views["ks"][h, :len(ref["ks"])], ref["ks"], rtol=1e-6, atol=0)
        assert np.allclose(views["vs"][h], ref["vs"], rtol=1e-6, atol=0)
        # padding rows are zero values (+0 or -0 codes) with unit Q scale
        assert np.all((views["q8"][h, S:] & 0x7F) == 0) and np.all((views["k8"][h, S:] & 0x7F) == 0)
        assert np.all(views["qs"][h, S:] == 1.0)
        assert np.all((_v_codes_from_gpu(views["v8t"][h], Sp)[S:] & 0x7F) == 0)  # keys S.. (permuted positions)
    assert Sp % 128 == 0 and Sp >= S


CASES = [  # (B, H, S, causal, rotate)
    (1, 2, 128, False, True),
    (1, 2, 200, True, True),
    (2, 1, 513, False, False),
    (1, 1, 1000, True, True),
    (1, 2, 64, True, False),
    (1, 1, 1, False, True),
]


@pytest.mark.parametrize("B,H,S,causal,rotate", CASES)
def test_fwd_fp8_matches_fp8_oracle(B, H, S, causal, rotate):
    import torch

    D = 128
    print(f"[fp8 fwd] B={B} H={H} S={S} causal={causal} rotate={rotate}", flush=True)
    q, k, v, _ = make_qkvdo(B, H, S, D, seed=32)
    sg = _signs(D)
    scale = 1.0 / math.sqrt(D)
    o, lse = L.attn_fwd_fp8(q.cuda(), k.cuda(), v.cuda(), sg.cuda() if rotate else None, scale=scale, causal=causal,
                            rescale_tau=0.0)
    torch.cuda.synchronize()
    o, lse = _np(o), _np(lse)
    sgn = sg.numpy() if rotate else None
    o_ref, lse_ref = F.fp8_attention_fwd_heads(_np(q), _np(k), _np(v), scale, causal, sgn)
    d = np.abs(o.reshape(B * H, S, D) - o_ref)
    dl = np.abs(lse.reshape(B * H, S) - lse_ref)
    qn, kn, vn = _np(q).reshape(B * H, S, D), _np(k).reshape(B * H, S, D), _np(v).reshape(B * H, S, D)
    slack = [_mfma_slack(qn[n], kn[n], vn[n], scale, sgn) for n in range(B * H)]
    ls = np.stack([a for a, _ in slack])
    os_ = np.stack([b for _, b in slack])
    print(f"    O: max-abs {d.max():.3e} mean-abs {d.mean():.3e}; LSE max-abs {dl.max():.3e} "
          f"(instruction slack up to {ls.max():.1e})", flush=True)
    assert np.all(d.max(axis=2) <= O_MAX + os_) and d.mean() <= O_MEAN
    assert np.all(dl <= LSE_MAX + ls)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_default_tau_has_the_methods_accuracy(causal):
    import torch

    B, H, S, D = 1, 2, 1024, 128
    print(f"[fp8 fwd tau=8] S={S} causal={causal}", flush=True)
    q, k, v, _ = make_qkvdo(B, H, S, D, seed=33)
    sg = _signs(D)
    scale = 1.0 / math.sqrt(D)
    o, _ = L.attn_fwd_fp8(q.cuda(), k.cuda(), v.cuda(), sg.cuda(), scale=scale, causal=causal)
    torch.cuda.synchronize()
    o = _np(o).reshape(B * H, S, D)
    qn, kn, vn = _np(q), _np(k), _np(v)
    o_exact, _ = A.attention_fwd(qn, kn, vn, scale, causal)
    o_f8, _ = F.fp8_attention_fwd_heads(qn, kn, vn, scale, causal, sg.numpy())
    o_exact = o_exact.reshape(B * H, S, D)
    e_gpu = np.abs(o - o_exact).mean()
    e_f8 = np.abs(o_f8 - o_exact).mean()
    print(f"    mean-abs error vs exact: gpu {e_gpu:.4e}, fp8 oracle {e_f8:.4e}", flush=True)
    assert e_gpu <= 1.25 * e_f8 + 1e-3


def test_fwd_fp8_transform_lowers_error_on_outliers():
    import torch

    B, H, S, D = 1, 2, 1024, 128
    print("[fp8 outliers]", flush=True)
    q, k, v, _ = make_qkvdo(B, H, S, D, seed=34, outlier_frac=0.01, outlier_scale=20.0)
    sg = _signs(D)
    scale = 1.0 / math.sqrt(D)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    o_rot, _ = L.attn_fwd_fp8(qc, kc, vc, sg.cuda(), scale=scale)
    o_naive, _ = L.attn_fwd_fp8(qc, kc, vc, None, scale=scale)
    torch.cuda.synchronize()
    o_exact, _ = A.attention_fwd(_np(q), _np(k), _np(v), scale, False)
    rms = lambda x: float(np.sqrt(np.mean(x * x)))
    e_rot = rms(_np(o_rot) - o_exact)
    e_naive = rms(_np(o_naive) - o_exact)
    print(f"    rms error vs exact: transformed {e_rot:.4e}, plain {e_naive:.4e} (ratio {e_naive / e_rot:.2f})",
          flush=True)
    assert e_rot < e_naive


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_headline_sampled_rows(causal):
    """B=2 H=16 S=8192 (the benchmark shape, same launch): sampled rows of two heads against the FP8 oracle."""
    import torch

    B, H, S, D = 2, 16, 8192, 128
    print(f"[fp8 headline] causal={causal}", flush=True)
    q, k, v, _ = make_qkvdo(B, H, S, D, seed=2, outlier_frac=0.01, outlier_scale=20.0)
    sg = _signs(D)
    scale = 1.0 / math.sqrt(D)
    o, lse = L.attn_fwd_fp8(q.cuda(), k.cuda(), v.cuda(), sg.cuda(), scale=scale, causal=causal, rescale_tau=0.0)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.sort(np.concatenate([[0, 1, 63, 64, 8191], rng.choice(S, 11, replace=False)]))
    for b, h in ((0, 0), (1, 15)):
        o_ref, l_ref = F.fp8_attention_fwd(_np(q[b, h]), _np(k[b, h]), _np(v[b, h]), scale, causal, sg.numpy(),
                                           rows=rows)
        d = np.abs(_np(o[b, h])[rows] - o_ref)
        dl = np.abs(_np(lse[b, h])[rows] - l_ref)
        ls, os_ = _mfma_slack(_np(q[b, h]), _np(k[b, h]), _np(v[b, h]), scale, sg.numpy(), rows)
        print(f"    head ({b},{h}): O max-abs {d.max():.3e} mean-abs {d.mean():.3e}; LSE {dl.max():.3e} "
              f"(instruction slack up to {ls.max():.1e})", flush=True)
        assert np.all(d.max(axis=1) <= O_MAX + os_) and d.mean() <= O_MEAN
        assert np.all(dl <= LSE_MAX + ls)


@pytest.mark.parametrize("scale", [0.0, -0.3])
def test_fwd_fp8_unusual_scale(scale):
    """A negative scale flips the sign of every Q code; scale 0 gives uniform attention."""
    import torch

    B, H, S, D = 1, 2, 300, 128
    print(f"[fp8 scale] {scale}", flush=True)
    q, k, v, _ = make_qkvdo(B, H, S, D, seed=35)
    sg = _signs(D)
    for causal in (False, True):
        o, lse = L.attn_fwd_fp8(q.cuda(), k.cuda(), v.cuda(), sg.cuda(), scale=scale, causal=causal, rescale_tau=0.0)
        torch.cuda.synchronize()
        o_ref, lse_ref = F.fp8_attention_fwd_heads(_np(q), _np(k), _np(v), scale, causal, sg.numpy())
        d = np.abs(_np(o).reshape(B * H, S, D) - o_ref)
        dl = np.abs(_np(lse).reshape(B * H, S) - lse_ref)
        qn, kn, vn = _np(q).reshape(B * H, S, D), _np(k).reshape(B * H, S, D), _np(v).reshape(B * H, S, D)
        slack = [_mfma_slack(qn[n], kn[n], vn[n], abs(scale), sg.numpy()) for n in range(B * H)]
        ls = np.stack([a for a, _ in slack])
        os_ = np.stack([b for _, b in slack])
        print(f"    causal={causal}: O max-abs {d.max():.3e} mean-abs {d.mean():.3e}; LSE {dl.max():.3e}", flush=True)
        assert np.all(d.max(axis=2) <= O_MAX + os_) and d.mean() <= O_MEAN
        assert np.all(dl <= LSE_MAX + ls)


def test_fwd_fp8_deterministic():
    import torch

    q, k, v, _ = make_qkvdo(2, 2, 700, 128, seed=36)
    qg, kg, vg, sg = q.cuda(), k.cuda(), v.cuda(), _signs(128).cuda()
    b1 = L.fp8_quantize(qg, kg, vg, sg)
    b2 = L.fp8_quantize(qg, kg, vg, sg)
    torch.cuda.synchronize()
    v1, v2 = L.fp8_buffer_views(b1, 2, 2, 700, 128), L.fp8_buffer_views(b2, 2, 2, 700, 128)
    for name in v1:
        assert bool((v1[name] == v2[name]).all()), f"quantizer region {name} not repeatable"
    for causal in (False, True):
        o1, l1 = L.attn_fwd_fp8_quantized(b1, 2, 2, 700, 128, causal=causal)
        o2, l2 = L.attn_fwd_fp8_quantized(b1, 2, 2, 700, 128, causal=causal)
        assert bool((o1 == o2).all()) and bool((l1 == l2).all()), "FP8 forward not bitwise repeatable"
