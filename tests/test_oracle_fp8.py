"""Pins for the FP8 oracle (oracle/fp8.py), each against something other than itself.

* The E4M3 codebook and its rounding against torch's float8_e4m3fn type (an
  independent library implementation of the same OCP format), plus closed
  forms of the format (largest value, smallest normal and subnormal).
* The Hadamard matrix against the closed form (-1)^popcount(i & j), and its
  orthogonality.
* Invariance of Q K^T under the transform (the reason it may be applied).
* With every rounding switched off, the tile-free FP8 reference and the
  tiled online softmax are exactly the softmax attention of the plain oracle
  (oracle/attention.py), causal and ragged included: this pins the mask, the
  row max, the tile loop, the running max and the rescale.
* A worked example of the reference by hand (two keys, P = [1, 0.3] with
  0.3 rounding to the code 0.3125, unrounded row sum), as a golden file.
* The rounding error bound of E4M3 (half a unit in the last place) and the
  per-element bound p_rounding_bound built on it: the rounded reference stays
  within it of the unrounded attention, and so does a tiled computation that
  rounds against the running max, for tiles of 1 to 200 keys and with the
  max allowed to lag by up to 8 (log2 units) as the conditional rescale does.
* The pages' claim, qualitatively: on inputs with outliers, the transform
  lowers the error of FP8 attention against the exact result.

The mutation tests at the bottom plant plausible mistakes in copies of the
oracle's steps and check that one of these pins catches each of them.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import fp8 as F


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def _torch_codes(x):
    import torch

    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _same_code(a, b):
    # +0 and -0 are the same value
    a = np.asarray(a, dtype=np.int64)
    b = np.asarray(b, dtype=np.int64)
    zero = ((a & 0x7F) == 0) & ((b & 0x7F) == 0)
    return (a == b) | zero


# ----------------------------------------------------------------------------
# the format
# ----------------------------------------------------------------------------


def test_table_matches_torch_float8_e4m3fn():
    import torch

    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = F.e4m3_table()
    assert np.array_equal(np.isnan(ref), np.isnan(tab))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], tab[ok])


def test_format_closed_forms():
    tab = F.e4m3_table()
    assert tab[0x7E] == 448.0 and F.E4M3_MAX == 448.0
    assert tab[0x08] == 2.0 ** -6  # smallest normal
    assert tab[0x01] == 2.0 ** -9  # smallest subnormal
    assert tab[0x38] == 1.0
    assert tab[0xB8] == -1.0
    assert np.isnan(tab[0x7F]) and np.isnan(tab[0xFF])
    assert np.all(np.diff(tab[:0x7F]) > 0)  # codes 0..0x7E increase


def test_rounding_matches_torch_on_random_and_ties():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.uniform(-448, 448, 4000),
        rng.standard_normal(4000) * 0.01,  # subnormal and small normal range
        rng.standard_normal(4000) * 3,
    ])
    tab = F.e4m3_table()[:0x7F]
    mids = (tab[1:] + tab[:-1]) / 2  # exact ties, representable in float32
    x = np.concatenate([x, mids, -mids]).astype(np.float32).astype(np.float64)
    got = F.quantize_e4m3(x)
    want = _torch_codes(x)
    assert np.all(_same_code(got, want))


def test_clamp_keeps_values_finite():
    x = np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e6, -1e6])
    codes = F.quantize_e4m3(x)
    assert np.all((codes & 0x7F) == 0x7E)


def test_rounding_error_bound():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.02])
    r = F.round_e4m3(x)
    err = np.abs(r - x)
    normal = np.abs(x) >= 2.0 ** -6
    # half a unit in the last place: 2^-4 relative for normals, 2^-10 absolute below
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x[normal]) + 1e-300)
    assert np.all(err[~normal] <= 2.0 ** -10)


# ----------------------------------------------------------------------------
# the transform
# ----------------------------------------------------------------------------


@pytest.mark.parametrize("d", [1, 2, 8, 64, 128])
def test_hadamard_closed_form_and_orthogonality(d):
    h = F.hadamard(d)
    closed = np.array([[(-1.0) ** bin(i & j).count("1") for j in range(d)] for i in range(d)])
    assert np.array_equal(h, closed)
    assert np.array_equal(h @ h.T, d * np.eye(d))


def test_rotation_keeps_scores():
    q = _rand((40, 128), 2)
    k = _rand((56, 128), 3)
    s = np.where(np.random.default_rng(4).random(128) < 0.5, -1.0, 1.0)
    qr, kr = F.rotate(q, s), F.rotate(k, s)
    assert np.max(np.abs(qr @ kr.T - q @ k.T)) <= 1e-12 * np.max(np.abs(q @ k.T))
    # and it changes the rows themselves (it is not the identity)
    assert np.max(np.abs(qr - q)) > 0.1


# ----------------------------------------------------------------------------
# the tiled online softmax
# ----------------------------------------------------------------------------


@pytest.mark.parametrize("sq,sk,causal", [(64, 64, False), (100, 100, True), (130, 130, False), (7, 200, True),
                                          (129, 129, True)])
def test_online_softmax_without_rounding_is_attention(sq, sk, causal):
    q = _rand((sq, 32), 5)
    k = _rand((sk, 32), 6)
    v = _rand((sk, 32), 7)
    scale = 1.0 / math.sqrt(32)
    o_ref, lse_ref = A.attention_fwd(q[None, None], k[None, None], v[None, None], scale, causal)
    for tile in (1, 37, 64):
        o, lse = F.online_softmax_fwd(q, k, v, scale, causal, lambda p: p, tile)
        assert np.max(np.abs(o - o_ref[0, 0])) <= 1e-12
        assert np.max(np.abs(lse - lse_ref[0, 0])) <= 1e-12
    if sq == sk:
        o, lse, _ = F.fp8_reference_fwd(q, k, v, scale, causal, round_p=lambda p: p)
        assert np.max(np.abs(o - o_ref[0, 0])) <= 1e-12
        assert np.max(np.abs(lse - lse_ref[0, 0])) <= 1e-12


def test_fp8_attention_close_to_exact():
    # FP8 is an approximation: on plain N(0,1) inputs its error against the
    # exact result stays at the level the E4M3 rounding allows
    q = _rand((256, 128), 8)
    k = _rand((256, 128), 9)
    v = _rand((256, 128), 10)
    scale = 1.0 / math.sqrt(128)
    o, lse = F.fp8_attention_fwd(q, k, v, scale, False)
    o_ref, lse_ref = A.attention_fwd(q[None, None], k[None, None], v[None, None], scale, False)
    err = np.abs(o - o_ref[0, 0])
    assert err.mean() < 2e-2 and err.max() < 0.15
    assert np.max(np.abs(lse - lse_ref[0, 0])) < 5e-2


def test_quantized_operands_reconstruct_inputs():
    q = _rand((100, 128), 11)
    k = _rand((100, 128), 12) * 3
    v = _rand((100, 128), 13)
    d = F.quantize_head(q, k, v)
    for name, x in (("qh", q), ("kh", k), ("vh", v)):
        rel = np.abs(d[name] - x).max() / np.abs(x).max()
        assert rel <= 2.0 ** -4, name
    assert np.shape(d["ks"]) == () and d["qs"].shape == (100,) and d["vs"].shape == (128,)
    assert np.all(np.abs(F.dequantize_e4m3(d["q8"])) <= 448.0)
    # the element of largest magnitude of each group is exactly +-448 times its scale
    assert np.max(np.abs(F.dequantize_e4m3(d["k8"]))) == 448.0 and d["ks"] == np.abs(k).max() / 448.0
    assert np.all(np.max(np.abs(F.dequantize_e4m3(d["q8"])), axis=1) == 448.0)
    assert np.all(np.max(np.abs(F.dequantize_e4m3(d["v8"])), axis=0) == 448.0)


def test_transform_lowers_error_on_outliers():
    # the pages' claim (error of FP8 attention with vs without the transform)
    rng = np.random.default_rng(14)
    sq, d = 256, 128
    q = rng.standard_normal((sq, d))
    k = rng.standard_normal((sq, d))
    v = rng.standard_normal((sq, d))
    q = np.where(rng.random((sq, d)) < 0.01, q * 20, q)
    k = np.where(rng.random((sq, d)) < 0.01, k * 20, k)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    scale = 1.0 / math.sqrt(d)
    o_ref, _ = A.attention_fwd(q[None, None], k[None, None], v[None, None], scale, False)
    o_naive, _ = F.fp8_attention_fwd(q, k, v, scale, False, None)
    o_rot, _ = F.fp8_attention_fwd(q, k, v, scale, False, s)
    rms = lambda e: math.sqrt(float(np.mean(e * e)))
    e_naive = rms(o_naive - o_ref[0, 0])
    e_rot = rms(o_rot - o_ref[0, 0])
    assert e_rot < e_naive, (e_rot, e_naive)


# ----------------------------------------------------------------------------
# the tile-free reference and the bound on the rounding of P
# ----------------------------------------------------------------------------


def test_reference_worked_example_golden():
    """tests/golden/fp8_two_keys.json, worked by hand: scores [0, ln 0.3] give
    P~ = [1, 0.3]; 0.3 lies between the E4M3 values 0.28125 and 0.3125 and is
    nearer the latter; O = (1 * 2 + 0.3125 * 4) / 1.3 = 2.5, LSE = ln 1.3."""
    import json
    import os

    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fp8_two_keys.json")))
    qh = np.array(g["qh"], dtype=np.float64)
    kh = np.array([[0.0], [math.log(0.3)]])
    vh = np.array(g["vh"], dtype=np.float64)
    o, lse, p = F.fp8_reference_fwd(qh, kh, vh, g["scale"], False)
    assert abs(o[0, 0] - g["O"]) <= 1e-12 and abs(lse[0] - g["LSE"]) <= 1e-12
    assert abs(F.round_e4m3(np.array([0.3]))[0] - g["P_rounded"][1]) == 0.0


def test_error_bound_holds_and_is_attained():
    rng = np.random.default_rng(40)
    x = np.concatenate([rng.uniform(0, 448, 50000), rng.uniform(0, 2.0 ** -5, 50000),
                        np.exp2(rng.uniform(-20, 8.8, 50000))])
    x = np.minimum(x, 448.0)
    err = np.abs(F.round_e4m3(x) - x)
    bnd = F.e4m3_error_bound(x)
    assert np.all(err <= bnd)
    # tight: at the first midpoint of a binade (1.0625 * 2^e) the error is 1 / 1.0625 of the bound
    tab = F.e4m3_table()[:0x7F]
    mids = (tab[1:] + tab[:-1]) / 2
    big = mids[mids >= 2.0 ** -6]
    assert np.max(np.abs(F.round_e4m3(big * (1 - 1e-9)) - big) / F.e4m3_error_bound(big)) > 0.94


def _lagging_online_softmax(qh, kh, vh, scale, tile, tau):
    """Tiled attention that moves its running max only when a row's max grows
    by more than tau (log2 units) and rounds P to E4M3 against that max."""
    n, sk = qh.shape[0], kh.shape[0]
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    acc = np.zeros((n, vh.shape[1]))
    for t0 in range(0, sk, tile):
        s = scale * (qh @ kh[t0:t0 + tile].T)
        mx = s.max(axis=1)
        grow = (mx - m) * math.log2(math.e) > tau
        m_new = np.where(grow, mx, m)
        alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
        p = np.exp(s - m_new[:, None])
        assert np.all(p <= 2.0 ** tau * (1 + 1e-12))
        acc = acc * alpha[:, None] + F.round_e4m3(p) @ vh[t0:t0 + tile]
        l = l * alpha + p.sum(axis=1)
        m = m_new
    return acc / l[:, None]


@pytest.mark.parametrize("outliers", [False, True])
def test_p_rounding_bound_covers_every_schedule(outliers):
    rng = np.random.default_rng(41)
    q = rng.standard_normal((64, 128))
    k = rng.standard_normal((200, 128))
    v = rng.standard_normal((200, 128))
    if outliers:
        q = np.where(rng.random(q.shape) < 0.01, 20 * q, q)
        k = np.where(rng.random(k.shape) < 0.01, 20 * k, k)
    d = F.quantize_head(q, k, v, np.where(rng.random(128) < 0.5, -1.0, 1.0))
    qh, kh, vh = d["qh"], d["kh"], d["vh"][:200]
    scale = 1.0 / math.sqrt(128)
    o_exact, _, p = F.fp8_reference_fwd(qh, kh, vh, scale, False, round_p=lambda x: x)
    o_ref, _, _ = F.fp8_reference_fwd(qh, kh, vh, scale, False)
    bnd = F.p_rounding_bound(p, vh)
    assert np.all(np.abs(o_ref - o_exact) <= bnd * (1 + 1e-9))
    assert np.max(np.abs(o_ref - o_exact)) > 0.0
    for tile in (1, 16, 64, 200):
        o_t, _ = F.online_softmax_fwd(qh, kh, vh, scale, False, F.round_e4m3, tile)
        assert np.all(np.abs(o_t - o_exact) <= bnd * (1 + 1e-9))
        assert np.all(np.abs(o_t - o_ref) <= 2 * bnd * (1 + 1e-9))
        for tau in (3.0, 8.0):
            o_l = _lagging_online_softmax(qh, kh, vh, scale, tile, tau)
            assert np.all(np.abs(o_l - o_exact) <= bnd * (1 + 1e-9))


# ----------------------------------------------------------------------------
# planted mistakes: each must fail a pin above
# ----------------------------------------------------------------------------


def _rotate_missing_norm(x, signs):
    return (np.asarray(x) * signs) @ F.hadamard(x.shape[-1])


def _round_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    pos = F.e4m3_table()[:0x7F]
    hi = np.minimum(np.searchsorted(pos, a), len(pos) - 1)
    lo = np.maximum(hi - 1, 0)
    code = np.where(pos[hi] - a <= a - pos[lo], hi, lo).astype(np.uint8)
    return np.where(x < 0, code | 0x80, code).astype(np.uint8)


def _softmax_without_rescale(qh, kh, vh, scale, causal, tile=64):
    sq, sk = qh.shape[0], kh.shape[0]
    m = np.full(sq, -np.inf)
    l = np.zeros(sq)
    acc = np.zeros((sq, vh.shape[1]))
    for t0 in range(0, sk, tile):
        s = scale * (qh @ kh[t0:t0 + tile].T)
        m = np.maximum(m, s.max(axis=1))
        p = np.exp(s - m[:, None])
        acc = acc + p @ vh[t0:t0 + tile]  # old tiles never rescaled
        l = l + p.sum(axis=1)
    return acc / l[:, None], m + np.log(l)


def test_planted_mistakes_are_caught():
    q = _rand((40, 128), 2)
    k = _rand((56, 128), 3)
    s = np.where(np.random.default_rng(4).random(128) < 0.5, -1.0, 1.0)
    qr, kr = _rotate_missing_norm(q, s), _rotate_missing_norm(k, s)
    assert np.max(np.abs(qr @ kr.T - q @ k.T)) > 1.0  # the invariance pin fails

    tab = F.e4m3_table()[:0x7F]
    mids = ((tab[1:] + tab[:-1]) / 2).astype(np.float32).astype(np.float64)
    assert not np.all(_same_code(_round_ties_away(mids), _torch_codes(mids)))  # the torch pin fails

    qq = _rand((130, 32), 5)
    kk = _rand((130, 32), 6)
    vv = _rand((130, 32), 7)
    o, _ = _softmax_without_rescale(qq, kk, vv, 0.2, False)
    o_ref, _ = A.attention_fwd(qq[None, None], kk[None, None], vv[None, None], 0.2, False)
    assert np.max(np.abs(o - o_ref[0, 0])) > 1e-6  # the online-softmax pin fails

    # the reference with its row sum over the rounded P: the golden fails
    qh, kh, vh = np.array([[1.0]]), np.array([[0.0], [math.log(0.3)]]), np.array([[2.0], [4.0]])
    p = np.exp(qh @ kh.T)
    o_bad = (F.round_e4m3(p) @ vh) / F.round_e4m3(p).sum(axis=1, keepdims=True)
    assert abs(o_bad[0, 0] - 2.5) > 1e-3
    # a bound that forgets the subnormal floor (2^-4 p only) fails the bound pin on rows with small P
    rng = np.random.default_rng(41)
    x = np.exp2(rng.uniform(-14, -7, 1000))
    assert np.any(np.abs(F.round_e4m3(x) - x) > 2.0 ** -4 * x)


def test_row_subset_equals_full_call():
    q = _rand((150, 128), 20)
    k = _rand((150, 128), 21)
    v = _rand((150, 128), 22)
    s = np.where(np.random.default_rng(23).random(128) < 0.5, -1.0, 1.0)
    rows = [0, 3, 64, 127, 149]
    for causal in (False, True):
        o, lse = F.fp8_attention_fwd(q, k, v, 0.09, causal, s)
        os_, ls_ = F.fp8_attention_fwd(q, k, v, 0.09, causal, s, rows=rows)
        # equal up to the summation order of the matrix library on a row subset
        assert np.max(np.abs(os_ - o[rows])) <= 1e-12 and np.max(np.abs(ls_ - lse[rows])) <= 1e-12
