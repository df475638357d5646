"""Pins for the CPU oracle: it is checked against things other than itself.

Every pin comes from the mathematics (the pages print no worked example):
brute force with scalar loops, closed forms for special cases, invariants of
softmax attention, central finite differences for the backward pass, a
hand-derived two-key example (tests/golden/two_keys.json) and an
independent library route (torch float64 autograd).  The pins are written
as functions of the implementation under check, so the mutation tests at
the bottom can show that plausible mistakes (a dropped scale, a flipped
mask, a transposed operand, a missing term) each fail at least one pin.
"""

from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


# ----------------------------------------------------------------------------
# brute force: scalar loops, no matrix library
# ----------------------------------------------------------------------------


def brute_force_fwd(q, k, v, scale, causal):
    """One head, [S, D] lists; every score, max, sum and output by hand."""
    sq, dd = len(q), len(q[0])
    sk, dv = len(k), len(v[0])
    out, lse = [], []
    for i in range(sq):
        allowed = [j for j in range(sk) if not (causal and j > i)]
        s = {}
        for j in allowed:
            acc = 0.0
            for d in range(dd):
                acc += q[i][d] * k[j][d]
            s[j] = scale * acc
        mx = max(s.values())
        w = {j: math.exp(s[j] - mx) for j in allowed}
        tot = math.fsum(w.values())
        out.append([math.fsum(w[j] * v[j][e] for j in allowed) / tot for e in range(dv)])
        lse.append(mx + math.log(tot))
    return out, lse


# ----------------------------------------------------------------------------
# pin suites, parametrised by the implementation (fwd, bwd)
# ----------------------------------------------------------------------------


def fwd_pin_failures(fwd, probs):
    """Run every forward pin; return a list of failure descriptions."""
    fails = []

    def check(name, ok):
        if not ok:
            fails.append(name)

    # brute force on tiny shapes
    for sq, dd, causal in itertools.product((1, 2, 3, 7, 16), (1, 4, 8), (False, True)):
        q = _rand((1, 1, sq, dd), 10 + sq * 7 + dd)
        k = _rand((1, 1, sq, dd), 20 + sq * 7 + dd)
        v = _rand((1, 1, sq, dd), 30 + sq * 7 + dd)
        scale = 0.7
        o, lse = fwd(q, k, v, scale, causal)
        bo, blse = brute_force_fwd(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), scale, causal)
        check(f"brute_force O S={sq} D={dd} causal={causal}",
              np.max(np.abs(o[0, 0] - np.array(bo))) <= 1e-12)
        check(f"brute_force LSE S={sq} D={dd} causal={causal}",
              np.max(np.abs(lse[0, 0] - np.array(blse))) <= 1e-12)

    for causal in (False, True):
        q = _rand((2, 2, 9, 5), 1)
        k = _rand((2, 2, 9, 5), 2)
        v = _rand((2, 2, 9, 5), 3)
        scale = 0.45
        # rows of P: non-negative, sum to one, zero where masked
        p = probs(q[1, 0], k[1, 0], scale, causal)
        check(f"P rows sum to 1 causal={causal}", np.allclose(p.sum(axis=1), 1.0, atol=1e-13))
        check(f"P >= 0 causal={causal}", bool(np.all(p >= 0)))
        if causal:
            check("P masked entries are 0", bool(np.all(np.triu(p, 1) == 0)))
        # constant V gives O equal to that constant
        c = np.full_like(v, 0.0) + np.arange(5)[None, None, None, :] * 0.5 - 1.0
        o, _ = fwd(q, k, c, scale, causal)
        check(f"constant V -> O = c causal={causal}", np.max(np.abs(o - c)) <= 1e-12)
        # scale = 0: O_i is the mean of the visible V rows, LSE_i = ln(n_i)
        o, lse = fwd(q, k, v, 0.0, causal)
        n = np.arange(1, 10) if causal else np.full(9, 9)
        if causal:
            mean = np.cumsum(v, axis=2) / n[None, None, :, None]
        else:
            mean = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        check(f"scale=0 -> mean of V causal={causal}", np.max(np.abs(o - mean)) <= 1e-12)
        check(f"scale=0 -> LSE=ln n causal={causal}",
              np.max(np.abs(lse - np.log(n)[None, None, :])) <= 1e-12)
        # each output row depends only on its own query row
        q2 = q.copy()
        q2[:, :, 4] += 3.0
        o1, l1 = fwd(q, k, v, scale, causal)
        o2, l2 = fwd(q2, k, v, scale, causal)
        keep = [i for i in range(9) if i != 4]
        check(f"row independence causal={causal}",
              np.array_equal(o1[:, :, keep], o2[:, :, keep]) and np.array_equal(l1[:, :, keep], l2[:, :, keep])
              and not np.allclose(o1[:, :, 4], o2[:, :, 4]))
        # adding one vector to every key: O unchanged, LSE_i shifts by scale q_i.c
        cvec = _rand((5,), 44)
        o3, l3 = fwd(q, k + cvec, v, scale, causal)
        check(f"key shift keeps O causal={causal}", np.max(np.abs(o3 - o1)) <= 1e-12)
        check(f"key shift moves LSE causal={causal}",
              np.max(np.abs(l3 - (l1 + scale * (q @ cvec)))) <= 1e-12)

    # a single key: O = V, LSE = scale q.k
    q = _rand((1, 3, 1, 6), 5)
    k = _rand((1, 3, 1, 6), 6)
    v = _rand((1, 3, 1, 6), 7)
    for causal in (False, True):
        o, lse = fwd(q, k, v, 0.8, causal)
        check(f"S=1 O=V causal={causal}", np.max(np.abs(o - v)) <= 1e-15)
        check(f"S=1 LSE causal={causal}", np.max(np.abs(lse - 0.8 * np.sum(q * k, axis=-1))) <= 1e-14)

    # causal row 0 sees only key 0
    q = _rand((1, 1, 6, 4), 8)
    k = _rand((1, 1, 6, 4), 9)
    v = _rand((1, 1, 6, 4), 10)
    o, lse = fwd(q, k, v, 1.3, True)
    check("causal row 0 O=V0", np.max(np.abs(o[0, 0, 0] - v[0, 0, 0])) <= 1e-15)
    check("causal row 0 LSE", abs(lse[0, 0, 0] - 1.3 * float(q[0, 0, 0] @ k[0, 0, 0])) <= 1e-14)

    # non-causal: jointly permuting the rows of K and V leaves O unchanged
    q = _rand((1, 2, 11, 4), 11)
    k = _rand((1, 2, 11, 4), 12)
    v = _rand((1, 2, 11, 4), 13)
    perm = np.random.default_rng(3).permutation(11)
    o1, l1 = fwd(q, k, v, 0.6, False)
    o2, l2 = fwd(q, k[:, :, perm], v[:, :, perm], 0.6, False)
    check("K/V permutation invariance", np.max(np.abs(o1 - o2)) <= 1e-12 and np.max(np.abs(l1 - l2)) <= 1e-12)

    # hand-derived two-key example (closed forms in the golden file)
    with open(os.path.join(GOLDEN, "two_keys.json")) as f:
        g = json.load(f)
    q = np.array(g["q"], dtype=np.float64)[None, None]
    k = np.array(g["k"], dtype=np.float64)[None, None]
    v = np.array(g["v"], dtype=np.float64)[None, None]
    for case in g["forward"]:
        o, lse = fwd(q, k, v, g["scale"], case["causal"])
        want_o = np.array([[_eval(e) for e in row] for row in case["O"]])
        want_l = np.array([_eval(e) for e in case["LSE"]])
        check(f"two_keys fwd causal={case['causal']}",
              np.max(np.abs(o[0, 0] - want_o)) <= 1e-14 and np.max(np.abs(lse[0, 0] - want_l)) <= 1e-14)
    return fails


def _eval(expr: str) -> float:
    """Evaluate a closed-form expression from the golden file (math names only)."""
    names = {"e": math.e, "exp": math.exp, "log": math.log, "sqrt": math.sqrt,
             "sig": lambda x: 1.0 / (1.0 + math.exp(-x))}
    return float(eval(expr, {"__builtins__": {}}, names))  # noqa: S307 - our own fixture


def _loss_fd(fwd, q, k, v, do, scale, causal):
    o, _ = fwd(q, k, v, scale, causal)
    return float(np.sum(o * do))


def bwd_pin_failures(fwd, bwd):
    """Run every backward pin; return a list of failure descriptions."""
    fails = []

    def check(name, ok):
        if not ok:
            fails.append(name)

    # central finite differences of L = sum(O * dO), every entry of Q, K, V
    for sq, dd, causal in ((3, 2, False), (5, 3, True), (8, 4, False), (8, 4, True)):
        q = _rand((1, 1, sq, dd), 50 + sq)
        k = _rand((1, 1, sq, dd), 60 + sq)
        v = _rand((1, 1, sq, dd), 70 + sq)
        do = _rand((1, 1, sq, dd), 80 + sq)
        scale = 0.9
        dq, dk, dv = bwd(q, k, v, do, scale, causal)
        h = 1e-6
        for name, x, grad in (("Q", q, dq), ("K", k, dk), ("V", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp = x.copy()
                xm = x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"Q": (xp, k, v), "K": (q, xp, v), "V": (q, k, xp)}[name]
                args_m = {"Q": (xm, k, v), "K": (q, xm, v), "V": (q, k, xm)}[name]
                num[idx] = (_loss_fd(fwd, *args_p, do, scale, causal)
                            - _loss_fd(fwd, *args_m, do, scale, causal)) / (2 * h)
            err = np.max(np.abs(num - grad)) / max(1.0, np.max(np.abs(grad)))
            check(f"finite differences d{name} S={sq} D={dd} causal={causal}", err <= 1e-6)

    for causal in (False, True):
        q = _rand((2, 2, 10, 6), 91)
        k = _rand((2, 2, 10, 6), 92)
        v = _rand((2, 2, 10, 6), 93)
        do = _rand((2, 2, 10, 6), 94)
        dq, dk, dv = bwd(q, k, v, do, 0.55, causal)
        # softmax ignores a common shift of all keys: the key gradients sum to 0
        check(f"sum_j dK_j = 0 causal={causal}", np.max(np.abs(dk.sum(axis=2))) <= 1e-12)
        # rows of P sum to one: the value gradients sum to the output gradients
        check(f"sum_j dV_j = sum_i dO_i causal={causal}",
              np.max(np.abs(dv.sum(axis=2) - do.sum(axis=2))) <= 1e-12)
        if causal:
            check("causal dQ_0 = 0", np.max(np.abs(dq[:, :, 0])) <= 1e-15)

    # hand-derived two-key gradients
    with open(os.path.join(GOLDEN, "two_keys.json")) as f:
        g = json.load(f)
    q = np.array(g["q"], dtype=np.float64)[None, None]
    k = np.array(g["k"], dtype=np.float64)[None, None]
    v = np.array(g["v"], dtype=np.float64)[None, None]
    do = np.array(g["do"], dtype=np.float64)[None, None]
    case = g["backward"]
    dq, dk, dv = bwd(q, k, v, do, g["scale"], False)
    for nm, got in (("dQ", dq), ("dK", dk), ("dV", dv)):
        want = np.array([[_eval(e) for e in row] for row in case[nm]])
        check(f"two_keys {nm}", np.max(np.abs(got[0, 0] - want)) <= 1e-14)
    return fails


# ----------------------------------------------------------------------------
# the oracle passes every pin
# ----------------------------------------------------------------------------


def test_forward_pins():
    fails = fwd_pin_failures(oracle.attention_fwd, oracle.attention_probs)
    assert not fails, fails


def test_backward_pins():
    fails = bwd_pin_failures(oracle.attention_fwd, oracle.attention_bwd)
    assert not fails, fails


def test_torch_autograd_cross_check():
    """Secondary cross-check through an independent library route."""
    torch = pytest.importorskip("torch")
    for causal in (False, True):
        g = torch.Generator().manual_seed(5)
        q, k, v, do = (torch.randn((2, 3, 13, 8), generator=g, dtype=torch.float64) for _ in range(4))
        qt, kt, vt = (x.clone().requires_grad_(True) for x in (q, k, v))
        s = (qt @ kt.transpose(-1, -2)) * 0.35
        if causal:
            s = s.masked_fill(torch.ones(13, 13, dtype=torch.bool).triu(1), float("-inf"))
        o = torch.softmax(s, dim=-1) @ vt
        lse = torch.logsumexp(s, dim=-1)
        o.backward(do)
        ro, rl = oracle.attention_fwd(q, k, v, 0.35, causal)
        dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.35, causal)
        assert np.max(np.abs(ro - o.detach().numpy())) < 1e-13
        assert np.max(np.abs(rl - lse.detach().numpy())) < 1e-13
        assert np.max(np.abs(dq - qt.grad.numpy())) < 1e-12
        assert np.max(np.abs(dk - kt.grad.numpy())) < 1e-12
        assert np.max(np.abs(dv - vt.grad.numpy())) < 1e-12


def test_row_sampled_forward_matches_full():
    q = _rand((2, 2, 40, 8), 1)
    k = _rand((2, 2, 40, 8), 2)
    v = _rand((2, 2, 40, 8), 3)
    for causal in (False, True):
        o, lse = oracle.attention_fwd(q, k, v, 0.4, causal)
        rows = [(1, 0, 0), (0, 1, 17), (1, 1, 39), (0, 0, 5)]
        ro, rl = oracle.attention_fwd_rows(q, k, v, 0.4, causal, rows)
        for n, (b, h, i) in enumerate(rows):
            assert np.max(np.abs(ro[n] - o[b, h, i])) < 1e-13
            assert abs(rl[n] - lse[b, h, i]) < 1e-13


def test_float32_oracle_close_to_float64():
    """The fp32 block-of-rows oracle used at scale errs far below the tolerances."""
    torch = pytest.importorskip("torch")
    g = torch.Generator().manual_seed(9)
    shape = (1, 2, 1000, 64)
    q, k, v, do = (torch.randn(shape, generator=g).to(torch.bfloat16) for _ in range(4))
    for causal in (False, True):
        o64, l64 = oracle.attention_fwd(q, k, v, 0.125, causal)
        o32, l32 = oracle.attention_fwd_f32(q, k, v, 0.125, causal, block_rows=300)
        assert np.max(np.abs(o32.numpy() - o64[0])) < 1e-5
        assert np.max(np.abs(l32.numpy() - l64[0])) < 1e-5
        dq64, dk64, dv64 = oracle.attention_bwd(q, k, v, do, 0.125, causal)
        dq32, dk32, dv32 = oracle.attention_bwd_f32(q, k, v, do, 0.125, causal, block_rows=300)
        assert np.max(np.abs(dq32.numpy() - dq64[0])) < 1e-5
        assert np.max(np.abs(dk32.numpy() - dk64[0])) < 1e-5
        assert np.max(np.abs(dv32.numpy() - dv64[0])) < 1e-5


def test_exp2_exact_is_exp2():
    x = np.array([-127.0, -3.5, -1.0, 0.0, 0.25, 8.0])
    assert np.all(oracle.exp2_exact(x) == np.array([2.0**-127, 2.0**-3.5, 0.5, 1.0, 2.0**0.25, 256.0]))


# ----------------------------------------------------------------------------
# mutation tests: plant plausible mistakes in copies of the oracle and show
# that the pins catch each of them
# ----------------------------------------------------------------------------


def _mut_fwd_factory(kind):
    def fwd(q, k, v, scale, causal):
        q, k, v = A._f64(q), A._f64(k), A._f64(v)
        bsz, nh, sq, _ = q.shape
        o = np.zeros((bsz, nh, sq, v.shape[-1]))
        lse = np.zeros((bsz, nh, sq))
        for b in range(bsz):
            for h in range(nh):
                sc = 1.0 if kind == "drop_scale" else scale
                s = sc * (q[b, h] @ k[b, h].T)
                if causal:
                    i = np.arange(sq)[:, None]
                    j = np.arange(sq)[None, :]
                    s = np.where((j < i) if kind == "flip_mask" else (j > i), -np.inf, s)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                l = e.sum(axis=1, keepdims=True)
                p = e / l
                if kind == "transpose_p":
                    o[b, h] = p.T @ v[b, h]
                else:
                    o[b, h] = p @ v[b, h]
                lse[b, h] = (m if kind == "lse_no_log" else m + np.log(l))[:, 0] if kind != "lse_no_max" else np.log(l)[:, 0]
        return o, lse

    def probs(q, k, scale, causal):
        p = A.attention_probs(q, k, scale, causal)
        return p
    return fwd, probs


def _mut_bwd_factory(kind):
    def bwd(q, k, v, do, scale, causal):
        q, k, v, do = A._f64(q), A._f64(k), A._f64(v), A._f64(do)
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(q.shape[0]):
            for h in range(q.shape[1]):
                p = A.attention_probs(q[b, h], k[b, h], scale, causal)
                dv[b, h] = (p @ do[b, h]) if kind == "dv_no_transpose" else p.T @ do[b, h]
                dp = do[b, h] @ v[b, h].T
                delta = np.sum(p * dp, axis=1, keepdims=True)
                ds = p * dp if kind == "drop_delta" else p * (dp - delta)
                sgn = -1.0 if kind == "dq_sign" else 1.0
                sc = 1.0 if kind == "dk_no_scale" else scale
                dq[b, h] = sgn * scale * (ds @ k[b, h])
                dk[b, h] = sc * (ds.T @ q[b, h])
        return dq, dk, dv
    return bwd


@pytest.mark.parametrize("kind", ["drop_scale", "flip_mask", "transpose_p", "lse_no_log", "lse_no_max"])
def test_forward_pins_catch_planted_mistakes(kind):
    fwd, probs = _mut_fwd_factory(kind)
    assert fwd_pin_failures(fwd, probs), f"planted mistake {kind} went unnoticed"


@pytest.mark.parametrize("kind", ["dv_no_transpose", "drop_delta", "dq_sign", "dk_no_scale"])
def test_backward_pins_catch_planted_mistakes(kind):
    bwd = _mut_bwd_factory(kind)
    assert bwd_pin_failures(oracle.attention_fwd, bwd), f"planted mistake {kind} went unnoticed"


# ----------------------------------------------------------------------------
# queries shorter than keys (split-KV forward): pinned to the square case
# ----------------------------------------------------------------------------


def _suffix_pin_failures(fwd):
    """Causal attention of the last Sq query positions over Sk keys equals the
    last Sq rows of the square problem whose earlier rows are any queries."""
    fails = []
    sk, dd = 37, 8
    qf = _rand((1, 2, sk, dd), 21)
    k = _rand((1, 2, sk, dd), 22)
    v = _rand((1, 2, sk, dd), 23)
    of, lf = fwd(qf, k, v, 0.45, True)
    for sq in (1, 5, 36):
        o, l = fwd(qf[:, :, sk - sq :], k, v, 0.45, True)
        if np.max(np.abs(o - of[:, :, sk - sq :])) > 1e-13 or np.max(np.abs(l - lf[:, :, sk - sq :])) > 1e-13:
            fails.append(f"suffix Sq={sq}")
    return fails


def test_rectangular_causal_is_suffix_of_square():
    assert not _suffix_pin_failures(oracle.attention_fwd)


def test_single_query_causal_sees_every_key():
    q = _rand((2, 2, 1, 8), 31)
    k = _rand((2, 2, 50, 8), 32)
    v = _rand((2, 2, 50, 8), 33)
    oc, lc = oracle.attention_fwd(q, k, v, 0.3, True)
    on, ln = oracle.attention_fwd(q, k, v, 0.3, False)
    assert np.max(np.abs(oc - on)) == 0.0 and np.max(np.abs(lc - ln)) == 0.0


def test_key_chunk_merge_identity():
    """Attention over all keys equals the log-sum-exp weighted merge of the
    attentions over disjoint key chunks (the decomposition split-KV uses):
    LSE = ln sum_c exp(LSE_c),  O = sum_c exp(LSE_c - LSE) O_c."""
    q = _rand((1, 2, 9, 8), 41)
    k = _rand((1, 2, 70, 8), 42)
    v = _rand((1, 2, 70, 8), 43)
    o, l = oracle.attention_fwd(q, k, v, 0.5, False)
    bounds = [0, 13, 40, 41, 70]
    parts = [oracle.attention_fwd(q, k[:, :, a:b], v[:, :, a:b], 0.5, False) for a, b in zip(bounds, bounds[1:])]
    lse = np.log(sum(np.exp(lc) for _, lc in parts))
    om = sum(np.exp(lc - lse)[..., None] * oc for oc, lc in parts)
    assert np.max(np.abs(lse - l)) < 1e-13
    assert np.max(np.abs(om - o)) < 1e-13


def test_rectangular_rows_and_float32_paths_agree():
    torch = pytest.importorskip("torch")
    g = torch.Generator().manual_seed(12)
    q = torch.randn((1, 2, 70, 16), generator=g).to(torch.bfloat16)
    k = torch.randn((1, 2, 300, 16), generator=g).to(torch.bfloat16)
    v = torch.randn((1, 2, 300, 16), generator=g).to(torch.bfloat16)
    o64, l64 = oracle.attention_fwd(q, k, v, 0.25, True)
    o32, l32 = oracle.attention_fwd_f32(q, k, v, 0.25, True, block_rows=32)
    assert np.max(np.abs(o32.numpy() - o64[0])) < 1e-5
    assert np.max(np.abs(l32.numpy() - l64[0])) < 1e-5
    rows = [(0, 0, 0), (0, 1, 33), (0, 0, 69)]
    ro, rl = oracle.attention_fwd_rows(q, k, v, 0.25, True, rows)
    for n, (b, h, i) in enumerate(rows):
        assert np.max(np.abs(ro[n] - o64[b, h, i])) < 1e-13
        assert abs(rl[n] - l64[b, h, i]) < 1e-13


def test_causal_needs_enough_keys():
    with pytest.raises(ValueError):
        oracle.attention_fwd(_rand((1, 1, 5, 4), 1), _rand((1, 1, 3, 4), 2), _rand((1, 1, 3, 4), 3), 1.0, True)


def test_suffix_pin_catches_top_left_alignment():
    """A planted mistake -- aligning short query blocks at the first key
    position -- fails the suffix pin."""

    def fwd_top_left(q, k, v, scale, causal):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        bsz, nh, sq, _ = q.shape
        o = np.zeros((bsz, nh, sq, v.shape[-1]))
        l = np.zeros((bsz, nh, sq))
        for b in range(bsz):
            for h in range(nh):
                s = scale * (q[b, h] @ k[b, h].T)
                if causal:
                    i = np.arange(sq)[:, None]
                    j = np.arange(k.shape[2])[None, :]
                    s = np.where(j > i, -np.inf, s)
                p, l[b, h] = A.softmax_rows(s)
                o[b, h] = p @ v[b, h]
        return o, l

    assert _suffix_pin_failures(fwd_top_left)


def test_poly_exp2_constants_are_the_fit():
    """The three constants of the kernels' software exp2 (exp2_poly in
    device_common.hpp, Horner form c3 f^3 + c2 f^2 + c1 f + 1) are the
    float32 rounding of fit_exp2.py's minimax fit, and that fit's maximum
    relative error on [0, 1) is the 8.6e-5 the kernels' comments state."""
    import importlib.util
    import os
    import re

    here = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    csrc = os.path.join(here, "exact_attention_97_amd", "csrc")
    spec = importlib.util.spec_from_file_location("fit_exp2", os.path.join(csrc, "fit_exp2.py"))
    fit_exp2 = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(fit_exp2)
    c, err = fit_exp2.fit(3)
    text = open(os.path.join(csrc, "device_common.hpp")).read()
    body = text[text.index("float exp2_poly(float x)"):]
    body = body[:body.index("}")]
    lits = [float(x) for x in re.findall(r"([0-9.]+e[-+][0-9]+)f", body)]
    assert len(lits) == 3, lits
    c3, c2, c1 = (np.float32(x) for x in lits)
    assert (c1, c2, c3) == tuple(np.float32(x) for x in c)
    assert 8.5e-5 < err < 8.65e-5
    f = np.linspace(0, 1, 200001, endpoint=False)
    rel = np.max(np.abs(fit_exp2.eval_f32(c, f).astype(np.float64) / np.exp2(f) - 1.0))
    assert rel < 8.7e-5
