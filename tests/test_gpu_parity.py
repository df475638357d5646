"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle.

Tolerances (elementwise absolute error, GPU bf16 outputs against the
unrounded oracle): O, dQ, dK, dV max <= 2e-2 and mean <= 2e-3; LSE max <=
1e-3.  Small shapes use the float64 oracle on every element; the full
workload sizes use sampled rows (float64) for the forward pass and whole
heads (float32 block-of-rows oracle, itself checked against float64 in
test_oracle.py) for the backward pass.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from exact_attention_97_amd import _lib as L
from exact_attention_97_amd.inputs import WORKLOADS, make_qkvdo, make_workload

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3


def _np(t):
    import torch

    return t.detach().to("cpu", torch.float64).numpy()


def _errs(got, want):
    d = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(want, dtype=np.float64))
    return float(d.max()), float(d.mean())


def _assert_close(name, got, want, max_tol=O_MAX, mean_tol=O_MEAN):
    mx, mn = _errs(got, want)
    print(f"    {name}: max-abs {mx:.3e} mean-abs {mn:.3e}", flush=True)
    assert mx <= max_tol and mn <= mean_tol, f"{name}: max {mx:.3e} (tol {max_tol}), mean {mn:.3e} (tol {mean_tol})"


def _assert_lse(got, want):
    mx, _ = _errs(got, want)
    print(f"    LSE: max-abs {mx:.3e}", flush=True)
    assert mx <= LSE_MAX, f"LSE max {mx:.3e} (tol {LSE_MAX})"


def _gpu(*ts):
    return [t.to("cuda") for t in ts]


def _bwd_rounding_bound(q, k, v, do, scale, causal, b, h):
    """Per-element error bound of the GPU backward pass for head (b, h), from
    the roundings it makes.  The kernels round P and dS to bf16 (relative
    2^-9) before the products dV = P^T dO, dK = scale dS^T Q and
    dQ = scale dS K, and those products then carry an error up to 2^-9 times
    the matching sum of absolute terms (e.g. |scale| |dS| |K| for dQ).  Delta_i
    is formed as sum_d dO_id O_id from the bf16 output O, off by up to
    e_i = 2^-9 sum_d |dO_id O_id|; that enters dS_ij as P_ij e_i and hence dQ_i
    as |scale| e_i sum_j P_ij |K_j| and dK_j as |scale| sum_i P_ij e_i |Q_i|.
    The bound is these first-order terms with a factor 2 margin, plus one bf16
    step of the output (2^-8 |ref|) and the usual 2e-2.  The terms are formed
    in float32 from the plain definitions."""
    import torch

    qf, kf, vf, dof = (x[b, h].float() for x in (q, k, v, do))
    sc = (qf @ kf.T) * scale
    if causal:
        sc = sc.masked_fill(torch.ones_like(sc, dtype=torch.bool).triu(1), float("-inf"))
    pr = torch.softmax(sc, dim=-1)
    dpr = dof @ vf.T
    dsr = pr * (dpr - (pr * dpr).sum(-1, keepdim=True))
    of = pr @ vf
    e = (dof * of).abs().sum(-1, keepdim=True)  # sum_d |dO O|; times 2^-9 in the bound
    a = abs(scale)
    terms = {"dQ": a * (dsr.abs() @ kf.abs() + (pr * e) @ kf.abs()),
             "dK": a * (dsr.abs().T @ qf.abs() + (pr * e).T @ qf.abs()),
             "dV": pr.T @ dof.abs()}
    return {nm: 2.0 * 2.0**-9 * t.double().numpy() for nm, t in terms.items()}


def _assert_within_bound(name, got, ref, extra, check_mean=True):
    err = np.abs(got - ref)
    bound = O_MAX + 2.0**-8 * np.abs(ref) + extra
    worst = float(np.max(err - bound))
    print(f"    {name}: max-abs {err.max():.3e} (|ref| max {np.abs(ref).max():.1f}) mean-abs {err.mean():.3e} "
          f"worst-vs-bound {worst:.3e}", flush=True)
    assert worst <= 0.0
    if check_mean:
        assert err.mean() <= O_MEAN


# ----------------------------------------------------------------------------
# small and ragged shapes, every element against the float64 oracle
# ----------------------------------------------------------------------------

SMALL_S = (1, 33, 128, 300)


@pytest.mark.parametrize("D", (64, 128, 256))
@pytest.mark.parametrize("S", SMALL_S)
@pytest.mark.parametrize("causal", (False, True))
def test_fwd_small(D, S, causal):
    print(f"[fwd small] D={D} S={S} causal={causal}", flush=True)
    q, k, v, _ = make_qkvdo(1, 2, S, D, seed=100 + S + D)
    scale = 1.0 / math.sqrt(D)
    o, lse = L.attn_fwd(*_gpu(q, k, v), scale=scale, causal=causal)
    ro, rl = oracle.attention_fwd(q, k, v, scale, causal)
    _assert_close("O", _np(o), ro)
    _assert_lse(_np(lse), rl)


@pytest.mark.parametrize("exp_mode,poly_fraction", (("native", 0.5), ("poly", 0.5), ("mixed", 0.25),
                                                    ("mixed", 0.5), ("mixed", 0.75)))
@pytest.mark.parametrize("tau", (0.0, 8.0))
@pytest.mark.parametrize("causal", (False, True))
def test_fwd_exp_modes_and_tau(exp_mode, poly_fraction, tau, causal):
    print(f"[fwd modes] exp={exp_mode} frac={poly_fraction} tau={tau} causal={causal}", flush=True)
    q, k, v, _ = make_qkvdo(2, 2, 300, 128, seed=7, outlier_frac=0.01)
    o, lse = L.attn_fwd(*_gpu(q, k, v), causal=causal, exp_mode=exp_mode, rescale_tau=tau,
                        poly_fraction=poly_fraction)
    ro, rl = oracle.attention_fwd(q, k, v, 1.0 / math.sqrt(128), causal)
    _assert_close("O", _np(o), ro)
    _assert_lse(_np(lse), rl)


@pytest.mark.parametrize("tau", (0.0, 3.0, 8.0, 64.0))
def test_fwd_tau_long_rows_with_outliers(tau):
    """Unmasked tiles take the exponentials against the running max as it
    stands and rescale only when a partial row sum of the tile exceeds 2^tau;
    rows of 4096 keys with the x20 outliers make the running max jump many
    times, at every tau the ABI accepts (0 .. 64), through the eight-
    wavefront tile."""
    print(f"[fwd tau long] tau={tau}", flush=True)
    q, k, v, _ = make_qkvdo(1, 2, 4100, 128, seed=17, outlier_frac=0.01)
    L.set_variant("fwd", 1)
    try:
        for causal in (False, True):
            o, lse = L.attn_fwd(*_gpu(q, k, v), causal=causal, rescale_tau=tau)
            rows = [(0, h, i) for h in range(2) for i in range(0, 4100, 37)] + [(0, 1, 4099)]
            ro, rl = oracle.attention_fwd_rows(q, k, v, 1.0 / math.sqrt(128), causal, rows)
            idx = tuple(np.array(rows).T)
            _assert_close("O rows", o.cpu()[idx].double().numpy(), ro)
            _assert_lse(lse.cpu()[idx].double().numpy(), rl)
    finally:
        L.set_variant("fwd", -1)


@pytest.mark.parametrize("scale", (0.0, -0.3, 2.0))
def test_fwd_unusual_scale(scale):
    print(f"[fwd scale] {scale}", flush=True)
    q, k, v, _ = make_qkvdo(1, 2, 200, 64, seed=3)
    for causal in (False, True):
        o, lse = L.attn_fwd(*_gpu(q, k, v), scale=scale, causal=causal)
        ro, rl = oracle.attention_fwd(q, k, v, scale, causal)
        _assert_close("O", _np(o), ro)
        _assert_lse(_np(lse), rl)


@pytest.mark.parametrize("scale", (0.0, -0.3, 2.0))
@pytest.mark.parametrize("D,bwd_mode", ((64, "split"), (128, "split"), (128, "atomic"), (256, "split")))
def test_bwd_unusual_scale(scale, D, bwd_mode):
    """Backward with scale 0 (uniform P; dQ = dK = 0 exactly), a negative
    scale and a large one, against the float64 oracle.  At |scale| = 0.3 and
    2 the gradients of N(0,1) inputs reach 5 to 90, where a flat 2e-2 is at
    or below one bf16 step, so every element is held to the rounding bound of
    the kernels' arithmetic (_bwd_rounding_bound) instead; at scale 0 to the
    plain tolerances."""
    print(f"[bwd scale] {scale} D={D} mode={bwd_mode}", flush=True)
    q, k, v, do = make_qkvdo(1, 2, 200, D, seed=4)
    qg, kg, vg, dog = _gpu(q, k, v, do)
    for causal in (False, True):
        o, lse = L.attn_fwd(qg, kg, vg, scale=scale, causal=causal)
        dq, dk, dv = L.attn_bwd(qg, kg, vg, o, dog, lse, scale=scale, causal=causal, bwd_mode=bwd_mode)
        rdq, rdk, rdv = oracle.attention_bwd(q, k, v, do, scale, causal)
        if scale == 0.0:
            _assert_close("dQ", _np(dq), rdq)
            _assert_close("dK", _np(dk), rdk)
            _assert_close("dV", _np(dv), rdv)
            assert float(dq.abs().max()) == 0.0 and float(dk.abs().max()) == 0.0
            continue
        for h in range(2):
            bnd = _bwd_rounding_bound(q, k, v, do, scale, causal, 0, h)
            for nm, g, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
                _assert_within_bound(f"{nm} head {h} causal={causal}", _np(g[0, h]), r[0, h], bnd[nm],
                                     check_mean=False)


def test_fwd_deterministic_and_row0():
    q, k, v, _ = make_qkvdo(2, 4, 1000, 128, seed=11)
    qg, kg, vg = _gpu(q, k, v)
    o1, l1 = L.attn_fwd(qg, kg, vg, causal=True)
    o2, l2 = L.attn_fwd(qg, kg, vg, causal=True)
    assert bool((o1 == o2).all()) and bool((l1 == l2).all()), "forward pass is not bitwise repeatable"
    # causal row 0 sees only key 0: O_0 = V_0 exactly, LSE_0 = scale q_0 . k_0
    assert bool((o1[:, :, 0] == vg[:, :, 0]).all())
    want = (q[:, :, 0].double() * k[:, :, 0].double()).sum(-1) / math.sqrt(128)
    assert float((l1[:, :, 0].double().cpu() - want).abs().max()) <= LSE_MAX


def test_fwd_constant_v():
    import torch

    q, k, _, _ = make_qkvdo(1, 2, 517, 64, seed=12)
    v = torch.full((1, 2, 517, 64), 0.75, dtype=torch.bfloat16)
    for causal in (False, True):
        o, _ = L.attn_fwd(*_gpu(q, k, v), causal=causal)
        _assert_close("O (constant V)", _np(o), np.full(o.shape, 0.75))


# the atomic mode supports D = 64 and 128; the split mode also D = 256
BWD_D_MODES = ((64, "atomic"), (64, "split"), (128, "atomic"), (128, "split"), (256, "split"))


@pytest.mark.parametrize("D,bwd_mode", BWD_D_MODES)
@pytest.mark.parametrize("S", SMALL_S)
@pytest.mark.parametrize("causal", (False, True))
def test_bwd_small(D, S, causal, bwd_mode):
    print(f"[bwd small] D={D} S={S} causal={causal} mode={bwd_mode}", flush=True)
    q, k, v, do = make_qkvdo(1, 2, S, D, seed=200 + S + D)
    scale = 1.0 / math.sqrt(D)
    qg, kg, vg, dog = _gpu(q, k, v, do)
    o, lse = L.attn_fwd(qg, kg, vg, scale=scale, causal=causal)
    dq, dk, dv = L.attn_bwd(qg, kg, vg, o, dog, lse, scale=scale, causal=causal, bwd_mode=bwd_mode)
    rdq, rdk, rdv = oracle.attention_bwd(q, k, v, do, scale, causal)
    _assert_close("dQ", _np(dq), rdq)
    _assert_close("dK", _np(dk), rdk)
    _assert_close("dV", _np(dv), rdv)
    # invariants on the GPU result: sum_j dK_j = 0, sum_j dV_j = sum_i dO_i, causal dQ_0 = 0
    n = S
    assert np.max(np.abs(_np(dk).sum(axis=2))) <= n * O_MEAN + O_MAX
    assert np.max(np.abs(_np(dv).sum(axis=2) - _np(dog).sum(axis=2))) <= n * O_MEAN + O_MAX
    if causal:
        assert np.max(np.abs(_np(dq)[:, :, 0])) <= 1e-3


def test_bwd_split_deterministic_and_matches_atomic():
    """The split backward pass uses no atomics: two runs are bitwise equal; it
    agrees with the atomic pass within the tolerances."""
    q, k, v, do = _gpu(*make_qkvdo(2, 4, 1100, 128, seed=21))
    for causal in (False, True):
        o, lse = L.attn_fwd(q, k, v, causal=causal)
        a = L.attn_bwd(q, k, v, o, do, lse, causal=causal, bwd_mode="split")
        b = L.attn_bwd(q, k, v, o, do, lse, causal=causal, bwd_mode="split")
        c = L.attn_bwd(q, k, v, o, do, lse, causal=causal, bwd_mode="atomic")
        for x, y, z, nm in zip(a, b, c, ("dQ", "dK", "dV")):
            assert bool((x == y).all()), f"split {nm} not bitwise repeatable"
            _assert_close(f"{nm} split vs atomic", _np(x), _np(z))


@pytest.mark.parametrize("B,H,S", [(1, 2, 128), (2, 2, 256), (1, 3, 640), (1, 2, 2048)])
@pytest.mark.parametrize("causal", (False, True))
def test_bwd_fused_atomic_small(B, H, S, causal):
    """The atomic mode at D = 128 with S a multiple of 128 runs the fused
    kernel (dQ formed beside dK and dV from dS in LDS, added with fp32
    atomics): every element against the float64 oracle."""
    print(f"[bwd fused] B={B} H={H} S={S} causal={causal}", flush=True)
    q, k, v, do = make_qkvdo(B, H, S, 128, seed=60 + S + B)
    scale = 1.0 / math.sqrt(128)
    qg, kg, vg, dog = _gpu(q, k, v, do)
    o, lse = L.attn_fwd(qg, kg, vg, scale=scale, causal=causal)
    dq, dk, dv = L.attn_bwd(qg, kg, vg, o, dog, lse, scale=scale, causal=causal, bwd_mode="atomic")
    rdq, rdk, rdv = oracle.attention_bwd(q, k, v, do, scale, causal)
    _assert_close("dQ", _np(dq), rdq)
    _assert_close("dK", _np(dk), rdk)
    _assert_close("dV", _np(dv), rdv)
    # dK and dV come from the same tile code as the split mode; non-causal
    # workgroups walk the query tiles in a rotated order, so the fp32 sums
    # differ in order only
    sq, sk, sv = L.attn_bwd(qg, kg, vg, o, dog, lse, scale=scale, causal=causal, bwd_mode="split")
    _assert_close("dK fused vs split", _np(dk), _np(sk), max_tol=4e-3, mean_tol=2e-4)
    _assert_close("dV fused vs split", _np(dv), _np(sv), max_tol=4e-3, mean_tol=2e-4)


def test_bwd_fused_atomic_full_size():
    """The fused atomic mode at the headline backward shape (B=2 H=16 S=8192
    D=128, iid inputs, the launch the benchmark times): whole heads against
    the float32 block-of-rows oracle."""
    import torch

    w = WORKLOADS["bwd8k"]
    q, k, v, do = make_workload(w)
    qg, kg, vg, dog = _gpu(q, k, v, do)
    for causal in w.causal:
        o, lse = L.attn_fwd(qg, kg, vg, scale=w.scale, causal=causal)
        dq, dk, dv = L.attn_bwd(qg, kg, vg, o, dog, lse, scale=w.scale, causal=causal, bwd_mode="atomic")
        torch.cuda.synchronize()
        _check_bwd_heads(w, q, k, v, do, dq, dk, dv, causal, [(0, 3), (1, 14)])


def test_bwd_split_full_size():
    import torch

    w = WORKLOADS["bwd8k"]
    q, k, v, do = make_workload(w)
    qg, kg, vg, dog = _gpu(q, k, v, do)
    for causal in w.causal:
        o, lse = L.attn_fwd(qg, kg, vg, scale=w.scale, causal=causal)
        dq, dk, dv = L.attn_bwd(qg, kg, vg, o, dog, lse, scale=w.scale, causal=causal, bwd_mode="split")
        torch.cuda.synchronize()
        _check_bwd_heads(w, q, k, v, do, dq, dk, dv, causal, [(1, 9)])


def test_bwd_d256_split_deterministic_atomic_unsupported():
    """D = 256: the split pass (dK / dV columns in two halves, one workgroup
    each) is bitwise repeatable; the atomic pass reports the head dim as
    unsupported."""
    q, k, v, do = _gpu(*make_qkvdo(1, 2, 333, 256, seed=1))
    for causal in (False, True):
        o, lse = L.attn_fwd(q, k, v, causal=causal)
        a = L.attn_bwd(q, k, v, o, do, lse, causal=causal, bwd_mode="split")
        b = L.attn_bwd(q, k, v, o, do, lse, causal=causal, bwd_mode="split")
        for x, y, nm in zip(a, b, ("dQ", "dK", "dV")):
            assert bool((x == y).all()), f"D=256 split {nm} not bitwise repeatable"
    with pytest.raises(L.AttnError) as e:
        L.attn_bwd(q, k, v, o, do, lse, bwd_mode="atomic")
    assert e.value.code == 3


# ----------------------------------------------------------------------------
# the named workloads at full size
# ----------------------------------------------------------------------------


def _sample_rows(w, n, seed):
    rng = np.random.default_rng(seed)
    rows = {(int(rng.integers(w.B)), int(rng.integers(w.H)), int(rng.integers(w.S))) for _ in range(n)}
    rows |= {(0, 0, 0), (w.B - 1, w.H - 1, w.S - 1)}
    return sorted(rows)


def _check_fwd_rows(w, q, k, v, o, lse, causal, nrows=512):
    rows = _sample_rows(w, nrows, w.seed)
    ro, rl = oracle.attention_fwd_rows(q, k, v, w.scale, causal, rows)
    idx = tuple(np.array(rows).T)
    og = o.cpu()[idx].double().numpy()
    lg = lse.cpu()[idx].double().numpy()
    _assert_close(f"O ({len(rows)} sampled rows)", og, ro)
    _assert_lse(lg, rl)


def _check_bwd_heads(w, q, k, v, do, dq, dk, dv, causal, heads):
    rdq, rdk, rdv = oracle.attention_bwd_f32(q, k, v, do, w.scale, causal, heads=heads)
    for n, (b, h) in enumerate(heads):
        _assert_close(f"dQ head {(b, h)}", _np(dq[b, h]), rdq[n].numpy())
        _assert_close(f"dK head {(b, h)}", _np(dk[b, h]), rdk[n].numpy())
        _assert_close(f"dV head {(b, h)}", _np(dv[b, h]), rdv[n].numpy())


def test_workload_tiny_full():
    w = WORKLOADS["tiny"]
    q, k, v, do = make_workload(w)
    qg, kg, vg, dog = _gpu(q, k, v, do)
    o, lse = L.attn_fwd(qg, kg, vg, scale=w.scale, causal=False)
    ro, rl = oracle.attention_fwd(q, k, v, w.scale, False)
    _assert_close("O", _np(o), ro)
    _assert_lse(_np(lse), rl)
    dq, dk, dv = L.attn_bwd(qg, kg, vg, o, dog, lse, scale=w.scale, causal=False)
    rdq, rdk, rdv = oracle.attention_bwd(q, k, v, do, w.scale, False)
    _assert_close("dQ", _np(dq), rdq)
    _assert_close("dK", _np(dk), rdk)
    _assert_close("dV", _np(dv), rdv)


@pytest.mark.parametrize("name", ("fwd2k", "long8k", "bwd4k", "bwd8k", "d64", "d256", "ctx32k"))
def test_workload_full_size(name):
    import torch

    w = WORKLOADS[name]
    print(f"[workload] {name} B={w.B} H={w.H} S={w.S} D={w.D}", flush=True)
    q, k, v, do = make_workload(w)
    qg, kg, vg, dog = _gpu(q, k, v, do)
    for causal in w.causal:
        print(f"  causal={causal}", flush=True)
        o, lse = L.attn_fwd(qg, kg, vg, scale=w.scale, causal=causal)
        torch.cuda.synchronize()
        _check_fwd_rows(w, q, k, v, o, lse, causal, nrows=1024)
        if "bwd" in w.passes:
            dq, dk, dv = L.attn_bwd(qg, kg, vg, o, dog, lse, scale=w.scale, causal=causal)
            torch.cuda.synchronize()
            _check_bwd_heads(w, q, k, v, do, dq, dk, dv, causal, [(0, 0), (w.B - 1, w.H - 1)])
        del o, lse


def test_bwd_outliers_rounding_bound():
    """Backward on the outlier inputs (Q, K entries x20 with probability 1%).

    Here the gradients reach magnitudes where an absolute 2e-2 is below what
    bf16 operands allow: the kernels round P and dS to bf16 (relative 2^-9)
    before the products dV = P^T dO, dK = scale dS^T Q and dQ = scale dS K,
    and those products then carry an error up to 2^-9 times the matching sum
    of absolute terms (e.g. scale |dS| |K| for dQ), which outlier rows of K
    make large even where dQ itself is small.  Second, Delta_i is formed as
    sum_d dO_id O_id from the bf16 output O (the forward pass keeps no fp32
    copy), which is off by up to e_i = 2^-9 sum_d |dO_id O_id|; that enters
    dS_ij as P_ij e_i and hence dQ_i as scale e_i sum_j P_ij |K_j| and dK_j
    as scale sum_i P_ij e_i |Q_i| (K and Q with x20 outliers amplify it).
    The per-element bound is these first-order terms (with a factor 2
    margin), plus one bf16 step of the output and the usual 2e-2; the mean
    bound stays 2e-3.  The absolute terms are formed here in float32 from
    the plain definitions.
    """
    import torch

    w = WORKLOADS["long8k"]
    q, k, v, do = make_qkvdo(1, 2, 4096, 128, seed=w.seed, outlier_frac=w.outlier_frac)
    qg, kg, vg, dog = _gpu(q, k, v, do)
    for causal in (False, True):
        o, lse = L.attn_fwd(qg, kg, vg, scale=w.scale, causal=causal)
        dq, dk, dv = L.attn_bwd(qg, kg, vg, o, dog, lse, scale=w.scale, causal=causal)
        torch.cuda.synchronize()
        rdq, rdk, rdv = oracle.attention_bwd_f32(q, k, v, do, w.scale, causal, heads=[(0, 0), (0, 1)])
        for n, h in enumerate((0, 1)):
            bnd = _bwd_rounding_bound(q, k, v, do, w.scale, causal, 0, h)
            for nm, g, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
                _assert_within_bound(f"{nm} head {h} causal={causal}", _np(g[0, h]), r[n].double().numpy(),
                                     bnd[nm])


def test_exp2_eval_against_exact():
    """The kernels' exp2 against float64 exp2: 1.6e7 evenly spaced points over
    [-127, 0] plus the positive range the kernels can meet (up to 2^8 with
    the conditional rescale), and every float32 value in [-1, 0]
    (1 065 353 217 values, evaluated in chunks on the device and compared
    there with torch's float64 exp2).  Native: the hardware instruction;
    poly: the degree-3 fit, max relative error 8.6e-5 by its fit.  Below
    x = -126 the exact result is a float32 subnormal, which the device
    flushes to zero: there the error is held to the smallest normal float32
    (2^-126) in absolute terms, a contribution no softmax row can see next to
    its largest term, 1."""
    import torch

    x = torch.cat([torch.linspace(-127.0, 0.0, 16_000_001, dtype=torch.float32),
                   torch.linspace(0.0, 8.0, 1_000_001, dtype=torch.float32)])
    want = oracle.exp2_exact(x.numpy())
    tiny = 2.0**-126
    normal = want >= tiny
    for mode, bound in (("native", 2e-6), ("poly", 1.0e-4)):
        y = L.exp2_eval(x.cuda(), mode).cpu().double().numpy()
        rel = np.max(np.abs(y[normal] / want[normal] - 1.0))
        sub = np.max(np.abs(y[~normal] - want[~normal]))
        print(f"    exp2 {mode} on {x.numel()} points: max rel err {rel:.3e} (normal results), "
              f"max abs err {sub:.3e} below 2^-126", flush=True)
        assert rel <= bound and sub <= tiny
    # every float32 in [-1, 0]: the bit patterns of [0, 1] with the sign bit set
    top = 0x3F800000  # bits of 1.0f
    chunk = 1 << 26
    worst = {"native": 0.0, "poly": 0.0}
    for start in range(0, top + 1, chunk):
        bits = torch.arange(start, min(start + chunk, top + 1), dtype=torch.int32, device="cuda")
        xs = (bits | torch.tensor(-0x80000000, dtype=torch.int32, device="cuda")).view(torch.float32)
        ref = torch.exp2(xs.double())
        for mode in worst:
            y = L.exp2_eval(xs, mode).double()
            worst[mode] = max(worst[mode], float((y / ref - 1.0).abs().max()))
    print(f"    exp2 on every float32 in [-1, 0]: max rel err {worst}", flush=True)
    assert worst["native"] <= 2e-6 and worst["poly"] <= 1.0e-4
    assert float(L.exp2_eval(torch.zeros(1, device="cuda"), "poly").item()) == 1.0
    assert float(L.exp2_eval(torch.full((1,), -0.0, device="cuda"), "poly").item()) == 1.0


# ----------------------------------------------------------------------------
# split-KV forward: queries and keys of different lengths, keys split into
# chunks merged by their log-sum-exp; against the float64 oracle
# ----------------------------------------------------------------------------

from exact_attention_97_amd.inputs import SPLITKV_WORKLOADS, make_qkv_rect  # noqa: E402

SPLIT_SHAPES = [  # (Sq, Sk)
    (1, 1), (1, 700), (7, 300), (128, 128), (130, 1000), (300, 4100), (33, 65),
]


@pytest.mark.parametrize("D", (64, 128, 256))
@pytest.mark.parametrize("shape", SPLIT_SHAPES)
@pytest.mark.parametrize("causal", (False, True))
@pytest.mark.parametrize("num_splits", (0, 1, 3, 1000))
def test_splitkv_small(D, shape, causal, num_splits):
    Sq, Sk = shape
    if causal and Sk < Sq:
        pytest.skip("causal needs Sk >= Sq")
    print(f"[splitkv small] D={D} Sq={Sq} Sk={Sk} causal={causal} splits={num_splits}", flush=True)
    q, k, v = make_qkv_rect(1, 2, Sq, Sk, D, seed=300 + Sq + Sk + D)
    scale = 1.0 / math.sqrt(D)
    o, lse = L.attn_fwd_splitkv(*_gpu(q, k, v), scale=scale, causal=causal, num_splits=num_splits)
    ro, rl = oracle.attention_fwd(q, k, v, scale, causal)
    _assert_close("O", _np(o), ro)
    _assert_lse(_np(lse), rl)


def test_splitkv_square_matches_fwd():
    """With Sq == Sk, split-KV agrees with the one-pass forward kernel."""
    import torch

    for causal in (False, True):
        q, k, v, _ = make_qkvdo(2, 4, 1000, 128, seed=11)
        q, k, v = _gpu(q, k, v)
        o1, l1 = L.attn_fwd(q, k, v, causal=causal)
        o2, l2 = L.attn_fwd_splitkv(q, k, v, causal=causal, num_splits=4)
        torch.cuda.synchronize()
        _assert_close("O split vs fwd", _np(o2), _np(o1), max_tol=4e-3, mean_tol=2e-4)
        assert float((l1 - l2).abs().max()) <= 1e-5


def test_splitkv_rejects_bad_arguments():
    import torch

    q, k, v = (t.cuda() for t in make_qkv_rect(1, 1, 8, 4, 64, seed=1))
    with pytest.raises(L.AttnError) as e:
        L.attn_fwd_splitkv(q, k, v, causal=True)  # Sk < Sq
    assert e.value.code == 2
    q, k, v = (t.cuda() for t in make_qkv_rect(1, 1, 4, 8, 64, seed=1))
    with pytest.raises(L.AttnError) as e:
        L.attn_fwd_splitkv(q, k, v, num_splits=-1)
    assert e.value.code == 7
    with pytest.raises(L.AttnError) as e:
        L.attn_fwd_splitkv(q, k, v, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert e.value.code == 5


@pytest.mark.parametrize("name", sorted(SPLITKV_WORKLOADS))
def test_splitkv_workload_full_size(name):
    """Full size, sampled rows against the float64 oracle (rows are independent)."""
    w = SPLITKV_WORKLOADS[name]
    print(f"[splitkv workload] {name}", flush=True)
    q, k, v = make_qkv_rect(w.B, w.H, w.Sq, w.Sk, w.D, w.seed, std=w.std)
    o, lse = L.attn_fwd_splitkv(*_gpu(q, k, v), scale=w.scale, causal=w.causal)
    rng = np.random.default_rng(w.seed)
    n = min(256, w.B * w.H * w.Sq)
    rows = sorted({(int(rng.integers(w.B)), int(rng.integers(w.H)), int(rng.integers(w.Sq))) for _ in range(n)})
    rows += [(0, 0, w.Sq - 1), (w.B - 1, w.H - 1, 0)]
    ro, rl = oracle.attention_fwd_rows(q, k, v, w.scale, w.causal, rows)
    on, ln = _np(o), _np(lse)
    got_o = np.stack([on[b, h, i] for b, h, i in rows])
    got_l = np.array([ln[b, h, i] for b, h, i in rows])
    _assert_close("O rows", got_o, ro)
    _assert_lse(got_l, rl)


# ----------------------------------------------------------------------------
# kernel variants kept for measurement (fwd 1 / 2: the eight- / four-wavefront
# tile at every length; dQ 1 / 2: the four- / eight-wavefront dQ tile):
# each against the float64 oracle, ragged length, both causal settings
# ----------------------------------------------------------------------------

VARIANTS = [("fwd", 1), ("fwd", 2), ("bwd_dq", 1), ("bwd_dq", 2)]


@pytest.mark.parametrize("kernel,variant", VARIANTS)
def test_kernel_variants_match_oracle(kernel, variant):
    print(f"[variant] {kernel} {variant}", flush=True)
    q, k, v, do = make_qkvdo(1, 2, 333, 128, seed=40 + variant)
    scale = 1.0 / math.sqrt(128)
    qg, kg, vg, dog = _gpu(q, k, v, do)
    L.set_variant(kernel, variant)
    try:
        for causal in (False, True):
            o, lse = L.attn_fwd(qg, kg, vg, scale=scale, causal=causal)
            ro, rl = oracle.attention_fwd(q, k, v, scale, causal)
            _assert_close("O", _np(o), ro)
            _assert_lse(_np(lse), rl)
            if kernel != "fwd":
                dq, dk, dv = L.attn_bwd(qg, kg, vg, o, dog, lse, scale=scale, causal=causal, bwd_mode="split")
                rdq, rdk, rdv = oracle.attention_bwd(q, k, v, do, scale, causal)
                _assert_close("dQ", _np(dq), rdq)
                _assert_close("dK", _np(dk), rdk)
                _assert_close("dV", _np(dv), rdv)
    finally:
        L.set_variant(kernel, -1)


# ----------------------------------------------------------------------------
# LDS tiles of two 64-key steps (the eight-wavefront forward, forced at every
# length by fwd variant 1, and the default D = 128 dQ kernel): lengths whose
# last tile ends inside its first step, at its boundary, or inside the second
# step (whose load is skipped when it starts at or past S); the forward's K
# tiles are offset by one step, so its boundaries fall 64 keys later
# ----------------------------------------------------------------------------

TWO_STEP_LENGTHS = (1, 33, 64, 65, 127, 128, 129, 191, 192, 193, 300, 320)


@pytest.mark.parametrize("S", TWO_STEP_LENGTHS)
def test_two_step_tiles_ragged(S):
    print(f"[two-step tiles] S={S}", flush=True)
    q, k, v, do = make_qkvdo(1, 2, S, 128, seed=300 + S)
    scale = 1.0 / math.sqrt(128)
    qg, kg, vg, dog = _gpu(q, k, v, do)
    for causal in (False, True):
        L.set_variant("fwd", 1)
        try:
            o, lse = L.attn_fwd(qg, kg, vg, scale=scale, causal=causal)
        finally:
            L.set_variant("fwd", -1)
        ro, rl = oracle.attention_fwd(q, k, v, scale, causal)
        _assert_close("O", _np(o), ro)
        _assert_lse(_np(lse), rl)
        dq, dk, dv = L.attn_bwd(qg, kg, vg, o, dog, lse, scale=scale, causal=causal, bwd_mode="split")
        rdq, rdk, rdv = oracle.attention_bwd(q, k, v, do, scale, causal)
        _assert_close("dQ", _np(dq), rdq)
        _assert_close("dK", _np(dk), rdk)
        _assert_close("dV", _np(dv), rdv)


# ----------------------------------------------------------------------------
# D = 64 and 256 split backward: the pipelined dK / dV tile (at D = 256 with
# the columns split between two workgroups; bwd_dkdv variant 1: the one-pass
# tile it replaced), every element against the float64 oracle.  Ragged
# lengths with an odd number of 64-query tiles (150, 700) walk one extra
# all-zero tile; 333 has an even count and a partial last tile.
# ----------------------------------------------------------------------------


@pytest.mark.parametrize("D", (64, 256))
@pytest.mark.parametrize("S", (128, 256, 640, 150, 333, 700))
@pytest.mark.parametrize("variant", (0, 1))
def test_bwd_dkdv_tiles_d64_d256(D, S, variant):
    print(f"[dkdv tiles] D={D} S={S} variant={variant}", flush=True)
    q, k, v, do = make_qkvdo(1, 2, S, D, seed=400 + S + D)
    scale = 1.0 / math.sqrt(D)
    qg, kg, vg, dog = _gpu(q, k, v, do)
    L.set_variant("bwd_dkdv", variant)
    try:
        for causal in (False, True):
            o, lse = L.attn_fwd(qg, kg, vg, scale=scale, causal=causal)
            dq, dk, dv = L.attn_bwd(qg, kg, vg, o, dog, lse, scale=scale, causal=causal, bwd_mode="split")
            rdq, rdk, rdv = oracle.attention_bwd(q, k, v, do, scale, causal)
            _assert_close("dQ", _np(dq), rdq)
            _assert_close("dK", _np(dk), rdk)
            _assert_close("dV", _np(dv), rdv)
    finally:
        L.set_variant("bwd_dkdv", -1)


# ----------------------------------------------------------------------------
# Block order with B*H a multiple of 8 (each XCD takes whole heads, one head's
# tiles together in non-causal passes) at small, ragged and tile-multiple
# lengths: every element of the forward and backward outputs against the
# float64 oracle (the other small tests have B*H of 2 to 6, the other order)
# ----------------------------------------------------------------------------


@pytest.mark.parametrize("B,H,S,D", ((2, 4, 300, 128), (1, 8, 640, 128), (2, 8, 256, 64), (1, 8, 384, 256)))
def test_grouped_block_order(B, H, S, D):
    """O and LSE to the plain tolerances; the gradients to the plain mean
    tolerance and, per element, to the rounding bound of the kernels'
    arithmetic (_bwd_rounding_bound): with eight and sixteen heads the
    early rows of a causal pass, which see few keys, carry gradients whose
    bf16 P and dS roundings alone can reach a flat 2e-2 (B=1, H=8, S=640:
    one dQ element 2.3e-2 off, |dQ| <= 3.6 there, mean error 2e-4)."""
    print(f"[grouped block order] B={B} H={H} S={S} D={D}", flush=True)
    q, k, v, do = make_qkvdo(B, H, S, D, seed=600 + S + D)
    scale = 1.0 / math.sqrt(D)
    qg, kg, vg, dog = _gpu(q, k, v, do)
    for causal in (False, True):
        o, lse = L.attn_fwd(qg, kg, vg, scale=scale, causal=causal)
        ro, rl = oracle.attention_fwd(q, k, v, scale, causal)
        _assert_close("O", _np(o), ro)
        _assert_lse(_np(lse), rl)
        dq, dk, dv = L.attn_bwd(qg, kg, vg, o, dog, lse, scale=scale, causal=causal, bwd_mode="split")
        rdq, rdk, rdv = oracle.attention_bwd(q, k, v, do, scale, causal)
        for nm, g, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
            assert float(np.abs(_np(g) - r).mean()) <= O_MEAN, nm
        for b in range(B):
            for h in range(H):
                bnd = _bwd_rounding_bound(q, k, v, do, scale, causal, b, h)
                for nm, g, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
                    _assert_within_bound(f"{nm} ({b}, {h}) causal={causal}", _np(g[b, h]), r[b, h], bnd[nm],
                                         check_mean=False)
