"""The no-allocation backward entry point (attn_bwd_noalloc) against attn_bwd.

attn_bwd_noalloc runs the same kernels as attn_bwd with the library's fixed
device scratch as the workspace, so in the split mode (no atomics) its
outputs are bitwise equal to attn_bwd's, and in the atomic mode equal within
the tolerances (the order of the fp32 atomic additions varies).  Two calls in
a row, the second with a smaller input, check that nothing an earlier call
left in the scratch leaks into a later one.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from exact_attention_97_amd import _lib as L
from exact_attention_97_amd.inputs import make_qkvdo

pytestmark = pytest.mark.gpu


def _run(shape, causal, mode, seed):
    import torch

    B, H, S, D = shape
    q, k, v, do = make_qkvdo(B, H, S, D, seed=seed)
    qg, kg, vg, dog = (t.cuda() for t in (q, k, v, do))
    scale = 1.0 / math.sqrt(D)
    o, lse = L.attn_fwd(qg, kg, vg, scale=scale, causal=causal)
    ref = L.attn_bwd(qg, kg, vg, o, dog, lse, scale=scale, causal=causal, bwd_mode=mode)
    out = tuple(torch.full_like(qg, float("nan")) for _ in range(3))
    L.attn_bwd_noalloc(qg, kg, vg, o, dog, lse, *out, scale=scale, causal=causal, bwd_mode=mode)
    torch.cuda.synchronize()
    return (q, k, v, do, scale), ref, out


@pytest.mark.parametrize("mode", ["split", "atomic"])
def test_noalloc_matches_workspace_entry_point_twice(mode):
    for n, (shape, causal) in enumerate((((2, 4, 1000, 128), True), ((1, 2, 300, 64), False))):
        print(f"[noalloc] call {n + 1} mode={mode} shape={shape} causal={causal}", flush=True)
        (q, k, v, do, scale), ref, out = _run(shape, causal, mode, seed=50 + n)
        for nm, a, b in zip(("dQ", "dK", "dV"), out, ref):
            if mode == "split":
                assert bool((a == b).all()), f"{nm}: no-allocation result differs from attn_bwd"
            else:
                d = (a.double() - b.double()).abs()
                assert float(d.max()) <= 4e-3 and bool(a.isfinite().all()), f"{nm}: max diff {float(d.max()):.3e}"
        # and to the oracle, on the smaller call (every element)
        if n == 1:
            rdq, rdk, rdv = oracle.attention_bwd(q, k, v, do, scale, causal)
            for nm, g, r in zip(("dQ", "dK", "dV"), out, (rdq, rdk, rdv)):
                err = np.abs(g.cpu().double().numpy() - r)
                print(f"    {nm}: max-abs {err.max():.3e} mean-abs {err.mean():.3e}", flush=True)
                assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_noalloc_rejects_beyond_scratch_on_device():
    import torch

    q = torch.zeros((1, 65, 65536, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 65, 65536), dtype=torch.float32, device="cuda")
    with pytest.raises(L.AttnError) as e:
        L.attn_bwd_noalloc(q, q, q, q, q, lse, q, q, q)
    assert e.value.code == 8
