"""GPU: the library's calls can be captured in a HIP graph (torch.cuda.CUDAGraph).

The forward, the split backward and the FP8 path launch kernels only (their
zero-fills are kernels, never memset nodes).  The graph is replayed several
times with eager work and synchronisations in between, and every replay is
compared bit for bit with the eager result (all of these kernels are
deterministic).
"""

from __future__ import annotations

import pytest

from exact_attention_97_amd import _lib as L
from exact_attention_97_amd.inputs import hadamard_signs, make_qkvdo

pytestmark = pytest.mark.gpu


def test_graph_capture_and_replay():
    import torch

    B, H, S, D = 1, 4, 777, 128
    print("[graph] capture fwd + split bwd + fp8 fwd", flush=True)
    q, k, v, do = (t.cuda() for t in make_qkvdo(B, H, S, D, seed=50))
    sg = hadamard_signs(D, 11).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(L.bwd_workspace_bytes(B, H, S, D, True), dtype=torch.uint8, device="cuda")
    buf = torch.empty(L.fp8_buffer_bytes(B, H, S, D), dtype=torch.uint8, device="cuda")
    o8 = torch.empty_like(q)
    lse8 = torch.empty_like(lse)

    def work():
        L.attn_fwd(q, k, v, causal=True, out=o, lse=lse)
        L.attn_bwd(q, k, v, o, do, lse, causal=True, workspace=ws, dq=dq, dk=dk, dv=dv)
        L.fp8_quantize(q, k, v, sg, buf=buf)
        L.attn_fwd_fp8_quantized(buf, B, H, S, D, causal=True, out=o8, lse=lse8)

    # eager reference (and warm-up on a side stream, as graph capture wants)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, dq, dk, dv, o8, lse8)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(3):
        for t in (o, lse, dq, dk, dv, o8, lse8):
            t.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("O", "LSE", "dQ", "dK", "dV", "O fp8", "LSE fp8"), (o, lse, dq, dk, dv, o8, lse8), ref):
            assert bool((t == r).all()), f"replay {rep}: {name} differs from the eager result"
        print(f"    replay {rep}: all outputs bitwise equal to eager", flush=True)
