"""Launch driver for hardware-counter and kernel-trace runs.

Runs, in one process: an optional device-to-device copy of known size (the
calibration kernel for the HBM byte counters: it reads and writes exactly
``--copy-mib`` MiB), then ``--iters`` launches of each requested attention
pass on the headline shape's synthetic inputs.  It prints one line per step
and nothing else, so a counter run over it sees only these kernels plus
input set-up.

    python3 -m exact_attention_97_amd.profile_driver --passes fwd,bwd --iters 2 --copy-mib 1024
    python3 -m exact_attention_97_amd.profile_driver --passes fwd --exp-mode poly --tau 0 --iters 5
    python3 -m exact_attention_97_amd.profile_driver --passes fwd,bwd --outliers --bwd-seed 7

``--bwd-seed N`` gives the backward pass inputs of its own (iid N(0,1), seed
N, with O and LSE from one forward call on them), as in the benchmark, whose
backward leg runs on the iid workload and its forward leg on the outlier one.
"""

from __future__ import annotations

import argparse
import math

import torch

from . import _lib as L
from .inputs import make_qkvdo


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--passes", default="fwd,bwd", help="comma list of fwd, bwd, fp8 (quantize + FP8 forward)")
    ap.add_argument("--causal", type=int, default=0)
    ap.add_argument("--B", type=int, default=2)
    ap.add_argument("--H", type=int, default=16)
    ap.add_argument("--S", type=int, default=8192)
    ap.add_argument("--D", type=int, default=128)
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--iters", type=int, default=2)
    ap.add_argument("--bwd-mode", default="split", choices=["split", "atomic"])
    ap.add_argument("--exp-mode", default="native", choices=["native", "poly", "mixed"], help="forward exp2")
    ap.add_argument("--poly-fraction", type=float, default=0.5, help="share of polynomial exp2 in the mixed mode")
    ap.add_argument("--bwd-seed", type=int, default=None, help="separate iid inputs for the backward pass")
    ap.add_argument("--tau", type=float, default=8.0, help="forward rescale threshold (log2 units)")
    ap.add_argument("--copy-mib", type=int, default=0, help="MiB of the calibration copy (0 = none)")
    ap.add_argument("--outliers", action="store_true", help="1%% of Q and K entries x20 (the benchmark's inputs)")
    a = ap.parse_args()
    if not torch.cuda.is_available():
        raise SystemExit("profile_driver needs a GPU")
    L.load()
    dev = torch.device("cuda:0")

    if a.copy_mib > 0:
        x = torch.ones(a.copy_mib << 18, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
        print(f"copy {a.copy_mib} MiB done", flush=True)
        del x, y

    extra = dict(outlier_frac=0.01, outlier_scale=20.0) if a.outliers else {}
    q, k, v, do = (t.to(dev) for t in make_qkvdo(a.B, a.H, a.S, a.D, a.seed, **extra))
    scale = 1.0 / math.sqrt(a.D)
    causal = bool(a.causal)
    o, lse = L.attn_fwd(q, k, v, scale=scale, causal=causal)
    torch.cuda.synchronize()
    passes = [p for p in a.passes.split(",") if p]
    for p in passes:
        if p == "fwd":
            for _ in range(a.iters):
                L.attn_fwd(q, k, v, scale=scale, causal=causal, exp_mode=a.exp_mode, rescale_tau=a.tau,
                           poly_fraction=a.poly_fraction, out=o, lse=lse)
        elif p == "fp8":
            from .inputs import hadamard_signs

            sg = hadamard_signs(a.D, 11).to(dev)
            buf = L.fp8_quantize(q, k, v, sg)
            for _ in range(a.iters):
                L.fp8_quantize(q, k, v, sg, buf=buf)
                L.attn_fwd_fp8_quantized(buf, a.B, a.H, a.S, a.D, scale=scale, causal=causal, out=o, lse=lse)
        elif p == "bwd":
            bq, bk, bv, bdo, bo, blse = q, k, v, do, o, lse
            if a.bwd_seed is not None:
                bq, bk, bv, bdo = (t.to(dev) for t in make_qkvdo(a.B, a.H, a.S, a.D, a.bwd_seed))
                bo, blse = L.attn_fwd(bq, bk, bv, scale=scale, causal=causal)
                torch.cuda.synchronize()
            ws = torch.empty(L.bwd_workspace_bytes(a.B, a.H, a.S, a.D, causal, bwd_mode=a.bwd_mode),
                             dtype=torch.uint8, device=dev)
            g = [torch.empty_like(q) for _ in range(3)]
            for _ in range(a.iters):
                L.attn_bwd(bq, bk, bv, bo, bdo, blse, scale=scale, causal=causal, bwd_mode=a.bwd_mode,
                           workspace=ws, dq=g[0], dk=g[1], dv=g[2])
        else:
            raise SystemExit(f"unknown pass {p!r}")
        torch.cuda.synchronize()
        print(f"{p} x{a.iters} done", flush=True)


if __name__ == "__main__":
    main()
