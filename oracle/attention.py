"""Plain, slow, obviously correct attention on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): the GPU library must
never import or call this module.

What is computed, and where it comes from
-----------------------------------------
* Attention is two matrix products with a softmax between them: the scores
  S = Q K^T and the output O = P V.  Stated on page "FlashAttention-4 : comment
  Together AI a accéléré l'attention sur GPU Blackwell", section "Pourquoi
  l'approche standard ne fonctionne plus" (and its Portuguese twin), and on
  page "FlashAttention-3 и FlashAttention-4", section "Режим 2-CTA MMA", which
  lists what sits between the two products: softmax, normalisation, masking
  and row reductions.
* The pages print neither the softmax nor the log-sum-exp nor the backward
  pass.  The plain definitions are used:
    S_ij = scale * q_i . k_j ;  causal: S_ij = -inf for key j > query i
    m_i = max_j S_ij ;  l_i = sum_j exp(S_ij - m_i)
    P_ij = exp(S_ij - m_i) / l_i ;  O = P V ;  LSE_i = m_i + ln l_i
  and, for a loss whose gradient with respect to O is dO, the chain rule:
    dV = P^T dO ;  dP = dO V^T ;  Delta_i = sum_j P_ij dP_ij
    dS = P * (dP - Delta) ;  dQ = scale * dS K ;  dK = scale * dS^T Q
* The backward oracle works from Q, K, V and dO only; it never consumes the
  GPU's O or LSE, so it stays independent of the code under test.

Precision: ``attention_fwd`` / ``attention_bwd`` / ``attention_fwd_rows`` work
in float64 with numpy.  ``attention_fwd_f32`` / ``attention_bwd_f32`` are the
same definitions in float32 with torch CPU matrix products, processed a block
of full score rows at a time so that the long sequences fit in memory (every
row of S and P is still formed in full; nothing is approximated).

The tiling, online softmax and conditional rescaling of the GPU kernels are
exact rearrangements of this definition in exact arithmetic, so this is the
result they must reproduce up to rounding.
"""

from __future__ import annotations

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)


def _f64(x) -> np.ndarray:
    """Upcast a numpy array or a CPU torch tensor (any float dtype) to float64."""
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu")
        import torch  # local: the fp64 oracle itself needs only numpy

        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def scores(q, k, scale: float, causal: bool) -> np.ndarray:
    """Scaled scores of one head: S = scale * Q K^T, with the causal mask.

    q: [Sq, D], k: [Sk, D] with Sk >= Sq when causal.  Causal masking uses
    0-based indices; the queries are the last Sq of the Sk positions (the
    plain reading for a query block that continues a longer key sequence),
    so key j is hidden from query i when j > i + (Sk - Sq).  With Sq == Sk
    this is j > i.
    """
    q = _f64(q)
    k = _f64(k)
    s = scale * (q @ k.T)
    if causal:
        sq, sk = s.shape
        if sk < sq:
            raise ValueError("causal attention needs at least as many keys as queries")
        i = np.arange(sq)[:, None]
        j = np.arange(sk)[None, :]
        s = np.where(j > i + (sk - sq), -np.inf, s)
    return s


def softmax_rows(s: np.ndarray):
    """Row softmax of a score matrix; returns (P, LSE) with LSE the natural log."""
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=1, keepdims=True)
    p = e / l
    lse = (m + np.log(l))[:, 0]
    return p, lse


def attention_probs(q, k, scale: float, causal: bool) -> np.ndarray:
    """The attention weights P = softmax(S) for one head, float64."""
    p, _ = softmax_rows(scores(q, k, scale, causal))
    return p


def attention_fwd(q, k, v, scale: float, causal: bool):
    """Forward pass over [B, H, Sq, D] queries and [B, H, Sk, D] keys/values.

    Returns (O, LSE), float64: O has shape [B, H, Sq, D]; LSE has shape
    [B, H, Sq] (natural log).  Sq == Sk is the square case of the rest of the
    path; Sq != Sk serves the split-KV forward (same definition, see scores).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    bsz, nh, sq, _ = q.shape
    o = np.zeros((bsz, nh, sq, v.shape[-1]))
    lse = np.zeros((bsz, nh, sq))
    for b in range(bsz):
        for h in range(nh):
            p, lse[b, h] = softmax_rows(scores(q[b, h], k[b, h], scale, causal))
            o[b, h] = p @ v[b, h]
    return o, lse


def attention_bwd(q, k, v, do, scale: float, causal: bool):
    """Backward pass over [B, H, S, D] inputs by the chain rule, float64.

    Returns (dQ, dK, dV) for the loss whose gradient with respect to the
    attention output O is ``do``.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    do = _f64(do)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    bsz, nh = q.shape[:2]
    for b in range(bsz):
        for h in range(nh):
            p = attention_probs(q[b, h], k[b, h], scale, causal)
            dv[b, h] = p.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T
            delta = np.sum(p * dp, axis=1, keepdims=True)
            ds = p * (dp - delta)
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
    return dq, dk, dv


def attention_fwd_rows(q, k, v, scale: float, causal: bool, rows):
    """Forward output for selected rows only, float64.

    ``rows`` is an iterable of (b, h, i).  Rows of attention are independent
    of one another, so each is the full definition applied to one query
    (causal: keys j <= i + Sk - Sq, as in ``scores``).  Returns
    (O_rows [n, D], LSE_rows [n]) in the order of ``rows``.
    """
    rows = list(rows)
    off = k.shape[2] - q.shape[2]
    dv = v.shape[-1]
    o = np.zeros((len(rows), dv))
    lse = np.zeros(len(rows))
    by_head = {}
    for n, (b, h, i) in enumerate(rows):
        by_head.setdefault((b, h), []).append((n, i))
    for (b, h), items in by_head.items():
        kk = _f64(k[b, h])
        vv = _f64(v[b, h])
        for n, i in items:
            qi = _f64(q[b, h, i : i + 1])
            s = scale * (qi @ kk.T)
            if causal:
                s[:, i + off + 1 :] = -np.inf
            p, l = softmax_rows(s)
            o[n] = (p @ vv)[0]
            lse[n] = l[0]
    return o, lse


# ----------------------------------------------------------------------------
# float32 versions for long sequences (torch CPU matrix products)
# ----------------------------------------------------------------------------


def _rows_block_f32(q_blk, k, scale, causal, r0):
    """Scores and softmax of rows r0.. of one head in float32 (torch)."""
    import torch

    s = (q_blk @ k.T) * scale
    if causal:  # r0 is the row's position among the keys (see scores)
        nr, sk = s.shape
        i = torch.arange(r0, r0 + nr).unsqueeze(1)
        j = torch.arange(sk).unsqueeze(0)
        s = s.masked_fill(j > i, float("-inf"))
    m = s.max(dim=1, keepdim=True).values
    e = torch.exp(s - m)
    l = e.sum(dim=1, keepdim=True)
    p = e / l
    lse = (m + torch.log(l)).squeeze(1)
    return p, lse


def attention_fwd_f32(q, k, v, scale: float, causal: bool, heads=None, block_rows: int = 2048):
    """Forward pass in float32 on the CPU for [B, H, S, D] torch tensors.

    ``heads`` optionally restricts the work to a list of (b, h) pairs; the
    result then has shape [len(heads), S, D] / [len(heads), S].  Rows are
    processed ``block_rows`` at a time (each row of S and P still complete).
    """
    import torch

    bsz, nh, sq, _ = q.shape
    if heads is None:
        heads = [(b, h) for b in range(bsz) for h in range(nh)]
    o = torch.empty((len(heads), sq, v.shape[-1]), dtype=torch.float32)
    lse = torch.empty((len(heads), sq), dtype=torch.float32)
    for n, (b, h) in enumerate(heads):
        kk = k[b, h].to(torch.float32)
        vv = v[b, h].to(torch.float32)
        for r0 in range(0, sq, block_rows):
            qb = q[b, h, r0 : r0 + block_rows].to(torch.float32)
            p, l = _rows_block_f32(qb, kk, scale, causal, r0 + kk.shape[0] - sq)
            o[n, r0 : r0 + qb.shape[0]] = p @ vv
            lse[n, r0 : r0 + qb.shape[0]] = l
    return o, lse


def attention_bwd_f32(q, k, v, do, scale: float, causal: bool, heads=None, block_rows: int = 2048):
    """Backward pass in float32 on the CPU for [B, H, S, D] torch tensors.

    Same chain rule as ``attention_bwd``.  dQ rows of a block need only that
    block; dK and dV are sums over all query rows and are accumulated block by
    block.  Returns (dQ, dK, dV), each [len(heads), S, D].
    """
    import torch

    bsz, nh, sq, dd = q.shape
    if heads is None:
        heads = [(b, h) for b in range(bsz) for h in range(nh)]
    dq = torch.empty((len(heads), sq, dd), dtype=torch.float32)
    dk = torch.zeros((len(heads), k.shape[2], dd), dtype=torch.float32)
    dv = torch.zeros((len(heads), v.shape[2], v.shape[-1]), dtype=torch.float32)
    for n, (b, h) in enumerate(heads):
        kk = k[b, h].to(torch.float32)
        vv = v[b, h].to(torch.float32)
        for r0 in range(0, sq, block_rows):
            qb = q[b, h, r0 : r0 + block_rows].to(torch.float32)
            dob = do[b, h, r0 : r0 + block_rows].to(torch.float32)
            p, _ = _rows_block_f32(qb, kk, scale, causal, r0)
            dv[n] += p.T @ dob
            dp = dob @ vv.T
            delta = (p * dp).sum(dim=1, keepdim=True)
            ds = p * (dp - delta)
            dq[n, r0 : r0 + qb.shape[0]] = scale * (ds @ kk)
            dk[n] += scale * (ds.T @ qb)
    return dq, dk, dv


def exp2_exact(x) -> np.ndarray:
    """2**x in float64: the exact function the kernels' exponentials approximate."""
    return np.exp2(np.asarray(x, dtype=np.float64))
