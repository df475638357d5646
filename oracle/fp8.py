"""FP8 forward attention with incoherent processing, step by step on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): the GPU library must
never import or call this module.

What is computed, and where it comes from
-----------------------------------------
Page "FlashAttention-3 и FlashAttention-4", section "Поддержка FP8 с контролем
ошибок": attention in FP8, where Q and K first go through a cheap transform
that spreads outlier values over the coordinates, so that the FP8 rounding
error is smaller and less concentrated in single elements (the page reports
2.6 times less numerical error than a naive FP8 attention).

The page fixes none of the details.  The readings taken here:

* Transform: x -> (x * s) H / sqrt(D) on every row of Q and of K, with H the
  D x D Sylvester-Hadamard matrix and s a vector of random signs.  The matrix
  diag(s) H / sqrt(D) is orthogonal, so Q K^T is unchanged in exact
  arithmetic; only the rounding to FP8 sees the transform.  V is not
  transformed.
* Format: OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa
  bits; no infinities; the all-ones pattern of each sign is NaN; largest
  finite value 448).  Rounding to nearest, ties to the even code.  Values
  are clamped to [-448, 448] after scaling, so nothing reaches the NaN code.
* Scales (float): Q one per row, K one per tile of 64 keys, V one per
  column (element of the head dimension); each is max|x| / 448 over its
  group, or 1 when the group is all zero.  x ~= scale * e4m3(x / scale).
* Both products in FP8: S = Q8 K8^T and O += P8 V8.  P is rounded to E4M3
  without a scale: its values lie in (0, 1] relative to the running max.
* Online softmax over tiles of 64 keys with a per-row running max m:
  P~ = exp(S - m_new) per tile, rounded to E4M3 for the product with V; the
  accumulator and the row sum are multiplied by exp(m_old - m_new) when the
  max grows; the row sum adds the unrounded P~.  O = acc / l and
  LSE = m + ln l.

Because P is rounded relative to the running max of the tiles seen so far,
the result depends on the tile size; 64 keys is the tile of the GPU kernel.
Every step above is exact in float64 except the roundings it names.
"""

from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
TILE = 64


def e4m3_table() -> np.ndarray:
    """Value of each of the 256 E4M3 codes (float64; NaN for 0x7F and 0xFF).

    code = s eeee mmm: exponent field 0 encodes m/8 * 2^-6 (subnormal),
    fields 1..15 encode (1 + m/8) * 2^(e - 7); e = 15 with m = 7 is NaN.
    """
    out = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            out[c] = np.nan
        elif e == 0:
            out[c] = sign * (m / 8.0) * 2.0 ** -6
        else:
            out[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_TABLE = e4m3_table()
_POS = _TABLE[:0x7F]  # codes 0x00 .. 0x7E: the non-negative finite values, increasing


def quantize_e4m3(x) -> np.ndarray:
    """Round to E4M3 codes (uint8): clamp to +-448, nearest value, ties to the even code.

    A value that rounds to zero keeps its sign bit (0x80 for negative).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left")  # first code with value >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(x < 0, code | 0x80, code).astype(np.uint8)


def dequantize_e4m3(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def round_e4m3(x) -> np.ndarray:
    """x rounded to the nearest E4M3 value (clamped to +-448), as float64."""
    return dequantize_e4m3(quantize_e4m3(x))


def hadamard(d: int) -> np.ndarray:
    """Sylvester-Hadamard matrix of order d (a power of two): H_1 = [1], H_2n = [[H, H], [H, -H]]."""
    if d < 1 or d & (d - 1):
        raise ValueError("order must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate(x, signs) -> np.ndarray:
    """Rows of x times diag(signs) H / sqrt(D): the incoherent-processing transform."""
    x = np.asarray(x, dtype=np.float64)
    s = np.asarray(signs, dtype=np.float64)
    d = x.shape[-1]
    return (x * s) @ hadamard(d) / math.sqrt(d)


def _scale_of(amax):
    amax = np.asarray(amax, dtype=np.float64)
    return np.where(amax > 0, amax / E4M3_MAX, 1.0)


def _codes(x, amax):
    """E4M3 codes of x / (amax / 448), formed as x * 448 / amax: one rounding,
    so a value exactly halfway between two codes stays exactly halfway (and
    goes to the even code).  amax = 0 gives code 0."""
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    return quantize_e4m3(np.where(amax > 0, x * E4M3_MAX / safe, 0.0))


def quantize_rows(x, norm: float = 1.0):
    """One scale per row: codes [S, D] (uint8) and scales [S] of the rows x * norm."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max(axis=-1)
    return _codes(x, amax[:, None]), _scale_of(amax * norm)


def quantize_tiles(x, tile: int = TILE, norm: float = 1.0):
    """One scale per tile of `tile` rows (the last tile may be shorter): codes and scales
    [ceil(S / tile)] of the rows x * norm."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    nt = (n + tile - 1) // tile
    amax = np.array([np.abs(x[t * tile:(t + 1) * tile]).max() for t in range(nt)])
    codes = np.empty(x.shape, dtype=np.uint8)
    for t in range(nt):
        codes[t * tile:(t + 1) * tile] = _codes(x[t * tile:(t + 1) * tile], amax[t])
    return codes, _scale_of(amax * norm)


def quantize_cols(x):
    """One scale per column: codes [S, D] and scales [D]."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max(axis=0)
    return _codes(x, amax[None, :]), _scale_of(amax)


def quantize_head(q, k, v, signs=None, tile: int = TILE):
    """Transform (when signs are given) and quantize one head's Q, K, V.

    Returns dict with codes (q8, k8, v8) and scales (qs [S], ks [ceil(S/tile)],
    vs [D]) and the dequantized float64 matrices (qh, kh, vh).

    The codes of a transformed row y = (x * s) H / sqrt(D) are the rounding of
    y * 448 / max|y|, in which the factor 1 / sqrt(D) cancels; they are formed
    from (x * s) H, which is exact in float64 for bf16 inputs, so that no
    rounding of that factor can move a value that lies exactly halfway
    between two codes.  The scales carry the factor.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    norm = 1.0
    if signs is not None:
        d = q.shape[-1]
        h = hadamard(d)
        s_ = np.asarray(signs, dtype=np.float64)
        q = (q * s_) @ h
        k = (k * s_) @ h
        norm = 1.0 / math.sqrt(d)
    q8, qs = quantize_rows(q, norm)
    k8, ks = quantize_tiles(k, tile, norm)
    v8, vs = quantize_cols(v)
    kt = np.repeat(ks, tile)[: k.shape[0]]
    return {
        "q8": q8, "qs": qs, "k8": k8, "ks": ks, "v8": v8, "vs": vs,
        "qh": dequantize_e4m3(q8) * qs[:, None],
        "kh": dequantize_e4m3(k8) * kt[:, None],
        "vh": dequantize_e4m3(v8) * vs[None, :],
    }


def online_softmax_fwd(qh, kh, vh, scale: float, causal: bool, round_p=round_e4m3, tile: int = TILE,
                       q_rows=None):
    """Tiled online-softmax forward of one head on given (dequantized) operands.

    For each tile of `tile` keys: S = scale * Q K_t^T (causal: key j > query i
    is -inf), m_new = max(m, rowmax S), P~ = exp(S - m_new), acc = acc *
    exp(m - m_new) + round_p(P~) V_t, l = l * exp(m - m_new) + rowsum P~.
    Returns O = acc / l and LSE = m + ln l.  With round_p the identity this is
    exactly the softmax attention of the operands.  q_rows: the positions of
    the given query rows among all Sq queries (for the causal mask), when qh
    holds only some rows; the default is all of them in order.
    """
    qh = np.asarray(qh, dtype=np.float64)
    kh = np.asarray(kh, dtype=np.float64)
    vh = np.asarray(vh, dtype=np.float64)
    n, sk = qh.shape[0], kh.shape[0]
    sq = n if q_rows is None else None
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    acc = np.zeros((n, vh.shape[1]))
    i = (np.arange(n) if q_rows is None else np.asarray(q_rows))[:, None]
    for t0 in range(0, sk, tile):
        s = scale * (qh @ kh[t0:t0 + tile].T)
        if causal:
            if sq is None:  # rows of a square problem
                sq = sk
            j = np.arange(t0, min(sk, t0 + tile))[None, :]
            s = np.where(j > i + (sk - sq), -np.inf, s)
        m_new = np.maximum(m, s.max(axis=1))
        # rows with every key so far masked keep m = -inf and contribute nothing
        live = np.isfinite(m_new)
        alpha = np.where(live & np.isfinite(m), np.exp(np.where(live, m - m_new, 0.0)), 0.0)
        p = np.where(live[:, None], np.exp(s - np.where(live, m_new, 0.0)[:, None]), 0.0)
        acc = acc * alpha[:, None] + round_p(p) @ vh[t0:t0 + tile]
        l = l * alpha + p.sum(axis=1)
        m = m_new
    o = acc / l[:, None]
    lse = m + np.log(l)
    return o, lse


def fp8_attention_fwd(q, k, v, scale: float, causal: bool, signs=None, tile: int = TILE, rows=None):
    """FP8 forward of one head ([S, D] each): transform, quantize, online softmax with P in E4M3.

    rows: compute only these query rows (of a square problem); Q is quantized
    per row, so the result is the same as those rows of the full call.
    """
    qd = quantize_head(q, k, v, signs, tile)
    qh = qd["qh"] if rows is None else qd["qh"][np.asarray(rows)]
    return online_softmax_fwd(qh, qd["kh"], qd["vh"], scale, causal, round_e4m3, tile, rows)


def fp8_attention_fwd_heads(q, k, v, scale: float, causal: bool, signs=None, heads=None, tile: int = TILE):
    """fp8_attention_fwd over [B, H, S, D] arrays (float64 results); `heads` picks (b, h) pairs."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, S, D = q.shape
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    o = np.zeros((len(heads), S, D))
    lse = np.zeros((len(heads), S))
    for n, (b, h) in enumerate(heads):
        o[n], lse[n] = fp8_attention_fwd(q[b, h], k[b, h], v[b, h], scale, causal, signs, tile)
    return o, lse
