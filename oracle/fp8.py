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

The page fixes none of the details.  The readings taken here, in the page's
order (transform, then quantize, then attention):

* Transform: x -> (x * s) H / sqrt(D) on every row of Q and of K, with H the
  D x D Sylvester-Hadamard matrix and s a vector of random signs.  The matrix
  diag(s) H / sqrt(D) is orthogonal, so Q K^T is unchanged in exact
  arithmetic; only the rounding to FP8 sees the transform.  V is not
  transformed.
* Format: OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa
  bits; no infinities; the all-ones pattern of each sign is NaN; largest
  finite value 448).  Rounding to nearest, ties to the even code.
* Scales (float): Q one per row, K one per (batch, head), V one per column
  (element of the head dimension); each is max|x| / 448 over its group, or 1
  when the group is all zero.  x ~= scale * e4m3(x / scale).  None of these
  groups depends on how a kernel tiles the sequence.  The code of x is the
  rounding of the float64 quotient x * 448 / max|x| (one correctly rounded
  division of an exact numerator), straight to E4M3.
* Attention (fp8_reference_fwd): S = scale * Q8 K8^T on the dequantized
  operands, m = the row max, P~ = exp(S - m) in (0, 1], O = E4M3(P~) V8 / l
  with l the row sum of the unrounded P~, LSE = m + ln l.  P is rounded to
  E4M3 without a scale, relative to the row's final max.

A kernel that walks the keys in tiles rounds P~ against the running max
instead: relative to a max that may still lag the final one, so on a grid
that is finer in absolute terms, tile by tile.  p_rounding_bound gives, per
output element, a bound that one rounding of P keeps to, whether against the
final max or against any running max not above it (any tiling, any
conditional-rescale threshold up to 8); two such results differ by at most
twice it.  online_softmax_fwd is the tiled form
of the same attention for a given tile size, rounding P per tile against the
running max (an emulation of that schedule, used as a second, tighter check).
Every step is exact in float64 except the roundings it names.
"""

from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


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
    """E4M3 codes of x / (amax / 448), formed as the float64 quotient
    (x * 448) / amax (the numerator is exact for the inputs here, the division
    is correctly rounded) and rounded from float64 straight to E4M3: a value
    exactly halfway between two codes stays exactly halfway (and goes to the
    even code).  amax = 0 gives code 0."""
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    return quantize_e4m3(np.where(amax > 0, (x * E4M3_MAX) / safe, 0.0))


def quantize_rows(x, norm: float = 1.0):
    """One scale per row: codes [S, D] (uint8) and scales [S] of the rows x * norm."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max(axis=-1)
    return _codes(x, amax[:, None]), _scale_of(amax * norm)


def quantize_whole(x, norm: float = 1.0):
    """One scale for the whole matrix: codes [S, D] and a scale (0-d array) of x * norm."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max()
    return _codes(x, amax), _scale_of(amax * norm)


def quantize_cols(x):
    """One scale per column: codes [S, D] and scales [D]."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max(axis=0)
    return _codes(x, amax[None, :]), _scale_of(amax)


def quantize_head(q, k, v, signs=None):
    """Transform (when signs are given) and quantize one head's Q, K, V.

    Returns dict with codes (q8, k8, v8), scales (qs [S], ks (one, for the
    head), vs [D]) and the dequantized float64 matrices (qh, kh, vh).

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
    k8, ks = quantize_whole(k, norm)
    v8, vs = quantize_cols(v)
    return {
        "q8": q8, "qs": qs, "k8": k8, "ks": ks, "v8": v8, "vs": vs,
        "qh": dequantize_e4m3(q8) * qs[:, None],
        "kh": dequantize_e4m3(k8) * ks,
        "vh": dequantize_e4m3(v8) * vs[None, :],
    }


def _causal_mask(n, sk, q_rows):
    """True where key j is hidden from query row i (queries are the last rows of sk positions)."""
    i = (np.arange(n) if q_rows is None else np.asarray(q_rows))[:, None]
    sq = n if q_rows is None else sk
    return np.arange(sk)[None, :] > i + (sk - sq)


def fp8_reference_fwd(qh, kh, vh, scale: float, causal: bool, round_p=None, q_rows=None):
    """Attention of one head on given (dequantized) operands with P rounded to
    E4M3 against each row's final max; no tiling.

    S = scale * Q K^T (causal: key j > query i is -inf), m = rowmax S,
    P~ = exp(S - m), O = round_p(P~) V / rowsum(P~), LSE = m + ln rowsum(P~).
    round_p defaults to round_e4m3; with the identity it is the softmax
    attention of the operands.  q_rows: the positions of the given query rows
    in a square problem (for the causal mask) when qh holds only some rows.
    Returns O, LSE and the unrounded P~ (for p_rounding_bound).
    """
    rp = round_e4m3 if round_p is None else round_p
    qh = np.asarray(qh, dtype=np.float64)
    kh = np.asarray(kh, dtype=np.float64)
    vh = np.asarray(vh, dtype=np.float64)
    s = scale * (qh @ kh.T)
    if causal:
        s = np.where(_causal_mask(qh.shape[0], kh.shape[0], q_rows), -np.inf, s)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    o = (rp(p) @ vh) / l[:, None]
    return o, m + np.log(l), p


def e4m3_error_bound(x) -> np.ndarray:
    """Largest |E4M3(x) - x| for 0 <= x <= 448: half a unit in the last place,
    2^-4 x for normal values (x >= 2^-6), 2^-10 below, and never more than x
    itself (a value under 2^-10 rounds to zero)."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(2.0 ** -4 * x, np.minimum(x, 2.0 ** -10))


def p_rounding_bound(p, vh) -> np.ndarray:
    """Per-element bound on how far rounding P to E4M3 moves O, for P~ = p
    (rows relative to their final max, values in (0, 1]) and operand V = vh:
        B_id = sum_j e(p_ij) |v_jd| / sum_j p_ij,   e = e4m3_error_bound.
    It holds for the rounding against the final max (fp8_reference_fwd) and,
    as well, for a rounding against any running max m_t <= m of a tiled
    kernel whose unnormalised probabilities stay at most 2^8 (no clamping at
    448): there the term c e4m3(p / c), c = exp(m_t - m) <= 1, is off from p
    by at most c e(p / c) <= max(2^-4 p, min(p, 2^-10 c)) <= e(p).  So two
    such results differ by at most 2 B."""
    p = np.asarray(p, dtype=np.float64)
    l = p.sum(axis=1)
    return (e4m3_error_bound(p) @ np.abs(np.asarray(vh, dtype=np.float64))) / l[:, None]


def online_softmax_fwd(qh, kh, vh, scale: float, causal: bool, round_p, tile: int, q_rows=None):
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
    mask = _causal_mask(n, sk, q_rows) if causal else None
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    acc = np.zeros((n, vh.shape[1]))
    for t0 in range(0, sk, tile):
        s = scale * (qh @ kh[t0:t0 + tile].T)
        if causal:
            s = np.where(mask[:, t0:t0 + tile], -np.inf, s)
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


def fp8_attention_fwd(q, k, v, scale: float, causal: bool, signs=None, rows=None, tile=None):
    """FP8 forward of one head ([S, D] each): transform, quantize, attention with P in E4M3.

    tile None: fp8_reference_fwd (P rounded against each row's final max, no
    tiling); an int: online_softmax_fwd over tiles of that many keys (P
    rounded per tile against the running max).  rows: compute only these
    query rows (of a square problem); Q is quantized per row, so the result is
    the same as those rows of the full call.  Returns O and LSE.
    """
    qd = quantize_head(q, k, v, signs)
    qh = qd["qh"] if rows is None else qd["qh"][np.asarray(rows)]
    if tile is None:
        o, lse, _ = fp8_reference_fwd(qh, qd["kh"], qd["vh"], scale, causal, q_rows=rows)
        return o, lse
    return online_softmax_fwd(qh, qd["kh"], qd["vh"], scale, causal, round_e4m3, tile, rows)


def fp8_attention_fwd_heads(q, k, v, scale: float, causal: bool, signs=None, heads=None, tile=None):
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
        o[n], lse[n] = fp8_attention_fwd(q[b, h], k[b, h], v[b, h], scale, causal, signs, tile=tile)
    return o, lse
