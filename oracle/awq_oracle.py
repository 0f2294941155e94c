"""Plain, slow CPU oracle for the AWQ W4A16 hot path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this module. The product path (the C-ABI library
and its Python binding) never calls it; it shares no code, header, table or
helper with the HIP implementation.

What it computes, step by step, in the pages' own order (calibration ->
activation statistic -> per-channel scale s = s_X^alpha -> quantize W*diag(s)
with group-wise round-to-nearest -> pack -> the W4A16 product with the
folded activation X*diag(s)^-1):

* Equivalence transform: W' = W diag(s), X' = diag(s)^-1 X, so W'X' = WX
  before quantization (hungho77 blog "AWQ explained" -- "Scaling instead of
  mixed precision"; AWQ Explained: Protecting the Weights That Matter Most --
  "Scaling instead of mixed precision").
* Scale parameterisation and search: s_j = mean_t |x_tj| ** alpha, alpha
  grid-searched in [0, 1] to minimise || W x - Q(W diag(s)) diag(s)^-1 x || on
  the calibration batch (AWQ Explained -- "How the scale is chosen"; hungho77
  blog -- "Scaling instead of mixed precision").
* Quantizer: plain round-to-nearest (ai360xpert "AWQ" -- "How It Works",
  step 4), group-wise, 3 or 4 bits, groups of 128 (Real Python glossary
  "activation-aware weight quantization (AWQ)"), asymmetric grid with an
  integer zero point, defaults bits=4 / group 128 / zero_point=true
  (AWQ Explained -- "How the scale is chosen", last paragraph); the grid step
  is the group's range divided by the number of levels and the rounding error
  is about half a step (AWQ Explained -- "Scaling instead of mixed precision").

Precision: the quantizer runs in float32 with single IEEE roundings
(multiply, subtract, divide) and round-half-to-even, exactly as the
hot path is required to; statistics, losses and the matmul run in float64.

Readings taken where the pages are silent or garbled (each one is also
listed in the design notes):

R1  s_X is the mean of |x| over calibration tokens (not RMS, not max).
R2  a channel whose statistic is exactly 0 gets s = 1 for every alpha.
R3  s = float32(pow(m, alpha)) with pow evaluated in double precision.
R3b s is not normalised.
R4  "number of levels" is read as the number of steps 2^b - 1, so that both
    ends of the range are on the grid.
R4b the range always contains 0: lo = min(0, min W'), hi = max(0, max W').
R5  q = clamp(rint(W' / delta) + z, 0, 2^b - 1), z = rint(-lo / delta): the
    zero point is an integer added after rounding.
R6  round-half-to-even everywhere; an all-zero group gets delta = 1, z = 0.
R7  the layer-output error is the squared Frobenius norm over calibration
    tokens and output channels, evaluated in exact (float64) arithmetic with
    the original fp16 W; the first minimum over the grid wins.
R9  packing: see ``code_position``.
R10 scales are stored as the float32 delta, zero points as uint8.
R18 the gated MLP that the fused gate/up product serves is LLaMA's:
    Y = silu(X' Wg^T) * (X' Wu^T), silu(v) = v / (1 + e^-v); the pages credit
    operator fusion for the speed-up (hungho77 blog -- "Why the engine is
    part of the method") but name no activation. Gate and up read the same
    normalized input, so they share one X' (one s). Evaluated here in
    float64 from the exact products.
R20 the fold of diag(s)^-1 into the normalization that precedes the layer
    (AWQ Explained -- "Scaling instead of mixed precision": it is done
    offline and what ships is a modified norm) is read for RMSNorm,
    y_k = x_k * r * gamma_k with r = (mean_k x_k^2 + eps)^-1/2: the folded
    weight is gamma'_k = fp16(float32(gamma_k) / s_k) (the weight keeps its
    fp16 storage, one rounding) and the norm with gamma' yields X' directly.
    Here r and the product are exact (float64) and rounded once to fp16.
R21 one norm carries one s, so layers that read the same normalized input
    (q/k/v; gate/up) share s, and its search minimizes the sum of their
    layer-output errors, summed in layer order; the first minimum wins.
R23 the ablations the pages report as perplexities are reported here as the
    layer-output error of R7 (no model or corpus exists here): keeping the
    salient fraction (1%, AWQ Explained -- "The premise: 1% of channels") of
    input channels in FP16 means quantizing W as usual and restoring those
    columns to their FP16 values; salient by activation is the largest
    mean |x| (the statistic of R1), by weight the largest mean |W| over the
    column's output channels; ties go to the lower channel index.
R24 compact storage of the group parameters (an AwqConfig storage variant):
    the step as fp16 (one rounding of the float32 delta) and the zero points
    as 4-bit fields, 8 per uint32 word in group order (group g of a row in
    word g // 8, bits 4 (g % 8)), each row padded to whole words. Every zero
    point fits 4 bits (at most 2^b - 1 <= 15). The product then dequantizes
    with the fp16 step: (q - z) * float(fp16(delta)).
R17 zero_point=false (the AwqConfig option, AWQ Explained -- "How the scale
    is chosen", last paragraph) is the symmetric grid: delta = max|W'| /
    (2^(b-1) - 1) per group, codes rint(W' / delta) in [-(2^(b-1) - 1),
    2^(b-1) - 1] stored with the offset z = 2^(b-1) (so the packed layout and
    the product are unchanged); an all-zero group gets delta = 1.
"""
from __future__ import annotations

import math

import numpy as np

# ----------------------------------------------------------------------------
# calibration statistic and scale candidates
# ----------------------------------------------------------------------------


def act_stats(xcal: np.ndarray) -> np.ndarray:
    """m_j = (1/T) * sum_t |x_tj| in float64 (R1).

    fp16 values are integer multiples of 2^-24 below 2^16, so for T < 8192
    the float64 sum is exact and independent of summation order; the only
    rounding is the final division by T.
    """
    x = np.abs(np.asarray(xcal, dtype=np.float16).astype(np.float64))
    return x.sum(axis=0) / x.shape[0]


def scale_from_stats(m: np.ndarray, alpha) -> np.ndarray:
    """s_j = float32(pow(m_j, alpha)) (R2, R3). alpha is taken as float32."""
    a = float(np.float32(alpha))
    out = np.empty(len(m), dtype=np.float32)
    for j, mj in enumerate(np.asarray(m, dtype=np.float64)):
        out[j] = np.float32(math.pow(float(mj), a)) if mj > 0.0 else np.float32(1.0)
    return out


# ----------------------------------------------------------------------------
# group-wise asymmetric round-to-nearest
# ----------------------------------------------------------------------------


def scaled_weight(W: np.ndarray, s) -> np.ndarray:
    """W' = W diag(s) as float32: one float32 multiply per element.

    s scales input channels, i.e. the columns of W [N, K] (p3/p4 "Scaling
    instead of mixed precision"). s = None means s = 1 (plain RTN).
    """
    w = np.asarray(W, dtype=np.float16).astype(np.float32)
    if s is None:
        return w
    s = np.asarray(s, dtype=np.float32)
    assert s.shape == (w.shape[1],)
    return (w * s[None, :]).astype(np.float32)


def quantize_groups(wp: np.ndarray, bits: int, group: int):
    """RTN quantization of float32 W' [N, K] in groups of `group` along K.

    Returns (q int64 [N, K], delta float32 [N, K/group], z int64 [N, K/group]).
    """
    wp = np.asarray(wp, dtype=np.float32)
    N, K = wp.shape
    assert K % group == 0
    qmax = (1 << bits) - 1
    g = wp.reshape(N, K // group, group)
    lo = np.minimum(g.min(axis=2), np.float32(0.0))          # R4b
    hi = np.maximum(g.max(axis=2), np.float32(0.0))
    r = (hi - lo).astype(np.float32)
    flat = r == 0                                            # all-zero group (R6)
    safe_r = np.where(flat, np.float32(1.0), r).astype(np.float32)
    delta = (safe_r / np.float32(qmax)).astype(np.float32)   # R4: range / (2^b - 1)
    delta = np.where(flat, np.float32(1.0), delta).astype(np.float32)
    z = np.rint((-lo / delta).astype(np.float32)).astype(np.int64)
    z = np.where(flat, 0, z)
    q = np.rint((g / delta[..., None]).astype(np.float32)).astype(np.int64) + z[..., None]
    q = np.clip(q, 0, qmax)                                  # R5
    return q.reshape(N, K), delta, z


def quantize_groups_symmetric(wp: np.ndarray, bits: int, group: int):
    """Symmetric RTN (R17) of float32 W' [N, K] in groups of `group` along K.

    Returns (q int64 [N, K] with the offset 2^(b-1) added, delta float32
    [N, K/group], z int64 [N, K/group] = 2^(b-1)).
    """
    wp = np.asarray(wp, dtype=np.float32)
    N, K = wp.shape
    assert K % group == 0
    half = 1 << (bits - 1)
    g = wp.reshape(N, K // group, group)
    amax = np.abs(g).max(axis=2).astype(np.float32)
    flat = amax == 0
    safe = np.where(flat, np.float32(1.0), amax).astype(np.float32)
    delta = (safe / np.float32(half - 1)).astype(np.float32)
    delta = np.where(flat, np.float32(1.0), delta).astype(np.float32)
    z = np.full(delta.shape, half, dtype=np.int64)
    q = np.rint((g / delta[..., None]).astype(np.float32)).astype(np.int64) + half
    q = np.clip(q, 0, (1 << bits) - 1)
    return q.reshape(N, K), delta, z


def quantize(W: np.ndarray, s, bits: int, group: int, zero_point: bool = True):
    """(q, scales fp32 [N, K/G], zeros uint8 [N, K/G]) of W diag(s)."""
    qg = quantize_groups if zero_point else quantize_groups_symmetric
    q, delta, z = qg(scaled_weight(W, s), bits, group)
    return q, delta.astype(np.float32), z.astype(np.uint8)


def dequantize(q: np.ndarray, scales: np.ndarray, zeros: np.ndarray, group: int) -> np.ndarray:
    """(q - z) * delta, exact in float64 [N, K]."""
    N, K = q.shape
    qq = q.reshape(N, K // group, group).astype(np.int64) - zeros.astype(np.int64)[..., None]
    return (qq.astype(np.float64) * scales.astype(np.float64)[..., None]).reshape(N, K)


# ----------------------------------------------------------------------------
# packing (R9)
# ----------------------------------------------------------------------------


def words_per_group(bits: int, group: int) -> int:
    """int4: 8 codes per 32-bit word; int3: 10 codes per word (bits 30-31
    unused) in blocks of 128 codes, 13 words per block (the last word holds
    8 codes). Groups are multiples of 128 codes."""
    if bits == 4:
        assert group % 8 == 0
        return group // 8
    if bits == 3:
        assert group % 128 == 0
        return 13 * (group // 128)
    raise ValueError("bits must be 3 or 4")


def words_per_row(K: int, bits: int, group: int) -> int:
    """Groups are stored back to back; the row is padded with zero words to
    a multiple of 4 words (16 bytes)."""
    assert K % group == 0
    w = (K // group) * words_per_group(bits, group)
    return -(-w // 4) * 4


def code_position(k, bits: int):
    """(word, bit offset) of the code at position k of a row (R9).

    int4: word k // 8, bits 4 (k % 8). int3: the row is cut into blocks of
    128 codes, each starting on a word boundary and taking 13 words; inside
    a block the code at j = k % 128 sits in word j // 10 at bits 3 (j % 10).
    The layout does not depend on the group size (groups are whole blocks).
    """
    k = np.asarray(k)
    if bits == 4:
        return k // 8, 4 * (k % 8)
    j = k % 128
    return 13 * (k // 128) + j // 10, 3 * (j % 10)


def pack(q: np.ndarray, bits: int, group: int) -> np.ndarray:
    """Pack codes q [N, K] into uint32 [N, words_per_row] at the positions
    of ``code_position``. Unused slots, the two top bits of an int3 word and
    the row padding are zero."""
    N, K = q.shape
    out = np.zeros((N, words_per_row(K, bits, group)), dtype=np.uint64)
    word, shift = code_position(np.arange(K), bits)
    qq = q.astype(np.uint64)
    for k in range(K):
        out[:, word[k]] |= qq[:, k] << np.uint64(shift[k])
    return out.astype(np.uint32)


def unpack(qpacked: np.ndarray, bits: int, group: int, K: int) -> np.ndarray:
    N = qpacked.shape[0]
    mask = np.uint64((1 << bits) - 1)
    w = qpacked.astype(np.uint64)
    word, shift = code_position(np.arange(K), bits)
    q = np.empty((N, K), dtype=np.int64)
    for k in range(K):
        q[:, k] = ((w[:, word[k]] >> np.uint64(shift[k])) & mask).astype(np.int64)
    return q


def quantize_pack(W: np.ndarray, s, bits: int, group: int, zero_point: bool = True):
    """The quantize-and-pack step: (qpacked uint32, scales fp32, zeros uint8)."""
    q, scales, zeros = quantize(W, s, bits, group, zero_point)
    return pack(q, bits, group), scales, zeros


# ----------------------------------------------------------------------------
# folding diag(s)^-1 into the activation, and the W4A16 product
# ----------------------------------------------------------------------------


def fold_inv_scale(X: np.ndarray, s: np.ndarray) -> np.ndarray:
    """X' = fp16(float32(X) / s): one float32 division, then one rounding to
    fp16 (AWQ Explained -- "Scaling instead of mixed precision": the
    activation channel is divided by the same s)."""
    x = np.asarray(X, dtype=np.float16).astype(np.float32)
    return (x / np.asarray(s, dtype=np.float32)[None, :]).astype(np.float32).astype(np.float16)


def matmul(Xp: np.ndarray, qpacked: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
           bits: int, group: int, K: int) -> np.ndarray:
    """Y = X' dequant(Q)^T in float64 [M, N]; X' is the fp16 activation."""
    Wd = dequantize(unpack(qpacked, bits, group, K), scales, zeros, group)
    return np.asarray(Xp, dtype=np.float16).astype(np.float64) @ Wd.T


def matmul_rows(Xp, qpacked, scales, zeros, bits, group, K, rows) -> np.ndarray:
    """Y[:, rows] only (for sampled checks at large N)."""
    rows = np.asarray(rows)
    return matmul(Xp, qpacked[rows], scales[rows], zeros[rows], bits, group, K)


def silu(v) -> np.ndarray:
    """silu(v) = v * sigmoid(v) = v / (1 + exp(-v)) in float64 (R18). For
    v below about -709, exp(-v) overflows to inf and the quotient is -0,
    the limit."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def gate_up_silu(Xp, qg, sg, zg, qu, su, zu, bits: int, group: int, K: int) -> np.ndarray:
    """Y = silu(X' Wg^T) * (X' Wu^T) in float64 [M, N] (R18): the gate and
    up projections of a gated MLP on one activation, then the elementwise
    product."""
    G = matmul(Xp, qg, sg, zg, bits, group, K)
    U = matmul(Xp, qu, su, zu, bits, group, K)
    return silu(G) * U


# ----------------------------------------------------------------------------
# layer-output loss and the alpha grid search
# ----------------------------------------------------------------------------


def quant_error(W: np.ndarray, s: np.ndarray, bits: int, group: int,
                zero_point: bool = True) -> np.ndarray:
    """D = W - Q(W diag(s)) diag(s)^-1 in float64 [N, K]."""
    q, scales, zeros = quantize(W, s, bits, group, zero_point)
    what = dequantize(q, scales, zeros, group)
    return np.asarray(W, dtype=np.float16).astype(np.float64) - what / np.asarray(s, np.float64)[None, :]


def layer_loss(xcal: np.ndarray, W: np.ndarray, s: np.ndarray, bits: int, group: int,
               zero_point: bool = True) -> float:
    """L = || Xcal D^T ||_F^2 (R7): the layer-output error on the calibration
    batch, sum over tokens t and output channels n of
    (sum_k x_tk (W_nk - Wq_nk / s_k))^2."""
    D = quant_error(W, s, bits, group, zero_point)
    E = np.asarray(xcal, dtype=np.float16).astype(np.float64) @ D.T
    return float(np.sum(E * E))


def scale_search(W: np.ndarray, xcal: np.ndarray, alpha_grid, bits: int, group: int,
                 zero_point: bool = True):
    """Grid search over alpha; returns (s float32 [K], best index, losses float64).

    The grid is scanned in the given order with a strict '<', so the first
    minimum wins (R7).
    """
    m = act_stats(xcal)
    losses = np.empty(len(alpha_grid), dtype=np.float64)
    best = 0
    for i, a in enumerate(alpha_grid):
        losses[i] = layer_loss(xcal, W, scale_from_stats(m, a), bits, group, zero_point)
        if losses[i] < losses[best]:
            best = i
    return scale_from_stats(m, alpha_grid[best]), best, losses


# ----------------------------------------------------------------------------
# the scale folded into the preceding RMSNorm, and the joint search of
# layers that share it
# ----------------------------------------------------------------------------


def fold_norm_weight(gamma: np.ndarray, s: np.ndarray) -> np.ndarray:
    """gamma' = fp16(float32(gamma) / s): the RMSNorm weight with diag(s)^-1
    folded in (R20), one float32 division and one rounding to fp16."""
    g = np.asarray(gamma, dtype=np.float16).astype(np.float32)
    return (g / np.asarray(s, dtype=np.float32)).astype(np.float32).astype(np.float16)


def rmsnorm(X: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """fp16(x_k * r * gamma_k), r = (mean_k x_k^2 + eps)^-1/2, per row of the
    fp16 X [M, K] with the fp16 weight gamma [K]; r and the product in
    float64, one rounding to fp16 (R20)."""
    x = np.asarray(X, dtype=np.float16).astype(np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + float(eps))
    g = np.asarray(gamma, dtype=np.float16).astype(np.float64)
    return (x * r * g[None, :]).astype(np.float16)


def joint_scale_search(Ws, xcal: np.ndarray, alpha_grid, bits: int, group: int,
                       zero_point: bool = True):
    """One s for the layers Ws (each [N_l, K]) that read the same input
    (R21): losses[i] = sum over layers, in order, of layer_loss at s_i; the
    first minimum wins. Returns (s float32 [K], best index, losses)."""
    m = act_stats(xcal)
    losses = np.empty(len(alpha_grid), dtype=np.float64)
    best = 0
    for i, a in enumerate(alpha_grid):
        s = scale_from_stats(m, a)
        total = 0.0
        for W in Ws:
            total += layer_loss(xcal, W, s, bits, group, zero_point)
        losses[i] = total
        if losses[i] < losses[best]:
            best = i
    return scale_from_stats(m, alpha_grid[best]), best, losses


# ----------------------------------------------------------------------------
# ablations (R23): FP16-kept salient channels against scaling
# ----------------------------------------------------------------------------


def weight_channel_magnitude(W: np.ndarray) -> np.ndarray:
    """mean_n |W[n, k]| per input channel k, in float64 (exact sums)."""
    return np.abs(np.asarray(W, dtype=np.float16).astype(np.float64)).mean(axis=0)


def salient_channels(score: np.ndarray, count: int) -> np.ndarray:
    """Indices of the `count` largest scores, ties to the lower index, in
    increasing order."""
    score = np.asarray(score, dtype=np.float64)
    order = sorted(range(len(score)), key=lambda k: (-score[k], k))
    return np.sort(np.asarray(order[:count], dtype=np.int64))


def layer_loss_fp16_kept(xcal: np.ndarray, W: np.ndarray, channels, bits: int, group: int,
                         zero_point: bool = True) -> float:
    """R7's loss with plain RTN (s = 1) except that the input channels
    `channels` keep their FP16 weights: D = W - Wq with those columns of Wq
    replaced by W's."""
    q, scales, zeros = quantize(W, None, bits, group, zero_point)
    what = dequantize(q, scales, zeros, group)
    w = np.asarray(W, dtype=np.float16).astype(np.float64)
    ch = np.asarray(channels, dtype=np.int64)
    what[:, ch] = w[:, ch]
    E = np.asarray(xcal, dtype=np.float16).astype(np.float64) @ (w - what).T
    return float(np.sum(E * E))


# ----------------------------------------------------------------------------
# compact storage of the group parameters (R24)
# ----------------------------------------------------------------------------


def compact_group_params(scales: np.ndarray, zeros: np.ndarray):
    """(fp16 steps [N, ng], uint32 packed zero points [N, ceil(ng / 8)])."""
    sc = np.asarray(scales, dtype=np.float32)
    z = np.asarray(zeros, dtype=np.uint8)
    assert np.all(z <= 15)
    N, ng = z.shape
    zw = np.zeros((N, -(-ng // 8)), dtype=np.uint64)
    for g in range(ng):
        zw[:, g // 8] |= z[:, g].astype(np.uint64) << np.uint64(4 * (g % 8))
    return sc.astype(np.float16), zw.astype(np.uint32)


def expand_group_params(scales16: np.ndarray, zeros4: np.ndarray, ng: int):
    """Inverse of the packing: (float32 steps as stored, uint8 zero points)."""
    N = scales16.shape[0]
    z = np.empty((N, ng), dtype=np.uint8)
    w = zeros4.astype(np.uint64)
    for g in range(ng):
        z[:, g] = ((w[:, g // 8] >> np.uint64(4 * (g % 8))) & np.uint64(15)).astype(np.uint8)
    return np.asarray(scales16, dtype=np.float16).astype(np.float32), z


def matmul_compact(Xp, qpacked, scales16, zeros4, bits: int, group: int, K: int) -> np.ndarray:
    """The W4A16 product with compactly stored group parameters (R24)."""
    sc, z = expand_group_params(scales16, zeros4, K // group)
    return matmul(Xp, qpacked, sc, z, bits, group, K)
