"""Pins that tie the CPU oracle to what the pages and the mathematics fix.

None of these re-types an oracle formula: each checks the oracle against a
closed form, a hand-derived fixture, an invariant, a textbook routine or
exact-rational brute force, chosen so that a plausible slip (a dropped term,
a wrong axis, a wrong rounding mode, a swapped operand) fails one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

import datagen
from oracle import awq_oracle as O
from tests.conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# P1: exactly representable groups (closed form, tests/golden/exact_groups.json)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", _golden("exact_groups.json")["cases"])
def test_exact_group(case):
    bits, G, L = case["bits"], case["group"], case["levels"]
    i = np.arange(G) % L
    v = ((i - case["num_offset"]) / case["den"]).astype(np.float16)
    W = np.stack([v, v[::-1]])  # second row: same values, reversed order
    q, scales, zeros = O.quantize(W, None, bits, G)
    assert scales.dtype == np.float32 and zeros.dtype == np.uint8
    assert np.all(scales == np.float32(case["delta"]))
    assert np.all(zeros == case["zero"])
    assert np.array_equal(q[0], i)
    assert np.array_equal(q[1], i[::-1])
    assert np.array_equal(O.dequantize(q, scales, zeros, G), W.astype(np.float64))


# ---------------------------------------------------------------------------
# P2/P3: half-step error bound and code ranges (hypothesis over awkward groups)
# ---------------------------------------------------------------------------

_f16 = st.floats(min_value=-8.0, max_value=8.0, allow_nan=False, width=16)


def _group_strategy():
    plain = st.lists(_f16, min_size=128, max_size=128)
    positive = st.lists(st.floats(0.0, 4.0, width=16), min_size=128, max_size=128)
    negative = st.lists(st.floats(-4.0, 0.0, width=16), min_size=128, max_size=128)
    # values on half-steps of a power-of-two grid: exact ties for rint
    ties = st.lists(st.integers(-16, 16), min_size=128, max_size=128).map(
        lambda xs: [x / 32.0 + 1.0 / 64.0 for x in xs])
    zeros = st.just([0.0] * 128)
    spike = st.tuples(st.integers(0, 127), st.floats(-1000, 1000, width=16)).map(
        lambda t: [t[1] if j == t[0] else 0.001 * (j % 7 - 3) for j in range(128)])
    return st.one_of(plain, positive, negative, ties, zeros, spike)


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(vals=_group_strategy(), bits=st.sampled_from([3, 4]),
       scale_exp=st.integers(-3, 3))
def test_half_step_bound_and_ranges(vals, bits, scale_exp):
    W = np.array(vals, dtype=np.float16)[None, :]
    s = np.full(128, np.float32(1.5 * 2.0 ** scale_exp), dtype=np.float32)
    wp = O.scaled_weight(W, s)
    q, scales, zeros = O.quantize(W, s, bits, 128)
    qmax = (1 << bits) - 1
    assert q.min() >= 0 and q.max() <= qmax
    assert int(zeros[0, 0]) <= qmax
    d = float(scales[0, 0])
    err = np.abs(O.dequantize(q, scales, zeros, 128)[0] - wp[0].astype(np.float64))
    assert err.max() <= d * (0.5 + 1e-5), (err.max() / d)
    lo = min(0.0, float(wp.min()))
    if lo < 0:  # the most negative entry lands on code 0 (round-half-even is odd-symmetric)
        assert q[0, int(np.argmin(wp[0]))] == 0
    if np.all(W == 0):
        assert d == 1.0 and zeros[0, 0] == 0 and np.all(q == 0)


def test_range_always_contains_zero():
    # a single-signed group still gets z in range and the half-step bound
    W = np.linspace(0.5, 1.0, 128).astype(np.float16)[None, :]
    q, sc, z = O.quantize(W, None, 4, 128)
    assert z[0, 0] == 0 and sc[0, 0] == np.float32(np.float32(W.max()) / np.float32(15))
    W2 = -W
    q2, sc2, z2 = O.quantize(W2, None, 4, 128)
    assert z2[0, 0] == 15 and np.array_equal(q2[0], 15 - q[0])


# ---------------------------------------------------------------------------
# P4: power-of-two equivariance of s (exact-arithmetic invariance)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("j", [-4, 1, 3])
def test_power_of_two_equivariance(bits, j):
    W = datagen.random_f16((8, 256), 0.02, seed=1)
    s = datagen.random_f32_positive(256, 0.3, 7.0, seed=2)
    q1, sc1, z1 = O.quantize(W, s, bits, 128)
    q2, sc2, z2 = O.quantize(W, (s * np.float32(2.0 ** j)).astype(np.float32), bits, 128)
    assert np.array_equal(q1, q2) and np.array_equal(z1, z2)
    assert np.array_equal(sc2, (sc1 * np.float32(2.0 ** j)).astype(np.float32))


# ---------------------------------------------------------------------------
# P5: W'X' = WX and the axis s acts on
# ---------------------------------------------------------------------------

def test_equivalence_transform_and_axis():
    K, N, T = 256, 16, 8
    W = datagen.random_f16((N, K), 0.02, seed=3)
    X = datagen.random_f16((T, K), 1.0, seed=4)
    s = datagen.random_f32_positive(K, 0.25, 8.0, seed=5)
    # W' and X' in exact float64: the product is unchanged
    Wp = W.astype(np.float64) * s.astype(np.float64)[None, :]
    Xp = X.astype(np.float64) / s.astype(np.float64)[None, :]
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.max(np.abs(Xp @ Wp.T - ref)) <= 1e-12 * np.max(np.abs(ref))
    # the oracle's W' multiplies columns (input channels) of W [N, K] ...
    assert np.array_equal(O.scaled_weight(W, s), (W.astype(np.float32) * s[None, :]))
    # ... and quantizing with s = 2 on channel c equals quantizing W with column c doubled
    c = 37
    s2 = np.ones(K, np.float32)
    s2[c] = 2.0
    W2 = W.copy()
    W2[:, c] = (W2[:, c].astype(np.float32) * 2).astype(np.float16)
    a = O.quantize(W, s2, 4, 128)
    b = O.quantize(W2, None, 4, 128)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    # the fold divides the same channel of X
    Xf = O.fold_inv_scale(X, s2)
    assert np.array_equal(Xf[:, c], (X[:, c].astype(np.float32) / 2).astype(np.float16))
    others = np.arange(K) != c
    assert np.array_equal(Xf[:, others], X[:, others])


# ---------------------------------------------------------------------------
# statistic and scale candidates: closed forms
# ---------------------------------------------------------------------------

def test_act_stats_closed_form():
    T, K = 6, 5
    X = np.zeros((T, K), np.float16)
    X[:, 0] = [1, -1, 1, -1, 1, -1]          # mean |x| = 1
    X[:, 1] = [0.5, 0, 0, 0, 0, 0]           # 0.5/6
    X[:, 2] = [-3, -3, -3, 3, 3, 3]          # 3
    X[:, 3] = 0                              # 0 -> s = 1 for every alpha (R2)
    X[:, 4] = [2 ** -24, 0, 0, 0, 0, 65504]  # fp16 extremes, sum stays exact
    m = O.act_stats(X)
    assert m[0] == 1.0 and m[1] == 0.5 / 6 and m[2] == 3.0 and m[3] == 0.0
    assert m[4] == (2.0 ** -24 + 65504.0) / 6
    # fp16 sums are exact in float64 for T < 8192: order does not matter
    rng = np.random.default_rng(0)
    Xb = (rng.standard_normal((4096, 64)) * 100).astype(np.float16)
    mb = O.act_stats(Xb)
    exact = [sum(Fraction(float(abs(v))) for v in Xb[:, j]) / 4096 for j in range(0, 64, 16)]
    for i, j in enumerate(range(0, 64, 16)):
        assert mb[j] == float(exact[i])
    s0 = O.scale_from_stats(m, 0.0)
    assert np.array_equal(s0, np.ones(K, np.float32))


def test_scale_candidates_closed_forms():
    m = np.array([1e-3, 0.37, 1.0, 2.5, 123.0, 0.0])
    assert np.array_equal(O.scale_from_stats(m, 1.0), np.array([np.float32(v) if v > 0 else 1 for v in m], np.float32))
    half = O.scale_from_stats(m, 0.5)
    assert np.array_equal(half[:5], np.sqrt(m[:5]).astype(np.float32))
    assert half[5] == 1.0
    quarter = O.scale_from_stats(m, 0.25)
    assert np.allclose(quarter[:5], m[:5] ** 0.25, rtol=1e-7)


# ---------------------------------------------------------------------------
# P6/P7: alpha = 0 is plain RTN; the search never does worse than alpha = 0
# ---------------------------------------------------------------------------

def test_alpha_zero_is_rtn():
    W, Xc, _ = datagen.small_layer(256, 32, 32, 3, 40.0, seed=11)
    m = O.act_stats(Xc)
    s0 = O.scale_from_stats(m, 0.0)
    a = O.quantize_pack(W, s0, 4, 128)
    b = O.quantize_pack(W, None, 4, 128)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    # L(0) equals the RTN layer-output error computed without any scale
    q, sc, z = O.quantize(W, None, 4, 128)
    D = W.astype(np.float64) - O.dequantize(q, sc, z, 128)
    E = Xc.astype(np.float64) @ D.T
    assert O.layer_loss(Xc, W, s0, 4, 128) == pytest.approx(float(np.sum(E * E)), rel=1e-12)


@pytest.mark.parametrize("bits", [3, 4])
def test_search_beats_rtn_with_outliers(bits):
    W, Xc, _ = datagen.small_layer(512, 64, 64, 5, 40.0, seed=12)
    s, best, losses = O.scale_search(W, Xc, datagen.alpha_grid(20), bits, 128)
    assert losses[best] <= losses[0]
    assert losses[best] < 0.9 * losses[0]   # outlier channels are protected
    assert best > 0
    # first minimum wins
    assert best == int(np.flatnonzero(losses == losses.min())[0])
    assert np.array_equal(s, O.scale_from_stats(O.act_stats(Xc), datagen.alpha_grid(20)[best]))


def test_first_minimum_wins_on_ties():
    W, Xc, _ = datagen.small_layer(128, 4, 8, 1, 10.0, seed=13)
    # alpha values that collapse to s = 1: every loss equal -> index 0
    grid = np.zeros(5, np.float32)
    _, best, losses = O.scale_search(W, Xc, grid, 4, 128)
    assert best == 0 and np.all(losses == losses[0])


# ---------------------------------------------------------------------------
# the loss: an independent identity and exact rationals
# ---------------------------------------------------------------------------

def test_loss_gram_identity():
    W, Xc, _ = datagen.small_layer(256, 24, 48, 3, 30.0, seed=14)
    s = O.scale_from_stats(O.act_stats(Xc), 0.5)
    D = O.quant_error(W, s, 4, 128)
    H = Xc.astype(np.float64).T @ Xc.astype(np.float64)   # K x K Gram matrix
    via_gram = float(np.einsum("nk,kl,nl->", D, H, D))
    assert O.layer_loss(Xc, W, s, 4, 128) == pytest.approx(via_gram, rel=1e-9)


def test_loss_exact_rationals():
    W, Xc, _ = datagen.small_layer(128, 2, 3, 1, 20.0, seed=15)
    s = O.scale_from_stats(O.act_stats(Xc), 0.35)
    q, sc, z = O.quantize(W, s, 3, 128)
    total = Fraction(0)
    for t in range(3):
        for n in range(2):
            acc = Fraction(0)
            for k in range(128):
                wq = (int(q[n, k]) - int(z[n, 0])) * Fraction(float(sc[n, 0]))
                d = Fraction(float(W[n, k])) - wq / Fraction(float(s[k]))
                acc += Fraction(float(Xc[t, k])) * d
            total += acc * acc
    assert O.layer_loss(Xc, W, s, 3, 128) == pytest.approx(float(total), rel=1e-12)


# ---------------------------------------------------------------------------
# P8/P8b: the 1/s error ratio and the growth limit (tests/golden/error_ratio.json)
# ---------------------------------------------------------------------------

def _ratio_group():
    g = datagen.rng(4242, 0).uniform(-0.1, 0.1, size=128)
    g[0], g[1] = 1.0, -1.0
    return g


def _salient_errors(s_val):
    base = _ratio_group()
    sweep = np.linspace(-0.2, 0.2, 10001).astype(np.float16)
    W = np.tile(base, (len(sweep), 1)).astype(np.float16)
    W[:, 2] = sweep
    s = np.ones(128, np.float32)
    s[2] = s_val
    q, sc, z = O.quantize(W, s, 4, 128)
    back = O.dequantize(q, sc, z, 128) / s.astype(np.float64)[None, :]
    err = np.abs(back - W.astype(np.float64))
    return err, sc[:, 0]


def test_error_ratio_one_over_s():
    spec = _golden("error_ratio.json")
    e1, d1 = _salient_errors(1.0)
    assert np.all(d1 == np.float32(2.0) / np.float32(15.0))
    for s_txt, expect in spec["expected_ratio"].items():
        es, ds = _salient_errors(float(s_txt))
        assert np.array_equal(ds, d1)           # delta' = delta exactly
        ratio = es[:, 2].mean() / e1[:, 2].mean()
        assert abs(ratio - expect) <= spec["relative_tolerance"] * expect, ratio


def test_step_growth_hurts_others():
    spec = _golden("error_ratio.json")
    base = _ratio_group().astype(np.float16)
    W = base.copy()
    W[2] = np.float16(0.2)
    prev_delta, prev_err = 0.0, -1.0
    for s_val in spec["growth_s"]:
        s = np.ones(128, np.float32)
        s[2] = s_val
        q, sc, z = O.quantize(W[None, :], s, 4, 128)
        back = O.dequantize(q, sc, z, 128)[0] / s.astype(np.float64)
        others = np.r_[0:2, 3:128]
        err = np.abs(back - W.astype(np.float64))[others].mean()
        assert sc[0, 0] > prev_delta
        assert err >= prev_err
        prev_delta, prev_err = float(sc[0, 0]), err


# ---------------------------------------------------------------------------
# P9: exact-rational brute force of the W4A16 product, with an independent
# bit-level unpack
# ---------------------------------------------------------------------------

def _unpack_by_hand(words, bits, group, K):
    # int3 words come in blocks of 128 codes (13 words), whatever the group
    cpw = 8 if bits == 4 else 10
    blk = group if bits == 4 else 128
    wpg = -(-blk // cpw)
    codes = []
    for k in range(K):
        g, j = divmod(k, blk)
        w = int(words[g * wpg + j // cpw])
        codes.append((w >> (bits * (j % cpw))) & ((1 << bits) - 1))
    return codes


@pytest.mark.parametrize("bits,K,N,M", [(4, 128, 3, 2), (3, 128, 2, 3), (4, 256, 4, 1), (3, 256, 3, 2)])
def test_matmul_exact_rationals(bits, K, N, M):
    W = datagen.random_f16((N, K), 0.02, seed=20 + K + bits)
    s = datagen.random_f32_positive(K, 0.5, 4.0, seed=21)
    X = datagen.random_f16((M, K), 1.0, seed=22)
    qp, sc, z = O.quantize_pack(W, s, bits, 128)
    Y = O.matmul(X, qp, sc, z, bits, 128, K)
    for n in range(N):
        codes = _unpack_by_hand(qp[n], bits, 128, K)
        w = [(codes[k] - int(z[n, k // 128])) * Fraction(float(sc[n, k // 128])) for k in range(K)]
        for m in range(M):
            exact = sum(Fraction(float(X[m, k])) * w[k] for k in range(K))
            assert Y[m, n] == pytest.approx(float(exact), rel=1e-12, abs=1e-15)
    # a unit vector picks out single dequantized weights
    e = np.zeros((1, K), np.float16)
    e[0, 5] = 1
    codes0 = _unpack_by_hand(qp[0], bits, 128, K)
    assert O.matmul(e, qp, sc, z, bits, 128, K)[0, 0] == (codes0[5] - int(z[0, 0])) * float(sc[0, 0])


def test_matmul_rows_selects_output_channels():
    """Row r of the weights holds the code r mod 16 everywhere (step 1,
    zero point 0), so column r of Y is (r mod 16) times the row sum of X:
    matmul_rows must return those columns in the order asked for."""
    N, K, M = 20, 128, 3
    q = (np.arange(N)[:, None] % 16) * np.ones((1, K), dtype=np.int64)
    qp = O.pack(q, 4, 128)
    sc = np.ones((N, 1), np.float32)
    z = np.zeros((N, 1), np.uint8)
    X = datagen.random_f16((M, K), 1.0, seed=40)
    rowsum = X.astype(np.float64).sum(axis=1)
    rows = [17, 2, 9, 2]
    Y = O.matmul_rows(X, qp, sc, z, 4, 128, K, rows)
    assert Y.shape == (M, len(rows))
    for i, r in enumerate(rows):
        assert np.allclose(Y[:, i], (r % 16) * rowsum, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# P10: textbook per-channel affine fake quantization
# ---------------------------------------------------------------------------

def test_matches_torch_affine_fake_quant_except_near_ties():
    torch = pytest.importorskip("torch")
    W = datagen.random_f16((64, 512), 0.02, seed=30)
    s = datagen.random_f32_positive(512, 0.5, 3.0, seed=31)
    wp = O.scaled_weight(W, s)
    q, sc, z = O.quantize(W, s, 4, 128)
    view = torch.from_numpy(wp.reshape(-1, 128).copy())
    out = torch.fake_quantize_per_channel_affine(
        view, torch.from_numpy(sc.reshape(-1).copy()),
        torch.from_numpy(z.reshape(-1).astype(np.int32)), 0, 0, 15).numpy()
    ours = O.dequantize(q, sc, z, 128).reshape(-1, 128).astype(np.float32)
    diff = out != ours
    t = wp.reshape(-1, 128).astype(np.float64) / sc.reshape(-1, 1).astype(np.float64)
    near_tie = np.abs(t - np.floor(t) - 0.5) < 1e-5
    assert np.all(near_tie[diff])
    assert diff.mean() < 1e-3


# ---------------------------------------------------------------------------
# P11/P12: packing layout (tests/golden/pack_layout.json) and storage size
# ---------------------------------------------------------------------------

def test_pack_layout_golden():
    spec = _golden("pack_layout.json")["cases"]
    q4 = (np.arange(128) % 16)[None, :]
    w4 = O.pack(q4, 4, 128)
    assert [format(int(v), "08x") for v in w4[0]] == spec[0]["words_hex"]
    q3 = (np.arange(128) % 8)[None, :]
    w3 = O.pack(q3, 3, 128)
    assert [format(int(v), "010o") for v in w3[0]] == spec[1]["words_oct"]
    q3b = (np.arange(256) % 8)[None, :]
    w3b = O.pack(q3b, 3, 128)
    assert w3b.shape[1] == spec[2]["words_per_row"]
    assert np.array_equal(w3b[0, 13:26], w3[0, :13]) and np.all(w3b[0, 26:] == 0)
    assert np.all((w3b.astype(np.uint64) >> np.uint64(30)) == 0)
    # groups are whole 128-code blocks: the layout does not depend on the group
    w3c = O.pack(q3b, 3, 256)
    assert w3c.shape[1] == spec[3]["words_per_row"] and np.array_equal(w3c, w3b)
    q3d = (np.arange(384) % 8)[None, :]
    w3d = O.pack(q3d, 3, 384)
    assert w3d.shape[1] == spec[4]["words_per_row"]
    for b in range(3):
        assert np.array_equal(w3d[0, 13 * b:13 * b + 13], w3[0, :13])
    assert w3d[0, 39] == 0


@pytest.mark.parametrize("bits", [3, 4])
def test_pack_roundtrip(bits):
    rng = np.random.default_rng(5)
    for K, group in ((128, 128), (384, 128), (4096, 128), (11008, 128), (1024, 256),
                     (2048, 512), (384, 384), (11008, 11008)):
        q = rng.integers(0, 1 << bits, size=(3, K))
        w = O.pack(q, bits, group)
        assert w.dtype == np.uint32 and w.shape == (3, O.words_per_row(K, bits, group))
        assert np.array_equal(O.unpack(w, bits, group, K), q)
        assert w.shape[1] % 4 == 0
        # every bit of a code shows up once, at its own position
        word, shift = O.code_position(np.arange(K), bits)
        assert len(set(zip(word.tolist(), shift.tolist()))) == K
        assert word.max() < w.shape[1] and shift.max() + bits <= 30 + 2 * (bits == 4)


def test_words_per_row_values():
    assert O.words_per_row(4096, 4, 128) == 512
    assert O.words_per_row(8192, 4, 128) == 1024
    assert O.words_per_row(4096, 3, 128) == 416       # 32 groups x 13 words
    assert O.words_per_row(11008, 3, 128) == 1120     # 86 x 13 = 1118 -> 1120
    assert O.words_per_row(512, 3, 128) == 52


def test_storage_ratio():
    # hungho77 blog -- "Why weight-only quantization fits decoding": FP16 -> INT4
    # cuts raw weight storage by about four times
    N, K = 4096, 4096
    packed_bytes = N * O.words_per_row(K, 4, 128) * 4
    assert packed_bytes * 4 == N * K * 2
    with_meta = packed_bytes + N * (K // 128) * (4 + 1)
    assert 3.7 < (N * K * 2) / with_meta < 3.72
    int3 = N * O.words_per_row(K, 3, 128) * 4 + N * (K // 128) * 5
    assert 4.4 < (N * K * 2) / int3 < 4.6


# ---------------------------------------------------------------------------
# fold: X' = fp16(fp32(X) / s), a closed form on powers of two
# ---------------------------------------------------------------------------

def test_fold_powers_of_two_exact():
    ints = datagen.rng(40, 0).integers(1, 64, size=(4, 256)) * np.where(np.arange(256) % 3, 1, -1)
    X = (ints / 8.0).astype(np.float16)          # |x| in [1/8, 8): no fp16 underflow or overflow
    s = np.float32(2.0) ** np.arange(-3, 5, dtype=np.float32)[np.arange(256) % 8]
    Xf = O.fold_inv_scale(X, s)
    assert np.array_equal(Xf.astype(np.float64), X.astype(np.float64) / s.astype(np.float64)[None, :])


def test_ties_round_half_even_and_zero_after_rint():
    spec = _golden("exact_groups.json")["ties"]
    i = np.arange(128) % 16
    v = ((i - 7) / 16.0)
    v[112:127] = (np.arange(15) - 6.5) / 16.0
    v[127] = 1.0 / 32.0
    W = v.astype(np.float16)[None, :]
    s = np.ones(128, np.float32)
    s[127] = np.nextafter(np.float32(1.0), np.float32(0.0))
    q, sc, z = O.quantize(W, s, 4, 128)
    assert sc[0, 0] == np.float32(1 / 16) and z[0, 0] == 7
    assert list(q[0, 112:127]) == spec["expected_tie_codes"]
    assert q[0, 127] == spec["expected_near_tie_code"]


# ---------------------------------------------------------------------------
# zero_point=false: the symmetric grid (R17)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", _golden("exact_groups_symmetric.json")["cases"])
def test_symmetric_exact_group(case):
    bits, G = case["bits"], case["group"]
    i = np.arange(G) % case["count"]
    v = ((i - case["h"]) / case["den"]).astype(np.float16)
    W = np.stack([v, v[::-1]])
    q, scales, zeros = O.quantize(W, None, bits, G, zero_point=False)
    assert np.all(scales == np.float32(case["delta"]))
    assert np.all(zeros == case["zero"])
    assert np.array_equal(q[0], i + 1) and np.array_equal(q[1], (i + 1)[::-1])
    assert np.array_equal(O.dequantize(q, scales, zeros, G), W.astype(np.float64))


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(vals=_group_strategy(), bits=st.sampled_from([3, 4]), scale_exp=st.integers(-3, 3))
def test_symmetric_half_step_bound_odd_symmetry(vals, bits, scale_exp):
    W = np.array(vals, dtype=np.float16)[None, :]
    s = np.full(128, np.float32(1.5 * 2.0 ** scale_exp), dtype=np.float32)
    wp = O.scaled_weight(W, s)
    q, scales, zeros = O.quantize(W, s, bits, 128, zero_point=False)
    half = 1 << (bits - 1)
    assert np.all(zeros == half)
    assert q.min() >= 1 and q.max() <= 2 * half - 1   # never the unused code -2^(b-1)
    d = float(scales[0, 0])
    err = np.abs(O.dequantize(q, scales, zeros, 128)[0] - wp[0].astype(np.float64))
    assert err.max() <= d * (0.5 + 1e-5), (err.max() / d)
    # rint is odd-symmetric and max|W'| is the same, so -W gets the negated codes
    qn, sn, zn = O.quantize(-W, s, bits, 128, zero_point=False)
    assert np.array_equal(sn, scales) and np.array_equal(qn - half, -(q - half))
    if np.all(W == 0):
        assert d == 1.0 and np.all(q == half)


@pytest.mark.parametrize("bits", [3, 4])
def test_symmetric_power_of_two_equivariance(bits):
    W = datagen.random_f16((8, 256), 0.02, seed=3)
    s = datagen.random_f32_positive(256, 0.3, 7.0, seed=4)
    q1, sc1, z1 = O.quantize(W, s, bits, 128, zero_point=False)
    q2, sc2, z2 = O.quantize(W, (s * np.float32(8.0)).astype(np.float32), bits, 128, zero_point=False)
    assert np.array_equal(q1, q2) and np.array_equal(z1, z2)
    assert np.array_equal(sc2, (sc1 * np.float32(8.0)).astype(np.float32))


@pytest.mark.parametrize("bits", [3, 4])
def test_symmetric_matmul_exact_rationals(bits):
    K, N, M = 256, 3, 2
    W = datagen.random_f16((N, K), 0.02, seed=30 + bits)
    s = datagen.random_f32_positive(K, 0.5, 4.0, seed=31)
    X = datagen.random_f16((M, K), 1.0, seed=32)
    qp, sc, z = O.quantize_pack(W, s, bits, 128, zero_point=False)
    Y = O.matmul(X, qp, sc, z, bits, 128, K)
    for n in range(N):
        codes = _unpack_by_hand(qp[n], bits, 128, K)
        w = [(codes[k] - int(z[n, k // 128])) * Fraction(float(sc[n, k // 128])) for k in range(K)]
        for m in range(M):
            exact = sum(Fraction(float(X[m, k])) * w[k] for k in range(K))
            assert Y[m, n] == pytest.approx(float(exact), rel=1e-12, abs=1e-15)


@pytest.mark.parametrize("bits", [3, 4])
def test_symmetric_search(bits):
    """alpha = 0 is plain symmetric RTN, and the search still protects the
    outlier channels."""
    W, Xc, _ = datagen.small_layer(512, 64, 64, 5, 40.0, seed=77)
    grid = datagen.alpha_grid(20)
    s, best, losses = O.scale_search(W, Xc, grid, bits, 128, zero_point=False)
    q0, sc0, z0 = O.quantize(W, None, bits, 128, zero_point=False)
    ones = O.scale_from_stats(O.act_stats(Xc), 0.0)
    assert np.all(ones == 1.0)
    assert losses[0] == O.layer_loss(Xc, W, ones, bits, 128, zero_point=False)
    qa, sca, za = O.quantize(W, ones, bits, 128, zero_point=False)
    assert np.array_equal(qa, q0) and np.array_equal(sca, sc0)
    assert losses[best] < losses[0]


# ---------------------------------------------------------------------------
# gated MLP: silu(X' Wg^T) * (X' Wu^T) (R18)
# ---------------------------------------------------------------------------

def test_silu_against_library_and_identities():
    torch = pytest.importorskip("torch")
    v = np.concatenate([np.linspace(-30, 30, 1201), [-800.0, -710.0, 0.0, 1e-300, 50.0, 800.0]])
    ref = torch.nn.functional.silu(torch.from_numpy(v)).numpy()
    got = O.silu(v)
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-300)
    assert O.silu(0.0) == 0.0 and O.silu(800.0) == 800.0 and O.silu(-800.0) == 0.0
    # sigmoid(-v) = 1 - sigmoid(v)  =>  silu(-v) = silu(v) - v
    w = np.linspace(-20, 20, 401)
    assert np.allclose(O.silu(-w), O.silu(w) - w, rtol=0, atol=1e-12)
    assert O.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)


@pytest.mark.parametrize("bits", [3, 4])
def test_gate_up_silu_picks_single_weights(bits):
    """A unit activation e_k selects column k of both matrices, so each output
    is silu(wg_nk) * wu_nk of the dequantized weights (read here with an
    independent bit-level unpack)."""
    K, N = 256, 5
    Wg = datagen.random_f16((N, K), 0.5, seed=50 + bits)
    Wu = datagen.random_f16((N, K), 0.5, seed=60 + bits)
    qg, sg, zg = O.quantize_pack(Wg, None, bits, 128)
    qu, su, zu = O.quantize_pack(Wu, None, bits, 128)
    for k in (0, 1, 127, 128, 255):
        X = np.zeros((1, K), np.float16)
        X[0, k] = 1.0
        Y = O.gate_up_silu(X, qg, sg, zg, qu, su, zu, bits, 128, K)[0]
        for n in range(N):
            cg = _unpack_by_hand(qg[n], bits, 128, K)[k]
            cu = _unpack_by_hand(qu[n], bits, 128, K)[k]
            wg = (cg - int(zg[n, k // 128])) * float(sg[n, k // 128])
            wu = (cu - int(zu[n, k // 128])) * float(su[n, k // 128])
            assert Y[n] == pytest.approx(wg / (1.0 + math.exp(-wg)) * wu, rel=1e-14, abs=1e-300)


def test_gate_up_silu_exact_products():
    """Exact-rational gate and up products, then silu in float64."""
    K, N, M = 256, 3, 2
    Wg = datagen.random_f16((N, K), 0.02, seed=71)
    Wu = datagen.random_f16((N, K), 0.02, seed=72)
    X = datagen.random_f16((M, K), 1.0, seed=73)
    qg, sg, zg = O.quantize_pack(Wg, None, 4, 128)
    qu, su, zu = O.quantize_pack(Wu, None, 4, 128)
    Y = O.gate_up_silu(X, qg, sg, zg, qu, su, zu, 4, 128, K)

    def exact(qp, sc, z, n, m):
        codes = _unpack_by_hand(qp[n], 4, 128, K)
        return sum(Fraction(float(X[m, k])) * (codes[k] - int(z[n, k // 128]))
                   * Fraction(float(sc[n, k // 128])) for k in range(K))
    for m in range(M):
        for n in range(N):
            g = float(exact(qg, sg, zg, n, m))
            u = float(exact(qu, su, zu, n, m))
            assert Y[m, n] == pytest.approx(g / (1.0 + math.exp(-g)) * u, rel=1e-12)


# ---------------------------------------------------------------------------
# RMSNorm with the folded scale (R20) and the joint search (R21)
# ---------------------------------------------------------------------------

def test_rmsnorm_against_library():
    """torch's functional rms_norm (a library routine) in float64, rounded
    once to fp16, agrees bit for bit except where the float64 value sits
    within rounding of an fp16 midpoint (then one ulp)."""
    torch = pytest.importorskip("torch")
    X = datagen.random_f16((7, 4096), 1.0, seed=81)
    gamma = (1.0 + datagen.random_f16((4096,), 0.1, seed=82)).astype(np.float16)
    eps = 1e-6
    ref = torch.nn.functional.rms_norm(torch.from_numpy(X.astype(np.float64)), (4096,),
                                       torch.from_numpy(gamma.astype(np.float64)), eps)
    ref16 = ref.numpy().astype(np.float16)
    got = O.rmsnorm(X, gamma, eps)
    diff = np.abs(got.astype(np.float32) - ref16.astype(np.float32))
    ulp = np.abs(np.spacing(ref16)).astype(np.float32)
    assert np.all(diff <= ulp)
    assert np.mean(got == ref16) > 0.999


def test_rmsnorm_closed_forms():
    """A row of equal values c normalizes to sign(c) * gamma / sqrt(1 + eps/c^2);
    scaling a row by 2^j leaves the output unchanged when eps = 0."""
    K = 256
    gamma = np.full(K, 0.5, np.float16)
    X = np.stack([np.full(K, 3.0), np.full(K, -0.25)]).astype(np.float16)
    Y = O.rmsnorm(X, gamma, 0.0)
    assert np.all(Y[0] == np.float16(0.5)) and np.all(Y[1] == np.float16(-0.5))
    Z = datagen.random_f16((3, K), 1.0, seed=83)
    g = datagen.random_f16((K,), 1.0, seed=84)
    assert np.array_equal(O.rmsnorm(Z, g, 0.0), O.rmsnorm((Z * np.float16(4)).astype(np.float16), g, 0.0))
    assert O.rmsnorm(np.zeros((1, K), np.float16), g, 1e-6).max() == 0


def test_folded_norm_equals_norm_then_division():
    """norm with gamma / s == (norm with gamma) / s, up to the fp16 roundings
    of gamma' and of the output (each 2^-11 relative)."""
    K = 1024
    X = datagen.random_f16((5, K), 1.0, seed=85)
    gamma = (1.0 + datagen.random_f16((K,), 0.1, seed=86)).astype(np.float16)
    s = datagen.random_f32_positive(K, 0.2, 9.0, seed=87)
    gp = O.fold_norm_weight(gamma, s)
    assert gp.dtype == np.float16
    assert np.array_equal(gp, (gamma.astype(np.float32) / s).astype(np.float16))
    a = O.rmsnorm(X, gp, 1e-6).astype(np.float64)
    x = X.astype(np.float64)
    b = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + 1e-6) * gamma.astype(np.float64) / s
    assert np.all(np.abs(a - b) <= (2.0 ** -10 + 2.0 ** -20) * np.abs(b) + 2.0 ** -24)
    # s = 1 folds to gamma itself
    assert np.array_equal(O.fold_norm_weight(gamma, np.ones(K, np.float32)), gamma)


def test_joint_search_equals_search_on_stacked_rows():
    """The loss is a sum over output channels and every group lies in one
    row, so the joint search over [W1, W2] is the plain search over the
    stacked matrix; with one layer it is the plain search."""
    W1, Xc, _ = datagen.small_layer(256, 48, 40, 3, 40.0, seed=88)
    W2 = datagen.random_f16((32, 256), 0.02, seed=89)
    grid = datagen.alpha_grid(10)
    for zp in (True, False):
        sj, bj, lj = O.joint_scale_search([W1, W2], Xc, grid, 4, 128, zp)
        ss, bs, ls = O.scale_search(np.vstack([W1, W2]), Xc, grid, 4, 128, zp)
        assert np.allclose(lj, ls, rtol=1e-12, atol=0)
        assert bj == bs and np.array_equal(sj, ss)
        s1, b1, l1 = O.joint_scale_search([W1], Xc, grid, 3, 128, zp)
        s0, b0, l0 = O.scale_search(W1, Xc, grid, 3, 128, zp)
        assert np.array_equal(l1, l0) and b1 == b0 and np.array_equal(s1, s0)


# ---------------------------------------------------------------------------
# ablations (R23)
# ---------------------------------------------------------------------------

def test_salient_channels_hand_cases():
    assert O.salient_channels([0.1, 5.0, 0.3, 5.0, 2.0], 2).tolist() == [1, 3]
    assert O.salient_channels([0.1, 5.0, 0.3, 5.0, 2.0], 3).tolist() == [1, 3, 4]
    assert O.salient_channels([1.0, 1.0, 1.0], 2).tolist() == [0, 1]  # ties: lower index
    assert O.salient_channels([3.0, 1.0], 0).tolist() == []
    W = np.array([[1, -4, 0.5], [-1, 2, 0.5]], np.float16)
    assert O.weight_channel_magnitude(W).tolist() == [1.0, 3.0, 0.5]


@pytest.mark.parametrize("bits", [3, 4])
def test_fp16_kept_limits_and_masked_identity(bits):
    """No kept channel is plain RTN; every channel kept is exact (loss 0);
    and keeping channels C is the RTN loss of the calibration batch with the
    columns C set to zero (D's columns C vanish)."""
    W, Xc, ch = datagen.small_layer(512, 64, 48, 5, 40.0, seed=95)
    rtn = O.layer_loss(Xc, W, np.ones(512, np.float32), bits, 128)
    assert O.layer_loss_fp16_kept(Xc, W, [], bits, 128) == rtn
    assert O.layer_loss_fp16_kept(Xc, W, np.arange(512), bits, 128) == 0.0
    Xm = Xc.copy()
    Xm[:, ch] = 0
    kept = O.layer_loss_fp16_kept(Xc, W, ch, bits, 128)
    assert kept == pytest.approx(O.layer_loss(Xm, W, np.ones(512, np.float32), bits, 128),
                                 rel=1e-12)


def test_ablation_orderings_on_outlier_layer():
    """The pages' qualitative findings, as layer-output errors on a layer
    whose 1% outlier channels carry large activations: keeping the
    activation-salient 1% in FP16 removes most of the RTN error, keeping
    the weight-salient 1% barely helps, and the scale search recovers most
    of the gap without mixed precision."""
    w = datagen.WORKLOADS["llama7b_attn_4096x4096_int4"]
    W, Xc = datagen.weight(w)[:512], datagen.calibration(w)
    n = round(0.01 * w.K)
    rtn = O.layer_loss(Xc, W, np.ones(w.K, np.float32), 4, 128)
    act = O.layer_loss_fp16_kept(Xc, W, O.salient_channels(O.act_stats(Xc), n), 4, 128)
    wgt = O.layer_loss_fp16_kept(Xc, W, O.salient_channels(O.weight_channel_magnitude(W), n),
                                 4, 128)
    _, _, losses = O.scale_search(W, Xc, datagen.alpha_grid(20), 4, 128)
    assert act < 0.1 * rtn
    assert wgt > 0.9 * rtn
    assert losses.min() < 0.3 * rtn


# ---------------------------------------------------------------------------
# compact storage of the group parameters (R24)
# ---------------------------------------------------------------------------

def test_compact_group_params_hand_words():
    """Zero points 0..15 of one row read back from a word printed in hex
    (slot 7 down to slot 0), and fp16 steps rounded once."""
    z = np.arange(16, dtype=np.uint8)[None, :]
    sc = np.full((1, 16), 0.1, np.float32)
    s16, z4 = O.compact_group_params(sc, z)
    assert [format(int(v), "08x") for v in z4[0]] == ["76543210", "fedcba98"]
    assert s16.dtype == np.float16 and np.all(s16 == np.float16(0.1))
    # 9 groups: the second word holds one zero point, the rest is zero
    s16, z4 = O.compact_group_params(sc[:, :9], np.full((1, 9), 13, np.uint8))
    assert z4.shape == (1, 2) and int(z4[0, 0]) == 0xDDDDDDDD and int(z4[0, 1]) == 0xD


@pytest.mark.parametrize("bits,group,K", [(4, 128, 1024), (3, 128, 640), (4, 256, 2048),
                                          (4, 384, 384), (3, 512, 1024)])
def test_compact_roundtrip_and_product(bits, group, K):
    W = datagen.random_f16((9, K), 0.02, seed=K + group)
    X = datagen.random_f16((3, K), 1.0, seed=7)
    qp, sc, z = O.quantize_pack(W, None, bits, group)
    s16, z4 = O.compact_group_params(sc, z)
    sc2, z2 = O.expand_group_params(s16, z4, K // group)
    assert np.array_equal(z2, z)
    assert np.array_equal(sc2, sc.astype(np.float16).astype(np.float32))
    # the compact product is the plain product with the fp16-rounded steps
    Yc = O.matmul_compact(X, qp, s16, z4, bits, group, K)
    Yr = O.matmul(X, qp, sc.astype(np.float16).astype(np.float32), z, bits, group, K)
    assert np.array_equal(Yc, Yr)
    # and within fp16's step rounding (2^-11 relative per group) of the exact one
    Y = O.matmul(X, qp, sc, z, bits, group, K)
    bound = 2.0 ** -11 * (np.abs(X.astype(np.float64)) @ np.abs(O.dequantize(
        O.unpack(qp, bits, group, K), sc, z, group)).T)
    assert np.all(np.abs(Yc - Y) <= bound * (1 + 1e-9))


def test_workload_search_golden_matches_oracle():
    """tests/golden/workload_search.json holds the oracle's full loss curves
    (written by make_workload_search.py from the oracle alone); the
    512 x 512 layer's curve is recomputed here and must agree exactly, and
    every stored curve has the default grid and its first minimum recorded."""
    import json
    import os
    with open(os.path.join(GOLDEN, "workload_search.json")) as f:
        doc = json.load(f)
    entries = {(e["kind"], e["workload"]): e for e in doc["entries"]}
    for name in datagen.WORKLOADS:
        assert ("single", name) in entries
    for e in doc["entries"]:
        grid = datagen.alpha_grid(20)
        assert np.array_equal(np.asarray(e["alpha_grid"], np.float32), grid)
        L = np.asarray(e["losses"])
        assert len(L) == 20 and np.all(L > 0)
        assert e["best_index"] == int(np.argmin(L))
        assert L[e["best_index"]] < L[0]  # the outlier channels make scaling pay
    w = datagen.WORKLOADS[datagen.SMALL]
    _, best, losses = O.scale_search(datagen.weight(w), datagen.calibration(w),
                                     datagen.alpha_grid(w.n_alpha), w.bits, w.group)
    e = entries[("single", w.name)]
    assert best == e["best_index"]
    assert np.array_equal(losses, np.asarray(e["losses"]))
