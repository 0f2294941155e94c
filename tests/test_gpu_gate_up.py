"""GPU parity of the fused gated-MLP product Y = silu(X' Wg^T) * (X' Wu^T)
(awq_w4a16_gate_up_silu) against the oracle.

Tolerance: the matmul contract (per output row, error <= 1e-3 of the row's
largest |value|) for each of the two products G and U, carried through
silu * mul to first order, plus the final fp16 rounding:
  |Y - Y*| <= 1e-3 (|silu'(G)| max|G_row| |U| + |silu(G)| max|U_row|)
              + 2^-11 |Y*| + 2^-24,
elementwise, with G, U the oracle's exact products. A plain 1e-3 on Y
would not do: Y's relative error is about the sum of G's and U's, and
where silu(G) is small while U is large, an error of G that is small
against max|G| is not small against Y."""
import functools

import numpy as np
import pytest

import datagen
from oracle import awq_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import weight_only_bit_w4a16_amd as awq  # noqa: E402
from tests.test_gpu_parity import dev, host, sample_rows, say  # noqa: E402


def _pair(N, K, bits, group, seed, with_s=True, zero_point=True):
    Wg = datagen.random_f16((N, K), 0.02, seed=seed)
    Wu = datagen.random_f16((N, K), 0.02, seed=seed + 1)
    s = datagen.random_f32_positive(K, 0.3, 5.0, seed=seed + 2) if with_s else None
    g = O.quantize_pack(Wg, s, bits, group, zero_point)
    u = O.quantize_pack(Wu, s, bits, group, zero_point)
    return g, u, s


def assert_gate_up_close(Yg, Xp, g, u, bits, group, K, tol=1e-3):
    Yg = np.asarray(Yg, dtype=np.float64)
    G = O.matmul(Xp, *g, bits, group, K)
    U = O.matmul(Xp, *u, bits, group, K)
    Y = O.gate_up_silu(Xp, *g, *u, bits, group, K)
    assert Yg.shape == Y.shape and np.all(np.isfinite(Yg))
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-G))
    dsilu = sig * (1.0 + G * (1.0 - sig))
    gmax = np.abs(G).max(axis=1, keepdims=True)
    umax = np.abs(U).max(axis=1, keepdims=True)
    bound = tol * (np.abs(dsilu) * gmax * np.abs(U) + np.abs(O.silu(G)) * umax) \
        + 2.0 ** -11 * np.abs(Y) + 2.0 ** -24
    err = np.abs(Yg - Y)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (bad[:5].tolist(), (err / bound).max())
    return float((err / bound).max())


def _dev3(t):
    """(qpacked, scales, zeros) of the oracle on the device; the binding
    takes the packed words as int32."""
    return (dev(t[0].view(np.int32)), dev(t[1]), dev(t[2]))


def _run(X, g, u, bits, group):
    return host(awq.gate_up_silu(dev(X), _dev3(g), _dev3(u), bits, group))


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("M", [1, 2, 5, 16, 100])
@pytest.mark.parametrize("N,K", [(16, 128), (17, 384), (100, 1024), (257, 4096)])
def test_gate_up_small(bits, M, N, K):
    say("gate_up", bits, M, N, K)
    g, u, _ = _pair(N, K, bits, 128, seed=N + K)
    X = datagen.random_f16((M, K), 1.0, seed=M + 7)
    assert_gate_up_close(_run(X, g, u, bits, 128), X, g, u, bits, 128, K)


@pytest.mark.parametrize("bits,M,N,K", [(4, 2, 70, 2048), (4, 2, 6200, 4096), (4, 2, 300, 8192),
                                        (4, 3, 6200, 4096), (4, 4, 33, 4096), (3, 2, 129, 6016),
                                        (3, 3, 77, 3968), (3, 4, 300, 2048), (3, 4, 90, 4096),
                                        (3, 3, 60, 6016), (3, 3, 40, 8192), (3, 3, 50, 11008)])
def test_gate_up_few_token_rows(bits, M, N, K):
    """2 <= M <= 4: the few-token kernels in their gated form (gate and up
    rows alternate; int4 at M = 2, int3 at M = 2-4 while the operands fit),
    partial last pieces, int3 pairs of token rows (4096 at M = 4) and an
    M = 1 launch for an odd last row (6016 at M = 3), the prefill kernel past
    that (8192, 11008 at M = 3) and the 16-row-block kernel for int4 at
    M = 3, 4."""
    say("gate_up few token rows", bits, M, N, K)
    g, u, _ = _pair(N, K, bits, 128, seed=N + 3 * K)
    X = datagen.random_f16((M, K), 1.0, seed=M + K)
    Y = _run(X, g, u, bits, 128)
    assert_gate_up_close(Y, X, g, u, bits, 128, K)
    assert np.array_equal(_run(X, g, u, bits, 128).view(np.uint16), Y.view(np.uint16))


@pytest.mark.parametrize("group", [256, 512])
@pytest.mark.parametrize("M", [1, 33])
def test_gate_up_int4_larger_groups(group, M):
    N, K = 130, 2048
    g, u, _ = _pair(N, K, 4, group, seed=group)
    X = datagen.random_f16((M, K), 1.0, seed=group + M)
    assert_gate_up_close(_run(X, g, u, 4, group), X, g, u, 4, group, K)


def test_gate_up_symmetric_and_long_rows():
    """Symmetric codes, and K = 16384 (past the M = 1 decode kernel's 96
    groups: the call runs the prefill kernel)."""
    for (N, K) in [(64, 4096), (40, 16384)]:
        g, u, _ = _pair(N, K, 4, 128, seed=K, zero_point=False)
        X = datagen.random_f16((1, K), 1.0, seed=5)
        assert_gate_up_close(_run(X, g, u, 4, 128), X, g, u, 4, 128, K)


def test_gate_up_saturating_gate():
    """Large gate sums push silu to its limits (e^-g overflows for very
    negative g; silu(g) = g for large g)."""
    N, K = 64, 1024
    Wg = (datagen.random_f16((N, K), 0.02, seed=3) * np.float16(40)).astype(np.float16)
    Wu = datagen.random_f16((N, K), 0.02, seed=4)
    g = O.quantize_pack(Wg, None, 4, 128)
    u = O.quantize_pack(Wu, None, 4, 128)
    X = (datagen.random_f16((3, K), 1.0, seed=6) * np.float16(4)).astype(np.float16)
    G = O.matmul(X, *g, 4, 128, K)
    assert G.max() > 60 and G.min() < -60
    for M in (1, 3):
        assert_gate_up_close(_run(X[:M], g, u, 4, 128), X[:M], g, u, 4, 128, K)


@functools.lru_cache(maxsize=1)
def _workload_pair(name):
    w = datagen.WORKLOADS[name]
    Wu = datagen.weight(w)
    Wg = datagen.gate_weight(w)
    s = O.scale_from_stats(O.act_stats(datagen.calibration(w)), 0.5)
    return Wg, Wu, s


@pytest.mark.parametrize("name,M", [("llama7b_mlp_up_4096x11008_int4", 1),
                                    ("llama7b_mlp_up_4096x11008_int4", 8),
                                    ("llama7b_mlp_up_4096x11008_int3", 1),
                                    ("llama7b_mlp_up_4096x11008_int3", 256),
                                    ("llama70b_mlp_8192x28672_int4", 1),
                                    ("llama70b_mlp_8192x28672_int4", 2048)])
def test_gate_up_workload(name, M):
    """Full size on the device (both matrices packed by the library); the
    oracle packs and multiplies sampled output rows."""
    w = datagen.WORKLOADS[name]
    say("gate_up workload", name, M)
    Wg, Wu, s = _workload_pair(name)
    X = datagen.decode_input(w, M)
    sd = dev(s)
    gd = awq.quantize_pack(dev(Wg), sd, w.bits, w.group)
    ud = awq.quantize_pack(dev(Wu), sd, w.bits, w.group)
    Xp = awq.fold_inv_scale(dev(X), sd)
    Y = host(awq.gate_up_silu(Xp, gd, ud, w.bits, w.group))
    rows = sample_rows(w.N, count=128)
    g = O.quantize_pack(Wg[rows], s, w.bits, w.group)
    u = O.quantize_pack(Wu[rows], s, w.bits, w.group)
    r = assert_gate_up_close(Y[:, rows], O.fold_inv_scale(X, s), g, u, w.bits, w.group, w.K)
    say("worst error / bound", r)


def test_gate_up_matches_separate_products():
    """The fused call against the library's own two products followed by
    silu * mul in float64 on the host. The separate products are rounded to
    fp16 (2^-11 relative each) and carry their own 1e-3 contract, so the
    bound is the fused one with both budgets added."""
    N, K, M = 300, 4096, 4
    g, u, _ = _pair(N, K, 4, 128, seed=11)
    X = datagen.random_f16((M, K), 1.0, seed=12)
    gd, ud = _dev3(g), _dev3(u)
    Xd = dev(X)
    Y = host(awq.gate_up_silu(Xd, gd, ud, 4, 128)).astype(np.float64)
    G = host(awq.w4a16_matmul(Xd, *gd, 4, 128)).astype(np.float64)
    U = host(awq.w4a16_matmul(Xd, *ud, 4, 128)).astype(np.float64)
    sig = 1.0 / (1.0 + np.exp(-G))
    Ys = G * sig * U
    bound = 2e-3 * (np.abs(sig * (1 + G * (1 - sig))) * np.abs(G).max(1, keepdims=True) * np.abs(U)
                    + np.abs(G * sig) * np.abs(U).max(1, keepdims=True)) + 2.0 ** -10 * np.abs(Ys) \
        + 2.0 ** -24
    assert np.all(np.abs(Y - Ys) <= bound)
