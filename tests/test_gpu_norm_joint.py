"""GPU parity of the scale folded into the RMSNorm (the folded weight
bit-exact, the norm within one fp16 ulp) and of the joint alpha search of
layers that share one input (losses within 1e-4, argmin contract, s
bit-exact), against the oracle."""
import numpy as np
import pytest

import datagen
from oracle import awq_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import weight_only_bit_w4a16_amd as awq  # noqa: E402
from tests.test_gpu_parity import (assert_rows_close, assert_same_bits, dev, host,  # noqa: E402
                                   sample_rows, say)


@pytest.mark.parametrize("K", [8, 128, 4096, 11008])
def test_fold_norm_weight_exact(K):
    gamma = (1.0 + datagen.random_f16((K,), 0.2, seed=K)).astype(np.float16)
    s = datagen.random_f32_positive(K, 0.05, 20.0, seed=K + 1)
    got = host(awq.fold_norm_weight(dev(gamma), dev(s)))
    assert_same_bits(got, O.fold_norm_weight(gamma, s))


def assert_within_one_ulp(got, ref):
    got = np.asarray(got, np.float16)
    ref = np.asarray(ref, np.float16)
    assert got.shape == ref.shape
    diff = np.abs(got.astype(np.float32) - ref.astype(np.float32))
    ulp = np.abs(np.spacing(ref)).astype(np.float32)
    assert np.all(diff <= ulp), float((diff / ulp).max())
    return float(np.mean(got == ref))


@pytest.mark.parametrize("M,K", [(1, 128), (3, 4096), (5, 11008), (2, 16384), (2048, 8192)])
@pytest.mark.parametrize("eps", [1e-6, 0.0])
def test_rmsnorm(M, K, eps):
    say("rmsnorm", M, K, eps)
    X = datagen.random_f16((M, K), 1.0, seed=M + K)
    X[0, : K // 2] *= np.float16(30)  # uneven rows
    gamma = (1.0 + datagen.random_f16((K,), 0.2, seed=K + 5)).astype(np.float16)
    got = host(awq.rmsnorm(dev(X), dev(gamma), eps))
    same = assert_within_one_ulp(got, O.rmsnorm(X, gamma, eps))
    assert same > 0.999


def test_rmsnorm_zero_row():
    X = np.zeros((2, 512), np.float16)
    X[1] = 1
    gamma = np.ones(512, np.float16)
    got = host(awq.rmsnorm(dev(X), dev(gamma), 1e-6))
    assert np.all(got[0] == 0)
    assert_within_one_ulp(got, O.rmsnorm(X, gamma, 1e-6))


def test_folded_norm_feeds_the_product():
    """search -> fold s into the norm weight -> norm -> W4A16 product, every
    step on the device, against the oracle's same chain."""
    w = datagen.WORKLOADS["llama7b_attn_4096x4096_int4"]
    W = datagen.weight(w)
    Xc = datagen.calibration(w)
    X = datagen.decode_input(w, 4)
    gamma = (1.0 + datagen.random_f16((w.K,), 0.1, seed=90)).astype(np.float16)
    grid = datagen.alpha_grid(w.n_alpha)
    s_g, best, _ = awq.scale_search(dev(W), dev(Xc), grid, w.bits, w.group)
    gp = awq.fold_norm_weight(dev(gamma), s_g)
    Xp = awq.rmsnorm(dev(X), gp, 1e-6)
    q, sc, z = awq.quantize_pack(dev(W), s_g, w.bits, w.group)
    Y = host(awq.w4a16_matmul(Xp, q, sc, z, w.bits, w.group))
    s_o = O.scale_from_stats(O.act_stats(Xc), grid[best])
    assert_same_bits(host(s_g), s_o)
    gp_o = O.fold_norm_weight(gamma, s_o)
    assert_same_bits(host(gp), gp_o)
    Xp_o = O.rmsnorm(X, gp_o, 1e-6)
    assert_within_one_ulp(host(Xp), Xp_o)
    rows = sample_rows(w.N)
    qo, so, zo = O.quantize_pack(W[rows], s_o, w.bits, w.group)
    assert_rows_close(Y[:, rows], O.matmul(host(Xp), qo, so, zo, w.bits, w.group, w.K))


def check_joint(Ws, Xc, grid, bits, group, zero_point=True, oracle_idx=None):
    s_g, best_g, loss_g = awq.scale_search_joint([dev(W) for W in Ws], dev(Xc), grid, bits,
                                                 group, zero_point=zero_point)
    m = O.act_stats(Xc)
    idx = range(len(grid)) if oracle_idx is None else sorted(set(oracle_idx) | {best_g})
    for i in idx:
        s = O.scale_from_stats(m, grid[i])
        lo = sum(O.layer_loss(Xc, W, s, bits, group, zero_point) for W in Ws)
        assert abs(loss_g[i] - lo) <= 1e-4 * lo, (i, loss_g[i], lo)
    assert best_g == int(np.argmin(loss_g))
    assert_same_bits(host(s_g), O.scale_from_stats(m, grid[best_g]))
    return best_g, loss_g


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("zero_point", [True, False])
def test_joint_search_small(bits, zero_point):
    """q/k/v-like: three matrices of different N on one input (hi/lo and
    scaled sizes mixed)."""
    K, T = 512, 64
    W1, Xc, _ = datagen.small_layer(K, 64, T, 5, 40.0, seed=91)
    W2 = datagen.random_f16((4096, K), 0.02, seed=92)
    W3 = datagen.random_f16((40, K), 0.02, seed=93)
    grid = datagen.alpha_grid(20)
    check_joint([W1, W2, W3], Xc, grid, bits, 128, zero_point)


def test_joint_one_layer_is_the_plain_search():
    W, Xc, _ = datagen.small_layer(1024, 300, 100, 10, 40.0, seed=94)
    grid = datagen.alpha_grid(20)
    s1, b1, l1 = awq.scale_search(dev(W), dev(Xc), grid, 4, 128)
    s2, b2, l2 = awq.scale_search_joint([dev(W)], dev(Xc), grid, 4, 128)
    assert b1 == b2 and np.array_equal(l1, l2)
    assert_same_bits(host(s1), host(s2))
