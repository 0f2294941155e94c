"""GPU parity for the group sizes beyond 128: int3 groups of 256 and 512
(stored as whole 128-code blocks, like group 128) and one group per output
channel (group_size = -1: the whole row) for int4 and int3, through the pack,
every matmul kernel family, the fused gate/up product and the search."""
import numpy as np
import pytest

import datagen
from oracle import awq_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import weight_only_bit_w4a16_amd as awq  # noqa: E402
from tests.test_gpu_parity import assert_rows_close, assert_same_bits, dev, host, say  # noqa: E402
from tests.test_gpu_gate_up import assert_gate_up_close  # noqa: E402

# (bits, group, K): group -1 is the whole row
CASES = [(3, 256, 1024), (3, 512, 2048), (3, -1, 384), (3, -1, 4096), (3, -1, 11008),
         (4, -1, 384), (4, -1, 4096), (4, -1, 11008), (4, -1, 28672)]


def _g(group, K):
    return K if group == -1 else group


@pytest.mark.parametrize("bits,group,K", CASES)
@pytest.mark.parametrize("zero_point", [True, False])
def test_pack(bits, group, K, zero_point):
    say("pack", bits, group, K, zero_point)
    N = 37
    W = datagen.random_f16((N, K), 0.02, seed=K + bits)
    s = datagen.random_f32_positive(K, 0.2, 9.0, seed=K)
    qo, so, zo = O.quantize_pack(W, s, bits, _g(group, K), zero_point)
    q, sc, z = awq.quantize_pack(dev(W), dev(s), bits, group, zero_point=zero_point)
    assert_same_bits(host(q), qo)
    assert_same_bits(host(sc), so)
    assert_same_bits(host(z), zo)


def test_pack_per_channel_without_scale():
    W = datagen.random_f16((5, 1024), 0.02, seed=7)
    W[2] = 0  # an all-zero row: delta 1, zero point 0
    for bits in (3, 4):
        qo, so, zo = O.quantize_pack(W, None, bits, 1024)
        q, sc, z = awq.quantize_pack(dev(W), None, bits, -1)
        assert_same_bits(host(q), qo)
        assert_same_bits(host(sc), so)
        assert_same_bits(host(z), zo)


@pytest.mark.parametrize("bits,group,K", CASES)
@pytest.mark.parametrize("M", [1, 3, 8, 40])
def test_matmul(bits, group, K, M):
    """M = 1 and 3 (int3: decode kernels up to 4 rows), 8 (int4: M <= 16
    decode kernels), 40 (prefill kernel)."""
    say("matmul", bits, group, K, M)
    N = 130
    W = datagen.random_f16((N, K), 0.02, seed=K + 3)
    X = datagen.random_f16((M, K), 1.0, seed=M + K)
    q, sc, z = awq.quantize_pack(dev(W), None, bits, group)
    Y = host(awq.w4a16_matmul(dev(X), q, sc, z, bits, group))
    qo, so, zo = O.quantize_pack(W, None, bits, _g(group, K))
    assert_rows_close(Y, O.matmul(X, qo, so, zo, bits, _g(group, K), K))


@pytest.mark.parametrize("kernel", [awq.KERNEL_DECODE, awq.KERNEL_DECODE_EXACT,
                                    awq.KERNEL_PREFILL])
def test_int4_per_channel_every_kernel(kernel):
    K, N, M = 4096, 70, 5
    W = datagen.random_f16((N, K), 0.02, seed=11)
    X = datagen.random_f16((M, K), 1.0, seed=12)
    q, sc, z = awq.quantize_pack(dev(W), None, 4, -1)
    Y = host(awq.w4a16_matmul(dev(X), q, sc, z, 4, -1, kernel=kernel))
    qo, so, zo = O.quantize_pack(W, None, 4, K)
    assert_rows_close(Y, O.matmul(X, qo, so, zo, 4, K, K))


@pytest.mark.parametrize("bits,group,K", [(3, 256, 1024), (3, -1, 4096), (4, -1, 4096)])
@pytest.mark.parametrize("M", [1, 4, 64])
def test_gate_up(bits, group, K, M):
    N = 96
    Wg = datagen.random_f16((N, K), 0.02, seed=21)
    Wu = datagen.random_f16((N, K), 0.02, seed=22)
    X = datagen.random_f16((M, K), 1.0, seed=23)
    gd = awq.quantize_pack(dev(Wg), None, bits, group)
    ud = awq.quantize_pack(dev(Wu), None, bits, group)
    Y = host(awq.gate_up_silu(dev(X), gd, ud, bits, group))
    g = O.quantize_pack(Wg, None, bits, _g(group, K))
    u = O.quantize_pack(Wu, None, bits, _g(group, K))
    assert_gate_up_close(Y, X, g, u, bits, _g(group, K), K)


@pytest.mark.parametrize("bits,group,K,N,T", [(3, 256, 1024, 64, 64), (3, -1, 1024, 64, 64),
                                              (4, -1, 4096, 1024, 256), (3, -1, 11008, 64, 64)])
@pytest.mark.parametrize("zero_point", [True, False])
def test_search(bits, group, K, N, T, zero_point):
    """hi/lo sizes and one scaled-domain size (T N = 2^18)."""
    say("search", bits, group, K, N, T, zero_point)
    W, Xc, _ = datagen.small_layer(K, N, T, max(1, K // 100), 40.0, seed=K + N)
    s_g, best_g, loss_g = awq.scale_search(dev(W), dev(Xc), datagen.alpha_grid(20), bits, group,
                                           zero_point=zero_point)
    m = O.act_stats(Xc)
    g = _g(group, K)
    for i in range(20):
        lo = O.layer_loss(Xc, W, O.scale_from_stats(m, datagen.alpha_grid(20)[i]), bits, g,
                          zero_point)
        assert abs(loss_g[i] - lo) <= 1e-4 * lo, (i, loss_g[i], lo)
    assert best_g == int(np.argmin(loss_g))
    assert_same_bits(host(s_g), O.scale_from_stats(m, datagen.alpha_grid(20)[best_g]))
