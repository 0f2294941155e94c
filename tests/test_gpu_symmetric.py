"""GPU parity of the symmetric grid (the AwqConfig zero_point=false option):
quantize-and-pack bit-exact against the oracle, the W4A16 / W3A16 product
on symmetric codes (the offset 2^(b-1) goes through the zeros array, so
every matmul kernel applies unchanged), and the alpha search with the
symmetric quantizer inside its loss."""
import numpy as np
import pytest

import datagen
from oracle import awq_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import weight_only_bit_w4a16_amd as awq  # noqa: E402
from tests.test_gpu_parity import (assert_rows_close, assert_same_bits, check_search, dev,  # noqa: E402
                                   host, sample_rows, say, workload_host)


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("N,K,group", [(1, 128, 128), (17, 384, 128), (33, 1024, 256),
                                       (5, 2048, 512), (40, 11008, 128)])
@pytest.mark.parametrize("with_s", [False, True])
def test_symmetric_pack_small(bits, N, K, group, with_s):
    say("symmetric pack", bits, N, K, group, with_s)
    W = datagen.random_f16((N, K), 0.02, seed=N + K + 1)
    s = datagen.random_f32_positive(K, 0.2, 9.0, seed=K + 1) if with_s else None
    qo, so, zo = O.quantize_pack(W, s, bits, group, zero_point=False)
    q, sc, z = awq.quantize_pack(dev(W), dev(s) if with_s else None, bits, group,
                                 zero_point=False)
    torch.cuda.synchronize()
    assert_same_bits(host(q), qo)
    assert_same_bits(host(sc), so)
    assert_same_bits(host(z), zo)


def test_symmetric_pack_degenerate_groups():
    """All-zero, single-signed, exactly representable and max-at-negative
    groups, plus a -0 group (max|W'| = 0 -> delta = 1)."""
    K = 512
    W = np.zeros((5, K), np.float16)
    W[1] = np.linspace(0.1, 0.5, K).astype(np.float16)
    W[2] = -np.linspace(0.1, 0.5, K).astype(np.float16)
    W[3] = ((np.arange(K) % 15 - 7) / 16).astype(np.float16)
    W[4] = np.float16(-0.0)
    for bits in (3, 4):
        qo, so, zo = O.quantize_pack(W, None, bits, 128, zero_point=False)
        q, sc, z = awq.quantize_pack(dev(W), None, bits, 128, zero_point=False)
        assert_same_bits(host(q), qo)
        assert_same_bits(host(sc), so)
        assert_same_bits(host(z), zo)


@pytest.mark.parametrize("name", ["llama7b_attn_4096x4096_int4", "llama7b_mlp_up_4096x11008_int3",
                                  "llama70b_mlp_8192x28672_int4"])
def test_symmetric_pack_workload(name):
    w = datagen.WORKLOADS[name]
    say("symmetric pack workload", name)
    W, Xc = workload_host(name)
    s = O.scale_from_stats(O.act_stats(Xc), 0.5)
    q, sc, z = awq.quantize_pack(dev(W), dev(s), w.bits, w.group, zero_point=False)
    rows = sample_rows(w.N)
    qo, so, zo = O.quantize_pack(W[rows], s, w.bits, w.group, zero_point=False)
    assert_same_bits(host(q)[rows], qo)
    assert_same_bits(host(sc)[rows], so)
    assert_same_bits(host(z)[rows], zo)


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("M", [1, 3, 16, 100])
def test_symmetric_matmul(bits, M):
    """Every kernel family on symmetric codes: M = 1 and 3 run the decode
    kernels (int3 only up to 4 rows), 16 and 100 the decode/prefill ones."""
    N, K = 257, 4096
    say("symmetric matmul", bits, M)
    W = datagen.random_f16((N, K), 0.02, seed=91 + bits)
    s = datagen.random_f32_positive(K, 0.3, 5.0, seed=92)
    X = datagen.random_f16((M, K), 1.0, seed=93 + M)
    q, sc, z = awq.quantize_pack(dev(W), dev(s), bits, 128, zero_point=False)
    Y = host(awq.w4a16_matmul(awq.fold_inv_scale(dev(X), dev(s)), q, sc, z, bits, 128))
    qo, so, zo = O.quantize_pack(W, s, bits, 128, zero_point=False)
    Yo = O.matmul(O.fold_inv_scale(X, s), qo, so, zo, bits, 128, K)
    assert_rows_close(Y, Yo)


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("N,K,T", [(64, 512, 64), (130, 1024, 100), (1024, 1024, 256)])
def test_symmetric_search_small(bits, N, K, T):
    """(64, 512, 64) and (130, 1024, 100) run the hi/lo contraction,
    (1024, 1024, 256) the scaled one."""
    say("symmetric search", bits, N, K, T)
    W, Xc, _ = datagen.small_layer(K, N, T, max(1, K // 100), 40.0, seed=N + K + T + 3)
    check_search(W, Xc, datagen.alpha_grid(20), bits, 128, zero_point=False)


def test_symmetric_search_workload_sampled():
    """Full grid on a 4096 x 4096 layer (scaled path); the oracle recomputes
    alpha = 0, the device's argmin and the last grid point."""
    w = datagen.WORKLOADS["llama7b_attn_4096x4096_int4"]
    say("symmetric search workload", w.name)
    W, Xc = workload_host(w.name)
    check_search(W, Xc, datagen.alpha_grid(w.n_alpha), w.bits, w.group,
                 oracle_idx=[0, w.n_alpha - 1], zero_point=False)
