"""GPU parity of the compact group parameters (fp16 steps, 4-bit zero points
8 per word): the conversion bit-exact against the oracle, and every product
kernel over them within the matmul contract against the oracle's product
with the same fp16 steps."""
import numpy as np
import pytest

import datagen
from oracle import awq_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import weight_only_bit_w4a16_amd as awq  # noqa: E402
from tests.test_gpu_parity import assert_rows_close, assert_same_bits, dev, host, say  # noqa: E402


def _g(group, K):
    return K if group == -1 else group


@pytest.mark.parametrize("bits,group,K", [(4, 128, 1024), (4, 256, 3072), (3, 128, 640),
                                          (3, 512, 2048), (4, -1, 4096), (3, -1, 384)])
def test_compact_params_exact(bits, group, K):
    N = 37
    W = datagen.random_f16((N, K), 0.02, seed=K + bits)
    q, sc, z = awq.quantize_pack(dev(W), None, bits, group)
    s16, z4 = awq.compact_group_params(sc, z, K, group)
    so, zo = O.compact_group_params(host(sc), host(z))
    assert_same_bits(host(s16), so)
    assert_same_bits(host(z4), zo)


CASES = [(4, 128, 4096, 300), (4, 256, 2048, 130), (4, -1, 4096, 130), (3, 128, 4096, 130),
         (3, -1, 11008, 64), (4, 128, 11008, 64), (4, 128, 28672, 40), (3, 128, 28672, 40)]


@pytest.mark.parametrize("bits,group,K,N", CASES)
@pytest.mark.parametrize("M,kernel", [(1, awq.KERNEL_AUTO), (2, awq.KERNEL_AUTO), (3, awq.KERNEL_AUTO),
                                      (8, awq.KERNEL_AUTO), (40, awq.KERNEL_AUTO),
                                      (5, awq.KERNEL_DECODE_EXACT), (2, awq.KERNEL_DECODE),
                                      (16, awq.KERNEL_PREFILL)])
def test_compact_product(bits, group, K, N, M, kernel):
    if kernel == awq.KERNEL_DECODE_EXACT and bits == 3:
        pytest.skip("the exact-dequant decode kernel is int4 only")
    if kernel == awq.KERNEL_DECODE and bits == 3 and K > 4096:
        pytest.skip("the int3 decode kernel for 2-4 rows holds K up to about 8000 in LDS")
    say("compact product", bits, group, K, N, M, kernel)
    W = datagen.random_f16((N, K), 0.02, seed=K + N)
    s = datagen.random_f32_positive(K, 0.3, 4.0, seed=K)
    X = datagen.random_f16((M, K), 1.0, seed=M)
    q, sc, z = awq.quantize_pack(dev(W), dev(s), bits, group)
    s16, z4 = awq.compact_group_params(sc, z, K, group)
    Y = host(awq.w4a16_matmul_compact(dev(X), q, s16, z4, bits, group, kernel=kernel))
    qo, so, zo = O.quantize_pack(W, s, bits, _g(group, K))
    s16o, z4o = O.compact_group_params(so, zo)
    assert_rows_close(Y, O.matmul_compact(X, qo, s16o, z4o, bits, _g(group, K), K))


def test_compact_decode_workload():
    """The 8192 x 28672 layer at M = 1 and 4 (every row checked at M = 1 on
    256 sampled rows)."""
    w = datagen.WORKLOADS["llama70b_mlp_8192x28672_int4"]
    say("compact workload")
    W = datagen.weight(w)
    q, sc, z = awq.quantize_pack(dev(W), None, 4, 128)
    s16, z4 = awq.compact_group_params(sc, z, w.K, 128)
    rows = np.sort(np.random.default_rng(3).choice(w.N, 256, replace=False))
    qo, so, zo = O.quantize_pack(W[rows], None, 4, 128)
    s16o, z4o = O.compact_group_params(so, zo)
    for M in (1, 4):
        X = datagen.decode_input(w, M)
        Y = host(awq.w4a16_matmul_compact(dev(X), q, s16, z4, 4, 128))
        assert_rows_close(Y[:, rows], O.matmul_compact(X, qo, s16o, z4o, 4, 128, w.K))
