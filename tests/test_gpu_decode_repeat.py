"""M = 1 decode on rows of 3 to 6 pieces, the shapes where the decode kernels
prepare their activation operands after the first weight loads, checked on
every output against the oracle and repeated bit for bit.

These kernels unpack codes with one AND-OR per pair and feed the result
straight to the matrix cores; gfx950 needs two wait states between a vector
write and an MFMA read of the same register. A write the compiler cannot see
(inline asm) gets none, and an MFMA issued right behind it can read the
register's previous value, which depends on how the wavefronts of a SIMD
interleave: wrong sums that change from call to call. Each case below is run
several times on the same inputs; every call must give the same bits and
match the oracle (the product within 1e-3 of each row's largest output,
HH "Why the engine is part of the method": the packed weights must be
unpacked, dequantized and multiplied efficiently, and here correctly).
"""
import numpy as np
import pytest

import datagen
from oracle import awq_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import weight_only_bit_w4a16_amd as awq  # noqa: E402
from tests.test_gpu_gate_up import assert_gate_up_close  # noqa: E402
from tests.test_gpu_parity import assert_rows_close, assert_same_bits, dev, host, say  # noqa: E402

REPEATS = 5
N_ROWS = 6007  # several rows per wavefront, and a ragged last round


def _packed(W, s, bits):
    q, sc, z = O.quantize_pack(W, s, bits, 128)
    return (q, sc, z), (dev(q.view(np.int32)), dev(sc), dev(z))


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("K", [6144, 8192, 11008])
def test_decode_m1_repeat(bits, K):
    say("decode M=1 repeat", bits, K)
    W = datagen.random_f16((N_ROWS, K), 0.02, seed=K + bits)
    s = datagen.random_f32_positive(K, 0.3, 4.0, seed=K + 21)
    X = datagen.random_f16((1, K), 1.0, seed=K + 22)
    (qo, so, zo), (q, sc, z) = _packed(W, s, bits)
    Xd = dev(X)
    Y = host(awq.w4a16_matmul(Xd, q, sc, z, bits, 128))
    assert_rows_close(Y, O.matmul(X, qo, so, zo, bits, 128, K))
    for _ in range(REPEATS - 1):
        assert_same_bits(host(awq.w4a16_matmul(Xd, q, sc, z, bits, 128)), Y)


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("K", [6144, 8192, 11008])
def test_gate_up_m1_repeat(bits, K):
    say("gate/up M=1 repeat", bits, K)
    Wg = datagen.random_f16((N_ROWS, K), 0.02, seed=K + 31)
    Wu = datagen.random_f16((N_ROWS, K), 0.02, seed=K + 32)
    s = datagen.random_f32_positive(K, 0.3, 4.0, seed=K + 33)
    X = datagen.random_f16((1, K), 1.0, seed=K + 34)
    g, gd = _packed(Wg, s, bits)
    u, ud = _packed(Wu, s, bits)
    Xd = dev(X)
    Y = host(awq.gate_up_silu(Xd, gd, ud, bits, 128))
    assert_gate_up_close(Y, X, g, u, bits, 128, K)
    for _ in range(REPEATS - 1):
        assert_same_bits(host(awq.gate_up_silu(Xd, gd, ud, bits, 128)), Y)


@pytest.mark.parametrize("M", [2, 3, 4])
def test_int3_few_token_late_form_shape(M):
    """The int3 few-token kernel at two wavefronts per row with two pieces
    each (K = 8192): every token row matches and repeats bit for bit."""
    K, N = 8192, 3001
    say("int3 few-token repeat", M)
    W = datagen.random_f16((N, K), 0.02, seed=M + 41)
    X = datagen.random_f16((M, K), 1.0, seed=M + 42)
    (qo, so, zo), (q, sc, z) = _packed(W, None, 3)
    Xd = dev(X)
    Y = host(awq.w4a16_matmul(Xd, q, sc, z, 3, 128))
    assert_rows_close(Y, O.matmul(X, qo, so, zo, 3, 128, K))
    for _ in range(REPEATS - 1):
        assert_same_bits(host(awq.w4a16_matmul(Xd, q, sc, z, 3, 128)), Y)
