"""Row assignment of the streaming decode kernels (one row per wavefront at a
time): when the grid is a multiple of 8 workgroups, XCD x takes the
contiguous eighth x of the rows; otherwise every wavefront interleaves over
all rows. Every output row is checked against the oracle (the product within
1e-3 of each token row's largest output) at row counts that put the
assignment at its edges, on 128-code rows (one piece):

- 200704 rows: 784 workgroups on 256 compute units, every wavefront exactly
  64 rows (the most a wavefront holds) in the XCD form;
- 32 rows: 8 workgroups, one per XCD, one row per wavefront;
- 36 and 1000 rows: 9 and 250 workgroups, the interleaved form.
The same shapes run through the gated gate/up form (M = 1) and, for int3,
the few-token kernel at M = 2.
"""
import numpy as np
import pytest

import datagen
from oracle import awq_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import weight_only_bit_w4a16_amd as awq  # noqa: E402
from tests.test_gpu_gate_up import assert_gate_up_close  # noqa: E402
from tests.test_gpu_parity import assert_rows_close, dev, host, say  # noqa: E402

K = 128
ROWS = [200704, 32, 36, 1000]


def _packed(W, bits):
    q, sc, z = O.quantize_pack(W, None, bits, 128)
    return (q, sc, z), (dev(q.view(np.int32)), dev(sc), dev(z))


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("N", ROWS)
def test_decode_m1_rows(bits, N):
    say("decode M=1 rows", bits, N)
    W = datagen.random_f16((N, K), 0.02, seed=N + bits)
    X = datagen.random_f16((1, K), 1.0, seed=N + 7)
    (qo, so, zo), (q, sc, z) = _packed(W, bits)
    Y = host(awq.w4a16_matmul(dev(X), q, sc, z, bits, 128))
    assert_rows_close(Y, O.matmul(X, qo, so, zo, bits, 128, K))


@pytest.mark.parametrize("N", ROWS)
def test_gate_up_m1_rows(N):
    say("gate/up M=1 rows", N)
    Wg = datagen.random_f16((N, K), 0.02, seed=N + 11)
    Wu = datagen.random_f16((N, K), 0.02, seed=N + 12)
    X = datagen.random_f16((1, K), 1.0, seed=N + 13)
    g, gd = _packed(Wg, 4)
    u, ud = _packed(Wu, 4)
    Y = host(awq.gate_up_silu(dev(X), gd, ud, 4, 128))
    assert_gate_up_close(Y, X, g, u, 4, 128, K)


@pytest.mark.parametrize("N", ROWS)
def test_int3_m2_rows(N):
    say("int3 M=2 rows", N)
    W = datagen.random_f16((N, K), 0.02, seed=N + 21)
    X = datagen.random_f16((2, K), 1.0, seed=N + 22)
    (qo, so, zo), (q, sc, z) = _packed(W, 3)
    Y = host(awq.w4a16_matmul(dev(X), q, sc, z, 3, 128))
    assert_rows_close(Y, O.matmul(X, qo, so, zo, 3, 128, K))
