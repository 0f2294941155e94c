"""The binding refuses malformed tensors before calling the library: wrong
output shape, dtype or contiguity, a scale vector of the wrong length, a
host tensor among device operands. (Each of these would otherwise become an
out-of-bounds device read or write.)"""
import numpy as np
import pytest

import datagen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import weight_only_bit_w4a16_amd as awq  # noqa: E402
from tests.test_gpu_parity import dev  # noqa: E402


@pytest.fixture(scope="module")
def layer():
    N, K = 64, 512
    W = dev(datagen.random_f16((N, K), 0.02, seed=1))
    s = dev(datagen.random_f32_positive(K, 0.5, 2.0, seed=2))
    X = dev(datagen.random_f16((3, K), 1.0, seed=3))
    q, sc, z = awq.quantize_pack(W, s)
    return N, K, W, s, X, q, sc, z


def test_matmul_out_checked(layer):
    N, K, W, s, X, q, sc, z = layer
    with pytest.raises(ValueError):
        awq.w4a16_matmul(X, q, sc, z, out=torch.empty((3, N - 1), dtype=torch.float16,
                                                        device="cuda"))
    with pytest.raises(TypeError):
        awq.w4a16_matmul(X, q, sc, z, out=torch.empty((3, N), dtype=torch.float32,
                                                        device="cuda"))
    with pytest.raises(ValueError):
        awq.w4a16_matmul(X, q, sc, z, out=torch.empty((N, 3), dtype=torch.float16,
                                                        device="cuda").t())
    y = torch.empty((3, N), dtype=torch.float16, device="cuda")
    assert awq.w4a16_matmul(X, q, sc, z, out=y) is y


def test_pack_out_checked(layer):
    N, K, W, s, X, q, sc, z = layer
    with pytest.raises(ValueError):
        awq.quantize_pack(W, s, out=(q[:-1], sc, z))
    with pytest.raises(TypeError):
        awq.quantize_pack(W, s, out=(q, sc.double(), z))
    with pytest.raises(ValueError):
        awq.quantize_pack(W, s[:-1])
    q2, sc2, z2 = torch.empty_like(q), torch.empty_like(sc), torch.empty_like(z)
    awq.quantize_pack(W, s, out=(q2, sc2, z2))
    assert torch.equal(q2, q) and torch.equal(sc2, sc) and torch.equal(z2, z)


def test_fold_checks_scale_length(layer):
    N, K, W, s, X, q, sc, z = layer
    with pytest.raises(ValueError):
        awq.fold_inv_scale(X, s[: K // 2])
    with pytest.raises(ValueError):
        awq.fold_inv_scale(X, s, out=torch.empty((3, K + 8), dtype=torch.float16, device="cuda"))


def test_host_operand_refused(layer):
    N, K, W, s, X, q, sc, z = layer
    with pytest.raises(ValueError):
        awq.w4a16_matmul(X, q, sc.cpu(), z)
    with pytest.raises(ValueError):
        awq.fold_inv_scale(X, s.cpu())


def test_gate_up_and_norm_out_checked(layer):
    N, K, W, s, X, q, sc, z = layer
    with pytest.raises(ValueError):
        awq.gate_up_silu(X, (q, sc, z), (q, sc, z),
                         out=torch.empty((3, N + 1), dtype=torch.float16, device="cuda"))
    gamma = dev(np.ones(K, np.float16))
    with pytest.raises(ValueError):
        awq.rmsnorm(X, gamma, out=torch.empty((2, K), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        awq.fold_norm_weight(gamma, s, out=torch.empty(K - 8, dtype=torch.float16, device="cuda"))
