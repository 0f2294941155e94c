"""Quantization steps below fp16's normal range (delta < 2^-14).

A group's step is its range over 2^b - 1 (AWQ Explained: Protecting the
Weights That Matter Most -- "Scaling instead of mixed precision"); with
small weights, or channels whose activation statistic is small at a large
alpha (s = mean|x|^alpha), W diag(s) and so delta fall far below 2^-14, where
fp16 has only a few significant bits left (and nothing below 2^-25). The
decode kernels apply delta in float32; the prefill kernels dequantize to
fp16 and scale each weight row by a power of two taken from its largest
step, so those rows keep fp16's full precision. Every product kernel is
checked here on such layers within the matmul contract per token row,
applied also to each class of output channels of the layers that mix large
and tiny weight rows.
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

# large activations, as X' = X / s is where s is small; they also keep the
# outputs in fp16's normal range
X_STD = 1000.0

def assert_class_rows_close(Yg, Yref, mixed):
    """The matmul contract per token row, over all outputs and, for layers
    whose weight rows alternate between two magnitudes, over each class of
    output channels by itself (a class of tiny rows would pass the check
    over all outputs whatever its error)."""
    assert_rows_close(Yg, Yref)
    if mixed:
        assert_rows_close(Yg[:, 0::2], Yref[:, 0::2])
        assert_rows_close(Yg[:, 1::2], Yref[:, 1::2])


def small_layer(N, K, seed, scale_lo, scale_hi, mixed_rows=False):
    """W ~ N(0, 0.02), s uniform in [scale_lo, scale_hi] (so W' = W s and
    the steps are tiny); with mixed_rows, every other row of W is 1e4 times
    larger, so neighbouring rows take different power-of-two exponents."""
    W = datagen.random_f16((N, K), 0.02, seed=seed)
    if mixed_rows:
        W = W.astype(np.float32)
        W[::2] *= 1e4
        W = W.astype(np.float16)
    s = datagen.random_f32_positive(K, scale_lo, scale_hi, seed=seed + 1)
    return W, s


@pytest.mark.parametrize("scale", [1e-3, 1e-5, 1e-7])
def test_steps_are_below_fp16_normal(scale):
    """The layers used below really have subnormal (or zero) fp16 steps."""
    W, s = small_layer(64, 1024, 3, scale, 2 * scale)
    _, so, _ = O.quantize_pack(W, s, 4, 128)
    assert so.max() < 2.0 ** -14
    if scale <= 1e-5:
        assert np.all(so.astype(np.float16).astype(np.float32) != so)


CASES = [
    # bits, M, N, K, kernel, mixed rows
    (4, 300, 700, 2048, awq.KERNEL_PREFILL, False),   # 128 x 128 tiles
    (4, 40, 130, 1024, awq.KERNEL_PREFILL, False),    # 64 x 64 tiles
    (4, 2048, 1100, 512, awq.KERNEL_AUTO, False),     # 256 x 256 rounds and the 128 x 256 tail
    (4, 300, 700, 2048, awq.KERNEL_PREFILL, True),
    (3, 300, 700, 2048, awq.KERNEL_PREFILL, False),
    (3, 40, 130, 1024, awq.KERNEL_PREFILL, True),
    (4, 17, 4096, 4096, awq.KERNEL_AUTO, False),      # split K
    (3, 33, 3000, 4096, awq.KERNEL_AUTO, True),       # split K
    (4, 1, 3000, 4096, awq.KERNEL_AUTO, True),        # decode kernels
    (4, 8, 3000, 4096, awq.KERNEL_AUTO, False),
    (3, 1, 3000, 4096, awq.KERNEL_AUTO, False),
    (3, 3, 3000, 4096, awq.KERNEL_AUTO, True),
]


@pytest.mark.parametrize("scale", [1e-5, 1e-7])
@pytest.mark.parametrize("bits,M,N,K,kernel,mixed", CASES)
def test_small_step_product(bits, M, N, K, kernel, mixed, scale):
    say("small steps", bits, M, N, K, kernel, mixed, scale)
    W, s = small_layer(N, K, seed=N + K + bits, scale_lo=scale, scale_hi=4 * scale,
                       mixed_rows=mixed)
    X = datagen.random_f16((M, K), X_STD, seed=M + 5)
    qo, so, zo = O.quantize_pack(W, s, bits, 128)
    q, sc, z = awq.quantize_pack(dev(W), dev(s), bits, 128)
    assert_same_bits(host(sc), so)
    if kernel == awq.KERNEL_AUTO and awq.matmul_workspace_bytes(M, N, K, bits, 128) > 0:
        say("  (split K)")
    Y = host(awq.w4a16_matmul(dev(X), q, sc, z, bits, 128, kernel=kernel))
    assert_class_rows_close(Y, O.matmul(X, qo, so, zo, bits, 128, K), mixed)


@pytest.mark.parametrize("bits,M", [(4, 1), (4, 40), (4, 300), (3, 1), (3, 40)])
def test_small_step_gate_up(bits, M):
    N, K = 700, 2048
    say("small steps gate/up", bits, M)
    Wg, s = small_layer(N, K, seed=71, scale_lo=1e-6, scale_hi=1e-5)
    Wu = datagen.random_f16((N, K), 0.02, seed=72)
    X = datagen.random_f16((M, K), X_STD, seed=73)
    g = O.quantize_pack(Wg, s, bits, 128)
    u = O.quantize_pack(Wu, s, bits, 128)
    d3 = lambda t: (dev(t[0].view(np.int32)), dev(t[1]), dev(t[2]))  # noqa: E731
    Y = host(awq.gate_up_silu(dev(X), d3(g), d3(u), bits, 128))
    assert_gate_up_close(Y, X, g, u, bits, 128, K)


@pytest.mark.parametrize("bits,M,kernel", [(4, 40, awq.KERNEL_AUTO), (4, 300, awq.KERNEL_PREFILL),
                                           (3, 40, awq.KERNEL_PREFILL), (4, 1, awq.KERNEL_AUTO),
                                           (4, 8, awq.KERNEL_AUTO), (3, 1, awq.KERNEL_AUTO)])
def test_small_step_compact(bits, M, kernel):
    """Compact storage keeps the steps in fp16, so a tiny step is stored
    with fp16's subnormal precision; the product must still be exact to the
    stored steps (the oracle uses the same fp16 values)."""
    N, K = 700, 2048
    say("small steps compact", bits, M, kernel)
    W, s = small_layer(N, K, seed=81, scale_lo=1e-5, scale_hi=4e-5, mixed_rows=True)
    X = datagen.random_f16((M, K), X_STD, seed=82)
    q, sc, z = awq.quantize_pack(dev(W), dev(s), bits, 128)
    s16, z4 = awq.compact_group_params(sc, z, K, 128)
    Y = host(awq.w4a16_matmul_compact(dev(X), q, s16, z4, bits, 128, kernel=kernel))
    qo, so, zo = O.quantize_pack(W, s, bits, 128)
    s16o, z4o = O.compact_group_params(so, zo)
    assert_class_rows_close(Y, O.matmul_compact(X, qo, s16o, z4o, bits, 128, K), True)


def test_ordinary_rows_unchanged_bits():
    """The power-of-two row exponent is exact for ordinary steps: a product
    repeated with the weights' rows permuted gives each row's outputs with
    the same bits (rows take different exponents, and no output depends on
    the neighbouring rows' exponents)."""
    M, N, K = 300, 512, 2048
    W = datagen.random_f16((N, K), 0.02, seed=91)
    W = (W.astype(np.float32) * np.where(np.arange(N) % 3 == 0, 8.0, 1.0)[:, None]).astype(np.float16)
    X = datagen.random_f16((M, K), 1.0, seed=92)
    q, sc, z = awq.quantize_pack(dev(W), None, 4, 128)
    Y = host(awq.w4a16_matmul(dev(X), q, sc, z, kernel=awq.KERNEL_PREFILL))
    perm = np.random.default_rng(5).permutation(N)
    qp, scp, zp = awq.quantize_pack(dev(np.ascontiguousarray(W[perm])), None, 4, 128)
    Yp = host(awq.w4a16_matmul(dev(X), qp, scp, zp, kernel=awq.KERNEL_PREFILL))
    assert_same_bits(Yp, np.ascontiguousarray(Y[:, perm]))
