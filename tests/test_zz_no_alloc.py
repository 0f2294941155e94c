"""The allocation-free product (awq_w4a16_matmul_noalloc), called through
the C ABI, against the product with a caller workspace
(awq_w4a16_matmul_ws): the same kernels and split plan, so the same bits.
Two calls in a row on one GPU, the second on a smaller problem (the scratch
keeps the first call's contents), for shapes that split K (int4 and int3),
a shape that does not, an M = 1 decode shape and decode shapes that split K."""
import ctypes

import numpy as np
import pytest

import datagen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import weight_only_bit_w4a16_amd as awq  # noqa: E402
from weight_only_bit_w4a16_amd import _lib  # noqa: E402


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _layer(N, K, bits, seed):
    W = torch.from_numpy(datagen.random_f16((N, K), 0.02, seed=seed)).cuda()
    s = torch.from_numpy(datagen.random_f32_positive(K, 0.3, 4.0, seed=seed + 1)).cuda()
    return awq.quantize_pack(W, s, bits, 128)


def _noalloc(X, q, sc, z, bits):
    M, K = X.shape
    N = q.shape[0]
    Y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    r = awq.lib().awq_w4a16_matmul_noalloc(_p(X), _p(q), _p(sc), _p(z), M, N, K, bits, 128,
                                          _p(Y), _stream())
    assert r == _lib.AWQ_OK, _lib.STATUS.get(r, r)
    return Y


def _with_workspace(X, q, sc, z, bits):
    M, K = X.shape
    N = q.shape[0]
    nb = awq.matmul_workspace_bytes(M, N, K, bits, 128)
    ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda") if nb else None
    Y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    r = awq.lib().awq_w4a16_matmul_ws(_p(X), _p(q), _p(sc), _p(z), M, N, K, bits, 128, _p(Y),
                                     _p(ws), nb, _stream())
    assert r == _lib.AWQ_OK, _lib.STATUS.get(r, r)
    return Y


# (M, N, K, bits) first call, then a smaller second call
PAIRS = [
    ((17, 4096, 4096, 4), (9, 1500, 4096, 4)),       # split K both times, 32-row tiles
    ((256, 4096, 11008, 4), (64, 2048, 8192, 4)),    # split K, 128- and 64-row tiles
    ((2048, 256, 4096, 4), (100, 256, 4096, 4)),     # the largest plan (16 MiB), then a small one
    ((33, 3000, 4096, 3), (20, 1000, 4096, 3)),      # int3 split K
    ((300, 2048, 2048, 4), (40, 700, 1024, 4)),      # no split
    ((1, 4096, 4096, 4), (1, 1024, 2048, 4)),        # decode
    ((16, 4096, 11008, 4), (8, 2000, 16384, 4)),     # decode split K, 16 then 8 token rows
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_workspace_product(first, second):
    for i, (M, N, K, bits) in enumerate((first, second)):
        print("noalloc", i, M, N, K, bits, flush=True)
        q, sc, z = _layer(N, K, bits, seed=N + K + i)
        X = torch.from_numpy(datagen.random_f16((M, K), 1.0, seed=M + i)).cuda()
        nb = awq.matmul_workspace_bytes(M, N, K, bits, 128)
        Y0 = _noalloc(X, q, sc, z, bits)
        Y1 = _with_workspace(X, q, sc, z, bits)
        torch.cuda.synchronize()
        assert torch.isfinite(Y0.float()).all()
        assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16)), (i, nb)


def test_noalloc_refuses_bad_arguments():
    h = awq.lib()
    X = torch.zeros((17, 4096), dtype=torch.float16, device="cuda")
    q, sc, z = _layer(4096, 4096, 4, seed=5)
    Y = torch.empty((17, 4096), dtype=torch.float16, device="cuda")
    st = _stream()
    assert h.awq_w4a16_matmul_noalloc(None, _p(q), _p(sc), _p(z), 17, 4096, 4096, 4, 128,
                                      _p(Y), st) == _lib.AWQ_ERR_INVALID_ARG
    assert h.awq_w4a16_matmul_noalloc(_p(X), _p(q), _p(sc), _p(z), 17, 4096, 4096, 5, 128,
                                      _p(Y), st) == _lib.AWQ_ERR_UNSUPPORTED
