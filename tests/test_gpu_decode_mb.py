"""GPU parity of the int4 decode kernel for 2 <= M <= 16 on 16-row blocks
(activations staged in LDS, K split over workgroups into float32 planes of
the workspace, added in split order by the split that finishes a row block
last), which the automatic choice takes for rows of more than 8192 codes:
the cases its plan and its loop have to get right, against the CPU oracle's
float64 product over the same dequantized weights (per output row m:
max_n |Y - Y*| <= 1e-3 * max_n |Y*|).

- several row blocks per wavefront (N = 22007: 1376 row blocks in 3 splits
  of 22 chunks, 2 row blocks per wavefront, the last block partial);
- K splits whose last split is shorter and whose chunk counts are not a
  multiple of the weight ring (K = 11008: 86 chunks in 8 splits of 11);
- 8 and 16 stored token rows, M from 2 to 16;
- groups of 256 and 512 codes and one group per row;
- the same shape without a workspace (the multi-pass kernel) and with one,
  and two calls with one workspace giving the same bits (the first call
  leaves the workspace's counters zero for the second);
- both weight-load forms: rows of 28672 codes on 8192 rows (the full-line
  form's staging would add K splits there, so the plan keeps the 16-row
  loads; at M = 16 with one workgroup per compute unit and the wide LDS)
  and the shapes above (full-line loads through LDS).
"""
import ctypes
import sys

import numpy as np
import pytest

import datagen
from oracle import awq_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import weight_only_bit_w4a16_amd as awq  # noqa: E402
from weight_only_bit_w4a16_amd import _lib  # noqa: E402

TOL = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.cpu().numpy()


def assert_rows_close(Yg, Yref, tol=TOL):
    Yg = np.asarray(Yg, dtype=np.float64)
    assert Yg.shape == Yref.shape
    assert np.all(np.isfinite(Yg))
    for m in range(Yref.shape[0]):
        scale = np.abs(Yref[m]).max()
        err = np.abs(Yg[m] - Yref[m]).max()
        assert err <= tol * scale, (m, err / scale)


def rows_of(N, seed=0, count=200):
    g = np.random.default_rng(seed)
    r = set(range(min(N, 48))) | set(range(max(0, N - 40), N)) | \
        set(g.choice(N, size=min(count, N), replace=False).tolist())
    return np.array(sorted(r))


def check(W, X, s, group, Y, rows=None):
    """Y [M, N] (host) against the oracle on all rows, or on `rows`."""
    K = W.shape[1]
    if rows is None:
        qo, so, zo = O.quantize_pack(W, s, 4, group)
        assert_rows_close(Y, O.matmul(X, qo, so, zo, 4, group, K))
    else:
        qo, so, zo = O.quantize_pack(W[rows], s, 4, group)
        assert_rows_close(Y[:, rows], O.matmul(X, qo, so, zo, 4, group, K))


def packed(W, s, group):
    return awq.quantize_pack(dev(W), dev(s) if s is not None else None, 4, group)


def test_mb_several_row_blocks_per_wavefront():
    N, K, M = 22007, 8320, 5
    say("mb several row blocks", M, N, K)
    assert awq.matmul_workspace_bytes(M, N, K, 4, 128) == (64 << 10) + 3 * M * N * 4
    W = datagen.random_f16((N, K), 0.02, seed=11)
    X = datagen.random_f16((M, K), 1.0, seed=12)
    q, sc, z = packed(W, None, 128)
    Y = host(awq.w4a16_matmul(dev(X), q, sc, z))
    check(W, X, None, 128, Y, rows_of(N, seed=1, count=400))


@pytest.mark.parametrize("M", [8, 16])
def test_mb_uneven_splits(M):
    N, K = 4100, 11008
    say("mb uneven splits", M, N, K)
    assert awq.matmul_workspace_bytes(M, N, K, 4, 128) > 0
    W = datagen.random_f16((N, K), 0.02, seed=M)
    s = datagen.random_f32_positive(K, 0.3, 4.0, seed=M + 1)
    X = datagen.random_f16((M, K), 1.0, seed=M + 2)
    q, sc, z = packed(W, s, 128)
    Y = host(awq.w4a16_matmul(dev(X), q, sc, z))
    check(W, X, s, 128, Y, rows_of(N, seed=M))


@pytest.mark.parametrize("M", [2, 3, 4, 6, 7, 9, 12, 15, 16])
def test_mb_token_rows(M):
    """16384 codes per row (128 chunks): M = 2 .. 4 too run on this kernel
    at this length."""
    N, K = 333, 16384
    say("mb token rows", M, N, K)
    W = datagen.random_f16((N, K), 0.02, seed=100 + M)
    X = datagen.random_f16((M, K), 1.0, seed=200 + M)
    q, sc, z = packed(W, None, 128)
    Y = host(awq.w4a16_matmul(dev(X), q, sc, z))
    check(W, X, None, 128, Y)


@pytest.mark.parametrize("group", [256, 512, -1])
@pytest.mark.parametrize("M", [5, 9])
def test_mb_groups(group, M):
    N, K = 200, 8704
    say("mb groups", group, M)
    W = datagen.random_f16((N, K), 0.02, seed=group % 1000 + M)
    X = datagen.random_f16((M, K), 1.0, seed=M)
    q, sc, z = packed(W, None, group)
    Y = host(awq.w4a16_matmul(dev(X), q, sc, z, 4, group))
    check(W, X, None, K if group == -1 else group, Y)


def _c(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def test_mb_with_and_without_workspace():
    """Without a workspace the shape runs on the multi-pass kernel (within
    the same contract); with one, two calls give the same bits, and a
    workspace one byte short is refused."""
    M, N, K = 16, 4096, 11008
    say("mb with and without workspace")
    W = datagen.random_f16((N, K), 0.02, seed=5)
    X = datagen.random_f16((M, K), 1.0, seed=6)
    q, sc, z = packed(W, None, 128)
    Xd = dev(X)
    nb = awq.matmul_workspace_bytes(M, N, K, 4, 128)
    assert nb == (64 << 10) + 8 * M * N * 4  # counters, then 8 planes (splits of 11 chunks)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    h = awq.lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = []
    for w, n in [(ws, nb), (ws, nb), (None, 0)]:
        y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        r = h.awq_w4a16_matmul_ws(_c(Xd), _c(q), _c(sc), _c(z), M, N, K, 4, 128, _c(y), _c(w), n,
                                  st)
        assert r == _lib.AWQ_OK, _lib.STATUS.get(r, r)
        out.append(host(y))
    r = h.awq_w4a16_matmul_ws(_c(Xd), _c(q), _c(sc), _c(z), M, N, K, 4, 128, _c(y), _c(ws),
                              nb - 1, st)
    assert r == _lib.AWQ_ERR_WORKSPACE
    assert np.array_equal(out[0].view(np.uint16), out[1].view(np.uint16))
    check(W, X, None, 128, out[0])
    check(W, X, None, 128, out[2])


@pytest.mark.parametrize("M", [8, 16])
def test_mb_long_rows_plain_loads(M):
    """28672 codes per row, 8192 rows: the plan keeps the 16-row loads here,
    and at M = 16 takes one workgroup per compute unit with the wide LDS
    (8 splits instead of 14; sampled rows against the oracle)."""
    N, K = 8192, 28672
    say("mb long rows", M, N, K)
    W = datagen.random_f16((N, K), 0.02, seed=31)
    X = datagen.random_f16((M, K), 1.0, seed=32)
    q, sc, z = packed(W, None, 128)
    Y = host(awq.w4a16_matmul(dev(X), q, sc, z))
    check(W, X, None, 128, Y, rows_of(N, seed=3, count=120))
