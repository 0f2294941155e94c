"""C-ABI checks that run without a GPU: the library loads, exports every
symbol include/awq.h declares, and rejects bad arguments before any HIP
call. With no device visible, valid requests return AWQ_ERR_NO_DEVICE."""
import ctypes
import os
import re

import numpy as np
import pytest

from tests.conftest import ROOT
from oracle import awq_oracle as O
import weight_only_bit_w4a16_amd as awq
from weight_only_bit_w4a16_amd import _lib

HEADER = os.path.join(ROOT, "include", "awq.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(awq_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    h = awq.lib()
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(h, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_status_strings_and_version():
    h = awq.lib()
    for code, name in _lib.STATUS.items():
        assert h.awq_status_string(code).decode() == name
    assert h.awq_status_string(99).decode() == "AWQ_ERR_UNKNOWN"
    assert h.awq_version() == 101


@pytest.mark.parametrize("K,bits,group", [(128, 4, 128), (4096, 4, 128), (8192, 4, 128),
                                          (11008, 4, 128), (512, 3, 128), (4096, 3, 128),
                                          (11008, 3, 128), (4096, 4, 256), (4096, 3, 512),
                                          (1024, 3, 256)])
def test_words_per_row_matches_layout(K, bits, group):
    assert awq.packed_words_per_row(K, bits, group) == O.words_per_row(K, bits, group)


@pytest.mark.parametrize("K,bits", [(384, 4), (384, 3), (11008, 4), (11008, 3), (28672, 4)])
def test_words_per_row_per_channel(K, bits):
    # group -1 (and group = K) is one group per output channel
    h = awq.lib()
    assert h.awq_packed_words_per_row(K, bits, -1) == O.words_per_row(K, bits, K)
    assert h.awq_packed_words_per_row(K, bits, K) == O.words_per_row(K, bits, K)
    assert O.words_per_row(K, bits, K) == O.words_per_row(K, bits, 128)


def test_words_per_row_rejects():
    h = awq.lib()
    assert h.awq_packed_words_per_row(4096, 5, 128) == 0
    assert h.awq_packed_words_per_row(4000, 4, 128) == 0
    assert h.awq_packed_words_per_row(4096, 4, 64) == 0
    assert h.awq_packed_words_per_row(256, 4, -1) == 256 // 8
    assert h.awq_packed_words_per_row(0, 4, 128) == 0
    assert h.awq_packed_words_per_row(200, 4, -1) == 0        # not a multiple of 128
    assert h.awq_packed_words_per_row(4096 * 8 + 128, 4, -1) == 0  # past the per-row kernels
    assert h.awq_packed_words_per_row(1024, 4, 1024 + 128) == 0


# fake, aligned, never-dereferenced device addresses
P = ctypes.c_void_p(0x10000)
P2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10008)
NULL = None


def _mm(*, X=P, q=P, s=P, z=P, M=1, N=64, K=256, bits=4, group=128, Y=P2, kernel=None):
    h = awq.lib()
    if kernel is None:
        return h.awq_w4a16_matmul(X, q, s, z, M, N, K, bits, group, Y, NULL)
    return h.awq_w4a16_matmul_kernel(X, q, s, z, M, N, K, bits, group, Y, kernel, NULL)


def test_matmul_validation():
    E = _lib
    assert _mm(X=NULL) == E.AWQ_ERR_INVALID_ARG
    assert _mm(Y=NULL) == E.AWQ_ERR_INVALID_ARG
    assert _mm(M=0) == E.AWQ_ERR_INVALID_ARG
    assert _mm(N=-1) == E.AWQ_ERR_INVALID_ARG
    assert _mm(X=MIS) == E.AWQ_ERR_INVALID_ARG
    assert _mm(bits=5) == E.AWQ_ERR_UNSUPPORTED
    assert _mm(K=200) == E.AWQ_ERR_INVALID_ARG
    assert _mm(group=64) == E.AWQ_ERR_UNSUPPORTED
    assert _mm(group=0) == E.AWQ_ERR_INVALID_ARG
    assert _mm(kernel=7) == E.AWQ_ERR_INVALID_ARG
    assert _mm(kernel=1, M=17) == E.AWQ_ERR_UNSUPPORTED
    assert _mm(kernel=2, bits=3) == E.AWQ_ERR_UNSUPPORTED
    assert _mm(kernel=1, bits=3, M=5) == E.AWQ_ERR_UNSUPPORTED


def test_matmul_workspace_plan():
    """The split plan on a 256-compute-unit part (the count assumed without a
    device): prefill tiles 128 wide and 32, 64 or 128 tall, split over K until
    about one workgroup per unit; int4 decode at 2 <= M <= 16 on rows of
    more than 8192 codes, 16-row blocks split over K until about 8
    wavefronts per unit (at M = 16 one workgroup per unit with a wider LDS
    when that needs far fewer splits); other decode shapes and shapes that
    fill the part need none. Bytes: one float32 [M, N] plane per split, after a 64 KiB
    counter region."""
    h = awq.lib()
    W = h.awq_w4a16_matmul_workspace_bytes
    C = 64 << 10  # the counter region at the head of a split workspace
    assert W(4, 4096, 4096, 3, 128) == 0  # int3 decode kernel
    assert W(1, 4096, 4096, 4, 128) == 0  # M = 1 decode kernel
    assert W(2, 4096, 4096, 4, 128) == 0  # M = 2 on the per-token-row decode kernel
    # int4 decode, 2 <= M <= 16: rows of up to 8192 codes run unsplit on the
    # one-pass kernel
    assert W(16, 4096, 4096, 4, 128) == 0
    assert W(8, 28672, 8192, 4, 128) == 0
    # longer rows: 16-row blocks, K split for 8 wavefronts per unit and the
    # LDS (29 chunks of 128 codes at M <= 8, 16 at M <= 16); 11008 = 86
    # chunks in 8 splits of 11 (the last one 9), one [M, N] plane per split
    assert W(8, 4096, 11008, 4, 128) == C + 8 * 8 * 4096 * 4
    # 28672 codes = 224 chunks at M = 16: 14 splits of 16 would take 308
    # workgroups for 256 units, so one workgroup per unit with the wide LDS
    # takes 8 splits of 28
    assert W(16, 8192, 28672, 4, 128) == C + 8 * 16 * 8192 * 4
    assert W(2048, 28672, 8192, 4, 128) == 0  # whole rounds of big tiles
    assert W(256, 11008, 4096, 3, 128) == 0  # 172 tiles of 128 x 128: no split
    # int4, M = 32: 32 tiles of 32 x 128, 8 splits of 8 steps (64 codes each)
    assert W(32, 4096, 4096, 4, 128) == C + 8 * 32 * 4096 * 4
    # int3, M = 64: 32 tiles of 64 x 128; 86 steps of 128 codes in 8 splits
    assert W(64, 4096, 11008, 3, 128) == C + 8 * 64 * 4096 * 4
    # M = 256: 64 tiles of 128 x 128 in 4 splits
    assert W(256, 4096, 11008, 3, 128) == C + 4 * 256 * 4096 * 4
    # few steps: at least 8 per split (K = 512: 8 steps, no split)
    assert W(32, 256, 512, 4, 128) == 0
    assert W(32, 4096, 4096, 5, 128) == 0  # invalid
    assert W(0, 4096, 4096, 4, 128) == 0


def test_matmul_noalloc_validation():
    """The allocation-free product validates like the others before any HIP
    call, and without a device returns AWQ_ERR_NO_DEVICE; no plan on a
    256-unit part needs more than its 16 MiB of scratch."""
    h = awq.lib()
    E = _lib
    f = lambda X=P, M=32, N=4096, K=4096, bits=4, group=128: h.awq_w4a16_matmul_noalloc(  # noqa: E731
        X, P, P, P, M, N, K, bits, group, P2, NULL)
    assert f(X=NULL) == E.AWQ_ERR_INVALID_ARG
    assert f(X=MIS) == E.AWQ_ERR_INVALID_ARG
    assert f(M=0) == E.AWQ_ERR_INVALID_ARG
    assert f(bits=5) == E.AWQ_ERR_UNSUPPORTED
    assert f() == E.AWQ_ERR_NO_DEVICE          # splits K
    assert f(M=1) == E.AWQ_ERR_NO_DEVICE       # decode
    assert f(M=2048, N=256) == E.AWQ_ERR_NO_DEVICE  # the largest plan: 16 MiB of planes
    assert h.awq_w4a16_matmul_workspace_bytes(2048, 256, 4096, 4, 128) == (16 << 20) + (64 << 10)


def test_matmul_ws_validation():
    h = awq.lib()
    E = _lib
    need = h.awq_w4a16_matmul_workspace_bytes(32, 4096, 4096, 4, 128)

    def ws(w, nbytes, M=32, K=4096):
        return h.awq_w4a16_matmul_ws(P, P, P, P, M, 4096, K, 4, 128, P2, w, nbytes, NULL)

    assert ws(P, need - 16) == E.AWQ_ERR_WORKSPACE
    assert ws(MIS, need) == E.AWQ_ERR_INVALID_ARG
    # the int4 decode kernel for 2 <= M <= 16 splits long rows with a
    # workspace too
    need8 = h.awq_w4a16_matmul_workspace_bytes(8, 4096, 11008, 4, 128)
    assert need8 > 0
    assert ws(P, need8 - 16, M=8, K=11008) == E.AWQ_ERR_WORKSPACE
    import torch
    if not torch.cuda.is_available():  # valid requests: no device to run them
        assert ws(P, need) == E.AWQ_ERR_NO_DEVICE
        assert ws(NULL, 0) == E.AWQ_ERR_NO_DEVICE
        assert ws(P, need8, M=8, K=11008) == E.AWQ_ERR_NO_DEVICE
        assert ws(NULL, 0, M=8, K=11008) == E.AWQ_ERR_NO_DEVICE  # runs on the multi-pass kernel
        assert ws(P, 0, M=1) == E.AWQ_ERR_NO_DEVICE  # the M = 1 kernel takes no workspace


def test_valid_calls_without_device_report_no_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    h = awq.lib()
    E = _lib
    assert _mm() == E.AWQ_ERR_NO_DEVICE
    assert _mm(M=2048, K=8192, N=128) == E.AWQ_ERR_NO_DEVICE
    assert h.awq_quantize_pack(P, NULL, 64, 256, 4, 128, P, P, P, NULL) == E.AWQ_ERR_NO_DEVICE
    assert h.awq_quantize_pack_ex(P, NULL, 64, 256, 4, 128, 0, P, P, P,
                                  NULL) == E.AWQ_ERR_NO_DEVICE
    assert h.awq_fold_inv_scale(P, P, 4, 256, P2, NULL) == E.AWQ_ERR_NO_DEVICE
    assert h.awq_act_stats(P, 64, 256, P2, NULL) == E.AWQ_ERR_NO_DEVICE
    assert h.awq_scale_candidates(P, 256, P, 20, P2, NULL) == E.AWQ_ERR_NO_DEVICE


def test_quantize_pack_validation():
    h = awq.lib()
    E = _lib
    assert h.awq_quantize_pack(NULL, NULL, 64, 256, 4, 128, P, P, P, NULL) == E.AWQ_ERR_INVALID_ARG
    assert h.awq_quantize_pack(P, MIS, 64, 256, 4, 128, P, P, P, NULL) == E.AWQ_ERR_INVALID_ARG
    assert h.awq_quantize_pack(P, NULL, 0, 256, 4, 128, P, P, P, NULL) == E.AWQ_ERR_INVALID_ARG
    assert h.awq_quantize_pack(P, NULL, 64, 256, 2, 128, P, P, P, NULL) == E.AWQ_ERR_UNSUPPORTED
    assert h.awq_quantize_pack(P, NULL, 64, 300, 4, 128, P, P, P, NULL) == E.AWQ_ERR_INVALID_ARG
    ex = h.awq_quantize_pack_ex
    assert ex(P, NULL, 64, 256, 4, 128, 2, P, P, P, NULL) == E.AWQ_ERR_INVALID_ARG
    assert ex(P, NULL, 64, 256, 4, 128, -1, P, P, P, NULL) == E.AWQ_ERR_INVALID_ARG
    assert ex(NULL, NULL, 64, 256, 4, 128, 0, P, P, P, NULL) == E.AWQ_ERR_INVALID_ARG
    assert ex(P, NULL, 64, 256, 2, 128, 0, P, P, P, NULL) == E.AWQ_ERR_UNSUPPORTED


def test_other_validation():
    h = awq.lib()
    E = _lib
    assert h.awq_fold_inv_scale(P, NULL, 4, 256, P2, NULL) == E.AWQ_ERR_INVALID_ARG
    assert h.awq_fold_inv_scale(P, P, 4, 250, P2, NULL) == E.AWQ_ERR_UNSUPPORTED
    assert h.awq_act_stats(P, 0, 256, P2, NULL) == E.AWQ_ERR_INVALID_ARG
    assert h.awq_act_stats(P, 8192, 256, P2, NULL) == E.AWQ_ERR_UNSUPPORTED
    assert h.awq_scale_candidates(P, 256, P, 0, P2, NULL) == E.AWQ_ERR_INVALID_ARG


def test_scale_search_validation():
    h = awq.lib()
    E = _lib
    a = np.arange(20, dtype=np.float32) / 20
    ap = a.ctypes.data_as(ctypes.c_void_p)
    loss = np.zeros(20)
    lp = loss.ctypes.data_as(ctypes.c_void_p)
    best = ctypes.c_int(0)
    need = h.awq_scale_search_workspace_bytes(64, 256, 32, 20, 4, 128)
    assert h.awq_scale_search_workspace_bytes(64, 256, 0, 20, 4, 128) == 0
    assert h.awq_scale_search_workspace_bytes(64, 250, 32, 20, 4, 128) == 0

    def call(ws=P, nbytes=need, alpha=ap, T=32, K=256):
        return h.awq_scale_search(P, P, 64, K, T, alpha, 20, 4, 128, P2, lp, ctypes.byref(best),
                                  ws, nbytes, NULL)
    assert need > 0
    assert call(alpha=NULL) == E.AWQ_ERR_INVALID_ARG
    assert call(T=0) == E.AWQ_ERR_INVALID_ARG
    assert call(ws=NULL) == E.AWQ_ERR_WORKSPACE
    assert call(nbytes=need - 1) == E.AWQ_ERR_WORKSPACE
    bad = a.copy()
    bad[3] = 1.5
    assert call(alpha=bad.ctypes.data_as(ctypes.c_void_p)) == E.AWQ_ERR_INVALID_ARG

    def call_ex(zp, ws=P, nbytes=need):
        return h.awq_scale_search_ex(P, P, 64, 256, 32, ap, 20, 4, 128, zp, P2, lp,
                                     ctypes.byref(best), ws, nbytes, NULL)
    assert call_ex(2) == E.AWQ_ERR_INVALID_ARG
    assert call_ex(0, ws=NULL) == E.AWQ_ERR_WORKSPACE


def test_gate_up_validation():
    h = awq.lib()
    E = _lib

    def call(X=P, qg=P, qu=P, M=1, N=64, K=256, bits=4, group=128, Y=P2):
        return h.awq_w4a16_gate_up_silu(X, qg, P, P, qu, P, P, M, N, K, bits, group, Y, NULL)
    assert call(X=NULL) == E.AWQ_ERR_INVALID_ARG
    assert call(qu=NULL) == E.AWQ_ERR_INVALID_ARG
    assert call(qg=MIS) == E.AWQ_ERR_INVALID_ARG
    assert call(M=0) == E.AWQ_ERR_INVALID_ARG
    assert call(K=200) == E.AWQ_ERR_INVALID_ARG
    assert call(bits=2) == E.AWQ_ERR_UNSUPPORTED
    assert call(group=64) == E.AWQ_ERR_UNSUPPORTED
    import torch
    if not torch.cuda.is_available():
        assert call() == E.AWQ_ERR_NO_DEVICE


def test_norm_and_joint_validation():
    h = awq.lib()
    E = _lib
    assert h.awq_fold_norm_weight(NULL, P, 256, P2, NULL) == E.AWQ_ERR_INVALID_ARG
    assert h.awq_fold_norm_weight(P, P, 0, P2, NULL) == E.AWQ_ERR_INVALID_ARG
    assert h.awq_fold_norm_weight(P, MIS, 256, P2, NULL) == E.AWQ_ERR_INVALID_ARG
    f = ctypes.c_float
    assert h.awq_rmsnorm(P, P, 4, 256, f(1e-6), NULL, NULL) == E.AWQ_ERR_INVALID_ARG
    assert h.awq_rmsnorm(P, P, 0, 256, f(1e-6), P2, NULL) == E.AWQ_ERR_INVALID_ARG
    assert h.awq_rmsnorm(P, P, 4, 256, f(-1.0), P2, NULL) == E.AWQ_ERR_INVALID_ARG
    assert h.awq_rmsnorm(P, P, 4, 250, f(1e-6), P2, NULL) == E.AWQ_ERR_UNSUPPORTED
    assert h.awq_rmsnorm(P, P, 4, 16392, f(1e-6), P2, NULL) == E.AWQ_ERR_UNSUPPORTED
    Ns = (ctypes.c_int * 3)(64, 64, 32)
    Ws = (ctypes.c_void_p * 3)(0x10000, 0x20000, 0x30000)
    a = np.arange(20, dtype=np.float32) / 20
    ap = a.ctypes.data_as(ctypes.c_void_p)
    need = h.awq_scale_search_joint_workspace_bytes(Ns, 3, 256, 32, 20, 4, 128)
    assert need > h.awq_scale_search_workspace_bytes(64, 256, 32, 20, 4, 128)
    one = (ctypes.c_int * 1)(64)
    assert h.awq_scale_search_joint_workspace_bytes(one, 1, 256, 32, 20, 4, 128) == \
        h.awq_scale_search_workspace_bytes(64, 256, 32, 20, 4, 128)
    assert h.awq_scale_search_joint_workspace_bytes(Ns, 0, 256, 32, 20, 4, 128) == 0
    assert h.awq_scale_search_joint_workspace_bytes(Ns, 17, 256, 32, 20, 4, 128) == 0
    best = ctypes.c_int(0)

    def call(W=Ws, n=3, ws=P, nbytes=need, zp=1):
        return h.awq_scale_search_joint(W, Ns, n, P, 256, 32, ap, 20, 4, 128, zp, P2, NULL,
                                        ctypes.byref(best), ws, nbytes, NULL)
    assert call(n=0) == E.AWQ_ERR_INVALID_ARG
    assert call(zp=3) == E.AWQ_ERR_INVALID_ARG
    bad = (ctypes.c_void_p * 3)(0x10000, None, 0x30000)
    assert call(W=bad) == E.AWQ_ERR_INVALID_ARG
    assert call(ws=NULL) == E.AWQ_ERR_WORKSPACE
    assert call(nbytes=need - 1) == E.AWQ_ERR_WORKSPACE
    import torch
    if not torch.cuda.is_available():
        assert call() == E.AWQ_ERR_NO_DEVICE
        assert h.awq_rmsnorm(P, P, 4, 256, f(1e-6), P2, NULL) == E.AWQ_ERR_NO_DEVICE
        assert h.awq_fold_norm_weight(P, P, 256, P2, NULL) == E.AWQ_ERR_NO_DEVICE


def test_compact_validation():
    h = awq.lib()
    E = _lib
    assert h.awq_compact_group_params(NULL, P, 64, 256, 128, P, P, NULL) == E.AWQ_ERR_INVALID_ARG
    assert h.awq_compact_group_params(P, P, 0, 256, 128, P, P, NULL) == E.AWQ_ERR_INVALID_ARG
    assert h.awq_compact_group_params(P, P, 64, 256, 64, P, P, NULL) == E.AWQ_ERR_UNSUPPORTED
    assert h.awq_compact_group_params(P, MIS, 64, 256, 128, P, P, NULL) == E.AWQ_ERR_INVALID_ARG

    def mm(X=P, M=1, kernel=0, bits=4):
        return h.awq_w4a16_matmul_compact(X, P, P, P, M, 64, 256, bits, 128, P2, kernel, NULL)
    assert mm(X=NULL) == E.AWQ_ERR_INVALID_ARG
    assert mm(kernel=5) == E.AWQ_ERR_INVALID_ARG
    assert mm(kernel=2, bits=3) == E.AWQ_ERR_UNSUPPORTED
    import torch
    if not torch.cuda.is_available():
        assert mm() == E.AWQ_ERR_NO_DEVICE
        assert h.awq_compact_group_params(P, P, 64, 256, 128, P, P, NULL) == E.AWQ_ERR_NO_DEVICE
