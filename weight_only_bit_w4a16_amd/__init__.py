"""AWQ W4A16 hot path for MI355X: a thin binding over libawq's C ABI.

The functions below only marshal arguments (dtype, device, contiguity and
shape checks, output allocation, the current HIP stream) and call the
library; every step of the computation runs in libawq's HIP kernels. There
is no CPU fallback: if the library is missing or no GPU is visible the calls
raise.

Notation follows the pages: W [N, K] (row = output channel), activations
[tokens, K], s [K] per input channel, delta/z per group of `group` codes
along K.
"""
from __future__ import annotations

import ctypes

import numpy as np

from ._lib import AwqError, check, lib  # noqa: F401

__all__ = [
    "AwqError", "lib", "packed_words_per_row", "act_stats", "scale_candidates",
    "quantize_pack", "fold_inv_scale", "w4a16_matmul", "gate_up_silu", "scale_search",
    "scale_search_joint", "scale_search_joint_workspace_bytes", "fold_norm_weight", "rmsnorm",
    "compact_group_params", "w4a16_matmul_compact",
    "scale_search_workspace_bytes", "KERNEL_AUTO", "KERNEL_DECODE", "KERNEL_DECODE_EXACT",
    "KERNEL_PREFILL",
]

KERNEL_AUTO, KERNEL_DECODE, KERNEL_DECODE_EXACT, KERNEL_PREFILL = 0, 1, 2, 3


def _torch():
    import torch
    return torch


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def _same_device(dev, *named):
    """Every tensor in (name, tensor) pairs sits on `dev` (the kernels read
    all operands on one device)."""
    for name, t in named:
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other operands on {dev}")


def _out(t, name, dtype, shape, device):
    """A caller-provided output: right dtype, exact shape, contiguous, on
    `device` (the library writes exactly shape's elements through its
    pointer)."""
    _need(t, name, dtype)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {device}")
    return t


def _group(K, group):
    return K if group == -1 else group


def packed_words_per_row(K: int, bits: int = 4, group: int = 128) -> int:
    n = lib().awq_packed_words_per_row(K, bits, group)
    if n == 0:
        raise ValueError(f"unsupported (K={K}, bits={bits}, group={group})")
    return int(n)


def act_stats(xcal, stream=None):
    """m[k] = mean_t |xcal[t, k]| (float64 [K])."""
    torch = _torch()
    _need(xcal, "xcal", torch.float16, 2)
    T, K = xcal.shape
    m = torch.empty(K, dtype=torch.float64, device=xcal.device)
    check(lib().awq_act_stats(_ptr(xcal), T, K, _ptr(m), _stream(stream)), "awq_act_stats")
    return m


def scale_candidates(m, alpha, stream=None):
    """s[a, k] = float32(m[k] ** alpha[a]) (float32 [n_alpha, K])."""
    torch = _torch()
    _need(m, "m", torch.float64, 1)
    _need(alpha, "alpha", torch.float32, 1)
    _same_device(m.device, ("alpha", alpha))
    s = torch.empty((alpha.numel(), m.numel()), dtype=torch.float32, device=m.device)
    check(lib().awq_scale_candidates(_ptr(m), m.numel(), _ptr(alpha), alpha.numel(), _ptr(s),
                                     _stream(stream)), "awq_scale_candidates")
    return s


def quantize_pack(W, s=None, bits: int = 4, group: int = 128, out=None, stream=None,
                  zero_point: bool = True):
    """Round-to-nearest quantize-and-pack of W diag(s) on the asymmetric grid
    (zero_point=True) or the symmetric one (zero_point=False).

    Returns (qpacked uint32-as-int32 [N, words_per_row], scales float32
    [N, K/group], zeros uint8 [N, K/group]).
    """
    torch = _torch()
    _need(W, "W", torch.float16, 2)
    N, K = W.shape
    if s is not None:
        _need(s, "s", torch.float32, 1)
        if s.numel() != K:
            raise ValueError("s must have K entries")
        _same_device(W.device, ("s", s))
    g = _group(K, group)
    wpr = packed_words_per_row(K, bits, group)
    if out is None:
        q = torch.empty((N, wpr), dtype=torch.int32, device=W.device)
        sc = torch.empty((N, K // g), dtype=torch.float32, device=W.device)
        z = torch.empty((N, K // g), dtype=torch.uint8, device=W.device)
    else:
        q, sc, z = out
        _out(q, "out qpacked", torch.int32, (N, wpr), W.device)
        _out(sc, "out scales", torch.float32, (N, K // g), W.device)
        _out(z, "out zeros", torch.uint8, (N, K // g), W.device)
    check(lib().awq_quantize_pack_ex(_ptr(W), _ptr(s), N, K, bits, group, int(bool(zero_point)),
                                     _ptr(q), _ptr(sc), _ptr(z), _stream(stream)),
          "awq_quantize_pack_ex")
    return q, sc, z


def fold_inv_scale(X, s, out=None, stream=None):
    """X' = fp16(float32(X) / s) (fp16 [M, K])."""
    torch = _torch()
    _need(X, "X", torch.float16, 2)
    _need(s, "s", torch.float32, 1)
    M, K = X.shape
    if s.numel() != K:
        raise ValueError("s must have K entries")
    _same_device(X.device, ("s", s))
    y = torch.empty_like(X) if out is None else _out(out, "out", torch.float16, (M, K), X.device)
    check(lib().awq_fold_inv_scale(_ptr(X), _ptr(s), M, K, _ptr(y), _stream(stream)),
          "awq_fold_inv_scale")
    return y


_MATMUL_WS = {}


def matmul_workspace_bytes(M: int, N: int, K: int, bits: int = 4, group: int = 128) -> int:
    """Bytes of workspace with which the product splits K for this shape (0: no split)."""
    return int(lib().awq_w4a16_matmul_workspace_bytes(M, N, K, bits, group))


def _matmul_workspace(device, stream_handle, nbytes: int):
    """A workspace of at least nbytes for calls on this device and stream,
    kept for reuse."""
    torch = _torch()
    key = (device.index if device.index is not None else torch.cuda.current_device(),
           int(getattr(stream_handle, "value", stream_handle) or 0))
    ws = _MATMUL_WS.get(key)
    if ws is None or ws.numel() < nbytes:
        # zero-filled: the split products keep their counters at its head
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _MATMUL_WS[key] = ws
    return ws


def w4a16_matmul(Xp, qpacked, scales, zeros, bits: int = 4, group: int = 128, out=None,
                 kernel: int = KERNEL_AUTO, stream=None, workspace=None):
    """Y = X' dequant(Q)^T (fp16 [M, N]) with X' already divided by s.

    With the automatic kernel choice, shapes that split K use `workspace`
    (a uint8 device tensor of at least matmul_workspace_bytes(...) bytes,
    zero-filled before its first use, shared only by calls ordered on one
    stream) or, when None, one kept per device and stream."""
    torch = _torch()
    _need(Xp, "Xp", torch.float16, 2)
    _need(qpacked, "qpacked", torch.int32, 2)
    _need(scales, "scales", torch.float32, 2)
    _need(zeros, "zeros", torch.uint8, 2)
    M, K = Xp.shape
    N = qpacked.shape[0]
    g = _group(K, group)
    if qpacked.shape[1] != packed_words_per_row(K, bits, group):
        raise ValueError("qpacked has the wrong row length for (K, bits, group)")
    if tuple(scales.shape) != (N, K // g) or tuple(zeros.shape) != (N, K // g):
        raise ValueError("scales/zeros must be [N, K/group]")
    _same_device(Xp.device, ("qpacked", qpacked), ("scales", scales), ("zeros", zeros),
                 ("workspace", workspace))
    y = torch.empty((M, N), dtype=torch.float16, device=Xp.device) if out is None else \
        _out(out, "out", torch.float16, (M, N), Xp.device)
    st = _stream(stream)
    if kernel == KERNEL_AUTO:
        nb = matmul_workspace_bytes(M, N, K, bits, group)
        if nb:
            ws = _matmul_workspace(Xp.device, st, nb) if workspace is None else workspace
            _need(ws, "workspace", torch.uint8, 1)
            r = lib().awq_w4a16_matmul_ws(_ptr(Xp), _ptr(qpacked), _ptr(scales), _ptr(zeros), M,
                                          N, K, bits, group, _ptr(y), _ptr(ws), ws.numel(), st)
        else:
            r = lib().awq_w4a16_matmul(_ptr(Xp), _ptr(qpacked), _ptr(scales), _ptr(zeros), M, N,
                                       K, bits, group, _ptr(y), st)
    else:
        r = lib().awq_w4a16_matmul_kernel(_ptr(Xp), _ptr(qpacked), _ptr(scales), _ptr(zeros), M,
                                          N, K, bits, group, _ptr(y), kernel, st)
    check(r, "awq_w4a16_matmul")
    return y


def compact_group_params(scales, zeros, K: int, group: int = 128, stream=None):
    """(fp16 steps [N, ng], int32 words of 4-bit zero points [N, ceil(ng/8)])
    from the plain float32 / uint8 group parameters of an [N, K] matrix."""
    torch = _torch()
    _need(scales, "scales", torch.float32, 2)
    _need(zeros, "zeros", torch.uint8, 2)
    N, ng = scales.shape
    if tuple(zeros.shape) != (N, ng) or ng != K // _group(K, group):
        raise ValueError("scales and zeros must be [N, K/group]")
    _same_device(scales.device, ("zeros", zeros))
    s16 = torch.empty((N, ng), dtype=torch.float16, device=scales.device)
    z4 = torch.empty((N, (ng + 7) // 8), dtype=torch.int32, device=scales.device)
    check(lib().awq_compact_group_params(_ptr(scales), _ptr(zeros), N, K, group, _ptr(s16),
                                         _ptr(z4), _stream(stream)), "awq_compact_group_params")
    return s16, z4


def w4a16_matmul_compact(Xp, qpacked, scales16, zeros4, bits: int = 4, group: int = 128,
                         out=None, kernel: int = KERNEL_AUTO, stream=None):
    """Y = X' dequant(Q)^T over compactly stored group parameters."""
    torch = _torch()
    _need(Xp, "Xp", torch.float16, 2)
    _need(qpacked, "qpacked", torch.int32, 2)
    _need(scales16, "scales16", torch.float16, 2)
    _need(zeros4, "zeros4", torch.int32, 2)
    M, K = Xp.shape
    N = qpacked.shape[0]
    g = _group(K, group)
    if qpacked.shape[1] != packed_words_per_row(K, bits, group):
        raise ValueError("qpacked has the wrong row length for (K, bits, group)")
    if tuple(scales16.shape) != (N, K // g) or tuple(zeros4.shape) != (N, (K // g + 7) // 8):
        raise ValueError("scales16 must be [N, K/group] and zeros4 [N, ceil(K/group / 8)]")
    _same_device(Xp.device, ("qpacked", qpacked), ("scales16", scales16), ("zeros4", zeros4))
    y = torch.empty((M, N), dtype=torch.float16, device=Xp.device) if out is None else \
        _out(out, "out", torch.float16, (M, N), Xp.device)
    check(lib().awq_w4a16_matmul_compact(_ptr(Xp), _ptr(qpacked), _ptr(scales16), _ptr(zeros4), M,
                                         N, K, bits, group, _ptr(y), kernel, _stream(stream)),
          "awq_w4a16_matmul_compact")
    return y


def gate_up_silu(Xp, gate, up, bits: int = 4, group: int = 128, out=None, stream=None):
    """Y = fp16(silu(X' Wg^T) * (X' Wu^T)) (fp16 [M, N]); `gate` and `up` are
    (qpacked, scales, zeros) triples of two [N, K] matrices."""
    torch = _torch()
    _need(Xp, "Xp", torch.float16, 2)
    M, K = Xp.shape
    g = _group(K, group)
    wpr = packed_words_per_row(K, bits, group)
    N = gate[0].shape[0]
    for name, (q, sc, z) in (("gate", gate), ("up", up)):
        _need(q, f"{name} qpacked", torch.int32, 2)
        _need(sc, f"{name} scales", torch.float32, 2)
        _need(z, f"{name} zeros", torch.uint8, 2)
        if tuple(q.shape) != (N, wpr):
            raise ValueError(f"{name} qpacked must be [N, words_per_row]")
        if tuple(sc.shape) != (N, K // g) or tuple(z.shape) != (N, K // g):
            raise ValueError(f"{name} scales/zeros must be [N, K/group]")
        _same_device(Xp.device, (f"{name} qpacked", q), (f"{name} scales", sc),
                     (f"{name} zeros", z))
    y = torch.empty((M, N), dtype=torch.float16, device=Xp.device) if out is None else \
        _out(out, "out", torch.float16, (M, N), Xp.device)
    check(lib().awq_w4a16_gate_up_silu(_ptr(Xp), _ptr(gate[0]), _ptr(gate[1]), _ptr(gate[2]),
                                       _ptr(up[0]), _ptr(up[1]), _ptr(up[2]), M, N, K, bits,
                                       group, _ptr(y), _stream(stream)),
          "awq_w4a16_gate_up_silu")
    return y


def scale_search_workspace_bytes(N, K, T, n_alpha, bits=4, group=128) -> int:
    return int(lib().awq_scale_search_workspace_bytes(N, K, T, n_alpha, bits, group))


def scale_search(W, xcal, alpha_grid=None, bits: int = 4, group: int = 128, workspace=None,
                 stream=None, zero_point: bool = True):
    """Grid search over alpha for s = mean|x| ** alpha, the weights quantized
    on the asymmetric (zero_point=True) or symmetric grid.

    Returns (s float32 [K] on the device, best index, losses float64 numpy).
    Synchronizes the stream.
    """
    torch = _torch()
    _need(W, "W", torch.float16, 2)
    _need(xcal, "xcal", torch.float16, 2)
    N, K = W.shape
    T = xcal.shape[0]
    if xcal.shape[1] != K:
        raise ValueError("xcal must be [T, K]")
    _same_device(W.device, ("xcal", xcal), ("workspace", workspace))
    if alpha_grid is None:
        alpha_grid = (np.arange(20, dtype=np.float64) / 20).astype(np.float32)
    a = np.ascontiguousarray(np.asarray(alpha_grid, dtype=np.float32))
    need = scale_search_workspace_bytes(N, K, T, len(a), bits, group)
    if need == 0:
        raise ValueError("unsupported scale_search sizes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=W.device)
    _need(workspace, "workspace", torch.uint8, 1)
    s = torch.empty(K, dtype=torch.float32, device=W.device)
    losses = np.zeros(len(a), dtype=np.float64)
    best = ctypes.c_int(-1)
    check(lib().awq_scale_search_ex(
        _ptr(W), _ptr(xcal), N, K, T, a.ctypes.data_as(ctypes.c_void_p), len(a), bits, group,
        int(bool(zero_point)), _ptr(s), losses.ctypes.data_as(ctypes.c_void_p),
        ctypes.byref(best), _ptr(workspace), workspace.numel(), _stream(stream)),
        "awq_scale_search_ex")
    return s, int(best.value), losses


def scale_search_joint_workspace_bytes(Ns, K, T, n_alpha, bits=4, group=128) -> int:
    arr = (ctypes.c_int * len(Ns))(*[int(n) for n in Ns])
    return int(lib().awq_scale_search_joint_workspace_bytes(arr, len(Ns), K, T, n_alpha, bits,
                                                            group))


def scale_search_joint(Ws, xcal, alpha_grid=None, bits: int = 4, group: int = 128,
                       workspace=None, stream=None, zero_point: bool = True):
    """One s for the layers Ws (each [N_l, K], fp16) that read the same
    input: the layers' losses are added per candidate before the argmin.

    Returns (s float32 [K] on the device, best index, summed losses float64
    numpy). Synchronizes the stream.
    """
    torch = _torch()
    Ws = list(Ws)
    if not Ws:
        raise ValueError("Ws must hold at least one matrix")
    _need(xcal, "xcal", torch.float16, 2)
    T, K = xcal.shape
    for i, W in enumerate(Ws):
        _need(W, f"Ws[{i}]", torch.float16, 2)
        if W.shape[1] != K:
            raise ValueError("every W must be [N_l, K] with the K of xcal")
        _same_device(xcal.device, (f"Ws[{i}]", W))
    if alpha_grid is None:
        alpha_grid = (np.arange(20, dtype=np.float64) / 20).astype(np.float32)
    a = np.ascontiguousarray(np.asarray(alpha_grid, dtype=np.float32))
    Ns = [int(W.shape[0]) for W in Ws]
    need = scale_search_joint_workspace_bytes(Ns, K, T, len(a), bits, group)
    if need == 0:
        raise ValueError("unsupported scale_search_joint sizes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=xcal.device)
    _need(workspace, "workspace", torch.uint8, 1)
    _same_device(xcal.device, ("workspace", workspace))
    s = torch.empty(K, dtype=torch.float32, device=xcal.device)
    losses = np.zeros(len(a), dtype=np.float64)
    best = ctypes.c_int(-1)
    ptrs = (ctypes.c_void_p * len(Ws))(*[W.data_ptr() for W in Ws])
    narr = (ctypes.c_int * len(Ws))(*Ns)
    check(lib().awq_scale_search_joint(
        ptrs, narr, len(Ws), _ptr(xcal), K, T, a.ctypes.data_as(ctypes.c_void_p), len(a), bits,
        group, int(bool(zero_point)), _ptr(s), losses.ctypes.data_as(ctypes.c_void_p),
        ctypes.byref(best), _ptr(workspace), workspace.numel(), _stream(stream)),
        "awq_scale_search_joint")
    return s, int(best.value), losses


def fold_norm_weight(gamma, s, out=None, stream=None):
    """gamma' = fp16(float32(gamma) / s): the RMSNorm weight with diag(s)^-1
    folded in (fp16 [K])."""
    torch = _torch()
    _need(gamma, "gamma", torch.float16, 1)
    _need(s, "s", torch.float32, 1)
    if s.numel() != gamma.numel():
        raise ValueError("gamma and s must have K entries each")
    _same_device(gamma.device, ("s", s))
    y = torch.empty_like(gamma) if out is None else \
        _out(out, "out", torch.float16, tuple(gamma.shape), gamma.device)
    check(lib().awq_fold_norm_weight(_ptr(gamma), _ptr(s), gamma.numel(), _ptr(y),
                                     _stream(stream)), "awq_fold_norm_weight")
    return y


def rmsnorm(X, gamma, eps: float = 1e-6, out=None, stream=None):
    """fp16(X r gamma) with r = (mean_k X^2 + eps)^-1/2 per row (fp16 [M, K])."""
    torch = _torch()
    _need(X, "X", torch.float16, 2)
    _need(gamma, "gamma", torch.float16, 1)
    M, K = X.shape
    if gamma.numel() != K:
        raise ValueError("gamma must have K entries")
    _same_device(X.device, ("gamma", gamma))
    y = torch.empty_like(X) if out is None else _out(out, "out", torch.float16, (M, K), X.device)
    check(lib().awq_rmsnorm(_ptr(X), _ptr(gamma), M, K, ctypes.c_float(eps), _ptr(y),
                            _stream(stream)), "awq_rmsnorm")
    return y
