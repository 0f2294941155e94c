"""ctypes declarations of libawq's C ABI (include/awq.h)."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libawq.so")

STATUS = {
    0: "AWQ_OK",
    1: "AWQ_ERR_INVALID_ARG",
    2: "AWQ_ERR_UNSUPPORTED",
    3: "AWQ_ERR_NO_DEVICE",
    4: "AWQ_ERR_HIP",
    5: "AWQ_ERR_WORKSPACE",
}
AWQ_OK, AWQ_ERR_INVALID_ARG, AWQ_ERR_UNSUPPORTED, AWQ_ERR_NO_DEVICE, AWQ_ERR_HIP, \
    AWQ_ERR_WORKSPACE = range(6)

_p = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t

# name -> (restype, argtypes), in header order
SIGNATURES = {
    "awq_status_string": (ctypes.c_char_p, [_i]),
    "awq_version": (_i, []),
    "awq_packed_words_per_row": (_sz, [_i, _i, _i]),
    "awq_act_stats": (_i, [_p, _i, _i, _p, _p]),
    "awq_scale_candidates": (_i, [_p, _i, _p, _i, _p, _p]),
    "awq_quantize_pack": (_i, [_p, _p, _i, _i, _i, _i, _p, _p, _p, _p]),
    "awq_quantize_pack_ex": (_i, [_p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p]),
    "awq_fold_inv_scale": (_i, [_p, _p, _i, _i, _p, _p]),
    "awq_w4a16_matmul": (_i, [_p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p]),
    "awq_w4a16_matmul_kernel": (_i, [_p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _i, _p]),
    "awq_w4a16_matmul_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "awq_w4a16_matmul_ws": (_i, [_p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _sz, _p]),
    "awq_w4a16_matmul_noalloc": (_i, [_p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p]),
    "awq_compact_group_params": (_i, [_p, _p, _i, _i, _i, _p, _p, _p]),
    "awq_w4a16_matmul_compact": (_i, [_p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _i, _p]),
    "awq_w4a16_gate_up_silu": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _p]),
    "awq_scale_search_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "awq_scale_search": (_i, [_p, _p, _i, _i, _i, _p, _i, _i, _i, _p, _p, _p, _p, _sz, _p]),
    "awq_scale_search_ex": (_i, [_p, _p, _i, _i, _i, _p, _i, _i, _i, _i, _p, _p, _p, _p, _sz,
                                 _p]),
    "awq_scale_search_joint_workspace_bytes": (_sz, [_p, _i, _i, _i, _i, _i, _i]),
    "awq_scale_search_joint": (_i, [_p, _p, _i, _p, _i, _i, _p, _i, _i, _i, _i, _p, _p, _p, _p,
                                    _sz, _p]),
    "awq_fold_norm_weight": (_i, [_p, _p, _i, _p, _p]),
    "awq_rmsnorm": (_i, [_p, _p, _i, _i, ctypes.c_float, _p, _p]),
}

_LIB = None


class AwqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


def lib() -> ctypes.CDLL:
    """The loaded library. Raises if it has not been built: there is no
    fallback path."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m weight_only_bit_w4a16_amd.build` (hipcc, gfx950)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _LIB = h
    return _LIB


def check(status: int, where: str) -> None:
    if status != AWQ_OK:
        raise AwqError(status, where)
