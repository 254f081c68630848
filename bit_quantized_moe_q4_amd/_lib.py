"""ctypes view of libmoe_q4.so (the C ABI in include/moe_q4.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation anywhere in this package.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_q4.so")

MOE_Q4_OK, MOE_Q4_EINVAL, MOE_Q4_EWORKSPACE, MOE_Q4_EHIP = 0, -1, -2, -3
MOE_Q4_F32, MOE_Q4_BF16 = 0, 1
STAGE_GATEUP, STAGE_DOWN, STAGE_COMBINE, STAGE_ALL = 1, 2, 4, 7
STAGE_TEST_WAIT_FAIL = 16

EXPORTS = [
    "q4_packed_bytes", "q4_pack", "q8_quantize",
    "moe_q4_route_workspace_bytes", "moe_q4_route",
    "moe_q4_prefill_workspace_bytes", "moe_q4_prefill", "moe_q4_prefill_stage",
    "moe_q4_decode_workspace_bytes", "moe_q4_decode",
    "moe_q4_w4a8_gemv", "moe_q4_rmsnorm", "moe_q4_last_error",
]


WEIGHTS_Q4_0, WEIGHTS_Q8_0 = 0, 1


class Layer(C.Structure):
    _fields_ = [
        ("hidden", C.c_int32), ("inter", C.c_int32), ("n_experts", C.c_int32),
        ("top_k", C.c_int32), ("has_shared", C.c_int32),
        ("w_router", C.c_void_p), ("router_bias", C.c_void_p),
        ("w_gate", C.c_void_p), ("w_up", C.c_void_p), ("w_down", C.c_void_p),
        ("s_gate", C.c_void_p), ("s_up", C.c_void_p), ("s_down", C.c_void_p),
        ("t_gate", C.c_void_p), ("t_up", C.c_void_p), ("t_down", C.c_void_p),
        ("ts_gate", C.c_void_p), ("ts_up", C.c_void_p), ("ts_down", C.c_void_p),
        ("weight_format", C.c_int32),
    ]


class Routing(C.Structure):
    _fields_ = [
        ("topk_ids", C.c_void_p), ("topk_w", C.c_void_p), ("expert_offsets", C.c_void_p),
        ("perm", C.c_void_p), ("inv_perm", C.c_void_p),
    ]


class DecodeTrace(C.Structure):
    _fields_ = [
        ("logits", C.c_void_p), ("ids", C.c_void_p), ("w", C.c_void_p),
        ("qx", C.c_void_p), ("dx", C.c_void_p), ("qh", C.c_void_p), ("dh", C.c_void_p),
    ]


_lock = threading.Lock()
_lib = None


def _declare(lib):
    P, I32, I64, SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    sig = {
        "q4_packed_bytes": (SZ, [I64, I64]),
        "q4_pack": (C.c_int, [P, I64, I64, P, P]),
        "q4_tile": (C.c_int, [P, I64, I64, P, P]),
        "q8w_packed_bytes": (SZ, [I64, I64]),
        "q8w_pack": (C.c_int, [P, I64, I64, P, P]),
        "q8w_tile": (C.c_int, [P, I64, I64, P, P]),
        "q8_quantize": (C.c_int, [P, I64, I64, P, P, P]),
        "moe_q4_route_workspace_bytes": (SZ, [P, I32]),
        "moe_q4_route": (C.c_int, [P, P, I32, I32, P, P, P, SZ, P]),
        "moe_q4_prefill_workspace_bytes": (SZ, [P, I32]),
        "moe_q4_prefill": (C.c_int, [P, P, I32, P, P, P, SZ, P]),
        "moe_q4_prefill_stage": (C.c_int, [P, P, I32, P, P, P, SZ, I32, P]),
        "moe_q4_prefill_status": (C.c_int, [P, I32, P, SZ, P, P]),
        "moe_q4_check_layer": (C.c_int, [P]),
        "moe_q4_prefill_w4a8": (C.c_int, [P, P, I32, P, P, P, P, SZ, P]),
        "moe_q4_prefill_w4a8_stage": (C.c_int, [P, P, I32, P, P, P, P, SZ, I32, P]),
        "moe_q4_decode_workspace_bytes": (SZ, [P]),
        "moe_q4_decode_batch_workspace_bytes": (SZ, [P, I32]),
        "moe_q4_decode_stack_workspace_bytes": (SZ, [P, I32]),
        "moe_q4_decode_stack": (C.c_int, [P, I32, P, P, C.c_float, P, SZ, P]),
        "moe_q4_decode_batch": (C.c_int, [P, P, I32, P, P, P, P, SZ, P]),
        "moe_q4_decode": (C.c_int, [P, P, P, P, P, SZ, P]),
        "moe_q4_decode_noalloc": (C.c_int, [P, P, P, P]),
        "moe_q4_decode_status": (C.c_int, [P, P, SZ, P, P]),
        "moe_q4_test_decode_wait_fail": (None, [I32]),
        "moe_q4_w4a8_gemv": (C.c_int, [P, I32, I32, P, P, P, P, P]),
        "moe_q4_w4a8_gemm": (C.c_int, [P, I32, I32, P, P, I32, P, P, P]),
        "moe_q4_rmsnorm": (C.c_int, [P, I32, I32, C.c_float, P, P, P]),
        "moe_q4_probe_mfma": (C.c_int, [I32, I32, I32, P, P, P]),
        "moe_q4_last_error": (C.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def lib():
    """The loaded library; raises if libmoe_q4.so is missing."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    "libmoe_q4.so is not built (%s); run "
                    "`python -m bit_quantized_moe_q4_amd.build` first" % LIB_PATH)
            _lib = _declare(C.CDLL(LIB_PATH))
    return _lib


def check(rc: int, what: str) -> None:
    if rc != MOE_Q4_OK:
        msg = lib().moe_q4_last_error().decode(errors="replace")
        raise RuntimeError("%s failed (%d): %s" % (what, rc, msg))
