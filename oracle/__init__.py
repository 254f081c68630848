"""CPU oracle for the Q4_0 Mixture-of-Experts expert FFN (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The product
library never loads it, and it shares no code with the HIP path.

The arithmetic lives in ``moe_q4_oracle.c`` (plain single-threaded C); this
file only compiles it (``build()``), loads it and marshals numpy arrays.  Each
wrapper names the C function whose header comment states the definition it
follows.  All arrays are host numpy arrays.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_q4_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_q4_oracle.so")
# -ffp-contract=off: a*b+c stays two roundings unless fmaf() is written.
CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]

_lock = threading.Lock()
_lib = None

BLK = 32
Q4_BYTES = 18
Q8W_BYTES = 34
Q4_0, Q8_0 = 0, 1          # weight formats of a layer (``orc_layer.wfmt``)


def build(out: str = _LIB, src: str = _SRC, extra: tuple = ()) -> str:
    """Compile the oracle with gcc into ``out`` (always recompiles)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *extra, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class Layer(C.Structure):
    """Mirror of ``orc_layer`` in moe_q4_oracle.c."""

    _fields_ = [
        ("H", C.c_int64), ("I", C.c_int64), ("E", C.c_int64),
        ("k", C.c_int32), ("has_shared", C.c_int32),
        ("w_router", C.c_void_p), ("bias", C.c_void_p),
        ("gate", C.c_void_p), ("up", C.c_void_p), ("down", C.c_void_p),
        ("s_gate", C.c_void_p), ("s_up", C.c_void_p), ("s_down", C.c_void_p),
        ("wfmt", C.c_int32),
    ]


class DecodeTrace(C.Structure):
    """Mirror of ``orc_decode_trace`` in moe_q4_oracle.c."""

    _fields_ = [
        ("logits", C.c_void_p), ("ids", C.c_void_p), ("w", C.c_void_p),
        ("qx", C.c_void_p), ("dx", C.c_void_p),
        ("gate", C.c_void_p), ("up", C.c_void_p),
        ("qh", C.c_void_p), ("dh", C.c_void_p), ("o", C.c_void_p),
    ]


def _declare(lib):
    P, I64, I32, F = C.c_void_p, C.c_int64, C.c_int32, C.c_float
    sig = {
        "orc_f32_to_f16": (C.c_uint16, [F]),
        "orc_f16_to_f32": (F, [C.c_uint16]),
        "orc_tree_sum": (F, [P, I64]),
        "orc_q4_row_bytes": (C.c_size_t, [I64]),
        "orc_q4_pack": (None, [P, I64, I64, P]),
        "orc_q4_dequant": (None, [P, I64, I64, P]),
        "orc_q8_quantize": (None, [P, I64, I64, P, P]),
        "orc_q8w_row_bytes": (C.c_size_t, [I64]),
        "orc_q8w_pack": (None, [P, I64, I64, P]),
        "orc_q8w_dequant": (None, [P, I64, I64, P]),
        "orc_w8a8_gemv": (None, [P, I64, I64, P, P, P, P]),
        "orc_exp_p": (F, [F]),
        "orc_silu_p": (F, [F]),
        "orc_router_logits": (None, [P, I64, I64, P, I64, P, P]),
        "orc_topk": (None, [P, I64, I64, I32, P, P, P]),
        "orc_route_permutation": (None, [P, I64, I32, I64, P, P, P, P]),
        "orc_prefill_ref": (None, [P, P, P, P, P, I64, P]),
        "orc_bf16_round": (F, [F]),
        "orc_bf16_round_n": (None, [P, I64, P]),
        "orc_prefill_bf16": (None, [P, P, P, P, P, I64, P]),
        "orc_w4a8_gemv": (None, [P, I64, I64, P, P, P, P]),
        "orc_decode": (None, [P, P, P, P]),
        "orc_rmsnorm": (None, [P, I64, I64, F, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def load(path: str | None = None):
    """Load the compiled oracle, compiling it first only if it is absent.

    ``MOE_Q4_ORACLE_LIB`` names another build to load instead (the planted-
    mistake tests use it to run the pins against deliberately broken copies).
    """
    global _lib
    if path is not None:
        return _declare(C.CDLL(path))
    with _lock:
        if _lib is None:
            alt = os.environ.get("MOE_Q4_ORACLE_LIB")
            if alt:
                _lib = _declare(C.CDLL(alt))
            else:
                if not os.path.exists(_LIB):
                    build()
                _lib = _declare(C.CDLL(_LIB))
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


# --------------------------------------------------------------------------
# Scalar helpers
# --------------------------------------------------------------------------
def f32_to_f16_bits(x: float, lib=None) -> int:
    return int((lib or load()).orc_f32_to_f16(float(np.float32(x))))


def f16_bits_to_f32(h: int, lib=None) -> float:
    return float(np.float32((lib or load()).orc_f16_to_f32(int(h))))


def exp_p(x, lib=None) -> np.ndarray:
    lib = lib or load()
    x = np.asarray(x, dtype=np.float32).ravel()
    return np.array([lib.orc_exp_p(float(v)) for v in x], dtype=np.float32)


def silu_p(x, lib=None) -> np.ndarray:
    lib = lib or load()
    x = np.asarray(x, dtype=np.float32).ravel()
    return np.array([lib.orc_silu_p(float(v)) for v in x], dtype=np.float32)


def tree_sum(v, lib=None) -> np.float32:
    v = _c(v, np.float32)
    return np.float32((lib or load()).orc_tree_sum(_p(v), v.size))


# --------------------------------------------------------------------------
# Formats
# --------------------------------------------------------------------------
def q4_row_bytes(K: int) -> int:
    return (K // BLK) * Q4_BYTES


def q4_pack(w, lib=None, threads: int = 1) -> np.ndarray:
    """``orc_q4_pack``: fp32 [..., rows, K] -> uint8 [..., rows, K/32*18].

    ``threads`` > 1 packs disjoint row ranges concurrently (each call is the
    same single-threaded C function; rows are independent)."""
    w = _c(w, np.float32)
    K = w.shape[-1]
    assert K % BLK == 0
    rows = w.size // K
    out = np.empty(w.shape[:-1] + (q4_row_bytes(K),), dtype=np.uint8)
    lib = lib or load()
    w2, o2 = w.reshape(rows, K), out.reshape(rows, q4_row_bytes(K))
    if threads <= 1 or rows < 2 * threads:
        lib.orc_q4_pack(_p(w2), rows, K, _p(o2))
        return out
    from concurrent.futures import ThreadPoolExecutor
    step = (rows + threads - 1) // threads
    def job(r0):
        r1 = min(rows, r0 + step)
        lib.orc_q4_pack(_p(w2[r0:r1]), r1 - r0, K, _p(o2[r0:r1]))
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(job, range(0, rows, step)))
    return out


def q4_dequant(packed, K: int, lib=None) -> np.ndarray:
    """``orc_q4_dequant``: uint8 [..., rows, K/32*18] -> fp32 [..., rows, K]."""
    packed = _c(packed, np.uint8)
    rb = q4_row_bytes(K)
    rows = packed.size // rb
    out = np.empty(packed.shape[:-1] + (K,), dtype=np.float32)
    (lib or load()).orc_q4_dequant(_p(packed), rows, K, _p(out))
    return out


def q8w_row_bytes(K: int) -> int:
    return (K // BLK) * Q8W_BYTES


def q8w_pack(w, lib=None, threads: int = 1) -> np.ndarray:
    """``orc_q8w_pack``: fp32 [..., rows, K] -> uint8 [..., rows, K/32*34] (Q8_0)."""
    w = _c(w, np.float32)
    K = w.shape[-1]
    assert K % BLK == 0
    rows = w.size // K
    out = np.empty(w.shape[:-1] + (q8w_row_bytes(K),), dtype=np.uint8)
    lib = lib or load()
    w2, o2 = w.reshape(rows, K), out.reshape(rows, q8w_row_bytes(K))
    if threads <= 1 or rows < 2 * threads:
        lib.orc_q8w_pack(_p(w2), rows, K, _p(o2))
        return out
    from concurrent.futures import ThreadPoolExecutor
    step = (rows + threads - 1) // threads
    def job(r0):
        r1 = min(rows, r0 + step)
        lib.orc_q8w_pack(_p(w2[r0:r1]), r1 - r0, K, _p(o2[r0:r1]))
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(job, range(0, rows, step)))
    return out


def q8w_dequant(packed, K: int, lib=None) -> np.ndarray:
    """``orc_q8w_dequant``: uint8 [..., rows, K/32*34] -> fp32 [..., rows, K]."""
    packed = _c(packed, np.uint8)
    rb = q8w_row_bytes(K)
    rows = packed.size // rb
    out = np.empty(packed.shape[:-1] + (K,), dtype=np.float32)
    (lib or load()).orc_q8w_dequant(_p(packed), rows, K, _p(out))
    return out


def q8_quantize(x, lib=None):
    """``orc_q8_quantize``: fp32 [..., K] -> (int8 [..., K], fp32 [..., K/32])."""
    x = _c(x, np.float32)
    K = x.shape[-1]
    rows = x.size // K
    q = np.empty(x.shape, dtype=np.int8)
    d = np.empty(x.shape[:-1] + (K // BLK,), dtype=np.float32)
    (lib or load()).orc_q8_quantize(_p(x), rows, K, _p(q), _p(d))
    return q, d


# --------------------------------------------------------------------------
# Routing
# --------------------------------------------------------------------------
def router_logits(x, w_router, bias=None, lib=None) -> np.ndarray:
    """``orc_router_logits``: x [T,H] fp32, W_r [H,E] -> logits [T,E] fp32."""
    x = _c(x, np.float32)
    w_router = _c(w_router, np.float32)
    bias = None if bias is None else _c(bias, np.float32)
    T, H = x.shape
    E = w_router.shape[1]
    out = np.empty((T, E), dtype=np.float32)
    (lib or load()).orc_router_logits(_p(x), T, H, _p(w_router), E, _p(bias), _p(out))
    return out


def topk(logits, k: int, lib=None):
    """``orc_topk``: -> (ids int32 [T,k], w32 fp32 [T,k], w64 fp64 [T,k])."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    assert 1 <= k <= min(E, 1024)
    ids = np.empty((T, k), dtype=np.int32)
    w32 = np.empty((T, k), dtype=np.float32)
    w64 = np.empty((T, k), dtype=np.float64)
    (lib or load()).orc_topk(_p(logits), T, E, k, _p(ids), _p(w32), _p(w64))
    return ids, w32, w64


def route_permutation(ids, E: int, lib=None):
    """``orc_route_permutation``: -> (counts [E], offsets [E+1], perm, inv_perm)."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(T * k, dtype=np.int32)
    inv = np.empty(T * k, dtype=np.int32)
    (lib or load()).orc_route_permutation(_p(ids), T, k, E, _p(counts), _p(offsets),
                                          _p(perm), _p(inv))
    return counts, offsets, perm, inv


# --------------------------------------------------------------------------
# Layer-level
# --------------------------------------------------------------------------
class PackedLayer:
    """Host copy of one packed layer, laid out as the oracle's ``orc_layer``.

    gate/up: uint8 [E, I, H/32*B]; down: uint8 [E, H, I/32*B] with B = 18
    (Q4_0) or 34 (Q8_0, wfmt = Q8_0: decode only); s_gate/s_up/s_down: the
    shared expert (single matrices) or None.
    """

    def __init__(self, w_router, bias, gate, up, down, s_gate=None, s_up=None,
                 s_down=None, k=1, wfmt=Q4_0):
        self.w_router = _c(w_router, np.float32)
        self.bias = None if bias is None else _c(bias, np.float32)
        self.gate = _c(gate, np.uint8)
        self.up = _c(up, np.uint8)
        self.down = _c(down, np.uint8)
        self.has_shared = s_gate is not None
        self.s_gate = None if s_gate is None else _c(s_gate, np.uint8)
        self.s_up = None if s_up is None else _c(s_up, np.uint8)
        self.s_down = None if s_down is None else _c(s_down, np.uint8)
        self.H, self.E = self.w_router.shape
        self.I = self.gate.shape[1]
        self.k = int(k)
        self.wfmt = int(wfmt)
        rb = q8w_row_bytes if self.wfmt == Q8_0 else q4_row_bytes
        assert self.gate.shape == (self.E, self.I, rb(self.H))
        assert self.down.shape == (self.E, self.H, rb(self.I))

    @classmethod
    def from_float(cls, w_router, bias, gate, up, down, s_gate=None, s_up=None,
                   s_down=None, k=1, lib=None, threads: int = 1, wfmt=Q4_0):
        """Pack fp32 expert weights with the oracle's own ``orc_q4_pack`` (or
        ``orc_q8w_pack`` for wfmt = Q8_0)."""
        pack = q8w_pack if wfmt == Q8_0 else q4_pack
        pk = lambda a: None if a is None else pack(a, lib=lib, threads=threads)  # noqa: E731
        return cls(w_router, bias, pk(gate), pk(up), pk(down), pk(s_gate),
                   pk(s_up), pk(s_down), k=k, wfmt=wfmt)

    def cstruct(self) -> Layer:
        L = Layer()
        L.H, L.I, L.E, L.k = self.H, self.I, self.E, self.k
        L.has_shared = 1 if self.has_shared else 0
        L.w_router, L.bias = _p(self.w_router), _p(self.bias)
        L.gate, L.up, L.down = _p(self.gate), _p(self.up), _p(self.down)
        L.s_gate, L.s_up, L.s_down = _p(self.s_gate), _p(self.s_up), _p(self.s_down)
        L.wfmt = self.wfmt
        return L


def route(layer: PackedLayer, x, lib=None) -> dict:
    """Router + top-k + permutation for a token batch x [T,H] fp32."""
    lib = lib or load()
    logits = router_logits(x, layer.w_router, layer.bias, lib=lib)
    ids, w32, w64 = topk(logits, layer.k, lib=lib)
    counts, offsets, perm, inv = route_permutation(ids, layer.E, lib=lib)
    return dict(logits=logits, ids=ids, w32=w32, w64=w64, counts=counts,
                offsets=offsets, perm=perm, inv_perm=inv)


def prefill_ref(layer: PackedLayer, x, ids, w64, tokens=None, lib=None, threads: int = 1) -> np.ndarray:
    """``orc_prefill_ref``: binary64 y for the listed tokens -> [n, H] fp64.

    ``threads`` > 1 runs the same single-threaded C function on disjoint
    slices of the token list concurrently (the layer is a per-token function,
    so each token's row is the same whatever the split)."""
    assert layer.wfmt == Q4_0, "the prefill reference is defined for Q4_0 layers"
    lib = lib or load()
    x = _c(x, np.float32)
    ids = _c(ids, np.int32)
    w64 = _c(w64, np.float64)
    T = x.shape[0]
    tok = np.arange(T, dtype=np.int64) if tokens is None else _c(tokens, np.int64)
    n = tok.size
    y = np.empty((n, layer.H), dtype=np.float64)
    L = layer.cstruct()

    def run(lo, hi):
        if hi > lo:
            lib.orc_prefill_ref(C.byref(L), _p(x), _p(ids), _p(w64), _p(tok[lo:hi]), hi - lo, _p(y[lo:hi]))
    if threads <= 1 or n < 2 * threads:
        run(0, n)
        return y
    step = (n + threads - 1) // threads
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda i: run(i, min(i + step, n)), range(0, n, step)))
    return y


def bf16_round(x, lib=None) -> np.ndarray:
    """``orc_bf16_round`` of each element: the nearest bfloat16 (ties to
    even), widened back to float32."""
    lib = lib or load()
    x = _c(np.atleast_1d(x), np.float32)
    out = np.empty_like(x)
    lib.orc_bf16_round_n(_p(x), x.size, _p(out))
    return out


def prefill_bf16(layer: PackedLayer, x, ids, w32, tokens=None, lib=None, threads: int = 1) -> np.ndarray:
    """``orc_prefill_bf16``: the bf16 prefill program for the listed tokens ->
    [n, H] float32 (x: bf16 values widened to float32; w32: the float32
    routing weights).  ``threads`` as in ``prefill_ref``."""
    assert layer.wfmt == Q4_0, "the prefill program is defined for Q4_0 layers"
    lib = lib or load()
    x = _c(x, np.float32)
    ids = _c(ids, np.int32)
    w32 = _c(w32, np.float32)
    T = x.shape[0]
    tok = np.arange(T, dtype=np.int64) if tokens is None else _c(tokens, np.int64)
    n = tok.size
    y = np.empty((n, layer.H), dtype=np.float32)
    L = layer.cstruct()

    def run(lo, hi):
        if hi > lo:
            lib.orc_prefill_bf16(C.byref(L), _p(x), _p(ids), _p(w32), _p(tok[lo:hi]), hi - lo, _p(y[lo:hi]))
    if threads <= 1 or n < 2 * threads:
        run(0, n)
        return y
    step = (n + threads - 1) // threads
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda i: run(i, min(i + step, n)), range(0, n, step)))
    return y


def w4a8_gemv(W, K: int, qa, da, lib=None):
    """``orc_w4a8_gemv``: -> (dots int32 [N, K/32], out fp32 [N])."""
    W = _c(W, np.uint8)
    N = W.size // q4_row_bytes(K)
    qa = _c(qa, np.int8)
    da = _c(da, np.float32)
    dots = np.empty((N, K // BLK), dtype=np.int32)
    out = np.empty(N, dtype=np.float32)
    (lib or load()).orc_w4a8_gemv(_p(W), N, K, _p(qa), _p(da), _p(dots), _p(out))
    return dots, out


def w8a8_gemv(W, K: int, qa, da, lib=None):
    """``orc_w8a8_gemv``: Q8_0 rows -> (dots int32 [N, K/32], out fp32 [N])."""
    W = _c(W, np.uint8)
    N = W.size // q8w_row_bytes(K)
    qa = _c(qa, np.int8)
    da = _c(da, np.float32)
    dots = np.empty((N, K // BLK), dtype=np.int32)
    out = np.empty(N, dtype=np.float32)
    (lib or load()).orc_w8a8_gemv(_p(W), N, K, _p(qa), _p(da), _p(dots), _p(out))
    return dots, out


def decode(layer: PackedLayer, x, trace: bool = False, lib=None):
    """``orc_decode``: one token x [H] fp32 -> y [H] fp32 (and the trace)."""
    lib = lib or load()
    x = _c(x, np.float32).ravel()
    H, I, E, k = layer.H, layer.I, layer.E, layer.k
    S = 1 if layer.has_shared else 0
    y = np.empty(H, dtype=np.float32)
    L = layer.cstruct()
    if not trace:
        lib.orc_decode(C.byref(L), _p(x), _p(y), None)
        return y
    tr = dict(
        logits=np.empty(E, np.float32), ids=np.empty(k, np.int32),
        w=np.empty(k, np.float32), qx=np.empty(H, np.int8),
        dx=np.empty(H // BLK, np.float32), gate=np.empty((k + S, I), np.float32),
        up=np.empty((k + S, I), np.float32), qh=np.empty((k + S, I), np.int8),
        dh=np.empty((k + S, I // BLK), np.float32), o=np.empty((k + S, H), np.float32))
    T = DecodeTrace(**{name: _p(a) for name, a in tr.items()})
    lib.orc_decode(C.byref(L), _p(x), _p(y), C.byref(T))
    return y, tr


def rmsnorm(y, eps: float = 1e-6, lib=None) -> np.ndarray:
    """``orc_rmsnorm``: y [T,H] fp32 -> normalised [T,H] fp32 (unit gain)."""
    y = _c(y, np.float32)
    T, H = y.shape
    out = np.empty_like(y)
    (lib or load()).orc_rmsnorm(_p(y), T, H, float(eps), _p(out))
    return out
