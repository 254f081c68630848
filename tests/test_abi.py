"""The C-ABI library without a GPU: exported symbols and host-side checks.

Nothing here launches a kernel: every call below fails (or returns) in the
library's argument checks before anything is enqueued.
"""
import ctypes as C
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_q4.h")


@pytest.fixture(scope="module")
def lib():
    from bit_quantized_moe_q4_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from bit_quantized_moe_q4_amd import build
        build.build()
    return _lib.lib()


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "sizeof")))


def test_header_declares_the_api():
    names = header_functions()
    for n in ["q4_packed_bytes", "q4_pack", "q4_tile", "q8w_packed_bytes", "q8w_pack", "q8w_tile", "q8_quantize",
              "moe_q4_route", "moe_q4_prefill",
              "moe_q4_decode", "moe_q4_decode_batch", "moe_q4_decode_batch_workspace_bytes",
              "moe_q4_decode_stack", "moe_q4_decode_stack_workspace_bytes",
              "moe_q4_route_workspace_bytes", "moe_q4_prefill_workspace_bytes",
              "moe_q4_decode_workspace_bytes", "moe_q4_w4a8_gemv", "moe_q4_w4a8_gemm", "moe_q4_rmsnorm",
              "moe_q4_prefill_status", "moe_q4_prefill_w4a8", "moe_q4_prefill_w4a8_stage", "moe_q4_check_layer",
              "moe_q4_decode_status",
              "moe_q4_test_decode_wait_fail", "moe_q4_probe_mfma",
              "moe_q4_last_error"]:
        assert n in names, n


def test_every_declared_symbol_is_exported(lib):
    from bit_quantized_moe_q4_amd import _lib
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in header_functions():
        assert n in exported, n
        assert getattr(lib, n) is not None


def _layer(hidden=256, inter=128, E=8, k=2, shared=0, ptr=0x10000):
    from bit_quantized_moe_q4_amd._lib import Layer
    L = Layer()
    L.hidden, L.inter, L.n_experts, L.top_k, L.has_shared = hidden, inter, E, k, shared
    L.w_router = L.w_gate = L.w_up = L.w_down = ptr
    if shared:
        L.s_gate = L.s_up = L.s_down = ptr
    return L


def _err(lib):
    return lib.moe_q4_last_error().decode()


def test_packed_bytes(lib):
    assert lib.q4_packed_bytes(512, 2048) == 512 * 64 * 18
    assert lib.q4_packed_bytes(3, 33) == 0
    assert lib.q4_packed_bytes(0, 32) == 0


def test_pack_and_quantize_argument_checks(lib):
    assert lib.q4_pack(C.c_void_p(0x1000), 4, 33, C.c_void_p(0x2000), None) == -1
    assert "K" in _err(lib)
    assert lib.q4_pack(None, 4, 32, C.c_void_p(0x2000), None) == -1
    assert lib.q4_pack(C.c_void_p(0x1004), 4, 32, C.c_void_p(0x2000), None) == -1   # misaligned
    assert lib.q4_pack(None, 0, 32, None, None) == 0                                 # nothing to do
    assert lib.q8_quantize(C.c_void_p(0x1000), 2, 31, C.c_void_p(0x2000), C.c_void_p(0x3000), None) == -1
    assert lib.q8_quantize(C.c_void_p(0x1000), -1, 32, C.c_void_p(0x2000), C.c_void_p(0x3000), None) == -1


@pytest.mark.parametrize("kw,frag", [
    (dict(hidden=33), "hidden"), (dict(inter=0), "inter"), (dict(E=0), "n_experts"),
    (dict(E=2000), "n_experts"), (dict(k=0), "top_k"), (dict(k=9, E=8), "top_k"),
    (dict(k=33, E=64), "top_k"), (dict(ptr=0x10008), "aligned"),
])
def test_layer_checks(lib, kw, frag):
    L = _layer(**kw)
    rc = lib.moe_q4_route(C.byref(L), C.c_void_p(0x1000), 1, 16, None, None, None, 0, None)
    assert rc == -1 and frag in _err(lib)
    assert lib.moe_q4_route_workspace_bytes(C.byref(L), 16) == 0


def test_shared_pointers_required(lib):
    L = _layer(shared=1)
    L.s_down = None
    assert lib.moe_q4_decode(C.byref(L), C.c_void_p(0x1000), C.c_void_p(0x2000), None, None, 0, None) == -1
    assert "shared" in _err(lib)


@pytest.mark.parametrize("setup,frag", [
    (lambda L: setattr(L, "t_gate", 0x20000), "together"),                 # t_up, t_down missing
    (lambda L: [setattr(L, n, 0x20000) for n in ("t_gate", "t_up", "t_down", "ts_gate")], "together"),
    (lambda L: [setattr(L, n, 0x20008) for n in ("t_gate", "t_up", "t_down")], "aligned"),
])
def test_tile_order_pointer_checks(lib, setup, frag):
    L = _layer()
    setup(L)
    rc = lib.moe_q4_route(C.byref(L), C.c_void_p(0x1000), 1, 16, None, None, None, 0, None)
    assert rc == -1 and frag in _err(lib)


def test_tile_order_needs_k_multiple_of_64(lib):
    L = _layer(hidden=96, inter=128)
    L.t_gate = L.t_up = L.t_down = 0x20000
    assert lib.moe_q4_route(C.byref(L), C.c_void_p(0x1000), 1, 16, None, None, None, 0, None) == -1
    assert "64" in _err(lib)


def test_q4_tile_argument_checks(lib):
    assert lib.q4_tile(C.c_void_p(0x1000), 33, 64, C.c_void_p(0x100000), None) == -1      # rows % 32
    assert lib.q4_tile(C.c_void_p(0x1000), 32, 96, C.c_void_p(0x100000), None) == -1      # K % 64
    assert lib.q4_tile(C.c_void_p(0x1000), 32, 64, C.c_void_p(0x100008), None) == -1      # misaligned
    assert "aligned" in _err(lib)
    assert lib.q4_tile(C.c_void_p(0x1000), 32, 64, C.c_void_p(0x1100), None) == -1        # overlap
    assert "overlap" in _err(lib)
    assert lib.q4_tile(None, 32, 64, C.c_void_p(0x100000), None) == -1
    assert lib.q4_tile(None, 0, 64, None, None) == 0                                        # nothing to do


def test_q8w_tile_argument_checks(lib):
    assert lib.q8w_tile(C.c_void_p(0x1000), 33, 64, C.c_void_p(0x100000), None) == -1     # rows % 32
    assert lib.q8w_tile(C.c_void_p(0x1000), 32, 96, C.c_void_p(0x100000), None) == -1     # K % 64
    assert lib.q8w_tile(C.c_void_p(0x1001), 32, 64, C.c_void_p(0x100000), None) == -1     # q8 misaligned
    assert lib.q8w_tile(C.c_void_p(0x1000), 32, 64, C.c_void_p(0x100008), None) == -1     # tiled misaligned
    assert "aligned" in _err(lib)
    # 32 rows x 2 blocks x 34 B = 2176 B: ranges that overlap by one byte
    assert lib.q8w_tile(C.c_void_p(0x1000), 32, 64, C.c_void_p(0x1000 + 2176 - 16), None) == -1
    assert "overlap" in _err(lib)
    assert lib.q8w_tile(None, 32, 64, C.c_void_p(0x100000), None) == -1
    assert lib.q8w_tile(None, 0, 64, None, None) == 0                                       # nothing to do


def test_w4a8_gemm_argument_checks(lib):
    ok = C.c_void_p(0x100000)
    assert lib.moe_q4_w4a8_gemm(ok, 48, 128, ok, ok, 4, None, ok, None) == -1       # N % 32
    assert lib.moe_q4_w4a8_gemm(ok, 2097152, 128, ok, ok, 4, None, ok, None) == -1  # N / 32 > 65535
    assert lib.moe_q4_w4a8_gemm(ok, 64, 96, ok, ok, 4, None, ok, None) == -1        # K % 64
    assert lib.moe_q4_w4a8_gemm(ok, 64, 8192, ok, ok, 4, None, ok, None) == -1      # K > 4096
    assert "4096" in _err(lib)
    assert lib.moe_q4_w4a8_gemm(ok, 64, 128, ok, ok, -1, None, ok, None) == -1      # M < 0
    assert lib.moe_q4_w4a8_gemm(C.c_void_p(0x100008), 64, 128, ok, ok, 4, None, ok, None) == -1   # Wt alignment
    assert lib.moe_q4_w4a8_gemm(ok, 64, 128, None, ok, 4, None, ok, None) == -1     # NULL
    assert lib.moe_q4_w4a8_gemm(None, 64, 128, None, None, 0, None, None, None) == 0   # nothing to do


def test_decode_batch_argument_checks(lib):
    L = _layer()
    ok = C.c_void_p(0x10000)
    assert lib.moe_q4_decode_batch_workspace_bytes(C.byref(L), 33) == 0
    assert lib.moe_q4_decode_batch_workspace_bytes(C.byref(L), -1) == 0
    need = lib.moe_q4_decode_batch_workspace_bytes(C.byref(L), 32)
    assert need > lib.moe_q4_decode_batch_workspace_bytes(C.byref(L), 1) > 0
    assert lib.moe_q4_decode_batch(C.byref(L), ok, 33, ok, None, None, ok, need, None) == -1
    assert "M=33" in _err(lib)
    assert lib.moe_q4_decode_batch(C.byref(L), None, 2, ok, None, None, ok, need, None) == -1
    assert lib.moe_q4_decode_batch(C.byref(L), C.c_void_p(0x10004), 2, ok, None, None, ok, need, None) == -1
    assert lib.moe_q4_decode_batch(C.byref(L), ok, 2, ok, None, None, ok, 64, None) == -2
    assert lib.moe_q4_decode_batch(C.byref(L), None, 0, None, None, None, None, 0, None) == 0   # nothing to do
    wide = _layer(hidden=16384 + 32)
    assert lib.moe_q4_decode_batch(C.byref(wide), ok, 1, ok, None, None, ok, need, None) == -1


def test_q8_weight_checks(lib):
    assert lib.q8w_packed_bytes(512, 2048) == 512 * 64 * 34
    assert lib.q8w_packed_bytes(3, 33) == 0
    assert lib.q8w_pack(C.c_void_p(0x1000), 4, 33, C.c_void_p(0x2000), None) == -1
    assert lib.q8w_pack(None, 4, 32, C.c_void_p(0x2000), None) == -1
    assert lib.q8w_pack(C.c_void_p(0x1004), 4, 32, C.c_void_p(0x2000), None) == -1   # misaligned
    assert lib.q8w_pack(None, 0, 32, None, None) == 0
    L = _layer()
    L.weight_format = 2
    assert lib.moe_q4_route(C.byref(L), C.c_void_p(0x1000), 1, 16, None, None, None, 0, None) == -1
    assert "weight_format" in _err(lib)
    L.weight_format = 1                     # Q8_0 tile-order copies follow the Q4_0 rules
    L.t_gate = L.t_up = 0x20000
    assert lib.moe_q4_route(C.byref(L), C.c_void_p(0x1000), 1, 16, None, None, None, 0, None) == -1
    assert "together" in _err(lib)
    L = _layer()
    L.weight_format = 1                     # prefill refuses Q8_0 before anything else
    from bit_quantized_moe_q4_amd._lib import Routing
    R = Routing()
    R.topk_ids = R.topk_w = R.expert_offsets = R.perm = R.inv_perm = 0x30000
    assert lib.moe_q4_prefill(C.byref(L), C.c_void_p(0x1000), 4, C.byref(R), C.c_void_p(0x2000),
                              C.c_void_p(0x40000), 1 << 30, None) == -1
    assert "Q4_0" in _err(lib)


def test_decode_stack_checks(lib):
    from bit_quantized_moe_q4_amd._lib import Layer
    arr = (Layer * 2)(_layer(), _layer())
    ok = C.c_void_p(0x10000)
    need = lib.moe_q4_decode_stack_workspace_bytes(arr, 2)
    assert need > 0
    assert lib.moe_q4_decode_stack(arr, 0, None, None, 1e-6, None, 0, None) == 0       # nothing to do
    assert lib.moe_q4_decode_stack(arr, -1, ok, ok, 1e-6, ok, need, None) == -1
    assert lib.moe_q4_decode_stack(None, 2, ok, ok, 1e-6, ok, need, None) == -1
    assert lib.moe_q4_decode_stack(arr, 2, ok, ok, -1.0, ok, need, None) == -1
    assert "eps" in _err(lib)
    assert lib.moe_q4_decode_stack(arr, 2, ok, ok, 1e-6, ok, 64, None) == -2
    arr[1].hidden = 512
    assert lib.moe_q4_decode_stack(arr, 2, ok, ok, 1e-6, ok, need, None) == -1
    assert "hidden" in _err(lib)


def test_workspace_checks(lib):
    from bit_quantized_moe_q4_amd._lib import Routing
    L = _layer()
    R = Routing()
    R.topk_ids = R.topk_w = R.expert_offsets = R.perm = R.inv_perm = 0x4000
    need = lib.moe_q4_route_workspace_bytes(C.byref(L), 100)
    assert need > 0 and need % 256 == 0
    rc = lib.moe_q4_route(C.byref(L), C.c_void_p(0x1000), 1, 100, C.byref(R), None,
                          C.c_void_p(0x100000), need - 1, None)
    assert rc == -2 and "workspace" in _err(lib)
    rc = lib.moe_q4_route(C.byref(L), C.c_void_p(0x1000), 1, 100, C.byref(R), None,
                          C.c_void_p(0x100010), need, None)
    assert rc == -2 and "aligned" in _err(lib)
    rc = lib.moe_q4_route(C.byref(L), C.c_void_p(0x1000), 7, 100, C.byref(R), None,
                          C.c_void_p(0x100000), need, None)
    assert rc == -1 and "dtype" in _err(lib)
    rc = lib.moe_q4_route(C.byref(L), C.c_void_p(0x1000), 1, -1, C.byref(R), None, None, 0, None)
    assert rc == -1
    pneed = lib.moe_q4_prefill_workspace_bytes(C.byref(L), 100)
    assert pneed >= 100 * 2 * 128 * 2 + 100 * 2 * 256 * 2
    rc = lib.moe_q4_prefill(C.byref(L), C.c_void_p(0x1000), 100, C.byref(R), C.c_void_p(0x2000),
                            C.c_void_p(0x100000), pneed - 256, None)
    assert rc == -2
    # no tokens: valid, nothing enqueued
    assert lib.moe_q4_prefill(C.byref(L), None, 0, None, None, None, 0, None) == 0
    dneed = lib.moe_q4_decode_workspace_bytes(C.byref(L))
    assert dneed > 0
    rc = lib.moe_q4_decode(C.byref(L), C.c_void_p(0x1000), C.c_void_p(0x2000), None,
                           C.c_void_p(0x100000), dneed - 1, None)
    assert rc == -2


def test_prefill_status_checks(lib):
    L = _layer()
    n = C.c_int32(-7)
    # no tokens: nothing was launched, nothing to report (no device access)
    assert lib.moe_q4_prefill_status(C.byref(L), 0, None, 0, C.byref(n), None) == 0 and n.value == 0
    assert lib.moe_q4_prefill_status(C.byref(L), -1, None, 0, C.byref(n), None) == -1
    assert lib.moe_q4_prefill_status(C.byref(L), 8, None, 0, None, None) == -1
    pneed = lib.moe_q4_prefill_workspace_bytes(C.byref(L), 8)
    assert lib.moe_q4_prefill_status(C.byref(L), 8, C.c_void_p(0x100000), pneed - 1, C.byref(n), None) == -2
    # the bit of the test-only forced wait failure is accepted on top of a stage mask
    assert lib.moe_q4_prefill_stage(C.byref(L), None, 0, None, None, None, 0, 3 | 16, None) == 0
    assert lib.moe_q4_prefill_stage(C.byref(L), None, 0, None, None, None, 0, 16, None) == -1


def test_prefill_w4a8_checks(lib):
    L = _layer()
    x, y, ws = C.c_void_p(0x1000), C.c_void_p(0x2000), C.c_void_p(0x100000)
    from bit_quantized_moe_q4_amd._lib import Routing
    R = Routing()
    R.topk_ids = R.topk_w = R.expert_offsets = R.perm = R.inv_perm = 0x3000
    # row-major layer: the W4A8 form needs the tile-order copies
    assert lib.moe_q4_prefill_w4a8(C.byref(L), x, 8, C.byref(R), y, None, ws, 1 << 30, None) == -1
    assert "tile-order" in _err(lib)
    L.t_gate = L.t_up = L.t_down = 0x20000
    assert lib.moe_q4_prefill_w4a8(C.byref(L), x, -1, C.byref(R), y, None, ws, 1 << 30, None) == -1
    # no tokens: valid, nothing enqueued
    assert lib.moe_q4_prefill_w4a8(C.byref(L), None, 0, None, None, None, None, 0, None) == 0
    assert lib.moe_q4_prefill_w4a8(C.byref(L), x, 8, None, y, None, ws, 1 << 30, None) == -1
    # one workspace size serves both prefill forms
    pneed = lib.moe_q4_prefill_workspace_bytes(C.byref(L), 100)
    rows = 100 * 2
    assert pneed >= rows * 128 * 2 + rows * 256 * 2                    # bf16 h + routed outputs
    assert pneed >= rows * 256 * 2 + rows * 128 + rows * 4 * 4 + 100 * 256 + 100 * 8 * 4
    rc = lib.moe_q4_prefill_w4a8(C.byref(L), x, 100, C.byref(R), y, None, ws, pneed - 1, None)
    assert rc == -2
    assert lib.moe_q4_prefill_w4a8(C.byref(L), C.c_void_p(0x1008), 100, C.byref(R), y, None, ws, pneed,
                                   None) == -1 and "aligned" in _err(lib)
    big = _layer(hidden=8192, inter=128)
    big.t_gate = big.t_up = big.t_down = 0x20000
    assert lib.moe_q4_prefill_w4a8(C.byref(big), x, 8, C.byref(R), y, None, ws, 1 << 40, None) == -1
    assert "4096" in _err(lib)
    L.weight_format = 1
    assert lib.moe_q4_prefill_w4a8(C.byref(L), x, 8, C.byref(R), y, None, ws, 1 << 30, None) == -1
    L.weight_format = 0
    for bad in (0, 8, 16, -1):
        assert lib.moe_q4_prefill_w4a8_stage(C.byref(L), x, 8, C.byref(R), y, None, ws, 1 << 30, bad, None) == -1
    assert lib.moe_q4_prefill_w4a8_stage(C.byref(L), None, 0, None, None, None, None, 0, 3, None) == 0


def test_check_layer_tile_only(lib):
    # one resident copy: the tile-order matrices without the row-major ones
    L = _layer(hidden=2048, inter=512, E=128, k=8, shared=1)
    assert lib.moe_q4_check_layer(C.byref(L)) == 0
    L.t_gate = L.t_up = L.t_down = L.ts_gate = L.ts_up = L.ts_down = 0x20000
    assert lib.moe_q4_check_layer(C.byref(L)) == 0                 # both copies
    L.w_gate = L.w_up = L.w_down = L.s_gate = L.s_up = L.s_down = None
    assert lib.moe_q4_check_layer(C.byref(L)) == 0                 # tile order only
    L0 = _layer(hidden=2048, inter=512, E=128, k=8, shared=1)
    L0.t_gate = L0.t_up = L0.t_down = L0.ts_gate = L0.ts_up = L0.ts_down = 0x20000
    L0.w_gate = L0.w_up = L0.w_down = L0.s_gate = L0.s_up = L0.s_down = None
    L.w_gate = 0x10000                                             # a partial row-major set
    assert lib.moe_q4_check_layer(C.byref(L)) == -1 and "together" in _err(lib)
    L.w_gate = None
    L.t_gate = L.t_up = L.t_down = L.ts_gate = L.ts_up = L.ts_down = None
    assert lib.moe_q4_check_layer(C.byref(L)) == -1                # no matrices at all
    # a shape the tile-order down kernel does not cover (I = 4096) keeps its rows
    W = _layer(hidden=256, inter=4096, E=8, k=2)
    W.w_gate = W.w_up = W.w_down = None
    W.t_gate = W.t_up = W.t_down = 0x20000
    assert lib.moe_q4_check_layer(C.byref(W)) == -1 and "cover" in _err(lib)
    # and the entry points refuse such layers before any device access
    assert lib.moe_q4_decode_workspace_bytes(C.byref(W)) == 0
    assert lib.moe_q4_check_layer(None) == -1
    # a batch whose bf16 tokens pass 2^32 bytes needs the generic GEMM, which
    # reads the row-major matrices: refused for a tile-only layer
    from bit_quantized_moe_q4_amd._lib import Routing
    R = Routing()
    R.topk_ids = R.topk_w = R.expert_offsets = R.perm = R.inv_perm = 0x3000
    T = (1 << 20) + 1                                              # T * 2048 * 2 > 2^32 - 1
    rc = lib.moe_q4_prefill(C.byref(L0), C.c_void_p(0x1000), T, C.byref(R), C.c_void_p(0x2000),
                            C.c_void_p(0x100000), 1 << 45, None)
    assert rc == -1 and "too large" in _err(lib)


def test_decode_noalloc_checks(lib):
    # a layer whose decode scratch exceeds the fixed array is refused before any device call
    L = _layer(hidden=8192, inter=64, E=1024, k=2)
    assert lib.moe_q4_decode_workspace_bytes(C.byref(L)) > (1 << 20)
    rc = lib.moe_q4_decode_noalloc(C.byref(L), C.c_void_p(0x1000), C.c_void_p(0x2000), None)
    assert rc == -2 and "fixed array" in _err(lib)
    assert lib.moe_q4_decode_noalloc(C.byref(L), None, C.c_void_p(0x2000), None) == -1
    assert lib.moe_q4_decode_noalloc(C.byref(L), C.c_void_p(0x1008), C.c_void_p(0x2000), None) == -1
    assert "MOE_Q4_NOALLOC_SCRATCH_BYTES (1u << 20)" in open(HEADER).read()


def test_gemv_and_rmsnorm_checks(lib):
    assert lib.moe_q4_w4a8_gemv(C.c_void_p(0x1000), 4, 48, C.c_void_p(0x2000), C.c_void_p(0x3000),
                                None, C.c_void_p(0x4000), None) == -1
    assert lib.moe_q4_w4a8_gemv(None, 0, 64, None, None, None, None, None) == 0
    assert lib.moe_q4_rmsnorm(C.c_void_p(0x1000), 4, 40, 1e-6, C.c_void_p(0x2000), None, None) == -1
    assert lib.moe_q4_rmsnorm(C.c_void_p(0x1000), 4, 64, 1e-6, None, None, None) == -1
    assert lib.moe_q4_rmsnorm(None, 0, 64, 1e-6, None, None, None) == 0


def test_probe_mfma_checks(lib):
    ops = C.c_int64(-1)
    out = C.c_void_p(0x1000)
    assert lib.moe_q4_probe_mfma(3, 512, 100, out, C.byref(ops), None) == -1
    assert "kind" in _err(lib)
    assert lib.moe_q4_probe_mfma(0, 0, 100, out, C.byref(ops), None) == -1
    assert lib.moe_q4_probe_mfma(0, 512, 0, out, C.byref(ops), None) == -1
    assert lib.moe_q4_probe_mfma(0, 512, 100, None, C.byref(ops), None) == -1
    assert lib.moe_q4_probe_mfma(1, 512, 100, out, None, None) == -1
    assert ops.value == -1                   # nothing launched, nothing written


def test_binding_fails_loudly_without_library(tmp_path):
    code = (
        "import bit_quantized_moe_q4_amd._lib as L\n"
        "L.LIB_PATH = %r\n"
        "try:\n    L.lib()\nexcept RuntimeError as e:\n    print('RAISED', 'not built' in str(e))\n"
    ) % str(tmp_path / "missing.so")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert "RAISED True" in r.stdout, r.stdout + r.stderr
