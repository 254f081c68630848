"""MI355X-native Q4_0 Mixture-of-Experts expert FFN (libmoe_q4.so binding).

Thin Python layer over the C ABI of include/moe_q4.h: the functions below
have the ABI's names and only marshal arguments (device pointers of torch
tensors, the current HIP stream, workspace buffers).  Every step of the
computation runs in the library's HIP kernels; torch only owns device memory
and streams.  If the library is not built, every call raises.

    layer = MoELayer.from_float(w_router, gate, up, down, top_k=8, s_gate=..)
    r = moe_q4_route(layer, x_bf16)             # router, top-k, permutation
    y = moe_q4_prefill(layer, x_bf16, r)        # grouped 4-bit GEMM prefill
    y1 = moe_q4_decode(layer, x_f32)            # one-token W4A8 decode
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import torch

from . import _lib

__all__ = [
    "q4_packed_bytes", "q4_pack", "q4_tile", "q8w_pack", "q8w_tile", "q8_quantize", "MoELayer", "Routing",
    "moe_q4_route_workspace_bytes", "moe_q4_route",
    "moe_q4_prefill_workspace_bytes", "moe_q4_prefill", "moe_q4_prefill_stage", "moe_q4_prefill_status",
    "moe_q4_prefill_w4a8", "moe_q4_prefill_w4a8_stage",
    "moe_q4_decode_workspace_bytes", "moe_q4_decode", "decode_workspace", "moe_q4_decode_noalloc", "moe_q4_decode_status",
    "moe_q4_decode_batch_workspace_bytes", "moe_q4_decode_batch",
    "LayerStack", "moe_q4_decode_stack_workspace_bytes", "moe_q4_decode_stack", "stack_workspace",
    "batch_workspace",
    "moe_q4_w4a8_gemv", "moe_q4_w4a8_gemm", "moe_q4_rmsnorm", "library_path",
]


def library_path() -> str:
    return _lib.LIB_PATH


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _s(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _dev(t, name):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


# ------------------------------------------------------------------ helpers
def q4_packed_bytes(rows: int, K: int) -> int:
    return int(_lib.lib().q4_packed_bytes(rows, K))


def q4_pack(w: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """fp32 [..., rows, K] device tensor -> uint8 [..., rows, K/32*18] Q4_0 blocks."""
    _dev(w, "w")
    K = w.shape[-1]
    rows = w.numel() // K
    if out is None:
        out = torch.empty(w.shape[:-1] + (K // 32 * 18,), dtype=torch.uint8, device=w.device)
    _lib.check(_lib.lib().q4_pack(_p(w), rows, K, _p(out), _s(stream)), "q4_pack")
    return out


def q8w_pack(w: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """fp32 [..., rows, K] device tensor -> uint8 [..., rows, K/32*34] Q8_0 blocks."""
    _dev(w, "w")
    K = w.shape[-1]
    rows = w.numel() // K
    if out is None:
        out = torch.empty(w.shape[:-1] + (K // 32 * 34,), dtype=torch.uint8, device=w.device)
    _lib.check(_lib.lib().q8w_pack(_p(w), rows, K, _p(out), _s(stream)), "q8w_pack")
    return out


def q4_tile(q4: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """uint8 [..., rows, K/32*18] Q4_0 blocks -> the same blocks in grouped-GEMM
    tile order (q4_tile in moe_q4.h); rows % 32 == 0, K % 64 == 0."""
    _dev(q4, "q4")
    rb = q4.shape[-1]
    K = rb // 18 * 32
    rows = q4.numel() // rb
    if out is None:
        out = torch.empty_like(q4)
    _lib.check(_lib.lib().q4_tile(_p(q4), rows, K, _p(out), _s(stream)), "q4_tile")
    return out


def q8w_tile(q8: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """uint8 [..., rows, K/32*34] Q8_0 blocks -> the same blocks in tile order
    (q8w_tile in moe_q4.h); rows % 32 == 0, K % 64 == 0."""
    _dev(q8, "q8")
    rb = q8.shape[-1]
    K = rb // 34 * 32
    rows = q8.numel() // rb
    if out is None:
        out = torch.empty_like(q8)
    _lib.check(_lib.lib().q8w_tile(_p(q8), rows, K, _p(out), _s(stream)), "q8w_tile")
    return out


def q8_quantize(x: torch.Tensor, stream=None):
    """fp32 [..., K] -> (int8 [..., K], fp32 scales [..., K/32])."""
    _dev(x, "x")
    K = x.shape[-1]
    rows = x.numel() // K
    q = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    d = torch.empty(x.shape[:-1] + (K // 32,), dtype=torch.float32, device=x.device)
    _lib.check(_lib.lib().q8_quantize(_p(x), rows, K, _p(q), _p(d), _s(stream)), "q8_quantize")
    return q, d


# ------------------------------------------------------------------ layer
class MoELayer:
    """Device-resident packed layer (moe_q4_layer).

    w_router fp32 [H, E]; gate/up uint8 [E, I, H/32*18]; down uint8
    [E, H, I/32*18]; optional router_bias fp32 [E] and shared expert
    s_gate/s_up uint8 [I, H/32*18], s_down uint8 [H, I/32*18].
    With `tiles` (the default) and H, I multiples of 64 the matrices are
    regrouped into the tile order (q4_tile), which every kernel reads; the
    row-major copies are then released (one resident copy of the weights)
    unless `rowmajor` is True or the library does not cover the shape
    without them (moe_q4_check_layer); `rowmajor=False` makes that an error.
    wfmt="q8": the matrices are Q8_0 blocks (34 bytes per 32 weights;
    routing and decode only), tiles by q8w_tile.
    """

    def __init__(self, w_router, gate, up, down, top_k, router_bias=None,
                 s_gate=None, s_up=None, s_down=None, tiles=True, stream=None, wfmt="q4",
                 rowmajor=None):
        for n, t in (("w_router", w_router), ("gate", gate), ("up", up), ("down", down),
                     ("router_bias", router_bias), ("s_gate", s_gate), ("s_up", s_up),
                     ("s_down", s_down)):
            _dev(t, n)
        if wfmt not in ("q4", "q8"):
            raise ValueError("wfmt must be 'q4' or 'q8'")
        self.w_router, self.router_bias = w_router, router_bias
        self.gate, self.up, self.down = gate, up, down
        self.s_gate, self.s_up, self.s_down = s_gate, s_up, s_down
        self.hidden, self.n_experts = int(w_router.shape[0]), int(w_router.shape[1])
        self.inter = int(gate.shape[1])
        self.top_k = int(top_k)
        self.has_shared = s_gate is not None
        self.wfmt = wfmt
        self.tiles = None
        if tiles and self.hidden % 64 == 0 and self.inter % 64 == 0:
            tile = q8w_tile if wfmt == "q8" else q4_tile
            tl = lambda t: None if t is None else tile(t, stream=stream)  # noqa: E731
            self.tiles = dict(gate=tl(gate), up=tl(up), down=tl(down),
                              s_gate=tl(s_gate), s_up=tl(s_up), s_down=tl(s_down))
        self._c = self._struct()
        if self.tiles is not None and rowmajor is not True:
            kept = (self.gate, self.up, self.down, self.s_gate, self.s_up, self.s_down)
            self.gate = self.up = self.down = self.s_gate = self.s_up = self.s_down = None
            st = self._struct()
            if _lib.lib().moe_q4_check_layer(C.byref(st)) == _lib.MOE_Q4_OK:
                self._c = st
                # the tile kernels read the row-major copies on `stream`: the
                # memory is reused only after them
                s_ = stream if stream is not None else torch.cuda.current_stream()
                for t in kept:
                    if t is not None:
                        t.record_stream(s_)
            elif rowmajor is False:
                raise RuntimeError("moe_q4_check_layer refused a layer without row-major matrices: %s"
                                   % _lib.lib().moe_q4_last_error().decode(errors="replace"))
            else:
                self.gate, self.up, self.down, self.s_gate, self.s_up, self.s_down = kept

    def _struct(self):
        st = _lib.Layer()
        st.hidden, st.inter, st.n_experts, st.top_k = self.hidden, self.inter, self.n_experts, self.top_k
        st.has_shared = 1 if self.has_shared else 0
        st.w_router, st.router_bias = _p(self.w_router), _p(self.router_bias)
        st.w_gate, st.w_up, st.w_down = _p(self.gate), _p(self.up), _p(self.down)
        st.s_gate, st.s_up, st.s_down = _p(self.s_gate), _p(self.s_up), _p(self.s_down)
        st.weight_format = _lib.WEIGHTS_Q8_0 if self.wfmt == "q8" else _lib.WEIGHTS_Q4_0
        if self.tiles is not None:
            T_ = self.tiles
            st.t_gate, st.t_up, st.t_down = _p(T_["gate"]), _p(T_["up"]), _p(T_["down"])
            st.ts_gate, st.ts_up, st.ts_down = _p(T_["s_gate"]), _p(T_["s_up"]), _p(T_["s_down"])
        return st

    @classmethod
    def from_float(cls, w_router, gate, up, down, top_k, router_bias=None,
                   s_gate=None, s_up=None, s_down=None, tiles=True, stream=None, wfmt="q4", rowmajor=None):
        """Pack fp32 device weights with the library's q4_pack (or q8w_pack) kernel."""
        pack = q8w_pack if wfmt == "q8" else q4_pack
        pk = lambda t: None if t is None else pack(t, stream=stream)  # noqa: E731
        return cls(w_router, pk(gate), pk(up), pk(down), top_k, router_bias,
                   pk(s_gate), pk(s_up), pk(s_down), tiles=tiles, stream=stream, wfmt=wfmt, rowmajor=rowmajor)

    @property
    def rowmajor(self) -> bool:
        """Whether the layer holds the row-major matrices."""
        return self.gate is not None

    def clone(self) -> "MoELayer":
        """A copy of the layer in new device memory (same layouts)."""
        c = MoELayer.__new__(MoELayer)
        c.__dict__.update(self.__dict__)
        cl = lambda t: None if t is None else t.clone()  # noqa: E731
        for n in ("w_router", "router_bias", "gate", "up", "down", "s_gate", "s_up", "s_down"):
            setattr(c, n, cl(getattr(self, n)))
        c.tiles = None if self.tiles is None else {n: cl(t) for n, t in self.tiles.items()}
        c._c = c._struct()
        return c

    def struct_ptr(self):
        return C.byref(self._c)

    def resident_bytes(self) -> int:
        """Device bytes the layer holds (router, packed matrices, tile-order copies)."""
        ts = [self.w_router, self.router_bias, self.gate, self.up, self.down, self.s_gate, self.s_up, self.s_down]
        if self.tiles:
            ts += list(self.tiles.values())
        return sum(t.numel() * t.element_size() for t in ts if t is not None)


@dataclass
class Routing:
    """Device buffers of moe_q4_routing for a T-token batch."""
    topk_ids: torch.Tensor      # int32 [T, k]
    topk_w: torch.Tensor        # fp32  [T, k]
    expert_offsets: torch.Tensor  # int32 [E+1]
    perm: torch.Tensor          # int32 [T*k]
    inv_perm: torch.Tensor      # int32 [T*k]
    logits: torch.Tensor | None = None

    @classmethod
    def empty(cls, T, k, E, device, logits=False):
        i32 = dict(dtype=torch.int32, device=device)
        return cls(torch.empty((T, k), **i32), torch.empty((T, k), dtype=torch.float32, device=device),
                   torch.empty(E + 1, **i32), torch.empty(T * k, **i32), torch.empty(T * k, **i32),
                   torch.empty((T, E), dtype=torch.float32, device=device) if logits else None)

    def cstruct(self):
        r = _lib.Routing()
        r.topk_ids, r.topk_w = _p(self.topk_ids), _p(self.topk_w)
        r.expert_offsets, r.perm, r.inv_perm = _p(self.expert_offsets), _p(self.perm), _p(self.inv_perm)
        return r


def _ws(nbytes, device, ws):
    if ws is not None:
        return ws
    # 256-byte aligned by the caching allocator
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ prefill
def moe_q4_route_workspace_bytes(layer: MoELayer, T: int) -> int:
    return int(_lib.lib().moe_q4_route_workspace_bytes(layer.struct_ptr(), T))


def moe_q4_route(layer: MoELayer, x: torch.Tensor, out: Routing | None = None,
                 logits: bool = False, ws: torch.Tensor | None = None, stream=None) -> Routing:
    """Router + top-k + permutation of x [T, H] (fp32 or bf16)."""
    _dev(x, "x")
    T = int(x.shape[0])
    if x.dtype == torch.bfloat16:
        dt = _lib.MOE_Q4_BF16
    elif x.dtype == torch.float32:
        dt = _lib.MOE_Q4_F32
    else:
        raise ValueError("x must be float32 or bfloat16")
    if out is None:
        out = Routing.empty(T, layer.top_k, layer.n_experts, x.device, logits=logits)
    nb = moe_q4_route_workspace_bytes(layer, T)
    w = _ws(nb, x.device, ws)
    rs = out.cstruct()
    _lib.check(_lib.lib().moe_q4_route(layer.struct_ptr(), _p(x), dt, T, C.byref(rs), _p(out.logits),
                                       _p(w), w.numel(), _s(stream)), "moe_q4_route")
    return out


def moe_q4_prefill_workspace_bytes(layer: MoELayer, T: int) -> int:
    return int(_lib.lib().moe_q4_prefill_workspace_bytes(layer.struct_ptr(), T))


def moe_q4_prefill(layer: MoELayer, x_bf16: torch.Tensor, routing: Routing,
                   y: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
    """Grouped 4-bit GEMM prefill: y [T, H] fp32."""
    _dev(x_bf16, "x_bf16")
    if x_bf16.dtype != torch.bfloat16:
        raise ValueError("x_bf16 must be bfloat16")
    T = int(x_bf16.shape[0])
    if y is None:
        y = torch.empty((T, layer.hidden), dtype=torch.float32, device=x_bf16.device)
    nb = moe_q4_prefill_workspace_bytes(layer, T)
    w = _ws(nb, x_bf16.device, ws)
    rs = routing.cstruct()
    _lib.check(_lib.lib().moe_q4_prefill(layer.struct_ptr(), _p(x_bf16), T, C.byref(rs), _p(y),
                                         _p(w), w.numel(), _s(stream)), "moe_q4_prefill")
    return y


def moe_q4_prefill_stage(layer: MoELayer, x_bf16: torch.Tensor, routing: Routing,
                         y: torch.Tensor, ws: torch.Tensor, stages: int, stream=None) -> torch.Tensor:
    """Run some stages of moe_q4_prefill (mask of _lib.STAGE_GATEUP | _DOWN | _COMBINE)
    with a caller-held workspace `ws` (its first bytes hold h after GATEUP)."""
    _dev(x_bf16, "x_bf16")
    T = int(x_bf16.shape[0])
    rs = routing.cstruct()
    _lib.check(_lib.lib().moe_q4_prefill_stage(layer.struct_ptr(), _p(x_bf16), T, C.byref(rs), _p(y),
                                               _p(ws), ws.numel(), int(stages), _s(stream)),
               "moe_q4_prefill_stage")
    return y


def moe_q4_prefill_status(layer: MoELayer, T: int, ws: torch.Tensor, stream=None) -> int:
    """Down units of the last fused prefill launch on `ws` whose bounded wait
    gave up (0: all waits ended normally).  Waits for the stream."""
    n = C.c_int32(-1)
    _lib.check(_lib.lib().moe_q4_prefill_status(layer.struct_ptr(), int(T), _p(ws), ws.numel(), C.byref(n),
                                                _s(stream)), "moe_q4_prefill_status")
    return int(n.value)


def moe_q4_prefill_w4a8(layer: MoELayer, x_bf16: torch.Tensor, routing: Routing,
                        y: torch.Tensor | None = None, gate_dots: torch.Tensor | None = None,
                        ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Grouped prefill in the W4A8 form (int8 block dots): y [T, H] fp32.
    gate_dots: None, or int32 [T*k + T*S, I, H/32] receiving every gate block dot."""
    _dev(x_bf16, "x_bf16")
    if x_bf16.dtype != torch.bfloat16:
        raise ValueError("x_bf16 must be bfloat16")
    T = int(x_bf16.shape[0])
    if y is None:
        y = torch.empty((T, layer.hidden), dtype=torch.float32, device=x_bf16.device)
    if gate_dots is not None:
        rows = T * layer.top_k + (T if layer.has_shared else 0)
        if gate_dots.dtype != torch.int32 or gate_dots.numel() < rows * layer.inter * (layer.hidden // 32):
            raise ValueError("gate_dots must be int32 with [T*k + T*S, I, H/32] elements")
        _dev(gate_dots, "gate_dots")
    nb = moe_q4_prefill_workspace_bytes(layer, T)
    w = _ws(nb, x_bf16.device, ws)
    rs = routing.cstruct()
    _lib.check(_lib.lib().moe_q4_prefill_w4a8(layer.struct_ptr(), _p(x_bf16), T, C.byref(rs), _p(y),
                                              _p(gate_dots), _p(w), w.numel(), _s(stream)),
               "moe_q4_prefill_w4a8")
    return y


def moe_q4_prefill_w4a8_stage(layer: MoELayer, x_bf16: torch.Tensor, routing: Routing, y: torch.Tensor,
                              ws: torch.Tensor, stages: int, gate_dots: torch.Tensor | None = None,
                              stream=None) -> torch.Tensor:
    """Some stages of moe_q4_prefill_w4a8 (mask of _lib.STAGE_GATEUP | _DOWN | _COMBINE)
    with a caller-held workspace."""
    _dev(x_bf16, "x_bf16")
    T = int(x_bf16.shape[0])
    rs = routing.cstruct()
    _lib.check(_lib.lib().moe_q4_prefill_w4a8_stage(layer.struct_ptr(), _p(x_bf16), T, C.byref(rs), _p(y),
                                                    _p(gate_dots), _p(ws), ws.numel(), int(stages), _s(stream)),
               "moe_q4_prefill_w4a8_stage")
    return y


# ------------------------------------------------------------------ decode
def moe_q4_decode_workspace_bytes(layer: MoELayer) -> int:
    return int(_lib.lib().moe_q4_decode_workspace_bytes(layer.struct_ptr()))


def decode_workspace(layer: MoELayer, device=None) -> torch.Tensor:
    """A decode workspace, zero-filled (the one-launch step keeps its call
    counter in it; each call leaves it ready for the next)."""
    dev = device if device is not None else layer.w_router.device
    return torch.zeros(max(moe_q4_decode_workspace_bytes(layer), 1), dtype=torch.uint8, device=dev)


def moe_q4_decode_status(layer: MoELayer, ws: torch.Tensor, stream=None) -> int:
    """Waits of the one-launch decode on `ws` that gave up since the last
    query (0: every step completed normally); resets the count.  Waits for the
    stream."""
    n = C.c_int32(-1)
    _lib.check(_lib.lib().moe_q4_decode_status(layer.struct_ptr(), _p(ws), ws.numel(), C.byref(n), _s(stream)),
               "moe_q4_decode_status")
    return int(n.value)


def moe_q4_decode(layer: MoELayer, x: torch.Tensor, y: torch.Tensor | None = None,
                  ws: torch.Tensor | None = None, trace: bool = False, stream=None):
    """One-token W4A8 decode: x [H] fp32 -> y [H] fp32 (and the trace dict)."""
    _dev(x, "x")
    if x.dtype != torch.float32:
        raise ValueError("x must be float32")
    if y is None:
        y = torch.empty(layer.hidden, dtype=torch.float32, device=x.device)
    if ws is None:
        ws = decode_workspace(layer, x.device)
    tr, tc = None, None
    if trace:
        H, I, k = layer.hidden, layer.inter, layer.top_k
        ns = k + (1 if layer.has_shared else 0)
        d = x.device
        tr = dict(logits=torch.empty(layer.n_experts, dtype=torch.float32, device=d),
                  ids=torch.empty(k, dtype=torch.int32, device=d),
                  w=torch.empty(k, dtype=torch.float32, device=d),
                  qx=torch.empty(H, dtype=torch.int8, device=d),
                  dx=torch.empty(H // 32, dtype=torch.float32, device=d),
                  qh=torch.empty((ns, I), dtype=torch.int8, device=d),
                  dh=torch.empty((ns, I // 32), dtype=torch.float32, device=d))
        tc = _lib.DecodeTrace(**{k_: _p(v) for k_, v in tr.items()})
    _lib.check(_lib.lib().moe_q4_decode(layer.struct_ptr(), _p(x), _p(y),
                                        C.byref(tc) if tc is not None else None,
                                        _p(ws), ws.numel(), _s(stream)), "moe_q4_decode")
    return (y, tr) if trace else y


def moe_q4_decode_noalloc(layer: MoELayer, x: torch.Tensor, y: torch.Tensor, stream=None) -> torch.Tensor:
    """One-token decode into the caller's y [H] fp32 with the library's fixed
    per-GPU scratch array (no workspace, nothing allocated)."""
    _dev(x, "x")
    _dev(y, "y")
    if x.dtype != torch.float32 or y.dtype != torch.float32:
        raise ValueError("x and y must be float32")
    _lib.check(_lib.lib().moe_q4_decode_noalloc(layer.struct_ptr(), _p(x), _p(y), _s(stream)),
               "moe_q4_decode_noalloc")
    return y


class LayerStack:
    """A host array of moe_q4_layer descriptors for moe_q4_decode_stack (the
    MoELayer objects must stay alive while it is used)."""

    def __init__(self, layers):
        self.layers = list(layers)
        arr = (_lib.Layer * len(self.layers))()
        for i, L in enumerate(self.layers):
            arr[i] = L._c
        self._arr = arr
        self.hidden = self.layers[0].hidden if self.layers else 0

    def __len__(self):
        return len(self.layers)

    def ptr(self):
        return C.cast(self._arr, C.c_void_p)


def moe_q4_decode_stack_workspace_bytes(stack: LayerStack) -> int:
    return int(_lib.lib().moe_q4_decode_stack_workspace_bytes(stack.ptr(), len(stack)))


def stack_workspace(stack: LayerStack, device=None) -> torch.Tensor:
    """A zero-filled workspace for moe_q4_decode_stack."""
    dev = device if device is not None else stack.layers[0].w_router.device
    return torch.zeros(max(1, moe_q4_decode_stack_workspace_bytes(stack)), dtype=torch.uint8, device=dev)


def moe_q4_decode_stack(stack: LayerStack, x: torch.Tensor, eps: float = 1e-6,
                        y: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None):
    """One decode step through the stack: x [H] fp32 -> y [H] fp32, the last
    layer's output (RMSNorm between layers, fused into each next layer)."""
    _dev(x, "x")
    if y is None:
        y = torch.empty(stack.hidden, dtype=torch.float32, device=x.device)
    if ws is None:
        ws = stack_workspace(stack, x.device)
    _lib.check(_lib.lib().moe_q4_decode_stack(stack.ptr(), len(stack), _p(x), _p(y), float(eps), _p(ws),
                                              ws.numel(), _s(stream)), "moe_q4_decode_stack")
    return y


def moe_q4_decode_batch_workspace_bytes(layer: MoELayer, M: int) -> int:
    return int(_lib.lib().moe_q4_decode_batch_workspace_bytes(layer.struct_ptr(), int(M)))


def batch_workspace(layer: MoELayer, M: int, device=None) -> torch.Tensor:
    """A zero-filled workspace for moe_q4_decode_batch of M tokens."""
    dev = device if device is not None else layer.w_router.device
    return torch.zeros(max(1, moe_q4_decode_batch_workspace_bytes(layer, M)), dtype=torch.uint8, device=dev)


def moe_q4_decode_batch(layer: MoELayer, x: torch.Tensor, y: torch.Tensor | None = None,
                        ws: torch.Tensor | None = None, routing: bool = False, stream=None):
    """Decode of M <= 32 independent tokens: x [M, H] fp32 -> y [M, H] fp32, each
    row bit-identical to moe_q4_decode of that token (with routing=True also
    the ids [M, k] int32 and weights [M, k] fp32)."""
    _dev(x, "x")
    if x.dtype != torch.float32 or x.dim() != 2:
        raise ValueError("x must be float32 [M, H]")
    M = int(x.shape[0])
    if y is None:
        y = torch.empty((M, layer.hidden), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = batch_workspace(layer, M, x.device)
    ids = w = None
    if routing:
        ids = torch.empty((M, layer.top_k), dtype=torch.int32, device=x.device)
        w = torch.empty((M, layer.top_k), dtype=torch.float32, device=x.device)
    _lib.check(_lib.lib().moe_q4_decode_batch(layer.struct_ptr(), _p(x), M, _p(y), _p(ids), _p(w),
                                              _p(ws), ws.numel(), _s(stream)), "moe_q4_decode_batch")
    return (y, ids, w) if routing else y


def moe_q4_w4a8_gemv(W: torch.Tensor, N: int, K: int, qa: torch.Tensor, da: torch.Tensor,
                     with_dots: bool = True, stream=None):
    """The decode row program on one packed matrix -> (dots int32 [N, K/32] | None, out fp32 [N])."""
    for n, t in (("W", W), ("qa", qa), ("da", da)):
        _dev(t, n)
    dots = torch.empty((N, K // 32), dtype=torch.int32, device=W.device) if with_dots else None
    out = torch.empty(N, dtype=torch.float32, device=W.device)
    _lib.check(_lib.lib().moe_q4_w4a8_gemv(_p(W), N, K, _p(qa), _p(da), _p(dots), _p(out), _s(stream)),
               "moe_q4_w4a8_gemv")
    return dots, out


def moe_q4_w4a8_gemm(Wt: torch.Tensor, N: int, K: int, qa: torch.Tensor, da: torch.Tensor,
                     with_dots: bool = False, stream=None):
    """The row program for M tokens on int8 MFMA: Wt (tile order, q4_tile), qa
    int8 [M, K], da fp32 [M, K/32] -> (dots int32 [M, N, K/32] | None, out fp32 [M, N])."""
    for n, t in (("Wt", Wt), ("qa", qa), ("da", da)):
        _dev(t, n)
    M = int(qa.shape[0])
    dots = torch.empty((M, N, K // 32), dtype=torch.int32, device=Wt.device) if with_dots else None
    out = torch.empty((M, N), dtype=torch.float32, device=Wt.device)
    _lib.check(_lib.lib().moe_q4_w4a8_gemm(_p(Wt), N, K, _p(qa), _p(da), M, _p(dots), _p(out), _s(stream)),
               "moe_q4_w4a8_gemm")
    return dots, out


PROBE_BF16, PROBE_I8, PROBE_F32_K1 = 0, 1, 2


def moe_q4_probe_mfma(kind: int, blocks: int, iters: int, out: torch.Tensor, stream=None) -> int:
    """One launch of the matrix-core rate probe (kind PROBE_BF16 / PROBE_I8 /
    PROBE_F32_K1) into `out` (device float32, blocks * 256 elements); returns
    the operation count of the launch (time it on `stream`)."""
    _dev(out, "out")
    if out.dtype != torch.float32 or out.numel() < blocks * 256:
        raise ValueError("out must be float32 with blocks * 256 elements")
    ops = C.c_int64(0)
    _lib.check(_lib.lib().moe_q4_probe_mfma(int(kind), int(blocks), int(iters), _p(out), C.byref(ops),
                                            _s(stream)), "moe_q4_probe_mfma")
    return int(ops.value)


def moe_q4_rmsnorm(y: torch.Tensor, eps: float = 1e-6, f32: bool = True, bf16: bool = False,
                   stream=None, out_f32: torch.Tensor | None = None, out_bf16: torch.Tensor | None = None):
    """Unit-gain RMSNorm of y [T, H] fp32 -> (fp32 | None, bf16 | None); out_f32 /
    out_bf16 may be given (then nothing is allocated)."""
    _dev(y, "y")
    T, H = int(y.shape[0]), int(y.shape[1])
    o32 = out_f32 if out_f32 is not None else (torch.empty_like(y) if f32 else None)
    o16 = out_bf16 if out_bf16 is not None else (
        torch.empty((T, H), dtype=torch.bfloat16, device=y.device) if bf16 else None)
    _lib.check(_lib.lib().moe_q4_rmsnorm(_p(y), T, H, float(eps), _p(o32), _p(o16), _s(stream)),
               "moe_q4_rmsnorm")
    return o32, o16
