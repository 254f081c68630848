"""Device-resident layers built from the seeded synthetic workloads.

The fp32 weights come from ``moe_synth`` (host), are copied to the device and
packed there by the library's ``q4_pack`` kernel; the fp32 copies are freed
afterwards, so only the packed layer stays resident in HBM.
"""
from __future__ import annotations

import numpy as np
import torch

import moe_synth

from . import MoELayer, q4_pack, q8w_pack


def _pack_host(a: np.ndarray, device, wfmt="q4") -> torch.Tensor:
    t = torch.from_numpy(a).to(device)
    p = q8w_pack(t) if wfmt == "q8" else q4_pack(t)
    del t
    return p


def device_layer(cfg: moe_synth.Config, layer: int = 0, device="cuda", weights=None,
                 threads: int = 16, tiles: bool = True, wfmt: str = "q4", rowmajor=None) -> MoELayer:
    """Pack layer `layer` of workload `cfg` on `device`.  `weights` (the dict
    from moe_synth.expert_weights) may be passed in to reuse a host copy;
    `tiles`, `wfmt` and `rowmajor` as in MoELayer."""
    W = weights if weights is not None else moe_synth.expert_weights(cfg, layer, threads=threads)
    wr = torch.from_numpy(moe_synth.router(cfg, layer)).to(device)
    b = moe_synth.router_bias(cfg, layer)
    bias = None if b is None else torch.from_numpy(b).to(device)
    pk = {k: (None if W[k] is None else _pack_host(W[k], device, wfmt))
          for k in ("gate", "up", "down", "s_gate", "s_up", "s_down")}
    L = MoELayer(wr, pk["gate"], pk["up"], pk["down"], cfg.k, router_bias=bias,
                 s_gate=pk["s_gate"], s_up=pk["s_up"], s_down=pk["s_down"], tiles=tiles, wfmt=wfmt,
                 rowmajor=rowmajor)
    torch.cuda.synchronize(device)
    return L


def device_tokens(cfg: moe_synth.Config, step: int = 0, T: int | None = None, layer: int = 0,
                  device="cuda"):
    """(x fp32 [T,H], x bf16 [T,H]) on the device; bf16 is round-to-nearest-even."""
    x = moe_synth.tokens(cfg, step=step, T=T, layer=layer)
    bits = moe_synth.to_bf16_bits(x)
    xb = torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(x).to(device), xb
