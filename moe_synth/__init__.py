"""Seeded synthetic inputs for the Q4_0 MoE expert-FFN layer.

This module only draws numbers: router matrices, fp32 expert weights (before
any quantisation), router biases and token activations.  It contains none of
the method's arithmetic (no packing, routing, quantisation or FFN); the
oracle and the HIP library each consume its arrays independently.

Every tensor has its own numpy PCG64 stream seeded by
``SeedSequence([config seed, layer, kind, index])`` so that any single expert
can be regenerated without the others and the result does not depend on the
order or the thread in which tensors are drawn.  Values are float32
standard normals (numpy's ziggurat) times sigma (one fp32 multiply).

The workloads (the pages give no model weights, prompts or datasets; these
shapes stand in for them):

=========  =======  =====  ===  ===  =  ======  ==================================
name       tokens   H      E    I    k  shared  notes
=========  =======  =====  ===  ===  =  ======  ==================================
tiny       16       256    8    128  2  no      x fp32 N(0,1), weights N(0,0.02)
decode     1/step   2048   128  512  8  yes     fresh x per step, 1000 steps
prefill    2048     2048   128  512  8  yes     x bf16 N(0,1)
skew       10240    2048   128  512  8  yes     bias b_e = 1.5*ln(1/(e+1))
stack      8192     2048   256  512  8  yes     40 layers, RMSNorm between
=========  =======  =====  ===  ===  =  ======  ==================================

128 routed experts is the 50%-pruned count of a 256-expert layer, as on the
pages' model; 256 is the unpruned count.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

# kinds of tensors (part of the seed)
K_ROUTER, K_GATE, K_UP, K_DOWN, K_SGATE, K_SUP, K_SDOWN, K_X, K_BIAS = range(9)
SEED_BASE = 0x5EED0000


@dataclass(frozen=True)
class Config:
    name: str
    index: int           # position in the workload list; part of the seed
    T: int               # tokens per prefill batch (1 for decode)
    H: int
    E: int
    I: int
    k: int
    shared: bool
    bias: str | None = None   # None or "zipf"
    layers: int = 1
    steps: int = 1            # decode steps with fresh inputs
    x_dtype: str = "bf16"     # prefill activations as handed to the layer
    sigma_w: float = 0.02
    sigma_r: float = 0.02
    sigma_x: float = 1.0
    extra: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    "tiny": Config("tiny", 0, T=16, H=256, E=8, I=128, k=2, shared=False, x_dtype="f32"),
    "decode": Config("decode", 1, T=1, H=2048, E=128, I=512, k=8, shared=True, steps=1000),
    "prefill": Config("prefill", 2, T=2048, H=2048, E=128, I=512, k=8, shared=True),
    "skew": Config("skew", 3, T=10240, H=2048, E=128, I=512, k=8, shared=True, bias="zipf"),
    "stack": Config("stack", 4, T=8192, H=2048, E=256, I=512, k=8, shared=True,
                    layers=40, steps=256),
}


def _rng(cfg_seed: int, layer: int, kind: int, index: int) -> np.random.Generator:
    ss = np.random.SeedSequence([cfg_seed, layer, kind, index])
    return np.random.Generator(np.random.PCG64(ss))


def normal(cfg_seed: int, layer: int, kind: int, index: int, shape, sigma: float,
           out: np.ndarray | None = None) -> np.ndarray:
    """One seeded float32 N(0, sigma) tensor."""
    if out is None:
        out = np.empty(shape, dtype=np.float32)
    _rng(cfg_seed, layer, kind, index).standard_normal(out=out, dtype=np.float32)
    np.multiply(out, np.float32(sigma), out=out)
    return out


def _fill_many(jobs, threads: int):
    if threads <= 1 or len(jobs) <= 1:
        for j in jobs:
            j()
        return
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda f: f(), jobs))


def router(cfg: Config, layer: int = 0) -> np.ndarray:
    """W_r [H, E] fp32."""
    return normal(cfg.seed, layer, K_ROUTER, 0, (cfg.H, cfg.E), cfg.sigma_r)


def router_bias(cfg: Config, layer: int = 0) -> np.ndarray | None:
    """Per-expert router bias [E] fp32 or None.  'zipf': 1.5*ln(1/(rank+1)),
    rank_e = e, which gives a Zipf-like expert load."""
    if cfg.bias is None:
        return None
    if cfg.bias == "zipf":
        return np.array([1.5 * math.log(1.0 / (e + 1)) for e in range(cfg.E)],
                        dtype=np.float32)
    raise ValueError(cfg.bias)


def expert_weights(cfg: Config, layer: int = 0, experts=None, threads: int = 8) -> dict:
    """fp32 expert weights.  gate/up [n, I, H], down [n, H, I] for the listed
    routed experts (default: all), plus the shared expert's s_gate/s_up [I, H]
    and s_down [H, I] when the layer has one."""
    ids = list(range(cfg.E)) if experts is None else list(experts)
    n = len(ids)
    gate = np.empty((n, cfg.I, cfg.H), np.float32)
    up = np.empty((n, cfg.I, cfg.H), np.float32)
    down = np.empty((n, cfg.H, cfg.I), np.float32)
    jobs = []
    for j, e in enumerate(ids):
        for kind, arr in ((K_GATE, gate), (K_UP, up), (K_DOWN, down)):
            jobs.append(lambda kind=kind, arr=arr, j=j, e=e:
                        normal(cfg.seed, layer, kind, e, arr.shape[1:], cfg.sigma_w, out=arr[j]))
    out = dict(gate=gate, up=up, down=down, s_gate=None, s_up=None, s_down=None)
    if cfg.shared:
        out["s_gate"] = np.empty((cfg.I, cfg.H), np.float32)
        out["s_up"] = np.empty((cfg.I, cfg.H), np.float32)
        out["s_down"] = np.empty((cfg.H, cfg.I), np.float32)
        for kind, key in ((K_SGATE, "s_gate"), (K_SUP, "s_up"), (K_SDOWN, "s_down")):
            arr = out[key]
            jobs.append(lambda kind=kind, arr=arr:
                        normal(cfg.seed, layer, kind, 0, arr.shape, cfg.sigma_w, out=arr))
    _fill_many(jobs, threads)
    return out


def tokens(cfg: Config, step: int = 0, T: int | None = None, layer: int = 0) -> np.ndarray:
    """Token activations [T, H] fp32 N(0, sigma_x).  `step` selects a fresh
    batch (decode steps use T=1 and step = 0..steps-1)."""
    T = cfg.T if T is None else T
    return normal(cfg.seed, layer, K_X, step, (T, cfg.H), cfg.sigma_x)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits to fp32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
