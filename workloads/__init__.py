"""Synthetic workloads: tensor shapes of the five shard configurations and seeded input generators.

This module holds only shapes and random draws.  It contains none of the sharded step's
arithmetic (no layout math, no reduction, no optimizer, no bf16 rounding) and is imported by the
tests and the benchmark, never by the oracle or by the GPU library.

bf16 inputs are drawn as float32 and keep the top 16 bits of the float32 pattern (rounded toward
zero), so the drawn gradients are bf16 values whose distribution is the stated normal one.
``N(0, s)`` means standard deviation s.
"""

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

ADAMW = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def llama_layer(d, n_q, n_kv, head_dim, ffn):
    """Parameter counts of one Llama-style decoder layer in flatten order:
    q, k, v, o projections, SwiGLU gate, up, down, attention norm, ffn norm."""
    q = d * n_q * head_dim
    kv = d * n_kv * head_dim
    return [q, kv, kv, q, d * ffn, d * ffn, ffn * d, d, d]


@dataclass
class Workload:
    name: str
    description: str
    sizes: List[int]
    pad_multiple: int
    world_size: int
    rank: int
    fan_in: int
    steps: int
    grad_std: float
    master_init: tuple                 # ("uniform", a) -> U(-a, a) ; ("normal", s) -> N(0, s)
    warm_steps: int = 0
    wd_mask: Optional[List[bool]] = None
    heavy_tail: Optional[tuple] = None  # (probability, factor) applied in float32 before bf16
    nan_padding_grads: bool = False
    hp: dict = field(default_factory=lambda: dict(ADAMW))

    @property
    def total(self):
        return sum(-(-s // self.pad_multiple) * self.pad_multiple for s in self.sizes)


def _many_small(seed=0, count=2000, top=4_000_000):
    rng = np.random.default_rng(seed)
    u = rng.uniform(0.0, math.log(top), count)
    sizes = np.clip(np.floor(np.exp(u)), 1, top).astype(np.int64)
    wd = rng.random(count) < 0.5
    return [int(s) for s in sizes], [bool(w) for w in wd]


LAYER_7B = llama_layer(4096, 32, 8, 128, 14336)        # 218,112,000 parameters
LAYER_70B = llama_layer(8192, 64, 8, 128, 28672)       # 855,654,400 parameters
_small_sizes, _small_wd = _many_small()

WORKLOADS = {
    "p1000003_n8_rank3": Workload(
        "p1000003_n8_rank3",
        "flat P=1,000,003, 8 ranks, rank 3's slice, fan-in 8, 3 steps",
        [1_000_003], 1, 8, 3, 8, 3, 1e-2, ("uniform", 0.05)),
    "llama_layer_n8_rank0": Workload(
        "llama_layer_n8_rank0",
        "one Llama-style layer (d 4096, 32/8 heads, ffn 14336, 218,112,000 params), 8 ranks, "
        "rank 0, fan-in 8, moments from 10 warm steps, 10 steps",
        list(LAYER_7B), 1, 8, 0, 8, 10, 1e-3, ("normal", 0.02), warm_steps=10),
    "dense7b_n8_rank0": Workload(
        "dense7b_n8_rank0",
        "7B-shaped dense model (embedding, 32 Llama layers, LM head; 7,241,728,000 params), "
        "8 ranks, rank 0's 905,216,000-element slice, fan-in 8, 5 steps",
        [32000 * 4096] + LAYER_7B * 32 + [32000 * 4096], 1, 8, 0, 8, 5, 1e-3, ("normal", 0.02)),
    "dense70b_n64_rank0": Workload(
        "dense70b_n64_rank0",
        "70B-shaped dense model (embedding, 80 layers d 8192 ffn 28672 64/8 heads, LM head; "
        "68,976,640,000 params), 64 ranks, rank 0's 1,077,760,000-element slice, pre-reduced "
        "gradient (fan-in 1) with 0.1% of entries x100, 5 steps",
        [32000 * 8192] + LAYER_70B * 80 + [32000 * 8192], 1, 64, 0, 1, 5, 1e-3, ("normal", 0.02),
        heavy_tail=(1e-3, 100.0)),
    "many_small_n16_rank3": Workload(
        "many_small_n16_rank3",
        "2,000 tensors, sizes log-uniform in [1, 4M] (seed 0; 529,495,435 real params), each "
        "padded to a multiple of 16, 16 ranks, rank 3's slice, per-tensor weight-decay mask, "
        "fan-in 4, NaN gradients in the padding, 5 steps",
        _small_sizes, 16, 16, 3, 4, 5, 1e-3, ("normal", 0.02), wd_mask=_small_wd,
        nan_padding_grads=True),
}

ORDER = ["p1000003_n8_rank3", "llama_layer_n8_rank0", "dense7b_n8_rank0", "dense70b_n64_rank0",
         "many_small_n16_rank3"]


# ----------------------------------------------------------------------------- numpy (host) draws

def _truncate_to_bf16_bits(x32):
    return (np.asarray(x32, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def np_state(w: Workload, n, seed):
    """Initial fp32 master, m, v of an n-element slice (m = v = 0)."""
    rng = np.random.default_rng([seed, 0xA11CE])
    kind, a = w.master_init
    if kind == "uniform":
        master = rng.uniform(-a, a, n).astype(np.float32)
    else:
        master = (rng.standard_normal(n, dtype=np.float32) * np.float32(a)).astype(np.float32)
    return master, np.zeros(n, np.float32), np.zeros(n, np.float32)


def np_grads(w: Workload, n, step, seed):
    """F bf16 contributions (uint16 bit patterns) of an n-element slice for 1-based ``step``."""
    out = []
    for r in range(w.fan_in):
        rng = np.random.default_rng([seed, step, r])
        x = rng.standard_normal(n, dtype=np.float32) * np.float32(w.grad_std)
        if w.heavy_tail is not None:
            p, f = w.heavy_tail
            x = np.where(rng.random(n) < p, x * np.float32(f), x).astype(np.float32)
        out.append(_truncate_to_bf16_bits(x))
    return out


def np_bf16_normal(key, n, std):
    """n bf16 bit patterns ~ N(0, std) (uint16), from a seed sequence ``key``."""
    rng = np.random.default_rng(key)
    return _truncate_to_bf16_bits(rng.standard_normal(n, dtype=np.float32) * np.float32(std))


def np_f32_normal(key, n, std):
    rng = np.random.default_rng(key)
    return (rng.standard_normal(n, dtype=np.float32) * np.float32(std)).astype(np.float32)


def np_f32_uniform(key, n, lo, hi):
    rng = np.random.default_rng(key)
    return rng.uniform(lo, hi, n).astype(np.float32)


# ----------------------------------------------------------------------------- torch (device) draws

def torch_state(w: Workload, n, seed, device):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 1_000_003 + 17)
    kind, a = w.master_init
    if kind == "uniform":
        master = torch.rand(n, generator=gen, device=device, dtype=torch.float32).mul_(2 * a).sub_(a)
    else:
        master = torch.randn(n, generator=gen, device=device, dtype=torch.float32).mul_(a)
    z = torch.zeros(n, device=device, dtype=torch.float32)
    return master, z, z.clone()


def torch_grads_into(w: Workload, bufs, step, seed):
    """Fill the F int16 device tensors ``bufs`` with bf16 bit patterns for 1-based ``step``."""
    import torch
    for r, buf in enumerate(bufs):
        gen = torch.Generator(device=buf.device)
        gen.manual_seed(((seed * 1009 + step) * 131 + r) * 7919 + 5)
        x = torch.randn(buf.numel(), generator=gen, device=buf.device, dtype=torch.float32)
        x.mul_(w.grad_std)
        if w.heavy_tail is not None:
            p, f = w.heavy_tail
            hit = torch.rand(buf.numel(), generator=gen, device=buf.device) < p
            x = torch.where(hit, x * f, x)
        buf.copy_((x.view(torch.int32) >> 16).to(torch.int16))
        del x
    return bufs
