"""Planted-Tucker synthetic KV caches and the named workload shapes.

A cache item is one layer group's K (or V) tensor X[L][H][T][d] (d fastest).
It is built as a Tucker tensor with orthonormal token and feature factors, a
core whose entries decay geometrically with the rank indices, plus iid
Gaussian noise; K items additionally get four boosted outlier channels per
(layer, head).  The pages measure on real Mistral-7B-v0.3 / LLaMA-2-13B /
LLaMA-3.1-8B prefill caches; these seeded tensors stand in for them, matching
only their shapes (layers per group, KV heads, head dim, context length).

Random stream: numpy ``default_rng([seed, sequence, group, kv])`` with kv 0 for
K and 1 for V.  Draw order per item: token factor, feature factor, core, noise,
outlier channels.  The fp64 tensor is rounded to fp32 (RNE) and then, for bf16
items, to bf16 (RNE).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np


# --------------------------------------------------------------------------
# dtype helpers (input casting only)
# --------------------------------------------------------------------------
def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 -> fp32 (RNE) -> bf16 (RNE); returns the uint16 bit patterns."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    # finite values stay below 2^32 after the rounding increment
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = bits.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# workload configurations
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class CacheConfig:
    name: str
    L: int                      # layers per group
    H: int                      # KV heads
    T: int                      # tokens
    d: int                      # head dim
    groups: int                 # layer groups per sequence
    sequences: int
    dtype: str                  # "bf16" | "f32"
    rank_t: Optional[int]       # planted token rank (None: per-sequence draw)
    rank_t_range: Optional[Tuple[int, int]]
    rank_f: int
    decay: float
    sigma: float
    k_outliers: bool
    seed: int
    # compressor settings that belong to the workload definition
    token_modes: Tuple[str, ...]          # "exact" and/or "randomized"
    ratios: Tuple[float, ...]             # budget = floor(dense bf16 bytes / ratio)
    fixed: Optional[Tuple[int, int, int]] = None   # (r_t, r_f, bits) when no budget
    rt_max: int = 0
    bits: Tuple[int, ...] = (0, 2, 3, 4)
    rank_step: int = 8
    oversample: int = 10
    power_iters: int = 1
    description: str = ""

    @property
    def items_per_sequence(self) -> int:
        return 2 * self.groups

    @property
    def n_items(self) -> int:
        return self.sequences * self.items_per_sequence

    @property
    def elems_per_item(self) -> int:
        return self.L * self.H * self.T * self.d

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


CONFIGS: Dict[str, CacheConfig] = {
    "tiny_exact_f32": CacheConfig(
        name="tiny_exact_f32", L=2, H=4, T=256, d=64, groups=1, sequences=1,
        dtype="f32", rank_t=16, rank_t_range=None, rank_f=12, decay=0.8,
        sigma=0.01, k_outliers=False, seed=0, token_modes=("exact",),
        ratios=(), fixed=(16, 12, 4), rt_max=16, bits=(4,),
        description="one group, 2 layers x 4 KV heads x 256 tokens x d=64, fp32, "
                    "exact token factor, fixed ranks (16, 12), 4-bit residual"),
    "mistral7b_gqa_1k": CacheConfig(
        name="mistral7b_gqa_1k", L=4, H=8, T=1024, d=128, groups=8, sequences=1,
        dtype="bf16", rank_t=64, rank_t_range=None, rank_f=48, decay=0.9,
        sigma=0.02, k_outliers=True, seed=0,
        token_modes=("randomized", "exact"), ratios=(2.0,), rt_max=128,
        description="Mistral-7B-v0.3-shaped GQA cache: 32 layers in 8 groups of 4, "
                    "8 KV heads, d=128, 1024 tokens, 2x budget"),
    "llama2_13b_mha_4k": CacheConfig(
        name="llama2_13b_mha_4k", L=4, H=40, T=4096, d=128, groups=10, sequences=1,
        dtype="bf16", rank_t=128, rank_t_range=None, rank_f=64, decay=0.9,
        sigma=0.02, k_outliers=True, seed=0, token_modes=("randomized",),
        ratios=(3.0,), rt_max=256,
        description="LLaMA-2-13B-shaped MHA cache: 40 layers in 10 groups of 4, "
                    "40 heads, d=128, 4096 tokens, 3x budget"),
    "llama31_8b_gqa_64k": CacheConfig(
        name="llama31_8b_gqa_64k", L=4, H=8, T=65536, d=128, groups=8, sequences=1,
        dtype="bf16", rank_t=256, rank_t_range=None, rank_f=64, decay=0.9,
        sigma=0.02, k_outliers=True, seed=0, token_modes=("randomized",),
        ratios=(2.0, 3.0, 4.0, 5.0), rt_max=256,
        description="LLaMA-3.1-8B-shaped GQA cache, one 65536-token sequence, "
                    "32 layers in 8 groups of 4, 8 KV heads, d=128"),
    "moe_gqa_batch16_8k": CacheConfig(
        name="moe_gqa_batch16_8k", L=4, H=8, T=8192, d=128, groups=8, sequences=16,
        dtype="bf16", rank_t=None, rank_t_range=(32, 192), rank_f=48, decay=0.9,
        sigma=0.02, k_outliers=True, seed=0, token_modes=("randomized",),
        ratios=(2.5,), rt_max=256,
        description="MoE-style GQA batch: 16 sequences x 8192 tokens, 8 groups of "
                    "4 layers, 8 KV heads, d=128, one shared 2.5x budget"),
}


def config(name: str, **overrides) -> CacheConfig:
    """A named configuration, optionally with fields replaced (smaller T, ...)."""
    base = CONFIGS[name]
    if not overrides:
        return base
    d = dict(base.__dict__)
    d.update(overrides)
    return CacheConfig(**d)


def budget_for_ratio(cfg: CacheConfig, ratio: float, n_items: Optional[int] = None) -> int:
    """Global byte budget: dense bf16 bytes of all items divided by the ratio."""
    n = cfg.n_items if n_items is None else n_items
    dense = n * 2 * cfg.elems_per_item
    return int(np.floor(dense / ratio))


# --------------------------------------------------------------------------
# items
# --------------------------------------------------------------------------
@dataclass
class Item:
    item_id: int
    seed: int            # seed of the item's random rotation / sketch streams
    sequence: int
    group: int
    kv: int              # 0 = K, 1 = V
    L: int
    H: int
    T: int
    d: int
    dtype: str
    rank_t: int
    rank_f: int
    x: Optional[np.ndarray] = None      # fp64 values of the stored tensor
    raw: Optional[np.ndarray] = None    # uint16 bf16 bits or float32, [L,H,T,d]
    planted: Dict[str, np.ndarray] = field(default_factory=dict)

    @property
    def N(self) -> int:
        return self.L * self.H * self.T * self.d


def _sequence_rank_t(cfg: CacheConfig, s: int) -> int:
    if cfg.rank_t is not None:
        return cfg.rank_t
    lo, hi = cfg.rank_t_range
    rng = np.random.default_rng([cfg.seed, s, 0x5EC])
    return int(rng.integers(lo, hi + 1))


def item_specs(cfg: CacheConfig, n_items: Optional[int] = None) -> List[Item]:
    """Item descriptors (no data) in (sequence, group, K/V) order."""
    out = []
    for s in range(cfg.sequences):
        rt = _sequence_rank_t(cfg, s)
        for g in range(cfg.groups):
            for kv in (0, 1):
                iid = (s * cfg.groups + g) * 2 + kv
                out.append(Item(item_id=iid, seed=cfg.seed + s, sequence=s, group=g,
                                kv=kv, L=cfg.L, H=cfg.H, T=cfg.T, d=cfg.d,
                                dtype=cfg.dtype, rank_t=rt, rank_f=cfg.rank_f))
    if n_items is not None:
        out = out[:n_items]
    return out


def make_item(cfg: CacheConfig, spec: Item, sigma: Optional[float] = None,
              keep_planted: bool = False, keep_x: bool = True) -> Item:
    """Fill ``spec`` with its seeded tensor (``keep_x=False``: the stored bits
    only, without the fp64 copy)."""
    L, H, T, d = spec.L, spec.H, spec.T, spec.d
    rt, rf = spec.rank_t, spec.rank_f
    sig = cfg.sigma if sigma is None else sigma
    rng = np.random.default_rng([cfg.seed, spec.sequence, spec.group, spec.kv])
    U = np.linalg.qr(rng.standard_normal((T, rt)))[0]
    V = np.linalg.qr(rng.standard_normal((d, rf)))[0]
    i = np.arange(rt)[:, None]
    j = np.arange(rf)[None, :]
    C = rng.standard_normal((L, H, rt, rf)) * (cfg.decay ** (i + j))
    X = np.matmul(np.matmul(U[None, None], C), V.T[None, None])
    noise = rng.standard_normal((L, H, T, d))
    X += sig * noise
    del noise
    if cfg.k_outliers and spec.kv == 0:
        for l in range(L):
            for h in range(H):
                ch = rng.choice(d, 4, replace=False)
                X[l, h][:, ch] *= 8.0
    if spec.dtype == "f32":
        raw = X.astype(np.float32)
        xv = raw.astype(np.float64) if keep_x else None
    else:
        raw = f64_to_bf16_bits(X)
        xv = bf16_bits_to_f64(raw) if keep_x else None
    del X
    spec.x = xv if keep_x else None
    spec.raw = raw
    if keep_planted:
        spec.planted = {"U": U, "V": V, "C": C}
    return spec


def make_items(cfg: CacheConfig, n_items: Optional[int] = None, **kw) -> List[Item]:
    return [make_item(cfg, s, **kw) for s in item_specs(cfg, n_items)]


def _raw_worker(args):
    cfg, spec = args
    try:
        import threadpoolctl
        with threadpoolctl.threadpool_limits(1):
            return make_item(cfg, spec, keep_x=False).raw
    except ImportError:
        return make_item(cfg, spec, keep_x=False).raw


def iter_raw_parallel(cfg: CacheConfig, specs: List[Item], workers: int = 0, start: str = "fork"):
    """Yield (index, stored bits) of every spec, in order, generated by a pool
    of worker processes (the same values as make_item).  With start="fork"
    call it before anything initialises a GPU in this process; "spawn" starts
    fresh interpreters and is safe afterwards."""
    import multiprocessing as mp
    import os
    if workers <= 0:
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
    workers = min(workers, max(1, len(specs)))
    if workers == 1:
        for i, s in enumerate(specs):
            yield i, make_item(cfg, s, keep_x=False).raw
        return
    ctx = mp.get_context(start)
    with ctx.Pool(workers) as pool:
        for i, raw in enumerate(pool.imap(_raw_worker, [(cfg, s) for s in specs], chunksize=1)):
            yield i, raw
        # every task is done: let the workers exit on their own rather than
        # terminating them with a signal (a profiler preloaded into them
        # handles that signal and can stall the parent waiting for them)
        pool.close()
        pool.join()


def gaussian_groups(n_groups: int, group: int = 64, seed: int = 0) -> np.ndarray:
    """iid N(0,1) fp64 groups, used to measure a quantizer's relative MSE."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n_groups, group))
