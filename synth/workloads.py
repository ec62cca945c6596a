"""Seeded synthetic workloads for the heterogeneous-batch LoRA delta.

This module only draws random inputs and lays out the page pool; it holds none
of the method's arithmetic (no products, no sums over pages), so both the fp64
oracle and the HIP path may take their inputs from it without sharing any
computation.

Sources for the shapes and distributions:
  * S-LoRA summary page ("S-LoRA: Serving Thousands of Concurrent LoRA
    Adapters", sections "What this paper explains" and "The mechanism"):
    A is d_in x r, B is r x d_out, adapters of different ranks share one page
    pool with KV blocks.
  * The five benchmark shapes (Tiny 256^2 fp32, Llama-7B decode and prefill,
    Llama-13B mixed q/k/v/o batch, Llama-70B-width MLP projection) with their
    adapter counts, rank sets, id distributions and pool occupancies.

Readings taken where the sources are silent:
  * "N(0, 0.02)" is a standard deviation of 0.02, drawn in fp32 and rounded to
    the storage dtype with round-to-nearest-even (numpy ``astype``).
  * x and the base y are N(0, 1) wherever a shape does not say otherwise.
  * Zipf(s) over N adapters has finite support: P(k) ~ k^-s, k = 1..N, and the
    adapter id is k - 1.
  * Ranks are drawn iid uniform per adapter from the listed set; prefill
    request lengths are uniform integers in [lo, hi] inclusive.
  * A pool with occupancy ``occ`` has P = ceil(N_adapter_pages / (1 - occ))
    pages per class; its free order is a seeded permutation of [0, P); the
    P - N_adapter_pages KV pages are taken first, then adapters load in id
    order, so adapter rows land at random places among the KV pages.
  * Adapters that no token references are reserved (pages taken, nothing
    written), which leaves their pages with whatever the pool holds; callers
    poison the pool with NaN so that a misdirected read shows up in y.

Seeding: every stream comes from ``SeedSequence([cfg_idx, seed, stream])``
(streams: 0 ranks, 1 token ids / lengths, 2 x, 3 y, 4 pool free order,
6 scales); the weights of adapter ``a`` for projection ``p`` come from
``SeedSequence([cfg_idx, seed, 5, a, p])`` so one adapter can be regenerated
alone, and the dense base weight W (h_in x h_out) of projection ``p``, for the
base-plus-delta product, from ``SeedSequence([cfg_idx, seed, 7, p])`` with the
adapters' distribution.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Sequence, Tuple

import numpy as np

STREAM_RANKS, STREAM_IDS, STREAM_X, STREAM_Y, STREAM_POOL, STREAM_W, STREAM_SCALE = 0, 1, 2, 3, 4, 5, 6
STREAM_BASE = 7

NP_DTYPE = {"f32": np.float32, "f16": np.float16}


@dataclass(frozen=True)
class Spec:
    """Shape of one workload; every random quantity is drawn in ``generate``."""

    name: str
    cfg_idx: int
    dtype: str                      # "f32" or "f16": storage type of x, y, A, B
    h_in: int
    h_out: int
    n_adapters: int
    rank_set: Tuple[int, ...] = (8, 16, 32, 64)
    fixed_ranks: Optional[Tuple[int, ...]] = None   # overrides rank_set draws
    n_proj: int = 1
    proj_x: Tuple[int, ...] = (0,)  # projection p reads x number proj_x[p]
    two_classes: bool = False       # A^T rows and B rows in separate page classes
    weight_std: float = 0.02
    scale: float = 2.0
    scale_set: Optional[Tuple[float, ...]] = None   # per-adapter scale drawn from this set
    # batch kinds:
    #   ("uniform", T)                         ids uniform over all adapters
    #   ("zipf", T, s)                         finite-support Zipf(s)
    #   ("requests", n_req, lo, hi)            prefill requests, one adapter each
    #   ("mixed", n_prefill, prefill_len, n_decode)
    batch: Tuple = ("uniform", 16)
    # pool kinds: ("fixed", P) or ("occ", num, den) meaning occupancy num/den
    pool: Tuple = ("occ", 1, 2)
    values: str = "normal"          # "normal" or "ternary" ({-1, 0, 1} everywhere)
    full_weights: bool = False      # write weights for unreferenced adapters too

    @property
    def n_x(self) -> int:
        return max(self.proj_x) + 1


# The five shapes of the benchmark suite.
TINY = Spec(name="tiny", cfg_idx=0, dtype="f32", h_in=256, h_out=256, n_adapters=4,
            fixed_ranks=(4, 8, 4, 8), batch=("uniform", 16), pool=("fixed", 128),
            full_weights=True)
DECODE_7B = Spec(name="decode7b", cfg_idx=1, dtype="f16", h_in=4096, h_out=4096,
                 n_adapters=1000, batch=("zipf", 256, 1.1), pool=("occ", 3, 5))
PREFILL_7B = Spec(name="prefill7b", cfg_idx=2, dtype="f16", h_in=4096, h_out=4096,
                  n_adapters=100, batch=("requests", 32, 64, 512), pool=("occ", 1, 2))
MIXED_13B = Spec(name="mixed13b", cfg_idx=3, dtype="f16", h_in=5120, h_out=5120,
                 n_adapters=2000, n_proj=4, proj_x=(0, 0, 0, 1),
                 batch=("mixed", 8, 256, 384), pool=("occ", 1, 2))
MLP_70B = Spec(name="mlp70b", cfg_idx=4, dtype="f16", h_in=8192, h_out=28672,
               n_adapters=5000, rank_set=(16, 32, 64, 128), two_classes=True,
               batch=("zipf", 512, 1.0), pool=("occ", 4, 5))

CONFIGS = {s.name: s for s in (TINY, DECODE_7B, PREFILL_7B, MIXED_13B, MLP_70B)}


@dataclass
class Workload:
    spec: Spec
    seed: int
    ranks: np.ndarray               # int32 [n_adapters]
    scales: np.ndarray              # float32 [n_adapters]
    ids: np.ndarray                 # int32 [T], adapter id per token in batch order
    x: list                         # n_x arrays [T, h_in] of the storage dtype
    y: list                         # n_proj arrays [T, h_out] of the storage dtype
    n_pages: Tuple[int, ...]        # pages per class
    free_order: list                # per class, int32 permutation of [0, P)
    kv_pages: Tuple[int, ...]       # KV pages allocated first, per class
    referenced: np.ndarray          # bool [n_adapters]: some token uses it
    _wcache: dict = field(default_factory=dict, repr=False)

    @property
    def T(self) -> int:
        return int(self.ids.shape[0])

    @property
    def np_dtype(self):
        return NP_DTYPE[self.spec.dtype]

    def page_elems(self, cls: int) -> int:
        """Elements per page of class ``cls`` (one H-element row)."""
        if self.spec.two_classes:
            return self.spec.h_in if cls == 0 else self.spec.h_out
        return self.spec.h_in

    def has_weights(self, a: int) -> bool:
        return bool(self.spec.full_weights or self.referenced[a])

    def weights(self, a: int, p: int = 0):
        """(A [h_in, r], B [r, h_out]) of adapter ``a``, projection ``p``."""
        key = (a, p)
        if key not in self._wcache:
            self._wcache[key] = _draw_weights(self.spec, self.seed, a, p, int(self.ranks[a]))
        return self._wcache[key]

    def base_weight(self, p: int = 0) -> np.ndarray:
        """Dense base weight W [h_in, h_out] of projection ``p`` (storage dtype)."""
        key = ("base", p)
        if key not in self._wcache:
            rng = _rng(self.spec, self.seed, STREAM_BASE, p)
            self._wcache[key] = _draw(rng, (self.spec.h_in, self.spec.h_out), self.spec.weight_std,
                                      self.spec.values, NP_DTYPE[self.spec.dtype])
        return self._wcache[key]

    def drop_weight_cache(self):
        self._wcache.clear()


def _rng(spec: Spec, seed: int, *stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([spec.cfg_idx, seed, *stream]))


def _draw(rng: np.random.Generator, shape, std: float, values: str, dtype):
    if values == "ternary":
        return rng.integers(-1, 2, size=shape).astype(dtype)
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(dtype)


def _draw_weights(spec: Spec, seed: int, a: int, p: int, r: int):
    rng = _rng(spec, seed, STREAM_W, a, p)
    dt = NP_DTYPE[spec.dtype]
    A = _draw(rng, (spec.h_in, r), spec.weight_std, spec.values, dt)
    B = _draw(rng, (r, spec.h_out), spec.weight_std, spec.values, dt)
    return A, B


def _finite_zipf(rng: np.random.Generator, n: int, s: float, size: int) -> np.ndarray:
    k = np.arange(1, n + 1, dtype=np.float64)
    p = k ** (-float(s))
    p /= p.sum()
    return rng.choice(n, size=size, p=p).astype(np.int32)


def _token_ids(spec: Spec, rng: np.random.Generator) -> np.ndarray:
    kind = spec.batch[0]
    if kind == "uniform":
        return rng.integers(0, spec.n_adapters, size=spec.batch[1]).astype(np.int32)
    if kind == "zipf":
        return _finite_zipf(rng, spec.n_adapters, spec.batch[2], spec.batch[1])
    if kind == "requests":
        n_req, lo, hi = spec.batch[1:]
        lengths = rng.integers(lo, hi + 1, size=n_req)
        req_adapter = rng.integers(0, spec.n_adapters, size=n_req)
        return np.repeat(req_adapter, lengths).astype(np.int32)
    if kind == "mixed":
        n_pre, pre_len, n_dec = spec.batch[1:]
        req_adapter = rng.integers(0, spec.n_adapters, size=n_pre + n_dec)
        pre = np.repeat(req_adapter[:n_pre], pre_len)
        return np.concatenate([pre, req_adapter[n_pre:]]).astype(np.int32)
    if kind == "explicit":
        return np.asarray(spec.batch[1], dtype=np.int32)
    raise ValueError(f"unknown batch kind {kind!r}")


def adapter_pages_per_class(spec: Spec, ranks: np.ndarray) -> Tuple[int, ...]:
    """Pages the adapters need per class: r A^T rows and r B rows per projection."""
    total_r = int(np.asarray(ranks, dtype=np.int64).sum()) * spec.n_proj
    if spec.two_classes:
        return (total_r, total_r)
    return (2 * total_r,)


def generate(spec: Spec, seed: int = 0) -> Workload:
    """Draw one workload of shape ``spec``; deterministic in (spec, seed)."""
    dt = NP_DTYPE[spec.dtype]
    if spec.fixed_ranks is not None:
        ranks = np.asarray(spec.fixed_ranks, dtype=np.int32)
        assert ranks.shape[0] == spec.n_adapters
    else:
        ranks = _rng(spec, seed, STREAM_RANKS).choice(
            np.asarray(spec.rank_set, dtype=np.int32), size=spec.n_adapters).astype(np.int32)
    if spec.scale_set is not None:
        scales = _rng(spec, seed, STREAM_SCALE).choice(
            np.asarray(spec.scale_set, dtype=np.float32), size=spec.n_adapters).astype(np.float32)
    else:
        scales = np.full(spec.n_adapters, spec.scale, dtype=np.float32)

    ids = _token_ids(spec, _rng(spec, seed, STREAM_IDS))
    T = ids.shape[0]
    rx = _rng(spec, seed, STREAM_X)
    x = [_draw(rx, (T, spec.h_in), 1.0, spec.values, dt) for _ in range(spec.n_x)]
    ry = _rng(spec, seed, STREAM_Y)
    y = [_draw(ry, (T, spec.h_out), 1.0, spec.values, dt) for _ in range(spec.n_proj)]

    need = adapter_pages_per_class(spec, ranks)
    if spec.pool[0] == "fixed":
        n_pages = tuple(int(spec.pool[1]) for _ in need)
        kv = tuple(0 for _ in need)
    else:
        num, den = spec.pool[1], spec.pool[2]
        # P = ceil(N / (1 - num/den)) = ceil(N * den / (den - num)), in integers
        n_pages = tuple(int(-(-n * den // (den - num))) for n in need)
        kv = tuple(P - n for P, n in zip(n_pages, need))
    for P, n in zip(n_pages, need):
        if n > P:
            raise ValueError(f"{spec.name}: pool of {P} pages cannot hold {n} adapter pages")
    rp = _rng(spec, seed, STREAM_POOL)
    free_order = [rp.permutation(P).astype(np.int32) for P in n_pages]

    referenced = np.zeros(spec.n_adapters, dtype=bool)
    referenced[ids[ids >= 0]] = True
    return Workload(spec=spec, seed=seed, ranks=ranks, scales=scales, ids=ids, x=x, y=y,
                    n_pages=n_pages, free_order=free_order, kv_pages=kv, referenced=referenced)


def small_spec(name: str = "small", **kw) -> Spec:
    """A custom small shape for tests; keyword arguments override Spec fields."""
    base = Spec(name=name, cfg_idx=100, dtype="f16", h_in=256, h_out=256, n_adapters=6,
                batch=("uniform", 24), pool=("occ", 1, 2), full_weights=True)
    return replace(base, **kw)
