"""Plain CPU oracle for the heterogeneous-batch LoRA delta (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and its
Python binding) never imports, calls or links it, and it imports nothing from
the product: the two share only the seeded input generator in ``synth/``.

What it computes, with its sources (S-LoRA pages):
  * LoRA forward h = xW + xAB with A in R^{d_in x r} and B in R^{r x d_out};
    the delta xAB is kept separate from the base product (summary page,
    "What this paper explains" and "How to read the paper" item 2; "The
    mechanism", "Separate base and delta").
  * Per-token delta with a scaling factor: each token of the batch names its
    own adapter and gets its product with A and B, times the adapter's
    scaling factor, added to its base output
    (blog page, section 2 pseudocode, "Batched S-LoRA Vector Matrix Addition").
  * Adapter factors live as non-contiguous pages of one pool shared with KV
    blocks, found through a block table (summary page, "Unified Paging";
    blog page, section 2; catalog page, mechanism paragraph).

Pieces, each written from its definition with no blocking or reordering:
  * ``AllocatorModel``: FIFO free list per page class seeded from the caller's
    free order; an adapter of rank r takes, for each projection in order,
    r pages for the rows of A^T (row j is column j of A) and then r pages for
    the rows of B; unloading appends its pages to the tail in allocation order.
  * ``segment_model``: tokens stably sorted by adapter id into segments in
    ascending id order, tokens with a negative id dropped; per segment the
    rank, scale, rank prefix offset and the concatenated page lists.
  * ``PoolImage``: host copy of the page contents the allocator model implies;
    every page not written by an adapter load reads as NaN.
  * ``lora_delta``: walks tokens in batch order, follows the block table to
    the page rows, converts them to float64 exactly and returns
    y_in + s * ((x A) B) unrounded, with s * (x A) B beside it.
  * ``lora_forward``: the base output plus the adapter output,
    x W + s * ((x A) B), unrounded (summary page, "How to read the paper"
    item 2, h = xW + xAB; blog page, section 2: the batched forward returns
    base_out + adapter_out); x W is NumPy's dense float64 product.

Parity: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, brute force, invariants and hand-worked fixtures); none is
"parity unpinned".
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


class OracleError(Exception):
    pass


@dataclass
class AdapterEntry:
    rank: int
    scale: float
    a_pages: List[List[int]]   # [n_proj][rank] page ids of the A^T rows
    b_pages: List[List[int]]   # [n_proj][rank] page ids of the B rows


class AllocatorModel:
    """Page allocator and block table, modelled with Python deques and dicts."""

    def __init__(self, n_pages: Sequence[int], free_order: Sequence[Optional[Sequence[int]]],
                 n_proj: int = 1, two_classes: bool = False):
        if len(n_pages) != (2 if two_classes else 1):
            raise OracleError("one page count per class")
        self.n_pages = [int(p) for p in n_pages]
        self.n_proj = int(n_proj)
        self.two_classes = bool(two_classes)
        self.free: List[deque] = []
        for P, order in zip(self.n_pages, free_order):
            ids = list(range(P)) if order is None else [int(i) for i in order]
            if sorted(ids) != list(range(P)):
                raise OracleError("free order must be a permutation of the page ids")
            self.free.append(deque(ids))
        self.table: Dict[int, AdapterEntry] = {}

    def b_class(self) -> int:
        return 1 if self.two_classes else 0

    def alloc(self, cls: int, n: int) -> List[int]:
        if n > len(self.free[cls]):
            raise OracleError("out of pages")
        return [self.free[cls].popleft() for _ in range(n)]

    def release(self, cls: int, pages: Sequence[int]) -> None:
        self.free[cls].extend(int(p) for p in pages)

    def load(self, a: int, rank: int, scale: float) -> AdapterEntry:
        if a in self.table:
            raise OracleError("adapter already loaded")
        need_a = rank * self.n_proj
        need_b = rank * self.n_proj
        if self.two_classes:
            if need_a > len(self.free[0]) or need_b > len(self.free[1]):
                raise OracleError("out of pages")
        elif need_a + need_b > len(self.free[0]):
            raise OracleError("out of pages")
        a_pages, b_pages = [], []
        for _p in range(self.n_proj):
            a_pages.append(self.alloc(0, rank))
            b_pages.append(self.alloc(self.b_class(), rank))
        entry = AdapterEntry(rank=int(rank), scale=float(np.float32(scale)),
                             a_pages=a_pages, b_pages=b_pages)
        self.table[a] = entry
        return entry

    def unload(self, a: int) -> None:
        entry = self.table.pop(a)
        for p in range(self.n_proj):
            self.release(0, entry.a_pages[p])
            self.release(self.b_class(), entry.b_pages[p])


@dataclass
class Segments:
    perm: np.ndarray          # int32 [T'], batch index of the i-th sorted token
    seg_start: np.ndarray     # int32 [S+1]
    seg_adapter: np.ndarray   # int32 [S]
    seg_rank: np.ndarray      # int32 [S]
    seg_scale: np.ndarray     # float32 [S]
    seg_page_off: np.ndarray  # int32 [S+1], prefix sum of ranks
    a_pages: np.ndarray       # int32 [n_proj * sum_r], index p*sum_r + seg_page_off[s] + j
    b_pages: np.ndarray       # int32 [n_proj * sum_r]


def segment_model(ids: Sequence[int], alloc: AllocatorModel) -> Segments:
    """Group the batch's tokens by adapter (ascending id, stable within an id)."""
    ids = np.asarray(ids, dtype=np.int64)
    for a in ids:
        if a >= 0 and int(a) not in alloc.table:
            raise OracleError(f"token names adapter {int(a)} which is not loaded")
    order = np.argsort(ids, kind="stable")
    perm = order[ids[order] >= 0].astype(np.int32)
    sorted_ids = ids[perm]
    seg_start, seg_adapter = [], []
    for i, a in enumerate(sorted_ids):
        if i == 0 or a != sorted_ids[i - 1]:
            seg_start.append(i)
            seg_adapter.append(int(a))
    seg_start.append(len(perm))
    ranks = [alloc.table[a].rank for a in seg_adapter]
    scales = [alloc.table[a].scale for a in seg_adapter]
    page_off = [0]
    for r in ranks:
        page_off.append(page_off[-1] + r)
    a_pages, b_pages = [], []
    for p in range(alloc.n_proj):
        for a in seg_adapter:
            a_pages.extend(alloc.table[a].a_pages[p])
            b_pages.extend(alloc.table[a].b_pages[p])
    return Segments(perm=perm, seg_start=np.asarray(seg_start, dtype=np.int32),
                    seg_adapter=np.asarray(seg_adapter, dtype=np.int32),
                    seg_rank=np.asarray(ranks, dtype=np.int32),
                    seg_scale=np.asarray(scales, dtype=np.float32),
                    seg_page_off=np.asarray(page_off, dtype=np.int32),
                    a_pages=np.asarray(a_pages, dtype=np.int32),
                    b_pages=np.asarray(b_pages, dtype=np.int32))


class PoolImage:
    """Contents of the page pool as the allocator model places them."""

    def __init__(self, page_elems: Sequence[int], dtype):
        self.page_elems = [int(e) for e in page_elems]
        self.dtype = np.dtype(dtype)
        self.rows: Dict[Tuple[int, int], np.ndarray] = {}

    def write_adapter(self, alloc: AllocatorModel, a: int, p: int, A: np.ndarray, B: np.ndarray):
        """Row j of the A^T pages is column j of A; row j of the B pages is row j of B."""
        entry = alloc.table[a]
        A = np.asarray(A)
        B = np.asarray(B)
        if A.shape != (self.page_elems[0], entry.rank):
            raise OracleError("A must be d_in x r")
        if B.shape != (entry.rank, self.page_elems[alloc.b_class()]):
            raise OracleError("B must be r x d_out")
        for j in range(entry.rank):
            self.rows[(0, entry.a_pages[p][j])] = A[:, j].astype(self.dtype).copy()
            self.rows[(alloc.b_class(), entry.b_pages[p][j])] = B[j, :].astype(self.dtype).copy()

    def row(self, cls: int, page: int) -> np.ndarray:
        r = self.rows.get((cls, int(page)))
        if r is None:
            return np.full(self.page_elems[cls], np.nan, dtype=self.dtype)
        return r


def lora_delta(alloc: AllocatorModel, image: PoolImage, ids: Sequence[int], x: np.ndarray,
               y_in: np.ndarray, proj: int = 0, tokens: Optional[Sequence[int]] = None):
    """Return (y_ref, sd_ref) in float64 for the tokens listed (all by default).

    For token t with adapter a of rank r and scale s:
        v[j]  = sum_k x[t, k] * A^T_row_j[k]        (j < r)
        d[o]  = sum_j v[j] * B_row_j[o]
        y_ref = y_in[t] + s * d,   sd_ref = s * d
    Tokens with a negative id keep y_in.  Both outputs are unrounded float64.
    """
    ids = np.asarray(ids)
    if tokens is None:
        tokens = range(ids.shape[0])
    tokens = list(tokens)
    y_ref = np.empty((len(tokens), y_in.shape[1]), dtype=np.float64)
    sd_ref = np.zeros_like(y_ref)
    b_cls = alloc.b_class()
    for out_i, t in enumerate(tokens):
        a = int(ids[t])
        y_ref[out_i] = y_in[t].astype(np.float64)
        if a < 0:
            continue
        entry = alloc.table[a]
        At = np.stack([image.row(0, pg) for pg in entry.a_pages[proj]]).astype(np.float64)
        Bm = np.stack([image.row(b_cls, pg) for pg in entry.b_pages[proj]]).astype(np.float64)
        v = At @ x[t].astype(np.float64)          # (x A)[j] = sum_k x[k] A[k, j]
        d = v @ Bm                                 # ((x A) B)[o] = sum_j v[j] B[j, o]
        sd_ref[out_i] = np.float64(entry.scale) * d
        y_ref[out_i] += sd_ref[out_i]
    return y_ref, sd_ref


def lora_forward(alloc: AllocatorModel, image: PoolImage, ids: Sequence[int], x: np.ndarray,
                 W: np.ndarray, proj: int = 0, tokens: Optional[Sequence[int]] = None):
    """Return (h_ref, sd_ref) in float64 for the tokens listed (all by default).

    h_ref[t] = x[t] W + s * (x[t] A) B: the base output of the dense weight W
    (d_in x d_out) plus the adapter output of token t's adapter; a token with
    a negative id gets x[t] W alone.  sd_ref is the adapter part, as in
    ``lora_delta``.  Both unrounded.
    """
    ids = np.asarray(ids)
    if tokens is None:
        tokens = range(ids.shape[0])
    tokens = list(tokens)
    base = x[tokens].astype(np.float64) @ W.astype(np.float64)
    # lora_delta over a base output of zeros gives the adapter output alone
    zeros = np.zeros((ids.shape[0], W.shape[1]), dtype=np.float64)
    _, sd_ref = lora_delta(alloc, image, ids, x, zeros, proj=proj, tokens=tokens)
    return base + sd_ref, sd_ref


def round_to(y: np.ndarray, dtype) -> np.ndarray:
    """One round-to-nearest-even of a float64 result to the output dtype."""
    return np.asarray(y, dtype=np.float64).astype(dtype)


# ---------------------------------------------------------------------------
# Building the oracle's view of a synthetic workload.


@dataclass
class OracleState:
    alloc: AllocatorModel
    image: PoolImage
    kv_pages: List[List[int]]


def build_from_workload(w, load_weights: bool = True) -> OracleState:
    """Replay the workload's pool set-up on the oracle's own allocator model.

    KV pages are taken first in each class, then adapters load in id order;
    only adapters with weights (referenced ones, unless the spec asks for all)
    get rows written into the image.
    """
    spec = w.spec
    alloc = AllocatorModel(w.n_pages, w.free_order, n_proj=spec.n_proj,
                           two_classes=spec.two_classes)
    kv = [alloc.alloc(c, n) for c, n in enumerate(w.kv_pages)]
    page_elems = [w.page_elems(c) for c in range(len(w.n_pages))]
    image = PoolImage(page_elems, w.np_dtype)
    for a in range(spec.n_adapters):
        alloc.load(a, int(w.ranks[a]), float(w.scales[a]))
        if load_weights and w.has_weights(a):
            for p in range(spec.n_proj):
                A, B = w.weights(a, p)
                image.write_adapter(alloc, a, p, A, B)
    return OracleState(alloc=alloc, image=image, kv_pages=kv)


def workload_delta(state: OracleState, w, proj: int = 0, tokens=None):
    """Oracle (y_ref, sd_ref) of projection ``proj`` of a synthetic workload."""
    x = w.x[w.spec.proj_x[proj]]
    return lora_delta(state.alloc, state.image, w.ids, x, w.y[proj], proj=proj, tokens=tokens)


def workload_forward(state: OracleState, w, proj: int = 0, tokens=None):
    """Oracle (h_ref, sd_ref) of the base-plus-delta product of projection ``proj``."""
    x = w.x[w.spec.proj_x[proj]]
    return lora_forward(state.alloc, state.image, w.ids, x, w.base_weight(proj), proj=proj,
                        tokens=tokens)
