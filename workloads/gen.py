"""Seeded synthetic inputs for tree-masked MLA verify attention.

This module builds inputs only: bf16 query/latent bits, the page_size=1 slot
layout, draft trees and their visibility masks, and the segmented metadata
buffers.  It holds none of the attention arithmetic; both the CPU oracle and the
HIP path consume what it returns, and neither is imported here.

Shapes and structure follow the workloads the verify step sees on the pages:
draft-tree query tokens with H heads over a 576-wide latent (512 compressed +
64 rope), prefix KV rows scattered over a paged pool with page size 1
("The Integration Chasm", Context: What Came Before), the segmented
qo_indptr / kv_indptr / kv_indices / out_cache_loc / custom_mask / mask_indptr
buffers ("The Capture-Safe Kernel", Decision 1), and draft-token rows already
resident in the pool at out_cache_loc ("The Launch Wrapper", The KV Cache
Ordering Insight).  The pages name no public benchmark; these synthetic
instances stand in for their unnamed long-context suite.

Draw order for one instance (numpy PCG64, one generator per seed):
  0. per-request prefix and tree sizes (segmented batch only)
  1. slot permutation of [0, num_slots)
  2. tree parents
  3. latent rows of the used slots, in logical order (each request's prefix,
     then its tree nodes)
  4. outlier rows (prefix rows whose 576 values are multiplied by 8)
  5. queries
Values are drawn as float32 N(0,1) and rounded to bf16 (round to nearest even).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

D_QK = 576          # latent width seen by Q.K^T (512 compressed + 64 rope)
D_V = 512           # V is the first 512 latent dims
MAX_TREE_NODES = 64
SM_SCALE = np.float32(1.0 / np.sqrt(192.0))
BF16_NAN = np.uint16(0xFFFF)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if not np.isfinite(x).all():
        raise ValueError("only finite values are rounded here")
    # finite inputs: |u| <= 0x7F7FFFFF (+ sign) so the sum cannot wrap in 32 bits
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def chain_parents(t: int) -> List[int]:
    return [-1] + list(range(t - 1))


def random_parents(rng: np.random.Generator, t: int) -> List[int]:
    """Node 0 is the root; node i >= 1 takes a parent uniform over 0..i-1."""
    parents = [-1]
    for i in range(1, t):
        parents.append(int(rng.integers(0, i)))
    return parents


def ancestor_or_self_mask(parents: Sequence[int]) -> np.ndarray:
    """T x T uint8, row = query node, column = key node, 1 where the key node
    is the query node itself or one of its ancestors."""
    t = len(parents)
    m = np.zeros((t, t), dtype=np.uint8)
    for i in range(t):
        j = i
        while j >= 0:
            m[i, j] = 1
            j = parents[j]
    return m


@dataclasses.dataclass
class Instance:
    """One verify call's inputs.  Everything is host numpy; bf16 as uint16 bits."""
    name: str
    seed: int
    num_heads: int
    num_slots: int
    q: np.ndarray              # uint16 [sumT, H, 576]
    rows: np.ndarray           # uint16 [n_used, 576] latent rows, logical order
    row_slots: np.ndarray      # int64  [n_used] slot of each row
    qo_indptr: np.ndarray      # int32  [B+1]
    kv_indptr: np.ndarray      # int32  [B+1]
    kv_indices: np.ndarray     # int32  [sumP]
    out_cache_loc: np.ndarray  # int64  [sumT]
    custom_mask: np.ndarray    # uint8  [sum T_b^2]
    mask_indptr: np.ndarray    # int32  [B+1]
    parents: List[List[int]]
    prefix_lens: List[int]
    tree_sizes: List[int]
    sm_scale: float = float(SM_SCALE)

    @property
    def batch(self) -> int:
        return len(self.prefix_lens)

    @property
    def total_q(self) -> int:
        return int(self.qo_indptr[-1])

    @property
    def total_kv(self) -> int:
        return int(self.kv_indptr[-1])

    def dense_pool(self, row_stride: int = D_QK, poison: bool = True) -> np.ndarray:
        """Materialise the full pool as uint16 [num_slots, row_stride]; unused
        slots (and padding columns) hold bf16 NaN when ``poison``."""
        fill = BF16_NAN if poison else np.uint16(0)
        pool = np.full((self.num_slots, row_stride), fill, dtype=np.uint16)
        pool[self.row_slots, :D_QK] = self.rows
        return pool

    def pool_view(self) -> "PoolView":
        return PoolView(self.num_slots, self.row_slots, self.rows)


class PoolView:
    """Read-only stand-in for a dense pool: ``view[slots]`` returns the rows a
    dense [num_slots, 576] pool would, without materialising it.  Unused slots
    read as bf16 NaN."""

    def __init__(self, num_slots: int, row_slots: np.ndarray, rows: np.ndarray):
        self.num_slots = int(num_slots)
        self.shape = (self.num_slots, rows.shape[1])
        self._lut = np.full(self.num_slots, -1, dtype=np.int64)
        self._lut[row_slots] = np.arange(len(row_slots))
        self._rows = np.concatenate([rows, np.full((1, rows.shape[1]), BF16_NAN, np.uint16)])

    def __getitem__(self, slots):
        idx = self._lut[np.asarray(slots, dtype=np.int64)]
        idx = np.where(idx < 0, len(self._rows) - 1, idx)
        return self._rows[idx]


def _build(name: str, seed: int, num_heads: int, num_slots: int,
           prefix_lens: Sequence[int], tree_sizes: Sequence[int], tree: str,
           outlier_frac: float, rng: np.random.Generator,
           slot_mode: str = "permutation") -> Instance:
    b = len(prefix_lens)
    assert len(tree_sizes) == b
    n_keys = [p + t for p, t in zip(prefix_lens, tree_sizes)]
    total_keys = int(sum(n_keys))
    if total_keys > num_slots:
        raise ValueError("pool too small for the instance")
    # 1. slots
    if slot_mode == "permutation":
        perm = rng.permutation(num_slots).astype(np.int64)
    elif slot_mode == "contiguous":
        perm = np.arange(num_slots, dtype=np.int64)
    else:
        raise ValueError(slot_mode)
    slots = perm[:total_keys]
    # 2. tree parents
    parents = []
    for t in tree_sizes:
        if t == 0:
            parents.append([])
        elif tree == "chain":
            parents.append(chain_parents(t))
        elif tree == "random":
            parents.append(random_parents(rng, t))
        else:
            raise ValueError(tree)
    # 3. latent rows, logical order (request by request: prefix then tree)
    vals = rng.standard_normal((total_keys, D_QK), dtype=np.float32)
    # 4. outliers among each request's prefix rows
    off = 0
    for p, nk in zip(prefix_lens, n_keys):
        n_out = int(np.floor(outlier_frac * p))
        if n_out > 0:
            pick = rng.choice(p, size=n_out, replace=False)
            vals[off + pick] *= np.float32(8.0)
        off += nk
    rows = f32_to_bf16_bits(vals)
    # 5. queries
    total_q = int(sum(tree_sizes))
    q = f32_to_bf16_bits(rng.standard_normal((total_q, num_heads, D_QK), dtype=np.float32))

    qo_indptr = np.zeros(b + 1, dtype=np.int32)
    kv_indptr = np.zeros(b + 1, dtype=np.int32)
    mask_indptr = np.zeros(b + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(tree_sizes)
    kv_indptr[1:] = np.cumsum(prefix_lens)
    mask_indptr[1:] = np.cumsum([t * t for t in tree_sizes])
    kv_indices = np.empty(int(kv_indptr[-1]), dtype=np.int32)
    out_cache_loc = np.empty(total_q, dtype=np.int64)
    masks = []
    off = 0
    for i, (p, t) in enumerate(zip(prefix_lens, tree_sizes)):
        kv_indices[kv_indptr[i]:kv_indptr[i + 1]] = slots[off:off + p]
        out_cache_loc[qo_indptr[i]:qo_indptr[i + 1]] = slots[off + p:off + p + t]
        masks.append(ancestor_or_self_mask(parents[i]).reshape(-1))
        off += p + t
    custom_mask = np.concatenate(masks) if masks else np.zeros(0, np.uint8)
    return Instance(name=name, seed=seed, num_heads=num_heads, num_slots=num_slots,
                    q=q, rows=rows, row_slots=slots.copy(), qo_indptr=qo_indptr,
                    kv_indptr=kv_indptr, kv_indices=kv_indices,
                    out_cache_loc=out_cache_loc, custom_mask=custom_mask.astype(np.uint8),
                    mask_indptr=mask_indptr, parents=parents,
                    prefix_lens=list(map(int, prefix_lens)),
                    tree_sizes=list(map(int, tree_sizes)))


def make_instance(prefix_lens: Sequence[int], tree_sizes: Sequence[int], num_heads: int,
                  num_slots: int, seed: int, tree: str = "random",
                  outlier_frac: float = 0.0, name: str = "custom",
                  slot_mode: str = "permutation") -> Instance:
    rng = np.random.default_rng(seed)
    return _build(name, seed, num_heads, num_slots, prefix_lens, tree_sizes, tree,
                  outlier_frac, rng, slot_mode)


# The five workload shapes (prefix length, tree, heads, pool size).
CONFIGS = {
    "tiny": dict(prefix_lens=[256], tree_sizes=[4], num_heads=8, num_slots=1024,
                 tree="chain", outlier_frac=0.0),
    "p5632_t16": dict(prefix_lens=[5632], tree_sizes=[16], num_heads=8, num_slots=65536,
                      tree="random", outlier_frac=0.0),
    "p23040_t32": dict(prefix_lens=[23040], tree_sizes=[32], num_heads=8, num_slots=262144,
                       tree="random", outlier_frac=0.0),
    "p91136_t32": dict(prefix_lens=[91136], tree_sizes=[32], num_heads=8, num_slots=1 << 20,
                       tree="random", outlier_frac=0.01),
    "p91136_t32_h64": dict(prefix_lens=[91136], tree_sizes=[32], num_heads=64,
                           num_slots=1 << 20, tree="random", outlier_frac=0.01),
}
CONFIG_SEEDS = {"tiny": 1001, "p5632_t16": 1002, "p23040_t32": 1003, "p91136_t32": 1004,
                "p91136_t32_h64": 1104}

# Decode: one query token per request (T_b = 1, its own key visible), many
# requests with prefixes drawn once, U[512, 8192], from fixed seeds.
DECODE_PREFIXES_B32 = [int(x) for x in np.random.default_rng(3032).integers(512, 8193, size=32)]
DECODE_PREFIXES_B64 = [int(x) for x in np.random.default_rng(3064).integers(512, 8193, size=64)]
CONFIGS["decode_b32_h16"] = dict(prefix_lens=DECODE_PREFIXES_B32, tree_sizes=[1] * 32, num_heads=16,
                                 num_slots=1 << 18, tree="random", outlier_frac=0.0)
CONFIGS["decode_b64_h128"] = dict(prefix_lens=DECODE_PREFIXES_B64, tree_sizes=[1] * 64, num_heads=128,
                                  num_slots=1 << 19, tree="random", outlier_frac=0.0)
CONFIG_SEEDS["decode_b32_h16"] = 1201
CONFIG_SEEDS["decode_b64_h128"] = 1202

# Segmented batch: 8 requests, prefixes U[1000, 185000], trees U[8, 64].
SEGMENTED = dict(batch=8, prefix_lo=1000, prefix_hi=185000, tree_lo=8, tree_hi=64,
                 num_heads=8, num_slots=1 << 21)
# Plan bounds for the segmented batch (every replay fits under them).
SEGMENTED_BOUNDS = dict(max_batch=8, max_q_tokens=512, max_tree_nodes=64,
                        max_kv_tokens=1_480_000, max_prefix_len=185_000)


def config(name: str, seed: Optional[int] = None) -> Instance:
    spec = dict(CONFIGS[name])
    s = CONFIG_SEEDS[name] if seed is None else seed
    return make_instance(name=name, seed=s, **spec)


def segmented(replay: int = 0, seed: Optional[int] = None) -> Instance:
    """The 8-request segmented batch; ``replay`` selects a fresh draw (seed 2000+replay)."""
    s = 2000 + replay if seed is None else seed
    rng = np.random.default_rng(s)
    sp = SEGMENTED
    prefix = rng.integers(sp["prefix_lo"], sp["prefix_hi"] + 1, size=sp["batch"]).tolist()
    trees = rng.integers(sp["tree_lo"], sp["tree_hi"] + 1, size=sp["batch"]).tolist()
    return _build(f"segmented_r{replay}", s, sp["num_heads"], sp["num_slots"], prefix, trees,
                  "random", 0.0, rng)


def segmented_pool(seed: int = 2999, num_slots: Optional[int] = None,
                   chunk_rows: int = 1 << 17, threads: int = 8) -> np.ndarray:
    """A fully populated bf16 pool [num_slots, 576] (N(0,1) rows) for replays
    that rewrite only metadata and queries between calls.  Chunk c of
    ``chunk_rows`` rows is drawn from child c of SeedSequence(seed), so the
    bits do not depend on the thread count."""
    from concurrent.futures import ThreadPoolExecutor
    n = SEGMENTED["num_slots"] if num_slots is None else num_slots
    pool = np.empty((n, D_QK), dtype=np.uint16)
    starts = list(range(0, n, chunk_rows))
    kids = np.random.SeedSequence(seed).spawn(len(starts))

    def fill(c):
        r0 = starts[c]
        r1 = min(n, r0 + chunk_rows)
        rng = np.random.default_rng(kids[c])
        pool[r0:r1] = f32_to_bf16_bits(rng.standard_normal((r1 - r0, D_QK), dtype=np.float32))

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(fill, range(len(starts))))
    return pool


@dataclasses.dataclass
class Replay:
    """Metadata and queries of one call over a fixed, fully populated pool."""
    seed: int
    num_heads: int
    num_slots: int
    q: np.ndarray
    qo_indptr: np.ndarray
    kv_indptr: np.ndarray
    kv_indices: np.ndarray
    out_cache_loc: np.ndarray
    custom_mask: np.ndarray
    mask_indptr: np.ndarray
    parents: List[List[int]]
    prefix_lens: List[int]
    tree_sizes: List[int]
    sm_scale: float = float(SM_SCALE)

    @property
    def batch(self) -> int:
        return len(self.prefix_lens)

    @property
    def total_q(self) -> int:
        return int(self.qo_indptr[-1])

    @property
    def total_kv(self) -> int:
        return int(self.kv_indptr[-1])


def segmented_replay(replay: int, num_slots: Optional[int] = None) -> Replay:
    """Replay ``replay`` of the segmented batch (seed 2000 + replay): fresh sizes,
    trees, slot placement and queries; rows come from ``segmented_pool``."""
    s = 2000 + replay
    rng = np.random.default_rng(s)
    sp = SEGMENTED
    n_slots = sp["num_slots"] if num_slots is None else num_slots
    prefix = rng.integers(sp["prefix_lo"], sp["prefix_hi"] + 1, size=sp["batch"]).tolist()
    trees = rng.integers(sp["tree_lo"], sp["tree_hi"] + 1, size=sp["batch"]).tolist()
    perm = rng.permutation(n_slots).astype(np.int64)
    parents = [random_parents(rng, t) for t in trees]
    total_q = int(sum(trees))
    q = f32_to_bf16_bits(rng.standard_normal((total_q, sp["num_heads"], D_QK), dtype=np.float32))
    b = sp["batch"]
    qo = np.zeros(b + 1, np.int32)
    kv = np.zeros(b + 1, np.int32)
    mi = np.zeros(b + 1, np.int32)
    qo[1:] = np.cumsum(trees)
    kv[1:] = np.cumsum(prefix)
    mi[1:] = np.cumsum([t * t for t in trees])
    kv_indices = np.empty(int(kv[-1]), np.int32)
    ocl = np.empty(total_q, np.int64)
    off = 0
    for i, (p, t) in enumerate(zip(prefix, trees)):
        kv_indices[kv[i]:kv[i + 1]] = perm[off:off + p]
        ocl[qo[i]:qo[i + 1]] = perm[off + p:off + p + t]
        off += p + t
    mask = np.concatenate([ancestor_or_self_mask(par).reshape(-1) for par in parents])
    return Replay(seed=s, num_heads=sp["num_heads"], num_slots=n_slots, q=q, qo_indptr=qo,
                  kv_indptr=kv, kv_indices=kv_indices, out_cache_loc=ocl,
                  custom_mask=mask.astype(np.uint8), mask_indptr=mi, parents=parents,
                  prefix_lens=prefix, tree_sizes=trees)
