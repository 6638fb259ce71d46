"""Seeded synthetic decode-attention inputs.

This module draws inputs and lays them out; it holds none of the attention
arithmetic.  The oracle and the HIP path both consume what it produces.

Seeding: every row's content (its query and its keys/values or latent rows,
and for sparse rows its top-k positions) comes from its own
``numpy.random.default_rng(row_seed)``.  Batch structure (lengths, page
permutation) comes from a separate ``default_rng(structure_seed)``.  A row's
content therefore does not depend on where it sits in a batch or on which
rows share the batch, which is what the batch-invariance checks need.

Values are drawn in float32 and rounded to bf16 with round-to-nearest-even;
the rounded values are what both sides see (as float32 here, as bf16 bits on
the device).
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

MLA_DQK = 576
MLA_DV = 512


# ----------------------------------------------------------------------------
# bf16 encoding of generated values (input preparation only)
# ----------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.

    Inputs are finite draws; NaN/Inf handling is not needed here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the exact float32 values they encode."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def draw_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    """N(0, std^2) draws rounded to bf16; returns uint16 bits."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_bits(x)


# ----------------------------------------------------------------------------
# Row content
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class GqaRow:
    q: np.ndarray        # [Hq, D] uint16 bf16 bits
    k: np.ndarray        # [L, Hkv, D] uint16
    v: np.ndarray        # [L, Hkv, D] uint16


@dataclasses.dataclass
class MlaRow:
    q: np.ndarray        # [Hq, 576] uint16
    latent: Optional[np.ndarray]   # [L, 576] uint16 (dense rows)
    # sparse rows: positions (slot order, padded with -1 to the index width)
    # and the latent rows at the attended positions only
    topk_idx: Optional[np.ndarray] = None     # [W] int32
    topk_len: int = 0
    gathered: Optional[np.ndarray] = None     # [topk_len, 576] uint16, slot order


def gqa_row(row_seed: int, length: int, hq: int, hkv: int, d: int, std: float) -> GqaRow:
    rng = np.random.default_rng(row_seed)
    q = draw_bf16(rng, (hq, d), std)
    k = draw_bf16(rng, (length, hkv, d), std)
    v = draw_bf16(rng, (length, hkv, d), std)
    return GqaRow(q, k, v)


def mla_row(row_seed: int, length: int, hq: int, std: float) -> MlaRow:
    rng = np.random.default_rng(row_seed)
    q = draw_bf16(rng, (hq, MLA_DQK), std)
    latent = draw_bf16(rng, (length, MLA_DQK), std)
    return MlaRow(q, latent)


def mla_sparse_row(row_seed: int, length: int, hq: int, std: float, width: int,
                   k: Optional[int] = None) -> MlaRow:
    """Sparse row: ``min(k, length)`` distinct positions drawn without
    replacement from ``[0, length)``, kept in drawn order, ``-1`` past them.

    Only the attended latent rows are drawn (in slot order); the other
    positions of the row are never read by the method.
    """
    k = width if k is None else k
    rng = np.random.default_rng(row_seed)
    q = draw_bf16(rng, (hq, MLA_DQK), std)
    n = min(k, length)
    idx = np.full(width, -1, dtype=np.int32)
    if n:
        idx[:n] = rng.choice(length, size=n, replace=False).astype(np.int32)
    gathered = draw_bf16(rng, (n, MLA_DQK), std)
    return MlaRow(q, None, idx, n, gathered)


# ----------------------------------------------------------------------------
# Lengths
# ----------------------------------------------------------------------------

def lens_uniform(rng: np.random.Generator, batch: int, lo: int, hi: int) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=batch).astype(np.int32)


def lens_lognormal(rng: np.random.Generator, batch: int, median: float, sigma: float,
                   lo: int, hi: int) -> np.ndarray:
    z = rng.standard_normal(batch)
    return np.clip(np.rint(median * np.exp(sigma * z)), lo, hi).astype(np.int32)


# ----------------------------------------------------------------------------
# Paging: logical rows -> a shared pool of fixed-size pages + block table
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Paging:
    page_size: int
    num_pages: int
    block_table: np.ndarray    # [B, max_pages_per_row] int32, -1 where unused

    @property
    def max_pages_per_row(self) -> int:
        return self.block_table.shape[1]

    def token_slots(self, b: int, positions: np.ndarray) -> np.ndarray:
        """Flat pool slot (page * page_size + offset) of row b's positions."""
        positions = np.asarray(positions, dtype=np.int64)
        pages = self.block_table[b, positions // self.page_size].astype(np.int64)
        return pages * self.page_size + positions % self.page_size


def make_paging(lens: Sequence[int], page_size: int, rng: Optional[np.random.Generator],
                max_pages_per_row: Optional[int] = None, spare_pages: int = 0) -> Paging:
    """Deal pages to rows.  ``rng=None`` gives the identity (contiguous) layout:
    row b's pages follow row b-1's in order.  Otherwise the page pool is a
    seeded permutation, so consecutive logical pages of a row sit at unrelated
    physical pages."""
    lens = np.asarray(lens, dtype=np.int64)
    need = [(int(l) + page_size - 1) // page_size for l in lens]
    total = int(sum(need)) + spare_pages
    width = max([1] + need) if max_pages_per_row is None else max_pages_per_row
    if max(need + [0]) > width:
        raise ValueError("a row needs more pages than max_pages_per_row")
    order = np.arange(total, dtype=np.int32) if rng is None else rng.permutation(total).astype(np.int32)
    table = np.full((len(lens), width), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = order[off:off + n]
        off += n
    return Paging(page_size, total, table)


# ----------------------------------------------------------------------------
# Whole cases
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class GqaCase:
    rows: List[GqaRow]
    lens: np.ndarray
    hq: int
    hkv: int
    d: int
    scale: float
    paging: Paging
    split_tokens: int = 0

    @property
    def batch(self) -> int:
        return len(self.rows)

    def q_bits(self) -> np.ndarray:
        return np.stack([r.q for r in self.rows])

    def pool_bits(self) -> np.ndarray:
        """[num_pages, 2, Hkv, P, D] uint16; slots past a row's length are 0."""
        P = self.paging.page_size
        pool = np.zeros((self.paging.num_pages, P, 2, self.hkv, self.d), np.uint16)
        flat = pool.reshape(self.paging.num_pages * P, 2, self.hkv, self.d)
        for b, r in enumerate(self.rows):
            L = int(self.lens[b])
            if L:
                s = self.paging.token_slots(b, np.arange(L))
                flat[s, 0] = r.k
                flat[s, 1] = r.v
        return np.ascontiguousarray(pool.transpose(0, 2, 3, 1, 4))


@dataclasses.dataclass
class MlaCase:
    rows: List[MlaRow]
    lens: np.ndarray
    hq: int
    scale: float
    paging: Paging
    topk_width: int = 0         # 0 = dense
    split_tokens: int = 0
    # sparse only: a second gathered set per row from its own cache (the
    # extra KV source); a sparse case of the same batch whose q is unused
    extra: Optional["MlaCase"] = None

    @property
    def batch(self) -> int:
        return len(self.rows)

    @property
    def sparse(self) -> bool:
        return self.topk_width > 0

    def q_bits(self) -> np.ndarray:
        return np.stack([r.q for r in self.rows])

    def topk_idx(self) -> np.ndarray:
        return np.stack([r.topk_idx for r in self.rows]).astype(np.int32)

    def topk_len(self) -> np.ndarray:
        return np.array([r.topk_len for r in self.rows], dtype=np.int32)

    def placed_slots(self, b: int) -> np.ndarray:
        """Slots of sparse row b whose position is attended: below topk_len and
        inside [0, len).  Their gathered rows are what the row's cache holds at
        those positions."""
        r = self.rows[b]
        n = min(max(int(r.topk_len), 0), len(r.topk_idx), len(r.gathered))
        idx = r.topk_idx[:n]
        return np.nonzero((idx >= 0) & (idx < int(self.lens[b])))[0]

    def fill_pool(self, flat_pool: np.ndarray) -> None:
        """Write every row's content into a flat [num_pages * P, 576] uint16 pool."""
        for b, r in enumerate(self.rows):
            if self.sparse:
                j = self.placed_slots(b)
                if len(j):
                    flat_pool[self.paging.token_slots(b, r.topk_idx[j])] = r.gathered[j]
            else:
                L = int(self.lens[b])
                if L:
                    flat_pool[self.paging.token_slots(b, np.arange(L))] = r.latent

    def pool_bits(self) -> np.ndarray:
        P = self.paging.page_size
        pool = np.zeros((self.paging.num_pages, P, MLA_DQK), np.uint16)
        self.fill_pool(pool.reshape(-1, MLA_DQK))
        return pool

    def logical_rows(self):
        """Per-row logical latent arrays (float32), for the oracle.  Sparse rows
        get zeros at positions they never attend."""
        for b, r in enumerate(self.rows):
            if self.sparse:
                L = int(self.lens[b])
                arr = np.zeros((L, MLA_DQK), np.float32)
                j = self.placed_slots(b)
                if len(j):
                    arr[r.topk_idx[j]] = bf16_value(r.gathered[j])
                yield arr
            else:
                yield bf16_value(r.latent)


def row_seed(structure_seed: int, b: int) -> int:
    return (structure_seed << 20) + b


def gqa_case(lens, hq, hkv, d, scale, page_size, structure_seed, std=1.0,
             permute=True, split_tokens=0, seeds: Optional[Sequence[int]] = None,
             max_pages_per_row=None, spare_pages=0) -> GqaCase:
    lens = np.asarray(lens, dtype=np.int32)
    rng = np.random.default_rng(structure_seed)
    seeds = [row_seed(structure_seed, b) for b in range(len(lens))] if seeds is None else list(seeds)
    rows = [gqa_row(s, int(L), hq, hkv, d, std) for s, L in zip(seeds, lens)]
    paging = make_paging(lens, page_size, rng if permute else None, max_pages_per_row, spare_pages)
    return GqaCase(rows, lens, hq, hkv, d, scale, paging, split_tokens)


def mla_case(lens, hq, scale, page_size, structure_seed, std=0.5, topk_width=0, topk=None,
             split_tokens=0, seeds: Optional[Sequence[int]] = None, max_pages_per_row=None,
             spare_pages=0, permute=True) -> MlaCase:
    lens = np.asarray(lens, dtype=np.int32)
    rng = np.random.default_rng(structure_seed)
    seeds = [row_seed(structure_seed, b) for b in range(len(lens))] if seeds is None else list(seeds)
    if topk_width:
        rows = [mla_sparse_row(s, int(L), hq, std, topk_width, topk) for s, L in zip(seeds, lens)]
    else:
        rows = [mla_row(s, int(L), hq, std) for s, L in zip(seeds, lens)]
    paging = make_paging(lens, page_size, rng if permute else None, max_pages_per_row, spare_pages)
    return MlaCase(rows, lens, hq, scale, paging, topk_width, split_tokens)


EXTRA_SEED_OFFSET = 1 << 40   # extra-set row seed = main row seed + this


def mla_extra_case(lens, extra_lens, hq, scale, page_size, structure_seed, topk_width, extra_width,
                   extra_page_size=None, std=0.5, topk=None, extra_topk=None, split_tokens=0,
                   seeds: Optional[Sequence[int]] = None) -> MlaCase:
    """Sparse MLA case with an extra KV source: each row also attends
    ``min(extra_topk, extra_len)`` positions of its own extra cache.  The
    extra set of a row is drawn from the row's seed plus EXTRA_SEED_OFFSET,
    so it too does not depend on the batch."""
    lens = np.asarray(lens, dtype=np.int32)
    seeds = [row_seed(structure_seed, b) for b in range(len(lens))] if seeds is None else list(seeds)
    case = mla_case(lens, hq, scale, page_size, structure_seed, std=std, topk_width=topk_width, topk=topk,
                    split_tokens=split_tokens, seeds=seeds)
    case.extra = mla_case(extra_lens, hq, scale, page_size if extra_page_size is None else extra_page_size,
                          structure_seed + 7919, std=std, topk_width=extra_width, topk=extra_topk,
                          split_tokens=split_tokens, seeds=[s + EXTRA_SEED_OFFSET for s in seeds])
    return case


# ----------------------------------------------------------------------------
# The five workloads (shapes, distributions and structure of the decode
# batches the pages describe; sizes as stated in each docstring)
# ----------------------------------------------------------------------------

def config1_gqa_tiny() -> GqaCase:
    """Dense GQA, B=4, Hq=8, Hkv=2, D=64, lens 17/100/256/1000, N(0,1),
    scale 1/8, contiguous KV (identity table, 64-token pages), 64-token splits."""
    return gqa_case([17, 100, 256, 1000], 8, 2, 64, 1.0 / 8.0, 64, structure_seed=1,
                    std=1.0, permute=False, split_tokens=64)


def config2_gqa_lens(seed: int = 2, batch: int = 32) -> np.ndarray:
    return lens_uniform(np.random.default_rng([seed, 1]), batch, 128, 8192)


def config2_gqa(batch: int = 32, lens=None) -> GqaCase:
    """Dense GQA, Llama-8B-like: B=32, Hq=32, Hkv=8, D=128, N(0,1),
    lens uniform in [128, 8192], 16-token pages, permuted block table."""
    lens = config2_gqa_lens(2, batch) if lens is None else lens
    return gqa_case(lens, 32, 8, 128, 1.0 / math.sqrt(128.0), 16, structure_seed=2, std=1.0)


def config3_mla_lens(seed: int = 3, batch: int = 64) -> np.ndarray:
    return lens_lognormal(np.random.default_rng([seed, 1]), batch, 4096.0, 1.0, 64, 32768)


def config3_mla(batch: int = 64, lens=None) -> MlaCase:
    """Absorbed MLA: B=64, Hq=128, latent 576 (512 + 64 rope), Dv=512,
    scale 1/sqrt(192), N(0, 0.5^2), lens lognormal (median 4096, sigma 1)
    clipped to [64, 32768], 64-token pages, permuted table."""
    lens = config3_mla_lens(3, batch) if lens is None else lens
    return mla_case(lens, 128, 1.0 / math.sqrt(192.0), 64, structure_seed=3, std=0.5)


def config4_sparse_lens(seed: int = 4, batch: int = 64) -> np.ndarray:
    return lens_uniform(np.random.default_rng([seed, 1]), batch, 2048, 65536)


def config4_sparse(batch: int = 64, lens=None, width: int = 2048) -> MlaCase:
    """Sparse MLA: config-3 heads/dims, lens uniform in [2048, 65536],
    2048 top-k positions per row drawn without replacement from [0, len),
    topk_len = min(2048, len), -1 past topk_len."""
    lens = config4_sparse_lens(4, batch) if lens is None else lens
    return mla_case(lens, 128, 1.0 / math.sqrt(192.0), 64, structure_seed=4, std=0.5,
                    topk_width=width)


def config4_extra_lens(seed: int = 4, batch: int = 64) -> np.ndarray:
    return lens_uniform(np.random.default_rng([seed, 2]), batch, 512, 8192)


def config4_sparse_extra(batch: int = 64) -> MlaCase:
    """Sparse MLA with an extra KV source: the config-4 main set (lens
    uniform in [2048, 65536], 2048 top-k positions) plus, per row, 512
    positions drawn without replacement from an extra cache of its own with
    lens uniform in [512, 8192] (64-token pages).  The pages name the extra
    source but give no sizes; these are this workload's choice."""
    return mla_extra_case(config4_sparse_lens(4, batch), config4_extra_lens(4, batch), 128,
                          1.0 / math.sqrt(192.0), 64, structure_seed=4, topk_width=2048, extra_width=512)


PROBE_LEN = 16384
PROBE_SEED = 0


def config5_composition(batch: int, composition_seed: int):
    """Invariance stress: the probe row (len 16384, row seed 0) at a random
    position among ``batch - 1`` batchmates with lens uniform in [1, 131072].
    Returns (lens, seeds, probe_position)."""
    rng = np.random.default_rng([5, batch, composition_seed])
    lens = lens_uniform(rng, batch, 1, 131072)
    seeds = [row_seed(5, 1000 * composition_seed + j) + (batch << 12) for j in range(batch)]
    pos = int(rng.integers(0, batch))
    lens[pos] = PROBE_LEN
    seeds[pos] = PROBE_SEED
    return lens, seeds, pos
