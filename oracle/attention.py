"""Oracle for batch-invariant split-KV decode attention: plain, slow, fp64, CPU.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it, and it shares no code,
tables or helpers with that path.

What it computes is the plain definition of decode attention, written out
with no splitting, tiling or reordering:

* FlashMLA issue "Sparse MLA decode is not batch-invariant ..." (section
  "Where it comes from"): a decode row's keys are cut into splits, each split
  produces a partial output plus a log-sum-exp scale, and a combine step
  merges the partials with weights derived from those scales.  Whatever the
  split points, the merged result is mathematically the single-pass softmax
  attention of the row over its whole key set.  That single-pass result is
  what every function here returns, so it is the target that any split rule
  (per-row or batch-balanced) must reach up to rounding.
* Same page, section "Measurement": the sparse call takes per-row top-k
  index arrays plus a valid-entry count (``topk_length``); only the first
  ``topk_length`` entries of a row's index array are used.
* Same page, section "Question": splitting is per row, decided from the row's
  own length only.  This changes which partials exist, never the value being
  approximated, so the oracle has no notion of splits at all except
  :func:`merge`, which states the partial-merge rule itself.

Readings of points the pages leave open:

* The log-sum-exp is the natural log of the sum of exp of the *scaled*
  scores.
* Grouped-query heads: query head ``h`` reads key/value head ``h // G`` with
  ``G = Hq / Hkv`` (consecutive query heads share a kv head).
* Absorbed MLA: one latent row of 576 values per token serves as the key; its
  first ``dv`` (512) values serve as the value.  The score scale is the one
  passed in (1/sqrt(192) for DeepSeek-style shapes), not 1/sqrt(576).
* Sparse indices are row-local token positions.  An entry is used iff its
  slot is below the row's ``topk_len`` and its value lies in ``[0, L_b)``;
  ``-1`` or any other out-of-range value is skipped.  Duplicated positions
  count once per occurrence.
* An empty key set gives ``out = 0`` and ``lse = -inf``.
* Extra KV source (same page, sections "Measurement" and "Environment": the
  sparse call also takes ``extra_indices_in_kvcache`` / ``extra_topk_length``
  into a second cache, ``extra_k_cache``).  The pages name these arguments
  without defining them; the reading taken here is the plainest one: a row
  attends, with one softmax, the multiset union of its main gathered set
  (positions in its main cache) and its extra gathered set (positions in its
  extra cache, validated against the extra cache's own length).

All inputs are taken as given numbers (the exact bf16 values, widened to
float64); all arithmetic is float64.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "attend",
    "gqa_decode",
    "mla_decode",
    "mla_sparse_decode",
    "mla_sparse_extra_decode",
    "sparse_positions",
    "merge",
    "merge_many",
]


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Single-pass softmax attention of query rows over one key/value set.

    q: [H, Dqk]; k: [T, Dqk]; v: [T, Dv]; returns (out [H, Dv], lse [H]).

    For each query row: s_t = scale * <q, k_t>; M = max_t s_t;
    Z = sum_t exp(s_t - M); lse = M + ln Z; p_t = exp(s_t - lse);
    out = sum_t p_t v_t.  T = 0 gives out = 0, lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    h = q.shape[0]
    if k.shape[0] == 0:
        return np.zeros((h, v.shape[1]), np.float64), np.full(h, -np.inf)
    s = scale * (q @ k.T)                       # [H, T]
    m = s.max(axis=1, keepdims=True)
    z = np.exp(s - m).sum(axis=1, keepdims=True)
    lse = m + np.log(z)                         # [H, 1]
    p = np.exp(s - lse)                         # rows sum to 1
    return p @ v, lse[:, 0]


def gqa_decode(q, k_rows, v_rows, scale: float):
    """Dense grouped-query decode over logical (unpaged) per-row caches.

    q: [B, Hq, D]; k_rows[b], v_rows[b]: [L_b, Hkv, D].
    Returns out [B, Hq, D] and lse [B, Hq] (float64).
    """
    q = np.asarray(q, dtype=np.float64)
    b_count, hq, _ = q.shape
    d_v = None
    outs, lses = [], []
    for b in range(b_count):
        kb = np.asarray(k_rows[b], dtype=np.float64)
        vb = np.asarray(v_rows[b], dtype=np.float64)
        hkv = kb.shape[1]
        if hq % hkv:
            raise ValueError("Hq must be a multiple of Hkv")
        g = hq // hkv
        d_v = vb.shape[2]
        ob = np.zeros((hq, d_v))
        lb = np.zeros(hq)
        for kvh in range(hkv):
            heads = slice(kvh * g, (kvh + 1) * g)   # query heads h with h // g == kvh
            ob[heads], lb[heads] = attend(q[b, heads], kb[:, kvh], vb[:, kvh], scale)
        outs.append(ob)
        lses.append(lb)
    return np.stack(outs), np.stack(lses)


def mla_decode(q, latent_rows, scale: float, dv: int = 512):
    """Dense absorbed-MLA decode: every query head attends one shared latent.

    q: [B, Hq, Dqk]; latent_rows[b]: [L_b, Dqk]; the key is the whole latent
    row and the value is its first ``dv`` entries.
    Returns out [B, Hq, dv] and lse [B, Hq] (float64).
    """
    q = np.asarray(q, dtype=np.float64)
    outs, lses = [], []
    for b in range(q.shape[0]):
        c = np.asarray(latent_rows[b], dtype=np.float64)
        o, l = attend(q[b], c, c[:, :dv], scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def sparse_positions(idx_row, topk_len: int, length: int) -> np.ndarray:
    """The positions a sparse row attends, in slot order, with multiplicity.

    Slot j is used iff j < topk_len and 0 <= idx_row[j] < length.
    """
    idx = np.asarray(idx_row, dtype=np.int64)[: max(int(topk_len), 0)]
    return idx[(idx >= 0) & (idx < length)]


def mla_sparse_decode(q, latent_rows, lens, topk_idx, topk_len, scale: float, dv: int = 512):
    """Sparse absorbed-MLA decode over gathered top-k positions of each row.

    latent_rows[b] holds at least lens[b] logical token rows; topk_idx [B, W]
    holds row-local positions; topk_len [B] the per-row valid-slot count.
    """
    q = np.asarray(q, dtype=np.float64)
    outs, lses = [], []
    for b in range(q.shape[0]):
        pos = sparse_positions(topk_idx[b], int(topk_len[b]), int(lens[b]))
        g = np.asarray(np.asarray(latent_rows[b])[pos], dtype=np.float64)
        o, l = attend(q[b], g, g[:, :dv], scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def mla_sparse_extra_decode(q, latent_rows, lens, topk_idx, topk_len,
                            extra_rows, extra_lens, extra_idx, extra_topk_len, scale: float, dv: int = 512):
    """Sparse absorbed-MLA decode over two gathered key sets per row.

    Row b attends the latent rows of its main cache at
    ``sparse_positions(topk_idx[b], topk_len[b], lens[b])`` together with
    the latent rows of its extra cache at
    ``sparse_positions(extra_idx[b], extra_topk_len[b], extra_lens[b])``,
    all in one softmax (keys are the whole latent rows, values their first
    ``dv`` entries).  Either set may be empty.
    """
    q = np.asarray(q, dtype=np.float64)
    outs, lses = [], []
    for b in range(q.shape[0]):
        pos = sparse_positions(topk_idx[b], int(topk_len[b]), int(lens[b]))
        xpos = sparse_positions(extra_idx[b], int(extra_topk_len[b]), int(extra_lens[b]))
        width = q.shape[2]
        main = np.asarray(latent_rows[b], dtype=np.float64).reshape(-1, width)[pos]
        extra = np.asarray(extra_rows[b], dtype=np.float64).reshape(-1, width)[xpos]
        g = np.concatenate([main, extra], axis=0)        # main set first, then the extra set
        o, l = attend(q[b], g, g[:, :dv], scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def merge(a, b):
    """Merge two partial results (out, lse) of attention over disjoint key sets.

    With lam = max(lse_a, lse_b) + ln(exp(lse_a - max) + exp(lse_b - max)),
    the merged output is exp(lse_a - lam) * out_a + exp(lse_b - lam) * out_b.
    (0, -inf) is the identity.  Works on scalars or on arrays whose last
    axis of ``out`` is the value dimension and ``lse`` matches the rest.
    """
    oa, la = np.asarray(a[0], np.float64), np.asarray(a[1], np.float64)
    ob, lb = np.asarray(b[0], np.float64), np.asarray(b[1], np.float64)
    m = np.maximum(la, lb)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    with np.errstate(invalid="ignore"):
        wa = np.where(finite, np.exp(la - m_safe), 0.0)
        wb = np.where(finite, np.exp(lb - m_safe), 0.0)
    tot = wa + wb
    lam = np.where(finite, m_safe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    ca = np.where(finite, wa / np.where(finite, tot, 1.0), 0.0)
    cb = np.where(finite, wb / np.where(finite, tot, 1.0), 0.0)
    out = ca[..., None] * oa + cb[..., None] * ob
    return out, lam


def merge_many(parts):
    """Left-to-right merge of a sequence of partials; empty sequence -> identity."""
    parts = list(parts)
    if not parts:
        raise ValueError("merge_many needs at least one partial to know the shape")
    acc = (np.zeros_like(np.asarray(parts[0][0], np.float64)),
           np.full_like(np.asarray(parts[0][1], np.float64), -np.inf))
    for p in parts:
        acc = merge(acc, p)
    return acc

