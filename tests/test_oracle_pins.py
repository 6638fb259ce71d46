"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against one of: a 50-digit brute-force evaluation
of the definition, a library routine (torch's scaled-dot-product attention in
float64), closed forms, invariants of the log-sum-exp merge, the semantics of
the sparse index array, and a hand-derived worked example under
tests/golden/.  ``test_planted_mistakes_are_caught`` plants plausible mistakes
in copies of the oracle's core and shows that these pins reject each one.
"""

import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import attention as oa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# Independent evaluations used as pins
# ----------------------------------------------------------------------------

def brute_force(q, k, v, scale, digits=50):
    """Definition evaluated directly at ``digits`` decimal digits, with no
    max-subtraction: out = sum e^{s_t} v_t / sum e^{s_t}, lse = ln sum e^{s_t}."""
    import mpmath as mp
    mp.mp.dps = digits
    H, T = q.shape[0], k.shape[0]
    outs, lses = [], []
    for h in range(H):
        e = []
        for t in range(T):
            s = mp.mpf(float(scale)) * mp.fsum(mp.mpf(float(q[h, d])) * mp.mpf(float(k[t, d]))
                                               for d in range(q.shape[1]))
            e.append(mp.exp(s))
        if T == 0:
            outs.append([0.0] * v.shape[1])
            lses.append(-math.inf)
            continue
        z = mp.fsum(e)
        outs.append([float(mp.fsum(e[t] * mp.mpf(float(v[t, d])) for t in range(T)) / z)
                     for d in range(v.shape[1])])
        lses.append(float(mp.log(z)))
    return np.array(outs), np.array(lses)


def sdpa_gqa(q, k_rows, v_rows, scale):
    """torch scaled_dot_product_attention (float64, CPU, enable_gqa) per row
    plus torch.logsumexp of the scaled scores, as a library cross-check."""
    import torch
    import torch.nn.functional as F
    outs, lses = [], []
    for b in range(q.shape[0]):
        qt = torch.tensor(q[b], dtype=torch.float64)[:, None, :][None]          # [1, Hq, 1, D]
        kt = torch.tensor(k_rows[b], dtype=torch.float64).permute(1, 0, 2)[None]  # [1, Hkv, L, D]
        vt = torch.tensor(v_rows[b], dtype=torch.float64).permute(1, 0, 2)[None]
        o = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=True)
        g = q.shape[1] // kt.shape[1]
        kr = kt.repeat_interleave(g, dim=1)                                      # head h -> kv h // g
        s = (qt @ kr.transpose(-1, -2)).squeeze(2) * scale                      # [1, Hq, L]
        outs.append(o[0, :, 0].numpy())
        lses.append(torch.logsumexp(s, dim=-1)[0].numpy())
    return np.stack(outs), np.stack(lses)


def rel_close(a, b, tol):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    err = np.where(both_inf, 0.0, np.abs(a - b) / np.maximum(1.0, np.abs(b)))
    return bool(np.all(err <= tol)), float(np.max(err, initial=0.0))


# ----------------------------------------------------------------------------
# Brute force at 50 digits
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_gqa_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    hq, hkv, d = 4, 2, 5
    lens = [int(rng.integers(1, 8)) for _ in range(2)]
    q = rng.standard_normal((2, hq, d))
    ks = [rng.standard_normal((L, hkv, d)) for L in lens]
    vs = [rng.standard_normal((L, hkv, d)) for L in lens]
    scale = 0.37
    out, lse = oracle.gqa_decode(q, ks, vs, scale)
    for b in range(2):
        for h in range(hq):
            bo, bl = brute_force(q[b, h:h + 1], ks[b][:, h // 2], vs[b][:, h // 2], scale)
            assert rel_close(out[b, h], bo[0], 1e-12)[0]
            assert rel_close(lse[b, h], bl[0], 1e-12)[0]


@pytest.mark.parametrize("seed", range(4))
def test_mla_matches_brute_force(seed):
    rng = np.random.default_rng(200 + seed)
    hq, dqk, dv = 3, 7, 4
    lens = [int(rng.integers(1, 9)) for _ in range(2)]
    q = rng.standard_normal((2, hq, dqk))
    cs = [rng.standard_normal((L, dqk)) for L in lens]
    scale = 0.29
    out, lse = oracle.mla_decode(q, cs, scale, dv=dv)
    for b in range(2):
        bo, bl = brute_force(q[b], cs[b], cs[b][:, :dv], scale)
        assert rel_close(out[b], bo, 1e-12)[0]
        assert rel_close(lse[b], bl, 1e-12)[0]


def test_sparse_matches_brute_force():
    rng = np.random.default_rng(7)
    hq, dqk, dv, L, W = 2, 6, 3, 9, 6
    q = rng.standard_normal((1, hq, dqk))
    c = rng.standard_normal((L, dqk))
    idx = np.array([[4, 0, 8, -1, 4, 2]], dtype=np.int32)   # -1 inside topk_len, a duplicate
    out, lse = oracle.mla_sparse_decode(q, [c], [L], idx, [5], 0.41, dv=dv)
    used = [4, 0, 8, 4]                                     # slot 3 skipped, slot 5 past topk_len
    bo, bl = brute_force(q[0], c[used], c[used][:, :dv], 0.41)
    assert rel_close(out[0], bo, 1e-12)[0] and rel_close(lse[0], bl, 1e-12)[0]


# ----------------------------------------------------------------------------
# Library cross-check
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (6, 1), (32, 8)])
def test_gqa_matches_torch_sdpa(hq, hkv):
    rng = np.random.default_rng(hq * 10 + hkv)
    d = 16
    lens = [1, 5, 33, 130]
    q = rng.standard_normal((len(lens), hq, d))
    ks = [rng.standard_normal((L, hkv, d)) for L in lens]
    vs = [rng.standard_normal((L, hkv, d)) for L in lens]
    scale = 1.0 / math.sqrt(d)
    out, lse = oracle.gqa_decode(q, ks, vs, scale)
    so, sl = sdpa_gqa(q, ks, vs, scale)
    assert np.max(np.abs(out - so)) < 1e-12
    assert np.max(np.abs(lse - sl)) < 1e-12


def test_mla_is_mqa_with_shared_latent_torch_sdpa():
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(11)
    hq, dqk, dv, L = 16, 40, 24, 70
    q = rng.standard_normal((1, hq, dqk))
    c = rng.standard_normal((L, dqk))
    scale = 1.0 / math.sqrt(12.0)
    out, lse = oracle.mla_decode(q, [c], scale, dv=dv)
    qt = torch.tensor(q)[0][None, :, None, :]
    ct = torch.tensor(c)[None, None]
    so = F.scaled_dot_product_attention(qt, ct, ct[..., :dv], scale=scale, enable_gqa=True)
    assert np.max(np.abs(out[0] - so[0, :, 0].numpy())) < 1e-12
    sl = torch.logsumexp((qt[0, :, 0] @ ct[0, 0].T) * scale, dim=-1).numpy()
    assert np.max(np.abs(lse[0] - sl)) < 1e-12


# ----------------------------------------------------------------------------
# Closed forms and the worked example
# ----------------------------------------------------------------------------

def test_worked_example_golden():
    g = json.load(open(os.path.join(GOLDEN, "three_token_worked_example.json")))
    q, k, v = np.array(g["q"]), np.array(g["k"]), np.array(g["v"])
    out, lse = oracle.attend(q, k, v, g["scale"])
    assert np.allclose(out, g["expected_out"], rtol=0, atol=1e-13)
    assert np.allclose(lse, g["expected_lse"], rtol=0, atol=1e-14)
    a = oracle.attend(q, k[:1], v[:1], g["scale"])
    b = oracle.attend(q, k[1:], v[1:], g["scale"])
    assert np.allclose(a[0], g["part_a"]["out"], atol=1e-14) and np.allclose(a[1], g["part_a"]["lse"], atol=1e-14)
    assert np.allclose(b[0], g["part_b"]["out"], atol=1e-13) and np.allclose(b[1], g["part_b"]["lse"], atol=1e-14)
    m = oracle.merge(a, b)
    assert np.allclose(m[0], g["expected_out"], atol=1e-13) and np.allclose(m[1], g["expected_lse"], atol=1e-14)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((5, 9)), rng.standard_normal((1, 9)), rng.standard_normal((1, 4))
    out, lse = oracle.attend(q, k, v, 0.5)
    assert np.array_equal(out, np.repeat(v, 5, axis=0))
    assert np.allclose(lse, 0.5 * (q @ k[0]), rtol=0, atol=1e-15)


def test_zero_query_gives_mean_and_log_length():
    rng = np.random.default_rng(4)
    L = 37
    k, v = rng.standard_normal((L, 8)), rng.standard_normal((L, 3))
    out, lse = oracle.attend(np.zeros((2, 8)), k, v, 0.9)
    assert np.allclose(out, v.mean(axis=0), rtol=0, atol=1e-14)
    assert np.allclose(lse, math.log(L), rtol=0, atol=1e-14)


def test_equal_values_give_that_value_and_probabilities_sum_to_one():
    rng = np.random.default_rng(5)
    L = 50
    q, k = rng.standard_normal((4, 8)), rng.standard_normal((L, 8)) * 3
    v = np.ones((L, 2)) * np.array([1.0, -2.5])
    out, _ = oracle.attend(q, k, v, 1.3)
    assert np.allclose(out, [1.0, -2.5], rtol=0, atol=1e-13)


def test_huge_scores_do_not_overflow():
    # s = [1000, 1000 + ln 3]: naive exp overflows; answer is (v0 + 3 v1) / 4
    q = np.array([[1.0]])
    k = np.array([[1000.0], [1000.0 + math.log(3.0)]])
    v = np.array([[4.0], [-4.0]])
    out, lse = oracle.attend(q, k, v, 1.0)
    assert np.allclose(out, [[(4.0 - 12.0) / 4.0]], atol=1e-12)
    assert np.allclose(lse, [1000.0 + math.log(4.0)], atol=1e-12)


def test_empty_key_set():
    out, lse = oracle.attend(np.ones((3, 4)), np.zeros((0, 4)), np.zeros((0, 2)), 1.0)
    assert np.array_equal(out, np.zeros((3, 2))) and np.all(lse == -np.inf)
    out, lse = oracle.mla_sparse_decode(np.ones((1, 2, 4)), [np.ones((5, 4))], [5],
                                        np.array([[-1, 7, 9]]), [3], 1.0, dv=2)
    assert np.array_equal(out, np.zeros((1, 2, 2))) and np.all(lse == -np.inf)


# ----------------------------------------------------------------------------
# Merge invariants and split-then-merge
# ----------------------------------------------------------------------------

def _rand_part(rng, h=3, d=4):
    return rng.standard_normal((h, d)), rng.standard_normal(h) * 5


def test_merge_associative_commutative_identity():
    rng = np.random.default_rng(9)
    a, b, c = _rand_part(rng), _rand_part(rng), _rand_part(rng)
    ident = (np.zeros((3, 4)), np.full(3, -np.inf))
    l = oracle.merge(oracle.merge(a, b), c)
    r = oracle.merge(a, oracle.merge(b, c))
    assert np.allclose(l[0], r[0], atol=1e-13) and np.allclose(l[1], r[1], atol=1e-13)
    ab, ba = oracle.merge(a, b), oracle.merge(b, a)
    assert np.allclose(ab[0], ba[0], atol=1e-14) and np.allclose(ab[1], ba[1], atol=1e-14)
    ai = oracle.merge(a, ident)
    assert np.allclose(ai[0], a[0], atol=1e-15) and np.allclose(ai[1], a[1], atol=1e-15)
    ii = oracle.merge(ident, ident)
    assert np.array_equal(ii[0], ident[0]) and np.all(ii[1] == -np.inf)


@settings(max_examples=60, deadline=None)
@given(L=st.integers(1, 60), cuts=st.lists(st.integers(0, 60), max_size=6), seed=st.integers(0, 10**6))
def test_split_anywhere_then_merge_equals_whole(L, cuts, seed):
    rng = np.random.default_rng(seed)
    q, k, v = rng.standard_normal((4, 6)), rng.standard_normal((L, 6)) * 2, rng.standard_normal((L, 5))
    bounds = sorted({0, L, *[c for c in cuts if c <= L]})
    parts = [oracle.attend(q, k[a:b], v[a:b], 0.7) for a, b in zip(bounds[:-1], bounds[1:])]
    got = oracle.merge_many(parts)
    whole = oracle.attend(q, k, v, 0.7)
    assert np.allclose(got[0], whole[0], rtol=0, atol=1e-12)
    assert np.allclose(got[1], whole[1], rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# Sparse semantics
# ----------------------------------------------------------------------------

def test_sparse_permutation_equals_dense():
    rng = np.random.default_rng(12)
    L, hq, dqk, dv = 40, 4, 12, 8
    q = rng.standard_normal((1, hq, dqk))
    c = rng.standard_normal((L, dqk))
    idx = rng.permutation(L).astype(np.int32)[None]
    so, sl = oracle.mla_sparse_decode(q, [c], [L], idx, [L], 0.3, dv=dv)
    do, dl = oracle.mla_decode(q, [c], 0.3, dv=dv)
    assert np.allclose(so, do, atol=1e-13) and np.allclose(sl, dl, atol=1e-13)


def test_sparse_masks_and_multiplicity():
    rng = np.random.default_rng(13)
    L, hq, dqk, dv = 10, 2, 6, 4
    q = rng.standard_normal((1, hq, dqk))
    c = rng.standard_normal((L, dqk))
    idx = np.array([[3, -1, 10, 3, 7, 12345, 1, 2]], dtype=np.int32)
    # topk_len 7: slots 0..6; -1, 10 (== L) and 12345 masked; 3 counted twice
    so, sl = oracle.mla_sparse_decode(q, [c], [L], idx, [7], 0.5, dv=dv)
    rows = c[[3, 3, 7, 1]]
    eo, el = oracle.attend(q[0], rows, rows[:, :dv], 0.5)
    assert np.allclose(so[0], eo, atol=1e-14) and np.allclose(sl[0], el, atol=1e-14)
    assert list(oracle.sparse_positions(idx[0], 7, L)) == [3, 3, 7, 1]
    assert list(oracle.sparse_positions(idx[0], 0, L)) == []


# ----------------------------------------------------------------------------
# Planted mistakes: each plausible error in the core formula fails a pin
# ----------------------------------------------------------------------------

def _mutant_attend(kind):
    def attend(q, k, v, scale):
        q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
        if k.shape[0] == 0:
            return np.zeros((q.shape[0], v.shape[1])), np.full(q.shape[0], -np.inf)
        sc = {"no_scale": 1.0, "sqrt_scale": math.sqrt(scale)}.get(kind, scale)
        s = sc * (q @ k.T)
        if kind == "neg_scores":
            s = -s
        m = s.max(axis=1, keepdims=True)
        if kind == "no_max_shift":
            m = np.zeros_like(m)
        z = np.exp(s - m).sum(axis=1, keepdims=True)
        lse = m + np.log(z)
        if kind == "log2_lse":
            lse = (m + np.log(z)) / math.log(2.0)
        p = np.exp(s - lse)
        if kind == "unnormalised":
            p = np.exp(s - m)
        out = p @ v
        if kind == "drop_last_token":
            out, lse = attend_ok(q, k[:-1], v[:-1], scale) if k.shape[0] > 1 else (out, lse[:, 0:1] * 0)
            return out, lse
        return out, lse[:, 0]
    return attend


attend_ok = oa.attend


def _pins_pass(monkeypatch, attend_impl, gqa_map=None):
    """Run a subset of the pins against a mutated oracle; True iff all pass."""
    monkeypatch.setattr(oa, "attend", attend_impl)
    try:
        if gqa_map is not None:
            monkeypatch.setattr(oa, "gqa_decode", gqa_map)
        checks = []
        rng = np.random.default_rng(77)
        # brute force, MLA shapes
        q = rng.standard_normal((1, 3, 7))
        c = rng.standard_normal((6, 7))
        out, lse = oa.mla_decode(q, [c], 0.29, dv=4)
        bo, bl = brute_force(q[0], c, c[:, :4], 0.29)
        checks.append(rel_close(out[0], bo, 1e-12)[0] and rel_close(lse[0], bl, 1e-12)[0])
        # torch library cross-check, GQA head mapping
        q = rng.standard_normal((2, 8, 16))
        ks = [rng.standard_normal((L, 2, 16)) for L in (5, 33)]
        vs = [rng.standard_normal((L, 2, 16)) for L in (5, 33)]
        out, lse = oa.gqa_decode(q, ks, vs, 0.25)
        so, sl = sdpa_gqa(q, ks, vs, 0.25)
        checks.append(np.max(np.abs(out - so)) < 1e-12 and np.max(np.abs(lse - sl)) < 1e-12)
        # overflow closed form
        o, l = oa.attend(np.array([[1.0]]), np.array([[1000.0], [1000.0 + math.log(3.0)]]),
                         np.array([[4.0], [-4.0]]), 1.0)
        checks.append(bool(np.all(np.isfinite(o))) and abs(o[0, 0] + 2.0) < 1e-12)
        return all(checks)
    finally:
        monkeypatch.undo()


def _gqa_wrong_head_map(q, k_rows, v_rows, scale):
    q = np.asarray(q, np.float64)
    outs, lses = [], []
    for b in range(q.shape[0]):
        kb, vb = np.asarray(k_rows[b]), np.asarray(v_rows[b])
        hkv = kb.shape[1]
        ob, lb = np.zeros((q.shape[1], vb.shape[2])), np.zeros(q.shape[1])
        for h in range(q.shape[1]):
            ob[h:h + 1], lb[h:h + 1] = oa.attend(q[b, h:h + 1], kb[:, h % hkv], vb[:, h % hkv], scale)
        outs.append(ob)
        lses.append(lb)
    return np.stack(outs), np.stack(lses)


def test_pins_accept_the_oracle(monkeypatch):
    assert _pins_pass(monkeypatch, attend_ok)


@pytest.mark.parametrize("kind", ["no_scale", "sqrt_scale", "neg_scores", "no_max_shift",
                                  "log2_lse", "unnormalised", "drop_last_token"])
def test_planted_mistakes_are_caught(monkeypatch, kind):
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        assert not _pins_pass(monkeypatch, _mutant_attend(kind))


def test_planted_head_mapping_mistake_is_caught(monkeypatch):
    assert not _pins_pass(monkeypatch, attend_ok, gqa_map=_gqa_wrong_head_map)


# ----------------------------------------------------------------------------
# Extra KV source: one softmax over the main and the extra gathered sets
# ----------------------------------------------------------------------------

def _extra_inputs(seed, hq=3, dqk=7, dv=4, L=11, LX=9, W=6, WX=5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, hq, dqk))
    c = rng.standard_normal((L, dqk))
    cx = rng.standard_normal((LX, dqk))
    idx = rng.permutation(L)[:W].astype(np.int32)[None]
    xidx = rng.permutation(LX)[:WX].astype(np.int32)[None]
    return q, c, cx, idx, xidx, dv


def test_extra_source_matches_brute_force_over_the_union():
    q, c, cx, idx, xidx, dv = _extra_inputs(21)
    # main: slots 0..3 used, slot 1 made -1 (skipped); extra: slots 0..2, one out of range
    idx = idx.copy(); idx[0, 1] = -1
    xidx = xidx.copy(); xidx[0, 2] = 9                      # == extra length: masked
    out, lse = oracle.mla_sparse_extra_decode(q, [c], [11], idx, [4], [cx], [9], xidx, [3], 0.37, dv=dv)
    keys = np.concatenate([c[[idx[0, 0], idx[0, 2], idx[0, 3]]], cx[[xidx[0, 0], xidx[0, 1]]]])
    bo, bl = brute_force(q[0], keys, keys[:, :dv], 0.37)
    assert rel_close(out[0], bo, 1e-12)[0] and rel_close(lse[0], bl, 1e-12)[0]


def test_extra_source_reduces_to_plain_sparse_when_either_set_is_empty():
    q, c, cx, idx, xidx, dv = _extra_inputs(22)
    so, sl = oracle.mla_sparse_decode(q, [c], [11], idx, [6], 0.5, dv=dv)
    eo, el = oracle.mla_sparse_extra_decode(q, [c], [11], idx, [6], [cx], [9], xidx, [0], 0.5, dv=dv)
    assert np.array_equal(so, eo) and np.array_equal(sl, el)
    xo, xl = oracle.mla_sparse_decode(q, [cx], [9], xidx, [5], 0.5, dv=dv)
    eo, el = oracle.mla_sparse_extra_decode(q, [c], [11], idx, [0], [cx], [9], xidx, [5], 0.5, dv=dv)
    assert np.array_equal(xo, eo) and np.array_equal(xl, el)
    eo, el = oracle.mla_sparse_extra_decode(q, [c], [11], idx, [0], [cx], [9], xidx, [0], 0.5, dv=dv)
    assert np.all(eo == 0.0) and np.all(np.isneginf(el))


def test_extra_source_is_the_merge_of_the_two_sets():
    q, c, cx, idx, xidx, dv = _extra_inputs(23)
    a = oracle.mla_sparse_decode(q, [c], [11], idx, [6], 0.45, dv=dv)
    x = oracle.mla_sparse_decode(q, [cx], [9], xidx, [5], 0.45, dv=dv)
    mo, ml = oracle.merge(a, x)
    eo, el = oracle.mla_sparse_extra_decode(q, [c], [11], idx, [6], [cx], [9], xidx, [5], 0.45, dv=dv)
    assert rel_close(eo, mo, 1e-12)[0] and rel_close(el, ml, 1e-12)[0]


def test_extra_source_with_full_permutations_equals_dense_over_both_caches():
    rng = np.random.default_rng(24)
    L, LX, hq, dqk, dv = 30, 17, 4, 10, 6
    q = rng.standard_normal((1, hq, dqk))
    c = rng.standard_normal((L, dqk))
    cx = rng.standard_normal((LX, dqk))
    idx = rng.permutation(L).astype(np.int32)[None]
    xidx = rng.permutation(LX).astype(np.int32)[None]
    eo, el = oracle.mla_sparse_extra_decode(q, [c], [L], idx, [L], [cx], [LX], xidx, [LX], 0.3, dv=dv)
    do, dl = oracle.mla_decode(q, [np.concatenate([c, cx])], 0.3, dv=dv)
    assert np.allclose(eo, do, atol=1e-13) and np.allclose(el, dl, atol=1e-13)


def test_extra_positions_are_checked_against_the_extra_length():
    # an extra position valid for the main cache (len 11) but not for the
    # extra cache (len 4) must be skipped
    q, c, cx, idx, xidx, dv = _extra_inputs(25, LX=9)
    xidx = np.array([[2, 7, 3, -1, 0]], dtype=np.int32)
    eo, el = oracle.mla_sparse_extra_decode(q, [c], [11], idx, [2], [cx], [4], xidx, [5], 0.6, dv=dv)
    keys = np.concatenate([c[idx[0, :2]], cx[[2, 3, 0]]])
    ro, rl = oracle.attend(q[0], keys, keys[:, :dv], 0.6)
    assert np.allclose(eo[0], ro, atol=1e-14) and np.allclose(el[0], rl, atol=1e-14)


def _extra_mutant(kind):
    def impl(q, rows, lens, idx, tl, xrows, xlens, xidx, xtl, scale, dv=512):
        q = np.asarray(q, np.float64)
        outs, lses = [], []
        for b in range(q.shape[0]):
            pos = oracle.sparse_positions(idx[b], int(tl[b]), int(lens[b]))
            xl = int(lens[b]) if kind == "main_len_for_extra" else int(xlens[b])
            xpos = oracle.sparse_positions(xidx[b], int(xtl[b]), xl)
            main = np.asarray(rows[b], np.float64)[pos]
            src = rows[b] if kind == "extra_from_main_cache" else xrows[b]
            xpos = xpos[xpos < len(src)]
            extra = np.asarray(src, np.float64)[xpos].reshape(-1, q.shape[2])
            if kind == "drop_extra":
                extra = extra[:0]
            if kind == "equal_weights" and len(main) and len(extra):
                oa_, la_ = oracle.attend(q[b], main, main[:, :dv], scale)
                ox_, lx_ = oracle.attend(q[b], extra, extra[:, :dv], scale)
                o, l = 0.5 * (oa_ + ox_), np.logaddexp(la_, lx_)
            else:
                g = np.concatenate([main.reshape(-1, q.shape[2]), extra])
                o, l = oracle.attend(q[b], g, g[:, :dv], scale)
            outs.append(o)
            lses.append(l)
        return np.stack(outs), np.stack(lses)
    return impl


_EXTRA_PINS = [test_extra_source_matches_brute_force_over_the_union,
               test_extra_source_reduces_to_plain_sparse_when_either_set_is_empty,
               test_extra_source_is_the_merge_of_the_two_sets,
               test_extra_source_with_full_permutations_equals_dense_over_both_caches,
               test_extra_positions_are_checked_against_the_extra_length]


@pytest.mark.parametrize("kind", ["drop_extra", "main_len_for_extra", "extra_from_main_cache", "equal_weights"])
def test_planted_extra_source_mistakes_are_caught(monkeypatch, kind):
    monkeypatch.setattr(oracle, "mla_sparse_extra_decode", _extra_mutant(kind))
    failed = 0
    for pin in _EXTRA_PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin rejects the planted mistake {kind}"


def test_extra_pins_accept_a_faithful_restatement(monkeypatch):
    monkeypatch.setattr(oracle, "mla_sparse_extra_decode", _extra_mutant("none"))
    for pin in _EXTRA_PINS:
        pin()
