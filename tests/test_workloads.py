"""Input-generation checks (no attention arithmetic here)."""
import numpy as np
import torch

from workloads import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 1e-30], np.float32)])
    ours = synth.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(synth.bf16_value(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_row_content_independent_of_batch_position():
    a = synth.gqa_case([5, 9], 4, 2, 8, 0.3, 4, structure_seed=7, seeds=[11, 12])
    b = synth.gqa_case([9, 3, 5], 4, 2, 8, 0.3, 4, structure_seed=8, seeds=[12, 13, 11])
    assert np.array_equal(a.rows[0].k, b.rows[2].k) and np.array_equal(a.rows[1].q, b.rows[0].q)


def test_paging_places_every_token_once():
    lens = [1, 16, 17, 100, 0]
    pg = synth.make_paging(lens, 16, np.random.default_rng(1))
    slots = np.concatenate([pg.token_slots(b, np.arange(L)) for b, L in enumerate(lens) if L])
    assert len(np.unique(slots)) == sum(lens)
    assert slots.max() < pg.num_pages * 16
    case = synth.gqa_case(lens, 4, 2, 8, 0.3, 16, structure_seed=3)
    pool = case.pool_bits()   # [NP, 2, Hkv, P, D]
    for b, L in enumerate(lens):
        for t in range(L):
            p, o = divmod(int(case.paging.token_slots(b, [t])[0]), 16)
            assert np.array_equal(pool[p, 0, :, o], case.rows[b].k[t])
            assert np.array_equal(pool[p, 1, :, o], case.rows[b].v[t])


def test_sparse_rows_shape_and_padding():
    r = synth.mla_sparse_row(5, 100, 4, 0.5, width=16, k=8)
    assert r.topk_len == 8 and np.all(r.topk_idx[8:] == -1)
    assert len(set(r.topk_idx[:8].tolist())) == 8 and r.topk_idx[:8].max() < 100
    short = synth.mla_sparse_row(5, 3, 4, 0.5, width=16)
    assert short.topk_len == 3 and sorted(short.topk_idx[:3].tolist()) == [0, 1, 2]
