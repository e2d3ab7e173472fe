"""The seeded generator produces the index structures the workloads name."""
import numpy as np
import torch

import sfag_inputs as si


def _idx(case, seed=3):
    d = si.make_inputs(case, seed)
    return d["sparse_indices"].reshape(case.T1, case.Kent).numpy()


def test_uniform_distinct_in_range():
    c = si.CONFIGS[1].replace(S1=16, S2=256, K=64)
    idx = _idx(c)
    for row in idx:
        assert len(set(row.tolist())) == 64 and row.min() >= 0 and row.max() < 256


def test_causal_mix_rule():
    c = si.CONFIGS[2].replace(S1=200, S2=200, G=2, K=64)
    idx = _idx(c)
    for t, row in enumerate(idx):
        v = row[row >= 0]
        assert len(set(v.tolist())) == len(v)
        assert v.max() <= t
        if t + 1 <= 64:
            assert sorted(v.tolist()) == list(range(t + 1))
            assert np.all(row[len(v):] == -1)
        else:
            assert len(v) == 64
            assert set(range(t - 16 + 1, t + 1)) <= set(v.tolist())


def test_tnd_rows_are_local():
    c = si.CONFIGS[3].replace(seqlens_q=(40, 8, 0, 30), seqlens_kv=(40, 8, 0, 30), G=2, K=16)
    idx = _idx(c)
    qs = 0
    for lq in c.seqlens_q:
        for t in range(lq):
            v = idx[qs + t][idx[qs + t] >= 0]
            assert v.max() <= t and len(v) == min(16, t + 1)
        qs += lq


def test_zipf_skews_to_recent_keys():
    c = si.CONFIGS[5].replace(S1=600, S2=600, G=2, K=64)
    idx = _idx(c)
    ages = []
    for t, row in enumerate(idx):
        v = row[row >= 0]
        assert len(set(v.tolist())) == len(v) == min(64, t + 1)
        assert v.max() <= t
        if t >= 500:
            ages.extend((t - v).tolist())
    ages = np.array(ages)
    assert (ages < 32).mean() > 0.2 and np.median(ages) < 150


def test_blocks_rule():
    c = si.CONFIGS[4].replace(B=1, S1=8, S2=1024, K=32)
    idx = _idx(c)
    assert np.all(idx % 16 == 0)
    for row in idx:
        assert len(set(row.tolist())) == 32 and row.max() <= 1024 - 16


def test_seeded():
    c = si.CONFIGS[1].replace(S1=4, S2=64, K=8)
    a, b = si.make_inputs(c, 5), si.make_inputs(c, 5)
    for k in a:
        assert torch.equal(a[k], b[k])
