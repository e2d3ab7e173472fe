"""Band (sliding-window or dense) attention through the sparse kernels.

sfag_band_indices turns the block-band test of the MindSpore FlashAttention
backward page ("flash_attention_bwd.py", compute_in_each_kv_block), taken per
query token and aligned on the bottom-right diagonal, into index rows; the
backward pass then runs unchanged.  The rows must equal the oracle's
band_indices bit for bit, and the backward on the library's rows must match
the float64 oracle on the oracle's own rows (relative L2: dQ/dQueryRope
<= 5e-3, dK/dV/dKeyRope <= 1e-2).
"""
import numpy as np
import pytest
import torch

import sfag_inputs as si
import top_sparse_attention_sfag_amd as sfag
from oracle import sfag_oracle as orc
from tests._helpers import add_oracle_stats, call_backward, geom_of, oracle_backward, to_device
from tests.test_gpu_parity import _check, _outs_np

pytestmark = pytest.mark.gpu

UNB = 2147483647

GEOMS = [
    dict(layout="BSND", B=2, S1=37, S2=53, pre=9, nxt=3, block=1),
    dict(layout="BSND", B=1, S1=70, S2=40, pre=UNB, nxt=0, block=1),
    dict(layout="BSND", B=1, S1=64, S2=64, pre=UNB, nxt=UNB, block=1),
    dict(layout="BSND", B=3, S1=20, S2=300, pre=45, nxt=17, block=16),
    dict(layout="TND", seqlens_q=(30, 0, 12, 50), seqlens_kv=(30, 7, 40, 50), pre=20, nxt=0, block=8),
    dict(layout="TND", seqlens_q=(5, 9), seqlens_kv=(200, 130), pre=UNB, nxt=UNB, block=64),
]


def _lib_rows(g, K):
    if g["layout"] == "BSND":
        return sfag.band_indices(pre_tokens=g["pre"], next_tokens=g["nxt"], block_size=g["block"], layout="BSND",
                                 B=g["B"], S1=g["S1"], S2=g["S2"], K=K)
    lq = torch.tensor(g["seqlens_q"], dtype=torch.int32, device="cuda")
    lk = torch.tensor(g["seqlens_kv"], dtype=torch.int32, device="cuda")
    return sfag.band_indices(pre_tokens=g["pre"], next_tokens=g["nxt"], block_size=g["block"], layout="TND",
                             seqlens_q=lq, seqlens_kv=lk, K=K)


def _geom(g):
    if g["layout"] == "BSND":
        return orc.geometry("BSND", g["B"], g["S1"], g["S2"])
    return orc.geometry("TND", len(g["seqlens_q"]), seqlens_q=g["seqlens_q"], seqlens_kv=g["seqlens_kv"])


@pytest.mark.parametrize("g", GEOMS, ids=[f"{g['layout']}_pre{g['pre']}_nxt{g['nxt']}_b{g['block']}" for g in GEOMS])
def test_band_indices_bit_exact(g):
    geom = _geom(g)
    max_lk = g["S2"] if g["layout"] == "BSND" else max(g["seqlens_kv"])
    K = orc.band_entries(max_lk, g["pre"], g["nxt"], g["block"])
    assert sfag.band_entries(max_lk, g["pre"], g["nxt"], g["block"]) == K
    print(f"band {g} K={K}", flush=True)
    got = _lib_rows(g, K)
    torch.cuda.synchronize()
    ref = orc.band_indices(geom, K, g["pre"], g["nxt"], g["block"])
    np.testing.assert_array_equal(got.reshape(geom["T1"], K).cpu().numpy(), ref)
    # a shorter K cuts rows after K entries
    if K > 2:
        cut = _lib_rows(g, K - 2)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(cut.reshape(geom["T1"], K - 2).cpu().numpy(), ref[:, : K - 2])


BAND_CASES = [
    (si.Case("band_dense_g16", S1=80, S2=80, G=16, K=80, mode=0), UNB, UNB),
    (si.Case("band_window_g64", S1=160, S2=160, G=64, K=48, mode=0), 47, 0),
    (si.Case("band_window_g128_blk16", S1=70, S2=150, G=128, K=1, block=16, mode=0), 40, 8),
    (si.Case("band_tnd_g32_fp16", layout="TND", B=3, seqlens_q=(40, 0, 25), seqlens_kv=(60, 9, 25), G=32, K=1,
             Dr=0, dtype="fp16", mode=0), 24, 0),
]


@pytest.mark.parametrize("case,pre,nxt", BAND_CASES, ids=[c[0].name for c in BAND_CASES])
def test_band_backward_against_oracle(case, pre, nxt):
    geom = geom_of(case)
    max_lk = case.S2 if case.layout == "BSND" else max(case.seqlens_kv)
    K = orc.band_entries(max_lk, pre, nxt, case.block)
    case = case.replace(K=K)
    inp = si.make_inputs(case, 21)
    shape = tuple(inp["sparse_indices"].shape)
    inp["sparse_indices"] = torch.from_numpy(orc.band_indices(geom, K, pre, nxt, case.block).astype(np.int32)
                                             ).reshape(shape)
    inp = add_oracle_stats(case, inp)
    ref = oracle_backward(case, inp)
    dev = to_device(inp)
    g = dict(layout=case.layout, pre=pre, nxt=nxt, block=case.block)
    if case.layout == "BSND":
        g.update(B=case.B, S1=case.S1, S2=case.S2)
    else:
        g.update(seqlens_q=case.seqlens_q, seqlens_kv=case.seqlens_kv)
    dev["sparse_indices"] = _lib_rows(g, K).reshape(shape)
    print(f"band backward {case.name} pre={pre} nxt={nxt} K={K}", flush=True)
    outs = call_backward(case, dev)
    torch.cuda.synchronize()
    _check(case, _outs_np(case, outs), ref, label=case.name)
