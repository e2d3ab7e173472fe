"""GPU parity of the forward pass (out, softmaxMax, softmaxSum) against the
oracle's forward, on seeded inputs small enough for the oracle.

Tolerances: out relative L2 <= 5e-3 (out is rounded to the 16-bit input type,
2^-9 relative per element, and P enters the P·V product in that type as
well); softmaxMax within 1e-4 + 1e-4·|max| (fp32 logits of 16-bit products
against float64); softmaxSum within 1e-3 relative (fp32 exponentials and
sums).  Tokens with no valid position must give max = -inf, sum = 0 and
out = 0 exactly.
"""
import numpy as np
import pytest
import torch

import sfag_inputs as si
from oracle import sfag_oracle as orc
from tests._helpers import flat, geom_of, rel_l2, to_device

pytestmark = pytest.mark.gpu

CASES = [
    si.Case("fwd_g128_causal", S1=70, S2=70, G=128, K=40, mode=3, index_rule="causal_mix"),
    si.Case("fwd_g64_tnd", layout="TND", B=4, seqlens_q=(17, 0, 33, 9), seqlens_kv=(40, 5, 33, 20), G=64, K=24,
            mode=3, index_rule="causal_mix"),
    si.Case("fwd_g20_uniform", S1=5, S2=300, G=20, K=130),
    si.Case("fwd_g16_fp16_blocks", S1=6, S2=512, G=16, Dr=0, K=9, block=16, dtype="fp16", std=0.5,
            index_rule="blocks", scale=1 / 512 ** 0.5),
    si.Case("fwd_g4_rope", S1=8, S2=256, G=4, K=100),
    si.Case("fwd_g48_more_queries_than_keys", S1=40, S2=24, G=48, K=16, mode=3, index_rule="causal_mix"),
]


def _oracle(case, inp):
    f = flat(case, inp)
    return orc.forward(f["q"], f["k"], f["v"], f["qr"], f["kr"], f["idx"], geom_of(case), case.block, case.mode,
                       case.scale_value)


def _run(case, seed, value_is_key=False):
    import top_sparse_attention_sfag_amd as sfag
    inp = si.make_inputs(case, seed)
    if value_is_key:
        inp["value"] = inp["key"]
    O, M, L = _oracle(case, inp)
    d = to_device(inp)
    if value_is_key:
        d["value"] = d["key"]
    print(f"forward case {case.name} seed {seed} value_is_key={value_is_key}", flush=True)
    out, smax, ssum = sfag.forward(d["query"], d["key"], d["value"], d["sparse_indices"],
                                   seqlens_q=d.get("seqlens_q"), seqlens_kv=d.get("seqlens_kv"),
                                   query_rope=d.get("query_rope"), key_rope=d.get("key_rope"),
                                   scale=case.scale_value, block_size=case.block, layout=case.layout,
                                   sparse_mode=case.mode)
    torch.cuda.synchronize()
    T1, G = case.T1, case.G
    go = out.float().cpu().numpy().astype(np.float64).reshape(T1, G, case.D)
    gm = smax.cpu().numpy().astype(np.float64).reshape(T1, G)
    gl = ssum.cpu().numpy().astype(np.float64).reshape(T1, G)
    empty = np.isinf(M) & (M < 0)
    live = ~empty
    assert np.all(np.isneginf(gm[empty])) and np.all(gl[empty] == 0) and np.all(go[empty] == 0)
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gm[live])) and np.all(np.isfinite(gl))
    err = rel_l2(go, O)
    dm = np.max(np.abs(gm[live] - M[live]) / (1.0 + np.abs(M[live]))) if live.any() else 0.0
    dl = np.max(np.abs(gl[live] - L[live]) / L[live]) if live.any() else 0.0
    print(case.name, f"out rel-L2 {err:.2e}, max dev {dm:.2e}, sum rel dev {dl:.2e}", flush=True)
    # out is rounded to 16 bits (relative step 2^-8 for bf16, so a rel-L2 of
    # ~1e-3 from rounding alone); max and sum are fp32 results of fp32 dot
    # products over at most 576 bf16 terms and sums of at most K*block fp32
    # exponentials, whose rounding stays near 1e-6 relative
    assert err <= 5e-3, err
    np.testing.assert_allclose(gm[live], M[live], rtol=1e-4, atol=1e-4)
    np.testing.assert_allclose(gl[live], L[live], rtol=1e-4, atol=0)
    return go, gm, gl


@pytest.mark.parametrize("case", CASES, ids=[c.name for c in CASES])
def test_forward_against_oracle(case):
    _run(case, seed=5)


@pytest.mark.parametrize("case", CASES[:2] + CASES[3:4], ids=[c.name for c in CASES[:2] + CASES[3:4]])
def test_forward_value_is_key(case):
    _run(case, seed=6, value_is_key=True)


def test_forward_duplicated_indices():
    case = si.Case("fwd_dup", S1=4, S2=64, G=32, K=40)
    inp = si.make_inputs(case, 3)
    idx = inp["sparse_indices"].reshape(4, 40)
    idx[0, 10:20] = idx[0, 0]          # one key ten times: ten softmax terms
    idx[1, :] = -1                     # a token with no valid position
    O, M, L = _oracle(case, inp)
    assert np.isneginf(M[1]).all()
    import top_sparse_attention_sfag_amd as sfag
    d = to_device(inp)
    out, smax, ssum = sfag.forward(d["query"], d["key"], d["value"], d["sparse_indices"],
                                   query_rope=d["query_rope"], key_rope=d["key_rope"], scale=case.scale_value)
    torch.cuda.synchronize()
    go = out.float().cpu().numpy().astype(np.float64).reshape(4, 32, case.D)
    assert rel_l2(go, O) <= 5e-3
    gm = smax.cpu().numpy().reshape(4, 32)
    assert np.isneginf(gm[1]).all() and np.all(go[1] == 0)


def test_forward_then_backward_matches_oracle_pair():
    """The library's own forward statistics feed its backward: gradients match
    the oracle's backward run on the oracle's forward statistics."""
    import top_sparse_attention_sfag_amd as sfag
    from tests._helpers import add_oracle_stats, call_backward, oracle_backward
    case = si.Case("fwd_bwd_g64", S1=40, S2=40, G=64, K=24, mode=3, index_rule="causal_mix")
    inp = si.make_inputs(case, 9)
    ref = oracle_backward(case, add_oracle_stats(case, inp))
    d = to_device(inp)
    out, smax, ssum = sfag.forward(d["query"], d["key"], d["value"], d["sparse_indices"],
                                   query_rope=d["query_rope"], key_rope=d["key_rope"], scale=case.scale_value,
                                   sparse_mode=case.mode)
    d["out"], d["softmax_max"], d["softmax_sum"] = out, smax, ssum
    dq, dk, dv, dqr, dkr = call_backward(case, d)
    torch.cuda.synchronize()
    T1, T2, G = case.T1, case.T2, case.G
    f = lambda x, shape: x.float().cpu().numpy().astype(np.float64).reshape(shape)
    # the backward's own tolerances: the library's fp32 statistics and its
    # bf16-rounded out differ from the oracle's by far less than the 16-bit
    # rounding of dS and the gradients that those tolerances already absorb
    errs = dict(dq=rel_l2(f(dq, (T1, G, case.D)), ref["dq"]), dk=rel_l2(f(dk, (T2, case.D)), ref["dk"]),
                dv=rel_l2(f(dv, (T2, case.D)), ref["dv"]), dqr=rel_l2(f(dqr, (T1, G, case.Dr)), ref["dqr"]),
                dkr=rel_l2(f(dkr, (T2, case.Dr)), ref["dkr"]))
    print("forward-fed backward", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for n, tol in dict(dq=5e-3, dqr=5e-3, dk=1e-2, dv=1e-2, dkr=1e-2).items():
        assert errs[n] <= tol, (n, errs[n])
