"""The rest of the operator's supported envelope, beyond the five workloads
(operator page "aclnnSparseFlashAttentionGrad": parameter table — N1 values and
sparseBlockSize; 规格约束 — S1 and S2 up to 128K and allowed to differ):
sparseBlockSize 32 and 64, head counts the workloads do not use, fp16 on the
workloads that are bf16, and sequences of 128K tokens.

Every case compares the HIP path with the float64 oracle at the same
tolerances as the workload tests (relative L2: dQ/dQueryRope <= 5e-3,
dK/dV/dKeyRope <= 1e-2); key rows that no valid position selects must be
exactly 0.
"""
import numpy as np
import pytest
import torch

import sfag_inputs as si
from oracle import sfag_oracle as orc
from tests._helpers import call_backward, geom_of, rel_l2
from tests.test_gpu_parity import REDUCED, TOL, _run

pytestmark = pytest.mark.gpu

ENVELOPE = [
    si.Case("blk32_g16_causal", S1=40, S2=512, G=16, K=6, block=32, mode=3, index_rule="blocks"),
    si.Case("blk64_g64_fp16_norope", S1=5, S2=1024, G=64, Dr=0, K=6, block=64, dtype="fp16", std=0.5,
            index_rule="blocks"),
    si.Case("blk32_g128_causal", S1=40, S2=512, G=128, K=6, block=32, mode=3, index_rule="blocks"),
    si.Case("blk64_g4_tnd", layout="TND", B=3, seqlens_q=(9, 0, 20), seqlens_kv=(300, 64, 200), G=4, K=4,
            block=64, mode=3, index_rule="blocks"),
    si.Case("g2_rope", S1=7, S2=128, G=2, K=50),
    si.Case("g6_fp16", S1=5, S2=100, G=6, K=33, dtype="fp16"),
    si.Case("g12_causal", S1=50, S2=50, G=12, K=20, mode=3, index_rule="causal_mix"),
    si.Case("g24_norope", S1=4, S2=120, G=24, Dr=0, K=70),
    si.Case("g32_zipf", S1=60, S2=60, G=32, K=30, mode=3, index_rule="zipf"),
]


@pytest.mark.parametrize("case", ENVELOPE, ids=[c.name for c in ENVELOPE])
def test_envelope_against_oracle(case):
    _run(case, seed=7)


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_fp16_workload_structures(cfg):
    """The bf16 workloads' structure (heads, rope, layout, mask, index rule,
    determinism) in fp16 at a token count the oracle finishes in seconds."""
    case = REDUCED[cfg]
    _run(case.replace(name=case.name + "_fp16", dtype="fp16"), seed=si.seed_for(cfg))


def test_long_keys_short_queries():
    """S2 = 128K keys for 48 query tokens, bottom-right causal (every bound is
    far past the first 64K keys): positions near the end of a long key
    sequence, compared in full."""
    case = si.Case("s2_128k", S1=48, S2=131072, G=8, K=256, mode=3, index_rule="uniform")
    _run(case, seed=11)


def test_long_context_sampled():
    """S1 = S2 = 128K tokens (blocks of 64, causal): too large for the whole
    oracle, so sampled dQ rows of tokens and dK/dV rows of keys are compared,
    as in the full-size workload tests."""
    case = si.Case("s128k_blk64", S1=131072, S2=131072, G=8, K=16, block=64, mode=3, index_rule="blocks")
    seed = 13
    print(f"long context {case.name} seed {seed}", flush=True)
    inp = si.make_inputs(case, seed, device="cuda")
    inp.update(si.standin_stats(case, inp, seed, device="cuda"))
    dq, dk, dv, dqr, dkr = call_backward(case, inp)
    torch.cuda.synchronize()
    idx = inp["sparse_indices"].reshape(case.T1, case.Kent).cpu()
    geom = geom_of(case)
    rows = orc.decode(idx, case.block, case.mode, geom)
    counts = np.bincount(rows[rows >= 0], minlength=case.T2)
    rng = np.random.default_rng(seed)
    tokens = np.unique(np.concatenate([[0, case.T1 - 1], rng.choice(case.T1, 4, replace=False)]))
    live = np.nonzero(counts)[0]
    keys = np.unique(np.concatenate([[int(np.argmax(counts)), int(live[-1])], rng.choice(live, 3, replace=False)]))
    print(f"tokens {tokens.tolist()} keys {keys.tolist()}", flush=True)
    ref = orc.backward_rows(inp["query"].reshape(case.T1, case.G, case.D), inp["key"].reshape(case.T2, case.D),
                            inp["value"].reshape(case.T2, case.D), inp["query_rope"].reshape(case.T1, case.G, case.Dr),
                            inp["key_rope"].reshape(case.T2, case.Dr), idx, inp["dout"].reshape(case.T1, case.G, case.D),
                            inp["out"].reshape(case.T1, case.G, case.D), inp["softmax_max"].reshape(case.T1, case.G),
                            inp["softmax_sum"].reshape(case.T1, case.G), geom, case.block, case.mode,
                            case.scale_value, tokens=tokens, keys=keys, rows=rows)
    T = torch.as_tensor(tokens, device="cuda")
    Kt = torch.as_tensor(keys, device="cuda")
    got = dict(dq=dq.reshape(case.T1, case.G, case.D)[T], dqr=dqr.reshape(case.T1, case.G, case.Dr)[T],
               dk=dk.reshape(case.T2, case.D)[Kt], dv=dv.reshape(case.T2, case.D)[Kt],
               dkr=dkr.reshape(case.T2, case.Dr)[Kt])
    errs = {n: rel_l2(x.float().cpu().numpy().astype(np.float64), ref[n]) for n, x in got.items()}
    print(case.name, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for n, e in errs.items():
        assert e <= TOL[n], (n, e)
    never = torch.as_tensor(counts == 0, device="cuda")
    for x, w in ((dk, case.D), (dv, case.D), (dkr, case.Dr)):
        assert torch.all(x.reshape(case.T2, w)[never] == 0)


def test_few_tokens_split_and_deterministic():
    """Few tokens with N1 <= 16: the default call splits each token's
    positions over several workgroups (fp32 dQ sums); a deterministic call
    does not, and repeats bit for bit.  Both match the oracle."""
    case = si.Case("few_tokens_g4", S1=8, S2=400, G=4, K=256, mode=0, index_rule="uniform")
    inp, ref, got, _ = _run(case, seed=17)                       # split (4 shares of 64 positions)
    dev_inp = {k: v.cuda() for k, v in inp.items()}
    runs = []
    for _ in range(3):
        outs = call_backward(case, dev_inp, deterministic=True)
        torch.cuda.synchronize()
        runs.append([None if x is None else x.clone() for x in outs])
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            if a is not None:
                assert torch.equal(a, b)
    d_np = [None if x is None else x.float().cpu().numpy().astype(np.float64) for x in runs[0]]
    assert rel_l2(d_np[0].reshape(ref["dq"].shape), ref["dq"]) <= TOL["dq"]
    assert rel_l2(d_np[1].reshape(ref["dk"].shape), ref["dk"]) <= TOL["dk"]
