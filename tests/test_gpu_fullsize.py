"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (default chunking and scatter path, deterministic as the
workload states).  The oracle cannot run these whole, so it computes sampled
output rows one by one: dQ/dQueryRope rows of sampled tokens (each depends only
on its own token) and dK/dV/dKeyRope rows of sampled key rows, including the
most-selected one (each is the sum over the pairs that select it, and the
saved statistics make every pair independent of the rest of its token's row).
Inputs are generated on the GPU; the softmax statistics are the generator's
stand-ins, which the backward pass takes as given.  Rows that no valid
position selects must be exactly 0 everywhere.
"""
import numpy as np
import pytest
import torch

import sfag_inputs as si
from oracle import sfag_oracle as orc
from tests._helpers import call_backward, geom_of, rel_l2

pytestmark = pytest.mark.gpu

TOL = dict(dq=5e-3, dqr=5e-3, dk=1e-2, dv=1e-2, dkr=1e-2)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_size_sampled(cfg):
    case = si.CONFIGS[cfg]
    seed = si.seed_for(cfg)
    print(f"full-size {case.name} seed {seed}", flush=True)
    inp = si.make_inputs(case, seed, device="cuda")
    inp.update(si.standin_stats(case, inp, seed, device="cuda"))
    outs = call_backward(case, inp)
    torch.cuda.synchronize()
    dq, dk, dv, dqr, dkr = outs
    idx = inp["sparse_indices"].reshape(case.T1, case.Kent).cpu()
    m = inp["softmax_max"].reshape(case.T1, case.G)
    l = inp["softmax_sum"].reshape(case.T1, case.G)
    geom = geom_of(case)
    rows = orc.decode(idx, case.block, case.mode, geom)
    counts = np.bincount(rows[rows >= 0], minlength=case.T2)
    rng = np.random.default_rng(seed)
    tokens = np.unique(np.concatenate([[0, case.T1 - 1, case.T1 // 2], rng.choice(case.T1, 3, replace=False)]))
    live_keys = np.nonzero(counts)[0]
    keys = np.unique(np.concatenate([[int(np.argmax(counts))], rng.choice(live_keys, 3, replace=False)]))
    print(f"tokens {tokens.tolist()} keys {keys.tolist()} (max hits {counts.max()})", flush=True)
    ref = orc.backward_rows(inp["query"].reshape(case.T1, case.G, case.D),
                            inp["key"].reshape(case.T2, case.D), inp["value"].reshape(case.T2, case.D),
                            inp["query_rope"].reshape(case.T1, case.G, case.Dr) if case.Dr else None,
                            inp["key_rope"].reshape(case.T2, case.Dr) if case.Dr else None,
                            idx, inp["dout"].reshape(case.T1, case.G, case.D),
                            inp["out"].reshape(case.T1, case.G, case.D), m, l, geom, case.block,
                            case.mode, case.scale_value, tokens=tokens, keys=keys, rows=rows)
    T = torch.as_tensor(tokens, device="cuda")
    Kt = torch.as_tensor(keys, device="cuda")
    got = dict(dq=dq.reshape(case.T1, case.G, case.D)[T], dk=dk.reshape(case.T2, case.D)[Kt],
               dv=dv.reshape(case.T2, case.D)[Kt])
    if case.Dr:
        got["dqr"] = dqr.reshape(case.T1, case.G, case.Dr)[T]
        got["dkr"] = dkr.reshape(case.T2, case.Dr)[Kt]
    errs = {}
    for n, x in got.items():
        x = x.float().cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(x)), n
        errs[n] = rel_l2(x, ref[n])
    print(case.name, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for n, e in errs.items():
        assert e <= TOL[n], (n, e)
    never = torch.as_tensor(counts == 0, device="cuda")
    for x, w in ((dk, case.D), (dv, case.D), (dkr, case.Dr)):
        if x is not None:
            assert torch.all(x.reshape(case.T2, w)[never] == 0)
