"""The entry point that allocates nothing (sfag_backward_static: the
library's own scratch array as workspace, for callers that cannot allocate)
against the ordinary entry point (sfag_backward with a caller workspace) on
the same plan options: two calls in a row, the second with a smaller input.
Deterministic calls give the same bits; every output is also within the
oracle's tolerance (relative L2: dQ/dQueryRope 5e-3, dK/dV/dKeyRope 1e-2)."""
import ctypes

import numpy as np
import pytest
import torch

import sfag_inputs as si
from tests._helpers import add_oracle_stats, call_backward, oracle_backward, rel_l2, to_device

pytestmark = pytest.mark.gpu

TOL = dict(dq=5e-3, dqr=5e-3, dk=1e-2, dv=1e-2, dkr=1e-2)
CASES = [
    si.Case("noalloc_g64_causal", S1=96, S2=512, G=64, K=200, mode=3, index_rule="causal_mix", deterministic=True),
    si.Case("noalloc_g16_blocks", S1=24, S2=256, G=16, Dr=0, K=6, block=16, dtype="fp16", std=0.5,
            index_rule="blocks", scale=1 / 512 ** 0.5, deterministic=True),
]


def _static_call(case, inp, outs, options):
    """sfag_backward_static through the C ABI."""
    import top_sparse_attention_sfag_amd as sfag
    dq, dk, dv, dqr, dkr = outs
    ws, p = sfag.plan(inp["query"], inp["key"], inp["value"], inp["sparse_indices"], inp["dout"], inp["out"],
                      inp["softmax_max"], inp["softmax_sum"], dq, dk, dv, dq_rope=dqr, dk_rope=dkr,
                      seqlens_q=inp.get("seqlens_q"), seqlens_kv=inp.get("seqlens_kv"),
                      query_rope=inp.get("query_rope"), key_rope=inp.get("key_rope"), scale=case.scale_value,
                      block_size=case.block, layout=case.layout, sparse_mode=case.mode,
                      deterministic=case.deterministic, options=options)
    assert ws <= sfag.STATIC_SCRATCH_BYTES, ws
    rc = sfag.lib().sfag_backward_static(p, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, sfag.lib().sfag_last_error()
    return outs


def test_static_scratch_matches_the_workspace_call():
    import top_sparse_attention_sfag_amd as sfag
    opts = dict(workspace_budget=sfag.STATIC_SCRATCH_BYTES)
    for case in CASES:   # the second input is smaller than the first
        print(f"no-alloc case {case.name}", flush=True)
        inp = add_oracle_stats(case, si.make_inputs(case, 31))
        ref = oracle_backward(case, inp)
        dev = to_device(inp)
        base = call_backward(case, dev, options=opts)
        mk = lambda x: None if x is None else torch.full_like(x, float("nan"))
        outs = _static_call(case, dev, tuple(mk(x) for x in base), opts)
        torch.cuda.synchronize()
        for n, a, b in zip(("dq", "dk", "dv", "dqr", "dkr"), base, outs):
            if a is None:
                continue
            assert torch.equal(a, b), n
            got = b.float().cpu().numpy().astype(np.float64).reshape(ref[n].shape)
            e = rel_l2(got, ref[n])
            print(case.name, n, f"{e:.2e}", flush=True)
            assert e <= TOL[n], (n, e)
