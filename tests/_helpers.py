"""Test plumbing: reshape generator outputs for the oracle and make forward
statistics with the oracle's forward pass."""
import numpy as np
import torch

import sfag_inputs as si
from oracle import sfag_oracle as orc


def geom_of(case):
    if case.layout == "BSND":
        return orc.geometry("BSND", case.B, case.S1, case.S2)
    return orc.geometry("TND", case.B, seqlens_q=case.seqlens_q, seqlens_kv=case.seqlens_kv)


def flat(case, inp):
    """CPU tensor views in the oracle's (T1,G,D)/(T2,D) shapes."""
    T1, T2, G = case.T1, case.T2, case.G
    c = lambda x: x.detach().cpu()
    f = dict(
        q=c(inp["query"]).reshape(T1, G, case.D),
        k=c(inp["key"]).reshape(T2, case.D),
        v=c(inp["value"]).reshape(T2, case.D),
        dO=c(inp["dout"]).reshape(T1, G, case.D),
        idx=c(inp["sparse_indices"]).reshape(T1, case.Kent),
        qr=c(inp["query_rope"]).reshape(T1, G, case.Dr) if case.Dr else None,
        kr=c(inp["key_rope"]).reshape(T2, case.Dr) if case.Dr else None,
    )
    if "out" in inp:
        f["O"] = c(inp["out"]).reshape(T1, G, case.D)
        f["m"] = c(inp["softmax_max"]).reshape(T1, G)
        f["l"] = c(inp["softmax_sum"]).reshape(T1, G)
    return f


def add_oracle_stats(case, inp):
    """out / softmaxMax / softmaxSum from the oracle forward: O rounded to the
    input dtype (RNE), max and sum rounded to float32."""
    f = flat(case, inp)
    O, M, L = orc.forward(f["q"], f["k"], f["v"], f["qr"], f["kr"], f["idx"], geom_of(case),
                          case.block, case.mode, case.scale_value)
    dev = inp["query"].device
    inp = dict(inp)
    inp["out"] = torch.from_numpy(O).to(si.DTYPES[case.dtype]).reshape(si.out_shape(case)).to(dev)
    inp["softmax_max"] = torch.from_numpy(M.astype(np.float32)).reshape(si.stats_shape(case)).to(dev)
    inp["softmax_sum"] = torch.from_numpy(L.astype(np.float32)).reshape(si.stats_shape(case)).to(dev)
    return inp


def oracle_backward(case, inp):
    f = flat(case, inp)
    return orc.backward(f["q"], f["k"], f["v"], f["qr"], f["kr"], f["idx"], f["dO"], f["O"], f["m"],
                        f["l"], geom_of(case), case.block, case.mode, case.scale_value)


def rel_l2(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    if den == 0:
        return 0.0 if num == 0 else float("inf")
    return float(num / den)


def call_backward(case, inp, **kw):
    """Run the library on generator inputs (all tensors on the GPU)."""
    import top_sparse_attention_sfag_amd as sfag
    return sfag.backward(
        inp["query"], inp["key"], inp["value"], inp["sparse_indices"], inp["dout"], inp["out"],
        inp["softmax_max"], inp["softmax_sum"], seqlens_q=inp.get("seqlens_q"), seqlens_kv=inp.get("seqlens_kv"),
        query_rope=inp.get("query_rope"), key_rope=inp.get("key_rope"), scale=case.scale_value,
        block_size=case.block, layout=case.layout, sparse_mode=case.mode,
        deterministic=kw.pop("deterministic", case.deterministic), **kw)


def to_device(inp, device="cuda"):
    return {k: v.to(device) for k, v in inp.items()}
