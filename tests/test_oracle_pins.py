"""Pins of the CPU oracle against facts that do not come from the oracle itself.

* central finite differences of L = <dO, O(Q,K,V,Qr,Kr)> (the backward pass is
  the gradient of the forward pass, 功能说明 stages 1-3);
* equality with dense attention backward (torch autograd, float64) when the
  indices select every key, for sparseMode 0 and for the bottom-right causal
  sparseMode 3 (Mask table) with S1 != S2;
* softmax-gradient invariants (rows of dS sum to zero, Σ_p dK[p] = 0,
  Σ_p dV[p] = Σ dO over live rows) and the one-key closed form;
* structural equalities: block entries == expanded positions, -1 padding ==
  removal, TND == per-sequence BSND, duplicated indices == repeated keys;
* the usage example of the operator page, whose constant inputs give a closed
  form (dP equals Delta, so dQ = dK = 0).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import sfag_oracle as orc

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _problem(seed, layout="BSND", B=1, S1=3, S2=8, G=2, D=8, Dr=4, Kent=5, block=1, mode=0,
             seqlens=None, neg_frac=0.2, dup=False):
    rng = np.random.default_rng(seed)
    if layout == "BSND":
        geom = orc.geometry("BSND", B, S1, S2)
    else:
        geom = orc.geometry("TND", len(seqlens[0]), seqlens_q=seqlens[0], seqlens_kv=seqlens[1])
    T1, T2 = geom["T1"], geom["T2"]
    q = rng.standard_normal((T1, G, D))
    k = rng.standard_normal((T2, D))
    v = rng.standard_normal((T2, D))
    qr = rng.standard_normal((T1, G, Dr)) if Dr else None
    kr = rng.standard_normal((T2, Dr)) if Dr else None
    dO = rng.standard_normal((T1, G, D))
    idx = np.zeros((T1, Kent), np.int64)
    for t in range(T1):
        Lk = int(geom["Lk"][t])
        nb = max(1, Lk // block) if block > 1 else Lk
        if block > 1:
            starts = rng.permutation(nb)[:Kent] * block
        else:
            starts = rng.choice(Lk, size=Kent, replace=dup or Kent > Lk)
        row = np.full(Kent, -1)
        row[: len(starts)] = starts
        drop = rng.random(Kent) < neg_frac
        row[drop] = -1
        idx[t] = row
    return dict(q=q, k=k, v=v, qr=qr, kr=kr, dO=dO, idx=idx, geom=geom, block=block, mode=mode)


def _loss(p, scale):
    O, _, _ = orc.forward(p["q"], p["k"], p["v"], p["qr"], p["kr"], p["idx"], p["geom"], p["block"],
                          p["mode"], scale)
    return float((p["dO"] * O).sum())


def _grads(p, scale):
    O, M, L = orc.forward(p["q"], p["k"], p["v"], p["qr"], p["kr"], p["idx"], p["geom"], p["block"],
                          p["mode"], scale)
    return orc.backward(p["q"], p["k"], p["v"], p["qr"], p["kr"], p["idx"], p["dO"], O, M, L,
                        p["geom"], p["block"], p["mode"], scale)


FD_CASES = [
    dict(seed=1),
    dict(seed=2, mode=3, S1=3, S2=8),
    dict(seed=3, mode=3, S1=6, S2=4, Kent=4),
    dict(seed=4, block=2, Kent=3, S2=9),
    dict(seed=5, block=2, Kent=3, S2=8, mode=3, S1=5),
    dict(seed=6, Dr=0),
    dict(seed=7, layout="TND", seqlens=((2, 3), (5, 4)), mode=3, Kent=4),
    dict(seed=8, dup=True, Kent=6, neg_frac=0.0),
]


@pytest.mark.parametrize("kw", FD_CASES, ids=[str(i) for i in range(len(FD_CASES))])
def test_finite_differences(kw):
    p = _problem(**kw)
    scale = 0.37
    g = _grads(p, scale)
    names = [("q", "dq"), ("k", "dk"), ("v", "dv")]
    if p["qr"] is not None:
        names += [("qr", "dqr"), ("kr", "dkr")]
    h = 1e-5
    for x, gx in names:
        X = p[x]
        fd = np.zeros_like(X)
        it = np.nditer(X, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = X[i]
            X[i] = old + h
            lp = _loss(p, scale)
            X[i] = old - h
            lm = _loss(p, scale)
            X[i] = old
            fd[i] = (lp - lm) / (2 * h)
        err = np.abs(fd - g[gx]).max()
        assert err <= 1e-7 * max(1.0, np.abs(fd).max()), (x, err)


def _dense_reference(q, k, v, qr, kr, dO, scale, mask):
    """Dense masked attention over one sequence (torch float64 autograd)."""
    sc = float(np.float32(scale))
    tq, tk, tv, tdO = (torch.tensor(a, requires_grad=True) for a in (q, k, v, dO))
    logits = torch.einsum("shd,pd->shp", tq, tk)
    if qr is not None:
        tqr, tkr = torch.tensor(qr, requires_grad=True), torch.tensor(kr, requires_grad=True)
        logits = logits + torch.einsum("shr,pr->shp", tqr, tkr)
    z = sc * logits
    m = torch.tensor(mask)[:, None, :]
    live = m.any(-1)                                         # (S, 1)
    z = z.masked_fill(~m, float("-inf"))
    zmax = torch.where(live, z.amax(-1), torch.zeros(()))
    e = torch.exp(z - zmax[..., None]).masked_fill(~m, 0.0)
    ssum = e.sum(-1)
    P = e / torch.where(live, ssum, torch.ones(()))[..., None]
    O = torch.einsum("shp,pd->shd", P, tv)
    (tdO * O).sum().backward()
    out = dict(O=O.detach().numpy(), m=torch.where(live, zmax, torch.full_like(zmax, -math.inf)).detach().numpy(),
               l=ssum.detach().numpy(), dq=tq.grad.numpy(), dk=tk.grad.numpy(), dv=tv.grad.numpy())
    if qr is not None:
        out["dqr"], out["dkr"] = tqr.grad.numpy(), tkr.grad.numpy()
    return out


@pytest.mark.parametrize("mode,S1,S2", [(0, 5, 7), (3, 5, 9), (3, 9, 5), (3, 6, 6)])
def test_dense_equivalence(mode, S1, S2):
    rng = np.random.default_rng(11 + mode + S1)
    G, D, Dr = 3, 6, 2
    geom = orc.geometry("BSND", 1, S1, S2)
    q = rng.standard_normal((S1, G, D))
    qr = rng.standard_normal((S1, G, Dr))
    k = rng.standard_normal((S2, D))
    kr = rng.standard_normal((S2, Dr))
    v = rng.standard_normal((S2, D))
    dO = rng.standard_normal((S1, G, D))
    idx = np.stack([rng.permutation(S2) for _ in range(S1)])      # every key, random order
    t = np.arange(S1)[:, None]
    p = np.arange(S2)[None, :]
    mask = np.ones((S1, S2), bool) if mode == 0 else (p <= t + S2 - S1)
    ref = _dense_reference(q, k, v, qr, kr, dO, 0.29, mask)
    O, M, L = orc.forward(q, k, v, qr, kr, idx, geom, 1, mode, 0.29)
    live = mask.any(1)
    np.testing.assert_allclose(O[live], ref["O"][live], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(M[live], ref["m"][live], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L[live], ref["l"][live], rtol=1e-12, atol=1e-12)
    assert np.all(L[~live] == 0) and np.all(O[~live] == 0)
    g = orc.backward(q, k, v, qr, kr, idx, dO, O, M, L, geom, 1, mode, 0.29)
    for name in ("dq", "dk", "dv", "dqr", "dkr"):
        np.testing.assert_allclose(g[name], ref[name], rtol=1e-10, atol=1e-11, err_msg=name)


def test_softmax_gradient_invariants():
    p = _problem(21, S1=4, S2=10, G=3, D=6, Dr=2, Kent=6, neg_frac=0.3)
    scale = 0.41
    O, M, L = orc.forward(p["q"], p["k"], p["v"], p["qr"], p["kr"], p["idx"], p["geom"], 1, 0, scale)
    rows = orc.decode(p["idx"], 1, 0, p["geom"])
    sc = orc.scale32(scale)
    for t in range(rows.shape[0]):
        sel = rows[t][rows[t] >= 0]
        if sel.size == 0:
            continue
        P, dP, delta, dS = orc.token_terms(p["q"][t], p["qr"][t], p["dO"][t], O[t], M[t], L[t],
                                           p["k"][sel], p["kr"][sel], p["v"][sel], sc)
        np.testing.assert_allclose(P.sum(1), 1.0, rtol=0, atol=1e-13)
        np.testing.assert_allclose(dS.sum(1), 0.0, rtol=0, atol=1e-12)
    g = orc.backward(p["q"], p["k"], p["v"], p["qr"], p["kr"], p["idx"], p["dO"], O, M, L, p["geom"], 1, 0, scale)
    np.testing.assert_allclose(g["dk"].sum(0), 0.0, atol=1e-12)
    np.testing.assert_allclose(g["dkr"].sum(0), 0.0, atol=1e-12)
    live = (rows >= 0).any(1)
    np.testing.assert_allclose(g["dv"].sum(0), p["dO"][live].sum((0, 1)), rtol=1e-12, atol=1e-12)
    # With O rounded (as the operator stores it), the dV column sum still holds.
    Or = O.astype(np.float32).astype(np.float64)
    g2 = orc.backward(p["q"], p["k"], p["v"], p["qr"], p["kr"], p["idx"], p["dO"], Or, M, L, p["geom"], 1, 0, scale)
    np.testing.assert_allclose(g2["dv"].sum(0), p["dO"][live].sum((0, 1)), rtol=1e-12, atol=1e-12)


def test_one_key_closed_form():
    """One valid key per row: P = 1 and O = v, so dS = 0 (dQ = dK = 0) and dV[p]
    is the sum of dO over every (token, head) selecting p."""
    rng = np.random.default_rng(5)
    S1, S2, G, D = 6, 4, 3, 5
    geom = orc.geometry("BSND", 1, S1, S2)
    q, dO = rng.standard_normal((S1, G, D)), rng.standard_normal((S1, G, D))
    k, v = rng.standard_normal((S2, D)), rng.standard_normal((S2, D))
    idx = np.full((S1, 3), -1)
    idx[:, 1] = rng.integers(0, S2, S1)
    O, M, L = orc.forward(q, k, v, None, None, idx, geom, 1, 0, 0.5)
    np.testing.assert_array_equal(L, 1.0)
    g = orc.backward(q, k, v, None, None, idx, dO, O, M, L, geom, 1, 0, 0.5)
    # dP and Delta are equal up to summation order, so dS vanishes to rounding.
    np.testing.assert_allclose(g["dq"], 0.0, atol=1e-14)
    np.testing.assert_allclose(g["dk"], 0.0, atol=1e-14)
    want = np.zeros((S2, D))
    for t in range(S1):
        want[idx[t, 1]] += dO[t].sum(0)
    np.testing.assert_allclose(g["dv"], want, rtol=1e-14, atol=1e-14)


def test_block_equals_expanded():
    rng = np.random.default_rng(9)
    S1, S2, G, D, Dr, bs = 5, 16, 2, 4, 2, 4
    for mode in (0, 3):
        geom = orc.geometry("BSND", 1, S1, S2)
        q, qr = rng.standard_normal((S1, G, D)), rng.standard_normal((S1, G, Dr))
        k, kr, v = rng.standard_normal((S2, D)), rng.standard_normal((S2, Dr)), rng.standard_normal((S2, D))
        dO = rng.standard_normal((S1, G, D))
        starts = np.stack([rng.permutation(S2 // bs)[:3] * bs for _ in range(S1)])
        starts[1, 2] = -1
        expanded = np.where(starts[:, :, None] >= 0, starts[:, :, None] + np.arange(bs), -1).reshape(S1, -1)
        a = orc.forward(q, k, v, qr, kr, starts, geom, bs, mode, 0.3)
        b = orc.forward(q, k, v, qr, kr, expanded, geom, 1, mode, 0.3)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)
        ga = orc.backward(q, k, v, qr, kr, starts, dO, *a, geom, bs, mode, 0.3)
        gb = orc.backward(q, k, v, qr, kr, expanded, dO, *a, geom, 1, mode, 0.3)
        for n in ga:
            np.testing.assert_array_equal(ga[n], gb[n])
        np.testing.assert_array_equal(orc.decode(starts, bs, mode, geom), orc.decode(expanded, 1, mode, geom))


def test_padding_equals_removal():
    p = _problem(31, S1=4, S2=12, Kent=8, neg_frac=0.0)
    O, M, L = orc.forward(p["q"], p["k"], p["v"], p["qr"], p["kr"], p["idx"], p["geom"], 1, 0, 0.3)
    g = orc.backward(p["q"], p["k"], p["v"], p["qr"], p["kr"], p["idx"], p["dO"], O, M, L, p["geom"], 1, 0, 0.3)
    rng = np.random.default_rng(3)
    padded = np.full((p["idx"].shape[0], 13), -1)
    for t in range(padded.shape[0]):
        slots = np.sort(rng.choice(13, 8, replace=False))
        padded[t, slots] = p["idx"][t]
    O2, M2, L2 = orc.forward(p["q"], p["k"], p["v"], p["qr"], p["kr"], padded, p["geom"], 1, 0, 0.3)
    g2 = orc.backward(p["q"], p["k"], p["v"], p["qr"], p["kr"], padded, p["dO"], O2, M2, L2, p["geom"], 1, 0, 0.3)
    for x, y in zip((O, M, L), (O2, M2, L2)):
        np.testing.assert_array_equal(x, y)
    for n in g:
        np.testing.assert_array_equal(g[n], g2[n])


def test_tnd_equals_bsnd_per_sequence():
    rng = np.random.default_rng(13)
    lq, lk = (3, 0, 4), (5, 2, 6)
    G, D, Dr, Kent = 2, 4, 2, 4
    geom = orc.geometry("TND", 3, seqlens_q=lq, seqlens_kv=lk)
    T1, T2 = sum(lq), sum(lk)
    q, qr, dO = rng.standard_normal((T1, G, D)), rng.standard_normal((T1, G, Dr)), rng.standard_normal((T1, G, D))
    k, kr, v = rng.standard_normal((T2, D)), rng.standard_normal((T2, Dr)), rng.standard_normal((T2, D))
    idx = np.full((T1, Kent), -1)
    qs = 0
    for b in range(3):
        for t in range(lq[b]):
            n = min(Kent, lk[b])
            idx[qs + t, :n] = rng.permutation(lk[b])[:n]
        qs += lq[b]
    O, M, L = orc.forward(q, k, v, qr, kr, idx, geom, 1, 3, 0.3)
    g = orc.backward(q, k, v, qr, kr, idx, dO, O, M, L, geom, 1, 3, 0.3)
    qs = ks = 0
    for b in range(3):
        if lq[b]:
            gb = orc.geometry("BSND", 1, lq[b], lk[b])
            sl, kl = slice(qs, qs + lq[b]), slice(ks, ks + lk[b])
            Ob, Mb, Lb = orc.forward(q[sl], k[kl], v[kl], qr[sl], kr[kl], idx[sl], gb, 1, 3, 0.3)
            np.testing.assert_array_equal(Ob, O[sl])
            gg = orc.backward(q[sl], k[kl], v[kl], qr[sl], kr[kl], idx[sl], dO[sl], Ob, Mb, Lb, gb, 1, 3, 0.3)
            for n, s in (("dq", sl), ("dqr", sl), ("dk", kl), ("dv", kl), ("dkr", kl)):
                np.testing.assert_allclose(g[n][s], gg[n], rtol=0, atol=1e-14)
        qs += lq[b]
        ks += lk[b]


def test_duplicates_equal_repeated_keys():
    """A row naming key j twice behaves as attention over a key list holding
    row j twice (torch autograd through the gather sums both uses)."""
    rng = np.random.default_rng(17)
    S1, S2, G, D = 2, 6, 2, 4
    geom = orc.geometry("BSND", 1, S1, S2)
    q, dO = rng.standard_normal((S1, G, D)), rng.standard_normal((S1, G, D))
    k, v = rng.standard_normal((S2, D)), rng.standard_normal((S2, D))
    idx = np.array([[1, 4, 1, 0], [5, 5, 5, 2]])
    O, M, L = orc.forward(q, k, v, None, None, idx, geom, 1, 0, 0.5)
    g = orc.backward(q, k, v, None, None, idx, dO, O, M, L, geom, 1, 0, 0.5)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    loss = 0
    for t in range(S1):
        sel = torch.tensor(idx[t])
        z = float(np.float32(0.5)) * (tq[t] @ tk[sel].T)
        loss = loss + (torch.tensor(dO[t]) * (torch.softmax(z, -1) @ tv[sel])).sum()
    loss.backward()
    np.testing.assert_allclose(g["dq"], tq.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g["dk"], tk.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g["dv"], tv.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_operator_page_example_closed_form():
    """The usage example of the operator page: TND, one query token, N1=16,
    D=512, Dr=64, T2=2048, indices 0..2047, softmaxMax = softmaxSum = 3.0,
    scale 0.088388, every data element the same constant c.  Then dP = Delta
    exactly (both are 512*c*c), so dS = 0: dQ = dK = dQr = dKr = 0 and every
    dV element equals 16 * exp(sc*576*c*c - 3) / 3 * c."""
    with open(os.path.join(GOLD, "operator_page_example.json")) as f:
        fx = json.load(f)
    geom = orc.geometry("TND", 1, seqlens_q=fx["actual_seq_q"], seqlens_kv=fx["actual_seq_kv"])
    G, D, Dr, T2 = fx["N1"], fx["D"], fx["Dr"], fx["T2"]
    for c in fx["constants"]:
        q = np.full((1, G, D), c)
        qr = np.full((1, G, Dr), c)
        k = np.full((T2, D), c)
        kr = np.full((T2, Dr), c)
        idx = np.arange(fx["K"])[None, :]
        m = np.full((1, G), fx["softmax_max"])
        l = np.full((1, G), fx["softmax_sum"])
        g = orc.backward(q, k, k.copy(), qr, kr, idx, q.copy(), q.copy(), m, l, geom, 1, 0, fx["scale"])
        assert np.all(g["dq"] == 0) and np.all(g["dk"] == 0)
        assert np.all(g["dqr"] == 0) and np.all(g["dkr"] == 0)
        sc = float(np.float32(fx["scale"]))
        want = G * math.exp(sc * (D + Dr) * c * c - fx["softmax_max"]) / fx["softmax_sum"] * c
        np.testing.assert_allclose(g["dv"], want, rtol=1e-13)


def test_csr_golden():
    with open(os.path.join(GOLD, "csr_small.json")) as f:
        fx = json.load(f)
    geom = orc.geometry("BSND", 1, fx["S1"], fx["S2"])
    rows = orc.decode(np.array(fx["indices"]), fx["block"], fx["mode"], geom)
    np.testing.assert_array_equal(rows, np.array(fx["rows"]))
    off, pairs = orc.csr(rows, fx["S2"])
    np.testing.assert_array_equal(off, fx["offsets"])
    np.testing.assert_array_equal(pairs, fx["pairs"])


def test_csr_properties():
    p = _problem(41, S1=7, S2=9, Kent=6, mode=3, neg_frac=0.3, dup=True)
    rows = orc.decode(p["idx"], 1, 3, p["geom"])
    off, pairs = orc.csr(rows, 9)
    flat = rows.reshape(-1)
    keys = flat[flat >= 0]
    assert off[-1] == keys.size
    for key in range(9):
        seg = pairs[off[key]:off[key + 1]]
        assert np.all(keys[seg] == key)
        assert np.all(np.diff(seg) > 0)


def test_sampled_rows_equal_full_backward():
    """The one-row-at-a-time evaluation used at full sizes equals the full
    backward pass on the sampled rows (including a duplicated index, rows
    past the causal bound and a token with no valid position)."""
    p = _problem(51, S1=6, S2=12, G=3, D=8, Dr=4, Kent=7, mode=3, neg_frac=0.25, dup=True)
    scale = 0.33
    O, M, L = orc.forward(p["q"], p["k"], p["v"], p["qr"], p["kr"], p["idx"], p["geom"], 1, 3, scale)
    g = orc.backward(p["q"], p["k"], p["v"], p["qr"], p["kr"], p["idx"], p["dO"], O, M, L, p["geom"], 1, 3, scale)
    tokens, keys = [0, 2, 5], [0, 3, 7, 11]
    r = orc.backward_rows(p["q"], p["k"], p["v"], p["qr"], p["kr"], p["idx"], p["dO"], O, M, L, p["geom"], 1, 3,
                          scale, tokens=tokens, keys=keys, batch=2)
    np.testing.assert_allclose(r["dq"], g["dq"][tokens], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["dqr"], g["dqr"][tokens], rtol=1e-12, atol=1e-13)
    for n in ("dk", "dv", "dkr"):
        np.testing.assert_allclose(r[n], g[n][keys], rtol=1e-12, atol=1e-13, err_msg=n)
    # token-subset backward: the same rows and the same per-key sums
    sub = orc.backward(p["q"], p["k"], p["v"], p["qr"], p["kr"], p["idx"], p["dO"], O, M, L, p["geom"], 1, 3, scale,
                       tokens=[1, 4])
    rest = orc.backward(p["q"], p["k"], p["v"], p["qr"], p["kr"], p["idx"], p["dO"], O, M, L, p["geom"], 1, 3, scale,
                        tokens=[0, 2, 3, 5])
    for n in ("dk", "dv", "dkr"):
        np.testing.assert_allclose(sub[n] + rest[n], g[n], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("S1,S2,pre,nxt,block", [(6, 6, 2, 1, 1), (5, 9, 3, 0, 1), (9, 5, 10**9, 0, 1),
                                                  (7, 7, 10**9, 10**9, 1), (6, 20, 4, 2, 4), (8, 8, 0, 0, 1)])
def test_band_equals_dense_band_mask(S1, S2, pre, nxt, block):
    """band_indices (sliding window from the FlashAttention backward page's
    block-band test, bottom-right aligned) through the sparse backward equals
    dense attention under the band mask written as a 2-D comparison: key p is
    live for query t iff its block holds a position within [d - pre, d + nxt]
    (d = t + S2 - S1) inside [0, S2)."""
    rng = np.random.default_rng(S1 * 31 + S2 + block)
    G, D, Dr = 2, 6, 2
    geom = orc.geometry("BSND", 1, S1, S2)
    K = orc.band_entries(S2, pre, nxt, block)
    idx = orc.band_indices(geom, K, pre, nxt, block)
    q, qr = rng.standard_normal((S1, G, D)), rng.standard_normal((S1, G, Dr))
    k, kr, v = rng.standard_normal((S2, D)), rng.standard_normal((S2, Dr)), rng.standard_normal((S2, D))
    dO = rng.standard_normal((S1, G, D))
    t = np.arange(S1)[:, None]
    p = np.arange(S2)[None, :]
    d = t + S2 - S1
    lo, hi = np.maximum(d - pre, 0), np.minimum(d + nxt, S2 - 1)
    mask = (lo <= hi) & (p // block >= lo // block) & (p // block <= hi // block)
    # every selected block lies inside the key range here, so positions are never cut
    ref = _dense_reference(q, k, v, qr, kr, dO, 0.31, mask)
    O, M, L = orc.forward(q, k, v, qr, kr, idx, geom, block, 0, 0.31)
    live = mask.any(1)
    np.testing.assert_allclose(O[live], ref["O"][live], rtol=1e-12, atol=1e-12)
    g = orc.backward(q, k, v, qr, kr, idx, dO, O, M, L, geom, block, 0, 0.31)
    for name in ("dq", "dk", "dv", "dqr", "dkr"):
        np.testing.assert_allclose(g[name], ref[name], rtol=1e-10, atol=1e-11, err_msg=name)


def test_band_special_cases_and_entry_count():
    """Unbounded band = every key in order; pre unbounded, next 0 = the
    sparseMode 3 causal set; band_entries is the largest row any alignment
    of the window needs (brute force over key lengths and offsets)."""
    geom = orc.geometry("TND", 3, seqlens_q=(4, 0, 6), seqlens_kv=(9, 3, 6))
    big = 10**9
    rows = orc.band_indices(geom, 9, big, big, 1)
    for t in range(geom["T1"]):
        Lk = int(geom["Lk"][t])
        np.testing.assert_array_equal(rows[t, :Lk], np.arange(Lk))
        assert np.all(rows[t, Lk:] == -1)
    causal = orc.band_indices(geom, 9, big, 0, 1)
    dec_band = orc.decode(causal, 1, 0, geom)
    dec_mode3 = orc.decode(np.tile(np.arange(9), (geom["T1"], 1)), 1, 3, geom)
    np.testing.assert_array_equal(dec_band, dec_mode3)
    for Lk in (1, 5, 16, 33):
        for pre in (0, 1, 3, 7, 20):
            for nxt in (0, 2, 5):
                for block in (1, 2, 4, 8):
                    g = orc.geometry("BSND", 1, Lk, Lk)
                    full = orc.band_indices(g, Lk, pre, nxt, block)
                    need = int((full >= 0).sum(1).max())
                    got = orc.band_entries(Lk, pre, nxt, block)
                    # the formula bounds every alignment; equality holds whenever the
                    # worst alignment occurs among the Lk diagonals
                    assert need <= got <= need + 1, (Lk, pre, nxt, block, need, got)


def test_flop_count():
    """oracle.flops: 2 flop per multiply-add of the five contractions per valid
    (head, position) pair, masked positions not counted.  Pinned by (a) the
    per-pair figures the workload definition states (5504 with D = 512 and
    Dr = 64, 5120 without rope) on a hand-counted row set, and (b) a scalar
    loop that performs S = q·k, dP = dO·v, dQ += dS·k, dK += dS·q, dV += P·dO
    for every valid pair and head of a tiny problem and counts its
    multiplications."""
    rows = np.array([[0, -1, 2, 5], [-1, -1, -1, -1], [7, 7, -1, 3]])   # 6 valid positions
    assert orc.flops(rows, 3, 512, 64) == 6 * 3 * 5504
    assert orc.flops(rows, 3, 512, 0) == 6 * 3 * 5120
    assert orc.flops(np.full((2, 3), -1), 128, 512, 64) == 0

    rng = np.random.default_rng(0)
    for G, D, Dr in ((2, 3, 2), (1, 4, 0), (3, 2, 1)):
        muls = 0
        for t in range(rows.shape[0]):
            for p in rows[t][rows[t] >= 0]:
                kq = rng.standard_normal(D + Dr)
                v = rng.standard_normal(D)
                for h in range(G):
                    q = rng.standard_normal(D + Dr)
                    dO = rng.standard_normal(D)
                    s = 0.0
                    for c in range(D + Dr):          # S over D + Dr
                        s += q[c] * kq[c]
                        muls += 1
                    dp = 0.0
                    for c in range(D):               # dP over D
                        dp += dO[c] * v[c]
                        muls += 1
                    ds, P = s * dp, s
                    for c in range(D + Dr):          # dQ and dK over D + Dr
                        _ = ds * kq[c]
                        _ = ds * q[c]
                        muls += 2
                    for c in range(D):               # dV over D
                        _ = P * dO[c]
                        muls += 1
        assert orc.flops(rows, G, D, Dr) == 2 * muls, (G, D, Dr)
