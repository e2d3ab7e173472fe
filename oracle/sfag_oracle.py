"""CPU oracle for the backward pass of top-k sparse flash attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library.

What it computes follows the operator description "aclnnSparseFlashAttentionGrad"
(CANN ops-transformer documentation):

* section 功能说明 (function description): the selected keys and values are
  gathered with the top-k indices in blocks of ``sparseBlockSize`` rows; stage 1
  forms dP = dO·Vᵀ and dV = Pᵀ·dO, stage 2 forms dS = P ∘ (dP − FlashSoftmaxGrad(dO, O))
  with FlashSoftmaxGrad(dO, O) = rowsum(dO ∘ O), stage 3 forms dQ = dS·K and
  dK = dSᵀ·Q, both times the scale (the page's 1/√d, replaced by ``scaleValue``
  as the parameter table recommends);
* parameter table of the GetWorkspaceSize section: softmaxMax / softmaxSum are
  the forward pass's per-(token, head) max and sum, queryRope / keyRope add a
  Dr-wide part to the logits and get their own gradients;
* section 约束说明, Mask table: sparseMode 0 applies no mask, sparseMode 3 is the
  causal mask whose diagonal passes through the bottom-right corner.

The recompute order (S = QKᵀ, subtract the saved max, divide by the saved sum,
Delta as a row sum of dO ∘ O, dS = P ∘ (dP − Delta)) is the one the MindSpore
page "flash_attention_bwd.py" (FlashAttention backward in TIK) uses in its
``compute_Pij``, ``compute_Di`` and ``compute_dSij`` steps.

Readings where the pages are silent or garbled (each is listed with its reason
in the design notes of the repository):

* an index entry i selects the key positions [i, i + blockSize); any negative
  entry selects nothing; positions at or beyond the sequence's key length are
  masked; under sparseMode 3 position p is valid for query position t of a
  sequence iff p <= t + Lk - Lq;
* a token with no valid position has P = 0 (its saved sum is 0);
* duplicated entries count once each (they behave as repeated keys);
* TND lengths are per-sequence counts and indices are local to the sequence.

Arithmetic is float64 on the exactly representable bf16/fp16 input values; the
scale is first rounded to float32 (the parameter table gives it as FLOAT32).
Matrix products and ``np.add.at`` are the only library primitives used.
"""
from __future__ import annotations

import numpy as np

try:  # torch CPU tensors (bf16) are accepted as inputs and converted row by row
    import torch
except Exception:  # pragma: no cover
    torch = None


def _f64(x, sel=None):
    """Rows ``sel`` of ``x`` (numpy array or torch CPU tensor) as float64."""
    if torch is not None and isinstance(x, torch.Tensor):
        y = x if sel is None else x[torch.as_tensor(np.asarray(sel))]
        return y.to(torch.float64).cpu().numpy()
    y = np.asarray(x) if sel is None else np.asarray(x)[sel]
    return np.asarray(y, dtype=np.float64)


def _i64(x):
    if torch is not None and isinstance(x, torch.Tensor):
        return x.to(torch.int64).cpu().numpy()
    return np.asarray(x, dtype=np.int64)


def scale32(scale_value: float) -> float:
    """scaleValue as the FLOAT32 the parameter table names."""
    return float(np.float32(scale_value))


# ---------------------------------------------------------------------------
# Geometry and index decode (parameter table: layouts BSND / TND,
# actualSeqLengths; 功能说明: gather of selectedBlockSize rows per index;
# Mask table: sparseMode 0 / 3).
# ---------------------------------------------------------------------------

def geometry(layout, B, S1=None, S2=None, seqlens_q=None, seqlens_kv=None):
    """Per-token (t_loc, Lq, Lk, kv_base) arrays of length T1.

    BSND: token t = b*S1 + s has t_loc = s, Lq = S1, Lk = S2, kv_base = b*S2.
    TND: sequence b owns tokens [sum(lq[:b]), sum(lq[:b+1])) and key rows
    [sum(lk[:b]), sum(lk[:b+1])); t_loc is the position inside the sequence.
    """
    if layout == "BSND":
        T1 = B * S1
        t = np.arange(T1, dtype=np.int64)
        b = t // S1
        return dict(t_loc=t % S1, Lq=np.full(T1, S1, np.int64), Lk=np.full(T1, S2, np.int64),
                    kv_base=b * S2, T1=T1, T2=B * S2)
    lq = _i64(seqlens_q)
    lk = _i64(seqlens_kv)
    T1, T2 = int(lq.sum()), int(lk.sum())
    t_loc = np.zeros(T1, np.int64)
    Lq = np.zeros(T1, np.int64)
    Lk = np.zeros(T1, np.int64)
    kv_base = np.zeros(T1, np.int64)
    qs = ks = 0
    for b in range(len(lq)):
        n = int(lq[b])
        t_loc[qs:qs + n] = np.arange(n)
        Lq[qs:qs + n] = n
        Lk[qs:qs + n] = lk[b]
        kv_base[qs:qs + n] = ks
        qs += n
        ks += int(lk[b])
    return dict(t_loc=t_loc, Lq=Lq, Lk=Lk, kv_base=kv_base, T1=T1, T2=T2)


def decode(idx, block: int, mode: int, geom, tokens=None) -> np.ndarray:
    """Selected global key rows, (n_tokens, Kent*block) int64, -1 where masked.

    Entry j of token t selects positions p = idx[t, j] + r for r < block, in
    that order (position e = j*block + r).  p is valid iff idx[t, j] >= 0,
    p < Lk, and, for sparseMode 3, p <= t_loc + Lk - Lq.
    """
    idx = _i64(idx)
    if tokens is None:
        tokens = np.arange(idx.shape[0])
    tokens = np.asarray(tokens, dtype=np.int64)
    ent = idx[tokens]                                   # (n, Kent)
    r = np.arange(block, dtype=np.int64)
    p = ent[:, :, None] + r[None, None, :]              # (n, Kent, block)
    Lk = geom["Lk"][tokens][:, None, None]
    valid = (ent[:, :, None] >= 0) & (p < Lk)
    if mode == 3:
        bound = (geom["t_loc"] + geom["Lk"] - geom["Lq"])[tokens][:, None, None]
        valid &= p <= bound
    rows = np.where(valid, p + geom["kv_base"][tokens][:, None, None], -1)
    return rows.reshape(len(tokens), -1)


# ---------------------------------------------------------------------------
# Per-token terms (功能说明 stages 1-3; MindSpore compute_Pij / compute_Di /
# compute_dSij).
# ---------------------------------------------------------------------------

def _logits(qt, qrt, Ks, Krs):
    s = qt @ Ks.T
    if qrt is not None:
        s = s + qrt @ Krs.T
    return s


def token_terms(qt, qrt, dOt, Ot, mt, lt, Ks, Krs, Vs, sc):
    """P, dP, Delta and dS of one token (heads x selected positions).

    P = exp(sc*S - max) / sum with the given per-head max and sum (0 where the
    sum is 0), Delta = rowsum(dO ∘ O), dP = dO·Vᵀ, dS = P ∘ (dP - Delta).
    """
    S = _logits(qt, qrt, Ks, Krs)
    live = (lt > 0)[:, None]
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        P = np.where(live, np.exp(sc * S - mt[:, None]) / np.where(live, lt[:, None], 1.0), 0.0)
    delta = (dOt * Ot).sum(axis=1)
    dP = dOt @ Vs.T
    dS = P * (dP - delta[:, None])
    return P, dP, delta, dS


def forward(q, k, v, qr, kr, idx, geom, block, mode, scale_value, tokens=None):
    """Forward pass over the selected keys (used only to make consistent inputs).

    Returns O (n, G, D), max (n, G) and sum (n, G) in float64 for ``tokens``:
    max = max over valid positions of sc*S, sum = Σ exp(sc*S - max),
    O = Σ (exp(sc*S - max)/sum)·V.  A token with no valid position gets
    max = -inf, sum = 0, O = 0.
    """
    sc = scale32(scale_value)
    T1 = geom["T1"]
    if tokens is None:
        tokens = np.arange(T1)
    tokens = np.asarray(tokens, dtype=np.int64)
    rows = decode(idx, block, mode, geom, tokens)
    G, D = q.shape[1], v.shape[1]
    O = np.zeros((len(tokens), G, D))
    M = np.full((len(tokens), G), -np.inf)
    L = np.zeros((len(tokens), G))
    for i, t in enumerate(tokens):
        sel = rows[i][rows[i] >= 0]
        if sel.size == 0:
            continue
        Ks, Vs = _f64(k, sel), _f64(v, sel)
        Krs = _f64(kr, sel) if qr is not None else None
        qt = _f64(q, [t])[0]
        qrt = _f64(qr, [t])[0] if qr is not None else None
        z = sc * _logits(qt, qrt, Ks, Krs)
        m = z.max(axis=1)
        e = np.exp(z - m[:, None])
        l = e.sum(axis=1)
        M[i], L[i] = m, l
        O[i] = (e / l[:, None]) @ Vs
    return O, M, L


def backward(q, k, v, qr, kr, idx, dO, O, smax, ssum, geom, block, mode, scale_value, tokens=None):
    """Full backward pass.  Shapes: q/dO/O (T1, G, D), qr (T1, G, Dr) or None,
    k/v (T2, D), kr (T2, Dr) or None, idx (T1, Kent), smax/ssum (T1, G).

    Returns float64 dq (T1,G,D), dk (T2,D), dv (T2,D), dqr, dkr (None without
    rope).  dK and dV rows are accumulated over every (token, position) that
    selects them (np.add.at, so duplicates add up); rows never selected stay 0.
    ``tokens`` restricts the pass to those query tokens (their dQ rows and
    their contributions to dK/dV); by default every token.
    """
    sc = scale32(scale_value)
    T1, T2 = geom["T1"], geom["T2"]
    G, D = q.shape[1], k.shape[1]
    rope = qr is not None
    tokens = np.arange(T1) if tokens is None else np.asarray(tokens, dtype=np.int64)
    rows = decode(idx, block, mode, geom, tokens)
    dq = np.zeros((T1, G, D))
    dk = np.zeros((T2, D))
    dv = np.zeros((T2, v.shape[1]))
    dqr = np.zeros((T1, G, qr.shape[2])) if rope else None
    dkr = np.zeros((T2, kr.shape[1])) if rope else None
    for i, t in enumerate(tokens):
        sel = rows[i][rows[i] >= 0]
        if sel.size == 0:
            continue
        Ks, Vs = _f64(k, sel), _f64(v, sel)
        Krs = _f64(kr, sel) if rope else None
        qt, dOt, Ot = _f64(q, [t])[0], _f64(dO, [t])[0], _f64(O, [t])[0]
        qrt = _f64(qr, [t])[0] if rope else None
        mt, lt = _f64(smax, [t])[0], _f64(ssum, [t])[0]
        P, _dP, _delta, dS = token_terms(qt, qrt, dOt, Ot, mt, lt, Ks, Krs, Vs, sc)
        dq[t] = sc * (dS @ Ks)
        np.add.at(dk, sel, sc * (dS.T @ qt))
        np.add.at(dv, sel, P.T @ dOt)
        if rope:
            dqr[t] = sc * (dS @ Krs)
            np.add.at(dkr, sel, sc * (dS.T @ qrt))
    return dict(dq=dq, dk=dk, dv=dv, dqr=dqr, dkr=dkr)


def backward_rows(q, k, v, qr, kr, idx, dO, O, smax, ssum, geom, block, mode, scale_value,
                  tokens=(), keys=(), rows=None, batch=256):
    """Selected output rows, each computed on its own.

    dQ (and dQueryRope) of a token depends only on that token's inputs and its
    selected keys.  dK / dV (and dKeyRope) of key row p is the sum over every
    (token, position) selecting p of that pair's contribution, which needs only
    that token's q, dO, O, max, sum and the key/value row p itself, since the
    saved statistics stand in for the rest of the row.  ``rows`` may carry a
    precomputed :func:`decode` of all tokens.
    Returns dict of arrays: dq (len(tokens),G,D), dqr, dk (len(keys),D), dv, dkr.
    """
    sc = scale32(scale_value)
    rope = qr is not None
    tokens = np.asarray(tokens, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    if rows is None:
        rows = decode(idx, block, mode, geom)
    G = q.shape[1]
    D = k.shape[1]
    out = dict(dq=np.zeros((len(tokens), G, D)), dk=np.zeros((len(keys), D)),
               dv=np.zeros((len(keys), v.shape[1])),
               dqr=np.zeros((len(tokens), G, qr.shape[2])) if rope else None,
               dkr=np.zeros((len(keys), kr.shape[1])) if rope else None)
    for i, t in enumerate(tokens):
        sel = rows[t][rows[t] >= 0]
        if sel.size == 0:
            continue
        Ks, Vs = _f64(k, sel), _f64(v, sel)
        Krs = _f64(kr, sel) if rope else None
        qt, dOt, Ot = _f64(q, [t])[0], _f64(dO, [t])[0], _f64(O, [t])[0]
        qrt = _f64(qr, [t])[0] if rope else None
        _P, _dP, _d, dS = token_terms(qt, qrt, dOt, Ot, _f64(smax, [t])[0], _f64(ssum, [t])[0],
                                      Ks, Krs, Vs, sc)
        out["dq"][i] = sc * (dS @ Ks)
        if rope:
            out["dqr"][i] = sc * (dS @ Krs)
    for i, p in enumerate(keys):
        tt, _e = np.nonzero(rows == p)                 # every (token, position) selecting p
        kp, vp = _f64(k, [p])[0], _f64(v, [p])[0]
        krp = _f64(kr, [p])[0] if rope else None
        for b0 in range(0, len(tt), batch):
            tb = tt[b0:b0 + batch]
            qb, dOb, Ob = _f64(q, tb), _f64(dO, tb), _f64(O, tb)   # (n, G, D)
            s = qb @ kp
            if rope:
                qrb = _f64(qr, tb)
                s = s + qrb @ krp
            mb, lb = _f64(smax, tb), _f64(ssum, tb)
            live = lb > 0
            with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
                P = np.where(live, np.exp(sc * s - mb) / np.where(live, lb, 1.0), 0.0)
            dP = dOb @ vp
            delta = (dOb * Ob).sum(axis=2)
            dS = P * (dP - delta)
            out["dk"][i] += sc * np.einsum("nh,nhd->d", dS, qb)
            out["dv"][i] += np.einsum("nh,nhd->d", P, dOb)
            if rope:
                out["dkr"][i] += sc * np.einsum("nh,nhd->d", dS, qrb)
    return out


# ---------------------------------------------------------------------------
# Key -> (token, position) inversion for the deterministic reduction.
# ---------------------------------------------------------------------------

def csr(rows: np.ndarray, T2: int):
    """CSR of the valid (token, position) pairs grouped by key row.

    Pairs are numbered in (token ascending, position ascending) order over the
    valid entries only.  offsets has T2+1 entries; pairs[offsets[p]:offsets[p+1]]
    lists the pairs selecting key row p in ascending pair order.
    """
    flat = rows.reshape(-1)
    keys = flat[flat >= 0]
    order = np.argsort(keys, kind="stable")
    counts = np.bincount(keys, minlength=T2)[:T2]
    offsets = np.zeros(T2 + 1, np.int64)
    np.cumsum(counts, out=offsets[1:])
    return offsets, order.astype(np.int64)


def flops(rows: np.ndarray, G: int, D: int, Dr: int) -> int:
    """Algorithmic flop count: 2*(3*(D+Dr) + 2*D) per valid (head, position) pair
    (S, dQ, dK over D+Dr; dP, dV over D)."""
    n = int((rows >= 0).sum())
    return n * G * 2 * (3 * (D + Dr) + 2 * D)


# ---------------------------------------------------------------------------
# Band (sliding-window or dense) selection expressed as sparse indices.  The
# MindSpore FlashAttention backward page ("flash_attention_bwd.py",
# compute_in_each_kv_block) computes a query block q against a key block k only
# when k - next_block_num <= q <= k + prev_block_num; here the same test is
# taken per query token and aligned, as sparseMode 3 is, on the diagonal
# through the bottom-right corner, so that dense and banded attention run
# through the sparse backward unchanged.
# ---------------------------------------------------------------------------

def band_entries(max_key_len: int, pre: int, nxt: int, block: int) -> int:
    """Index entries per row that hold every block a band can touch."""
    if max_key_len <= 0:
        return 0
    width = min(max_key_len, pre + nxt + 1)
    return min(-(-max_key_len // block), -(-(width - 1) // block) + 1)


def band_indices(geom, K: int, pre: int, nxt: int, block: int) -> np.ndarray:
    """(T1, K) int64 index rows of the band.

    Query position t of a sequence (Lq queries, Lk keys) covers key positions
    d - pre .. d + nxt, d = t + Lk - Lq, clipped to [0, Lk).  Its row lists, in
    ascending order, the start of every block of ``block`` positions (block
    starts are multiples of ``block``) that holds at least one covered
    position, then -1; rows are cut at K entries.
    """
    T1 = geom["T1"]
    out = np.full((T1, K), -1, np.int64)
    for t in range(T1):
        Lk = int(geom["Lk"][t])
        d = int(geom["t_loc"][t]) + Lk - int(geom["Lq"][t])
        covered = [p for p in range(max(0, d - pre), min(Lk - 1, d + nxt) + 1)]
        starts = sorted({(p // block) * block for p in covered})[:K]
        out[t, :len(starts)] = starts
    return out
