"""Seeded synthetic inputs for the sparse flash attention backward.

This module draws random numbers and nothing else: it holds none of the
attention arithmetic (no logits, softmax, statistics or gradients).  Both the
CPU oracle and the HIP path receive what it produces, so it is the only code the
two share.  Tensors are drawn with a seeded ``torch.Generator`` on the device
requested (CPU for oracle-sized cases, the GPU for full-size ones) and cast to
bf16/fp16 with round-to-nearest-even.

Shapes follow the operator description "aclnnSparseFlashAttentionGrad" (the
parameter table of its GetWorkspaceSize section): query/dOut/out are
(B,S1,N1,D) or (T1,N1,D), key/value (B,S2,1,D) or (T2,1,D), sparseIndices
(B,S1,1,K) or (T1,1,K) int32, softmaxMax/softmaxSum (B,1,S1,N1) or (1,T1,N1)
fp32, rope parts with Dr=64.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import torch

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}


@dataclasses.dataclass(frozen=True)
class Case:
    """One synthetic workload.  Index rules:

    * ``uniform``: K distinct key positions drawn uniformly from [0, Lk).
    * ``blocks``: K distinct block starts drawn uniformly from the multiples of
      ``block`` below Lk.
    * ``causal_mix``: for token t with causal bound b = t_loc + Lk - Lq, if b+1 <= K
      every key in [0, b] is selected and the rest of the row is -1; otherwise
      the K/4 most recent keys (b-K/4, b] plus 3K/4 distinct uniform keys from
      [0, b-K/4].
    * ``zipf``: min(K, b+1) distinct keys from [0, b] without replacement, key s
      weighted by (b - s + 1)^-zipf_s (Gumbel top-k).
    * ``all``: every key of the sequence once (K = Lk), a random permutation.
    * ``all_causal``: every key in [0, b], random order, -1 padding.

    Valid entries are emitted in a seeded random order with any -1 padding at
    the tail (``interleave_pad`` scatters the padding among the valid entries).
    """

    name: str
    layout: str = "BSND"
    B: int = 1
    S1: int = 128
    S2: int = 2048
    seqlens_q: Optional[Sequence[int]] = None
    seqlens_kv: Optional[Sequence[int]] = None
    G: int = 4
    D: int = 512
    Dr: int = 64
    K: int = 1024
    block: int = 1
    mode: int = 0
    dtype: str = "bf16"
    std: float = 1.0
    index_rule: str = "uniform"
    zipf_s: float = 1.1
    deterministic: bool = False
    scale: Optional[float] = None
    interleave_pad: bool = False
    extra_pad: int = 0  # append this many -1 entries to every row (K grows by it)

    @property
    def T1(self) -> int:
        return int(sum(self.seqlens_q)) if self.layout == "TND" else self.B * self.S1

    @property
    def T2(self) -> int:
        return int(sum(self.seqlens_kv)) if self.layout == "TND" else self.B * self.S2

    @property
    def Kent(self) -> int:
        return self.K + self.extra_pad

    @property
    def scale_value(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.D + self.Dr)

    def sequences(self):
        """Yield (b, q_start, Lq, kv_start, Lk) per batch entry."""
        if self.layout == "TND":
            qs = ks = 0
            for b, (lq, lk) in enumerate(zip(self.seqlens_q, self.seqlens_kv)):
                yield b, qs, int(lq), ks, int(lk)
                qs += int(lq)
                ks += int(lk)
        else:
            for b in range(self.B):
                yield b, b * self.S1, self.S1, b * self.S2, self.S2

    def replace(self, **kw) -> "Case":
        return dataclasses.replace(self, **kw)


# The five workloads: shapes, index structure, value distributions.
CONFIGS = {
    1: Case("cfg1_bsnd_g4_k1024", layout="BSND", B=1, S1=128, S2=2048, G=4, K=1024,
            block=1, mode=0, dtype="bf16", std=1.0, index_rule="uniform"),
    2: Case("cfg2_bsnd_g128_s4096_k2048_causal", layout="BSND", B=1, S1=4096, S2=4096, G=128,
            K=2048, block=1, mode=3, dtype="bf16", std=1.0, index_rule="causal_mix"),
    3: Case("cfg3_tnd_g64_k2048_causal", layout="TND", B=4, seqlens_q=(1024, 3072, 512, 3584),
            seqlens_kv=(1024, 3072, 512, 3584), G=64, K=2048, block=1, mode=3, dtype="bf16",
            std=1.0, index_rule="causal_mix"),
    4: Case("cfg4_bsnd_g16_s16384_blk16x512_fp16", layout="BSND", B=2, S1=16384, S2=16384, G=16,
            Dr=0, K=512, block=16, mode=0, dtype="fp16", std=0.5, index_rule="blocks",
            scale=1.0 / math.sqrt(512)),
    5: Case("cfg5_bsnd_g128_s32768_k8192_zipf_det", layout="BSND", B=1, S1=32768, S2=32768, G=128,
            K=8192, block=1, mode=3, dtype="bf16", std=1.0, index_rule="zipf", deterministic=True),
}


def seed_for(cfg: int) -> int:
    return 1000 + cfg


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, std, dtype, g, device):
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(DTYPES[dtype])


def _shuffle_rows(sel: torch.Tensor, g, device) -> torch.Tensor:
    """Random order for the valid (>=0) entries of each row, -1 entries last."""
    key = torch.rand(sel.shape, generator=g, device=device)
    key = torch.where(sel >= 0, key, torch.full_like(key, 2.0))
    order = torch.argsort(key, dim=1)
    return torch.gather(sel, 1, order)


def _interleave(sel: torch.Tensor, g, device) -> torch.Tensor:
    key = torch.rand(sel.shape, generator=g, device=device)
    return torch.gather(sel, 1, torch.argsort(key, dim=1))


def _rows_for_sequence(case: Case, Lq: int, Lk: int, g, device, row_chunk: int = 1024) -> torch.Tensor:
    K, bs, rule = case.K, case.block, case.index_rule
    out = torch.full((Lq, K), -1, dtype=torch.int64, device=device)
    for r0 in range(0, Lq, row_chunk):
        r1 = min(Lq, r0 + row_chunk)
        n = r1 - r0
        t_loc = torch.arange(r0, r1, device=device)
        if case.mode == 3:
            bound = t_loc + (Lk - Lq)
        else:
            bound = torch.full((n,), Lk - 1, device=device)
        s = torch.arange(Lk, device=device)
        if rule == "blocks":
            nb = Lk // bs
            u = torch.rand(n, nb, generator=g, device=device)
            sb = torch.arange(nb, device=device) * bs
            eligible = sb[None, :] <= bound[:, None]
            score = torch.where(eligible, u, torch.full_like(u, -1.0))
            kk = min(K, nb)
            val, pos = torch.topk(score, kk, dim=1)
            sel = torch.where(val >= 0, sb[pos], torch.full_like(pos, -1))
        else:
            u = torch.rand(n, Lk, generator=g, device=device)
            eligible = s[None, :] <= bound[:, None]
            if rule in ("uniform", "all", "all_causal"):
                score = u
            elif rule == "causal_mix":
                local = s[None, :] > (bound[:, None] - K // 4)
                score = torch.where(local, u + 2.0, u)
            elif rule == "zipf":
                age = (bound[:, None] - s[None, :] + 1).clamp(min=1).to(torch.float32)
                gum = -torch.log(-torch.log(u.clamp(min=1e-20, max=1 - 1e-7)))
                score = -case.zipf_s * torch.log(age) + gum + 1e3
            else:
                raise ValueError(rule)
            score = torch.where(eligible, score, torch.full_like(score, -1.0))
            kk = min(K, Lk)
            val, pos = torch.topk(score, kk, dim=1)
            sel = torch.where(val >= 0, pos, torch.full_like(pos, -1))
        out[r0:r1, : sel.shape[1]] = sel
    return out


def make_indices(case: Case, g, device) -> torch.Tensor:
    """(T1, Kent) int32 index rows, local to each sequence."""
    rows = []
    for _b, _qs, Lq, _ks, Lk in case.sequences():
        if Lq == 0:
            continue
        rows.append(_rows_for_sequence(case, Lq, Lk, g, device))
    if rows:
        sel = torch.cat(rows, 0)
    else:
        sel = torch.full((0, case.K), -1, dtype=torch.int64, device=device)
    sel = _shuffle_rows(sel, g, device)
    if case.extra_pad:
        sel = torch.cat([sel, torch.full((sel.shape[0], case.extra_pad), -1, dtype=sel.dtype, device=device)], 1)
    if case.interleave_pad:
        sel = _interleave(sel, g, device)
    return sel.to(torch.int32)


def make_inputs(case: Case, seed: int, device="cpu") -> dict:
    """Q, K, V, rope parts, dO and indices for ``case`` in the operator layouts.

    Returns a dict of tensors on ``device``.  ``out``, ``softmax_max`` and
    ``softmax_sum`` are not drawn here: they come from the oracle's forward
    pass (tests) or from :func:`standin_stats`.
    """
    g = _gen(seed, device)
    T1, T2, G, D, Dr = case.T1, case.T2, case.G, case.D, case.Dr
    bsnd = case.layout == "BSND"
    qshape = (case.B, case.S1, G) if bsnd else (T1, G)
    kshape = (case.B, case.S2, 1) if bsnd else (T2, 1)
    ishape = (case.B, case.S1, 1) if bsnd else (T1, 1)
    d = {}
    d["query"] = _normal((*qshape, D), case.std, case.dtype, g, device)
    d["key"] = _normal((*kshape, D), case.std, case.dtype, g, device)
    d["value"] = _normal((*kshape, D), case.std, case.dtype, g, device)
    d["dout"] = _normal((*qshape, D), case.std, case.dtype, g, device)
    if Dr:
        d["query_rope"] = _normal((*qshape, Dr), case.std, case.dtype, g, device)
        d["key_rope"] = _normal((*kshape, Dr), case.std, case.dtype, g, device)
    idx = make_indices(case, g, device)
    d["sparse_indices"] = idx.reshape(*ishape, case.Kent).contiguous()
    if not bsnd:
        d["seqlens_q"] = torch.tensor(list(case.seqlens_q), dtype=torch.int32, device=device)
        d["seqlens_kv"] = torch.tensor(list(case.seqlens_kv), dtype=torch.int32, device=device)
    return d


def stats_shape(case: Case):
    return (case.B, 1, case.S1, case.G) if case.layout == "BSND" else (1, case.T1, case.G)


def out_shape(case: Case):
    return (case.B, case.S1, case.G, case.D) if case.layout == "BSND" else (case.T1, case.G, case.D)


def standin_stats(case: Case, inputs: dict, seed: int, device="cpu") -> dict:
    """Stand-in forward statistics for sizes where the oracle's forward pass is
    too slow to run: softmaxMax = 0, softmaxSum = the number of selected
    positions of the token (entries >= 0 times the block size), out drawn from
    N(0, (std/4)^2).  Tokens with no selected position get max = -inf, sum = 0,
    out = 0.  The backward pass takes these as given inputs, so it is defined
    for them exactly as for statistics that came from a forward pass.
    """
    g = _gen(seed + 7919, device)
    idx = inputs["sparse_indices"].reshape(case.T1, case.Kent)
    nsel = (idx >= 0).sum(1).to(torch.float32) * case.block
    none = nsel == 0
    m = torch.zeros(case.T1, case.G, dtype=torch.float32, device=device)
    m[none] = float("-inf")
    l = nsel[:, None].expand(case.T1, case.G).contiguous()
    o = torch.randn(case.T1, case.G, case.D, generator=g, device=device) * (case.std / 4)
    o[none] = 0
    return {
        "out": o.to(DTYPES[case.dtype]).reshape(out_shape(case)).contiguous(),
        "softmax_max": m.reshape(stats_shape(case)).contiguous(),
        "softmax_sum": l.reshape(stats_shape(case)).contiguous(),
    }
