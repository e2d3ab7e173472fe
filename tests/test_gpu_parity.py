"""GPU parity: the HIP path against the CPU oracle, element by element, on
seeded inputs small enough for the oracle (several tiles and a ragged tail),
with forward statistics from the oracle's forward pass.

Tolerances (relative L2 against the float64 oracle): dQ and dQueryRope
<= 5e-3, dK, dV and dKeyRope <= 1e-2.  Index decode and the CSR are compared
bit for bit; the deterministic path must be bitwise reproducible.
"""
import os

import numpy as np
import pytest
import torch

import sfag_inputs as si
from oracle import sfag_oracle as orc
from tests._helpers import add_oracle_stats, call_backward, flat, geom_of, oracle_backward, rel_l2, to_device

pytestmark = pytest.mark.gpu

TOL = dict(dq=5e-3, dqr=5e-3, dk=1e-2, dv=1e-2, dkr=1e-2)


def _outs_np(case, outs):
    dq, dk, dv, dqr, dkr = outs
    T1, T2, G = case.T1, case.T2, case.G
    f = lambda x, shape: None if x is None else x.detach().float().cpu().numpy().astype(np.float64).reshape(shape)
    return dict(dq=f(dq, (T1, G, case.D)), dk=f(dk, (T2, case.D)), dv=f(dv, (T2, case.D)),
                dqr=f(dqr, (T1, G, case.Dr)), dkr=f(dkr, (T2, case.Dr)))


def _check(case, got, ref, tol=TOL, label=""):
    errs = {}
    for n in ("dq", "dk", "dv", "dqr", "dkr"):
        if ref[n] is None:
            assert got[n] is None
            continue
        assert np.all(np.isfinite(got[n])), (label, n, "non-finite output")
        errs[n] = rel_l2(got[n], ref[n])
    print(label, {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for n, e in errs.items():
        assert e <= tol[n], (label, n, e)
    return errs


def _never_selected(case, inp):
    f = flat(case, inp)
    rows = orc.decode(f["idx"], case.block, case.mode, geom_of(case))
    sel = np.zeros(case.T2, bool)
    sel[rows[rows >= 0]] = True
    return ~sel


def _run(case, seed, deterministic=None, inp=None, options=None):
    if inp is None:
        inp = add_oracle_stats(case, si.make_inputs(case, seed))
    ref = oracle_backward(case, inp)
    print(f"case {case.name} seed {seed} det={deterministic} options={options}", flush=True)
    kw = {} if deterministic is None else dict(deterministic=deterministic)
    if options:
        kw["options"] = options
    outs = call_backward(case, to_device(inp), **kw)
    torch.cuda.synchronize()
    got = _outs_np(case, outs)
    _check(case, got, ref, label=case.name)
    never = _never_selected(case, inp)
    for n in ("dk", "dv", "dkr"):
        if got[n] is not None:
            assert np.all(got[n][never] == 0), (n, "unselected key rows must be exactly 0")
    return inp, ref, got, outs


SMALL = [
    si.Case("g1_rope_uniform", S1=5, S2=96, G=1, K=70),
    si.Case("g3_fp16_norope", S1=4, S2=80, G=3, Dr=0, K=45, dtype="fp16"),
    si.Case("g4_cfg1_shape", S1=8, S2=256, G=4, K=100),
    si.Case("g16_fp16_blocks", S1=6, S2=512, G=16, Dr=0, K=9, block=16, dtype="fp16", std=0.5,
            index_rule="blocks", scale=1 / 512 ** 0.5),
    si.Case("g20_causal_mix", S1=80, S2=80, G=20, K=40, mode=3, index_rule="causal_mix"),
    si.Case("g64_tnd_causal", layout="TND", B=4, seqlens_q=(17, 0, 33, 9), seqlens_kv=(40, 5, 33, 20), G=64, K=24,
            mode=3, index_rule="causal_mix"),
    si.Case("g96_uniform", S1=3, S2=200, G=96, K=130),
    si.Case("g128_zipf", S1=100, S2=100, G=128, K=64, mode=3, index_rule="zipf"),
    si.Case("g128_fp16_interleaved_pad", S1=6, S2=150, G=128, Dr=0, K=50, dtype="fp16", interleave_pad=True,
            extra_pad=13),
    si.Case("g48_more_queries_than_keys", S1=40, S2=24, G=48, K=24, mode=3, index_rule="all_causal"),
    si.Case("g8_bsnd_b3_blocks8", B=3, S1=5, S2=64, G=8, K=5, block=8, mode=3, index_rule="blocks"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c.name for c in SMALL])
def test_small_against_oracle(case):
    _run(case, seed=7)


# Value passed as the key tensor itself (the operator page supports only
# value identical to key): the library gathers each row once and reads it for
# both S and dP.  dK and dV stay separate outputs.
VALUE_IS_KEY = [
    si.Case("vk_g128_rope", S1=6, S2=300, G=128, K=100),
    si.Case("vk_g64_causal", S1=70, S2=70, G=64, K=40, mode=3, index_rule="causal_mix"),
    si.Case("vk_g96_norope_fp16", S1=5, S2=150, G=96, Dr=0, K=77, dtype="fp16"),
    si.Case("vk_g16_blocks", S1=6, S2=512, G=16, Dr=0, K=9, block=16, dtype="fp16", std=0.5,
            index_rule="blocks", scale=1 / 512 ** 0.5),
    si.Case("vk_g4_rope", S1=8, S2=256, G=4, K=100),
]


@pytest.mark.parametrize("case", VALUE_IS_KEY, ids=[c.name for c in VALUE_IS_KEY])
def test_value_is_key(case):
    inp = si.make_inputs(case, 11)
    inp["value"] = inp["key"]
    inp = add_oracle_stats(case, inp)
    ref = oracle_backward(case, inp)
    dev = to_device(inp)
    dev["value"] = dev["key"]          # one device tensor passed twice
    print(f"case {case.name} value is key", flush=True)
    outs = call_backward(case, dev)
    torch.cuda.synchronize()
    _check(case, _outs_np(case, outs), ref, label=case.name)


@pytest.mark.parametrize("name", ["g64_tnd_causal", "g128_zipf"])
def test_token_paths_agree(name):
    """The fused token kernel (k_row, 64 heads per workgroup) and the split
    one (k_sdp + k_dq) both match the oracle on the same N1 >= 32 inputs."""
    case = next(c for c in SMALL if c.name == name)
    inp = add_oracle_stats(case, si.make_inputs(case, 21))
    for path in ("fused", "split"):
        _run(case, seed=21, inp=inp, options=dict(token_path=path))


@pytest.mark.parametrize("G,options", [(16, None), (128, dict(scatter="keyblock")), (112, dict(scatter="keyblock"))],
                         ids=["g16", "g128_keyblock", "g112_keyblock"])
def test_duplicated_indices(G, options):
    case = si.Case("dup", S1=4, S2=300 if G > 16 else 64, G=G, K=40)
    inp = si.make_inputs(case, 3)
    idx = inp["sparse_indices"].reshape(4, 40)
    idx[0, 10:20] = idx[0, 0]          # one key ten times
    idx[2, :] = idx[2, 5]              # a whole row of one key
    idx[3, 1] = idx[3, 0]              # one key twice
    inp = add_oracle_stats(case, inp)
    _run(case, 3, inp=inp, options=options)


@pytest.mark.parametrize("K", [200, 400], ids=["k200", "k400_long_visits"])
def test_duplicated_indices_key_blocks(K):
    """128 heads, key-block path, three key blocks and three token ranges of
    8: keys listed several times by tokens past the first two of a range
    (slot maps built from pairs copied ahead), and, with K = 400, one key
    listed 300 times (a visit of more pairs than the 256 copied ahead, the
    rest read from memory) and another 280 times by the first token of a
    range (a map built before the pipeline starts)."""
    case = si.Case("dup_maps", S1=24, S2=600, G=128, K=K)
    inp = si.make_inputs(case, 4)
    idx = inp["sparse_indices"].reshape(24, K)
    idx[3, 20:40] = idx[3, 0]          # twenty times
    idx[12, :] = idx[12, 7]            # a whole row of one key
    idx[20, 1] = idx[20, 0]            # twice
    if K > 255:
        idx[5, :300] = 17              # 300 times, fifth token of its range
        idx[8, :280] = 300             # 280 times, first token of its range
    inp = add_oracle_stats(case, inp)
    _run(case, 4, inp=inp, options=dict(scatter="keyblock"))


def test_masked_rows_never_read():
    """Key rows named only by masked entries (after the causal bound, or past
    the key length) hold NaN: every output must stay finite, match the oracle,
    and leave those rows' gradients at exactly 0."""
    case = si.Case("nan_sentinel", S1=30, S2=30, G=16, K=12, mode=3, index_rule="uniform")
    inp = si.make_inputs(case, 11)
    idx = inp["sparse_indices"].view(30, 12)
    for t in range(30):
        row = idx[t]
        row[row >= 25] = -1                      # no valid entry names rows 25..29
        if t < 25:
            row[-5:] = torch.arange(25, 30)      # masked: beyond token t's causal bound
        if t % 3 == 0:
            row[0] = 1000                        # masked: beyond the key length
    for p in range(25, 30):
        inp["key"].view(-1, 512)[p] = float("nan")
        inp["value"].view(-1, 512)[p] = float("nan")
        inp["key_rope"].view(-1, 64)[p] = float("nan")
    inp = add_oracle_stats(case, inp)
    _, ref, got, _ = _run(case, 11, inp=inp)
    assert np.all(got["dk"][25:] == 0) and np.all(got["dv"][25:] == 0)


def test_empty_query():
    case = si.Case("empty", S1=0, S2=32, G=4, K=8)
    inp = si.make_inputs(case, 1)
    inp["out"] = torch.zeros(si.out_shape(case), dtype=torch.bfloat16)
    inp["softmax_max"] = torch.zeros(si.stats_shape(case))
    inp["softmax_sum"] = torch.zeros(si.stats_shape(case))
    dev = to_device(inp)
    outs = call_backward(case, dev)
    torch.cuda.synchronize()
    dq, dk, dv, dqr, dkr = outs
    assert dq.numel() == 0
    assert torch.all(dk == 0) and torch.all(dv == 0) and torch.all(dkr == 0)


DET_CASE = si.Case("det_zipf", S1=64, S2=64, G=128, K=48, mode=3, index_rule="zipf", deterministic=True)


def test_deterministic_bitwise_and_parity():
    inp = add_oracle_stats(DET_CASE, si.make_inputs(DET_CASE, 5))
    _, ref, got, outs = _run(DET_CASE, 5, deterministic=True, inp=inp)
    dev = to_device(inp)
    first = [o.clone() for o in outs if o is not None]
    for _ in range(3):
        again = [o for o in call_backward(DET_CASE, dev, deterministic=True) if o is not None]
        torch.cuda.synchronize()
        for a, b in zip(first, again):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("path", ["keyblock", "partials"])
def test_deterministic_independent_of_chunking(path):
    """The deterministic bits do not depend on how the tokens are chunked
    (chunk limit, workspace budget): every chunking gives the same bits as
    one chunk, on both deterministic dK/dV paths."""
    inp = to_device(add_oracle_stats(DET_CASE, si.make_inputs(DET_CASE, 6)))
    base = [o.clone() for o in call_backward(DET_CASE, inp, deterministic=True, options=dict(scatter=path))
            if o is not None]
    for opts in (dict(chunk_tokens=7), dict(chunk_tokens=20), dict(workspace_budget=1 << 20)):
        opts["scatter"] = path
        print(f"det chunking {opts}", flush=True)
        chunked = [o for o in call_backward(DET_CASE, inp, deterministic=True, options=opts) if o is not None]
        torch.cuda.synchronize()
        for a, b in zip(base, chunked):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), opts


# The key-block contraction at head counts that pad to 128 (the two-waves-per-
# SIMD kernel, heads past N1 in its last 32-head stage) and to 64; the last
# two cases have more key blocks than twice the positions per token, where the
# pairs are grouped by the global radix sort instead of per-token counting.
KEYBLOCK_HEADS = [
    si.Case("kb_g112_causal", S1=48, S2=300, G=112, K=96, mode=3, index_rule="causal_mix"),
    si.Case("kb_g100_fp16_norope", S1=20, S2=280, G=100, Dr=0, K=80, dtype="fp16"),
    si.Case("kb_g40_rope", S1=30, S2=270, G=40, K=70),
    si.Case("kb_g128_radix_grouping", S1=40, S2=4096, G=128, K=4),
    si.Case("kb_g16_radix_grouping", S1=24, S2=3000, G=16, K=5),
]


@pytest.mark.parametrize("case", KEYBLOCK_HEADS, ids=[c.name for c in KEYBLOCK_HEADS])
def test_keyblock_head_counts(case):
    _run(case, seed=11, options=dict(scatter="keyblock"))


@pytest.mark.parametrize("path", ["keyblock", "atomic", "partials"])
@pytest.mark.parametrize("chunk", [0, 9])
def test_scatter_paths_agree(path, chunk):
    """Every dK/dV path (key-block contraction, fp32 atomics, per-pair rows with
    the CSR reduction), with and without token chunking, against the oracle."""
    case = si.Case("paths", S1=50, S2=300, G=64, K=60, mode=3, index_rule="causal_mix")
    inp = add_oracle_stats(case, si.make_inputs(case, 8))
    ref = oracle_backward(case, inp)
    dev = to_device(inp)
    opts = dict(scatter=path)
    if chunk:
        opts["chunk_tokens"] = chunk
    got = _outs_np(case, call_backward(case, dev, deterministic=False, options=opts))
    _check(case, got, ref, label=f"paths {path} chunk {chunk}")


@pytest.mark.parametrize("path", ["keyblock", "partials"])
def test_deterministic_paths_bitwise(path):
    case = si.Case("detpaths", S1=40, S2=260, G=32, K=50, mode=3, index_rule="zipf", deterministic=True)
    inp = to_device(add_oracle_stats(case, si.make_inputs(case, 4)))
    first = [o.clone() for o in call_backward(case, inp, options=dict(scatter=path)) if o is not None]
    for _ in range(2):
        again = [o for o in call_backward(case, inp, options=dict(scatter=path)) if o is not None]
        torch.cuda.synchronize()
        for x, y in zip(first, again):
            assert torch.equal(x, y)


def test_build_index_bit_exact():
    import top_sparse_attention_sfag_amd as sfag
    cases = [
        si.Case("idx_bsnd_causal", S1=70, S2=90, G=1, K=50, mode=3, index_rule="causal_mix", interleave_pad=True,
                extra_pad=5),
        si.Case("idx_blocks", B=2, S1=9, S2=256, G=1, Dr=0, K=10, block=16, index_rule="blocks", mode=3),
        si.Case("idx_tnd", layout="TND", B=3, seqlens_q=(20, 0, 31), seqlens_kv=(25, 4, 31), G=1, K=16, mode=3,
                index_rule="causal_mix"),
    ]
    for case in cases:
        inp = si.make_inputs(case, 2)
        idx = inp["sparse_indices"]
        # some out-of-range and negative entries the mask must drop
        flat_idx = idx.view(-1)
        flat_idx[::17] = 10 ** 6
        flat_idx[::23] = -5
        geom = geom_of(case)
        rows_ref = orc.decode(idx.reshape(case.T1, case.Kent), case.block, case.mode, geom)
        off_ref, pairs_ref = orc.csr(rows_ref, case.T2)
        E = case.Kent * case.block
        nvalid_ref = (rows_ref >= 0).sum(1)
        # oracle pair ids (valid pairs in (token, position) order) -> t*E + rank in token
        tt, _ = np.nonzero(rows_ref >= 0)
        rank = np.concatenate([np.arange(n) for n in nvalid_ref]) if len(nvalid_ref) else np.zeros(0, int)
        pair_code = tt * E + rank
        dev = idx.cuda()
        kw = dict(T2=case.T2, block_size=case.block, layout=case.layout, sparse_mode=case.mode)
        if case.layout == "TND":
            kw.update(seqlens_q=inp["seqlens_q"].cuda(), seqlens_kv=inp["seqlens_kv"].cuda())
        else:
            kw.update(B=case.B, S1=case.S1, S2=case.S2)
        nv, rows, off, pairs = sfag.build_index(dev.reshape(case.T1, case.Kent), **kw)
        torch.cuda.synchronize()
        nv, rows, off, pairs = (x.cpu().numpy() for x in (nv, rows, off, pairs))
        np.testing.assert_array_equal(nv, nvalid_ref)
        for t in range(case.T1):
            np.testing.assert_array_equal(rows[t, :nv[t]], rows_ref[t][rows_ref[t] >= 0])
        np.testing.assert_array_equal(off, off_ref)
        np.testing.assert_array_equal(pairs[: off[-1]], pair_code[pairs_ref])


REDUCED = {
    1: si.CONFIGS[1],
    2: si.CONFIGS[2].replace(name="cfg2_reduced", S1=320, S2=320, K=256),
    3: si.CONFIGS[3].replace(name="cfg3_reduced", seqlens_q=(96, 160, 32, 224), seqlens_kv=(96, 160, 32, 224),
                             K=128),
    4: si.CONFIGS[4].replace(name="cfg4_reduced", B=2, S1=96, S2=1024, K=24),
    5: si.CONFIGS[5].replace(name="cfg5_reduced", S1=256, S2=256, K=128),
}


@pytest.mark.parametrize("cfg", sorted(REDUCED))
def test_reduced_configs(cfg):
    """Each workload's structure (heads, rope, dtype, layout, mask, index rule,
    block size, determinism) at a token count the oracle finishes in seconds."""
    _run(REDUCED[cfg], seed=si.seed_for(cfg))


@pytest.mark.parametrize("G", [16, 64])
def test_no_keys(G):
    """S2 = 0: every position is masked, so dQ is 0 and the key gradients are
    empty (the key-block path, which needs key rows, is not chosen)."""
    case = si.Case(f"no_keys_g{G}", S1=6, S2=0, G=G, K=8)
    inp = add_oracle_stats(case, si.make_inputs(case, 2))
    _, ref, got, outs = _run(case, 2, inp=inp)
    assert torch.all(outs[0] == 0) and outs[1].numel() == 0


def test_validation_flags():
    """Opt-in device checks: consistent inputs raise no flag and leave the
    results unchanged; TND lengths that are negative or do not add up to
    T1 / T2, and index entries at or past their sequence's key length, are
    reported (such entries are masked, never read)."""
    import top_sparse_attention_sfag_amd as sfag
    case = si.Case("validate_tnd", layout="TND", B=3, seqlens_q=(5, 7, 4), seqlens_kv=(20, 10, 30), G=32, K=12,
                   mode=3, index_rule="causal_mix")
    inp = add_oracle_stats(case, si.make_inputs(case, 3))
    dev = to_device(inp)
    base = [o.clone() for o in call_backward(case, dev) if o is not None]
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")
    got = [o for o in call_backward(case, dev, options=dict(validate=True), workspace=ws) if o is not None]
    assert sfag.validation_read(ws) == dict(flags=0, bad_entries=0)
    for a, b in zip(base, got):
        assert torch.equal(a, b)
    # entries past the key length of their sequence
    idx = dev["sparse_indices"].clone().view(case.T1, case.Kent)
    geom = geom_of(case)
    plant = [(0, 0, 25), (6, 3, 10), (6, 4, 11), (15, 0, 30)]   # (token, entry, value): Lk 20, 10, 10, 30
    for t, j, val in plant:
        idx[t, j] = val
    bad = sum(1 for t, _j, val in plant if val >= geom["Lk"][t])
    d2 = dict(dev, sparse_indices=idx.view_as(dev["sparse_indices"]))
    call_backward(case, d2, options=dict(validate=True), workspace=ws)
    assert sfag.validation_read(ws) == dict(flags=sfag.BAD_INDEX_RANGE, bad_entries=bad)
    # lengths: a negative one, and sums that differ from T1 / T2
    d3 = dict(dev, seqlens_q=torch.tensor([5, -1, 4], dtype=torch.int32, device="cuda"),
              seqlens_kv=torch.tensor([20, 10, 31], dtype=torch.int32, device="cuda"))
    call_backward(case, d3, options=dict(validate=True), workspace=ws)
    r = sfag.validation_read(ws)
    assert r["flags"] & (sfag.BAD_LENGTH_NEGATIVE | sfag.BAD_LENGTH_SUM_Q | sfag.BAD_LENGTH_SUM_KV) == \
        sfag.BAD_LENGTH_NEGATIVE | sfag.BAD_LENGTH_SUM_Q | sfag.BAD_LENGTH_SUM_KV


def test_auxiliary_stream_of_the_caller():
    """A concurrent call on a second stream the caller passes gives the same
    bits as the serial call."""
    case = si.Case("aux_g64", S1=60, S2=300, G=64, K=60, mode=3, index_rule="causal_mix")
    inp = to_device(add_oracle_stats(case, si.make_inputs(case, 12)))
    serial = [o.clone() for o in call_backward(case, inp, options=dict(concurrent="off")) if o is not None]
    aux = torch.cuda.Stream()
    got = [o for o in call_backward(case, inp, options=dict(concurrent="on", aux_stream=aux)) if o is not None]
    torch.cuda.synchronize()
    for a, b in zip(serial, got):
        assert torch.equal(a, b)


# Listing-order invariance: each token's entries are walked in ascending key
# order whatever order the listing gives them (no key listed twice, keys
# below 65536), so a permuted listing gives the same bits, forward and
# backward, on the 128-head, N1 <= 16 (blocks) and TND paths.
ORDER_CASES = [
    si.Case("order_g128_causal", S1=48, S2=300, G=128, K=96, mode=3, index_rule="causal_mix"),
    si.Case("order_g16_blocks", S1=20, S2=512, G=16, Dr=0, K=12, block=16, dtype="fp16", std=0.5,
            index_rule="blocks"),
    si.Case("order_g64_tnd", layout="TND", B=3, seqlens_q=(20, 0, 31), seqlens_kv=(60, 4, 90), G=64, K=40,
            mode=3, index_rule="causal_mix"),
]


@pytest.mark.parametrize("case", ORDER_CASES, ids=[c.name for c in ORDER_CASES])
def test_listing_order_does_not_change_bits(case):
    import top_sparse_attention_sfag_amd as sfag
    inp = add_oracle_stats(case, si.make_inputs(case, 8))
    idx = inp["sparse_indices"].cpu()
    rows = idx.reshape(-1, idx.shape[-1])
    g = torch.Generator().manual_seed(11)
    perm = torch.stack([torch.randperm(rows.shape[1], generator=g) for _ in range(rows.shape[0])])
    shuffled = torch.gather(rows, 1, perm).reshape(idx.shape).contiguous()
    assert not torch.equal(shuffled, idx)
    runs = []
    for listing in (idx, shuffled):
        dev = to_device(dict(inp, sparse_indices=listing))
        print(f"listing order {case.name}", flush=True)
        outs = [o.clone() for o in call_backward(case, dev, deterministic=True) if o is not None]
        fwd = sfag.forward(dev["query"], dev["key"], dev["value"], dev["sparse_indices"],
                           seqlens_q=dev.get("seqlens_q"), seqlens_kv=dev.get("seqlens_kv"),
                           query_rope=dev.get("query_rope"), key_rope=dev.get("key_rope"), scale=case.scale_value,
                           block_size=case.block, layout=case.layout, sparse_mode=case.mode)
        torch.cuda.synchronize()
        runs.append(outs + [fwd[0].clone(), fwd[1].clone(), fwd[2].clone()])
    for a, b in zip(*runs):
        assert torch.equal(a.view(torch.int16) if a.element_size() == 2 else a.view(torch.int32),
                           b.view(torch.int16) if b.element_size() == 2 else b.view(torch.int32))
