"""C ABI on the CPU: the library loads and exports what include/sfag.h declares,
and phase-1 validation returns the status codes of the operator page's 返回值
table (161001 null pointer, 161002 invalid dtype/format, 561002 attribute or
shape outside the supported range).  Phase 1 reads no tensor data, so these
tests run without a GPU."""
import ctypes
import os
import re

import pytest
import torch

import top_sparse_attention_sfag_amd as sfag

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "sfag.h")


def test_exports_every_declared_function():
    src = open(HDR).read()
    names = set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s+(sfag_\w+)\s*\(", src, re.M))
    assert {"sfag_workspace_size", "sfag_backward", "sfag_plan_destroy", "sfag_last_error",
            "sfag_index_workspace_size", "sfag_build_index"} <= names
    L = ctypes.CDLL(sfag.LIB_PATH)
    for n in sorted(names):
        assert hasattr(L, n), n


def _tensors(layout="BSND", B=1, S1=2, S2=8, G=4, D=512, Dr=64, K=4, dtype=torch.bfloat16):
    if layout == "BSND":
        q = torch.zeros(B, S1, G, D, dtype=dtype)
        k = torch.zeros(B, S2, 1, D, dtype=dtype)
        idx = torch.zeros(B, S1, 1, K, dtype=torch.int32)
        st = torch.zeros(B, 1, S1, G)
        qr = torch.zeros(B, S1, G, Dr, dtype=dtype) if Dr else None
        kr = torch.zeros(B, S2, 1, Dr, dtype=dtype) if Dr else None
        lq = lk = None
    else:
        T1, T2 = B * S1, B * S2
        q = torch.zeros(T1, G, D, dtype=dtype)
        k = torch.zeros(T2, 1, D, dtype=dtype)
        idx = torch.zeros(T1, 1, K, dtype=torch.int32)
        st = torch.zeros(1, T1, G)
        qr = torch.zeros(T1, G, Dr, dtype=dtype) if Dr else None
        kr = torch.zeros(T2, 1, Dr, dtype=dtype) if Dr else None
        lq = torch.full((B,), S1, dtype=torch.int32)
        lk = torch.full((B,), S2, dtype=torch.int32)
    return dict(query=q, key=k, value=k.clone(), sparse_indices=idx, dout=q.clone(), out=q.clone(),
                softmax_max=st, softmax_sum=st.clone(), dq=q.clone(), dk=k.clone(), dv=k.clone(),
                query_rope=qr, key_rope=kr, dq_rope=None if qr is None else qr.clone(),
                dk_rope=None if kr is None else kr.clone(), seqlens_q=lq, seqlens_kv=lk, layout=layout)


def _plan(t, **over):
    t = dict(t)
    t.update(over)
    args = [t.pop(n) for n in ("query", "key", "value", "sparse_indices", "dout", "out", "softmax_max",
                               "softmax_sum", "dq", "dk", "dv")]
    return sfag.plan(*args, **t)


def _code(t, **over):
    try:
        ws, p = _plan(t, **over)
    except sfag.SfagError as e:
        return e.code
    sfag.destroy(p)
    return 0


def test_valid_plans():
    for layout in ("BSND", "TND"):
        for Dr in (0, 64):
            t = _tensors(layout, Dr=Dr)
            ws, p = _plan(t)
            assert ws > 0
            sfag.destroy(p)
    t = _tensors("BSND", dtype=torch.float16)
    assert _code(t, block_size=16, sparse_mode=3, deterministic=True) == 0


def test_empty_query_needs_no_workspace():
    t = _tensors(S1=0)
    ws, p = _plan(t)
    assert ws == 0
    sfag.destroy(p)


@pytest.mark.parametrize("over,code", [
    (dict(layout="BNSD"), 561002),
    (dict(sparse_mode=1), 561002),
    (dict(sparse_mode=4), 561002),
    (dict(block_size=2), 561002),
    (dict(pre_tokens=100), 561002),
    (dict(next_tokens=0), 561002),
    (dict(scale=float("nan")), 161002),
    (dict(key_rope=None), 161002),
    (dict(dq_rope=None), 161001),
    (dict(query=None), 161001),
    (dict(dk=None), 161001),
])
def test_attribute_and_presence_errors(over, code):
    assert _code(_tensors(), **over) == code


def test_dtype_and_format_errors():
    t = _tensors()
    assert _code(t, key=t["key"].half()) == 161002
    assert _code(t, sparse_indices=t["sparse_indices"].long()) == 161002
    assert _code(t, softmax_max=t["softmax_max"].half()) == 161002
    assert _code(t, query=t["query"].float(), dout=t["dout"].float(), out=t["out"].float(),
                 dq=t["dq"].float()) == 161002
    nc = t["query"].transpose(1, 2).contiguous().transpose(1, 2)
    assert not nc.is_contiguous()
    assert _code(t, query=nc) == 161002
    tt = _tensors("TND")
    assert _code(tt, seqlens_q=tt["seqlens_q"].long()) == 161002


def test_shape_errors():
    assert _code(_tensors(D=256)) == 561002
    assert _code(_tensors(Dr=32)) == 561002
    assert _code(_tensors(G=129, S1=1, K=1, Dr=0)) == 561002
    assert _code(_tensors(B=257, S1=1, S2=1, K=1, Dr=0, G=1)) == 561002
    t = _tensors()
    k2 = torch.zeros(1, 8, 2, 512, dtype=torch.bfloat16)
    assert _code(t, key=k2, value=k2.clone(), dk=k2.clone(), dv=k2.clone()) == 561002   # N2 != 1
    assert _code(t, sparse_indices=torch.zeros(1, 3, 1, 4, dtype=torch.int32)) == 561002
    assert _code(t, softmax_sum=torch.zeros(1, 1, 2, 5)) == 561002
    assert _code(t, dv=torch.zeros(1, 9, 1, 512, dtype=torch.bfloat16)) == 561002
    tt = _tensors("TND")
    assert _code(tt, seqlens_q=None) == 561002
    assert _code(tt, seqlens_kv=torch.zeros(2, dtype=torch.int32)) == 561002
    assert _code(_tensors(S1=131073, G=1, K=1, Dr=0)) == 561002


def test_backward_rejects_small_workspace_before_launch():
    t = _tensors()
    ws, p = _plan(t)
    rc = sfag.lib().sfag_backward(None, ctypes.c_uint64(ws - 1), p, None)   # consumes the plan
    assert rc == 161002
    assert b"workspace" in sfag.lib().sfag_last_error()


def test_null_plan():
    assert sfag.lib().sfag_backward(None, ctypes.c_uint64(0), None, None) == 161001


def _fwd_plan(t, drop=None):
    """Phase 1 of the forward call through the C ABI; returns (rc, ws, plan)."""
    from top_sparse_attention_sfag_amd._binding import _desc
    t = dict(t)
    if drop:
        t[drop] = None
    ws = ctypes.c_uint64(0)
    p = ctypes.c_void_p(None)
    rc = sfag.lib().sfag_forward_workspace_size(
        _desc(t["query"]), _desc(t["key"]), _desc(t["value"]), _desc(t["sparse_indices"]), _desc(t["seqlens_q"]),
        _desc(t["seqlens_kv"]), _desc(t["query_rope"]), _desc(t["key_rope"]), 0.04, 1, t["layout"].encode(), 0,
        _desc(t["out"]), _desc(t["softmax_max"]), _desc(t["softmax_sum"]), ctypes.byref(ws), ctypes.byref(p))
    return rc, int(ws.value), p


def test_forward_plans():
    for layout in ("BSND", "TND"):
        for Dr in (0, 64):
            rc, ws, p = _fwd_plan(_tensors(layout, Dr=Dr))
            assert rc == 0 and ws > 0
            sfag.destroy(p)
    rc, ws, p = _fwd_plan(_tensors(S1=0))
    assert rc == 0 and ws == 0
    sfag.destroy(p)
    for missing, code in (("out", 161001), ("softmax_sum", 161001), ("query", 161001), ("key_rope", 161002)):
        rc, _, p = _fwd_plan(_tensors(), drop=missing)
        assert rc == code, (missing, rc)
        assert not p.value


def test_plans_are_not_interchangeable():
    # a forward plan given to the backward call and the other way round: both
    # fail before anything is enqueued, and consume the plan
    rc, ws, p = _fwd_plan(_tensors())
    assert rc == 0
    assert sfag.lib().sfag_backward(None, ctypes.c_uint64(ws), p, None) == 161002
    assert b"forward" in sfag.lib().sfag_last_error()
    ws, p = _plan(_tensors())
    assert sfag.lib().sfag_forward(None, ctypes.c_uint64(ws), p, None) == 161002
    assert b"backward" in sfag.lib().sfag_last_error()


def test_band_entries_and_argument_errors():
    """Band selection: the entry count and every host-side rejection (these
    return before anything is launched, so no GPU is needed)."""
    L = sfag.lib()
    assert L.sfag_band_entries(4096, 2147483647, 0, 1) == 4096
    assert L.sfag_band_entries(4096, 127, 0, 1) == 128
    assert L.sfag_band_entries(4096, 127, 0, 16) == 9      # 128 positions can straddle 9 blocks of 16
    assert L.sfag_band_entries(100, 2147483647, 2147483647, 64) == 2
    assert L.sfag_band_entries(0, 5, 5, 1) == 0 and L.sfag_band_entries(10, -1, 0, 1) == 0
    null = ctypes.c_void_p(None)
    dummy = ctypes.c_void_p(16)
    call = lambda *a: L.sfag_band_indices(*a)
    assert call(dummy, null, null, 1, 8, 8, 8, 8, 1, 2, 0, 0, null) == sfag.ERR_TILING        # layout
    assert call(dummy, null, null, 1, 8, 8, 8, 8, 0, 0, 0, 0, null) == sfag.ERR_TILING        # block
    assert call(dummy, null, null, 1, 8, 8, 8, 8, 1, 0, -1, 0, null) == sfag.ERR_TILING       # preTokens
    assert call(dummy, null, null, 1, 8, 8, 9, 8, 1, 0, 0, 0, null) == sfag.ERR_TILING        # T1 != B*S1
    assert call(dummy, null, null, 0, 0, 0, 4, 8, 1, 1, 0, 0, null) == sfag.ERR_TILING        # TND B = 0
    assert call(dummy, null, null, 2, 0, 0, 4, 8, 1, 1, 0, 0, null) == sfag.ERR_NULLPTR       # TND lengths
    assert call(null, null, null, 1, 8, 8, 8, 8, 1, 0, 0, 0, null) == sfag.ERR_NULLPTR        # output


def test_few_token_split_needs_a_dq_buffer_only_when_not_deterministic():
    """Phase 1 plans the few-token split of the fused token kernel (N1 <= 16)
    with an fp32 dQ|dQrope buffer of chunk x N1 x (512 + Dr) floats; a
    deterministic call never splits, so its workspace lacks exactly that."""
    t = _tensors("BSND", B=1, S1=8, S2=400, G=4, Dr=64, K=256)
    ws_split, p = _plan(t)
    sfag.destroy(p)
    ws_det, p = _plan(t, deterministic=True)
    sfag.destroy(p)
    assert ws_split - ws_det == 8 * 4 * (512 + 64) * 4
    # many heads: the split kernel is not used, the workspaces are equal
    t = _tensors("BSND", B=1, S1=8, S2=400, G=64, Dr=64, K=256)
    a, p = _plan(t)
    sfag.destroy(p)
    b, p = _plan(t, deterministic=True)
    sfag.destroy(p)
    assert a == b


def test_band_entries_match_the_oracle_count():
    """sfag_band_entries (host C) against the oracle's band_entries over a
    grid of key lengths, windows and block sizes, including unbounded ones."""
    from oracle import sfag_oracle as orc
    L = sfag.lib()
    big = 2147483647
    for lk in (1, 2, 7, 16, 33, 100, 4096, 131072):
        for pre in (0, 1, 5, 63, 1023, big):
            for nxt in (0, 3, 64, big):
                for block in (1, 8, 16, 64):
                    assert L.sfag_band_entries(lk, pre, nxt, block) == orc.band_entries(lk, pre, nxt, block), \
                        (lk, pre, nxt, block)


def _configure(p, **opts):
    o = sfag.make_options(opts) if opts else None
    ws = ctypes.c_uint64(0)
    rc = sfag.lib().sfag_plan_configure(p, ctypes.byref(o) if o is not None else None, ctypes.byref(ws))
    return rc, int(ws.value)


def test_configure_defaults_and_budget():
    """sfag_plan_configure re-plans from the shapes: no options = the phase-1
    size; a smaller budget gives a smaller workspace (more, smaller chunks);
    validation adds exactly the 256-byte result region."""
    t = _tensors("BSND", B=1, S1=512, S2=1024, G=64, Dr=64, K=256)
    ws0, p = _plan(t, sparse_mode=3)
    assert _configure(p) == (0, ws0)
    rc, ws_small = _configure(p, workspace_budget=64 << 20)
    assert rc == 0 and ws_small < ws0
    rc, ws_val = _configure(p, validate=True)
    assert rc == 0 and ws_val == ws0 + 256
    rc, ws_chunk = _configure(p, chunk_tokens=8)
    assert rc == 0 and ws_chunk < ws0
    sfag.destroy(p)


@pytest.mark.parametrize("field,value", [("scatter", 4), ("tokenPath", 3), ("tokenOrder", -1), ("concurrent", 3),
                                         ("rowSplit", 9), ("keyBlockRanges", -2), ("chunkTokens", -1),
                                         ("validate", 2)])
def test_configure_rejects_bad_fields(field, value):
    t = _tensors()
    ws0, p = _plan(t)
    o = sfag._binding.SfagOptions()
    setattr(o, field, value)
    ws = ctypes.c_uint64(0)
    assert sfag.lib().sfag_plan_configure(p, ctypes.byref(o), ctypes.byref(ws)) == 161002
    assert _configure(p) == (0, ws0)   # the plan is left as it was
    sfag.destroy(p)
    assert sfag.lib().sfag_plan_configure(None, None, ctypes.byref(ws)) == 161001


def test_configure_forward_plan():
    rc, ws0, p = _fwd_plan(_tensors("BSND", S1=64, S2=128, K=32))
    assert rc == 0
    rc, ws1 = _configure(p, workspace_budget=1 << 16)
    assert rc == 0 and ws1 < ws0
    rc, ws2 = _configure(p, validate=True)
    assert rc == 0 and ws2 == ws0 + 256
    sfag.destroy(p)


def test_empty_query_validation_workspace():
    t = _tensors("TND", S1=0)
    ws, p = _plan(t)
    assert ws == 0
    rc, ws = _configure(p, validate=True)
    assert rc == 0 and ws >= 256
    sfag.destroy(p)


def test_validation_read_null_arguments():
    v = sfag._binding.SfagValidation()
    assert sfag.lib().sfag_validation_read(None, None, ctypes.byref(v)) == 161001
    assert sfag.lib().sfag_validation_read(ctypes.c_void_p(256), None, None) == 161001


def _fake(shape, dtype_code):
    """A descriptor with a placeholder data pointer: phase 1 reads no data."""
    d = sfag._binding.SfagTensor()
    d.data = 4096
    d.dtype = dtype_code
    d.ndim = len(shape)
    stride = 1
    for i in reversed(range(len(shape))):
        d.shape[i] = shape[i]
        d.stride[i] = stride
        stride *= shape[i]
    return ctypes.pointer(d)


def test_long_keys_cap_the_chunk_instead_of_failing():
    """128K keys make 512 key blocks: the key-block sort key (block x chunk +
    token) must stay below 2^31, so phase 1 caps the chunk (here 128K query
    tokens, which would not fit in one chunk) instead of failing."""
    B, S1, S2, G, K = 1, 131072, 131072, 1, 65536
    bf, i32, f32 = 1, 4, 3
    q = lambda: _fake((B, S1, G, 512), bf)
    k = lambda: _fake((B, S2, 1, 512), bf)
    st = lambda: _fake((B, 1, S1, G), f32)
    ws = ctypes.c_uint64(0)
    p = ctypes.c_void_p(None)
    rc = sfag.lib().sfag_workspace_size(q(), k(), k(), _fake((B, S1, 1, K), i32), q(), q(), st(), st(), None, None,
                                        None, None, 0.04, 1, b"BSND", 0, 2147483647, 2147483647, True, q(), k(), k(),
                                        None, None, ctypes.byref(ws), ctypes.byref(p))
    assert rc == 0, sfag.lib().sfag_last_error()
    o = sfag.make_options(dict(scatter="keyblock"))
    assert sfag.lib().sfag_plan_configure(p, ctypes.byref(o), ctypes.byref(ws)) == 0
    sfag.destroy(p)


def test_product_sources_read_no_environment():
    """Every tuning choice is an sfag_options field: the library's sources
    never read the environment."""
    csrc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "top_sparse_attention_sfag_amd",
                        "csrc")
    for f in sorted(os.listdir(csrc)):
        src = open(os.path.join(csrc, f)).read()
        assert "getenv" not in src and "environ" not in src, f


def test_static_entry_rejects_a_plan_larger_than_its_scratch():
    """sfag_backward_static checks the plan's workspace against its scratch
    array before anything is enqueued (no GPU needed), and frees the plan."""
    B, S1, S2, G, K = 1, 2048, 4096, 128, 2048
    bf, i32, f32 = 1, 4, 3
    q = lambda: _fake((B, S1, G, 512), bf)
    k = lambda: _fake((B, S2, 1, 512), bf)
    st = lambda: _fake((B, 1, S1, G), f32)
    ws = ctypes.c_uint64(0)
    p = ctypes.c_void_p(None)
    rc = sfag.lib().sfag_workspace_size(q(), k(), k(), _fake((B, S1, 1, K), i32), q(), q(), st(), st(), None, None,
                                        None, None, 0.04, 1, b"BSND", 3, 2147483647, 2147483647, False, q(), k(), k(),
                                        None, None, ctypes.byref(ws), ctypes.byref(p))
    assert rc == 0 and ws.value > sfag.STATIC_SCRATCH_BYTES
    assert sfag.lib().sfag_backward_static(p, None) == sfag.ERR_PARAM_INVALID
    assert b"scratch" in sfag.lib().sfag_last_error()
    assert sfag.lib().sfag_backward_static(None, None) == sfag.ERR_NULLPTR
