"""ctypes binding of libsfag (argument marshalling only: every step of the
backward pass runs in the library's HIP kernels).

PyTorch provides the device memory (outputs and workspace) and the stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libsfag.so")

OK = 0
ERR_NULLPTR = 161001
ERR_PARAM_INVALID = 161002
ERR_RUNTIME = 361001
ERR_TILING = 561002

_DTYPE = {torch.bfloat16: 1, torch.float16: 2, torch.float32: 3, torch.int32: 4}
WINDOW = 2147483647


class SfagTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class SfagOptions(ctypes.Structure):
    _fields_ = [("workspaceBudget", ctypes.c_uint64), ("chunkTokens", ctypes.c_int64), ("scatter", ctypes.c_int32),
                ("tokenPath", ctypes.c_int32), ("tokenOrder", ctypes.c_int32), ("concurrent", ctypes.c_int32),
                ("rowSplit", ctypes.c_int32), ("keyBlockRanges", ctypes.c_int32), ("validate", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("auxStream", ctypes.c_void_p)]


class SfagValidation(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_uint32), ("reserved", ctypes.c_uint32), ("badEntries", ctypes.c_uint64)]


# Names of the sfag_options values (include/sfag.h).
SCATTER = {"auto": 0, "keyblock": 1, "partials": 2, "atomic": 3}
TOKEN_PATH = {"auto": 0, "fused": 1, "split": 2}
TOKEN_ORDER = {"auto": 0, "ascending": 1, "descending": 2}
CONCURRENT = {"auto": 0, "off": 1, "on": 2}
BAD_LENGTH_NEGATIVE, BAD_LENGTH_SUM_Q, BAD_LENGTH_SUM_KV, BAD_INDEX_RANGE = 1, 2, 4, 8


def make_options(options=None):
    """sfag_options from a dict with keys workspace_budget (bytes),
    chunk_tokens, scatter, token_path, token_order, concurrent, row_split,
    key_block_ranges, validate and aux_stream (a torch.cuda.Stream); None when
    ``options`` is None or empty."""
    if not options:
        return None
    known = {"workspace_budget", "chunk_tokens", "scatter", "token_path", "token_order", "concurrent", "row_split",
             "key_block_ranges", "validate", "aux_stream"}
    bad = set(options) - known
    if bad:
        raise SfagValueError(ERR_PARAM_INVALID, f"unknown options {sorted(bad)}")
    o = SfagOptions()
    o.workspaceBudget = int(options.get("workspace_budget", 0))
    o.chunkTokens = int(options.get("chunk_tokens", 0))
    o.scatter = SCATTER[options.get("scatter", "auto")]
    o.tokenPath = TOKEN_PATH[options.get("token_path", "auto")]
    o.tokenOrder = TOKEN_ORDER[options.get("token_order", "auto")]
    o.concurrent = CONCURRENT[options.get("concurrent", "auto")]
    o.rowSplit = int(options.get("row_split", 0))
    o.keyBlockRanges = int(options.get("key_block_ranges", 0))
    o.validate = 1 if options.get("validate", False) else 0
    aux = options.get("aux_stream")
    o.auxStream = aux.cuda_stream if aux is not None else None
    return o


class SfagError(Exception):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libsfag error {code}: {msg}")
        self.code = code


class SfagValueError(SfagError, ValueError):
    pass


class SfagRuntimeError(SfagError, RuntimeError):
    pass


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(or python top_sparse_attention_sfag_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        T = ctypes.POINTER(SfagTensor)
        L.sfag_workspace_size.restype = ctypes.c_int
        L.sfag_workspace_size.argtypes = [T] * 12 + [ctypes.c_double, ctypes.c_int64, ctypes.c_char_p, ctypes.c_int64,
                                                     ctypes.c_int64, ctypes.c_int64, ctypes.c_bool] + [T] * 5 + [
            ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_void_p)]
        L.sfag_backward.restype = ctypes.c_int
        L.sfag_backward.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
        L.sfag_forward_workspace_size.restype = ctypes.c_int
        L.sfag_forward_workspace_size.argtypes = [T] * 8 + [ctypes.c_double, ctypes.c_int64, ctypes.c_char_p,
                                                           ctypes.c_int64] + [T] * 3 + [
            ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_void_p)]
        L.sfag_forward.restype = ctypes.c_int
        L.sfag_forward.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
        L.sfag_backward_static.restype = ctypes.c_int
        L.sfag_backward_static.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.sfag_plan_configure.restype = ctypes.c_int
        L.sfag_plan_configure.argtypes = [ctypes.c_void_p, ctypes.POINTER(SfagOptions), ctypes.POINTER(ctypes.c_uint64)]
        L.sfag_validation_read.restype = ctypes.c_int
        L.sfag_validation_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(SfagValidation)]
        L.sfag_plan_destroy.restype = None
        L.sfag_plan_destroy.argtypes = [ctypes.c_void_p]
        L.sfag_last_error.restype = ctypes.c_char_p
        L.sfag_last_error.argtypes = []
        L.sfag_index_workspace_size.restype = ctypes.c_uint64
        L.sfag_index_workspace_size.argtypes = [ctypes.c_int64] * 4
        L.sfag_build_index.restype = ctypes.c_int
        L.sfag_build_index.argtypes = ([ctypes.c_void_p] * 3 + [ctypes.c_int64] * 7 + [ctypes.c_int32, ctypes.c_int64]
                                       + [ctypes.c_void_p, ctypes.c_uint64] + [ctypes.c_void_p] * 5)
        L.sfag_band_entries.restype = ctypes.c_int64
        L.sfag_band_entries.argtypes = [ctypes.c_int64] * 4
        L.sfag_band_indices.restype = ctypes.c_int
        L.sfag_band_indices.argtypes = ([ctypes.c_void_p] * 3 + [ctypes.c_int64] * 6 + [ctypes.c_int32]
                                        + [ctypes.c_int64] * 2 + [ctypes.c_void_p])
        L.sfag_profile_enable.restype = None
        L.sfag_profile_enable.argtypes = [ctypes.c_int]
        L.sfag_profile_reset.restype = None
        L.sfag_profile_reset.argtypes = []
        L.sfag_profile_read.restype = ctypes.c_int
        L.sfag_profile_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int64)]
        _lib = L
    return _lib


KERNEL_GROUPS = ("seq_offsets", "delta", "fill", "decode", "row", "sdp", "dq", "col", "csr", "key_reduce", "kb_sort",
                 "keyblock", "kb_reduce", "cast", "fwd")


def profile_enable(on: bool = True):
    lib().sfag_profile_enable(1 if on else 0)


def profile_reset():
    lib().sfag_profile_reset()


def profile_read():
    """{kernel group: (total ms, launches)} since the last reset."""
    out = {}
    for n in KERNEL_GROUPS:
        ms, cnt = ctypes.c_double(0), ctypes.c_int64(0)
        lib().sfag_profile_read(n.encode(), ctypes.byref(ms), ctypes.byref(cnt))
        if cnt.value:
            out[n] = (ms.value, cnt.value)
    return out


def _desc(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if t.dim() > 4:
        raise SfagValueError(ERR_PARAM_INVALID, "tensors have at most 4 dims")
    d = SfagTensor()
    d.data = t.data_ptr() if t.numel() > 0 else None
    d.dtype = _DTYPE.get(t.dtype, 0)
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return ctypes.pointer(d)


def _raise(code: int):
    msg = lib().sfag_last_error().decode()
    if code == ERR_RUNTIME:
        raise SfagRuntimeError(code, msg)
    raise SfagValueError(code, msg)


def plan(query, key, value, sparse_indices, dout, out, softmax_max, softmax_sum, dq, dk, dv, *, dq_rope=None,
         dk_rope=None, seqlens_q=None, seqlens_kv=None, query_rope=None, key_rope=None, scale=None, block_size=1,
         layout: Optional[str] = "BSND", sparse_mode=0, pre_tokens=WINDOW, next_tokens=WINDOW, deterministic=False,
         options=None):
    """Phase 1: returns (workspace bytes, plan handle).  Reads no tensor data.
    ``options`` (see make_options) re-plans with sfag_plan_configure."""
    if scale is None and query is not None:
        scale = 1.0 / (query.shape[-1] + (query_rope.shape[-1] if query_rope is not None else 0)) ** 0.5
    if scale is None:
        scale = 1.0
    ws = ctypes.c_uint64(0)
    p = ctypes.c_void_p(None)
    rc = lib().sfag_workspace_size(
        _desc(query), _desc(key), _desc(value), _desc(sparse_indices), _desc(dout), _desc(out), _desc(softmax_max),
        _desc(softmax_sum), _desc(seqlens_q), _desc(seqlens_kv), _desc(query_rope), _desc(key_rope), float(scale),
        int(block_size), None if layout is None else layout.encode(), int(sparse_mode), int(pre_tokens),
        int(next_tokens), bool(deterministic), _desc(dq), _desc(dk), _desc(dv), _desc(dq_rope), _desc(dk_rope),
        ctypes.byref(ws), ctypes.byref(p))
    if rc != OK:
        _raise(rc)
    return _configure(p, ws, options), p


def _configure(p, ws, options):
    o = make_options(options)
    if o is not None:
        rc = lib().sfag_plan_configure(p, ctypes.byref(o), ctypes.byref(ws))
        if rc != OK:
            destroy(p)
            _raise(rc)
    return int(ws.value)


def destroy(p):
    lib().sfag_plan_destroy(p)


def _stream_ptr(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def backward(query, key, value, sparse_indices, dout, out, softmax_max, softmax_sum, *, seqlens_q=None,
             seqlens_kv=None, query_rope=None, key_rope=None, scale=None, block_size=1, layout="BSND", sparse_mode=0,
             pre_tokens=WINDOW, next_tokens=WINDOW, deterministic=False, outputs=None, workspace=None, stream=None,
             options=None):
    """Backward pass of top-k sparse flash attention on the GPU.

    Returns (dq, dk, dv, dq_rope, dk_rope); the rope gradients are None without
    rope inputs.  ``outputs`` may supply preallocated gradients and
    ``workspace`` a uint8 device buffer of at least the planned size; what is
    allocated here is allocated on the stream the kernels run on.
    ``options``: tuning choices (see make_options).
    """
    if not query.is_cuda:
        raise SfagValueError(ERR_PARAM_INVALID, "tensors must be on the GPU")
    s = stream if stream is not None else torch.cuda.current_stream(query.device)
    with torch.cuda.stream(s):
        if outputs is None:
            dq, dk, dv = torch.empty_like(query), torch.empty_like(key), torch.empty_like(value)
            dqr = torch.empty_like(query_rope) if query_rope is not None else None
            dkr = torch.empty_like(key_rope) if key_rope is not None else None
        else:
            dq, dk, dv, dqr, dkr = outputs
        ws, p = plan(query, key, value, sparse_indices, dout, out, softmax_max, softmax_sum, dq, dk, dv, dq_rope=dqr,
                     dk_rope=dkr, seqlens_q=seqlens_q, seqlens_kv=seqlens_kv, query_rope=query_rope,
                     key_rope=key_rope, scale=scale, block_size=block_size, layout=layout, sparse_mode=sparse_mode,
                     pre_tokens=pre_tokens, next_tokens=next_tokens, deterministic=deterministic, options=options)
        if workspace is None or workspace.numel() < ws:
            workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=query.device)
    rc = lib().sfag_backward(ctypes.c_void_p(workspace.data_ptr()), ctypes.c_uint64(workspace.numel()), p,
                             ctypes.c_void_p(s.cuda_stream))
    if rc != OK:
        _raise(rc)
    return dq, dk, dv, dqr, dkr


STATIC_SCRATCH_BYTES = 256 << 20   # SFAG_STATIC_SCRATCH_BYTES


def backward_static(query, key, value, sparse_indices, dout, out, softmax_max, softmax_sum, outputs, *,
                    seqlens_q=None, seqlens_kv=None, query_rope=None, key_rope=None, scale=None, block_size=1,
                    layout="BSND", sparse_mode=0, deterministic=False, stream=None, options=None):
    """sfag_backward_static: the backward pass with the library's own scratch
    array as workspace (nothing is allocated; ``outputs`` = (dq, dk, dv,
    dq_rope, dk_rope) must be given).  The plan is made with
    workspace_budget = STATIC_SCRATCH_BYTES unless ``options`` sets one."""
    if not query.is_cuda:
        raise SfagValueError(ERR_PARAM_INVALID, "tensors must be on the GPU")
    dq, dk, dv, dqr, dkr = outputs
    opts = dict(options or {})
    opts.setdefault("workspace_budget", STATIC_SCRATCH_BYTES)
    _ws, p = plan(query, key, value, sparse_indices, dout, out, softmax_max, softmax_sum, dq, dk, dv, dq_rope=dqr,
                  dk_rope=dkr, seqlens_q=seqlens_q, seqlens_kv=seqlens_kv, query_rope=query_rope, key_rope=key_rope,
                  scale=scale, block_size=block_size, layout=layout, sparse_mode=sparse_mode,
                  deterministic=deterministic, options=opts)
    s = stream if stream is not None else torch.cuda.current_stream(query.device)
    rc = lib().sfag_backward_static(p, ctypes.c_void_p(s.cuda_stream))
    if rc != OK:
        _raise(rc)
    return dq, dk, dv, dqr, dkr


def validation_read(workspace, stream=None):
    """Result of the device-side input checks of a finished call planned with
    options={"validate": True}: dict(flags=..., bad_entries=...).  Waits for
    ``stream`` (default: the current stream)."""
    s = stream if stream is not None else torch.cuda.current_stream(workspace.device)
    v = SfagValidation()
    rc = lib().sfag_validation_read(ctypes.c_void_p(workspace.data_ptr()), ctypes.c_void_p(s.cuda_stream),
                                    ctypes.byref(v))
    if rc != OK:
        _raise(rc)
    return dict(flags=int(v.flags), bad_entries=int(v.badEntries))


def forward(query, key, value, sparse_indices, *, seqlens_q=None, seqlens_kv=None, query_rope=None, key_rope=None,
            scale=None, block_size=1, layout="BSND", sparse_mode=0, outputs=None, workspace=None, stream=None,
            options=None):
    """Forward pass on the GPU: returns (out, softmax_max, softmax_sum), the
    inputs the backward pass takes from the forward.  ``outputs`` may supply
    preallocated tensors of those shapes."""
    if not query.is_cuda:
        raise SfagValueError(ERR_PARAM_INVALID, "tensors must be on the GPU")
    if scale is None:
        scale = 1.0 / (query.shape[-1] + (query_rope.shape[-1] if query_rope is not None else 0)) ** 0.5
    s = stream if stream is not None else torch.cuda.current_stream(query.device)
    with torch.cuda.stream(s):
        if outputs is None:
            G = query.shape[-2]
            stats = (1, query.shape[0], G) if layout == "TND" else (query.shape[0], 1, query.shape[1], G)
            out = torch.empty_like(query)
            smax = torch.empty(stats, dtype=torch.float32, device=query.device)
            ssum = torch.empty(stats, dtype=torch.float32, device=query.device)
        else:
            out, smax, ssum = outputs
        ws = ctypes.c_uint64(0)
        p = ctypes.c_void_p(None)
        rc = lib().sfag_forward_workspace_size(
            _desc(query), _desc(key), _desc(value), _desc(sparse_indices), _desc(seqlens_q), _desc(seqlens_kv),
            _desc(query_rope), _desc(key_rope), float(scale), int(block_size),
            None if layout is None else layout.encode(), int(sparse_mode), _desc(out), _desc(smax), _desc(ssum),
            ctypes.byref(ws), ctypes.byref(p))
        if rc != OK:
            _raise(rc)
        ws = _configure(p, ws, options)
        if workspace is None or workspace.numel() < ws:
            workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=query.device)
    rc = lib().sfag_forward(ctypes.c_void_p(workspace.data_ptr()), ctypes.c_uint64(workspace.numel()), p,
                            ctypes.c_void_p(s.cuda_stream))
    if rc != OK:
        _raise(rc)
    return out, smax, ssum


def workspace_size(*args, **kw) -> int:
    ws, p = plan(*args, **kw)
    destroy(p)
    return ws


def build_index(sparse_indices, *, T2, block_size=1, layout="BSND", sparse_mode=0, B=None, S1=None, S2=None,
                seqlens_q=None, seqlens_kv=None, stream=None):
    """Index decode and key -> (token, position) CSR on the GPU.

    Returns (n_valid (T1,), rows (T1, K*block), csr_offsets (T2+1,),
    csr_pairs (T1*K*block,)) as int32 device tensors; see sfag_build_index.
    """
    dev = sparse_indices.device
    K = sparse_indices.shape[-1]
    T1 = sparse_indices.numel() // max(K, 1) if K else sparse_indices.shape[0]
    lay = 0 if layout == "BSND" else 1
    if lay == 0:
        B = B if B is not None else sparse_indices.shape[0]
        S1 = S1 if S1 is not None else sparse_indices.shape[1]
        S2 = S2 if S2 is not None else T2 // max(B, 1)
    else:
        B = seqlens_q.numel()
        S1 = S2 = 0
    E = K * block_size
    n_valid = torch.empty(T1, dtype=torch.int32, device=dev)
    rows = torch.empty((T1, E), dtype=torch.int32, device=dev)
    off = torch.empty(T2 + 1, dtype=torch.int32, device=dev)
    pairs = torch.empty(max(T1 * E, 1), dtype=torch.int32, device=dev)
    wsz = lib().sfag_index_workspace_size(T1, T2, K, block_size)
    ws = torch.empty(max(int(wsz), 1), dtype=torch.uint8, device=dev)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(None)
    rc = lib().sfag_build_index(ptr(sparse_indices), ptr(seqlens_q), ptr(seqlens_kv), B, S1, S2, T1, T2, K,
                                block_size, lay, sparse_mode, ptr(ws), ctypes.c_uint64(ws.numel()), ptr(n_valid),
                                ptr(rows), ptr(off), ptr(pairs), _stream_ptr(dev, stream))
    if rc != OK:
        _raise(rc)
    return n_valid, rows, off, pairs[: T1 * E]


def band_entries(max_key_len, pre_tokens, next_tokens, block_size=1):
    """Index entries per row that keep every block of a band (sfag_band_entries)."""
    return int(lib().sfag_band_entries(max_key_len, pre_tokens, next_tokens, block_size))


def band_indices(*, pre_tokens, next_tokens, block_size=1, layout="BSND", B=1, S1=None, S2=None, seqlens_q=None,
                 seqlens_kv=None, K=None, device="cuda", stream=None):
    """Sparse index rows of a band (sliding-window or dense) selection, made on
    the GPU by sfag_band_indices.  Returns int32 (B, S1, 1, K) for BSND or
    (T1, 1, K) for TND; K defaults to band_entries over the longest key
    sequence."""
    lay = 0 if layout == "BSND" else 1
    if lay == 0:
        T1, max_lk = B * S1, S2
    else:
        B = seqlens_q.numel()
        T1 = int(seqlens_q.clamp(min=0).sum().item())
        max_lk = int(seqlens_kv.max().item()) if seqlens_kv.numel() else 0
        S1 = S2 = 0
    if K is None:
        K = band_entries(max_lk, pre_tokens, next_tokens, block_size)
    dev = torch.device(device) if seqlens_q is None else seqlens_q.device
    shape = (B, S1, 1, K) if lay == 0 else (T1, 1, K)
    idx = torch.empty(shape, dtype=torch.int32, device=dev)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(None)
    rc = lib().sfag_band_indices(ptr(idx), ptr(seqlens_q), ptr(seqlens_kv), B, S1 or 0, S2 or 0, T1, K, block_size,
                                 lay, pre_tokens, next_tokens, _stream_ptr(dev, stream))
    if rc != OK:
        _raise(rc)
    return idx
