"""ctypes binding of libattn (include/attn.h): argument marshalling only.

PyTorch supplies device memory and the stream; every step of the attention
forward runs in the HIP kernels of libattn.so.  There is no Python or CPU
implementation behind these functions: if the library is not built they
raise.
"""

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

ATTN_OK, ATTN_E_INVALID, ATTN_E_UNSUPPORTED, ATTN_E_WORKSPACE, ATTN_E_LAUNCH = range(5)
# attn_path values (include/attn.h) by name
PATH_NAMES = {0: "none", 1: "prefill_mfma", 2: "decode_split", 3: "per_row", 4: "bwd_mfma",
              5: "bwd_per_row"}
NORMALIZER_IDS = {"softmax": 0, "softmax1": 1, "sparsemax": 2, "entmax15": 3}
_DTYPE_IDS = {torch.float32: 0, torch.bfloat16: 1}
_DTYPE_UNKNOWN = 99


class AttnError(RuntimeError):
    """A non-zero attn_status returned by libattn."""

    def __init__(self, status, detail):
        self.status = status
        self.detail = detail
        super().__init__(f"{attn_strerror(status)} ({detail})")


class _Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class _Paged(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("block_size", ctypes.c_int32), ("max_blocks", ctypes.c_int32)]


class _Varlen(ctypes.Structure):
    _fields_ = [("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
                ("num_seqs", ctypes.c_int32), ("max_seqlen_q", ctypes.c_int32)]


class _BlockMask(ctypes.Structure):
    _fields_ = [("kv_num_blocks", ctypes.c_void_p), ("kv_indices", ctypes.c_void_p),
                ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("max_kv_blocks", ctypes.c_int32)]


class _Params(ctypes.Structure):
    _fields_ = [("normalizer", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("window", ctypes.c_int32), ("softcap", ctypes.c_float),
                ("scaling", ctypes.c_float), ("sinks", ctypes.c_void_p),
                ("block_mask", ctypes.POINTER(_BlockMask))]


_lib = None


def load_library(path=None):
    """Load libattn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"libattn.so not found at {path}: build it first "
                           "(python -m attention_pluggable_normalizers_amd.build)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.attn_fwd.argtypes = [P(_Tensor), P(_Tensor), P(_Tensor), P(_Paged), P(_Params),
                             P(_Tensor), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                             ctypes.c_void_p]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd_varlen.argtypes = [P(_Tensor), P(_Tensor), P(_Tensor), P(_Varlen), P(_Params),
                                    P(_Tensor), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                    ctypes.c_void_p]
    lib.attn_fwd_varlen.restype = ctypes.c_int
    lib.attn_fwd_workspace_bytes.argtypes = [P(_Tensor), P(_Tensor), P(_Tensor), P(_Paged),
                                             P(_Params), P(ctypes.c_size_t)]
    lib.attn_fwd_workspace_bytes.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [P(_Tensor), P(_Tensor), P(_Tensor), P(_Tensor), P(_Tensor),
                             ctypes.c_void_p, P(_Params), P(_Tensor), P(_Tensor), P(_Tensor),
                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd_varlen.argtypes = [P(_Tensor), P(_Tensor), P(_Tensor), P(_Tensor), P(_Tensor),
                                    ctypes.c_void_p, P(_Varlen), P(_Params), P(_Tensor),
                                    P(_Tensor), P(_Tensor), ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_size_t, ctypes.c_void_p]
    lib.attn_bwd_varlen.restype = ctypes.c_int
    lib.attn_bwd_workspace_bytes.argtypes = [P(_Tensor), P(_Tensor), P(_Tensor), P(_Params),
                                             P(ctypes.c_size_t)]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_int
    lib.attn_fwd_noalloc.argtypes = [P(_Tensor), P(_Tensor), P(_Tensor), P(_Paged), P(_Params),
                                     P(_Tensor), ctypes.c_void_p, ctypes.c_void_p]
    lib.attn_fwd_noalloc.restype = ctypes.c_int
    lib.attn_fwd_path.argtypes = [P(_Tensor), P(_Tensor), P(_Tensor), P(_Paged), P(_Params),
                                  P(_Tensor), P(ctypes.c_int)]
    lib.attn_fwd_path.restype = ctypes.c_int
    lib.attn_fwd_varlen_path.argtypes = [P(_Tensor), P(_Tensor), P(_Tensor), P(_Varlen),
                                         P(_Params), P(_Tensor), P(ctypes.c_int)]
    lib.attn_fwd_varlen_path.restype = ctypes.c_int
    lib.attn_bwd_path.argtypes = [P(_Tensor), P(_Tensor), P(_Tensor), P(_Tensor), P(_Tensor),
                                  P(_Params), P(_Tensor), P(_Tensor), P(_Tensor), P(ctypes.c_int)]
    lib.attn_bwd_path.restype = ctypes.c_int
    lib.attn_strerror.argtypes = [ctypes.c_int]
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_last_error_detail.argtypes = []
    lib.attn_last_error_detail.restype = ctypes.c_char_p
    lib.attn_abi_version.argtypes = []
    lib.attn_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def attn_strerror(status):
    return load_library().attn_strerror(int(status)).decode()


def attn_last_error_detail():
    return load_library().attn_last_error_detail().decode()


def attn_abi_version():
    return load_library().attn_abi_version()


def _desc(t):
    if t.dim() != 4:
        raise ValueError("attn tensors are 4-D")
    d = _Tensor()
    d.data = t.data_ptr()
    d.dtype = _DTYPE_IDS.get(t.dtype, _DTYPE_UNKNOWN)
    d.reserved = 0
    for i in range(4):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _block_mask(block_mask):
    """(kv_num_blocks int32 [B, Hm, nqb], kv_indices int32 [B, Hm, nqb, max], block_q,
    block_k) -> the C descriptor (device tensors, contiguous)."""
    num, idx, bq, bk = block_mask
    for t, name, nd in ((num, "kv_num_blocks", 3), (idx, "kv_indices", 4)):
        if (t.dtype != torch.int32 or t.dim() != nd or not t.is_contiguous()
                or t.device.type != "cuda"):
            raise ValueError(f"{name} must be a contiguous int32 device tensor with {nd} dims")
    if tuple(idx.shape[:3]) != tuple(num.shape):
        raise ValueError("kv_indices must be [B, heads, q-blocks, max_kv_blocks] over kv_num_blocks")
    m = _BlockMask()
    m.kv_num_blocks = num.data_ptr()
    m.kv_indices = idx.data_ptr()
    m.block_q, m.block_k = int(bq), int(bk)
    m.num_heads = int(num.shape[1])
    m.max_kv_blocks = int(idx.shape[3])
    return m


def _params(normalizer, causal, window, softcap, scaling, head_dim, sinks=None, num_heads=None,
            block_mask=None):
    p = _Params()
    p.normalizer = NORMALIZER_IDS.get(normalizer, -1) if isinstance(normalizer, str) else int(normalizer)
    p.causal = 1 if causal else 0
    p.window = int(window)
    p.softcap = float(softcap)
    p.scaling = float(1.0 / math.sqrt(head_dim) if scaling is None else scaling)
    if sinks is not None:
        # the library reads Hq float32 values from this device address
        if (sinks.dtype != torch.float32 or sinks.dim() != 1 or sinks.numel() != num_heads
                or not sinks.is_contiguous() or sinks.device.type != "cuda"):
            raise ValueError("sinks must be a contiguous float32 device tensor of shape [Hq]")
        p.sinks = sinks.data_ptr()
    else:
        p.sinks = None
    if block_mask is not None:
        p._bm = _block_mask(block_mask)  # kept alive with the params
        p.block_mask = ctypes.pointer(p._bm)
    return p


def _paged_desc(paged):
    if paged is None:
        return None
    pd = _Paged()
    pd.block_table = paged["block_table"].data_ptr()
    pd.seq_lens = paged["seq_lens"].data_ptr()
    pd.block_size = int(paged["block_size"])
    pd.max_blocks = int(paged["max_blocks"])
    return pd


def _check(status):
    if status != ATTN_OK:
        raise AttnError(status, attn_last_error_detail())


def _on_stream(stream, device, *tensors):
    """The raw stream handle to enqueue on (torch's current stream when
    ``stream`` is None).  Tensors allocated here for the call (outputs,
    workspace) are marked as used by a foreign stream, so torch's caching
    allocator does not hand their memory to other work before the kernels
    on that stream have finished."""
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    ext = torch.cuda.ExternalStream(stream, device=device)
    for t in tensors:
        if t is not None:
            t.record_stream(ext)
    return stream


def attn_fwd_workspace_bytes(q, k, v, *, normalizer, causal=False, window=0, softcap=0.0,
                             scaling=None, paged=None):
    """Workspace bytes ``attn_fwd`` needs for these arguments."""
    lib = load_library()
    n = ctypes.c_size_t(0)
    pd = _paged_desc(paged)
    p = _params(normalizer, causal, window, softcap, scaling, q.shape[-1])
    _check(lib.attn_fwd_workspace_bytes(ctypes.byref(_desc(q)), ctypes.byref(_desc(k)),
                                        ctypes.byref(_desc(v)),
                                        ctypes.byref(pd) if pd is not None else None,
                                        ctypes.byref(p), ctypes.byref(n)))
    return n.value


def attn_fwd_path(q, k, v, out=None, *, normalizer, causal=False, window=0, softcap=0.0,
                  scaling=None, paged=None, sinks=None, block_mask=None):
    """Name of the kernel family ``attn_fwd`` takes for these arguments
    ("prefill_mfma", "decode_split", "per_row" or "none"); nothing runs."""
    lib = load_library()
    if out is None:
        out = q  # same shape, dtype and alignment class as the output attn_fwd allocates
    pd = _paged_desc(paged)
    p = _params(normalizer, causal, window, softcap, scaling, q.shape[-1], sinks, q.shape[1],
                block_mask)
    path = ctypes.c_int(-1)
    _check(lib.attn_fwd_path(ctypes.byref(_desc(q)), ctypes.byref(_desc(k)),
                             ctypes.byref(_desc(v)), ctypes.byref(pd) if pd is not None else None,
                             ctypes.byref(p), ctypes.byref(_desc(out)), ctypes.byref(path)))
    return PATH_NAMES[path.value]


def attn_fwd(q, k, v, out=None, row_stats=None, *, normalizer, causal=False, window=0,
             softcap=0.0, scaling=None, paged=None, workspace=None, stream=None, sinks=None,
             block_mask=None):
    """Enqueue the forward on ``stream`` (default: torch's current stream).

    q [B,Hq,Lq,D]; k, v [B,Hkv,Lk,D], or paged caches [NB,bs,Hkv,D] with
    ``paged = {"block_table", "seq_lens", "block_size", "max_blocks"}``.
    ``out`` (allocated like q when None) and ``row_stats`` (float32
    [B,Hq,Lq,2] or None) receive the results; returns ``(out, row_stats)``.
    ``sinks`` (softmax1 only): float32 device tensor [Hq] of learned sink
    logits, the virtual key's logit per query head (default 0).
    ``block_mask``: ``(kv_num_blocks, kv_indices, block_q, block_k)``, a
    full-block CSR key mask (int32 device tensors [B, 1 or Hq, q-blocks] and
    [B, 1 or Hq, q-blocks, max_kv_blocks] with ascending block indices).
    """
    lib = load_library()
    new_out = None
    if out is None:
        out = new_out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if row_stats is not None and (row_stats.dtype != torch.float32 or not row_stats.is_contiguous()
                                  or tuple(row_stats.shape) != (*q.shape[:3], 2)):
        raise ValueError("row_stats must be a contiguous float32 tensor [B, Hq, Lq, 2]")
    pd = _paged_desc(paged)
    p = _params(normalizer, causal, window, softcap, scaling, q.shape[-1], sinks, q.shape[1],
                block_mask)
    new_ws = None
    if workspace is None:
        nbytes = attn_fwd_workspace_bytes(q, k, v, normalizer=normalizer, causal=causal,
                                          window=window, softcap=softcap, scaling=scaling,
                                          paged=paged)
        workspace = new_ws = (torch.empty(nbytes, dtype=torch.uint8, device=q.device)
                              if nbytes else None)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    stream = _on_stream(stream, q.device, new_out, new_ws)
    st = lib.attn_fwd(ctypes.byref(_desc(q)), ctypes.byref(_desc(k)), ctypes.byref(_desc(v)),
                      ctypes.byref(pd) if pd is not None else None, ctypes.byref(p),
                      ctypes.byref(_desc(out)),
                      row_stats.data_ptr() if row_stats is not None else None,
                      ws_ptr, ws_len, stream)
    _check(st)
    return out, row_stats


def attn_fwd_noalloc(q, k, v, out, row_stats=None, *, normalizer, causal=False, window=0,
                     softcap=0.0, scaling=None, paged=None, stream=None, sinks=None,
                     block_mask=None):
    """``attn_fwd`` without any device allocation: ``out`` must be given, and
    the paged-decode workspace is the library's fixed per-GPU scratch (calls
    that overlap on one GPU race).  Returns ``(out, row_stats)``."""
    lib = load_library()
    if row_stats is not None and (row_stats.dtype != torch.float32 or not row_stats.is_contiguous()
                                  or tuple(row_stats.shape) != (*q.shape[:3], 2)):
        raise ValueError("row_stats must be a contiguous float32 tensor [B, Hq, Lq, 2]")
    pd = _paged_desc(paged)
    p = _params(normalizer, causal, window, softcap, scaling, q.shape[-1], sinks, q.shape[1],
                block_mask)
    stream = _on_stream(stream, q.device)
    _check(lib.attn_fwd_noalloc(ctypes.byref(_desc(q)), ctypes.byref(_desc(k)),
                                ctypes.byref(_desc(v)),
                                ctypes.byref(pd) if pd is not None else None, ctypes.byref(p),
                                ctypes.byref(_desc(out)),
                                row_stats.data_ptr() if row_stats is not None else None, stream))
    return out, row_stats


def _packed_view(t):
    """[tokens, heads, D] -> the [1, heads, tokens, D] view (no copy)."""
    return t.permute(1, 0, 2).unsqueeze(0)


def _varlen_desc(query, key, value, cu_seqlens_q, cu_seqlens_k, max_seqlen_q):
    if query.dim() != 3 or key.dim() != 3 or value.dim() != 3:
        raise ValueError("packed query/key/value are [tokens, heads, head_dim]")
    for t, name in ((cu_seqlens_q, "cu_seqlens_q"), (cu_seqlens_k, "cu_seqlens_k")):
        if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 tensor [num_seqs + 1]")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have num_seqs + 1 entries")
    vl = _Varlen()
    vl.cu_seqlens_q = cu_seqlens_q.data_ptr()
    vl.cu_seqlens_k = cu_seqlens_k.data_ptr()
    vl.num_seqs = cu_seqlens_q.numel() - 1
    vl.max_seqlen_q = int(max_seqlen_q)
    return vl


def attn_fwd_varlen(query, key, value, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, out=None,
                    row_stats=None, *, normalizer, causal=False, window=0, softcap=0.0,
                    scaling=None, stream=None, sinks=None):
    """Packed variable-length forward ("HF Attention Normalizers", "Packed
    Variable-Length Attention").

    query [total_q, Hq, D], key/value [total_k, Hkv, D]; cu_seqlens_q/k int32
    device tensors [num_seqs + 1]; request r attends its own key range with
    bottom-right causal alignment.  ``out`` [total_q, Hq, D] (allocated when
    None) and ``row_stats`` (float32 [Hq, total_q, 2] or None) receive the
    results; returns ``(out, row_stats)``.
    """
    lib = load_library()
    vl = _varlen_desc(query, key, value, cu_seqlens_q, cu_seqlens_k, max_seqlen_q)
    new_out = None
    if out is None:
        out = new_out = torch.empty(query.shape, dtype=query.dtype, device=query.device)
    if row_stats is not None and (row_stats.dtype != torch.float32 or not row_stats.is_contiguous()
                                  or tuple(row_stats.shape) != (query.shape[1], query.shape[0], 2)):
        raise ValueError("row_stats must be a contiguous float32 tensor [Hq, total_q, 2]")
    view = _packed_view
    p = _params(normalizer, causal, window, softcap, scaling, query.shape[-1], sinks, query.shape[1])
    stream = _on_stream(stream, query.device, new_out)
    st = lib.attn_fwd_varlen(ctypes.byref(_desc(view(query))), ctypes.byref(_desc(view(key))),
                             ctypes.byref(_desc(view(value))), ctypes.byref(vl), ctypes.byref(p),
                             ctypes.byref(_desc(view(out))),
                             row_stats.data_ptr() if row_stats is not None else None,
                             None, 0, stream)
    _check(st)
    return out, row_stats


def attn_bwd_path(q, k, v, dout, *, normalizer, causal=False, window=0, softcap=0.0,
                  scaling=None, sinks=None, dq=None, dk=None, dv=None, out=None,
                  block_mask=None):
    """Name of the kernel family ``attn_bwd`` takes ("bwd_mfma", "bwd_per_row"
    or "none"); gradients default to tensors laid out like q, k, v."""
    lib = load_library()
    p = _params(normalizer, causal, window, softcap, scaling, q.shape[-1], sinks, q.shape[1],
                block_mask)
    path = ctypes.c_int(-1)
    od = ctypes.byref(_desc(out)) if out is not None else None
    _check(lib.attn_bwd_path(ctypes.byref(_desc(q)), ctypes.byref(_desc(k)),
                             ctypes.byref(_desc(v)), od, ctypes.byref(_desc(dout)),
                             ctypes.byref(p), ctypes.byref(_desc(q if dq is None else dq)),
                             ctypes.byref(_desc(k if dk is None else dk)),
                             ctypes.byref(_desc(v if dv is None else dv)), ctypes.byref(path)))
    return PATH_NAMES[path.value]


def attn_bwd(q, k, v, dout, row_stats, *, normalizer, causal=False, window=0, softcap=0.0,
             scaling=None, sinks=None, dq=None, dk=None, dv=None, sink_grad=False, out=None,
             stream=None, block_mask=None):
    """Gradients of ``attn_fwd`` for the same q, k, v and parameters, given the
    forward's ``row_stats`` and the upstream gradient ``dout``: returns
    ``(dq, dk, dv, dsinks)`` (``dsinks`` float32 [Hq] when ``sink_grad``,
    softmax1 only, else None).  ``out`` (optional): the forward's output; the
    softmax family then takes its row constant from dout . out (one pass
    fewer).  ``block_mask``: the forward's (kv_num_blocks, kv_indices,
    block_q, block_k)."""
    lib = load_library()
    if (row_stats is None or row_stats.dtype != torch.float32 or not row_stats.is_contiguous()
            or tuple(row_stats.shape) != (*q.shape[:3], 2)):
        raise ValueError("row_stats must be the forward's float32 [B, Hq, Lq, 2]")
    fresh = []

    def alloc(shape, dtype):
        t = torch.empty(shape, dtype=dtype, device=q.device)
        fresh.append(t)
        return t
    dq = alloc(q.shape, q.dtype) if dq is None else dq
    dk = alloc(k.shape, k.dtype) if dk is None else dk
    dv = alloc(v.shape, v.dtype) if dv is None else dv
    ds = alloc(q.shape[1], torch.float32) if sink_grad else None
    p = _params(normalizer, causal, window, softcap, scaling, q.shape[-1], sinks, q.shape[1],
                block_mask)
    qd, kd, vd = _desc(q), _desc(k), _desc(v)
    n = ctypes.c_size_t(0)
    _check(lib.attn_bwd_workspace_bytes(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd),
                                        ctypes.byref(p), ctypes.byref(n)))
    ws = alloc(max(n.value, 1), torch.uint8)
    stream = _on_stream(stream, q.device, *fresh)
    od = ctypes.byref(_desc(out)) if out is not None else None
    _check(lib.attn_bwd(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd), od,
                        ctypes.byref(_desc(dout)), row_stats.data_ptr(), ctypes.byref(p),
                        ctypes.byref(_desc(dq)), ctypes.byref(_desc(dk)), ctypes.byref(_desc(dv)),
                        ds.data_ptr() if ds is not None else None, ws.data_ptr(), n.value,
                        stream))
    return dq, dk, dv, ds


def attn_bwd_varlen(query, key, value, dout, row_stats, cu_seqlens_q, cu_seqlens_k,
                    max_seqlen_q, *, normalizer, causal=False, window=0, softcap=0.0,
                    scaling=None, sinks=None, dq=None, dk=None, dv=None, sink_grad=False,
                    out=None, stream=None):
    """Gradients of ``attn_fwd_varlen`` ("HF Attention Normalizers", "Packed
    Variable-Length Attention"): query, dout [total_q, Hq, D], key, value
    [total_k, Hkv, D], row_stats the forward's float32 [Hq, total_q, 2].
    Returns ``(dq, dk, dv, dsinks)`` in the packed layouts; tokens outside
    every request get zeros."""
    lib = load_library()
    vl = _varlen_desc(query, key, value, cu_seqlens_q, cu_seqlens_k, max_seqlen_q)
    if (row_stats is None or row_stats.dtype != torch.float32 or not row_stats.is_contiguous()
            or tuple(row_stats.shape) != (query.shape[1], query.shape[0], 2)):
        raise ValueError("row_stats must be the forward's float32 [Hq, total_q, 2]")
    fresh = []

    def alloc(shape, dtype):
        t = torch.empty(shape, dtype=dtype, device=query.device)
        fresh.append(t)
        return t
    dq = alloc(query.shape, query.dtype) if dq is None else dq
    dk = alloc(key.shape, key.dtype) if dk is None else dk
    dv = alloc(value.shape, value.dtype) if dv is None else dv
    ds = alloc(query.shape[1], torch.float32) if sink_grad else None
    p = _params(normalizer, causal, window, softcap, scaling, query.shape[-1], sinks,
                query.shape[1])
    view = _packed_view
    qd, kd, vd = _desc(view(query)), _desc(view(key)), _desc(view(value))
    n = ctypes.c_size_t(0)
    _check(lib.attn_bwd_workspace_bytes(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd),
                                        ctypes.byref(p), ctypes.byref(n)))
    ws = alloc(max(n.value, 1), torch.uint8)
    stream = _on_stream(stream, query.device, *fresh)
    od = ctypes.byref(_desc(view(out))) if out is not None else None
    _check(lib.attn_bwd_varlen(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd), od,
                               ctypes.byref(_desc(view(dout))), row_stats.data_ptr(),
                               ctypes.byref(vl), ctypes.byref(p), ctypes.byref(_desc(view(dq))),
                               ctypes.byref(_desc(view(dk))), ctypes.byref(_desc(view(dv))),
                               ds.data_ptr() if ds is not None else None, ws.data_ptr(), n.value,
                               stream))
    return dq, dk, dv, ds


def custom_attention(module, query, key, value, attention_mask, *, normalizer, dropout=0.0,
                     scaling=None, is_causal=True, sliding_window=0, softcap=0.0,
                     output_attentions=False, sinks=None, **kwargs):
    """The custom-attention signature of the transformers attention interface.

    ("attention interface", "custom attention registration": the function
    receives the module, query, key, value and attention_mask and returns
    ``(attn_output, attn_weights)``; "Attention" (factory.ai), "What every
    backend must support".)  query [B,Hq,L,D], key/value [B,Hkv,Lk,D] (GQA
    handled natively).  Only structured masks are supported, so a dense
    ``attention_mask`` is rejected, as are dropout and returned weights.
    ``sinks`` (softmax1): per-head learned sink logits, float32 [Hq].
    Returns ``(out [B, L, Hq, D], None)``.
    """
    if attention_mask is not None:
        raise AttnError(ATTN_E_UNSUPPORTED, "dense attention_mask; use is_causal/sliding_window")
    if dropout:
        raise AttnError(ATTN_E_UNSUPPORTED, "dropout is not part of this forward")
    if output_attentions:
        raise AttnError(ATTN_E_UNSUPPORTED, "attention weights are never materialized")
    out, _ = attn_fwd(query, key, value, normalizer=normalizer, causal=is_causal,
                      window=sliding_window or 0, softcap=softcap or 0.0, scaling=scaling,
                      sinks=sinks)
    return out.transpose(1, 2).contiguous(), None
