"""The C ABI library: it loads, exports what include/attn.h declares, and
rejects invalid arguments before touching the GPU (host-side checks only)."""

import ctypes
import os
import re

import pytest
import torch

import attention_pluggable_normalizers_amd as apn
from attention_pluggable_normalizers_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libattn.so is not built (python -m attention_pluggable_normalizers_amd.build)")
    return B.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert names == sorted(["attn_fwd", "attn_fwd_varlen", "attn_fwd_workspace_bytes", "attn_strerror",
                            "attn_last_error_detail", "attn_abi_version", "attn_bwd",
                            "attn_bwd_workspace_bytes", "attn_fwd_path", "attn_fwd_varlen_path",
                            "attn_bwd_path", "attn_fwd_noalloc", "attn_bwd_varlen"])
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strerror(lib):
    assert apn.attn_abi_version() == 8
    for code in range(5):
        assert apn.attn_strerror(code).startswith("ATTN_")
    assert "unknown" in apn.attn_strerror(77)


# fake device pointers: validation never dereferences them
def _t(shape, dtype=torch.bfloat16, strides=None):
    d = B._Tensor()
    d.data = 0x1000
    d.dtype = B._DTYPE_IDS.get(dtype, 99)
    d.reserved = 0
    if strides is None:
        strides = [0] * 4
        acc = 1
        for i in (3, 2, 1, 0):
            strides[i] = acc
            acc *= shape[i]
    for i in range(4):
        d.shape[i] = shape[i]
        d.stride[i] = strides[i]
    return d


def _p(norm=0, causal=1, window=0, softcap=0.0, scaling=0.125):
    p = B._Params()
    p.normalizer, p.causal, p.window, p.softcap, p.scaling = norm, causal, window, softcap, scaling
    return p


def _call(lib, q, k, v, p, out=None, paged=None, ws=0, wsp=None):
    out = out or q
    r = lib.attn_fwd(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                     ctypes.byref(paged) if paged else None, ctypes.byref(p), ctypes.byref(out),
                     None, wsp, ws, None)
    return r, apn.attn_last_error_detail()


Q = (2, 8, 64, 64)
KV = (2, 2, 64, 64)


@pytest.mark.parametrize("mutate,code,needle", [
    (lambda a: a["p"].__setattr__("normalizer", 7), 1, "normalizer"),
    (lambda a: a["p"].__setattr__("causal", 2), 1, "causal"),
    (lambda a: a["p"].__setattr__("window", -1), 1, "window"),
    (lambda a: (a["p"].__setattr__("window", 4), a["p"].__setattr__("causal", 0)), 1, "causal"),
    (lambda a: a["p"].__setattr__("softcap", -1.0), 1, "softcap"),
    (lambda a: a["p"].__setattr__("softcap", float("inf")), 1, "softcap"),
    (lambda a: a["p"].__setattr__("scaling", float("nan")), 1, "scaling"),
    (lambda a: a.__setitem__("k", _t((2, 3, 64, 64))), 1, "k and v"),
    (lambda a: (a.__setitem__("k", _t((2, 3, 64, 64))), a.__setitem__("v", _t((2, 3, 64, 64)))),
     1, "multiple"),
    (lambda a: a.__setitem__("v", _t((2, 2, 64, 32))), 1, "head dim"),
    (lambda a: a.__setitem__("k", _t((1, 2, 64, 64))), 1, "batch"),
    (lambda a: a.__setitem__("k", _t(KV, torch.float32)), 1, "dtype"),
    (lambda a: a.__setitem__("q", _t(Q, torch.float16)), 2, "dtype"),
    (lambda a: a.__setitem__("q", _t((2, 8, 64, 512))), 1, "head dim"),
    (lambda a: a.__setitem__("out", _t((2, 8, 63, 64))), 1, "out shape"),
    (lambda a: a.__setitem__("q", _t(Q, strides=[8 * 64 * 128, 64 * 128, 128, 2])), 1,
     "contiguous"),
    (lambda a: a["q"].__setattr__("data", 0), 1, "NULL"),
    (lambda a: a["q"].__setattr__("reserved", 3), 1, "reserved"),
    (lambda a: a["p"].__setattr__("sinks", 0x4000), 1, "softmax1"),  # sinks with softmax
    (lambda a: (a["p"].__setattr__("sinks", 0x4000), a["p"].__setattr__("normalizer", 3)), 1,
     "softmax1"),
])
def test_invalid_arguments_rejected(lib, mutate, code, needle):
    a = {"q": _t(Q), "k": _t(KV), "v": _t(KV), "p": _p(), "out": _t(Q)}
    mutate(a)
    r, detail = _call(lib, a["q"], a["k"], a["v"], a["p"], a["out"])
    assert r == code, detail
    assert needle in detail


def test_head_dim_256_bf16_ok_for_sizes(lib):
    n = ctypes.c_size_t(123)
    r = lib.attn_fwd_workspace_bytes(ctypes.byref(_t((1, 16, 8, 256))),
                                     ctypes.byref(_t((1, 8, 8, 256))),
                                     ctypes.byref(_t((1, 8, 8, 256))), None,
                                     ctypes.byref(_p()), ctypes.byref(n))
    assert r == 0 and n.value == 0


def test_null_params_and_bytes(lib):
    r = lib.attn_fwd(ctypes.byref(_t(Q)), ctypes.byref(_t(KV)), ctypes.byref(_t(KV)), None, None,
                     ctypes.byref(_t(Q)), None, None, 0, None)
    assert r == 1
    r = lib.attn_fwd_workspace_bytes(ctypes.byref(_t(Q)), ctypes.byref(_t(KV)),
                                     ctypes.byref(_t(KV)), None, ctypes.byref(_p()), None)
    assert r == 1


def _paged(bs=16, max_blocks=8, table=0x2000, lens=0x3000):
    pd = B._Paged()
    pd.block_table, pd.seq_lens, pd.block_size, pd.max_blocks = table, lens, bs, max_blocks
    return pd


def test_paged_validation(lib):
    q = _t((4, 32, 1, 128))
    cache = _t((100, 16, 8, 128))
    r, d = _call(lib, q, cache, cache, _p(), paged=_paged(bs=32))
    assert r == 1 and "block_size" in d
    r, d = _call(lib, q, cache, cache, _p(), paged=_paged(table=0))
    assert r == 1 and "NULL" in d
    r, d = _call(lib, q, cache, cache, _p(), paged=_paged(max_blocks=0))
    assert r == 1 and "max_blocks" in d
    r, d = _call(lib, q, cache, _t((100, 16, 4, 128)), _p(), paged=_paged())
    assert r == 1


def test_workspace_query_needs_no_device(lib):
    # a pure host computation: works in a process without a GPU
    n = ctypes.c_size_t(7)
    q = _t((4, 32, 1, 128))
    cache = _t((100, 16, 8, 128))
    pd = _paged(table=0, lens=0)
    r = lib.attn_fwd_workspace_bytes(ctypes.byref(q), ctypes.byref(cache), ctypes.byref(cache),
                                     ctypes.byref(pd), ctypes.byref(_p(norm=2)), ctypes.byref(n))
    assert r == 0
    assert n.value >= 0


def test_python_wrapper_rejects_dense_mask_and_dropout():
    q = torch.zeros(1, 2, 4, 16)
    with pytest.raises(apn.AttnError):
        apn.custom_attention(None, q, q, q, torch.ones(4, 4, dtype=torch.bool), normalizer="softmax")
    with pytest.raises(apn.AttnError):
        apn.custom_attention(None, q, q, q, None, normalizer="softmax", dropout=0.1)
    with pytest.raises(apn.AttnError):
        apn.custom_attention(None, q, q, q, None, normalizer="softmax", output_attentions=True)


def test_varlen_validation(lib):
    q = _t((1, 8, 100, 64))
    kv = _t((1, 2, 120, 64))
    vl = B._Varlen()
    vl.cu_seqlens_q, vl.cu_seqlens_k, vl.num_seqs, vl.max_seqlen_q = 0x5000, 0x6000, 3, 50
    call = lambda q_, kv_, v_: (lib.attn_fwd_varlen(ctypes.byref(q_), ctypes.byref(kv_),
                                                    ctypes.byref(kv_), v_, ctypes.byref(_p()),
                                                    ctypes.byref(q_), None, None, 0, None),
                                apn.attn_last_error_detail())
    r, d = call(q, kv, None)
    assert r == 1 and "varlen" in d
    r, d = call(_t((2, 8, 100, 64)), _t((2, 2, 120, 64)), ctypes.byref(vl))
    assert r == 1 and "batch extent 1" in d
    vl.num_seqs = -1
    r, d = call(q, kv, ctypes.byref(vl))
    assert r == 1 and "num_seqs" in d
    vl.num_seqs, vl.cu_seqlens_k = 3, 0
    r, d = call(q, kv, ctypes.byref(vl))
    assert r == 1 and "NULL" in d


def _bm(bq=128, bk=128, heads=1, maxb=4, num=0x7000, idx=0x8000):
    m = B._BlockMask()
    m.kv_num_blocks, m.kv_indices = num, idx
    m.block_q, m.block_k, m.num_heads, m.max_kv_blocks = bq, bk, heads, maxb
    return m


@pytest.mark.parametrize("kw,code,needle", [
    (dict(bq=0), 1, "block sizes"),
    (dict(bk=-1), 1, "block sizes"),
    (dict(heads=3), 1, "num_heads"),
    (dict(maxb=-2), 1, "max_kv_blocks"),
    (dict(num=0), 1, "NULL"),
    (dict(idx=0), 1, "NULL"),
    (dict(bk=1, maxb=1), 2, "16384"),  # 200000 keys in blocks of 1
])
def test_block_mask_validation(lib, kw, code, needle):
    m = _bm(**kw)
    p = _p()
    p.block_mask = ctypes.pointer(m)
    kv = _t((2, 2, 200000 if "16384" in needle else 64, 64))
    r, d = _call(lib, _t(Q), kv, kv, p)
    assert r == code and needle in d, d


def test_block_mask_rejected_with_paged_cache(lib):
    p = _p()
    m = _bm()
    p.block_mask = ctypes.pointer(m)
    cache = _t((100, 16, 8, 128))
    r, d = _call(lib, _t((4, 32, 3, 128)), cache, cache, p, paged=_paged())
    assert r == 2 and "contiguous" in d


def test_backward_validation(lib):
    q, kv = _t(Q), _t(KV)
    n = ctypes.c_size_t(0)
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(q), ctypes.byref(kv), ctypes.byref(kv),
                                        ctypes.byref(_p()), ctypes.byref(n)) == 0
    # per-row kernels: 8 bytes per query row; matrix-core kernels: a 384-byte
    # record per 32 rows of each (batch, head), 4 bytes per row, and (G > 1)
    # fp32 partial dK and dV per query head
    part_off = (2 * 8 * 2 * 384 + 2 * 8 * 64 * 4 + 255) // 256 * 256
    assert n.value == max(2 * 8 * 64 * 8, part_off + 2 * 2 * 8 * 64 * 64 * 4)

    def call(dout=None, dq=None, dk=None, dv=None, stats=0x9000, p=None, dsinks=None, ws=0x9100,
             wsn=1 << 20, out=None):
        r = lib.attn_bwd(ctypes.byref(q), ctypes.byref(kv), ctypes.byref(kv),
                         ctypes.byref(out) if out is not None else None,
                         ctypes.byref(dout or _t(Q)), stats, ctypes.byref(p or _p()),
                         ctypes.byref(dq or _t(Q)), ctypes.byref(dk or _t(KV)),
                         ctypes.byref(dv or _t(KV)), dsinks, ws, wsn, None)
        return r, apn.attn_last_error_detail()
    r, d = call(dq=_t((2, 8, 63, 64)))
    assert r == 1 and "dq" in d
    r, d = call(dk=_t(KV, torch.float32))
    assert r == 1 and "dk" in d
    r, d = call(stats=None)
    assert r == 1 and "row_stats" in d
    r, d = call(dsinks=0x9200)
    assert r == 1 and "softmax1" in d
    r, d = call(wsn=8)
    assert r == 3 and "workspace" in d
    r, d = call(out=_t((2, 8, 64, 32)))
    assert r == 1 and "out" in d
    pb = _p()
    m = _bm(bq=1, bk=1)  # 64 query blocks: accepted; see test_bwd_path
    pb.block_mask = ctypes.pointer(m)
    r, d = call(p=pb, wsn=8)
    assert r == 3 and "workspace" in d


def test_bwd_block_mask_query_block_limit(lib):
    # the per-row key kernel keeps a bitmap of at most 16384 query blocks
    q, kv = _t((1, 2, 16385, 64)), _t((1, 2, 64, 64))
    pb = _p()
    m = _bm(bq=1, bk=64)
    pb.block_mask = ctypes.pointer(m)
    path = ctypes.c_int(-1)
    r = lib.attn_bwd_path(ctypes.byref(q), ctypes.byref(kv), ctypes.byref(kv), None,
                          ctypes.byref(q), ctypes.byref(pb), ctypes.byref(q), ctypes.byref(kv),
                          ctypes.byref(kv), ctypes.byref(path))
    assert r == 2 and "16384 query blocks" in apn.attn_last_error_detail()
    m.block_q = 2
    r = lib.attn_bwd_path(ctypes.byref(q), ctypes.byref(kv), ctypes.byref(kv), None,
                          ctypes.byref(q), ctypes.byref(pb), ctypes.byref(q), ctypes.byref(kv),
                          ctypes.byref(kv), ctypes.byref(path))
    assert r == 0 and B.PATH_NAMES[path.value] == "bwd_per_row"


def _vl(num_seqs=3, max_q=50, cu_q=0x5000, cu_k=0x6000):
    vl = B._Varlen()
    vl.cu_seqlens_q, vl.cu_seqlens_k, vl.num_seqs, vl.max_seqlen_q = cu_q, cu_k, num_seqs, max_q
    return vl


def test_bwd_varlen_validation(lib):
    # every case fails validation before anything is launched
    def call(q=None, kv=None, vl="default", p=None, stats=0x9000, wsn=1 << 20, dsinks=None):
        q = q or _t((1, 8, 100, 64))
        kv = kv or _t((1, 2, 120, 64))
        vl = _vl() if vl == "default" else vl
        r = lib.attn_bwd_varlen(ctypes.byref(q), ctypes.byref(kv), ctypes.byref(kv), None,
                                ctypes.byref(q), stats,
                                ctypes.byref(vl) if vl is not None else None,
                                ctypes.byref(p or _p()), ctypes.byref(q), ctypes.byref(kv),
                                ctypes.byref(kv), dsinks, 0x9100, wsn, None)
        return r, apn.attn_last_error_detail()
    r, d = call(vl=None)
    assert r == 1 and "varlen" in d
    r, d = call(vl=_vl(num_seqs=-1))
    assert r == 1 and "num_seqs" in d
    r, d = call(vl=_vl(cu_q=0))
    assert r == 1 and "cu_seqlens" in d
    r, d = call(q=_t((2, 8, 100, 64)), kv=_t((2, 2, 120, 64)))
    assert r == 1 and "batch extent" in d
    r, d = call(stats=None)
    assert r == 1 and "row_stats" in d
    r, d = call(dsinks=0x9200)
    assert r == 1 and "softmax1" in d
    r, d = call(wsn=8 * 8 * 100 - 1)
    assert r == 3 and "workspace" in d
    pb = _p()
    m = _bm()
    pb.block_mask = ctypes.pointer(m)
    r, d = call(p=pb)
    assert r == 2 and "padded batch" in d


def _fwd_path(lib, q, k, v, p, out=None, paged=None):
    path = ctypes.c_int(-1)
    r = lib.attn_fwd_path(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                          ctypes.byref(paged) if paged else None, ctypes.byref(p),
                          ctypes.byref(out or q), ctypes.byref(path))
    return r, B.PATH_NAMES.get(path.value)


@pytest.mark.parametrize("q,kv,dtype,paged,p,want", [
    # the five workloads' shapes (bf16, aligned): tiled kernels
    ((4, 32, 2048, 64), (4, 8, 2048, 64), torch.bfloat16, None, dict(), "prefill_mfma"),
    ((2, 16, 8192, 128), (2, 8, 8192, 128), torch.bfloat16, None, dict(norm=3), "prefill_mfma"),
    ((1, 16, 8192, 256), (1, 8, 8192, 256), torch.bfloat16, None,
     dict(window=4096, softcap=50.0, scaling=0.0625), "prefill_mfma"),
    ((64, 32, 1, 128), (70000, 16, 8, 128), torch.bfloat16, 16, dict(norm=2), "decode_split"),
    ((64, 32, 512, 128), (70000, 16, 8, 128), torch.bfloat16, 16, dict(), "prefill_mfma"),
    # what the per-row kernel takes
    ((1, 2, 8, 16), (1, 2, 8, 16), torch.float32, None, dict(scaling=0.25), "per_row"),
    ((1, 4, 100, 64), (1, 2, 100, 64), torch.float32, None, dict(), "per_row"),
    ((1, 4, 100, 96), (1, 2, 100, 96), torch.bfloat16, None, dict(), "per_row"),
    ((1, 4, 100, 64), (1, 2, 100, 64), torch.bfloat16, None, dict(scaling=-0.1), "per_row"),
    ((2, 34, 1, 128), (100, 16, 2, 128), torch.bfloat16, 16, dict(), "per_row"),  # G = 17
    ((2, 4, 7, 128), (100, 12, 2, 128), torch.bfloat16, 12, dict(), "per_row"),  # pages of 12
    ((0, 4, 7, 64), (0, 2, 7, 64), torch.bfloat16, None, dict(), "none"),
])
def test_fwd_path(lib, q, kv, dtype, paged, p, want):
    pd = _paged(bs=paged, max_blocks=2048) if paged else None
    r, path = _fwd_path(lib, _t(q, dtype), _t(kv, dtype), _t(kv, dtype), _p(**p), paged=pd)
    assert r == 0, apn.attn_last_error_detail()
    assert path == want


def test_fwd_path_unaligned(lib):
    # a pointer off the 16-byte grid, or a row stride that is not a multiple
    # of 8 elements, leaves the tiled kernels
    q = _t((1, 4, 100, 64))
    kv = _t((1, 2, 100, 64))
    assert _fwd_path(lib, q, kv, kv, _p())[1] == "prefill_mfma"
    q.data = 0x1002
    assert _fwd_path(lib, q, kv, kv, _p())[1] == "per_row"
    q2 = _t((1, 4, 100, 64), strides=[4 * 100 * 68, 100 * 68, 68, 1])
    assert _fwd_path(lib, q2, kv, kv, _p())[1] == "per_row"
    r, _ = _fwd_path(lib, q, kv, kv, _p(norm=9))
    assert r == 1


def test_fwd_varlen_path(lib):
    q = _t((1, 8, 100, 64))
    kv = _t((1, 2, 120, 64))
    vl = B._Varlen()
    vl.cu_seqlens_q, vl.cu_seqlens_k, vl.num_seqs, vl.max_seqlen_q = 0x5000, 0x6000, 3, 50
    path = ctypes.c_int(-1)
    r = lib.attn_fwd_varlen_path(ctypes.byref(q), ctypes.byref(kv), ctypes.byref(kv),
                                 ctypes.byref(vl), ctypes.byref(_p()), ctypes.byref(q),
                                 ctypes.byref(path))
    assert r == 0 and B.PATH_NAMES[path.value] == "prefill_mfma"
    qf, kvf = _t((1, 8, 100, 64), torch.float32), _t((1, 2, 120, 64), torch.float32)
    r = lib.attn_fwd_varlen_path(ctypes.byref(qf), ctypes.byref(kvf), ctypes.byref(kvf),
                                 ctypes.byref(vl), ctypes.byref(_p()), ctypes.byref(qf),
                                 ctypes.byref(path))
    assert r == 0 and B.PATH_NAMES[path.value] == "per_row"


def test_bwd_path(lib):
    def path_of(q, kv, p=None):
        path = ctypes.c_int(-1)
        r = lib.attn_bwd_path(ctypes.byref(q), ctypes.byref(kv), ctypes.byref(kv), None,
                              ctypes.byref(q), ctypes.byref(p or _p()), ctypes.byref(q),
                              ctypes.byref(kv), ctypes.byref(kv), ctypes.byref(path))
        return r, B.PATH_NAMES.get(path.value)
    assert path_of(_t((4, 32, 2048, 64)), _t((4, 8, 2048, 64))) == (0, "bwd_mfma")
    assert path_of(_t((1, 4, 64, 96)), _t((1, 2, 64, 96))) == (0, "bwd_per_row")
    assert path_of(_t((1, 4, 64, 64), torch.float32), _t((1, 2, 64, 64), torch.float32)) == \
        (0, "bwd_per_row")
    pb = _p()
    m = _bm()
    pb.block_mask = ctypes.pointer(m)
    assert path_of(_t(Q), _t(KV), pb) == (0, "bwd_per_row")


def test_noalloc_rejects_oversized_workspace(lib):
    # the sparse decode lists of 64 sequences x 32 heads over 64 splits of
    # 512 keys need far more than the fixed 128 MiB scratch: rejected before
    # anything runs (no device is touched)
    q = _t((64, 32, 1, 128))
    cache = _t((70000, 16, 8, 128))
    r = lib.attn_fwd_noalloc(ctypes.byref(q), ctypes.byref(cache), ctypes.byref(cache),
                             ctypes.byref(_paged(max_blocks=2048)), ctypes.byref(_p(norm=2)),
                             ctypes.byref(q), None, None)
    assert r == 3 and "scratch" in apn.attn_last_error_detail()
    r = lib.attn_fwd_noalloc(ctypes.byref(q), ctypes.byref(cache), ctypes.byref(cache),
                             ctypes.byref(_paged(max_blocks=2048)), ctypes.byref(_p(norm=9)),
                             ctypes.byref(q), None, None)
    assert r == 1
