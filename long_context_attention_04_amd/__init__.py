"""Python binding of libcsa.so, the CSA / HCA attention hot path for gfx950.

Argument marshalling only: every function here forwards to the C ABI function
of the same name (declared in include/csa.h) and raises CsaError when it
returns a non-zero status.  Pointer arguments accept torch tensors (their
data_ptr() is passed), plain ints or None (NULL).  Device memory and streams
come from torch; all computation happens in the library's HIP kernels.

torch is imported before the library is loaded so the process holds a single
HIP runtime (torch's), which the library then shares.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede the library load: one HIP runtime per process)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python long_context_attention_04_amd/build.py` "
        "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)

F32, BF16, FP8_E4M3, MXFP4 = 0, 1, 2, 3
_STATUS = {0: "CSA_OK", 1: "CSA_ERR_NULL", 2: "CSA_ERR_SHAPE", 3: "CSA_ERR_DTYPE",
           4: "CSA_ERR_UNSUPPORTED", 5: "CSA_ERR_WORKSPACE", 6: "CSA_ERR_HIP"}


class CsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class CsaTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("scale", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("stride_b", ctypes.c_int64),
        ("stride_row", ctypes.c_int64),
        ("scale_stride_b", ctypes.c_int64),
        ("scale_stride_row", ctypes.c_int64),
    ]


class CsaCompressJob(ctypes.Structure):
    _fields_ = [
        ("raw", CsaTensor),
        ("raw_base", ctypes.c_void_p),
        ("logits", ctypes.c_void_p),
        ("m", ctypes.c_int32),
        ("dim", ctypes.c_int32),
        ("block_first", ctypes.c_void_p),
        ("block_count", ctypes.c_void_p),
        ("max_blocks", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("out", CsaTensor),
    ]


MAX_COMPRESS_JOBS = 4

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t
_TP = ctypes.POINTER(CsaTensor)


def _proto(name, restype, *argtypes):
    fn = getattr(_lib, name)
    fn.restype = restype
    fn.argtypes = list(argtypes)
    return fn


_c = {
    "csa_abi_version": _proto("csa_abi_version", _I32),
    "csa_status_string": _proto("csa_status_string", ctypes.c_char_p, _I32),
    "csa_last_error": _proto("csa_last_error", ctypes.c_char_p),
    "csa_compress": _proto("csa_compress", _I32, _TP, _P, _P, _I32, _I32, _P, _P, _I32, _I32, _TP, _P),
    "csa_compress_jobs": _proto("csa_compress_jobs", _I32, ctypes.POINTER(CsaCompressJob), _I32, _P),
    "csa_index_scores": _proto("csa_index_scores", _I32, _TP, _P, _TP, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P),
    "csa_topk": _proto("csa_topk", _I32, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _SZ, _P),
    "csa_topk_workspace_size": _proto("csa_topk_workspace_size", _SZ, _I32, _I32, _I32, _I32),
    "csa_index_topk": _proto("csa_index_topk", _I32, _TP, _P, _TP, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P,
                             _P, _P, _SZ, _P),
    "csa_index_topk_part": _proto("csa_index_topk_part", _I32, _TP, _P, _TP, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                  _I32, _P, _P, _P, _SZ, _I32, _P),
    "csa_index_topk_workspace_size": _proto("csa_index_topk_workspace_size", _SZ, _I32, _I32, _I32, _I32, _I32),
    "csa_compress_index_topk": _proto("csa_compress_index_topk", _I32, ctypes.POINTER(CsaCompressJob),
                                      ctypes.POINTER(CsaCompressJob), _TP, _P, _TP, _P, _I32, _I32, _I32, _I32,
                                      _I32, _I32, _I32, _P, _P, _P, _SZ, _I32, _P),
    "csa_sparse_attn": _proto("csa_sparse_attn", _I32, _TP, _TP, _P, _I32, _TP, _P, _I32, _P, _I32, _I32, _I32,
                              _I32, _F, _P, _P, _P, _SZ, _P),
    "hca_attn": _proto("hca_attn", _I32, _TP, _TP, _I32, _I32, _TP, _P, _I32, _P, _I32, _I32, _I32, _I32, _F, _P,
                       _P, _P, _SZ, _P),
    "csa_attn_workspace_size": _proto("csa_attn_workspace_size", _SZ, _I32, _I32, _I32, _I32, _I32),
    "csa_index_query": _proto("csa_index_query", _I32, _TP, _TP, _TP, _TP, _I32, _I32, _I32, _I32, _I32, _I32, _TP,
                              _P, _P, _SZ, _P),
    "csa_index_query_workspace_size": _proto("csa_index_query_workspace_size", _SZ, _I32, _I32, _I32, _I32, _I32,
                                             _I32),
    "csa_latent_query": _proto("csa_latent_query", _I32, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _SZ, _P),
    "csa_latent_query_workspace_size": _proto("csa_latent_query_workspace_size", _SZ, _I32, _I32, _I32, _I32),
    "csa_latent_output": _proto("csa_latent_output", _I32, _P, _P, _I32, _I32, _I32, _I32, _P, _I32, _P, _SZ, _P),
    "csa_latent_output_workspace_size": _proto("csa_latent_output_workspace_size", _SZ, _I32, _I32, _I32, _I32),
    "csa_sparse_attn_noalloc": _proto("csa_sparse_attn_noalloc", _I32, _TP, _TP, _P, _I32, _TP, _P, _I32, _P, _I32,
                                      _I32, _I32, _I32, _F, _P, _P, _P),
    "csa_quantize_mxfp4": _proto("csa_quantize_mxfp4", _I32, _P, _I64, _I32, _P, _P, _P),
    "csa_quantize_fp8": _proto("csa_quantize_fp8", _I32, _P, _I64, _I32, _P, _P, _P),
    "csa_stream_read": _proto("csa_stream_read", _I32, _P, _SZ, _P, _P),
    "csa_stream_read_sink_size": _proto("csa_stream_read_sink_size", _SZ),
}


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != 0:
        raise CsaError(status, _c["csa_last_error"]().decode())


def desc(data, dtype: int, scale=None) -> CsaTensor:
    """CsaTensor for a torch tensor viewed as [batch, rows, ...].

    Strides are taken from the tensor (in its own elements: bytes for uint8
    code tensors).  `scale` is the FP8 row-scale tensor [batch, rows] or the
    MXFP4 scale tensor [batch, rows, cols/32].  The descriptor holds references
    to both tensors, so their memory stays valid while it is in use."""
    t = CsaTensor()
    t._keep = (data, scale)  # the descriptor keeps its tensors alive
    t.data = _ptr(data)
    t.scale = _ptr(scale)
    t.dtype = dtype
    t.stride_b = data.stride(0) if data.dim() >= 1 else 0
    t.stride_row = data.stride(1) if data.dim() >= 2 else 0
    if scale is not None:
        t.scale_stride_b = scale.stride(0) if scale.dim() >= 1 else 0
        t.scale_stride_row = scale.stride(1) if scale.dim() >= 2 else 0
    return t


def abi_version() -> int:
    return _c["csa_abi_version"]()


def csa_status_string(status: int) -> str:
    return _c["csa_status_string"](status).decode()


def csa_last_error() -> str:
    return _c["csa_last_error"]().decode()


def csa_compress(raw, raw_base, logits, m, dim, block_first, block_count, max_blocks, batch, out, stream=None):
    _check(_c["csa_compress"](ctypes.byref(raw), _ptr(raw_base), _ptr(logits), m, dim, _ptr(block_first),
                              _ptr(block_count), max_blocks, batch, ctypes.byref(out), _stream(stream)))


def csa_compress_jobs(jobs, stream=None):
    """jobs: sequence of (raw, raw_base, logits, m, dim, block_first, block_count, max_blocks, batch, out),
    each exactly the arguments of one csa_compress call; one launch for all of them."""
    arr = (CsaCompressJob * max(len(jobs), 1))()
    for i, (raw, raw_base, logits, m, dim, first, count, max_blocks, batch, out) in enumerate(jobs):
        arr[i] = CsaCompressJob(raw, _ptr(raw_base), _ptr(logits), m, dim, _ptr(first), _ptr(count), max_blocks,
                                batch, out)
    _check(_c["csa_compress_jobs"](arr, len(jobs), _stream(stream)))


def csa_index_scores(q_idx, w, k_idx, q_pos, batch, tq, n_idx_heads, idx_dim, m, n_cap, scores, stream=None):
    _check(_c["csa_index_scores"](ctypes.byref(q_idx), _ptr(w), ctypes.byref(k_idx), _ptr(q_pos), batch, tq,
                                  n_idx_heads, idx_dim, m, n_cap, _ptr(scores), _stream(stream)))


def csa_topk_workspace_size(batch, tq, n_cap, k) -> int:
    return _c["csa_topk_workspace_size"](batch, tq, n_cap, k)


def csa_topk(scores, q_pos, batch, tq, n_cap, m, k, idx, ws=None, ws_bytes=0, stream=None):
    _check(_c["csa_topk"](_ptr(scores), _ptr(q_pos), batch, tq, n_cap, m, k, _ptr(idx), _ptr(ws), ws_bytes,
                          _stream(stream)))


def csa_index_topk_workspace_size(batch, tq, n_cap, k, scores_kept=True) -> int:
    return _c["csa_index_topk_workspace_size"](batch, tq, n_cap, k, int(bool(scores_kept)))


def csa_index_topk(q_idx, w, k_idx, q_pos, batch, tq, n_idx_heads, idx_dim, m, n_cap, k, scores, idx, ws=None,
                   ws_bytes=0, stream=None):
    _check(_c["csa_index_topk"](ctypes.byref(q_idx), _ptr(w), ctypes.byref(k_idx), _ptr(q_pos), batch, tq,
                                n_idx_heads, idx_dim, m, n_cap, k, _ptr(scores), _ptr(idx), _ptr(ws), ws_bytes,
                                _stream(stream)))


def csa_index_topk_part(q_idx, w, k_idx, q_pos, batch, tq, n_idx_heads, idx_dim, m, n_cap, k, scores, idx, ws,
                        ws_bytes, part, stream=None):
    _check(_c["csa_index_topk_part"](ctypes.byref(q_idx), _ptr(w), ctypes.byref(k_idx), _ptr(q_pos), batch, tq,
                                     n_idx_heads, idx_dim, m, n_cap, k, _ptr(scores), _ptr(idx), _ptr(ws), ws_bytes,
                                     part, _stream(stream)))


def _job(j):
    if j is None:
        return None
    raw, raw_base, logits, m, dim, first, count, max_blocks, batch, out = j
    return ctypes.byref(CsaCompressJob(raw, _ptr(raw_base), _ptr(logits), m, dim, _ptr(first), _ptr(count),
                                       max_blocks, batch, out))


def csa_compress_index_topk(kv_job, key_job, q_idx, w, k_idx, q_pos, batch, tq, n_idx_heads, idx_dim, m, n_cap, k,
                            scores, idx, ws, ws_bytes, part=3, stream=None):
    """csa_compress_jobs([kv_job, key_job]) then csa_index_topk_part(..., part), in as few launches as
    the shapes allow; each job is a csa_compress argument tuple or None."""
    _check(_c["csa_compress_index_topk"](_job(kv_job), _job(key_job), ctypes.byref(q_idx), _ptr(w),
                                         ctypes.byref(k_idx), _ptr(q_pos), batch, tq, n_idx_heads, idx_dim, m, n_cap,
                                         k, _ptr(scores), _ptr(idx), _ptr(ws), ws_bytes, part, _stream(stream)))


def csa_attn_workspace_size(batch, tq, heads, dim, n_entries_max) -> int:
    return _c["csa_attn_workspace_size"](batch, tq, heads, dim, n_entries_max)


def csa_sparse_attn(q, kv_cmp, idx, k, kv_raw, raw_base, window, q_pos, batch, tq, heads, dim, scale, out, lse=None,
                    ws=None, ws_bytes=0, stream=None):
    _check(_c["csa_sparse_attn"](ctypes.byref(q), ctypes.byref(kv_cmp), _ptr(idx), k, ctypes.byref(kv_raw),
                                 _ptr(raw_base), window, _ptr(q_pos), batch, tq, heads, dim, scale, _ptr(out),
                                 _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))


def csa_index_query(h, w_dq, w_uq, w_w, batch, tq, d_model, rank, n_idx_heads, idx_dim, q_idx, w, ws, ws_bytes,
                    stream=None):
    _check(_c["csa_index_query"](ctypes.byref(h), ctypes.byref(w_dq), ctypes.byref(w_uq), ctypes.byref(w_w), batch,
                                 tq, d_model, rank, n_idx_heads, idx_dim, ctypes.byref(q_idx), _ptr(w), _ptr(ws),
                                 ws_bytes, _stream(stream)))


def csa_index_query_workspace_size(batch, tq, d_model, rank, n_idx_heads, idx_dim):
    return _c["csa_index_query_workspace_size"](batch, tq, d_model, rank, n_idx_heads, idx_dim)


def csa_latent_query(q, w_uk_t, rows, heads, head_dim, dim, q_lat, ws, ws_bytes, stream=None):
    _check(_c["csa_latent_query"](_ptr(q), _ptr(w_uk_t), rows, heads, head_dim, dim, _ptr(q_lat), _ptr(ws), ws_bytes,
                                  _stream(stream)))


def csa_latent_query_workspace_size(rows, heads, head_dim, dim):
    return _c["csa_latent_query_workspace_size"](rows, heads, head_dim, dim)


def csa_latent_output(o_lat, w_uv, rows, heads, head_dim, dim, out, out_dtype, ws, ws_bytes, stream=None):
    _check(_c["csa_latent_output"](_ptr(o_lat), _ptr(w_uv), rows, heads, head_dim, dim, _ptr(out), out_dtype,
                                   _ptr(ws), ws_bytes, _stream(stream)))


def csa_latent_output_workspace_size(rows, heads, head_dim, dim):
    return _c["csa_latent_output_workspace_size"](rows, heads, head_dim, dim)


def csa_sparse_attn_noalloc(q, kv_cmp, idx, k, kv_raw, raw_base, window, q_pos, batch, tq, heads, dim, scale, out,
                            lse=None, stream=None):
    _check(_c["csa_sparse_attn_noalloc"](ctypes.byref(q), ctypes.byref(kv_cmp), _ptr(idx), k, ctypes.byref(kv_raw),
                                         _ptr(raw_base), window, _ptr(q_pos), batch, tq, heads, dim, scale, _ptr(out),
                                         _ptr(lse), _stream(stream)))


CSA_NOALLOC_SCRATCH_BYTES = 64 << 20  # the static scratch of csa_sparse_attn_noalloc (csa.h)


def hca_attn(q, kv_hc, m_hc, n_cap_hc, kv_raw, raw_base, window, q_pos, batch, tq, heads, dim, scale, out, lse=None,
             ws=None, ws_bytes=0, stream=None):
    _check(_c["hca_attn"](ctypes.byref(q), ctypes.byref(kv_hc), m_hc, n_cap_hc, ctypes.byref(kv_raw), _ptr(raw_base),
                          window, _ptr(q_pos), batch, tq, heads, dim, scale, _ptr(out), _ptr(lse), _ptr(ws),
                          ws_bytes, _stream(stream)))


def csa_quantize_mxfp4(x, rows, cols, codes, scales, stream=None):
    _check(_c["csa_quantize_mxfp4"](_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream(stream)))


def csa_quantize_fp8(x, rows, cols, codes, row_scale, stream=None):
    _check(_c["csa_quantize_fp8"](_ptr(x), rows, cols, _ptr(codes), _ptr(row_scale), _stream(stream)))


def csa_stream_read(data, nbytes, sink, stream=None):
    _check(_c["csa_stream_read"](_ptr(data), nbytes, _ptr(sink), _stream(stream)))


def csa_stream_read_sink_size() -> int:
    return _c["csa_stream_read_sink_size"]()


EXPORTED = [k for k in _c]
