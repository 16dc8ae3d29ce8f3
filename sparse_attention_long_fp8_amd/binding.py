"""ctypes binding of libdsa (include/libdsa.h).

Argument marshalling only: every step of the path runs in the HIP library.
Tensor arguments are torch tensors on the GPU (their data_ptr() is passed),
or None for NULL; the stream defaults to torch's current stream.  Each
wrapper keeps the C entry point's name and raises DsaError (carrying the
dsa_status_t and the library's message) when the status is not DSA_OK.
If libdsa.so is missing, loading fails loudly: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdsa.so")
PROJ_LIB_PATH = os.path.join(PKG, "libdsa_proj.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "libdsa.h")
PROJ_HEADER = os.path.join(os.path.dirname(PKG), "include", "libdsa_proj.h")

DSA_OK, DSA_ERR_INVALID_ARGUMENT, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE_TOO_SMALL, DSA_ERR_HIP = range(5)
DSA_F32, DSA_BF16, DSA_FP8_E4M3 = range(3)
DSA_CHECK_OK, DSA_CHECK_BATCH, DSA_CHECK_ROWS, DSA_CHECK_PAGE, DSA_CHECK_INDEX, DSA_CHECK_NAN_SCORE = range(6)

c_i32, c_i64, c_f32, c_ptr, c_size = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class dsa_batch_t(ctypes.Structure):
    _fields_ = [("num_seqs", c_i32), ("num_queries", c_i32), ("q_seq_start", c_ptr),
                ("k_len", c_ptr), ("max_q_per_seq", c_i32), ("max_k_len", c_i32)]


class dsa_kv_layout_t(ctypes.Structure):
    _fields_ = [("paged", c_i32), ("k_seq_start", c_ptr), ("page_table", c_ptr),
                ("page_table_stride", c_i32), ("page_size", c_i32), ("num_rows", c_i64)]


class dsa_forward_args_t(ctypes.Structure):
    _fields_ = [("batch", dsa_batch_t), ("layout", dsa_kv_layout_t),
                ("index_dtype", c_i32), ("h_i", c_i32), ("d_i", c_i32),
                ("q_idx", c_ptr), ("q_scale", c_ptr), ("w", c_ptr), ("k_idx", c_ptr),
                ("k_scale", c_ptr), ("index_scale", c_f32),
                ("top_k", c_i32), ("scores", c_ptr), ("ld_scores", c_i64), ("indices", c_ptr),
                ("mla_dtype", c_i32), ("heads", c_i32), ("d_qk", c_i32), ("d_v", c_i32),
                ("q", c_ptr), ("kv", c_ptr), ("sm_scale", c_f32), ("out", c_ptr), ("lse", c_ptr)]


class DsaError(RuntimeError):
    def __init__(self, status, where, detail):
        super().__init__("%s: %s (%s)" % (where, _STATUS_NAMES.get(status, status), detail))
        self.status = status


_STATUS_NAMES = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARGUMENT", 2: "DSA_ERR_UNSUPPORTED",
                 3: "DSA_ERR_WORKSPACE_TOO_SMALL", 4: "DSA_ERR_HIP"}

_SIGS = {
    "dsa_indexer_scores": [ctypes.POINTER(dsa_batch_t), ctypes.POINTER(dsa_kv_layout_t), c_i32, c_i32, c_i32,
                           c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_f32, c_ptr, c_i64, c_ptr],
    "dsa_topk": [ctypes.POINTER(dsa_batch_t), c_ptr, c_i64, c_i32, c_ptr, c_ptr, c_size, c_ptr],
    "dsa_validate": [ctypes.POINTER(dsa_batch_t), ctypes.POINTER(dsa_kv_layout_t), c_ptr, c_i32, c_ptr, c_i64, c_ptr,
                     c_ptr],
    "dsa_topk_workspace_size": [ctypes.POINTER(dsa_batch_t), c_i32, ctypes.POINTER(c_size)],
    "dsa_sparse_mla_fwd": [ctypes.POINTER(dsa_batch_t), ctypes.POINTER(dsa_kv_layout_t), c_i32, c_i32, c_i32,
                           c_i32, c_ptr, c_ptr, c_ptr, c_i32, c_f32, c_ptr, c_ptr, c_ptr, c_size, c_ptr],
    "dsa_sparse_mla_workspace_size": [ctypes.POINTER(dsa_batch_t), c_i32, c_i32, c_i32, c_i32, c_i32,
                                      ctypes.POINTER(c_size)],
    "dsa_forward": [ctypes.POINTER(dsa_forward_args_t), c_ptr, c_size, c_ptr],
    "dsa_forward_workspace_size": [ctypes.POINTER(dsa_forward_args_t), ctypes.POINTER(c_size)],
    "dsa_forward_noalloc": [ctypes.POINTER(dsa_forward_args_t), c_ptr],
    "dsa_indexer_topk": [ctypes.POINTER(dsa_batch_t), ctypes.POINTER(dsa_kv_layout_t), c_i32, c_i32, c_i32,
                         c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_f32, c_i32, c_ptr, c_ptr, c_size, c_ptr],
    "dsa_indexer_topk_workspace_size": [ctypes.POINTER(dsa_batch_t), ctypes.POINTER(dsa_kv_layout_t), c_i32, c_i32,
                                        c_i32, c_i32, ctypes.POINTER(c_size)],
    "dsa_cache_append": [ctypes.POINTER(dsa_kv_layout_t), c_i32, c_ptr, c_ptr, c_i32, c_ptr, c_ptr, c_ptr,
                         c_i32, c_ptr, c_ptr, c_ptr],
    "dsa_module_forward": [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32] + [c_ptr] * 11
                          + [c_ptr, c_size, c_ptr],
    "dsa_module_forward_workspace_size": [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                          ctypes.POINTER(c_size)],
    "dsa_status_string": [c_i32],
    "dsa_last_error": [],
    "dsa_abi_version": [],
}
# libdsa_proj.so (include/libdsa_proj.h): the hipBLASLt output projections
_PROJ_SIGS = {
    "dsa_output_projection": [c_ptr, c_i32, c_i32, c_i32, c_i32, c_i32, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_size,
                              c_ptr],
    "dsa_output_projection_workspace_size": [c_i32, c_i32, c_i32, ctypes.POINTER(c_size)],
    "dsa_blaslt_create": [ctypes.POINTER(c_ptr)],
    "dsa_blaslt_destroy": [c_ptr],
}
_RESTYPES = {"dsa_status_string": ctypes.c_char_p, "dsa_last_error": ctypes.c_char_p,
             "dsa_abi_version": c_i32}

_LIB = None
_PROJ_LIB = None


def lib():
    """The loaded libdsa.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libdsa.so not found at %s; build it with "
                               "`python -m sparse_attention_long_fp8_amd.build`" % LIB_PATH)
        handle = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = _RESTYPES.get(name, c_i32)
        _LIB = handle
    return _LIB


def proj_lib():
    """The loaded libdsa_proj.so, the output projections (raises if it has
    not been built).  It links hipBLASLt; libdsa.so does not."""
    global _PROJ_LIB
    if _PROJ_LIB is None:
        lib()  # its status helpers live in libdsa.so
        if not os.path.exists(PROJ_LIB_PATH):
            raise RuntimeError("libdsa_proj.so not found at %s; build it with "
                               "`python -m sparse_attention_long_fp8_amd.build`" % PROJ_LIB_PATH)
        handle = ctypes.CDLL(PROJ_LIB_PATH)
        for name, args in _PROJ_SIGS.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = c_i32
        _PROJ_LIB = handle
    return _PROJ_LIB


def header_functions(header=HEADER):
    """Names of the functions a header (default include/libdsa.h) declares."""
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:dsa_status_t|const char \*|int32_t)\s*(dsa_\w+)\s*\(", text, re.M)))


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------
def _p(x):
    """Device address of a tensor (None -> NULL, int -> itself)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        if not torch.cuda.is_available():
            return None  # NULL stream; only argument-validation paths run without a GPU
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, where):
    if status != DSA_OK:
        raise DsaError(status, where, dsa_last_error())


# The descriptors hold raw device pointers; each keeps a reference to the
# tensors it points at (`_keep`), so that a temporary passed in is not freed
# (and its memory handed to another tensor) while the descriptor is in use.

def make_batch(q_seq_start, k_len, num_seqs, num_queries, max_q_per_seq, max_k_len):
    """dsa_batch_t from device int32 tensors and host-side counts / bounds."""
    bt = dsa_batch_t(int(num_seqs), int(num_queries), _p(q_seq_start), _p(k_len), int(max_q_per_seq),
                     int(max_k_len))
    bt._keep = (q_seq_start, k_len)
    return bt


def make_contiguous_layout(k_seq_start, num_rows):
    ly = dsa_kv_layout_t(0, _p(k_seq_start), None, 0, 64, int(num_rows))
    ly._keep = (k_seq_start,)
    return ly


def make_paged_layout(page_table, stride, num_pages, page_size=64):
    ly = dsa_kv_layout_t(1, None, _p(page_table), int(stride), int(page_size), int(num_pages))
    ly._keep = (page_table,)
    return ly


# --------------------------------------------------------------------------
# entry points (same names as the C ABI)
# --------------------------------------------------------------------------
def dsa_status_string(status):
    return lib().dsa_status_string(int(status)).decode()


def dsa_last_error():
    return lib().dsa_last_error().decode()


def dsa_abi_version():
    return int(lib().dsa_abi_version())


def dsa_indexer_scores(batch, keys, dtype, h_i, d_i, q_idx, q_scale, w, k_idx, k_scale, scale, scores,
                       ld_scores, stream=None, check=True):
    st = lib().dsa_indexer_scores(ctypes.byref(batch), ctypes.byref(keys), dtype, h_i, d_i, _p(q_idx),
                                  _p(q_scale), _p(w), _p(k_idx), _p(k_scale), float(scale), _p(scores),
                                  int(ld_scores), _stream(stream))
    if check:
        _check(st, "dsa_indexer_scores")
    return st


def dsa_topk_workspace_size(batch, k):
    n = c_size(0)
    _check(lib().dsa_topk_workspace_size(ctypes.byref(batch), int(k), ctypes.byref(n)), "dsa_topk_workspace_size")
    return n.value


def dsa_validate(batch, layout, indices, k, scores, ld_scores, report, stream=None, check=True):
    """Enqueue the precondition checks; `report` is a device int32[4] (see libdsa.h)."""
    st = lib().dsa_validate(ctypes.byref(batch), None if layout is None else ctypes.byref(layout), _p(indices),
                            int(k), _p(scores), int(ld_scores), _p(report), _stream(stream))
    if check:
        _check(st, "dsa_validate")
    return st


def dsa_topk(batch, scores, ld_scores, k, indices, workspace=None, workspace_bytes=0, stream=None, check=True):
    st = lib().dsa_topk(ctypes.byref(batch), _p(scores), int(ld_scores), int(k), _p(indices), _p(workspace),
                        int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "dsa_topk")
    return st


def dsa_sparse_mla_workspace_size(batch, dtype, heads, d_qk, d_v, k):
    n = c_size(0)
    _check(lib().dsa_sparse_mla_workspace_size(ctypes.byref(batch), dtype, heads, d_qk, d_v, int(k),
                                               ctypes.byref(n)), "dsa_sparse_mla_workspace_size")
    return n.value


def dsa_sparse_mla_fwd(batch, kv_layout, dtype, heads, d_qk, d_v, q, kv, indices, k, sm_scale, out, lse,
                       workspace=None, workspace_bytes=0, stream=None, check=True):
    st = lib().dsa_sparse_mla_fwd(ctypes.byref(batch), ctypes.byref(kv_layout), dtype, heads, d_qk, d_v, _p(q),
                                  _p(kv), _p(indices), int(k), float(sm_scale), _p(out), _p(lse), _p(workspace),
                                  int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "dsa_sparse_mla_fwd")
    return st


def dsa_forward_workspace_size(args):
    n = c_size(0)
    _check(lib().dsa_forward_workspace_size(ctypes.byref(args), ctypes.byref(n)), "dsa_forward_workspace_size")
    return n.value


def dsa_forward(args, workspace=None, workspace_bytes=0, stream=None, check=True):
    st = lib().dsa_forward(ctypes.byref(args), _p(workspace), int(workspace_bytes),
                           _stream(stream))
    if check:
        _check(st, "dsa_forward")
    return st


def dsa_forward_noalloc(args, stream=None, check=True):
    st = lib().dsa_forward_noalloc(ctypes.byref(args), _stream(stream))
    if check:
        _check(st, "dsa_forward_noalloc")
    return st


def dsa_indexer_topk_workspace_size(batch, keys, dtype, h_i, d_i, k):
    n = c_size(0)
    _check(lib().dsa_indexer_topk_workspace_size(ctypes.byref(batch), ctypes.byref(keys), dtype, h_i, d_i, int(k),
                                                 ctypes.byref(n)), "dsa_indexer_topk_workspace_size")
    return n.value


def dsa_indexer_topk(batch, keys, dtype, h_i, d_i, q_idx, q_scale, w, k_idx, k_scale, scale, k, indices,
                     workspace=None, workspace_bytes=0, stream=None, check=True):
    st = lib().dsa_indexer_topk(ctypes.byref(batch), ctypes.byref(keys), dtype, h_i, d_i, _p(q_idx), _p(q_scale),
                                _p(w), _p(k_idx), _p(k_scale), float(scale), int(k), _p(indices), _p(workspace),
                                int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "dsa_indexer_topk")
    return st


def dsa_cache_append(layout, num_tokens, seq, pos, d_i, k_new, k_pool, k_scale_pool, d_c=0, latent_new=None,
                     latent_pool=None, stream=None, check=True):
    st = lib().dsa_cache_append(ctypes.byref(layout), int(num_tokens), _p(seq), _p(pos), int(d_i), _p(k_new),
                                _p(k_pool), _p(k_scale_pool), int(d_c), _p(latent_new), _p(latent_pool),
                                _stream(stream))
    if check:
        _check(st, "dsa_cache_append")
    return st


def dsa_blaslt_create():
    h = c_ptr()
    _check(proj_lib().dsa_blaslt_create(ctypes.byref(h)), "dsa_blaslt_create")
    return h.value


def dsa_blaslt_destroy(handle):
    _check(proj_lib().dsa_blaslt_destroy(handle), "dsa_blaslt_destroy")


def dsa_output_projection_workspace_size(num_queries, heads, d_h):
    n = c_size(0)
    _check(proj_lib().dsa_output_projection_workspace_size(int(num_queries), int(heads), int(d_h), ctypes.byref(n)),
           "dsa_output_projection_workspace_size")
    return n.value


def dsa_output_projection(blaslt, num_queries, heads, d_c, d_h, hidden, o, w_uv, w_o, out, workspace,
                          workspace_bytes, stream=None, check=True):
    st = proj_lib().dsa_output_projection(blaslt, int(num_queries), int(heads), int(d_c), int(d_h), int(hidden), _p(o),
                                     _p(w_uv), _p(w_o), _p(out), _p(workspace), int(workspace_bytes),
                                     _stream(stream))
    if check:
        _check(st, "dsa_output_projection")
    return st


def dsa_module_forward_workspace_size(batch, seq_len, hidden, heads, head_dim, latent_dim, index_dim):
    n = c_size(0)
    _check(lib().dsa_module_forward_workspace_size(int(batch), int(seq_len), int(hidden), int(heads),
                                                   int(head_dim), int(latent_dim), int(index_dim),
                                                   ctypes.byref(n)),
           "dsa_module_forward_workspace_size")
    return n.value


def dsa_module_forward(batch, seq_len, hidden, heads, head_dim, latent_dim, index_dim, top_k, q_hidden, hist,
                       latent, w_qi, w_ki, w_q, w_uk, w_uv, w_out, out, indices, workspace, workspace_bytes,
                       stream=None, check=True):
    st = lib().dsa_module_forward(int(batch), int(seq_len), int(hidden), int(heads), int(head_dim),
                                  int(latent_dim), int(index_dim), int(top_k), _p(q_hidden), _p(hist), _p(latent),
                                  _p(w_qi), _p(w_ki), _p(w_q), _p(w_uk), _p(w_uv), _p(w_out), _p(out), _p(indices),
                                  _p(workspace), int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "dsa_module_forward")
    return st


def forward_args(batch, layout, *, index_dtype, h_i, d_i, q_idx, q_scale, w, k_idx, k_scale, index_scale,
                 top_k, scores=None, ld_scores=0, indices=None, mla_dtype, heads, d_qk, d_v, q, kv, sm_scale,
                 out, lse=None):
    """dsa_forward_args_t from tensors (marshalling only)."""
    return dsa_forward_args_t(batch, layout, index_dtype, h_i, d_i, _p(q_idx), _p(q_scale), _p(w), _p(k_idx),
                              _p(k_scale), float(index_scale), int(top_k), _p(scores), int(ld_scores),
                              _p(indices), mla_dtype, heads, d_qk, d_v, _p(q), _p(kv), float(sm_scale), _p(out),
                              _p(lse))
