"""Thin ctypes binding of ``libmp.so`` (the C ABI declared in ``include/mp.h``).

Argument marshalling only: each function takes torch device tensors, checks
nothing the library does not check itself, passes raw pointers and sizes, and
raises :class:`MPError` on a non-zero status.  Every step of the path runs in
the library's HIP kernels; there is no fallback.  Workspaces are plain device
byte buffers obtained through torch's allocator.

All calls are asynchronous on ``stream`` (default: torch's current stream).
"""

import collections
import ctypes
import os

import torch

# MP_LIB may name another build of the library (e.g. the host-sanitized test
# build); a missing library is an error either way.
_LIB_PATH = os.environ.get("MP_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmp.so")
_lib = None

MP_F32, MP_BF16 = 0, 1
MP_ACT_NONE, MP_ACT_GELU_ERF, MP_ACT_GELU_TANH = 0, 1, 2
ACTS = {"none": MP_ACT_NONE, "erf": MP_ACT_GELU_ERF, "tanh": MP_ACT_GELU_TANH}
MP_MAX_SHARDS = 16

ERRORS = {0: "MP_OK", -1: "MP_ERR_NULL", -2: "MP_ERR_SHAPE", -3: "MP_ERR_DTYPE", -4: "MP_ERR_UNSUPPORTED",
          -5: "MP_ERR_ALIGN", -6: "MP_ERR_WORKSPACE", -7: "MP_ERR_HIP", -8: "MP_ERR_ARG", -9: "MP_ERR_DATA"}

c_i64, c_i32, c_u64, c_f32, c_p, c_sz = (ctypes.c_int64, ctypes.c_int, ctypes.c_uint64, ctypes.c_float,
                                         ctypes.c_void_p, ctypes.c_size_t)

# name -> (restype, argtypes); the order follows include/mp.h.
_SIGS = {
    "mp_version": (c_i32, []),
    "mp_device_supported": (c_i32, [c_i32]),
    "mp_last_error": (ctypes.c_char_p, []),
    "mp_check_indices": (c_i32, [c_p, c_i64, c_i64, c_i64, c_p, c_p]),
    "mp_column_linear_gelu": (c_i32, [c_i32, c_i32, c_i64, c_i64, c_i64, c_p, c_p, c_p, c_i32, c_p, c_p, c_p]),
    "mp_column_linear_gelu_bwd_workspace": (c_sz, [c_i32, c_i64, c_i64, c_i64]),
    "mp_column_linear_gelu_bwd": (c_i32, [c_i32, c_i64, c_i64, c_i64, c_p, c_p, c_p, c_p, c_i32, c_p, c_p, c_p,
                                          c_p, c_sz, c_p]),
    "mp_row_linear_partial": (c_i32, [c_i32, c_i64, c_i64, c_i64, c_p, c_p, c_p, c_p]),
    "mp_row_linear_partial_bwd_workspace": (c_sz, [c_i32, c_i64, c_i64, c_i64]),
    "mp_row_linear_partial_bwd": (c_i32, [c_i32, c_i64, c_i64, c_i64, c_p, c_p, c_p, c_p, c_p, c_p, c_sz, c_p]),
    "mp_row_linear_partial_bwd_static_max_bytes": (c_sz, []),
    "mp_row_linear_partial_bwd_static": (c_i32, [c_i32, c_i64, c_i64, c_i64, c_p, c_p, c_p, c_p, c_p, c_p]),
    "mp_row_linear_partial_bwd_dact": (c_i32, [c_i32, c_i64, c_i64, c_i64, c_p, c_p, c_p, c_p, c_i32, c_p, c_p, c_p,
                                               c_sz, c_p]),
    "mp_shard_reduce": (c_i32, [c_i32, c_i32, c_i64, c_i64, c_p, c_p, c_p, c_f32, c_u64, c_u64, c_u64, c_p, c_p,
                                c_p]),
    "mp_shared_seed_dropout": (c_i32, [c_i32, c_i64, c_p, c_p, c_p, c_f32, c_u64, c_u64, c_u64, c_p]),
    "mp_shard_reduce_layernorm": (c_i32, [c_i32, c_i32, c_i64, c_i64, c_p, c_p, c_p, c_f32, c_u64, c_u64, c_u64,
                                          c_p, c_p, c_p, c_p, c_f32, c_p, c_p, c_p, c_p]),
    "mp_shard_reduce_layernorm_bwd_workspace": (c_sz, [c_i64, c_i64]),
    "mp_shard_reduce_layernorm_bwd": (c_i32, [c_i32, c_i32, c_i64, c_i64, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p,
                                              c_p, c_p, c_sz, c_p]),
    "mp_shard_reduce_layernorm_bwd_dropout": (c_i32, [c_i32, c_i32, c_i64, c_i64, c_p, c_p, c_p, c_p, c_p, c_p, c_p,
                                                      c_p, c_p, c_f32, c_p, c_p, c_p, c_p, c_sz, c_p]),
    "mp_all_gather_rows": (c_i32, [c_i32, c_i32, c_i64, c_i64, c_p, c_p, c_p]),
    "mp_vocab_parallel_embedding_bwd": (c_i32, [c_i32, c_i64, c_i64, c_i64, c_i64, c_p, c_p, c_p, c_i32, c_p]),
    "mp_vocab_parallel_logits_xent_workspace": (c_sz, [c_i64, c_i64, c_i64]),
    "mp_vocab_parallel_logits_xent": (c_i32, [c_i32, c_i64, c_i64, c_i64, c_i64, c_p, c_p, c_p, c_p, c_p, c_sz, c_p]),
    "mp_dropout_mask_bwd_workspace": (c_sz, [c_i64, c_i64]),
    "mp_dropout_mask_bwd": (c_i32, [c_i32, c_i64, c_i64, c_p, c_p, c_f32, c_p, c_p, c_p, c_sz, c_p]),
    "mp_bias_grad_workspace": (c_sz, [c_i64, c_i64]),
    "mp_bias_grad": (c_i32, [c_i32, c_i64, c_i64, c_p, c_p, c_p, c_sz, c_p]),
    "mp_head_attention": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_p, c_p, c_p, c_p, c_p, c_p,
                                  c_p]),
    "mp_head_attention_bwd_workspace": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "mp_head_attention_bwd": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_p, c_p, c_p, c_p, c_p,
                                      c_p, c_p, c_p, c_p, c_p, c_sz, c_p]),
    "mp_vocab_parallel_embedding": (c_i32, [c_i32, c_i64, c_i64, c_i64, c_i64, c_p, c_p, c_p, c_p]),
    "mp_vocab_parallel_xent": (c_i32, [c_i64, c_i64, c_i64, c_p, c_p, c_p, c_p]),
    "mp_vocab_xent_combine": (c_i32, [c_i32, c_i64, c_p, c_p, c_p, c_p, c_p]),
    "mp_vocab_parallel_xent_bwd": (c_i32, [c_i64, c_i64, c_i64, c_p, c_p, c_p, c_f32, c_i32, c_p, c_p]),
    "mp_grouped_expert_gemm_workspace": (c_sz, [c_i64, c_i64, c_i64, c_i32, c_i32]),
    "mp_grouped_expert_gemm": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_i32, c_i32, c_p, c_p, c_p, c_p, c_p, c_p, c_p,
                                       c_p, c_p, c_sz, c_p]),
    "mp_grouped_expert_gemm_weighted_act": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_i32, c_i32, c_p, c_p, c_p, c_p,
                                                    c_p, c_p, c_p, c_p, c_p, c_sz, c_p]),
    "mp_grouped_expert_gemm_fwd_train": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_i32, c_i32, c_p, c_p, c_p, c_p, c_p,
                                                 c_p, c_p, c_p, c_sz, c_p]),
    "mp_grouped_expert_gemm_weighted_act_fwd_train": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_i32, c_i32, c_p, c_p,
                                                              c_p, c_p, c_p, c_p, c_p, c_p, c_sz, c_p]),
    "mp_grouped_expert_gemm_weighted_act_bwd": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_i32, c_p, c_p, c_p, c_p, c_p,
                                                        c_p, c_p, c_sz, c_p, c_p, c_p, c_p, c_p, c_sz, c_p]),
    "mp_grouped_expert_gemm_bwd_workspace": (c_sz, [c_i64, c_i64, c_i64, c_i32, c_i32]),
    "mp_grouped_expert_gemm_bwd": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_i32, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_sz,
                                           c_p, c_p, c_p, c_p, c_p, c_sz, c_p]),
    "mp_mxfp8_quantize": (c_i32, [c_i64, c_i64, c_p, c_i64, c_p, c_p, c_p]),
    "mp_grouped_expert_gemm_mxfp8_workspace": (c_sz, [c_i64, c_i64, c_i64, c_i32, c_i32]),
    "mp_grouped_expert_gemm_mxfp8": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_i32, c_i32, c_p, c_p, c_p, c_p, c_p, c_p,
                                             c_p, c_p, c_p, c_p, c_p, c_sz, c_p]),
    "mp_layernorm": (c_i32, [c_i32, c_i64, c_i64, c_p, c_p, c_p, c_f32, c_p, c_p, c_p, c_p]),
    "mp_layernorm_bwd_workspace": (c_sz, [c_i64, c_i64]),
    "mp_layernorm_bwd": (c_i32, [c_i32, c_i64, c_i64, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_sz, c_p]),
}

EXPORTED = tuple(_SIGS)


class MPError(RuntimeError):
    def __init__(self, name, code, msg):
        super().__init__(f"{name} failed with {ERRORS.get(code, code)}: {msg}")
        self.code = code


def lib_path():
    return _LIB_PATH


def lib():
    """Open libmp.so (once).  A missing library is an error: there is no
    fallback path."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() first")
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _call(name, *args):
    rc = getattr(lib(), name)(*args)
    if rc != 0:
        raise MPError(name, rc, lib().mp_last_error().decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _s(stream):
    return ctypes.c_void_p((stream if stream is not None else torch.cuda.current_stream()).cuda_stream)


def _dt(t):
    if t.dtype == torch.bfloat16:
        return MP_BF16
    if t.dtype == torch.float32:
        return MP_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


# Cached scratch buffers, one per (device, stream handle), least recently
# used first; at most _WS_ENTRIES are kept.
_WS_ENTRIES = 8
_ws_cache = collections.OrderedDict()


def _stream_of(stream, dev):
    return stream if stream is not None else torch.cuda.current_stream(dev)


def workspace(nbytes, device=None, stream=None):
    """A cached device byte buffer of at least ``nbytes``, one per (device,
    stream): calls enqueued on one stream run in order and may share it; calls
    on different streams get different buffers.  Its contents do not survive
    the next call that uses it.

    The buffer is allocated while ``stream`` is torch's current stream, so
    the caching allocator files it under that stream: when a larger request
    replaces it (or it is evicted), its memory is reused only by later work
    on the same stream, never while kernels enqueued there may still use it.
    A stream handle destroyed with work pending and issued again to a new
    stream would share the old entry, as with any tensor torch allocated on
    it."""
    if nbytes == 0:
        return None
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    strm = _stream_of(stream, dev)
    key = (dev, strm.cuda_stream)
    buf = _ws_cache.pop(key, None)
    if buf is None or buf.numel() < nbytes:
        buf = None
        with torch.cuda.stream(strm):
            buf = torch.empty(int(nbytes), dtype=torch.uint8, device=dev)
    _ws_cache[key] = buf
    while len(_ws_cache) > _WS_ENTRIES:
        _ws_cache.popitem(last=False)
    return buf


def _nbytes(t):
    """Byte size of a caller's (or cached) buffer, passed to the library so
    its workspace check sees the real size."""
    return 0 if t is None else t.numel() * t.element_size()


def _act(act):
    return ACTS[act] if isinstance(act, str) else int(act)


def _ptr_array(tensors):
    arr = (ctypes.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])
    return arr


# ----------------------------------------------------------------- utilities

def mp_version():
    return lib().mp_version()


def mp_device_supported(device=0):
    return lib().mp_device_supported(device)


def mp_last_error():
    return lib().mp_last_error().decode()


def mp_check_indices(idx, lo, hi, bad_count, stream=None):
    """Counts the entries of the int32 device tensor ``idx`` outside
    [lo, hi) into ``bad_count`` (a one-element int64 device tensor),
    asynchronously on ``stream``."""
    _call("mp_check_indices", _p(idx), idx.numel(), lo, hi, _p(bad_count), _s(stream))


# -------------------------------------------------------------- MLP pieces

def mp_column_linear_gelu(X, A_i, a_i, act, Y_i, Z_save=None, stream=None):
    T, K = X.shape
    Fi = A_i.shape[0]
    _call("mp_column_linear_gelu", _dt(X), _dt(Y_i), T, K, Fi, _p(X), _p(A_i), _p(a_i), _act(act), _p(Y_i),
          _p(Z_save), _s(stream))


def mp_column_linear_gelu_bwd(X, A_i, Z_save, dY_i, act, dX_partial, dA_i, da_i=None, ws=None, stream=None):
    T, K = X.shape
    Fi = A_i.shape[0]
    dt = _dt(X)
    need = lib().mp_column_linear_gelu_bwd_workspace(dt, T, K, Fi)
    ws = ws if ws is not None else workspace(need, X.device, stream)
    _call("mp_column_linear_gelu_bwd", dt, T, K, Fi, _p(X), _p(A_i), _p(Z_save), _p(dY_i), _act(act),
          _p(dX_partial), _p(dA_i), _p(da_i), _p(ws), _nbytes(ws), _s(stream))


def mp_row_linear_partial(Y_i, B_i, P_i, stream=None):
    T, Fi = Y_i.shape
    K = B_i.shape[0]
    _call("mp_row_linear_partial", _dt(Y_i), T, Fi, K, _p(Y_i), _p(B_i), _p(P_i), _s(stream))


def mp_row_linear_partial_bwd(Y_i, B_i, dOut, dY_i, dB_i, ws=None, stream=None):
    T, Fi = Y_i.shape
    K = B_i.shape[0]
    dt = _dt(Y_i)
    need = lib().mp_row_linear_partial_bwd_workspace(dt, T, Fi, K)
    ws = ws if ws is not None else workspace(need, Y_i.device, stream)
    _call("mp_row_linear_partial_bwd", dt, T, Fi, K, _p(Y_i), _p(B_i), _p(dOut), _p(dY_i), _p(dB_i), _p(ws),
          _nbytes(ws), _s(stream))


def mp_row_linear_partial_bwd_static(Y_i, B_i, dOut, dY_i, dB_i, stream=None):
    """mp_row_linear_partial_bwd on the library's static scratch: no
    workspace argument, nothing allocated (for code under graph capture or
    other callers that cannot allocate).  Calls overlapping on one GPU race."""
    T, Fi = Y_i.shape
    K = B_i.shape[0]
    _call("mp_row_linear_partial_bwd_static", _dt(Y_i), T, Fi, K, _p(Y_i), _p(B_i), _p(dOut), _p(dY_i), _p(dB_i),
          _s(stream))


def mp_row_linear_partial_bwd_dact(Y_i, B_i, dOut, Z_save, act, dZ_i, dB_i, ws=None, stream=None):
    T, Fi = Y_i.shape
    K = B_i.shape[0]
    dt = _dt(Y_i)
    need = lib().mp_row_linear_partial_bwd_workspace(dt, T, Fi, K)
    ws = ws if ws is not None else workspace(need, Y_i.device, stream)
    _call("mp_row_linear_partial_bwd_dact", dt, T, Fi, K, _p(Y_i), _p(B_i), _p(dOut), _p(Z_save), _act(act),
          _p(dZ_i), _p(dB_i), _p(ws), _nbytes(ws), _s(stream))


# ------------------------------------------------------- reduce and dropout

def mp_shard_reduce(partials, out, bias=None, residual=None, p=0.0, seed=0, offset=0, index_base=0,
                    mask_out=None, stream=None):
    rows, cols = partials[0].shape
    arr = _ptr_array(partials)
    _call("mp_shard_reduce", _dt(partials[0]), len(partials), rows, cols, arr, _p(bias), _p(residual), p, seed,
          offset, index_base, _p(out), _p(mask_out), _s(stream))


def mp_shard_reduce_layernorm(partials, out, gamma, beta, y, mean=None, rstd=None, bias=None, residual=None, p=0.0,
                              seed=0, offset=0, index_base=0, mask_out=None, eps=1e-5, stream=None):
    rows, cols = partials[0].shape
    arr = _ptr_array(partials)
    _call("mp_shard_reduce_layernorm", _dt(partials[0]), len(partials), rows, cols, arr, _p(bias), _p(residual), p,
          seed, offset, index_base, _p(out), _p(mask_out), _p(gamma), _p(beta), eps, _p(y), _p(mean), _p(rstd),
          _s(stream))


def mp_shard_reduce_layernorm_bwd(partials, x, gamma, mean, rstd, dx, dres=None, dgamma=None, dbeta=None, ws=None,
                                  stream=None):
    rows, cols = x.shape
    arr = _ptr_array(partials)
    need = lib().mp_shard_reduce_layernorm_bwd_workspace(rows, cols) if (dgamma is not None or dbeta is not None) \
        else 0
    ws = ws if ws is not None else workspace(need, x.device, stream)
    _call("mp_shard_reduce_layernorm_bwd", _dt(x), len(partials), rows, cols, arr, _p(x), _p(gamma), _p(mean),
          _p(rstd), _p(dres), _p(dx), _p(dgamma), _p(dbeta), _p(ws), _nbytes(ws), _s(stream))


def mp_shard_reduce_layernorm_bwd_dropout(partials, x, gamma, mean, rstd, dx, p, keep_bits, ddrop, dres=None,
                                          dgamma=None, dbeta=None, dbias=None, ws=None, stream=None):
    rows, cols = x.shape
    arr = _ptr_array(partials)
    params = dgamma is not None or dbeta is not None or dbias is not None
    need = lib().mp_shard_reduce_layernorm_bwd_workspace(rows, cols) if params else 0
    ws = ws if ws is not None else workspace(need, x.device, stream)
    _call("mp_shard_reduce_layernorm_bwd_dropout", _dt(x), len(partials), rows, cols, arr, _p(x), _p(gamma), _p(mean),
          _p(rstd), _p(dres), _p(dx), _p(dgamma), _p(dbeta), p, _p(keep_bits), _p(ddrop), _p(dbias), _p(ws),
          _nbytes(ws), _s(stream))


def mp_vocab_parallel_embedding_bwd(ids, dOut, v_start, dE_i, accumulate=False, stream=None):
    T, K = dOut.shape
    Vi = dE_i.shape[0]
    _call("mp_vocab_parallel_embedding_bwd", _dt(dOut), T, Vi, v_start, K, _p(ids), _p(dOut), _p(dE_i),
          int(bool(accumulate)), _s(stream))


def mp_all_gather_rows(slices, out, stream=None):
    rows, cols = slices[0].shape
    _call("mp_all_gather_rows", _dt(out), len(slices), rows, cols, _ptr_array(slices), _p(out), _s(stream))


def mp_dropout_mask_bwd(dy, keep_bits, p, dx, dbias=None, ws=None, stream=None):
    rows, cols = dy.shape
    need = lib().mp_dropout_mask_bwd_workspace(rows, cols) if dbias is not None else 0
    ws = ws if ws is not None else workspace(need, dy.device, stream)
    _call("mp_dropout_mask_bwd", _dt(dy), rows, cols, _p(dy), _p(keep_bits), p, _p(dx), _p(dbias), _p(ws),
          _nbytes(ws), _s(stream))


def mp_shared_seed_dropout(x, y, p, seed, offset, index_base=0, mask_out=None, stream=None):
    _call("mp_shared_seed_dropout", _dt(x), x.numel(), _p(x), _p(y), _p(mask_out), p, seed, offset, index_base,
          _s(stream))


def mp_bias_grad(dy, db, ws=None, stream=None):
    rows, cols = dy.shape
    need = lib().mp_bias_grad_workspace(rows, cols)
    ws = ws if ws is not None else workspace(need, dy.device, stream)
    _call("mp_bias_grad", _dt(dy), rows, cols, _p(dy), _p(db), _p(ws), _nbytes(ws), _s(stream))


# ---------------------------------------------------------------- attention

def mp_head_attention(X, Wqkv_i, bqkv_i, B, L, h, d, ctx_i, qkv, lse, causal=True, stream=None):
    K = X.shape[1]
    _call("mp_head_attention", _dt(X), B, L, K, h, d, int(causal), _p(X), _p(Wqkv_i), _p(bqkv_i), _p(ctx_i),
          _p(qkv), _p(lse), _s(stream))


def mp_head_attention_bwd(X, Wqkv_i, qkv, ctx_i, lse, dctx_i, B, L, h, d, dX_partial, dWqkv_i, dbqkv_i=None,
                          causal=True, ws=None, stream=None):
    K = X.shape[1]
    dt = _dt(X)
    need = lib().mp_head_attention_bwd_workspace(dt, B, L, K, h, d)
    ws = ws if ws is not None else workspace(need, X.device, stream)
    _call("mp_head_attention_bwd", dt, B, L, K, h, d, int(causal), _p(X), _p(Wqkv_i), _p(qkv), _p(ctx_i), _p(lse),
          _p(dctx_i), _p(dX_partial), _p(dWqkv_i), _p(dbqkv_i), _p(ws), _nbytes(ws), _s(stream))


# ------------------------------------------------------------- vocab path

def mp_vocab_parallel_embedding(ids, E_i, v_start, out_partial, stream=None):
    Vi, K = E_i.shape
    _call("mp_vocab_parallel_embedding", _dt(E_i), ids.numel(), Vi, v_start, K, _p(ids), _p(E_i),
          _p(out_partial), _s(stream))


def mp_vocab_parallel_xent(Z_i, labels, v_start, triples, stream=None):
    T, Vi = Z_i.shape
    _call("mp_vocab_parallel_xent", T, Vi, v_start, _p(Z_i), _p(labels), _p(triples), _s(stream))


def mp_vocab_parallel_logits_xent(H, E_i, labels, v_start, triples, ws=None, stream=None):
    T, K = H.shape
    Vi = E_i.shape[0]
    need = lib().mp_vocab_parallel_logits_xent_workspace(T, K, Vi)
    ws = ws if ws is not None else workspace(need, H.device, stream)
    _call("mp_vocab_parallel_logits_xent", _dt(H), T, K, Vi, v_start, _p(H), _p(E_i), _p(labels), _p(triples), _p(ws),
          _nbytes(ws), _s(stream))


def mp_vocab_xent_combine(triples, loss, stats=None, mean_loss=None, stream=None):
    arr = _ptr_array(triples)
    _call("mp_vocab_xent_combine", len(triples), loss.numel(), arr, _p(loss), _p(stats), _p(mean_loss),
          _s(stream))


def mp_vocab_parallel_xent_bwd(Z_i, labels, v_start, stats, g, dZ_i, stream=None):
    T, Vi = Z_i.shape
    _call("mp_vocab_parallel_xent_bwd", T, Vi, v_start, _p(Z_i), _p(labels), _p(stats), g, _dt(dZ_i), _p(dZ_i),
          _s(stream))


# ---------------------------------------------------------------------- MoE

def _grouped_expert_gemm(name, X, topk_ids, topk_w, W_gu, W_d, e_start, out, perm_picks, expert_offsets, ws,
                         stream):
    T, Hd = X.shape
    topk = topk_ids.shape[1]
    E_loc, two_fe, _ = W_gu.shape
    Fe = two_fe // 2
    need = lib().mp_grouped_expert_gemm_workspace(T, Hd, Fe, topk, E_loc)
    ws = ws if ws is not None else workspace(need, X.device, stream)
    _call(name, T, Hd, Fe, topk, E_loc, e_start, _p(X), _p(topk_ids), _p(topk_w), _p(W_gu),
          _p(W_d), _p(out), _p(perm_picks), _p(expert_offsets), _p(ws), _nbytes(ws), _s(stream))


def mp_grouped_expert_gemm(X, topk_ids, topk_w, W_gu, W_d, e_start, out, perm_picks=None, expert_offsets=None,
                           ws=None, stream=None):
    _grouped_expert_gemm("mp_grouped_expert_gemm", X, topk_ids, topk_w, W_gu, W_d, e_start, out, perm_picks,
                         expert_offsets, ws, stream)


def mp_grouped_expert_gemm_weighted_act(X, topk_ids, topk_w, W_gu, W_d, e_start, out, perm_picks=None,
                                        expert_offsets=None, ws=None, stream=None):
    _grouped_expert_gemm("mp_grouped_expert_gemm_weighted_act", X, topk_ids, topk_w, W_gu, W_d, e_start, out,
                         perm_picks, expert_offsets, ws, stream)


def mp_grouped_expert_gemm_fwd_train(X, topk_ids, topk_w, W_gu, W_d, e_start, out, gu_save, ws=None, stream=None,
                                     weighted_act=False):
    """Training forward (``weighted_act``: the memory-efficient form);
    returns the workspace, which holds the state the matching backward reads
    (keep it and gu_save until then).  It is a buffer of its own, not the
    shared scratch of :func:`workspace`."""
    name = "mp_grouped_expert_gemm_weighted_act_fwd_train" if weighted_act else "mp_grouped_expert_gemm_fwd_train"
    T, Hd = X.shape
    topk = topk_ids.shape[1]
    E_loc, two_fe, _ = W_gu.shape
    Fe = two_fe // 2
    need = lib().mp_grouped_expert_gemm_workspace(T, Hd, Fe, topk, E_loc)
    if ws is None:
        with torch.cuda.stream(_stream_of(stream, X.device)):
            ws = torch.empty(max(int(need), 1), dtype=torch.uint8, device=X.device)
    _call(name, T, Hd, Fe, topk, E_loc, e_start, _p(X), _p(topk_ids), _p(topk_w),
          _p(W_gu), _p(W_d), _p(out), _p(gu_save), _p(ws), _nbytes(ws),
          _s(stream))
    return ws


def mp_grouped_expert_gemm_bwd(X, topk_w, W_gu, W_d, dOut, gu_save, fwd_ws, dX, dW_gu, dW_d, dtopk_w, ws=None,
                               stream=None, weighted_act=False):
    name = "mp_grouped_expert_gemm_weighted_act_bwd" if weighted_act else "mp_grouped_expert_gemm_bwd"
    T, Hd = X.shape
    topk = topk_w.shape[1]
    E_loc, two_fe, _ = W_gu.shape
    Fe = two_fe // 2
    need = lib().mp_grouped_expert_gemm_bwd_workspace(T, Hd, Fe, topk, E_loc)
    ws = ws if ws is not None else workspace(need, X.device, stream)
    _call(name, T, Hd, Fe, topk, E_loc, _p(X), _p(topk_w), _p(W_gu), _p(W_d), _p(dOut),
          _p(gu_save), _p(fwd_ws), _nbytes(fwd_ws), _p(dX),
          _p(dW_gu), _p(dW_d), _p(dtopk_w), _p(ws), _nbytes(ws),
          _s(stream))


# ------------------------------------------------------------------ MXFP8

def mxfp8_scale_width(K):
    return 4 * ((K + 127) // 128)


def mp_mxfp8_quantize(x, q, scales, stream=None):
    rows, K = x.shape
    _call("mp_mxfp8_quantize", rows, K, _p(x), x.stride(0), _p(q), _p(scales), _s(stream))


def mp_grouped_expert_gemm_mxfp8(X, topk_ids, topk_w, W_gu_q, W_gu_s, W_d_q, W_d_s, e_start, out, perm_picks=None,
                                 expert_offsets=None, ws=None, stream=None):
    T, Hd = X.shape
    topk = topk_ids.shape[1]
    E_loc, two_fe, _ = W_gu_q.shape
    Fe = two_fe // 2
    need = lib().mp_grouped_expert_gemm_mxfp8_workspace(T, Hd, Fe, topk, E_loc)
    ws = ws if ws is not None else workspace(need, X.device, stream)
    _call("mp_grouped_expert_gemm_mxfp8", T, Hd, Fe, topk, E_loc, e_start, _p(X), _p(topk_ids), _p(topk_w),
          _p(W_gu_q), _p(W_gu_s), _p(W_d_q), _p(W_d_s), _p(out), _p(perm_picks), _p(expert_offsets), _p(ws),
          _nbytes(ws), _s(stream))


# ---------------------------------------------------------------- LayerNorm

def mp_layernorm(x, gamma, beta, y, mean=None, rstd=None, eps=1e-5, stream=None):
    T, K = x.shape
    _call("mp_layernorm", _dt(x), T, K, _p(x), _p(gamma), _p(beta), eps, _p(y), _p(mean), _p(rstd), _s(stream))


def mp_layernorm_bwd(x, gamma, mean, rstd, dy, dx, dres=None, dgamma=None, dbeta=None, ws=None, stream=None):
    T, K = x.shape
    need = lib().mp_layernorm_bwd_workspace(T, K) if (dgamma is not None or dbeta is not None) else 0
    ws = ws if ws is not None else workspace(need, x.device, stream)
    _call("mp_layernorm_bwd", _dt(x), T, K, _p(x), _p(gamma), _p(mean), _p(rstd), _p(dy), _p(dres), _p(dx),
          _p(dgamma), _p(dbeta), _p(ws), _nbytes(ws), _s(stream))
