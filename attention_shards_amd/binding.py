"""Thin ctypes binding of libtpshard.so (the C ABI in include/tp_shard.h).

Argument marshalling only: torch tensors are turned into device pointers,
sizes and dtype codes, the current HIP stream is passed along, and a
non-success status is raised as TPError.  Every step of the computation runs
in the library's HIP kernels; there is no fallback path.  If the library is
missing, load() raises.

The functions carry the C names.  Shapes are taken from the tensors and
checked against each other here, because the C side only sees pointers.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtpshard.so")

TP_F32 = 0
TP_BF16 = 1
TP_MAX_PARTIALS = 64

STATUS = {
    0: "TP_SUCCESS", 1: "TP_ERR_NULL", 2: "TP_ERR_SHAPE", 3: "TP_ERR_SHARD",
    4: "TP_ERR_DIVISIBILITY", 5: "TP_ERR_DTYPE", 6: "TP_ERR_WORKSPACE",
    7: "TP_ERR_ALIAS", 8: "TP_ERR_HIP", 9: "TP_ERR_UNSUPPORTED",
    10: "TP_ERR_ALIGNMENT",
}

# name -> (restype, argtypes); mirrors include/tp_shard.h
_c_i64, _c_i32, _c_sz, _c_p = ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
SIGNATURES = {
    "tp_ffn_shard_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i32, _c_i32]),
    "tp_ffn_shard": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32,
                              _c_i32, _c_i64, _c_i32, _c_i32, _c_p, _c_sz, _c_p]),
    "tp_attn_shard_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i32, _c_i32, _c_i32]),
    "tp_attn_shard": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i32,
                               _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_p,
                               _c_sz, _c_p]),
    "tp_partial_reduce": (_c_i32, [ctypes.POINTER(_c_p), _c_i32, _c_p, _c_p, _c_i64,
                                   _c_i64, _c_i32, _c_i32, _c_i32, _c_p]),
    "tp_partial_reduce_slice": (_c_i32, [ctypes.POINTER(_c_p), _c_i32, _c_p, _c_p, _c_i64,
                                         _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                         _c_p]),
    "tp_ffn_shard_reduce_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i32, _c_i32]),
    "tp_ffn_shard_reduce": (_c_i32, [_c_p, _c_p, _c_p, ctypes.POINTER(_c_p), _c_p, _c_p,
                                     _c_i64, _c_i64, _c_i64, _c_i32, _c_i32, _c_i64, _c_i32,
                                     _c_i32, _c_i32, _c_i32, _c_p, _c_sz, _c_p]),
    "tp_ffn_shard_noalloc": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64,
                                      _c_i32, _c_i32, _c_i64, _c_i32, _c_i32, _c_p]),
    "tp_sp_reduce_layernorm": (_c_i32, [ctypes.POINTER(_c_p), _c_i32, _c_p, _c_p, _c_p, _c_p,
                                        _c_p, ctypes.c_float, _c_i64, _c_i64, _c_i32, _c_i32,
                                        _c_i32, _c_i32, _c_i32, _c_i32, _c_p]),
    "tp_status_string": (ctypes.c_char_p, [_c_i32]),
    "tp_last_error_message": (ctypes.c_char_p, []),
    "tp_abi_version": (_c_i32, []),
}

_lib = None


class TPError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


def load() -> ctypes.CDLL:
    """Load libtpshard.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m attention_shards_amd.build`")
        # PyTorch ships its own HIP runtime with the same soname as the
        # system one; importing it first makes this library bind to the
        # runtime torch's tensors and streams live in.
        _torch()
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int) -> None:
    if status != 0:
        msg = load().tp_last_error_message().decode()
        raise TPError(status, msg)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return TP_F32
    if t.dtype == torch.bfloat16:
        return TP_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return t


def _dense(t, name: str):
    _dev(t, name)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _same_device(device, **tensors):
    """Every tensor on `device`: the kernels run there and take the others'
    addresses as its own."""
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, the call runs on {device}")


def _stream_of(stream, device):
    """The torch stream the call is enqueued on: the current stream of
    `device` for None, a torch stream as given, or a raw hipStream_t handle
    (int; 0 is the device's default stream) wrapped as an external stream.
    Temporaries a call allocates (its workspace) are allocated while this
    stream is current, so the caching allocator only hands their memory out
    again in this stream's order, after the call's kernels."""
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, int):
        if stream == 0:
            return torch.cuda.default_stream(device)
        return torch.cuda.ExternalStream(stream, device=device)
    return stream


def tp_ffn_shard_workspace_bytes(tokens: int, hidden: int, ffn: int, t: int,
                                 in_dtype: int) -> int:
    return int(load().tp_ffn_shard_workspace_bytes(tokens, hidden, ffn, t, in_dtype))


def tp_ffn_shard_reduce_workspace_bytes(tokens: int, hidden: int, ffn: int, t: int,
                                        in_dtype: int) -> int:
    return int(load().tp_ffn_shard_reduce_workspace_bytes(tokens, hidden, ffn, t, in_dtype))


def tp_attn_shard_workspace_bytes(batch: int, seq: int, n_heads: int,
                                  head_dim: int, t: int) -> int:
    return int(load().tp_attn_shard_workspace_bytes(batch, seq, n_heads, head_dim, t))


def _workspace(ws, nbytes: int, device):
    torch = _torch()
    if ws is None:
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    _dense(ws, "workspace")
    _same_device(device, workspace=ws)
    return ws


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def tp_ffn_shard(X, W1_i, W2_i, Y_i, i: int, t: int, workspace=None,
                 stream=None):
    """Y_i = GeLU(X W1_i) W2_i on the GPU.

    W1_i may be a column view of a full W1 (stride(1) == 1, any stride(0)).
    Returns Y_i.
    """
    lib = load()
    _dense(X, "X")
    _dense(W2_i, "W2_i")
    _dense(Y_i, "Y_i")
    _dev(W1_i, "W1_i")
    if W1_i.dim() != 2 or W1_i.stride(1) != 1:
        raise ValueError("W1_i must be 2-D with unit column stride")
    tokens, hidden = X.shape
    fs = W1_i.shape[1]
    if W1_i.shape[0] != hidden or tuple(W2_i.shape) != (fs, hidden) or \
            tuple(Y_i.shape) != (tokens, hidden):
        raise ValueError(f"shape mismatch: X{tuple(X.shape)} W1_i{tuple(W1_i.shape)} "
                         f"W2_i{tuple(W2_i.shape)} Y_i{tuple(Y_i.shape)}")
    in_dt = _dtype_code(X)
    if _dtype_code(W1_i) != in_dt or _dtype_code(W2_i) != in_dt:
        raise TypeError("X, W1_i and W2_i must share a dtype")
    _same_device(X.device, W1_i=W1_i, W2_i=W2_i, Y_i=Y_i)
    ffn = fs * t
    need = tp_ffn_shard_workspace_bytes(tokens, hidden, ffn, t, in_dt)
    torch = _torch()
    s = _stream_of(stream, X.device)
    with torch.cuda.device(X.device), torch.cuda.stream(s):
        ws = _workspace(workspace, need, X.device)
        _check(lib.tp_ffn_shard(X.data_ptr(), W1_i.data_ptr(), W2_i.data_ptr(),
                                Y_i.data_ptr(), tokens, hidden, ffn, i, t,
                                W1_i.stride(0), in_dt, _dtype_code(Y_i),
                                ws.data_ptr(), _nbytes(ws), s.cuda_stream))
    return Y_i


TP_FFN_NOALLOC_MAX_WORKSPACE = 64 << 20


def tp_ffn_shard_noalloc(X, W1_i, W2_i, Y_i, i: int, t: int, stream=None):
    """Y_i = GeLU(X W1_i) W2_i through tp_ffn_shard_noalloc: no workspace,
    nothing allocated (GeLU(Z_i) lives in the library's own device array of
    TP_FFN_NOALLOC_MAX_WORKSPACE bytes).  Returns Y_i."""
    lib = load()
    _dense(X, "X")
    _dense(W2_i, "W2_i")
    _dense(Y_i, "Y_i")
    _dev(W1_i, "W1_i")
    if W1_i.dim() != 2 or W1_i.stride(1) != 1:
        raise ValueError("W1_i must be 2-D with unit column stride")
    tokens, hidden = X.shape
    fs = W1_i.shape[1]
    if W1_i.shape[0] != hidden or tuple(W2_i.shape) != (fs, hidden) or \
            tuple(Y_i.shape) != (tokens, hidden):
        raise ValueError(f"shape mismatch: X{tuple(X.shape)} W1_i{tuple(W1_i.shape)} "
                         f"W2_i{tuple(W2_i.shape)} Y_i{tuple(Y_i.shape)}")
    in_dt = _dtype_code(X)
    if _dtype_code(W1_i) != in_dt or _dtype_code(W2_i) != in_dt:
        raise TypeError("X, W1_i and W2_i must share a dtype")
    _same_device(X.device, W1_i=W1_i, W2_i=W2_i, Y_i=Y_i)
    torch = _torch()
    s = _stream_of(stream, X.device)
    with torch.cuda.device(X.device):
        _check(lib.tp_ffn_shard_noalloc(X.data_ptr(), W1_i.data_ptr(), W2_i.data_ptr(),
                                        Y_i.data_ptr(), tokens, hidden, fs * t, i, t,
                                        W1_i.stride(0), in_dt, _dtype_code(Y_i),
                                        s.cuda_stream))
    return Y_i


def tp_ffn_shard_reduce(X, W1_i, W2_i, peer_partials, residual, out, i: int,
                        workspace=None, stream=None):
    """out = (sum_{j != i} P_j + residual) + P_i with P_i = GeLU(X W1_i) W2_i
    computed here and added unrounded; peer_partials is the list of the t
    partials (entry i is not read and may be None).  Returns out."""
    lib = load()
    t = len(peer_partials)
    if not 1 <= t <= TP_MAX_PARTIALS:
        raise ValueError(f"need 1..{TP_MAX_PARTIALS} partials, got {t}")
    _dense(X, "X")
    _dense(W2_i, "W2_i")
    _dense(out, "out")
    _dev(W1_i, "W1_i")
    if W1_i.dim() != 2 or W1_i.stride(1) != 1:
        raise ValueError("W1_i must be 2-D with unit column stride")
    tokens, hidden = X.shape
    fs = W1_i.shape[1]
    if W1_i.shape[0] != hidden or tuple(W2_i.shape) != (fs, hidden) or \
            tuple(out.shape) != (tokens, hidden):
        raise ValueError(f"shape mismatch: X{tuple(X.shape)} W1_i{tuple(W1_i.shape)} "
                         f"W2_i{tuple(W2_i.shape)} out{tuple(out.shape)}")
    in_dt = _dtype_code(X)
    if _dtype_code(W1_i) != in_dt or _dtype_code(W2_i) != in_dt:
        raise TypeError("X, W1_i and W2_i must share a dtype")
    peers = [p for k, p in enumerate(peer_partials) if k != i]
    pdt = TP_F32
    for k, p in enumerate(peer_partials):
        if k == i:
            continue
        _dense(p, f"peer_partials[{k}]")
        if tuple(p.shape) != (tokens, hidden):
            raise ValueError(f"peer_partials[{k}] shape {tuple(p.shape)} != {(tokens, hidden)}")
    if peers:
        pdt = _dtype_code(peers[0])
        if any(_dtype_code(p) != pdt for p in peers):
            raise TypeError("all peer partials must share a dtype")
    rdt, rptr = TP_F32, None
    if residual is not None:
        _dense(residual, "residual")
        if tuple(residual.shape) != (tokens, hidden):
            raise ValueError("residual shape mismatch")
        rdt, rptr = _dtype_code(residual), residual.data_ptr()
    _same_device(X.device, W1_i=W1_i, W2_i=W2_i, out=out, residual=residual,
                 **{f"peer_partials[{k}]": p for k, p in enumerate(peer_partials) if k != i})
    arr = (ctypes.c_void_p * t)(*[None if (k == i or p is None) else p.data_ptr()
                                  for k, p in enumerate(peer_partials)])
    ffn = fs * t
    need = tp_ffn_shard_reduce_workspace_bytes(tokens, hidden, ffn, t, in_dt)
    torch = _torch()
    s = _stream_of(stream, X.device)
    with torch.cuda.device(X.device), torch.cuda.stream(s):
        ws = _workspace(workspace, need, X.device)
        _check(lib.tp_ffn_shard_reduce(X.data_ptr(), W1_i.data_ptr(), W2_i.data_ptr(), arr,
                                       rptr, out.data_ptr(), tokens, hidden, ffn, i, t,
                                       W1_i.stride(0), in_dt, pdt, rdt, _dtype_code(out),
                                       ws.data_ptr(), _nbytes(ws), s.cuda_stream))
    return out


def tp_attn_shard(X, Wqkv_i, Wo_i, Y_i, batch: int, seq: int, n_heads: int,
                  head_dim: int, i: int, t: int, causal: bool = True,
                  workspace=None, stream=None):
    """Y_i = concat_h(softmax(Q_h K_h^T/sqrt d) V_h) Wo_i for this GPU's heads.

    Wqkv_i is the held [hidden, 3*nl*d] buffer laid out [W_Q,i | W_K,i | W_V,i].
    Returns Y_i.
    """
    lib = load()
    for name, tens in (("X", X), ("Wqkv_i", Wqkv_i), ("Wo_i", Wo_i), ("Y_i", Y_i)):
        _dense(tens, name)
    nl = n_heads // t if t > 0 else 0
    hidden = X.shape[1]
    if tuple(X.shape) != (batch * seq, hidden) or \
            tuple(Wqkv_i.shape) != (hidden, 3 * nl * head_dim) or \
            tuple(Wo_i.shape) != (nl * head_dim, hidden) or \
            tuple(Y_i.shape) != (batch * seq, hidden):
        raise ValueError(f"shape mismatch: X{tuple(X.shape)} Wqkv_i{tuple(Wqkv_i.shape)} "
                         f"Wo_i{tuple(Wo_i.shape)} Y_i{tuple(Y_i.shape)}")
    if _dtype_code(Wqkv_i) != _dtype_code(X) or _dtype_code(Wo_i) != _dtype_code(X):
        raise TypeError("X, Wqkv_i and Wo_i must share a dtype")
    _same_device(X.device, Wqkv_i=Wqkv_i, Wo_i=Wo_i, Y_i=Y_i)
    torch = _torch()
    s = _stream_of(stream, X.device)
    with torch.cuda.device(X.device), torch.cuda.stream(s):
        need = tp_attn_shard_workspace_bytes(batch, seq, n_heads, head_dim, t)
        ws = _workspace(workspace, need, X.device)
        _check(lib.tp_attn_shard(X.data_ptr(), Wqkv_i.data_ptr(), Wo_i.data_ptr(),
                                 Y_i.data_ptr(), batch, seq, hidden, n_heads,
                                 head_dim, i, t, 1 if causal else 0,
                                 _dtype_code(X), _dtype_code(Y_i), ws.data_ptr(),
                                 _nbytes(ws), s.cuda_stream))
    return Y_i


def tp_partial_reduce(partials, residual, out, stream=None, slice_of=None):
    """out = sum(partials) + residual (residual may be None).  Returns out.
    slice_of=(slice, nslices) computes only that row block (see
    tp_partial_reduce_slice)."""
    lib = load()
    t = len(partials)
    if not 1 <= t <= TP_MAX_PARTIALS:
        raise ValueError(f"need 1..{TP_MAX_PARTIALS} partials, got {t}")
    _dense(out, "out")
    rows, cols = out.shape
    for k, p in enumerate(partials):
        _dense(p, f"partials[{k}]")
        if tuple(p.shape) != (rows, cols):
            raise ValueError(f"partials[{k}] shape {tuple(p.shape)} != {(rows, cols)}")
    pdt = _dtype_code(partials[0])
    if any(_dtype_code(p) != pdt for p in partials):
        raise TypeError("all partials must share a dtype")
    rdt = TP_F32
    rptr = None
    if residual is not None:
        _dense(residual, "residual")
        if tuple(residual.shape) != (rows, cols):
            raise ValueError("residual shape mismatch")
        rdt = _dtype_code(residual)
        rptr = residual.data_ptr()
    _same_device(out.device, residual=residual,
                 **{f"partials[{k}]": p for k, p in enumerate(partials)})
    arr = (ctypes.c_void_p * t)(*[p.data_ptr() for p in partials])
    torch = _torch()
    s = _stream_of(stream, out.device)
    with torch.cuda.device(out.device):
        if slice_of is None:
            _check(lib.tp_partial_reduce(arr, t, rptr, out.data_ptr(), rows, cols, pdt,
                                         rdt, _dtype_code(out), s.cuda_stream))
        else:
            slice_, nslices = slice_of
            _check(lib.tp_partial_reduce_slice(arr, t, rptr, out.data_ptr(), rows, cols,
                                               slice_, nslices, pdt, rdt, _dtype_code(out),
                                               s.cuda_stream))
    return out


def tp_partial_reduce_slice(partials, residual, out, slice_, nslices, stream=None):
    """Rows block `slice_` of `nslices` of sum(partials) + residual, written into
    the same rows of out (the reduce-scatter half of the all-reduce).  Returns out."""
    return tp_partial_reduce(partials, residual, out, stream, slice_of=(slice_, nslices))


def tp_sp_reduce_layernorm(partials, residual, x_out, ln_out, gamma=None, beta=None,
                           eps: float = 1e-5, slice_of=(0, 1), stream=None):
    """Rows block slice_of = (slice, nslices) of x = sum(partials) + residual and
    y = LayerNorm(x) (per row; gamma/beta fp32 [cols] or None), written into
    the same rows of x_out (may be None) and ln_out.  Returns ln_out."""
    lib = load()
    t = len(partials)
    if not 1 <= t <= TP_MAX_PARTIALS:
        raise ValueError(f"need 1..{TP_MAX_PARTIALS} partials, got {t}")
    _dense(ln_out, "ln_out")
    rows, cols = ln_out.shape
    for k, p in enumerate(partials):
        _dense(p, f"partials[{k}]")
        if tuple(p.shape) != (rows, cols):
            raise ValueError(f"partials[{k}] shape {tuple(p.shape)} != {(rows, cols)}")
    pdt = _dtype_code(partials[0])
    if any(_dtype_code(p) != pdt for p in partials):
        raise TypeError("all partials must share a dtype")
    rdt, rptr = TP_F32, None
    if residual is not None:
        _dense(residual, "residual")
        if tuple(residual.shape) != (rows, cols):
            raise ValueError("residual shape mismatch")
        rdt, rptr = _dtype_code(residual), residual.data_ptr()
    xdt, xptr = TP_F32, None
    if x_out is not None:
        _dense(x_out, "x_out")
        if tuple(x_out.shape) != (rows, cols):
            raise ValueError("x_out shape mismatch")
        xdt, xptr = _dtype_code(x_out), x_out.data_ptr()
    torch = _torch()
    gb = []
    for name, v in (("gamma", gamma), ("beta", beta)):
        if v is None:
            gb.append(None)
            continue
        _dense(v, name)
        if v.dtype != torch.float32 or tuple(v.shape) != (cols,):
            raise ValueError(f"{name} must be float32 [{cols}]")
        gb.append(v.data_ptr())
    _same_device(ln_out.device, residual=residual, x_out=x_out, gamma=gamma, beta=beta,
                 **{f"partials[{k}]": p for k, p in enumerate(partials)})
    arr = (ctypes.c_void_p * t)(*[p.data_ptr() for p in partials])
    s = _stream_of(stream, ln_out.device)
    slice_, nslices = slice_of
    with torch.cuda.device(ln_out.device):
        _check(lib.tp_sp_reduce_layernorm(arr, t, rptr, xptr, ln_out.data_ptr(), gb[0], gb[1],
                                          float(eps), rows, cols, slice_, nslices, pdt, rdt,
                                          xdt, _dtype_code(ln_out), s.cuda_stream))
    return ln_out
