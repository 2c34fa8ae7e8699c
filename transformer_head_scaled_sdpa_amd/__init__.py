"""MI355X (gfx950) multi-head scaled dot-product attention forward.

Thin torch-facing binding over libmha.so (C ABI in include/mha.h).  It only
marshals arguments: device pointers, strides, sizes and torch's current HIP
stream.  Every step of the computation runs in the library's HIP kernels;
there is no CPU or PyTorch fallback, and a missing library raises.

    sdpa_forward(q, k, v, valid_lens=None, causal=False, out_dtype=None,
                 return_weights=False)
        q [B,h,Lq,64], k [B,h,Lk,64], v [B,h,Lk,64] on the GPU (bf16 or fp32)
    mha_forward(x_q, x_kv, w_q, w_k, w_v, w_o, b_q=None, ..., h=8,
                valid_lens=None, causal=False, out_dtype=None,
                return_weights=False)
        x_q [B,Lq,D], x_kv [B,Lk,D], W [D,D] stored [out, in], b [D]
    mha_sublayer_forward(x, w_q, w_k, w_v, w_o, ..., ln_gain=None, ln_bias=None,
                         ln_kind=0, ln_eps=1e-6, memory=None, ...)
        x + MHA(norm(x), ...): the pre-norm residual sublayer
    sdpa_forward(..., return_lse=True) -> o, lse
        also each query's log-sum-exp [B, h, Lq] (fp32), kept for the backward
    sdpa_backward(q, k, v, o, dout, valid_lens=None, causal=False, lse=None)
        -> dq, dk, dv (gradients of sdpa_forward for the output gradient dout;
        with the forward's lse the weights are recomputed from it)
    mha_forward_train(x_q, x_kv, w_q, ..., h=8, valid_lens=None, causal=False)
        -> out, saved (Q, K, V, merged heads and statistic kept for the backward)
    mha_backward(x_q, x_kv, w_q, w_k, w_v, w_o, dout, b_q=None, ..., h=8,
                 valid_lens=None, causal=False) -> dict of fp32 gradients
        dx_q, dx_kv (None for self-attention: x_kv is x_q, dx_q holds the
        whole input gradient), dw_q, dw_k, dw_v, dw_o, db_q, ..., db_o
        (bf16 inputs; the bias gradients when b_q is given)
    sdpa_decode(q, k_cache, v_cache, lens)
        one decoding step: q [B,h,64] against caches [B,h,L,64]
    sdpa_decode_noalloc(q, k_cache, v_cache, lens, out=None)
        the same step with no workspace (for callers that cannot allocate)

valid_lens is [B] (one length per sequence) or [B, Lq] (one per query).
return_weights=True also returns the attention weights [B, h, Lq, Lk]
(fp32).  Lengths per query or the weights take the inspection path
(sdpa_forward_ex / mha_forward_ex: fp32 arithmetic, two passes).
"""
import ctypes

from . import _lib
from ._lib import MhaError, MHA_BF16, MHA_F32, MHA_OK, Strides

__all__ = ["sdpa_forward", "sdpa_backward", "sdpa_decode", "sdpa_decode_noalloc", "mha_forward", "mha_sublayer_forward", "mha_backward", "mha_forward_train", "workspace_bytes", "kernel_timing", "MhaError", "library"]


def library():
    """The loaded ctypes handle of libmha.so (raises if it is not built)."""
    return _lib.load()


def _torch():
    import torch
    return torch


def _dtype_code(dt):
    torch = _torch()
    if dt == torch.bfloat16:
        return MHA_BF16
    if dt == torch.float32:
        return MHA_F32
    raise TypeError(f"unsupported dtype {dt}: use torch.bfloat16 or torch.float32")


def _check_gpu(name, t):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _strides4(t):
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("attention operands are [B, h, L, d] views with a contiguous last axis")
    s = t.stride()
    return Strides(s[0], s[1], s[2])


def _valid_lens(valid_lens, B, device, Lq=None):
    """Lengths as a device int32 tensor: [B], or [B, Lq] when Lq is given."""
    torch = _torch()
    if valid_lens is None:
        return None
    vl = torch.as_tensor(valid_lens, dtype=torch.int32, device=device).contiguous()
    if vl.shape != (B,) and (Lq is None or vl.shape != (B, Lq)):
        raise ValueError(f"valid_lens must have shape ({B},)" + ("" if Lq is None else f" or ({B}, {Lq})"))
    return vl


def _raise(status, what):
    if status != MHA_OK:
        raise MhaError(status, what)


def sdpa_forward(q, k, v, valid_lens=None, causal=False, out_dtype=None, out=None, return_weights=False,
                 weights=None, return_lse=False):
    """softmax(q k^T / sqrt(d_k)) v per (batch, head) with key-padding
    ``valid_lens`` ([B] or [B, Lq]) and/or the causal mask; returns
    o [B, h, Lq, d_v], and the weights [B, h, Lq, Lk] (fp32) when
    ``return_weights`` (written into ``weights`` if given: an fp32 tensor of
    that shape whose last axis is contiguous), or each query's log-sum-exp
    of its scaled scores [B, h, Lq] (fp32) when ``return_lse`` (lengths per
    sequence only; not with the weights)."""
    torch = _torch()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_gpu(n, t)
    B, h, Lq, dk = q.shape
    Lk, dv = k.shape[2], v.shape[3]
    in_dt = _dtype_code(q.dtype)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, h, Lq, dv), dtype=out_dtype, device=q.device)
    vl = _valid_lens(valid_lens, B, q.device, Lq)
    lib = _lib.load()
    head = (in_dt, _dtype_code(out.dtype), _ptr(q), _strides4(q), _ptr(k), _strides4(k), _ptr(v), _strides4(v),
            _ptr(out), _strides4(out), B, h, Lq, Lk, dk, dv, _ptr(vl))
    if return_lse:
        if return_weights or (vl is not None and vl.dim() != 1):
            raise ValueError("return_lse takes lengths per sequence and no weights")
        lse = torch.empty((B, h, Lq), dtype=torch.float32, device=q.device)
        _raise(lib.sdpa_forward_lse(*head, int(bool(causal)), _ptr(lse), _stream()), "sdpa_forward_lse")
        return out, lse
    if not return_weights and (vl is None or vl.dim() == 1):
        _raise(lib.sdpa_forward(*head, int(bool(causal)), _stream()), "sdpa_forward")
        return out
    p = None
    if return_weights:
        if weights is None:
            p = torch.empty((B, h, Lq, Lk), dtype=torch.float32, device=q.device)
        else:
            _check_gpu("weights", weights)
            if weights.dtype != torch.float32 or tuple(weights.shape) != (B, h, Lq, Lk) or weights.stride(3) != 1:
                raise ValueError(f"weights must be fp32 [{B}, {h}, {Lq}, {Lk}] with a contiguous last axis")
            p = weights
    sp = _strides4(p) if p is not None else Strides(0, 0, 0)
    st = lib.sdpa_forward_ex(*head, 1 if vl is None else vl.dim(), int(bool(causal)), _ptr(p), sp, _stream())
    _raise(st, "sdpa_forward_ex")
    return (out, p) if return_weights else out


def sdpa_backward(q, k, v, o, dout, valid_lens=None, causal=False, out_dtype=None, workspace=None, lse=None):
    """Gradients (dq, dk, dv) of sdpa_forward(q, k, v, valid_lens, causal),
    whose output was ``o``, for the output gradient ``dout``; ``lse`` is the
    forward's log-sum-exp (sdpa_forward(..., return_lse=True)), if kept."""
    torch = _torch()
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_gpu(n, t)
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, o and dout must share one dtype")
    B, h, Lq, dk = q.shape
    Lk, dv = k.shape[2], v.shape[3]
    out_dtype = q.dtype if out_dtype is None else out_dtype
    gq = torch.empty((B, h, Lq, dk), dtype=out_dtype, device=q.device)
    gk = torch.empty((B, h, Lk, dk), dtype=out_dtype, device=q.device)
    gv = torch.empty((B, h, Lk, dv), dtype=out_dtype, device=q.device)
    vl = _valid_lens(valid_lens, B, q.device, Lq)
    lib = _lib.load()
    need = int(lib.sdpa_backward_workspace_bytes(B, h, Lq))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    args = []
    for t in (q, k, v, o, dout, gq, gk, gv):
        args += [_ptr(t), _strides4(t)]
    if lse is not None:
        _check_gpu("lse", lse)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, h, Lq) or not lse.is_contiguous():
            raise ValueError(f"lse must be a contiguous fp32 [{B}, {h}, {Lq}] tensor")
        st = lib.sdpa_backward_lse(_dtype_code(q.dtype), _dtype_code(out_dtype), *args, B, h, Lq, Lk, dk, dv,
                                   _ptr(vl), 1 if vl is None else vl.dim(), int(bool(causal)), _ptr(lse),
                                   _ptr(workspace), workspace.numel(), _stream())
        _raise(st, "sdpa_backward_lse")
        return gq, gk, gv
    st = lib.sdpa_backward(_dtype_code(q.dtype), _dtype_code(out_dtype), *args, B, h, Lq, Lk, dk, dv, _ptr(vl),
                           1 if vl is None else vl.dim(), int(bool(causal)), _ptr(workspace), workspace.numel(),
                           _stream())
    _raise(st, "sdpa_backward")
    return gq, gk, gv


def sdpa_decode(q, k_cache, v_cache, lens, out_dtype=None, out=None, workspace=None):
    """One decoding step: q [B, h, d_k] attends to positions 0 .. lens[b]-1 of
    the caches k_cache, v_cache [B, h, L, d]; returns o [B, h, d_v]."""
    torch = _torch()
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_gpu(n, t)
    B, h, dk = q.shape
    L, dv = k_cache.shape[2], v_cache.shape[3]
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share one dtype")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, h, dv), dtype=out_dtype, device=q.device)
    ln = _valid_lens(lens, B, q.device)
    if ln is None:
        raise ValueError("lens is required")
    lib = _lib.load()
    need = int(lib.sdpa_decode_workspace_bytes(B, h, L))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    S3 = lambda t: _lib.Strides(t.stride(0), t.stride(1), 0)
    st = lib.sdpa_decode(_dtype_code(q.dtype), _dtype_code(out.dtype), _ptr(q), S3(q), _ptr(k_cache),
                         _strides4(k_cache), _ptr(v_cache), _strides4(v_cache), _ptr(out), S3(out), B, h, L, dk, dv,
                         _ptr(ln), _ptr(workspace), workspace.numel(), _stream())
    _raise(st, "sdpa_decode")
    return out


def sdpa_decode_noalloc(q, k_cache, v_cache, lens, out_dtype=None, out=None):
    """sdpa_decode whose partial results live in the library's own device
    array (no workspace); the C entry point allocates nothing.  Pass ``out``
    and a device int32 ``lens`` to keep the whole call allocation-free."""
    torch = _torch()
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_gpu(n, t)
    B, h, dk = q.shape
    L, dv = k_cache.shape[2], v_cache.shape[3]
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share one dtype")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, h, dv), dtype=out_dtype, device=q.device)
    ln = _valid_lens(lens, B, q.device)
    if ln is None:
        raise ValueError("lens is required")
    S3 = lambda t: _lib.Strides(t.stride(0), t.stride(1), 0)
    st = _lib.load().sdpa_decode_noalloc(_dtype_code(q.dtype), _dtype_code(out.dtype), _ptr(q), S3(q),
                                         _ptr(k_cache), _strides4(k_cache), _ptr(v_cache), _strides4(v_cache),
                                         _ptr(out), S3(out), B, h, L, dk, dv, _ptr(ln), _stream())
    _raise(st, "sdpa_decode_noalloc")
    return out


def workspace_bytes(dtype, B, Lq, Lk, d_model, h):
    return int(_lib.load().mha_workspace_bytes(_dtype_code(dtype), B, Lq, Lk, d_model, h))


def mha_forward(x_q, x_kv, w_q, w_k, w_v, w_o, b_q=None, b_k=None, b_v=None, b_o=None, h=8,
                valid_lens=None, causal=False, out_dtype=None, out=None, workspace=None, return_weights=False):
    """Multi-head attention forward; returns [B, Lq, d_model], and the
    per-head weights [B, h, Lq, Lk] (fp32) when ``return_weights``."""
    torch = _torch()
    args = dict(x_q=x_q, x_kv=x_kv, w_q=w_q, w_k=w_k, w_v=w_v, w_o=w_o, b_q=b_q, b_k=b_k, b_v=b_v, b_o=b_o)
    for n, t in args.items():
        _check_gpu(n, t)
        if t is not None and (not t.is_contiguous() or t.dtype != x_q.dtype):
            raise ValueError(f"{n} must be contiguous and share x_q's dtype")
    B, Lq, D = x_q.shape
    Lk = x_kv.shape[1]
    in_dt = _dtype_code(x_q.dtype)
    out_dtype = (torch.float32 if x_q.dtype == torch.bfloat16 else x_q.dtype) if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, Lq, D), dtype=out_dtype, device=x_q.device)
    vl = _valid_lens(valid_lens, B, x_q.device, Lq)
    ex = return_weights or (vl is not None and vl.dim() == 2)
    lib = _lib.load()
    need = int((lib.mha_workspace_bytes_ex if ex else lib.mha_workspace_bytes)(in_dt, B, Lq, Lk, D, h))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x_q.device)
    head = (in_dt, _dtype_code(out.dtype), _ptr(x_q), _ptr(x_kv), _ptr(w_q), _ptr(b_q), _ptr(w_k), _ptr(b_k),
            _ptr(w_v), _ptr(b_v), _ptr(w_o), _ptr(b_o), _ptr(out), B, Lq, Lk, D, h, D // h if h else 0, _ptr(vl))
    if not ex:
        st = lib.mha_forward(*head, int(bool(causal)), _ptr(workspace), workspace.numel(), _stream())
        _raise(st, "mha_forward")
        return out
    p = torch.empty((B, h, Lq, Lk), dtype=torch.float32, device=x_q.device) if return_weights else None
    sp = _strides4(p) if p is not None else Strides(0, 0, 0)
    st = lib.mha_forward_ex(*head, 1 if vl is None else vl.dim(), int(bool(causal)), _ptr(p), sp,
                            _ptr(workspace), workspace.numel(), _stream())
    _raise(st, "mha_forward_ex")
    return (out, p) if return_weights else out


def mha_sublayer_forward(x, w_q, w_k, w_v, w_o, b_q=None, b_k=None, b_v=None, b_o=None, h=8, ln_gain=None,
                         ln_bias=None, ln_kind=0, ln_eps=1e-6, memory=None, valid_lens=None, causal=False,
                         out_dtype=None, out=None, workspace=None):
    """x + MHA(norm(x), kv, kv), kv = norm(x) or ``memory``; returns [B, L, d_model]."""
    torch = _torch()
    args = dict(x=x, memory=memory, w_q=w_q, w_k=w_k, w_v=w_v, w_o=w_o, b_q=b_q, b_k=b_k, b_v=b_v, b_o=b_o,
                ln_gain=ln_gain, ln_bias=ln_bias)
    for n, t in args.items():
        _check_gpu(n, t)
        if t is not None and (not t.is_contiguous() or t.dtype != x.dtype):
            raise ValueError(f"{n} must be contiguous and share x's dtype")
    B, L, D = x.shape
    Lk = L if memory is None else memory.shape[1]
    in_dt = _dtype_code(x.dtype)
    out_dtype = (torch.float32 if x.dtype == torch.bfloat16 else x.dtype) if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, L, D), dtype=out_dtype, device=x.device)
    lib = _lib.load()
    need = int(lib.mha_sublayer_workspace_bytes(in_dt, B, L, Lk, D, h))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    vl = _valid_lens(valid_lens, B, x.device)
    st = lib.mha_sublayer_forward(in_dt, _dtype_code(out.dtype), _ptr(x), _ptr(memory), _ptr(ln_gain), _ptr(ln_bias),
                                  int(ln_kind), float(ln_eps), _ptr(w_q), _ptr(b_q), _ptr(w_k), _ptr(b_k), _ptr(w_v),
                                  _ptr(b_v), _ptr(w_o), _ptr(b_o), _ptr(out), B, L, Lk, D, h, D // h if h else 0,
                                  _ptr(vl), int(bool(causal)), _ptr(workspace), workspace.numel(), _stream())
    _raise(st, "mha_sublayer_forward")
    return out


def mha_forward_train(x_q, x_kv, w_q, w_k, w_v, w_o, b_q=None, b_k=None, b_v=None, b_o=None, h=8, valid_lens=None,
                      causal=False, out_dtype=None, out=None, saved=None):
    """mha_forward for training (bf16): returns (out, saved), where ``saved``
    (a uint8 device tensor) holds Q, K, V, the merged heads and each query's
    log-sum-exp for mha_backward(..., saved=saved)."""
    torch = _torch()
    args = dict(x_q=x_q, x_kv=x_kv, w_q=w_q, w_k=w_k, w_v=w_v, w_o=w_o, b_q=b_q, b_k=b_k, b_v=b_v, b_o=b_o)
    for n, t in args.items():
        _check_gpu(n, t)
        if t is not None and (not t.is_contiguous() or t.dtype != x_q.dtype):
            raise ValueError(f"{n} must be contiguous and share x_q's dtype")
    B, Lq, D = x_q.shape
    Lk = x_kv.shape[1]
    in_dt = _dtype_code(x_q.dtype)
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, Lq, D), dtype=out_dtype, device=x_q.device)
    lib = _lib.load()
    need = int(lib.mha_saved_bytes(in_dt, B, Lq, Lk, D, h))
    if saved is None:
        saved = torch.empty(max(need, 1), dtype=torch.uint8, device=x_q.device)
    vl = _valid_lens(valid_lens, B, x_q.device)
    st = lib.mha_forward_train(in_dt, _dtype_code(out.dtype), _ptr(x_q), _ptr(x_kv), _ptr(w_q), _ptr(b_q), _ptr(w_k),
                               _ptr(b_k), _ptr(w_v), _ptr(b_v), _ptr(w_o), _ptr(b_o), _ptr(out), B, Lq, Lk, D, h,
                               D // h if h else 0, _ptr(vl), int(bool(causal)), _ptr(saved), saved.numel(), _stream())
    _raise(st, "mha_forward_train")
    return out, saved


def mha_backward(x_q, x_kv, w_q, w_k, w_v, w_o, dout, b_q=None, b_k=None, b_v=None, h=8, valid_lens=None,
                 causal=False, bias_grads=None, workspace=None, saved=None):
    """Gradients of mha_forward (bf16) for the output gradient ``dout``
    [B, Lq, d_model]: a dict of fp32 tensors dx_q, dx_kv, dw_q, dw_k, dw_v,
    dw_o and, with ``bias_grads`` (default: when b_q is given), db_q, db_k,
    db_v, db_o.  When x_kv is x_q (self-attention) dx_kv is None and dx_q is
    the input's whole gradient.  With ``saved`` from mha_forward_train (same
    inputs) the forward is not recomputed."""
    torch = _torch()
    args = dict(x_q=x_q, x_kv=x_kv, w_q=w_q, w_k=w_k, w_v=w_v, w_o=w_o, dout=dout, b_q=b_q, b_k=b_k, b_v=b_v)
    for n, t in args.items():
        _check_gpu(n, t)
        if t is not None and (not t.is_contiguous() or t.dtype != x_q.dtype):
            raise ValueError(f"{n} must be contiguous and share x_q's dtype")
    B, Lq, D = x_q.shape
    Lk = x_kv.shape[1]
    dev = x_q.device
    f32 = dict(dtype=torch.float32, device=dev)
    self_attn = x_kv is x_q or (x_kv.data_ptr() == x_q.data_ptr() and x_kv.shape == x_q.shape)
    bias_grads = (b_q is not None) if bias_grads is None else bool(bias_grads)
    r = {"dx_q": torch.empty((B, Lq, D), **f32),
         "dx_kv": None if self_attn else torch.empty((B, Lk, D), **f32)}
    for n in "qkvo":
        r["dw_" + n] = torch.empty((D, D), **f32)
        r["db_" + n] = torch.empty((D,), **f32) if bias_grads else None
    lib = _lib.load()
    in_dt = _dtype_code(x_q.dtype)
    size_fn = lib.mha_backward_workspace_bytes if saved is None else lib.mha_backward_saved_workspace_bytes
    need = int(size_fn(in_dt, B, Lq, Lk, D, h))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    vl = _valid_lens(valid_lens, B, dev)
    grads = [_ptr(r["dx_q"]), _ptr(r["dx_kv"]), _ptr(r["dw_q"]), _ptr(r["db_q"]), _ptr(r["dw_k"]), _ptr(r["db_k"]),
             _ptr(r["dw_v"]), _ptr(r["db_v"]), _ptr(r["dw_o"]), _ptr(r["db_o"])]
    tail = [B, Lq, Lk, D, h, D // h if h else 0, _ptr(vl), int(bool(causal)), _ptr(workspace), workspace.numel(),
            _stream()]
    if saved is None:
        st = lib.mha_backward(in_dt, _ptr(x_q), _ptr(x_kv), _ptr(w_q), _ptr(b_q), _ptr(w_k), _ptr(b_k), _ptr(w_v),
                              _ptr(b_v), _ptr(w_o), _ptr(dout), *grads, *tail)
        _raise(st, "mha_backward")
    else:
        _check_gpu("saved", saved)
        st = lib.mha_backward_saved(in_dt, _ptr(x_q), _ptr(x_kv), _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(w_o),
                                    _ptr(saved), saved.numel() * saved.element_size(), _ptr(dout), *grads, *tail)
        _raise(st, "mha_backward_saved")
    return r


class kernel_timing:
    """Context manager: per-kernel GPU time (HIP events around each launch).

        with kernel_timing(repeat=10) as kt:
            ...library calls...
        kt.result  # {kernel name: (total_ms, launches)}

    With repeat > 1 each kernel runs `repeat` times back to back inside one
    event pair (same results: the kernels are pure functions of their
    inputs), so total_ms / launches approaches the kernel's own duration.
    """

    def __init__(self, repeat=1):
        self.result = {}
        self.repeat = int(repeat)

    def __enter__(self):
        _raise(_lib.load().mha_timing_enable(self.repeat), "mha_timing_enable")
        return self

    def __exit__(self, *exc):
        lib = _lib.load()
        n = 16
        names = (ctypes.c_char_p * n)()
        tot = (ctypes.c_double * n)()
        cnt = (ctypes.c_int * n)()
        k = lib.mha_timing_read(names, tot, cnt, n)
        lib.mha_timing_enable(0)
        if k < 0:
            raise RuntimeError("mha_timing_read failed")
        self.result = {names[x].decode(): (tot[x], cnt[x]) for x in range(k)}
        return False
