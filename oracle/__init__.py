"""fp64 CPU oracle for multi-head scaled dot-product attention (forward).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; the product library never loads it.
It shares no code with the HIP path.  The arithmetic lives in ``oracle.c``
(plain fp64 loops); this module only converts numpy arrays to float64 and
calls it through ctypes.

Functions and the passages they follow:

* ``linear``  -- y = x W^T + b, a torch linear layer's stored orientation
  ("Transformer" study notes, multi-head attention section).
* ``sdpa``    -- softmax(Q K^T / sqrt(d_k)) V with masked scores replaced by
  -1e9 (The Annotated Transformer, "Attention" section), key-padding
  ``valid_lens`` (d2l Transformer digest, multi-head attention prerequisites)
  and the lower-triangular causal mask ("Transformer" study notes,
  mask-generation section), combined by AND.
* ``sdpa_backward`` -- the gradients of ``sdpa`` with respect to q, k, v
  for a given gradient of the output: the softmax Jacobian written out
  (the pages train these models end to end).
* ``mha``     -- the four projections, head split, sdpa per head, head merge
  and the output projection ("Transformer" study notes, multi-head attention
  formula and class).
* ``layer_norm`` -- per-row normalisation in the two forms the pages print:
  The Annotated Transformer's class (std with Bessel's correction, eps added
  to the std) and the study notes' torch layer (biased variance, eps inside
  the root).
* ``mha_sublayer`` -- the pre-norm residual sublayer around attention, x +
  attention(norm(x), ...) (The Annotated Transformer, sublayer connection;
  no dropout at inference).
* ``round_bf16`` -- nearest bfloat16, ties to even (used by the optional
  bf16-storage mode of ``mha``).

Every function is pinned by tests in ``tests/test_oracle_*.py`` against values
the pages print, closed forms, invariants, brute force and torch's float64
CPU routines; none is "parity unpinned".
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)


def _open(path):
    lib = ctypes.CDLL(path)
    lib.oracle_round_bf16_f64.restype = ctypes.c_double
    lib.oracle_round_bf16_f64.argtypes = [ctypes.c_double]
    lib.oracle_linear_f64.restype = None
    lib.oracle_linear_f64.argtypes = [_dp, _dp, _dp, _dp, ctypes.c_long, ctypes.c_int, ctypes.c_int]
    lib.oracle_sdpa_f64.restype = ctypes.c_int
    lib.oracle_sdpa_f64.argtypes = [_dp, _dp, _dp, _dp, _dp] + [ctypes.c_int] * 6 + [
        _ip, ctypes.c_int, ctypes.c_int, _ip, ctypes.c_int]
    lib.oracle_sdpa_lse_f64.restype = ctypes.c_int
    lib.oracle_sdpa_lse_f64.argtypes = [_dp, _dp, _dp] + [ctypes.c_int] * 5 + [_ip, ctypes.c_int, ctypes.c_int]
    lib.oracle_mha_f64.restype = ctypes.c_int
    lib.oracle_mha_f64.argtypes = [_dp] * 11 + [ctypes.c_int] * 5 + [
        _ip, ctypes.c_int, ctypes.c_int, _ip, ctypes.c_int, ctypes.c_int]
    lib.oracle_mha_backward_f64.restype = ctypes.c_int
    lib.oracle_mha_backward_f64.argtypes = [_dp] * 20 + [ctypes.c_int] * 5 + [_ip, ctypes.c_int, ctypes.c_int,
                                                                             ctypes.c_int]
    lib.oracle_sdpa_backward_f64.restype = ctypes.c_int
    lib.oracle_sdpa_backward_f64.argtypes = [_dp] * 7 + [ctypes.c_int] * 6 + [_ip, ctypes.c_int, ctypes.c_int]
    lib.oracle_layer_norm_f64.restype = None
    lib.oracle_layer_norm_f64.argtypes = [_dp, _dp, _dp, _dp, ctypes.c_long, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_double]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        _lib = _open(_LIB_PATH)
    return _lib


class use_library:
    """Context manager: run the oracle functions from another build of
    ``oracle.c`` (the mutation tests build copies with a planted mistake)."""

    def __init__(self, path):
        self.path = path
        self.saved = None

    def __enter__(self):
        global _lib
        self.saved = _load()
        _lib = _open(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def _iptr(a):
    return None if a is None else a.ctypes.data_as(_ip)


def _i32(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def round_bf16(x):
    """Nearest bfloat16 value of each element (returned as float64)."""
    lib = _load()
    flat = _f64(x).ravel()
    out = np.array([lib.oracle_round_bf16_f64(float(v)) for v in flat], dtype=np.float64)
    return out.reshape(np.shape(x))


def linear(x, w, b=None):
    """y = x W^T + b over the last axis; W is [out, in]."""
    x = _f64(x)
    w = _f64(w)
    b = None if b is None else _f64(b)
    din = x.shape[-1]
    dout = w.shape[0]
    assert w.shape == (dout, din)
    m = int(np.prod(x.shape[:-1]))
    y = np.empty(x.shape[:-1] + (dout,), dtype=np.float64)
    _load().oracle_linear_f64(_ptr(x), _ptr(w), _ptr(b), _ptr(y), m, din, dout)
    return y


def sdpa(q, k, v, valid_lens=None, causal=False, rows=None, return_weights=False):
    """Attention on split heads: q [B,h,Lq,dk], k [B,h,Lk,dk], v [B,h,Lk,dv].

    Returns o [B,h,R,dv] (and the weights [B,h,R,Lk] if asked), where R is
    ``len(rows)`` if ``rows`` (query indices) is given, else Lq.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, h, Lq, dk = q.shape
    Lk = k.shape[2]
    dv = v.shape[3]
    assert k.shape == (B, h, Lk, dk) and v.shape == (B, h, Lk, dv)
    vl = _i32(valid_lens)
    if vl is not None:
        assert vl.shape in ((B,), (B, Lq))
    rr = _i32(rows)
    R = Lq if rr is None else int(rr.shape[0])
    o = np.empty((B, h, R, dv), dtype=np.float64)
    p = np.empty((B, h, R, Lk), dtype=np.float64) if return_weights else None
    rc = _load().oracle_sdpa_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(p),
                                 B, h, Lq, Lk, dk, dv, _iptr(vl), int(vl is not None and vl.ndim == 2),
                                 int(bool(causal)), _iptr(rr), 0 if rr is None else R)
    if rc != 0:
        raise ValueError("oracle_sdpa_f64 rejected its arguments")
    return (o, p) if return_weights else o


def sdpa_lse(q, k, valid_lens=None, causal=False):
    """Log of each query row's softmax normaliser, log sum_j exp(s_ij), for
    ``sdpa(q, k, v, valid_lens, causal)``: [B, h, Lq] (masked scores take the
    fill, so a row with every key masked gives fill + log(Lk))."""
    q, k = _f64(q), _f64(k)
    B, h, Lq, dk = q.shape
    Lk = k.shape[2]
    assert k.shape == (B, h, Lk, dk)
    vl = _i32(valid_lens)
    if vl is not None:
        assert vl.shape in ((B,), (B, Lq))
    lse = np.empty((B, h, Lq), dtype=np.float64)
    rc = _load().oracle_sdpa_lse_f64(_ptr(q), _ptr(k), _ptr(lse), B, h, Lq, Lk, dk, _iptr(vl),
                                     int(vl is not None and vl.ndim == 2), int(bool(causal)))
    if rc != 0:
        raise ValueError("oracle_sdpa_lse_f64 rejected its arguments")
    return lse


def sdpa_backward(q, k, v, dout, valid_lens=None, causal=False):
    """Gradients (dq, dk, dv) of ``sdpa(q, k, v, valid_lens, causal)`` for the
    output gradient ``dout`` [B,h,Lq,dv]."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, h, Lq, dk = q.shape
    Lk = k.shape[2]
    dv = v.shape[3]
    assert k.shape == (B, h, Lk, dk) and v.shape == (B, h, Lk, dv) and g.shape == (B, h, Lq, dv)
    vl = _i32(valid_lens)
    if vl is not None:
        assert vl.shape in ((B,), (B, Lq))
    dq, dkk, dvv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    rc = _load().oracle_sdpa_backward_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(dq), _ptr(dkk), _ptr(dvv),
                                          B, h, Lq, Lk, dk, dv, _iptr(vl), int(vl is not None and vl.ndim == 2),
                                          int(bool(causal)))
    if rc != 0:
        raise ValueError("oracle_sdpa_backward_f64 rejected its arguments")
    return dq, dkk, dvv


def mha_backward(x_q, x_kv, w_q, w_k, w_v, w_o, dout, b_q=None, b_k=None, b_v=None, h=8, valid_lens=None,
                 causal=False, bf16_stages=False):
    """Gradients of ``mha(x_q, x_kv, ...)`` (all query rows) for the output
    gradient ``dout`` [B, Lq, D].  Returns a dict: dx_q [B,Lq,D] (through the
    query projection), dx_kv [B,Lk,D] (through the key and value projections;
    with self-attention the input's gradient is dx_q + dx_kv), dw_q, dw_k,
    dw_v, dw_o [D,D] and db_q, db_k, db_v, db_o [D].  The output bias does
    not enter any gradient."""
    xq, xkv, g = _f64(x_q), _f64(x_kv), _f64(dout)
    B, Lq, D = xq.shape
    Lk = xkv.shape[1]
    assert xkv.shape == (B, Lk, D) and g.shape == (B, Lq, D)
    ws = [_f64(w) for w in (w_q, w_k, w_v, w_o)]
    for w in ws:
        assert w.shape == (D, D)
    bs = [None if b is None else _f64(b) for b in (b_q, b_k, b_v)]
    vl = _i32(valid_lens)
    if vl is not None:
        assert vl.shape in ((B,), (B, Lq))
    r = {"dx_q": np.empty((B, Lq, D)), "dx_kv": np.empty((B, Lk, D))}
    for n in ("q", "k", "v", "o"):
        r["dw_" + n] = np.empty((D, D))
        r["db_" + n] = np.empty(D)
    rc = _load().oracle_mha_backward_f64(
        _ptr(xq), _ptr(xkv), _ptr(ws[0]), _ptr(bs[0]), _ptr(ws[1]), _ptr(bs[1]), _ptr(ws[2]), _ptr(bs[2]),
        _ptr(ws[3]), _ptr(g), _ptr(r["dx_q"]), _ptr(r["dx_kv"]),
        _ptr(r["dw_q"]), _ptr(r["db_q"]), _ptr(r["dw_k"]), _ptr(r["db_k"]),
        _ptr(r["dw_v"]), _ptr(r["db_v"]), _ptr(r["dw_o"]), _ptr(r["db_o"]),
        B, Lq, Lk, D, h, _iptr(vl), int(vl is not None and vl.ndim == 2), int(bool(causal)),
        int(bool(bf16_stages)))
    if rc != 0:
        raise ValueError("oracle_mha_backward_f64 rejected its arguments")
    return r


def layer_norm(x, gain=None, bias=None, kind=0, eps=1e-6):
    """Normalise each row of x [..., D]: kind 0 (std with Bessel's correction,
    eps added to the std) or kind 1 (biased variance, eps inside the root)."""
    x = _f64(x)
    D = x.shape[-1]
    y = np.empty_like(x)
    a = None if gain is None else _f64(gain)
    b = None if bias is None else _f64(bias)
    _load().oracle_layer_norm_f64(_ptr(x), _ptr(a), _ptr(b), _ptr(y), x.size // D, D, int(kind), float(eps))
    return y


def mha_sublayer(x, w_q, w_k, w_v, w_o, b_q=None, b_k=None, b_v=None, b_o=None, h=8, ln_gain=None,
                 ln_bias=None, ln_kind=0, ln_eps=1e-6, memory=None, valid_lens=None, causal=False, rows=None):
    """x + MHA(norm(x), kv, kv) with kv = norm(x) (self-attention) or the
    given memory (source attention); the result's rows ``rows`` if given."""
    x = _f64(x)
    xn = layer_norm(x, ln_gain, ln_bias, ln_kind, ln_eps)
    kv = xn if memory is None else _f64(memory)
    att = mha(xn, kv, w_q, w_k, w_v, w_o, b_q, b_k, b_v, b_o, h=h, valid_lens=valid_lens, causal=causal,
              rows=rows)
    xr = x if rows is None else x[:, np.asarray(rows)]
    return xr + att


def mha(x_q, x_kv, w_q, w_k, w_v, w_o, b_q=None, b_k=None, b_v=None, b_o=None,
        h=8, valid_lens=None, causal=False, rows=None, bf16_stages=False):
    """Multi-head attention forward: x_q [B,Lq,D], x_kv [B,Lk,D] -> [B,R,D]."""
    xq, xkv = _f64(x_q), _f64(x_kv)
    B, Lq, D = xq.shape
    Lk = xkv.shape[1]
    assert xkv.shape == (B, Lk, D)
    ws = [_f64(w) for w in (w_q, w_k, w_v, w_o)]
    for w in ws:
        assert w.shape == (D, D)
    bs = [None if b is None else _f64(b) for b in (b_q, b_k, b_v, b_o)]
    vl = _i32(valid_lens)
    if vl is not None:
        assert vl.shape in ((B,), (B, Lq))
    rr = _i32(rows)
    R = Lq if rr is None else int(rr.shape[0])
    out = np.empty((B, R, D), dtype=np.float64)
    rc = _load().oracle_mha_f64(_ptr(xq), _ptr(xkv),
                                _ptr(ws[0]), _ptr(bs[0]), _ptr(ws[1]), _ptr(bs[1]),
                                _ptr(ws[2]), _ptr(bs[2]), _ptr(ws[3]), _ptr(bs[3]),
                                _ptr(out), B, Lq, Lk, D, h, _iptr(vl), int(vl is not None and vl.ndim == 2),
                                int(bool(causal)),
                                _iptr(rr), 0 if rr is None else R, int(bool(bf16_stages)))
    if rc != 0:
        raise ValueError("oracle_mha_f64 rejected its arguments")
    return out
