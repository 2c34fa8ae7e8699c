"""(Batch, head) views that begin past 2^31 elements of their buffer (beyond
4 GiB of bf16): the entry points that take strided views form each view's
base address in 64-bit arithmetic.  Every operand here is a [2, 1, L, 64]
view of a buffer of its own whose second batch starts at element
2^31 + 4096; only the two views are written (and read by the kernels), the
rest of each buffer is never touched.  Results against the oracle on the
same values."""
import numpy as np
import pytest

import oracle
import workloads
from parity import assert_bf16, assert_fp32, to_device, to_host

pytestmark = pytest.mark.gpu

S = 2 ** 31 + 4096      # batch stride in elements: batch 1 begins past 2^31
L = 64


def _far(shape, dtype, values=None):
    """A view of the given shape ([2, ...], last axes contiguous) whose batch
    stride is S, over a fresh buffer of S + 4096 elements."""
    import torch
    inner = int(np.prod(shape[1:]))
    assert shape[0] == 2 and inner <= 4096
    buf = torch.empty(S + 4096, dtype=dtype, device="cuda")
    strides = [S]
    for n in range(1, len(shape)):
        strides.append(int(np.prod(shape[n + 1:])))
    t = buf.as_strided(tuple(shape), tuple(strides))
    if values is not None:
        t.copy_(to_device(values, dtype))
    return t


def _release():
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _qkv(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return [workloads._finish(rng.standard_normal((2, 1, L, 64)), "bf16") for _ in range(3)]


@pytest.mark.parametrize("causal,lens", [(False, [64, 37]), (True, None)])
def test_sdpa_forward_far_views(causal, lens):
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    q, k, v = _qkv(11 + causal)
    vl = None if lens is None else np.array(lens, dtype=np.int32)
    tq, tk, tv = (_far((2, 1, L, 64), torch.bfloat16, x) for x in (q, k, v))
    to = _far((2, 1, L, 64), torch.float32)
    o = mha.sdpa_forward(tq, tk, tv, valid_lens=vl, causal=causal, out=to)
    torch.cuda.synchronize()
    assert o.data_ptr() == to.data_ptr()
    assert_bf16(to_host(o), oracle.sdpa(q, k, v, valid_lens=vl, causal=causal), f"far views causal={causal}")
    del tq, tk, tv, to, o
    _release()


def test_sdpa_weights_far_views():
    """The weights export (scores kept in registers: Lk <= 512) with its
    inputs, output and fp32 weights all in far views."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    q, k, v = _qkv(21)
    vl = np.array([[min(L, 1 + (3 * i) % 70) for i in range(L)], [L] * L], dtype=np.int32)   # per query
    tq, tk, tv = (_far((2, 1, L, 64), torch.bfloat16, x) for x in (q, k, v))
    to = _far((2, 1, L, 64), torch.float32)
    tp = _far((2, 1, L, L), torch.float32)
    o, p = mha.sdpa_forward(tq, tk, tv, valid_lens=vl, out=to, return_weights=True, weights=tp)
    torch.cuda.synchronize()
    ro, rp = oracle.sdpa(q, k, v, valid_lens=vl, return_weights=True)
    assert_fp32(to_host(p), rp, "far weights")
    assert_bf16(to_host(o), ro, "far output")
    del tq, tk, tv, to, tp, o, p
    _release()


def test_sdpa_decode_far_views():
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    q, k, v = _qkv(31)
    lens = np.array([L, 20], dtype=np.int32)
    tq = _far((2, 1, 64), torch.bfloat16, q[:, :, 0])
    tk, tv = (_far((2, 1, L, 64), torch.bfloat16, x) for x in (k, v))
    to = _far((2, 1, 64), torch.float32)
    o = mha.sdpa_decode(tq, tk, tv, lens, out=to)
    torch.cuda.synchronize()
    assert_bf16(to_host(o), oracle.sdpa(q[:, :, :1], k, v, valid_lens=lens)[:, :, 0], "far decode")
    del tq, tk, tv, to, o
    _release()


def test_sdpa_backward_far_views():
    """The backward given the forward's log-sum-exp, every input in far views."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    q, k, v = _qkv(41)
    g = workloads._finish(np.random.Generator(np.random.PCG64(42)).standard_normal((2, 1, L, 64)), "bf16")
    tq, tk, tv, tg = (_far((2, 1, L, 64), torch.bfloat16, x) for x in (q, k, v, g))
    to = _far((2, 1, L, 64), torch.bfloat16)
    o, lse = mha.sdpa_forward(tq, tk, tv, causal=True, out=to, return_lse=True)
    grads = mha.sdpa_backward(tq, tk, tv, o, tg, causal=True, out_dtype=torch.float32, lse=lse)
    torch.cuda.synchronize()
    ref = oracle.sdpa_backward(q, k, v, g, causal=True)
    for name, got, r in zip(("dq", "dk", "dv"), grads, ref):
        assert_bf16(to_host(got), r, f"far backward {name}")
    del tq, tk, tv, tg, to, o, lse, grads
    _release()
