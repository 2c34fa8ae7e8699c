"""Streamed row tiles must stop at the view's last row.

The bf16 MFMA backward and weights-export kernels stream K/V (or Q/dO) in
128-row steps; a step that runs past row L - 1 must read zeros, not the
memory after the view.  Here every [B, h, L, 64] operand is a slice of a
longer [B, h, L + 160, 64] tensor whose rows from L on are NaN, so any read
past the view turns the affected results into NaN (0 * NaN) and fails the
finite check of the parity bar.  L = 260 and 300 leave ragged last steps."""
import numpy as np
import pytest

import oracle
import workloads
from parity import assert_bf16, assert_fp32, to_host

pytestmark = pytest.mark.gpu

PAD = 160


def _nan_padded(x):
    """bf16 device tensor [B, h, L + PAD, 64] holding x in rows < L and NaN
    after them; returns the [B, h, L, 64] view."""
    import torch
    B, h, L, d = x.shape
    t = torch.full((B, h, L + PAD, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    t[:, :, :L] = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda().to(torch.bfloat16)
    return t[:, :, :L]


@pytest.mark.parametrize("L,causal", [(260, False), (300, True), (300, False)])
def test_backward_reads_nothing_past_the_view(L, causal):
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    rng = np.random.Generator(np.random.PCG64(4000 + L + causal))
    B, h = 2, 2
    q, k, v, g = (workloads._finish(rng.standard_normal((B, h, L, 64)), "bf16") for _ in range(4))
    vl = None if causal else np.array([L, L - 37], np.int32)
    tq, tk, tv, tg = (_nan_padded(x) for x in (q, k, v, g))
    o = mha.sdpa_forward(tq, tk, tv, valid_lens=vl, causal=causal)
    # the forward output too lives in a NaN-padded buffer
    to = _nan_padded(to_host(o).astype(np.float32))
    gq, gk, gv = mha.sdpa_backward(tq, tk, tv, to, tg, valid_lens=vl, causal=causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.sdpa_backward(q, k, v, g, valid_lens=vl, causal=causal)
    for name, got, r in zip(("dq", "dk", "dv"), (gq, gk, gv), ref):
        e = assert_bf16(to_host(got), r, f"{name} L{L} causal={causal} NaN after the view")
        print(name, e)


@pytest.mark.parametrize("L,causal", [(260, False), (300, True)])
def test_weights_export_reads_nothing_past_the_view(L, causal):
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    rng = np.random.Generator(np.random.PCG64(5000 + L + causal))
    B, h = 2, 2
    q, k, v = (workloads._finish(rng.standard_normal((B, h, L, 64)), "bf16") for _ in range(3))
    vl = np.array([L, L - 51], np.int32)
    tq, tk, tv = (_nan_padded(x) for x in (q, k, v))
    o, p = mha.sdpa_forward(tq, tk, tv, valid_lens=vl, causal=causal, out_dtype=torch.float32,
                            return_weights=True)
    torch.cuda.synchronize()
    ref_o, ref_p = oracle.sdpa(q, k, v, valid_lens=vl, causal=causal, return_weights=True)
    assert_bf16(to_host(o), ref_o, f"output L{L} NaN after the view")
    assert_fp32(to_host(p), ref_p, f"weights L{L} NaN after the view")
