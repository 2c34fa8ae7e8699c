"""GPU parity of the inspection path (sdpa_forward_ex, mha_forward_ex):
attention weights returned beside the output, and key-padding lengths per
query [B, Lq], against the fp64 oracle.

The path computes in fp32 (FMA) on the exact input values, so the weights
and fp32 outputs are held to the fp32 bar (norm-wise 1e-5); bf16 outputs and
the multi-head layer in bf16 (whose projections are bf16 MFMA products) to
the bf16 bar."""
import numpy as np
import pytest

import oracle
import workloads
from parity import assert_bf16, assert_fp32, to_device, to_host

pytestmark = pytest.mark.gpu

SDPA_CASES = [
    # B, h, Lq, Lk, causal, lengths: None | "1d" | "2d", input dtype
    (2, 3, 70, 70, True, "2d", "bf16"),
    (2, 2, 45, 100, False, "2d", "bf16"),
    (3, 2, 64, 96, False, "1d", "f32"),
    (2, 2, 33, 33, True, None, "f32"),
    (1, 4, 130, 77, False, "2d", "f32"),
]


def _lengths(kind, rng, B, Lq, Lk):
    if kind is None:
        return None
    if kind == "1d":
        vl = rng.integers(0, Lk + 1, size=B).astype(np.int32)
        vl[0] = 0                                            # a fully masked sequence
        return vl
    vl = rng.integers(-1, Lk + 3, size=(B, Lq)).astype(np.int32)   # incl. <= 0 and > Lk
    vl[0, :3] = [0, 1, Lk]
    return vl


@pytest.mark.parametrize("B,h,Lq,Lk,causal,kind,dt", SDPA_CASES)
def test_sdpa_weights_and_lengths_per_query(B, h, Lq, Lk, causal, kind, dt):
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    rng = np.random.Generator(np.random.PCG64(B * 1000 + Lq * 7 + Lk))
    q = workloads._finish(rng.standard_normal((B, h, Lq, 64)), dt)
    k = workloads._finish(rng.standard_normal((B, h, Lk, 64)), dt)
    v = workloads._finish(rng.standard_normal((B, h, Lk, 64)), dt)
    vl = _lengths(kind, rng, B, Lq, Lk)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    tq, tk, tv = (to_device(x, tdt) for x in (q, k, v))
    o, p = mha.sdpa_forward(tq, tk, tv, valid_lens=vl, causal=causal, out_dtype=torch.float32, return_weights=True)
    torch.cuda.synchronize()
    ro, rp = oracle.sdpa(q, k, v, valid_lens=vl, causal=causal, return_weights=True)
    assert_fp32(to_host(p), rp, "weights")
    assert_fp32(to_host(o), ro, "output")
    # masked keys get exactly zero weight; every row sums to one
    g = to_host(p)
    assert np.all(g[rp == 0.0] == 0.0)
    assert np.allclose(g.sum(axis=-1), 1.0, atol=1e-5)
    if kind == "2d" and dt == "bf16":
        # bf16 output without the weights takes the same path
        ob = mha.sdpa_forward(tq, tk, tv, valid_lens=vl, causal=causal, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert_bf16(to_host(ob), ro, "bf16 output, lengths per query")


def test_lengths_i_plus_1_match_the_causal_kernel():
    """Query lengths i + 1 (the decoder's training lengths) on the inspection
    path equal the causal mask on the fast path."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    rng = np.random.Generator(np.random.PCG64(77))
    B, h, L = 2, 4, 200
    q, k, v = (workloads._finish(rng.standard_normal((B, h, L, 64)), "bf16") for _ in range(3))
    tq, tk, tv = (to_device(x, torch.bfloat16) for x in (q, k, v))
    vl2 = np.tile(np.arange(1, L + 1, dtype=np.int32), (B, 1))
    a = mha.sdpa_forward(tq, tk, tv, valid_lens=vl2, out_dtype=torch.float32)
    c = mha.sdpa_forward(tq, tk, tv, causal=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.sdpa(q, k, v, causal=True)
    assert_fp32(to_host(a), ref, "lengths i + 1")
    assert_bf16(to_host(c), ref, "causal fast path")


def _oracle_mha_weights(inp, vl):
    """Per-head weights of the multi-head layer from the oracle's own pieces:
    its linear layers, the head split, and its attention with weights."""
    t = inp.tensors
    w = inp.workload
    B, Lq, D = t["x_q"].shape
    Lk = t["x_kv"].shape[1]
    dk = D // w.h
    Q = oracle.linear(t["x_q"], t["w_q"], t["b_q"]).reshape(B, Lq, w.h, dk).transpose(0, 2, 1, 3)
    K = oracle.linear(t["x_kv"], t["w_k"], t["b_k"]).reshape(B, Lk, w.h, dk).transpose(0, 2, 1, 3)
    V = oracle.linear(t["x_kv"], t["w_v"], t["b_v"]).reshape(B, Lk, w.h, dk).transpose(0, 2, 1, 3)
    return oracle.sdpa(Q, K, V, valid_lens=vl, causal=w.causal, return_weights=True)[1]


MHA_CASES = [
    # B, Lq, Lk, D, h, causal, lengths, dtype, self-attention
    (2, 40, 40, 256, 4, True, "2d", "bf16", True),
    (2, 30, 50, 128, 2, False, "1d", "bf16", False),
    (2, 20, 20, 256, 4, False, "2d", "f32", True),
]


@pytest.mark.parametrize("B,Lq,Lk,D,h,causal,kind,dt,self_attn", MHA_CASES)
def test_mha_weights_and_lengths_per_query(B, Lq, Lk, D, h, causal, kind, dt, self_attn):
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    inp = workloads.make_mha_inputs(B, Lq, Lk, D, h, dt, seed=B * 31 + Lq + Lk, vl_range=None, causal=causal,
                                    self_attn=self_attn, bias=True)
    rng = np.random.Generator(np.random.PCG64(Lq * 13 + Lk))
    vl = _lengths(kind, rng, B, Lq, Lk)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    t = {n: (None if a is None else to_device(a, tdt)) for n, a in inp.tensors.items()}
    if self_attn:
        t["x_kv"] = t["x_q"]
    out, p = mha.mha_forward(t["x_q"], t["x_kv"], t["w_q"], t["w_k"], t["w_v"], t["w_o"], t["b_q"], t["b_k"],
                             t["b_v"], t["b_o"], h=h, valid_lens=vl, causal=causal, out_dtype=torch.float32,
                             return_weights=True)
    torch.cuda.synchronize()
    tt = inp.tensors
    ref = oracle.mha(tt["x_q"], tt["x_kv"], tt["w_q"], tt["w_k"], tt["w_v"], tt["w_o"], tt["b_q"], tt["b_k"],
                     tt["b_v"], tt["b_o"], h=h, valid_lens=vl, causal=causal)
    rp = _oracle_mha_weights(inp, vl)
    if dt == "f32":
        assert_fp32(to_host(out), ref, "mha output")
        assert_fp32(to_host(p), rp, "mha weights")
    else:
        assert_bf16(to_host(out), ref, "mha output")
        assert_bf16(to_host(p), rp, "mha weights")
    assert np.all(to_host(p)[rp == 0.0] == 0.0)


def test_inspect_weights_workload_full_size():
    """The weights-export workload at full size (B=4 h=8 L=512, per-sequence
    lengths) as the benchmark launches it: every weight and output."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    w = workloads.BY_NAME["inspect_weights"]
    inp = workloads.make_inputs(w)
    q, k, v = (inp.tensors[n] for n in ("q", "k", "v"))
    tq, tk, tv = (to_device(x, torch.bfloat16) for x in (q, k, v))
    o, p = mha.sdpa_forward(tq, tk, tv, valid_lens=inp.valid_lens, out_dtype=torch.bfloat16, return_weights=True)
    torch.cuda.synchronize()
    ro, rp = oracle.sdpa(q, k, v, valid_lens=inp.valid_lens, return_weights=True)
    print("weights", assert_fp32(to_host(p), rp, "inspect_weights weights"))
    print("output", assert_bf16(to_host(o), ro, "inspect_weights output (bf16, as benchmarked)"))


@pytest.mark.parametrize("B,h,L,causal,kind", [
    (2, 2, 200, True, None),      # causal without lengths: keys past each block's triangle are zero-filled
    (1, 2, 70, True, None),       # rows of 70 weights: the last 16-byte piece of a row is partial
    (2, 3, 150, False, "1d"),
    (2, 2, 99, True, "2d"),
    (2, 2, 512, False, "2d"),     # the longest rows whose scores stay in registers
    (2, 2, 512, True, None),      # the same length, causal without lengths: the two-pass kernel
    (1, 2, 513, True, None),
    (1, 2, 600, False, "1d"),     # past 512 keys: the two-pass kernel with lengths
    (1, 2, 530, True, "2d"),      # ... causal with lengths per query, rows not 16-byte aligned
])
def test_weights_overwrite_every_entry(B, h, L, causal, kind):
    """bf16 inputs (MFMA inspection kernels) into a weights buffer pre-filled
    with NaN: every entry must be written, masked ones as exact zeros.  Rows
    of up to 512 keys take the kernel that keeps its scores in registers,
    longer rows and causal launches without lengths the two-pass one."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    rng = np.random.Generator(np.random.PCG64(B * 31 + L))
    q, k, v = (workloads._finish(rng.standard_normal((B, h, L, 64)), "bf16") for _ in range(3))
    vl = _lengths(kind, rng, B, L, L)
    tq, tk, tv = (to_device(x, torch.bfloat16) for x in (q, k, v))
    buf = torch.full((B, h, L, L), float("nan"), dtype=torch.float32, device="cuda")
    o, p = mha.sdpa_forward(tq, tk, tv, valid_lens=vl, causal=causal, out_dtype=torch.float32,
                            return_weights=True, weights=buf)
    torch.cuda.synchronize()
    assert p.data_ptr() == buf.data_ptr()
    g = to_host(p)
    assert not np.isnan(g).any(), "weights left unwritten"
    ro, rp = oracle.sdpa(q, k, v, valid_lens=vl, causal=causal, return_weights=True)
    assert_fp32(g, rp, "weights")
    assert np.all(g[rp == 0.0] == 0.0)
    assert_fp32(to_host(o), ro, "output")


@pytest.mark.parametrize("B,h,L", [(2, 3, 300), (1, 2, 512), (2, 2, 97)])
def test_weights_kernels_agree_bit_for_bit(B, h, L):
    """Causal rows with every length equal to L take the kernel that keeps its
    scores in registers; causal rows without lengths take the two-pass
    kernel.  Both allow the same keys and do the same arithmetic in the same
    order (the extra steps of the first are wholly masked and leave the
    running statistics unchanged), so weights and outputs agree bit for
    bit; both also match the oracle."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    rng = np.random.Generator(np.random.PCG64(B * 7 + L))
    q, k, v = (workloads._finish(rng.standard_normal((B, h, L, 64)), "bf16") for _ in range(3))
    tq, tk, tv = (to_device(x, torch.bfloat16) for x in (q, k, v))
    full = np.full(B, L, dtype=np.int32)
    o1, p1 = mha.sdpa_forward(tq, tk, tv, valid_lens=full, causal=True, out_dtype=torch.float32, return_weights=True)
    o2, p2 = mha.sdpa_forward(tq, tk, tv, causal=True, out_dtype=torch.float32, return_weights=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(p1), to_host(p2))
    np.testing.assert_array_equal(to_host(o1), to_host(o2))
    ro, rp = oracle.sdpa(q, k, v, causal=True, return_weights=True)
    assert_fp32(to_host(p1), rp, "weights")
    assert_bf16(to_host(o1), ro, "output")
