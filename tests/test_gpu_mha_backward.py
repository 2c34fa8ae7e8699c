"""GPU parity of mha_backward (gradients of the multi-head layer) through the
C ABI against the fp64 oracle's chain rule on the same bf16 inputs.

The GPU path stores Q, K, V, the merged heads and the gradients of those four
in bf16 (as the forward does its intermediates) and multiplies on bf16 MFMA
with fp32 sums; every gradient is graded against the plain fp64 oracle with
the gradient bar (relative to the gradient's rms), and the distance to the
oracle's bf16-storage reading is printed beside it."""
import numpy as np
import pytest

import oracle
import workloads
from parity import assert_grad_bf16, assert_grad_rows_bf16, to_device, to_host

pytestmark = pytest.mark.gpu

GRADS = ("dx_q", "dx_kv", "dw_q", "dw_k", "dw_v", "dw_o", "db_q", "db_k", "db_v", "db_o")


def make(B, Lq, Lk, D, h, causal, vlr, bias, self_attn, seed):
    inp = workloads.make_mha_inputs(B, Lq, Lk, D, h, "bf16", seed=seed, vl_range=vlr, causal=causal,
                                    self_attn=self_attn, bias=bias)
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    g = workloads.round_to_bf16(rng.standard_normal((B, Lq, D)).astype(np.float32))
    return inp, g


def run_gpu(inp, g, separate_kv=False):
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    w = inp.workload
    t = {n: (None if a is None else to_device(a, torch.bfloat16)) for n, a in inp.tensors.items()}
    if w.self_attn:
        t["x_kv"] = t["x_q"].clone() if separate_kv else t["x_q"]
    r = mha.mha_backward(t["x_q"], t["x_kv"], t["w_q"], t["w_k"], t["w_v"], t["w_o"], to_device(g, torch.bfloat16),
                         t["b_q"], t["b_k"], t["b_v"], h=w.h, valid_lens=inp.valid_lens, causal=w.causal,
                         bias_grads=True)
    torch.cuda.synchronize()
    return {n: (None if a is None else to_host(a)) for n, a in r.items()}


def run_oracle(inp, g, bf16_stages):
    t = inp.tensors
    w = inp.workload
    return oracle.mha_backward(t["x_q"], t["x_kv"], t["w_q"], t["w_k"], t["w_v"], t["w_o"], g,
                               t["b_q"], t["b_k"], t["b_v"], h=w.h, valid_lens=inp.valid_lens, causal=w.causal,
                               bf16_stages=bf16_stages)


def check(got, inp, g, what, storage_diag=True):
    ref = run_oracle(inp, g, False)
    ref16 = run_oracle(inp, g, True) if storage_diag else ref
    if got["dx_kv"] is None:               # self-attention: one input, both paths summed
        for r in ((ref, ref16) if storage_diag else (ref,)):
            r["dx_q"] = r["dx_q"] + r["dx_kv"]
            r["dx_kv"] = None
    rms = lambda a: float(np.sqrt(np.mean(np.square(a))))
    for n in GRADS:
        if ref[n] is None:
            continue
        if n.startswith("dx_"):
            # Input gradients sequence by sequence and row by row: padding and
            # the causal mask make rows differ in scale, and padded keys get
            # exactly zero.
            for b in range(ref[n].shape[0]):
                e = assert_grad_rows_bf16(got[n][b], ref[n][b], f"{what} {n} sequence {b}")
                print(what, n, b, e)
            continue
        scale = max(rms(ref[n]), rms(ref["dw_" + n[-1]])) if n.startswith("db_") else rms(ref[n])
        if scale == 0.0 and n[-1] in "qk":
            # Every row has one allowed key: the softmax is the constant 1
            # and passes Q and K no gradient.  The GPU's is the rounding
            # left where dP and its row sum cancel; those terms have the
            # size of the value gradient.
            scale = rms(ref["dw_v"])
        e = assert_grad_bf16(got[n], ref[n], scale, f"{what} {n}")
        e16 = float(np.max(np.abs(got[n] - ref16[n])) / scale)
        print(what, n, "vs fp64", e, "max vs bf16-storage", e16 if storage_diag else "-")


CASES = [
    # B, Lq, Lk, D, h, causal, vl_range, bias, self_attn
    (2, 100, 100, 256, 4, True, (1, 100), True, True),
    (2, 70, 150, 192, 3, False, (0, 150), True, False),
    (1, 256, 256, 512, 8, False, None, False, True),
    (2, 129, 129, 128, 2, False, (60, 129), True, True),
    (3, 33, 65, 64, 1, False, (1, 65), True, False),
    (2, 300, 300, 256, 4, True, None, True, True),
]


@pytest.mark.parametrize("B,Lq,Lk,D,h,causal,vlr,bias,self_attn", CASES)
def test_mha_backward_vs_oracle(B, Lq, Lk, D, h, causal, vlr, bias, self_attn):
    inp, g = make(B, Lq, Lk, D, h, causal, vlr, bias, self_attn, seed=7 * B + Lq + 3 * Lk + D)
    check(run_gpu(inp, g), inp, g, f"mha_backward B{B} Lq{Lq} Lk{Lk} D{D} h{h} causal{int(causal)}")


def test_mha_backward_self_attention_split_equals_fused():
    """The same input passed as two tensors gives dx_q and dx_kv apart; their
    sum is the fused self-attention gradient up to fp32 summation order, and
    every weight gradient is the same."""
    inp, g = make(2, 96, 96, 256, 4, True, (1, 96), True, True, seed=11)
    fused = run_gpu(inp, g)
    split = run_gpu(inp, g, separate_kv=True)
    assert fused["dx_kv"] is None and split["dx_kv"] is not None
    total = split["dx_q"] + split["dx_kv"]
    scale = np.sqrt(np.mean(total ** 2))
    assert np.max(np.abs(fused["dx_q"] - total)) <= 1e-5 * max(scale, 1.0)
    for n in GRADS[2:]:
        np.testing.assert_array_equal(fused[n], split[n])


def test_mha_backward_no_queries_gives_zero_gradients():
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    B, Lk, D, h = 2, 40, 128, 2
    inp, _ = make(B, 8, Lk, D, h, False, None, True, False, seed=5)
    t = {n: (None if a is None else to_device(a, torch.bfloat16)) for n, a in inp.tensors.items()}
    xq = torch.empty((B, 0, D), dtype=torch.bfloat16, device="cuda")
    dout = torch.empty((B, 0, D), dtype=torch.bfloat16, device="cuda")
    r = mha.mha_backward(xq, t["x_kv"], t["w_q"], t["w_k"], t["w_v"], t["w_o"], dout, t["b_q"], t["b_k"], t["b_v"],
                         h=h, bias_grads=True)
    torch.cuda.synchronize()
    for n, a in r.items():
        assert a is not None and torch.all(a == 0).item(), n


def test_mha_backward_full_size_decoder():
    """The decoder's masked self-attention at full size (B=64, L=512,
    d_model=512, h=8, causal with padding lengths in [256, 512]) as the
    benchmark launches its training pass: every gradient, whole, against the
    oracle."""
    w = workloads.BY_NAME["decoder_causal"]
    inp = workloads.make_inputs(w)
    rng = np.random.Generator(np.random.PCG64(w.seed + 1000))
    g = workloads.round_to_bf16(rng.standard_normal((w.B, w.Lq, w.d_model)).astype(np.float32))
    check(run_gpu(inp, g), inp, g, "mha_backward decoder_causal full size", storage_diag=False)
