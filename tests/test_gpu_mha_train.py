"""GPU parity of the training pair: mha_forward_train (the layer's output,
with Q, K, V, the merged heads and each query's log-sum-exp kept) and
mha_backward_saved (the gradients from those kept tensors).

The output is graded against the fp64 oracle with the bf16 bar, as
mha_forward's is.  The gradients are graded against the oracle's chain rule
with the gradient bar and must equal, bit for bit, mha_backward's on the
same inputs: both run the same projection and attention launches, one of
them in the forward call and the other inside the backward."""
import numpy as np
import pytest

import oracle
import workloads
from parity import assert_bf16, errors, to_device, to_host
from test_gpu_mha_backward import GRADS, check, make

pytestmark = pytest.mark.gpu


def run_pair(inp, g, out_f32=True):
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    w = inp.workload
    t = {n: (None if a is None else to_device(a, torch.bfloat16)) for n, a in inp.tensors.items()}
    if w.self_attn:
        t["x_kv"] = t["x_q"]
    out, saved = mha.mha_forward_train(t["x_q"], t["x_kv"], t["w_q"], t["w_k"], t["w_v"], t["w_o"], t["b_q"],
                                       t["b_k"], t["b_v"], t["b_o"], h=w.h, valid_lens=inp.valid_lens,
                                       causal=w.causal, out_dtype=torch.float32 if out_f32 else torch.bfloat16)
    dout = to_device(g, torch.bfloat16)
    kept = mha.mha_backward(t["x_q"], t["x_kv"], t["w_q"], t["w_k"], t["w_v"], t["w_o"], dout, h=w.h,
                            valid_lens=inp.valid_lens, causal=w.causal, bias_grads=True, saved=saved)
    again = mha.mha_backward(t["x_q"], t["x_kv"], t["w_q"], t["w_k"], t["w_v"], t["w_o"], dout, t["b_q"], t["b_k"],
                             t["b_v"], h=w.h, valid_lens=inp.valid_lens, causal=w.causal, bias_grads=True)
    torch.cuda.synchronize()
    host = lambda r: {n: (None if a is None else to_host(a)) for n, a in r.items()}
    return to_host(out), host(kept), host(again)


def oracle_out(inp, bf16_stages):
    t = inp.tensors
    w = inp.workload
    return oracle.mha(t["x_q"], t["x_kv"], t["w_q"], t["w_k"], t["w_v"], t["w_o"], t["b_q"], t["b_k"], t["b_v"],
                      t["b_o"], h=w.h, valid_lens=inp.valid_lens, causal=w.causal, bf16_stages=bf16_stages)


CASES = [
    # B, Lq, Lk, D, h, causal, vl_range, bias, self_attn
    (2, 100, 100, 256, 4, True, (1, 100), True, True),
    (2, 70, 150, 192, 3, False, (0, 150), True, False),
    (1, 300, 300, 512, 8, True, None, False, True),
    (3, 33, 65, 64, 1, False, (1, 65), True, False),
]


@pytest.mark.parametrize("B,Lq,Lk,D,h,causal,vlr,bias,self_attn", CASES)
@pytest.mark.parametrize("out_f32", [True, False])
def test_training_pair_vs_oracle(B, Lq, Lk, D, h, causal, vlr, bias, self_attn, out_f32):
    what = f"training pair B{B} Lq{Lq} Lk{Lk} D{D} h{h} causal{int(causal)}"
    inp, g = make(B, Lq, Lk, D, h, causal, vlr, bias, self_attn, seed=5 * B + Lq + 2 * Lk + D)
    out, kept, again = run_pair(inp, g, out_f32)
    e = assert_bf16(out, oracle_out(inp, False), what + " output")
    print(what, "output vs fp64", e, "vs bf16-storage", errors(out, oracle_out(inp, True)))
    for n in GRADS:
        if again[n] is None:
            assert kept[n] is None, n
            continue
        np.testing.assert_array_equal(kept[n], again[n], err_msg=f"{what} {n}: saved vs recomputed forward")
    check(kept, inp, g, what, storage_diag=False)


def test_training_pair_no_queries():
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    B, Lk, D, h = 2, 40, 128, 2
    inp, _ = make(B, 8, Lk, D, h, False, None, True, False, seed=5)
    t = {n: (None if a is None else to_device(a, torch.bfloat16)) for n, a in inp.tensors.items()}
    xq = torch.empty((B, 0, D), dtype=torch.bfloat16, device="cuda")
    out, saved = mha.mha_forward_train(xq, t["x_kv"], t["w_q"], t["w_k"], t["w_v"], t["w_o"], t["b_q"], t["b_k"],
                                       t["b_v"], t["b_o"], h=h)
    r = mha.mha_backward(xq, t["x_kv"], t["w_q"], t["w_k"], t["w_v"], t["w_o"], xq, h=h, bias_grads=True,
                         saved=saved)
    torch.cuda.synchronize()
    assert out.shape == (B, 0, D)
    for n, a in r.items():
        assert a is not None and torch.all(a == 0).item(), n


def test_training_pair_full_size_decoder():
    """The decoder workload (B=64, L=512, d_model=512, h=8, causal, lengths in
    [256, 512]) as the benchmark runs its training pass: the saved-tensor
    gradients equal the recomputing backward's bit for bit, and the output
    meets the bar on sampled rows of every sequence."""
    from parity import sample_rows
    w = workloads.BY_NAME["decoder_causal"]
    inp = workloads.make_inputs(w)
    rng = np.random.Generator(np.random.PCG64(w.seed + 1000))
    g = workloads.round_to_bf16(rng.standard_normal((w.B, w.Lq, w.d_model)).astype(np.float32))
    out, kept, again = run_pair(inp, g, out_f32=True)
    for n in GRADS:
        if again[n] is None:
            assert kept[n] is None, n
            continue
        np.testing.assert_array_equal(kept[n], again[n], err_msg=f"decoder_causal {n}: saved vs recomputed forward")
    rows = sample_rows(w.Lq, 24, np.random.Generator(np.random.PCG64(17)))
    batches = np.array([0, 17, 41, 63])
    t = inp.tensors
    sel = lambda a: None if a is None else a[batches]
    ref = oracle.mha(sel(t["x_q"]), sel(t["x_kv"]), t["w_q"], t["w_k"], t["w_v"], t["w_o"], t["b_q"], t["b_k"],
                     t["b_v"], t["b_o"], h=w.h, valid_lens=inp.valid_lens[batches], causal=True, rows=rows)
    e = assert_bf16(out[batches][:, rows], ref, "training pair decoder_causal output")
    print("training pair decoder_causal output vs fp64", e)
