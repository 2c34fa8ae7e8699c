"""GPU parity of mha_forward (projections, head split, attention, merge,
output projection) through the C ABI against the fp64 oracle.

bf16 path: graded against the plain fp64 oracle on the same bf16 inputs and
weights.  The oracle's bf16-storage mode (Q, K, V and the merged heads
rounded to bf16 between steps) is printed beside it as a diagnostic."""
import numpy as np
import pytest

import oracle
import workloads
from parity import assert_bf16, assert_fp32, errors, to_device, to_host

pytestmark = pytest.mark.gpu


def run_gpu(inp, out_f32=True):
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    w = inp.workload
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = {n: (None if a is None else to_device(a, dt)) for n, a in inp.tensors.items()}
    if w.self_attn:
        t["x_kv"] = t["x_q"]
    out_dtype = torch.float32 if (out_f32 or w.dtype == "f32") else torch.bfloat16
    out = mha.mha_forward(t["x_q"], t["x_kv"], t["w_q"], t["w_k"], t["w_v"], t["w_o"],
                          t["b_q"], t["b_k"], t["b_v"], t["b_o"], h=w.h,
                          valid_lens=inp.valid_lens, causal=w.causal, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return to_host(out)


def run_oracle(inp, bf16_stages, batches=None, rows=None):
    t = inp.tensors
    sel = (lambda a: a) if batches is None else (lambda a: None if a is None else a[batches])
    vl = inp.valid_lens
    if vl is not None and batches is not None:
        vl = vl[batches]
    return oracle.mha(sel(t["x_q"]), sel(t["x_kv"]), t["w_q"], t["w_k"], t["w_v"], t["w_o"],
                      t["b_q"], t["b_k"], t["b_v"], t["b_o"], h=inp.workload.h, valid_lens=vl,
                      causal=inp.workload.causal, rows=rows, bf16_stages=bf16_stages)


MHA_BF16_CASES = [
    # B, Lq, Lk, D, h, causal, vl_range, bias, self_attn
    (2, 37, 37, 512, 8, True, (1, 37), False, True),
    (2, 50, 90, 256, 4, False, (10, 90), True, False),
    (3, 130, 130, 128, 2, False, (0, 130), True, True),
    (1, 1, 1, 64, 1, False, None, False, True),
    (2, 200, 140, 192, 3, False, None, True, False),
    # self-attention with L <= 128 takes the single-pass kernel: full 128
    # rows with fully masked rows possible, a causal length between the key
    # halves, and exactly one key half
    (4, 128, 128, 256, 4, False, (0, 128), True, True),
    (2, 100, 100, 128, 2, True, None, False, True),
    (3, 64, 64, 192, 3, False, (1, 64), True, True),
]


@pytest.mark.parametrize("B,Lq,Lk,D,h,causal,vlr,bias,self_attn", MHA_BF16_CASES)
@pytest.mark.parametrize("out_f32", [True, False])
def test_mha_bf16_vs_oracle(B, Lq, Lk, D, h, causal, vlr, bias, self_attn, out_f32):
    inp = workloads.make_mha_inputs(B, Lq, Lk, D, h, "bf16", seed=B * 100 + Lq + Lk, vl_range=vlr,
                                    causal=causal, self_attn=self_attn, bias=bias)
    g = run_gpu(inp, out_f32)
    e = assert_bf16(g, run_oracle(inp, bf16_stages=False), f"mha bf16 B{B} Lq{Lq} Lk{Lk} D{D} h{h}")
    print("vs fp64 oracle", e, "vs bf16-storage oracle", errors(g, run_oracle(inp, bf16_stages=True)))


# Several 256-query blocks and more than four 128-key chunks, with ragged key
# lengths that include 0 (a fully masked sequence) and the full length.
# These shapes take the projected route (Q/K/V GEMM, then attention on the
# hi + lo projections); the last two keep the single-kernel route with two
# causal blocks.
MULTI_BLOCK_CASES = [
    # B, Lq, Lk, D, h, self_attn, causal, lengths
    (3, 600, 600, 128, 2, True, False, [0, 600, 333]),
    (3, 300, 700, 256, 4, False, False, [700, 0, 517]),
    (2, 513, 513, 192, 3, True, False, [513, 257]),
    (2, 1000, 1000, 128, 2, True, True, [1000, 611]),
    (2, 260, 900, 256, 4, False, False, [900, 1]),
    (2, 512, 512, 128, 2, True, True, [0, 300]),
    (2, 400, 400, 192, 3, True, True, [400, 129]),
]


@pytest.mark.parametrize("B,Lq,Lk,D,h,self_attn,causal,lens", MULTI_BLOCK_CASES)
def test_mha_bf16_multi_block_ragged(B, Lq, Lk, D, h, self_attn, causal, lens):
    inp = workloads.make_mha_inputs(B, Lq, Lk, D, h, "bf16", seed=7000 + Lq + Lk, vl_range=(1, Lk),
                                    causal=causal, self_attn=self_attn, bias=True)
    inp.valid_lens = np.array(lens, dtype=np.int32)
    g = run_gpu(inp, True)
    e = assert_bf16(g, run_oracle(inp, bf16_stages=False), f"mha bf16 B{B} Lq{Lq} Lk{Lk} lengths {lens}")
    print("vs fp64 oracle", e)


def test_mha_bf16_projected_route_large_logits():
    """The projected route on embeddings scaled by sqrt(d_model) plus the
    positional encoding (logits with std in the hundreds, as in the encoder
    workload) at a length that takes that route: Q and K travel as hi + lo
    bf16 planes, so the result stays within the bar."""
    inp = workloads.make_mha_inputs(2, 600, 600, 256, 4, "bf16", seed=4242, vl_range=(300, 600),
                                    x_kind="embed_pe", self_attn=True, bias=True)
    g = run_gpu(inp, True)
    e = assert_bf16(g, run_oracle(inp, bf16_stages=False), "projected route, large logits")
    print("vs fp64 oracle", e)


# Projections large enough for the 256 x 256 GEMM tiles: self-attention
# (Q/K/V over one input) with a row count past the last full tile, and
# cross-attention whose query projection, key/value projections and output
# projection all take them, the last two with ragged row counts.  The oracle
# checks sampled rows of every batch.
LARGE_PROJECTION_CASES = [
    # B, Lq, Lk, D, h, self_attn, lengths
    (2, 5500, 5500, 512, 8, True, [5500, 3001]),
    (2, 8200, 300, 1024, 16, False, [300, 17]),
]


@pytest.mark.parametrize("B,Lq,Lk,D,h,self_attn,lens", LARGE_PROJECTION_CASES)
@pytest.mark.parametrize("out_f32", [True, False])
def test_mha_bf16_large_projections(B, Lq, Lk, D, h, self_attn, lens, out_f32):
    from parity import sample_rows
    inp = workloads.make_mha_inputs(B, Lq, Lk, D, h, "bf16", seed=9100 + Lq, vl_range=(1, Lk),
                                    self_attn=self_attn, bias=True)
    inp.valid_lens = np.array(lens, dtype=np.int32)
    g = run_gpu(inp, out_f32)
    rows = sample_rows(Lq, 40, np.random.Generator(np.random.PCG64(Lq)))
    e = assert_bf16(g[:, rows], run_oracle(inp, bf16_stages=False, rows=rows),
                    f"mha bf16 large projections B{B} Lq{Lq} Lk{Lk} D{D}")
    print("vs fp64 oracle", e)


MHA_F32_CASES = [
    (2, 10, 10, 512, 8, False, (3, 10), False, True),
    (2, 33, 45, 256, 4, False, (0, 45), True, False),
    (2, 70, 70, 128, 2, True, (1, 70), True, True),
]


@pytest.mark.parametrize("B,Lq,Lk,D,h,causal,vlr,bias,self_attn", MHA_F32_CASES)
def test_mha_f32_vs_oracle(B, Lq, Lk, D, h, causal, vlr, bias, self_attn):
    inp = workloads.make_mha_inputs(B, Lq, Lk, D, h, "f32", seed=B * 10 + Lq + Lk, vl_range=vlr,
                                    causal=causal, self_attn=self_attn, bias=bias)
    g = run_gpu(inp)
    assert_fp32(g, run_oracle(inp, bf16_stages=False), f"mha f32 B{B} Lq{Lq} Lk{Lk} D{D}")


def test_mha_empty_batch_is_noop():
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    x = torch.zeros((0, 8, 128), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((128, 128), dtype=torch.bfloat16, device="cuda")
    out = mha.mha_forward(x, x, w, w, w, w, h=2)
    assert out.shape == (0, 8, 128)


def test_mha_invalid_arguments_raise():
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    x = torch.zeros((1, 8, 128), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((128, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mha.MhaError):
        mha.mha_forward(x, x, w, w, w, w, h=4)            # d_k = 32: unsupported
    y = torch.zeros((1, 9, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mha.MhaError):
        mha.mha_forward(x, y, w, w, w, w, h=2, causal=True)   # causal needs Lq == Lk
