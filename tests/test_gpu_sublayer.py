"""GPU parity of mha_sublayer_forward, the pre-norm residual sublayer
x + MHA(norm(x), ...), against the fp64 oracle, in both printed LayerNorm
forms.  The normalisation is a row-wise kernel that writes norm(x) to the
workspace before the attention layer runs on it; the residual add is fused
into the output projection's epilogue."""
import numpy as np
import pytest

import oracle
import workloads
from parity import assert_bf16, assert_fp32, to_device, to_host

pytestmark = pytest.mark.gpu

CASES = [
    # B, L, Lk (None: self-attention), D, h, causal, lengths, ln_kind, eps, gain/bias, dtype
    (3, 128, None, 256, 4, False, (20, 128), 0, 1e-6, True, "bf16"),
    (2, 100, None, 512, 8, True, None, 1, 1e-5, False, "bf16"),
    (2, 200, None, 128, 2, False, (50, 200), 0, 1e-6, True, "bf16"),
    (2, 64, 90, 256, 4, False, (30, 90), 1, 1e-5, True, "bf16"),
    (2, 20, None, 256, 4, True, None, 0, 1e-6, True, "f32"),
    (2, 33, 47, 128, 2, False, (5, 47), 1, 1e-5, False, "f32"),
]


@pytest.mark.parametrize("B,L,Lk,D,h,causal,vlr,kind,eps,affine,dt", CASES)
def test_sublayer_vs_oracle(B, L, Lk, D, h, causal, vlr, kind, eps, affine, dt):
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    inp = workloads.make_mha_inputs(B, L, Lk or L, D, h, dt, seed=B * 17 + L + D, vl_range=vlr, causal=causal,
                                    self_attn=Lk is None, bias=True)
    rng = np.random.Generator(np.random.PCG64(L * 3 + D))
    t = inp.tensors
    x = workloads._finish(np.asarray(t["x_q"], np.float64) * 2.0 + 0.5, dt)     # rows with a nonzero mean
    g = workloads._finish(1.0 + 0.2 * rng.standard_normal(D), dt) if affine else None
    bb = workloads._finish(0.1 * rng.standard_normal(D), dt) if affine else None
    mem = None if Lk is None else t["x_kv"]
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    dv = lambda a: None if a is None else to_device(a, tdt)
    out = mha.mha_sublayer_forward(dv(x), dv(t["w_q"]), dv(t["w_k"]), dv(t["w_v"]), dv(t["w_o"]), dv(t["b_q"]),
                                   dv(t["b_k"]), dv(t["b_v"]), dv(t["b_o"]), h=h, ln_gain=dv(g), ln_bias=dv(bb),
                                   ln_kind=kind, ln_eps=eps, memory=dv(mem), valid_lens=inp.valid_lens,
                                   causal=causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.mha_sublayer(x, t["w_q"], t["w_k"], t["w_v"], t["w_o"], t["b_q"], t["b_k"], t["b_v"], t["b_o"], h=h,
                              ln_gain=g, ln_bias=bb, ln_kind=kind, ln_eps=eps, memory=mem,
                              valid_lens=inp.valid_lens, causal=causal)
    check = assert_fp32 if dt == "f32" else assert_bf16
    print(check(to_host(out), ref, f"sublayer B{B} L{L} Lk{Lk} D{D} kind{kind} {dt}"))


def test_sublayer_at_the_encoder_shape():
    """The encoder self-attention shape (B=32, L=128, d_model=512, h=8,
    embeddings scaled by sqrt(d_model) plus positional encoding), with the
    Annotated Transformer's LayerNorm: sampled batches against the oracle."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    w = workloads.BY_NAME["encoder_self"]
    inp = workloads.make_inputs(w)
    t = inp.tensors
    dv = lambda a: None if a is None else to_device(a, torch.bfloat16)
    out = mha.mha_sublayer_forward(dv(t["x_q"]), dv(t["w_q"]), dv(t["w_k"]), dv(t["w_v"]), dv(t["w_o"]), h=w.h,
                                   valid_lens=inp.valid_lens, out_dtype=torch.float32)
    torch.cuda.synchronize()
    bs = [0, 13, 31]
    ref = oracle.mha_sublayer(t["x_q"][bs], t["w_q"], t["w_k"], t["w_v"], t["w_o"], h=w.h,
                              valid_lens=inp.valid_lens[bs])
    print(assert_bf16(to_host(out)[bs], ref, "sublayer at the encoder shape"))
