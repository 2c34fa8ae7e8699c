"""GPU parity of sdpa_backward (dq, dk, dv) through the C ABI against the
fp64 oracle's backward.

fp32 inputs run on FMA kernels in fp32 on the exact input values and are
held to the fp32 bar (norm-wise 1e-5).  bf16 inputs run on bf16 MFMA with
fp32 accumulation: the weights and ds are rounded to bf16 for their products
(as the forward rounds its weights), and the forward output o, which enters
D_i = do_i . o_i, is itself bf16; they are held to the bf16 bar."""
import numpy as np
import pytest

import oracle
import workloads
from parity import assert_bf16, assert_fp32, to_device, to_host

pytestmark = pytest.mark.gpu

CASES = [
    # B, h, Lq, Lk, causal, lengths, dtype
    (2, 3, 70, 70, True, None, "f32"),
    (2, 2, 45, 100, False, "2d", "bf16"),
    (2, 4, 130, 77, False, "1d", "f32"),
    (2, 2, 33, 33, True, "2d", "bf16"),
    (3, 1, 64, 96, False, "1d", "bf16"),
    (2, 4, 512, 512, True, None, "bf16"),
    # several 64-row workgroups and 128-row steps with ragged tails
    (2, 2, 300, 260, False, "1d", "bf16"),
    (1, 3, 200, 200, True, "2d", "bf16"),
    (2, 2, 257, 257, True, None, "bf16"),
    (1, 2, 129, 1, False, None, "bf16"),
]


def _lengths(kind, rng, B, Lq, Lk):
    if kind is None:
        return None
    if kind == "1d":
        vl = rng.integers(1, Lk + 1, size=B).astype(np.int32)
        vl[0] = 0                                            # a fully masked sequence
        return vl
    vl = rng.integers(-1, Lk + 3, size=(B, Lq)).astype(np.int32)
    vl[0, :3] = [0, 1, Lk]
    return vl


@pytest.mark.parametrize("B,h,Lq,Lk,causal,kind,dt", CASES)
def test_backward_vs_oracle(B, h, Lq, Lk, causal, kind, dt):
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    rng = np.random.Generator(np.random.PCG64(B * 7919 + Lq * 31 + Lk))
    q = workloads._finish(rng.standard_normal((B, h, Lq, 64)), dt)
    k = workloads._finish(rng.standard_normal((B, h, Lk, 64)), dt)
    v = workloads._finish(rng.standard_normal((B, h, Lk, 64)), dt)
    g = workloads._finish(rng.standard_normal((B, h, Lq, 64)), dt)
    vl = _lengths(kind, rng, B, Lq, Lk)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    tq, tk, tv, tg = (to_device(x, tdt) for x in (q, k, v, g))
    o = mha.sdpa_forward(tq, tk, tv, valid_lens=vl, causal=causal)          # the forward output, in dt
    gq, gk, gv = mha.sdpa_backward(tq, tk, tv, o, tg, valid_lens=vl, causal=causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.sdpa_backward(q, k, v, g, valid_lens=vl, causal=causal)
    check = assert_fp32 if dt == "f32" else assert_bf16
    for name, got, ref in (("dq", gq, rq), ("dk", gk, rk), ("dv", gv, rv)):
        e = check(to_host(got), ref, f"{name} B{B} h{h} Lq{Lq} Lk{Lk} causal={causal} lengths={kind} {dt}")
        print(name, e)


@pytest.mark.parametrize("B,h,Lq,Lk,causal,kind,dt", [c for c in CASES if c[6] == "bf16"])
def test_backward_with_forward_lse_vs_oracle(B, h, Lq, Lk, causal, kind, dt):
    """The path a training step takes: the forward keeps each query's
    log-sum-exp and the backward recomputes the weights from it (one launch
    for the query- and key-side workgroups).  Lengths per query have no
    forward with the statistic, so there the oracle's log-sum-exp (in fp32,
    a fully masked row's fill taken out) is the input."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    rng = np.random.Generator(np.random.PCG64(B * 7919 + Lq * 31 + Lk))
    q = workloads._finish(rng.standard_normal((B, h, Lq, 64)), dt)
    k = workloads._finish(rng.standard_normal((B, h, Lk, 64)), dt)
    v = workloads._finish(rng.standard_normal((B, h, Lk, 64)), dt)
    g = workloads._finish(rng.standard_normal((B, h, Lq, 64)), dt)
    vl = _lengths(kind, rng, B, Lq, Lk)
    tq, tk, tv, tg = (to_device(x, torch.bfloat16) for x in (q, k, v, g))
    if kind == "2d":
        o = mha.sdpa_forward(tq, tk, tv, valid_lens=vl, causal=causal)
        ref_lse = oracle.sdpa_lse(q, k, valid_lens=vl, causal=causal)
        ref_lse[ref_lse < -1e8] += 1e9
        lse = torch.from_numpy(ref_lse.astype(np.float32)).cuda()
    else:
        o, lse = mha.sdpa_forward(tq, tk, tv, valid_lens=vl, causal=causal, return_lse=True)
    gq, gk, gv = mha.sdpa_backward(tq, tk, tv, o, tg, valid_lens=vl, causal=causal, out_dtype=torch.float32,
                                   lse=lse)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.sdpa_backward(q, k, v, g, valid_lens=vl, causal=causal)
    for name, got, ref in (("dq", gq, rq), ("dk", gk, rk), ("dv", gv, rv)):
        e = assert_bf16(to_host(got), ref, f"{name} with lse B{B} h{h} Lq{Lq} Lk{Lk} causal={causal} lengths={kind}")
        print(name, e)


def test_backward_bf16_outputs_and_strided_views():
    """bf16 gradients into [B, L, h, d] views (strided), lengths per sequence."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    rng = np.random.Generator(np.random.PCG64(99))
    B, h, L = 2, 3, 90
    x = [workloads._finish(rng.standard_normal((B, L, h, 64)), "bf16") for _ in range(4)]
    vl = np.array([90, 41], np.int32)
    tq, tk, tv, tg = (to_device(a, torch.bfloat16).transpose(1, 2) for a in x)   # [B, h, L, d] views
    o = mha.sdpa_forward(tq, tk, tv, valid_lens=vl)
    gq, gk, gv = mha.sdpa_backward(tq, tk, tv, o, tg, valid_lens=vl)
    torch.cuda.synchronize()
    q, k, v, g = (a.transpose(0, 2, 1, 3) for a in x)
    for got, ref in zip((gq, gk, gv), oracle.sdpa_backward(q, k, v, g, valid_lens=vl)):
        assert got.dtype == torch.bfloat16
        assert_bf16(to_host(got), ref, "bf16 gradients")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_backward_no_queries_zeroes_key_gradients(dt):
    """No query rows: dk and dv are empty sums, written as zeros over
    whatever the buffers held."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    B, h, Lk = 2, 3, 50
    q = torch.empty((B, h, 0, 64), dtype=tdt, device="cuda")
    k, v = (torch.randn((B, h, Lk, 64), device="cuda").to(tdt) for _ in range(2))
    gq, gk, gv = mha.sdpa_backward(q, k, v, q, q, valid_lens=[50, 7])
    torch.cuda.synchronize()
    assert gq.numel() == 0
    assert torch.all(gk == 0).item() and torch.all(gv == 0).item()


def test_backward_full_size_sampled_heads():
    """The causal backward workload at full size (B=4 h=8 L=1024, bf16 in,
    fp32 gradients) as the benchmark launches it; two (batch, head) slices,
    the first and the last, are checked whole against the oracle."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    w = workloads.BY_NAME["backward_causal"]
    inp = workloads.make_inputs(w)
    q, k, v = (inp.tensors[n] for n in "qkv")
    rng = np.random.Generator(np.random.PCG64(w.seed + 1000))
    g = workloads._finish(rng.standard_normal(q.shape), "bf16")
    tq, tk, tv, tg = (to_device(x, torch.bfloat16) for x in (q, k, v, g))
    o, lse = mha.sdpa_forward(tq, tk, tv, causal=True, return_lse=True)
    grads = {"own statistics": mha.sdpa_backward(tq, tk, tv, o, tg, causal=True, out_dtype=torch.float32),
             "forward lse": mha.sdpa_backward(tq, tk, tv, o, tg, causal=True, out_dtype=torch.float32, lse=lse)}
    torch.cuda.synchronize()
    for b, hd in ((0, 0), (w.B - 1, w.h - 1)):
        sl = lambda x: x[b:b + 1, hd:hd + 1]
        ref = oracle.sdpa_backward(sl(q), sl(k), sl(v), sl(g), causal=True)
        for path, (gq, gk, gv) in grads.items():
            for name, got, r in (("dq", gq, ref[0]), ("dk", gk, ref[1]), ("dv", gv, ref[2])):
                e = assert_bf16(sl(to_host(got)), r, f"{name} full size b{b} h{hd} ({path})")
                print(path, name, b, hd, e)
