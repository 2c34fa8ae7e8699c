"""A seeded sweep of odd shapes through the bf16 entry points against the
fp64 oracle: query and key counts on either side of the kernels' tile edges
(32, 64, 128, 256), Lq different from Lk, lengths of 0, 1, the full count
and past it, with and without the causal rule, both output dtypes; the
attention core's backward on both of its statistic paths, the layer's
training pair against its recomputing backward, the weights export of the
attention core and of the multi-head layer, the pre-norm sublayer, and the
fp32 entry points.  The shapes come from a fixed generator, so every run
checks the same cases."""
import numpy as np
import pytest

import oracle
import workloads
from parity import assert_bf16, assert_fp32, to_device, to_host
from test_gpu_mha_backward import GRADS, check, make
from test_gpu_mha_train import oracle_out, run_pair

pytestmark = pytest.mark.gpu

EDGES = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300]


def _cases(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for c in range(n):
        B = int(rng.integers(1, 4))
        causal = bool(rng.integers(0, 2))
        Lq = int(rng.choice(EDGES))
        Lk = Lq if causal else int(rng.choice(EDGES))
        kind = int(rng.integers(0, 4))          # 0: none, 1: random, 2: with 0 and full, 3: past the end
        if kind == 0:
            lens = None
        elif kind == 1:
            lens = rng.integers(1, Lk + 1, size=B).tolist()
        elif kind == 2:
            lens = ([0, Lk] + rng.integers(1, Lk + 1, size=B).tolist())[:B]
        else:
            lens = (Lk + rng.integers(1, 50, size=B)).tolist()
        out.append((c, B, Lq, Lk, causal, lens))
    return out


SDPA_CASES = _cases(24, 2024)


@pytest.mark.parametrize("c,B,Lq,Lk,causal,lens", SDPA_CASES)
def test_sweep_sdpa_bf16(c, B, Lq, Lk, causal, lens):
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    h = 1 + c % 3
    inp = workloads.make_sdpa_inputs(B, h, Lq, Lk, 64, "bf16", seed=500 + c)
    vl = None if lens is None else np.array(lens, dtype=np.int32)
    q, k, v = (inp.tensors[n] for n in ("q", "k", "v"))
    out_dtype = torch.float32 if c % 2 else torch.bfloat16
    o = mha.sdpa_forward(to_device(q, torch.bfloat16), to_device(k, torch.bfloat16), to_device(v, torch.bfloat16),
                         valid_lens=vl, causal=causal, out_dtype=out_dtype)
    torch.cuda.synchronize()
    e = assert_bf16(to_host(o), oracle.sdpa(q, k, v, valid_lens=vl, causal=causal),
                    f"sweep sdpa case {c}: B{B} h{h} Lq{Lq} Lk{Lk} causal{int(causal)} lengths {lens}")
    print(c, e)


MHA_CASES = _cases(12, 77)


@pytest.mark.parametrize("c,B,Lq,Lk,causal,lens", MHA_CASES)
def test_sweep_mha_bf16(c, B, Lq, Lk, causal, lens):
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    h = 1 + c % 4
    D = 64 * h
    self_attn = causal or c % 3 == 0
    if self_attn:
        Lk = Lq
        if lens is not None:
            lens = [min(x, Lq + 7) if x > Lq else x for x in lens]
    inp = workloads.make_mha_inputs(B, Lq, Lk, D, h, "bf16", seed=900 + c, causal=causal, self_attn=self_attn,
                                    bias=c % 2 == 0)
    vl = None if lens is None else np.array(lens, dtype=np.int32)
    t = {n: (None if a is None else to_device(a, torch.bfloat16)) for n, a in inp.tensors.items()}
    if self_attn:
        t["x_kv"] = t["x_q"]
    out = mha.mha_forward(t["x_q"], t["x_kv"], t["w_q"], t["w_k"], t["w_v"], t["w_o"], t["b_q"], t["b_k"], t["b_v"],
                          t["b_o"], h=h, valid_lens=vl, causal=causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    r = inp.tensors
    ref = oracle.mha(r["x_q"], r["x_kv"], r["w_q"], r["w_k"], r["w_v"], r["w_o"], r["b_q"], r["b_k"], r["b_v"], r["b_o"],
                     h=h, valid_lens=vl, causal=causal)
    e = assert_bf16(to_host(out), ref,
                    f"sweep mha case {c}: B{B} Lq{Lq} Lk{Lk} D{D} causal{int(causal)} lengths {lens}")
    print(c, e)


DECODE_CASES = [(c, B, Lk, lens) for c, B, Lq, Lk, causal, lens in _cases(10, 5)]


@pytest.mark.parametrize("c,B,L,lens", DECODE_CASES)
def test_sweep_decode_bf16(c, B, L, lens):
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    h = 1 + c % 4
    inp = workloads.make_sdpa_inputs(B, h, 1, L, 64, "bf16", seed=1300 + c)
    lens = lens if lens is not None else [L] * B
    vl = np.array(lens, dtype=np.int32)
    q, k, v = (inp.tensors[n] for n in ("q", "k", "v"))
    o = mha.sdpa_decode(to_device(q[:, :, 0], torch.bfloat16), to_device(k, torch.bfloat16),
                        to_device(v, torch.bfloat16), vl)
    torch.cuda.synchronize()
    ref = oracle.sdpa(q, k, v, valid_lens=vl)[:, :, 0]
    e = assert_bf16(to_host(o), ref, f"sweep decode case {c}: B{B} h{h} L{L} lengths {lens}")
    print(c, e)


BWD_CASES = _cases(16, 4242)


@pytest.mark.parametrize("c,B,Lq,Lk,causal,lens", BWD_CASES)
def test_sweep_backward_bf16(c, B, Lq, Lk, causal, lens):
    """sdpa_backward on both of its paths (the statistic found in its own
    pass, and given by the forward) against the oracle's gradients."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    h = 1 + c % 3
    rng = np.random.Generator(np.random.PCG64(7700 + c))
    q, k, v, g = (workloads._finish(rng.standard_normal((B, h, L, 64)), "bf16") for L in (Lq, Lk, Lk, Lq))
    vl = None if lens is None else np.array(lens, dtype=np.int32)
    tq, tk, tv, tg = (to_device(x, torch.bfloat16) for x in (q, k, v, g))
    o, lse = mha.sdpa_forward(tq, tk, tv, valid_lens=vl, causal=causal, return_lse=True)
    own = mha.sdpa_backward(tq, tk, tv, o, tg, valid_lens=vl, causal=causal, out_dtype=torch.float32)
    given = mha.sdpa_backward(tq, tk, tv, o, tg, valid_lens=vl, causal=causal, out_dtype=torch.float32, lse=lse)
    torch.cuda.synchronize()
    ref = oracle.sdpa_backward(q, k, v, g, valid_lens=vl, causal=causal)
    for path, grads in (("own statistic", own), ("forward statistic", given)):
        for name, got, r in zip(("dq", "dk", "dv"), grads, ref):
            e = assert_bf16(to_host(got), r, f"sweep backward case {c} ({path}) {name}: B{B} h{h} Lq{Lq} Lk{Lk} "
                                             f"causal{int(causal)} lengths {lens}")
            print(c, path, name, e)


LAYER_BWD_CASES = _cases(10, 31337)


@pytest.mark.parametrize("c,B,Lq,Lk,causal,lens", LAYER_BWD_CASES)
def test_sweep_layer_backward_bf16(c, B, Lq, Lk, causal, lens):
    """mha_forward_train, mha_backward_saved and mha_backward on odd shapes:
    the output and every gradient against the oracle, and the saved-tensor
    gradients equal, bit for bit, to the recomputing backward's."""
    h = 1 + c % 4
    D = 64 * h
    self_attn = causal or c % 3 == 0
    if self_attn:
        Lk = Lq
        if lens is not None:
            lens = [min(x, Lq + 7) if x > Lq else x for x in lens]
    inp, g = make(B, Lq, Lk, D, h, causal, None, c % 2 == 0, self_attn, seed=2600 + c)
    inp.valid_lens = None if lens is None else np.array(lens, dtype=np.int32)
    what = f"sweep layer backward case {c}: B{B} Lq{Lq} Lk{Lk} D{D} causal{int(causal)} lengths {lens}"
    out, kept, again = run_pair(inp, g, out_f32=c % 2 == 1)
    e = assert_bf16(out, oracle_out(inp, False), what + " output")
    print(what, "output", e)
    for n in GRADS:
        if again[n] is None:
            assert kept[n] is None, n
            continue
        np.testing.assert_array_equal(kept[n], again[n], err_msg=f"{what} {n}: saved vs recomputed forward")
    check(again, inp, g, what, storage_diag=False)


WEIGHTS_CASES = _cases(14, 8080)


@pytest.mark.parametrize("c,B,Lq,Lk,causal,lens", WEIGHTS_CASES)
def test_sweep_weights_bf16(c, B, Lq, Lk, causal, lens):
    """The weights export on odd shapes; odd cases take one length per query
    (drawn around the case's per-sequence length, 0 and past Lk included)."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    h = 1 + c % 3
    inp = workloads.make_sdpa_inputs(B, h, Lq, Lk, 64, "bf16", seed=3100 + c)
    q, k, v = (inp.tensors[n] for n in ("q", "k", "v"))
    vl = None if lens is None else np.array(lens, dtype=np.int32)
    if vl is not None and c % 2:
        rng = np.random.Generator(np.random.PCG64(3200 + c))
        vl = np.clip(vl[:, None] + rng.integers(-8, 9, size=(B, Lq)), 0, Lk + 20).astype(np.int32)
    o, p = mha.sdpa_forward(to_device(q, torch.bfloat16), to_device(k, torch.bfloat16), to_device(v, torch.bfloat16),
                            valid_lens=vl, causal=causal, out_dtype=torch.float32, return_weights=True)
    torch.cuda.synchronize()
    ro, rp = oracle.sdpa(q, k, v, valid_lens=vl, causal=causal, return_weights=True)
    what = f"sweep weights case {c}: B{B} h{h} Lq{Lq} Lk{Lk} causal{int(causal)} lengths {lens}"
    assert_fp32(to_host(p), rp, what + " weights")
    assert_bf16(to_host(o), ro, what + " output")


MHA_WEIGHTS_CASES = _cases(8, 4321)


@pytest.mark.parametrize("c,B,Lq,Lk,causal,lens", MHA_WEIGHTS_CASES)
def test_sweep_mha_weights_bf16(c, B, Lq, Lk, causal, lens):
    """The multi-head layer exporting its weights on odd shapes (projections
    to fp32 Q, K, V, then the inspection kernel): output and per-head
    weights against the oracle."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    from test_gpu_inspect import _oracle_mha_weights
    h = 1 + c % 4
    D = 64 * h
    self_attn = causal or c % 2 == 0
    if self_attn:
        Lk = Lq
        if lens is not None:
            lens = [min(x, Lq + 3) for x in lens]
    inp = workloads.make_mha_inputs(B, Lq, Lk, D, h, "bf16", seed=4400 + c, causal=causal, self_attn=self_attn,
                                    bias=c % 3 == 0)
    vl = None if lens is None else np.array(lens, dtype=np.int32)
    t = {n: (None if a is None else to_device(a, torch.bfloat16)) for n, a in inp.tensors.items()}
    if self_attn:
        t["x_kv"] = t["x_q"]
    out, p = mha.mha_forward(t["x_q"], t["x_kv"], t["w_q"], t["w_k"], t["w_v"], t["w_o"], t["b_q"], t["b_k"], t["b_v"],
                             t["b_o"], h=h, valid_lens=vl, causal=causal, out_dtype=torch.float32, return_weights=True)
    torch.cuda.synchronize()
    r = inp.tensors
    ref = oracle.mha(r["x_q"], r["x_kv"], r["w_q"], r["w_k"], r["w_v"], r["w_o"], r["b_q"], r["b_k"], r["b_v"], r["b_o"],
                     h=h, valid_lens=vl, causal=causal)
    what = f"sweep mha weights case {c}: B{B} Lq{Lq} Lk{Lk} D{D} causal{int(causal)} lengths {lens}"
    assert_bf16(to_host(out), ref, what + " output")
    assert_bf16(to_host(p), _oracle_mha_weights(inp, vl), what + " weights")


SUBLAYER_CASES = _cases(8, 2718)


@pytest.mark.parametrize("c,B,Lq,Lk,causal,lens", SUBLAYER_CASES)
def test_sweep_sublayer_bf16(c, B, Lq, Lk, causal, lens):
    """x + MHA(LayerNorm(x)) on odd shapes, both LayerNorm forms, with and
    without gain and bias, self-attention or attention to a memory."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    h = 1 + c % 4
    D = 64 * h
    self_attn = causal or c % 2 == 0
    if self_attn:
        Lk = Lq
        if lens is not None:
            lens = [min(x, Lq + 3) for x in lens]
    inp = workloads.make_mha_inputs(B, Lq, Lk, D, h, "bf16", seed=5500 + c, causal=causal, self_attn=self_attn,
                                    bias=True)
    vl = None if lens is None else np.array(lens, dtype=np.int32)
    t = inp.tensors
    rng = np.random.Generator(np.random.PCG64(5600 + c))
    x = workloads._finish(np.asarray(t["x_q"], np.float64) * 1.5 - 0.25, "bf16")
    affine = c % 3 != 0
    g = workloads._finish(1.0 + 0.2 * rng.standard_normal(D), "bf16") if affine else None
    bb = workloads._finish(0.1 * rng.standard_normal(D), "bf16") if affine else None
    kind, eps = c % 2, (1e-6 if c % 2 == 0 else 1e-5)
    mem = None if self_attn else t["x_kv"]
    dv = lambda a: None if a is None else to_device(a, torch.bfloat16)
    out = mha.mha_sublayer_forward(dv(x), dv(t["w_q"]), dv(t["w_k"]), dv(t["w_v"]), dv(t["w_o"]), dv(t["b_q"]),
                                   dv(t["b_k"]), dv(t["b_v"]), dv(t["b_o"]), h=h, ln_gain=dv(g), ln_bias=dv(bb),
                                   ln_kind=kind, ln_eps=eps, memory=dv(mem), valid_lens=vl, causal=causal,
                                   out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.mha_sublayer(x, t["w_q"], t["w_k"], t["w_v"], t["w_o"], t["b_q"], t["b_k"], t["b_v"], t["b_o"], h=h,
                              ln_gain=g, ln_bias=bb, ln_kind=kind, ln_eps=eps, memory=mem, valid_lens=vl,
                              causal=causal)
    assert_bf16(to_host(out), ref, f"sweep sublayer case {c}: B{B} Lq{Lq} Lk{Lk} D{D} causal{int(causal)} "
                                   f"lengths {lens} kind{kind}")


F32_CASES = _cases(10, 1234)


@pytest.mark.parametrize("c,B,Lq,Lk,causal,lens", F32_CASES)
def test_sweep_fp32(c, B, Lq, Lk, causal, lens):
    """The fp32 entry points on odd shapes against the fp32 bar: the
    attention core and, on even cases, the multi-head layer."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    h = 1 + c % 3
    vl = None if lens is None else np.array(lens, dtype=np.int32)
    inp = workloads.make_sdpa_inputs(B, h, Lq, Lk, 64, "f32", seed=6600 + c)
    q, k, v = (inp.tensors[n] for n in ("q", "k", "v"))
    o = mha.sdpa_forward(to_device(q, torch.float32), to_device(k, torch.float32), to_device(v, torch.float32),
                         valid_lens=vl, causal=causal)
    torch.cuda.synchronize()
    what = f"sweep fp32 case {c}: B{B} h{h} Lq{Lq} Lk{Lk} causal{int(causal)} lengths {lens}"
    assert_fp32(to_host(o), oracle.sdpa(q, k, v, valid_lens=vl, causal=causal), what + " sdpa")
    if c % 2:
        return
    D = 64 * h
    self_attn = causal
    Lk2 = Lq if self_attn else Lk
    lens2 = None if lens is None else [min(x, Lk2 + 3) for x in lens]
    vl2 = None if lens2 is None else np.array(lens2, dtype=np.int32)
    mi = workloads.make_mha_inputs(B, Lq, Lk2, D, h, "f32", seed=6700 + c, causal=causal, self_attn=self_attn,
                                   bias=True)
    t = {n: (None if a is None else to_device(a, torch.float32)) for n, a in mi.tensors.items()}
    if self_attn:
        t["x_kv"] = t["x_q"]
    out = mha.mha_forward(t["x_q"], t["x_kv"], t["w_q"], t["w_k"], t["w_v"], t["w_o"], t["b_q"], t["b_k"], t["b_v"],
                          t["b_o"], h=h, valid_lens=vl2, causal=causal)
    torch.cuda.synchronize()
    r = mi.tensors
    ref = oracle.mha(r["x_q"], r["x_kv"], r["w_q"], r["w_k"], r["w_v"], r["w_o"], r["b_q"], r["b_k"], r["b_v"], r["b_o"],
                     h=h, valid_lens=vl2, causal=causal)
    assert_fp32(to_host(out), ref, what + f" mha D{D}")
