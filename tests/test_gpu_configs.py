"""The five workloads at their full sizes, in the launch configuration the
benchmark times: the GPU computes everything; the oracle checks sampled
batches and query rows (tile edges, first/last rows, random rows), which it
computes one by one."""
import numpy as np
import pytest

import oracle
import workloads
from parity import assert_bf16, assert_fp32, errors, sample_rows, to_device, to_host
from test_gpu_mha import run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def test_mha_f32_tiny_full():
    inp = workloads.make_inputs(workloads.BY_NAME["mha_f32_tiny"])
    g = run_gpu(inp)
    e = assert_fp32(g, run_oracle(inp, bf16_stages=False), "mha_f32_tiny")
    print("mha_f32_tiny", e)


@pytest.mark.parametrize("name,n_batches,n_rows", [
    ("encoder_self", 8, 40),
    ("decoder_causal", 4, 48),
    ("enc_dec_source", 3, 40),
])
def test_mha_bf16_full(name, n_batches, n_rows):
    w = workloads.BY_NAME[name]
    inp = workloads.make_inputs(w)
    g = run_gpu(inp)
    rng = np.random.Generator(np.random.PCG64(99))
    vl = inp.valid_lens
    # the batches with the shortest and longest valid length, plus random ones
    pick = [int(np.argmin(vl)), int(np.argmax(vl))]
    for x in rng.permutation(w.B):
        if len(pick) >= n_batches:
            break
        if int(x) not in pick:
            pick.append(int(x))
    batches = np.array(sorted(set(pick)))
    rows = sample_rows(w.Lq, n_rows, rng)
    got = g[batches][:, rows]
    e = assert_bf16(got, run_oracle(inp, bf16_stages=False, batches=batches, rows=rows), name)
    stages = errors(got, run_oracle(inp, bf16_stages=True, batches=batches, rows=rows))
    print(name, "vs fp64 oracle", e, "vs bf16-storage oracle", stages)


def test_sdpa_long_causal_full():
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    w = workloads.BY_NAME["sdpa_long_causal"]
    inp = workloads.make_inputs(w)
    q, k, v = (inp.tensors[n] for n in ("q", "k", "v"))
    o = mha.sdpa_forward(to_device(q, torch.bfloat16), to_device(k, torch.bfloat16),
                         to_device(v, torch.bfloat16), causal=True)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(5))
    rows = sample_rows(w.Lq, 24, rng, tile=512)
    ref = oracle.sdpa(q, k, v, causal=True, rows=rows)
    e = assert_bf16(to_host(o[:, :, rows]), ref, "sdpa_long_causal")
    print("sdpa_long_causal", e)
