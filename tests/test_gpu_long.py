"""Long key ranges at the large end of what the kernels take: tens of
thousands of keys per (batch, head) through sdpa_forward, sdpa_decode and
sdpa_backward, against the fp64 oracle (every output; the oracle finishes
these in seconds because the query side is short)."""
import numpy as np
import pytest

import oracle
import workloads
from parity import assert_bf16, assert_fp32, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,h,Lq,Lk,lens", [
    (1, 2, 100, 20000, [17003]),     # ~270 key tiles, a ragged valid length
    (2, 1, 64, 12345, None),         # Lk not a multiple of the tile
])
def test_sdpa_forward_long_keys(B, h, Lq, Lk, lens):
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    inp = workloads.make_sdpa_inputs(B, h, Lq, Lk, 64, "bf16", seed=Lk)
    q, k, v = (inp.tensors[n] for n in ("q", "k", "v"))
    vl = None if lens is None else np.array(lens * B, dtype=np.int32)[:B]
    o = mha.sdpa_forward(to_device(q, torch.bfloat16), to_device(k, torch.bfloat16), to_device(v, torch.bfloat16),
                         valid_lens=vl, out_dtype=torch.float32)
    torch.cuda.synchronize()
    print(assert_bf16(to_host(o), oracle.sdpa(q, k, v, valid_lens=vl), f"sdpa Lk={Lk}"))


@pytest.mark.parametrize("B,h,L,lens", [
    (1, 8, 32768, [32768]),          # 64 slices of 512 keys, merged
    (2, 4, 20000, [19999, 7]),       # slices past a short cache are empty
])
def test_decode_long_cache(B, h, L, lens):
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    inp = workloads.make_sdpa_inputs(B, h, 1, L, 64, "bf16", seed=L + 1)
    q, k, v = (inp.tensors[n] for n in ("q", "k", "v"))
    ln = np.array(lens, dtype=np.int32)
    o = mha.sdpa_decode(to_device(q[:, :, 0, :], torch.bfloat16), to_device(k, torch.bfloat16),
                        to_device(v, torch.bfloat16), ln, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.sdpa(q, k, v, valid_lens=ln)[:, :, 0, :]
    print(assert_fp32(to_host(o), ref, f"decode L={L}"))


def test_backward_long_keys():
    """64 queries against 8000 keys (bf16 MFMA path), lengths per sequence."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    rng = np.random.Generator(np.random.PCG64(8000))
    B, h, Lq, Lk = 2, 1, 64, 8000
    q = workloads._finish(rng.standard_normal((B, h, Lq, 64)), "bf16")
    k = workloads._finish(rng.standard_normal((B, h, Lk, 64)), "bf16")
    v = workloads._finish(rng.standard_normal((B, h, Lk, 64)), "bf16")
    g = workloads._finish(rng.standard_normal((B, h, Lq, 64)), "bf16")
    vl = np.array([8000, 5123], dtype=np.int32)
    tq, tk, tv, tg = (to_device(x, torch.bfloat16) for x in (q, k, v, g))
    o = mha.sdpa_forward(tq, tk, tv, valid_lens=vl)
    gq, gk, gv = mha.sdpa_backward(tq, tk, tv, o, tg, valid_lens=vl, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.sdpa_backward(q, k, v, g, valid_lens=vl)
    for name, got, ref in (("dq", gq, rq), ("dk", gk, rk), ("dv", gv, rv)):
        print(name, assert_bf16(to_host(got), ref, f"{name} Lk={Lk}"))
