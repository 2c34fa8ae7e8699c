"""GPU parity of sdpa_decode (one incremental-decoding step through the C
ABI) against the fp64 oracle.  The step is attention with one query row and
the cache length as key-padding length, so the oracle is oracle.sdpa with
Lq = 1 and valid_lens = lens.  The kernel computes in fp32 from the bf16
inputs, so fp32 outputs are held to the fp32 bar and bf16 outputs to the bf16
bar."""
import numpy as np
import pytest

import oracle
import workloads
from parity import assert_bf16, assert_fp32, to_device, to_host

pytestmark = pytest.mark.gpu

CASES = [
    # B, h, L (cache capacity), lens
    (1, 1, 1, [1]),
    (2, 3, 5, [5, 2]),
    (2, 2, 256, [256, 255]),
    (3, 2, 257, [257, 1, 0]),          # 0: fully masked row -> uniform over all L positions
    (2, 4, 700, [700, 513]),
    (2, 2, 300, [999, 300]),           # lens above L count as L
    (4, 8, 1024, "random"),
    # grids of at least 512 workgroups take 512-key slices: one slice written
    # in place, or several merged
    (64, 8, 512, "random0"),
    (32, 16, 1000, "random0"),
    (128, 4, 200, "random0"),
]


def _lens(mode, B, L, rng):
    if mode in ("random", "random0"):
        ln = rng.integers(1, L, size=B, endpoint=True).astype(np.int32)
        if mode == "random0":
            ln[:3] = [0, L, 1]       # a fully masked row, a full cache, one position
        return ln
    return np.array(mode, dtype=np.int32)


def _run(q, k, v, lens, out_dtype, layout="bhld"):
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    B, h, L, d = k.shape
    qd = to_device(q, torch.bfloat16)
    if layout == "bhld":
        kd, vd = to_device(k, torch.bfloat16), to_device(v, torch.bfloat16)
    else:
        # caches stored [B, L, h, d] (a linear layer's output per position), viewed [B, h, L, d]
        kd = to_device(np.ascontiguousarray(k.transpose(0, 2, 1, 3)), torch.bfloat16).transpose(1, 2)
        vd = to_device(np.ascontiguousarray(v.transpose(0, 2, 1, 3)), torch.bfloat16).transpose(1, 2)
    o = mha.sdpa_decode(qd, kd, vd, lens, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return to_host(o)


@pytest.mark.parametrize("B,h,L,lens", CASES)
@pytest.mark.parametrize("out_f32", [True, False])
def test_decode_vs_oracle(B, h, L, lens, out_f32):
    import torch
    rng = np.random.Generator(np.random.PCG64(L * 7 + B))
    inp = workloads.make_sdpa_inputs(B, h, 1, L, 64, "bf16", seed=L + h)
    q, k, v = (inp.tensors[n] for n in ("q", "k", "v"))
    ln = _lens(lens, B, L, rng)
    g = _run(q[:, :, 0, :], k, v, ln, torch.float32 if out_f32 else torch.bfloat16)
    ref = oracle.sdpa(q, k, v, valid_lens=ln)[:, :, 0, :]
    if out_f32:
        assert_fp32(g, ref, f"decode B{B} h{h} L{L}")
    else:
        assert_bf16(g, ref, f"decode B{B} h{h} L{L}")


def test_decode_strided_cache_and_sharp_rows():
    """Caches in the [B, L, h, d] layout, queries with large logits."""
    import torch
    B, h, L = 2, 4, 600
    inp = workloads.make_sdpa_inputs(B, h, 1, L, 64, "bf16", seed=5)
    q = workloads.round_to_bf16(inp.tensors["q"] * 6.0)
    k, v = inp.tensors["k"], inp.tensors["v"]
    ln = np.array([600, 333], dtype=np.int32)
    g = _run(q[:, :, 0, :], k, v, ln, torch.float32, layout="blhd")
    ref = oracle.sdpa(q, k, v, valid_lens=ln)[:, :, 0, :]
    assert_fp32(g, ref, "decode strided sharp")


def test_decode_step_workload_full_size():
    """The decode workload at full size: every (batch, head) output."""
    import torch
    w = workloads.BY_NAME["decode_step"]
    inp = workloads.make_inputs(w)
    q, k, v = (inp.tensors[n] for n in ("q", "k", "v"))
    g = _run(q[:, :, 0, :], k, v, inp.valid_lens, torch.bfloat16)
    ref = oracle.sdpa(q, k, v, valid_lens=inp.valid_lens)[:, :, 0, :]
    print("decode_step", assert_bf16(g, ref, "decode_step full"))
