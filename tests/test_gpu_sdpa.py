"""GPU parity of sdpa_forward (through the C ABI) against the fp64 oracle,
element by element, at sizes the oracle finishes in seconds that span several
query/key tiles and ragged tails, plus the degenerate cases of the masks."""
import numpy as np
import pytest

import oracle
import workloads
from parity import assert_bf16, assert_fp32, to_device, to_host

pytestmark = pytest.mark.gpu


def _vl(mode, B, Lk, rng):
    if mode is None:
        return None
    if mode == "random":
        return rng.integers(1, Lk, size=B, endpoint=True).astype(np.int32)
    return np.array(mode, dtype=np.int32)


BF16_CASES = [
    # B, h, Lq, Lk, causal, valid_lens
    (1, 1, 1, 1, False, None),
    (1, 1, 4, 4, True, None),
    (1, 2, 3, 5, False, [2]),
    (2, 3, 130, 130, True, "random"),
    (2, 2, 77, 200, False, "random"),
    (3, 2, 257, 257, True, [0, 1, 257]),
    (2, 2, 128, 64, False, [0, 64]),
    (1, 4, 300, 1000, False, [999]),
    (2, 2, 384, 384, True, None),
    (1, 1, 129, 700, False, [640]),
]


@pytest.mark.parametrize("B,h,Lq,Lk,causal,vl", BF16_CASES)
@pytest.mark.parametrize("out_f32", [False, True])
def test_sdpa_bf16_vs_oracle(B, h, Lq, Lk, causal, vl, out_f32):
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    rng = np.random.Generator(np.random.PCG64(B * 1000 + Lq * 7 + Lk))
    inp = workloads.make_sdpa_inputs(B, h, Lq, Lk, 64, "bf16", seed=Lq + Lk, causal=causal)
    q, k, v = (inp.tensors[n] for n in ("q", "k", "v"))
    vls = _vl(vl, B, Lk, rng)
    o = mha.sdpa_forward(to_device(q, torch.bfloat16), to_device(k, torch.bfloat16),
                         to_device(v, torch.bfloat16), valid_lens=vls, causal=causal,
                         out_dtype=torch.float32 if out_f32 else torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.sdpa(q, k, v, valid_lens=vls, causal=causal)
    assert_bf16(to_host(o), ref, f"sdpa bf16 B{B} h{h} Lq{Lq} Lk{Lk} causal{causal} vl{vls}")


def test_sdpa_bf16_sharp_softmax_and_strided_layout():
    """Large logits (nearly one-hot rows) through a [B, L, h, d] strided view,
    the layout the projections produce."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    B, h, L = 2, 4, 200
    inp = workloads.make_sdpa_inputs(B, h, L, L, 64, "bf16", seed=77)
    q = workloads.round_to_bf16(inp.tensors["q"] * 6.0)
    k, v = inp.tensors["k"], inp.tensors["v"]
    vls = np.array([150, 200], dtype=np.int32)
    # device tensors stored [B, L, h, d]; pass [B, h, L, d] views
    dev = lambda x: to_device(np.ascontiguousarray(x.transpose(0, 2, 1, 3)), torch.bfloat16).transpose(1, 2)
    o = mha.sdpa_forward(dev(q), dev(k), dev(v), valid_lens=vls, causal=True)
    torch.cuda.synchronize()
    ref = oracle.sdpa(q, k, v, valid_lens=vls, causal=True)
    assert_bf16(to_host(o), ref, "sharp softmax, strided")


@pytest.mark.parametrize("causal", [False, True])
def test_sdpa_bf16_later_tile_far_above_the_first(causal):
    """Key 200 scores about 350 log2 units above every key of the first tile
    (q in [1, ~4], k_200 = 16): its weight overflows fp32 under the first
    tile's offset, and the kernel must move the offset and recompute rather
    than let infinities (or NaNs from them) into the output.  Rows that see
    key 200 put almost all their weight on it."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    rng = np.random.Generator(np.random.PCG64(2024))
    B, h, L = 1, 2, 300
    q = workloads.round_to_bf16((1.0 + np.abs(rng.standard_normal((B, h, L, 64)))).astype(np.float32))
    k = workloads.round_to_bf16(rng.standard_normal((B, h, L, 64)).astype(np.float32))
    v = workloads.round_to_bf16(rng.standard_normal((B, h, L, 64)).astype(np.float32))
    k[:, :, 200, :] = 16.0
    o = mha.sdpa_forward(*(to_device(x, torch.bfloat16) for x in (q, k, v)), causal=causal,
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.sdpa(q, k, v, causal=causal)
    assert_bf16(to_host(o), ref, f"score jump above the first tile, causal={causal}")


@pytest.mark.parametrize("out_f32,row", [(False, 64), (False, 72), (False, 136), (True, 64), (True, 68)])
def test_sdpa_bf16_output_views(out_f32, row):
    """The output written through a view whose rows are padded (row stride
    `row` elements): the values match the oracle and nothing outside the view
    is touched."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    B, h, L = 2, 2, 300
    inp = workloads.make_sdpa_inputs(B, h, L, L, 64, "bf16", seed=row, causal=True)
    q, k, v = (inp.tensors[n] for n in ("q", "k", "v"))
    vls = np.array([300, 100], dtype=np.int32)
    dt = torch.float32 if out_f32 else torch.bfloat16
    n = B * h * L * row
    buf = torch.full((n,), float("nan"), dtype=dt, device="cuda")
    out = buf.view(B, h, L, row)[..., :64]
    mha.sdpa_forward(to_device(q, torch.bfloat16), to_device(k, torch.bfloat16), to_device(v, torch.bfloat16),
                     valid_lens=vls, causal=True, out=out)
    torch.cuda.synchronize()
    ref = oracle.sdpa(q, k, v, valid_lens=vls, causal=True)
    assert_bf16(to_host(out), ref, f"output view row {row} f32 {out_f32}")
    assert torch.isnan(buf.view(B, h, L, row)[..., 64:]).all(), "a store landed outside the output view"


@pytest.mark.parametrize("out_f32,row,offset", [(False, 68, 0), (False, 64, 1), (True, 66, 0)])
def test_sdpa_rejects_misaligned_output(out_f32, row, offset):
    """Output rows that would not start 16-byte aligned are refused before
    anything is enqueued, and the buffer is left as it was."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    from transformer_head_scaled_sdpa_amd._lib import MhaError
    B, h, L = 1, 2, 40
    x = torch.zeros((B, h, L, 64), dtype=torch.bfloat16, device="cuda")
    dt = torch.float32 if out_f32 else torch.bfloat16
    n = B * h * L * row
    buf = torch.full((n + 8,), float("nan"), dtype=dt, device="cuda")
    out = buf[offset:offset + n].view(B, h, L, row)[..., :64]
    with pytest.raises(MhaError, match="MHA_EINVAL"):
        mha.sdpa_forward(x, x, x, causal=True, out=out)
    torch.cuda.synchronize()
    assert torch.isnan(buf).all()


F32_CASES = [
    (2, 8, 10, 10, False, "random"),
    (1, 1, 1, 1, False, None),
    (2, 3, 70, 70, True, "random"),
    (1, 2, 65, 130, False, [0]),
    (2, 2, 100, 33, False, [33, 5]),
]


@pytest.mark.parametrize("B,h,Lq,Lk,causal,vl", F32_CASES)
def test_sdpa_f32_vs_oracle(B, h, Lq, Lk, causal, vl):
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    rng = np.random.Generator(np.random.PCG64(Lq * 31 + Lk))
    inp = workloads.make_sdpa_inputs(B, h, Lq, Lk, 64, "f32", seed=Lq * 3 + Lk, causal=causal)
    q, k, v = (inp.tensors[n] for n in ("q", "k", "v"))
    vls = _vl(vl, B, Lk, rng)
    o = mha.sdpa_forward(to_device(q, torch.float32), to_device(k, torch.float32),
                         to_device(v, torch.float32), valid_lens=vls, causal=causal)
    torch.cuda.synchronize()
    ref = oracle.sdpa(q, k, v, valid_lens=vls, causal=causal)
    assert_fp32(to_host(o), ref, f"sdpa f32 B{B} h{h} Lq{Lq} Lk{Lk}")


def test_sdpa_fully_masked_rows_are_uniform():
    """valid_len 0: the GPU must give the mean of all Lk values (uniform
    weights), exactly as the -1e9 replacement does."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    B, h, L = 2, 2, 150
    inp = workloads.make_sdpa_inputs(B, h, L, L, 64, "bf16", seed=5)
    q, k, v = (inp.tensors[n] for n in ("q", "k", "v"))
    vls = np.array([0, 0], dtype=np.int32)
    for causal in (False, True):
        o = to_host(mha.sdpa_forward(to_device(q, torch.bfloat16), to_device(k, torch.bfloat16),
                                     to_device(v, torch.bfloat16), valid_lens=vls, causal=causal,
                                     out_dtype=torch.float32))
        mean = v.astype(np.float64).mean(axis=2, keepdims=True)
        assert_bf16(o, np.broadcast_to(mean, o.shape), "fully masked rows")


# The log-sum-exp the forward keeps for the backward.  Bar: the bf16 kernel
# sums the bf16-rounded weights (relative error at most 2^-9 each, so at most
# 2^-9 in the sum and in its log) and scores the bf16 inputs in fp32; the
# fp32 kernel is fp32 throughout.  So |lse - ref| <= 2^-9 + 1e-5 max(1, |ref|)
# (bf16 inputs) or 1e-5 max(1, |ref|) (fp32).  A row with every key masked
# weighs its keys equally; the oracle's fill makes that fill + log(Lk), the
# library reports log(Lk) (scores all 0): the test adds the fill back.
LSE_CASES = [
    # B, h, Lq, Lk, causal, valid_lens, dtype
    (2, 3, 200, 200, True, None, "bf16"),
    (2, 2, 77, 300, False, [0, 150], "bf16"),
    (1, 4, 513, 513, True, None, "bf16"),
    (3, 1, 64, 1, False, None, "bf16"),
    (2, 2, 70, 90, False, [5, 90], "f32"),
    (2, 3, 64, 64, True, [0, 64], "f32"),
]


@pytest.mark.parametrize("B,h,Lq,Lk,causal,vl,dt", LSE_CASES)
def test_sdpa_forward_lse_vs_oracle(B, h, Lq, Lk, causal, vl, dt):
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    inp = workloads.make_sdpa_inputs(B, h, Lq, Lk, 64, dt, seed=B * 131 + Lq + Lk)
    q, k, v = (inp.tensors[n] for n in ("q", "k", "v"))
    vls = None if vl is None else np.array(vl, np.int32)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    tq, tk, tv = (to_device(x, tdt) for x in (q, k, v))
    o, lse = mha.sdpa_forward(tq, tk, tv, valid_lens=vls, causal=causal, return_lse=True)
    o_plain = mha.sdpa_forward(tq, tk, tv, valid_lens=vls, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain), "the output must not change when the statistic is kept"
    ref = oracle.sdpa_lse(q, k, valid_lens=vls, causal=causal)
    if vls is not None:
        ref[vls <= 0] += 1e9                               # the fill, added back
    got = to_host(lse)
    bar = (2.0 ** -9 if dt == "bf16" else 0.0) + 1e-5 * np.maximum(1.0, np.abs(ref))
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)) and np.all(err <= bar), f"lse error {err.max()} (bar {bar.min()})"
    print("max lse error", err.max())
