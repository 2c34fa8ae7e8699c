"""Seeded synthetic inputs for multi-head scaled dot-product attention.

Shared by the tests, the benchmark and the smoke check; feeds both the HIP
library and the fp64 oracle.  It holds none of the attention arithmetic: only
the workload table, the random draws, the sinusoidal position signal that one
workload adds to its inputs, and rounding of inputs to bfloat16.

Workloads (shapes from the pages' hyper-parameters: d_model = 512, h = 8,
d_k = d_v = d_model / h = 64, "Transformer" study notes, multi-head attention
parameter list):

  mha_f32_tiny     MHA, fp32: B=2, L=10, d_model=512, h=8; X ~ N(0,1);
                   Xavier-uniform weights, zero bias; valid_lens ~ U{3..10}
  encoder_self     MHA, bf16: B=32, L=128, d_model=512, h=8;
                   X = N(0,1) * sqrt(d_model) + sinusoidal position encoding;
                   valid_lens ~ U{64..128}
  decoder_causal   MHA, bf16: B=64, L=512, d_model=512, h=8; X ~ N(0,1);
                   causal AND valid_lens ~ U{256..512}
  enc_dec_source   MHA, bf16: B=16, Lq=256, Lk=384, d_model=1024, h=16;
                   queries and memory ~ N(0,1); valid_lens ~ U{192..384}
  sdpa_long_causal SDPA only, bf16: B=4, h=16, L=4096, d_k=64;
                   Q, K, V ~ N(0,1); causal

Draw order for seed s (numpy PCG64(s)): valid_lens, then X (or X_q then
memory, or Q then K then V), then W_Q, W_K, W_V, W_O, then (only when asked)
biases.  Values are drawn in float64, cast to float32 and, for bf16 workloads,
rounded to the nearest bfloat16 (ties to even).
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "mha", "sdpa" or "decode" (sdpa with one query against a cache)
    dtype: str                # "f32" or "bf16"
    B: int
    Lq: int
    Lk: int
    h: int
    d_k: int
    causal: bool
    vl_range: Optional[Tuple[int, int]]   # inclusive [lo, hi] or None
    x_kind: str = "normal"    # "normal" or "embed_pe"
    self_attn: bool = True
    seed: int = 1
    description: str = ""

    @property
    def d_model(self) -> int:
        return self.h * self.d_k

    def attention_flops(self) -> int:
        """Dense-equivalent attention flops 4*B*h*Lq*Lk*d_k."""
        return 4 * self.B * self.h * self.Lq * self.Lk * self.d_k


WORKLOADS = [
    Workload("mha_f32_tiny", "mha", "f32", 2, 10, 10, 8, 64, False, (3, 10), seed=1,
             description="MHA forward fp32, B=2 L=10 d_model=512 h=8, padding valid_lens U{3..10}"),
    Workload("encoder_self", "mha", "bf16", 32, 128, 128, 8, 64, False, (64, 128),
             x_kind="embed_pe", seed=2,
             description="encoder self-attention MHA forward bf16, B=32 L=128 d_model=512 h=8, "
                         "padding valid_lens U{64..128}"),
    Workload("decoder_causal", "mha", "bf16", 64, 512, 512, 8, 64, True, (256, 512), seed=3,
             description="decoder masked self-attention MHA forward bf16, B=64 L=512 d_model=512 "
                         "h=8, causal and padding valid_lens U{256..512}"),
    Workload("enc_dec_source", "mha", "bf16", 16, 256, 384, 16, 64, False, (192, 384),
             self_attn=False, seed=4,
             description="encoder-decoder source attention MHA forward bf16, B=16 Lq=256 Lk=384 "
                         "d_model=1024 h=16, source valid_lens U{192..384}"),
    Workload("sdpa_long_causal", "sdpa", "bf16", 4, 4096, 4096, 16, 64, True, None, seed=5,
             description="long causal SDPA core bf16, B=4 h=16 L=4096 d_k=64"),
    # One incremental-decoding step of the decoder workload's shape: a single
    # query per (batch, head) against a 512-position cache holding U{256..512}
    # valid keys.
    Workload("decode_step", "decode", "bf16", 64, 1, 512, 8, 64, False, (256, 512), seed=6,
             description="decoding step bf16, B=64 h=8 d_k=64, one query against a K/V cache of "
                         "512 positions with U{256..512} valid"),
    # The backward pass over a decoder-sized causal attention (q, k, v and the
    # output gradient ~ N(0,1)).
    Workload("backward_causal", "sdpa", "bf16", 4, 1024, 1024, 8, 64, True, None, seed=7,
             description="attention backward bf16 in / fp32 gradients, B=4 h=8 L=1024 d_k=64, causal"),
    # The inspection path: weights of a padded self-attention, B=4 h=8 L=512
    # with per-sequence lengths U{256..512}.
    Workload("inspect_weights", "sdpa", "bf16", 4, 512, 512, 8, 64, False, (256, 512), seed=8,
             description="attention with weights export bf16, B=4 h=8 L=512 d_k=64, valid_lens U{256..512}"),
]
BY_NAME = {w.name: w for w in WORKLOADS}


# ----------------------------------------------------------------------------
# bfloat16 rounding of inputs (float32 -> nearest bf16, ties to even)
# ----------------------------------------------------------------------------
def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of the nearest bfloat16 to each float32 element."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x32: np.ndarray) -> np.ndarray:
    """float32 array holding the nearest-bf16 values."""
    return bf16_bits_to_f32(bf16_bits(x32))


# ----------------------------------------------------------------------------
# random draws
# ----------------------------------------------------------------------------
def xavier_uniform(rng: np.random.Generator, fan_out: int, fan_in: int) -> np.ndarray:
    a = math.sqrt(6.0 / (fan_in + fan_out))
    return rng.uniform(-a, a, size=(fan_out, fan_in))


def sinusoidal_positions(L: int, D: int) -> np.ndarray:
    """Position signal added to embeddings: sin at even feature 2i, cos at odd
    feature 2i+1, both of pos / 10000^(2i/D) ("Transformer" study notes,
    position-encoder section; the page-5 copy of the formula is garbled)."""
    pos = np.arange(L, dtype=np.float64)[:, None]
    two_i = np.arange(0, D, 2, dtype=np.float64)[None, :]
    ang = pos / np.power(10000.0, two_i / D)
    pe = np.zeros((L, D), dtype=np.float64)
    pe[:, 0::2] = np.sin(ang)
    pe[:, 1::2] = np.cos(ang)
    return pe


def draw_valid_lens(rng, B, vl_range):
    if vl_range is None:
        return None
    lo, hi = vl_range
    return rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)


def _finish(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = np.asarray(x64, dtype=np.float32)
    return round_to_bf16(x32) if dtype == "bf16" else x32


@dataclass
class Inputs:
    """Host copies of one workload's inputs.  Float arrays are float32 holding
    exactly the values the device receives (bf16-exact for bf16 workloads)."""
    workload: Workload
    valid_lens: Optional[np.ndarray]
    tensors: dict = field(default_factory=dict)

    def digest(self) -> dict:
        out = {}
        for k, v in self.tensors.items():
            if v is not None:
                out[k] = hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()[:16]
        if self.valid_lens is not None:
            out["valid_lens"] = hashlib.sha256(self.valid_lens.tobytes()).hexdigest()[:16]
        return out


def make_mha_inputs(B, Lq, Lk, D, h, dtype="bf16", seed=0, vl_range=None, causal=False,
                    x_kind="normal", self_attn=True, bias=False, name="custom") -> Inputs:
    w = Workload(name, "mha", dtype, B, Lq, Lk, h, D // h, causal, vl_range, x_kind,
                 self_attn, seed)
    return make_inputs(w, bias=bias)


def make_sdpa_inputs(B, h, Lq, Lk, d, dtype="bf16", seed=0, vl_range=None, causal=False,
                     name="custom") -> Inputs:
    w = Workload(name, "sdpa", dtype, B, Lq, Lk, h, d, causal, vl_range, seed=seed)
    return make_inputs(w)


def make_inputs(w: Workload, bias: bool = False) -> Inputs:
    rng = np.random.Generator(np.random.PCG64(w.seed))
    vl = draw_valid_lens(rng, w.B, w.vl_range)
    t = {}
    if w.kind in ("sdpa", "decode"):
        for name in ("q", "k", "v"):
            L = w.Lq if name == "q" else w.Lk
            t[name] = _finish(rng.standard_normal((w.B, w.h, L, w.d_k)), w.dtype)
        return Inputs(w, vl, t)
    D = w.d_model
    if w.x_kind == "embed_pe":
        x = rng.standard_normal((w.B, w.Lq, D)) * math.sqrt(D) + sinusoidal_positions(w.Lq, D)[None]
    else:
        x = rng.standard_normal((w.B, w.Lq, D))
    t["x_q"] = _finish(x, w.dtype)
    if w.self_attn:
        assert w.Lq == w.Lk
        t["x_kv"] = t["x_q"]
    else:
        t["x_kv"] = _finish(rng.standard_normal((w.B, w.Lk, D)), w.dtype)
    for name in ("w_q", "w_k", "w_v", "w_o"):
        t[name] = _finish(xavier_uniform(rng, D, D), w.dtype)
    for name in ("b_q", "b_k", "b_v", "b_o"):
        if bias:
            a = 1.0 / math.sqrt(D)
            t[name] = _finish(rng.uniform(-a, a, size=(D,)), w.dtype)
        else:
            t[name] = None
    return Inputs(w, vl, t)
