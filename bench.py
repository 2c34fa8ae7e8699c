"""Benchmark: scaled dot-product attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

The headline workload is the long causal attention core (B=4 h=16 L=4096
d_k=64, bf16, Q/K/V given): a step is one sdpa_forward over it with inputs
resident in HBM.  `value` is the algorithmic attention throughput (4*d_k
flops per mask-allowed pair / step time); the literal 4*B*h*Lq*Lk*d_k rate is
reported beside it as the dense equivalent.  Prints ONE JSON line with the
dominant kernel's roofline (its duration from HIP events on the launch
stream), the other four configurations (the MHA forward steps, each with its
own dominant kernel's roofline), the NEXT-row paths, and the fp64 CPU oracle
timed on the host's cores on a bounded sample of the headline workload.
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work (what the method itself must do: masked pairs skipped,
# keys beyond the valid length not read)
# ---------------------------------------------------------------------------
def allowed_pairs(w, valid_lens):
    """Number of (batch, head, query, key) pairs the masks allow."""
    Lq, Lk = w.Lq, w.Lk
    vl = np.full(w.B, Lk) if valid_lens is None else np.asarray(valid_lens, dtype=np.int64)
    total = 0
    i = np.arange(Lq)
    for v in vl:
        if v <= 0:
            total += Lq * Lk          # fully masked rows weight every key
            continue
        v = min(int(v), Lk)
        total += int(np.minimum(i + 1, v).sum()) if w.causal else Lq * v
    return total * w.h


def sdpa_alg(w, valid_lens, in_bytes, out_bytes):
    """Algorithmic flops and HBM bytes of one fused attention launch."""
    pairs = allowed_pairs(w, valid_lens)
    flops = 4 * w.d_k * pairs
    vl = np.full(w.B, w.Lk) if valid_lens is None else np.asarray(valid_lens, dtype=np.int64)
    keys = sum(w.Lk if v <= 0 else min(int(v), w.Lk) for v in vl)   # K/V rows that carry weight
    byts = w.h * w.d_k * (w.B * w.Lq * (in_bytes + out_bytes) + 2 * keys * in_bytes)
    return flops, byts


def gemm_alg(M, N, K, nprob, in_bytes, out_bytes):
    return 2 * M * N * K * nprob, nprob * ((M * K + N * K + N) * in_bytes + M * N * out_bytes)


def fused_alg(w, valid_lens, in_bytes):
    """Algorithmic flops and HBM bytes of the kernel that projects Q, K, V and
    attends (merged-head output in the input dtype).  K and V are needed only
    for keys below each batch's valid length; every query row is projected."""
    D = w.d_model
    vl = np.full(w.B, w.Lk) if valid_lens is None else np.asarray(valid_lens, dtype=np.int64)
    kv_rows = sum(w.Lk if v <= 0 else min(int(v), w.Lk) for v in vl)
    f_attn, _ = sdpa_alg(w, valid_lens, in_bytes, in_bytes)
    flops = 2 * w.B * w.Lq * D * D + 2 * 2 * kv_rows * D * D + f_attn
    x_bytes = w.B * w.Lq * D * in_bytes + (0 if w.self_attn else w.B * w.Lk * D * in_bytes)
    byts = x_bytes + 3 * (D * D + D) * in_bytes + w.B * w.Lq * D * in_bytes
    return flops, byts


def roofline(flops, byts, ms, mfma_peak):
    t_mfma = flops / (mfma_peak * 1e12)
    t_hbm = byts / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm:
        ach = flops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": round(ach / mfma_peak, 4)}
    ach = byts / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4)}


# ---------------------------------------------------------------------------
# GPU side
# ---------------------------------------------------------------------------
class PreparedMha:
    """mha_forward with its arguments marshalled once (device pointers of
    preallocated tensors); each call only passes torch's current stream."""

    def __init__(self, inp):
        import torch
        import transformer_head_scaled_sdpa_amd as mha
        from transformer_head_scaled_sdpa_amd import _lib
        w = inp.workload
        self.w = w
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        dev = torch.device("cuda:0")
        self.t = {n: (None if a is None else torch.from_numpy(a).to(dev).to(dt)) for n, a in inp.tensors.items()}
        if w.self_attn:
            self.t["x_kv"] = self.t["x_q"]
        self.out = torch.empty((w.B, w.Lq, w.d_model), dtype=torch.float32, device=dev)
        need = mha.workspace_bytes(dt, w.B, w.Lq, w.Lk, w.d_model, w.h)
        self.ws = torch.empty(need, dtype=torch.uint8, device=dev)
        self.vl = None if inp.valid_lens is None else torch.from_numpy(inp.valid_lens).to(dev)
        self.lib = _lib.load()
        p = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())
        t = self.t
        self.in_dt = _lib.MHA_BF16 if w.dtype == "bf16" else _lib.MHA_F32
        self.args = [self.in_dt, _lib.MHA_F32, p(t["x_q"]), p(t["x_kv"]), p(t["w_q"]), p(t["b_q"]),
                     p(t["w_k"]), p(t["b_k"]), p(t["w_v"]), p(t["b_v"]), p(t["w_o"]), p(t["b_o"]),
                     p(self.out), w.B, w.Lq, w.Lk, w.d_model, w.h, w.d_k, p(self.vl), int(w.causal),
                     p(self.ws), need]
        self.torch = torch

    def __call__(self):
        st = self.lib.mha_forward(*self.args, ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"mha_forward failed with status {st}")


class PreparedSdpa:
    def __init__(self, inp):
        import torch
        from transformer_head_scaled_sdpa_amd import _lib
        w = inp.workload
        self.w = w
        dev = torch.device("cuda:0")
        self.q, self.k, self.v = (torch.from_numpy(inp.tensors[n]).to(dev).to(torch.bfloat16) for n in "qkv")
        self.o = torch.empty_like(self.q)
        self.vl = None if inp.valid_lens is None else torch.from_numpy(inp.valid_lens).to(dev)
        self.lib = _lib.load()
        s = lambda x: _lib.Strides(*x.stride()[:3])
        p = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())
        self.args = [_lib.MHA_BF16, _lib.MHA_BF16, p(self.q), s(self.q), p(self.k), s(self.k), p(self.v), s(self.v),
                     p(self.o), s(self.o), w.B, w.h, w.Lq, w.Lk, w.d_k, w.d_k, p(self.vl), int(w.causal)]
        self.torch = torch

    def __call__(self):
        st = self.lib.sdpa_forward(*self.args, ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"sdpa_forward failed with status {st}")


class PreparedDecode:
    """sdpa_decode on one decoding step's query and K/V caches."""

    def __init__(self, inp):
        import torch
        from transformer_head_scaled_sdpa_amd import _lib
        w = inp.workload
        self.w = w
        dev = torch.device("cuda:0")
        self.q = torch.from_numpy(inp.tensors["q"][:, :, 0, :]).to(dev).to(torch.bfloat16)
        self.k, self.v = (torch.from_numpy(inp.tensors[n]).to(dev).to(torch.bfloat16) for n in "kv")
        self.o = torch.empty_like(self.q)
        self.lens = torch.from_numpy(inp.valid_lens).to(dev)
        self.lib = _lib.load()
        need = int(self.lib.sdpa_decode_workspace_bytes(w.B, w.h, w.Lk))
        self.ws = torch.empty(need, dtype=torch.uint8, device=dev)
        s3 = lambda x: _lib.Strides(x.stride(0), x.stride(1), 0)
        s4 = lambda x: _lib.Strides(*x.stride()[:3])
        p = lambda x: ctypes.c_void_p(x.data_ptr())
        self.args = [_lib.MHA_BF16, _lib.MHA_BF16, p(self.q), s3(self.q), p(self.k), s4(self.k), p(self.v),
                     s4(self.v), p(self.o), s3(self.o), w.B, w.h, w.Lk, w.d_k, w.d_k, p(self.lens), p(self.ws),
                     need]
        self.torch = torch

    def __call__(self):
        st = self.lib.sdpa_decode(*self.args, ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"sdpa_decode failed with status {st}")


def decode_alg(w, lens):
    """Algorithmic flops and HBM bytes of one decoding step: every valid cached
    key and value is read once, the query read and the output written."""
    n = sum(w.Lk if v <= 0 else min(int(v), w.Lk) for v in lens)
    flops = 4 * w.d_k * w.h * n
    byts = w.h * w.d_k * 2 * (2 * n + 2 * w.B)
    return flops, byts


class PreparedBackward:
    """sdpa_backward on q, k, v, the forward output and an output gradient;
    with ``use_lse`` sdpa_backward_lse, given the forward's log-sum-exp (the
    training step's path)."""

    def __init__(self, inp, use_lse=False):
        import torch
        import transformer_head_scaled_sdpa_amd as mha
        from transformer_head_scaled_sdpa_amd import _lib
        w = inp.workload
        dev = torch.device("cuda:0")
        self.t = [torch.from_numpy(inp.tensors[n]).to(dev).to(torch.bfloat16) for n in "qkv"]
        rng = np.random.Generator(np.random.PCG64(w.seed + 1000))
        self.g = torch.from_numpy(rng.standard_normal(self.t[0].shape).astype(np.float32)).to(dev).to(torch.bfloat16)
        self.vl = None if inp.valid_lens is None else torch.from_numpy(inp.valid_lens).to(dev)
        self.o, self.lse = mha.sdpa_forward(*self.t, valid_lens=self.vl, causal=w.causal, return_lse=True)
        self.use_lse = use_lse
        self.grads = [torch.empty(x.shape, dtype=torch.float32, device=dev) for x in self.t]
        self.lib = _lib.load()
        need = int(self.lib.sdpa_backward_workspace_bytes(w.B, w.h, w.Lq))
        self.ws = torch.empty(need, dtype=torch.uint8, device=dev)
        s4 = lambda x: _lib.Strides(*x.stride()[:3])
        p = lambda x: ctypes.c_void_p(x.data_ptr())
        args = []
        for x in self.t + [self.o, self.g] + self.grads:
            args += [p(x), s4(x)]
        self.args = [_lib.MHA_BF16, _lib.MHA_F32] + args + [w.B, w.h, w.Lq, w.Lk, 64, 64,
                                                             None if self.vl is None else p(self.vl), 1,
                                                             int(w.causal)]
        self.args += ([p(self.lse)] if use_lse else []) + [p(self.ws), need]
        self.fn = self.lib.sdpa_backward_lse if use_lse else self.lib.sdpa_backward
        self.torch = torch

    def __call__(self):
        st = self.fn(*self.args, ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"sdpa_backward failed with status {st}")


class PreparedMhaBackward:
    """mha_backward (bf16 inputs, fp32 gradients) on an MHA workload's inputs
    and a seeded output gradient, its arguments marshalled once."""

    def __init__(self, inp):
        import torch
        from transformer_head_scaled_sdpa_amd import _lib
        w = inp.workload
        dev = torch.device("cuda:0")
        T = lambda a: None if a is None else torch.from_numpy(a).to(dev).to(torch.bfloat16)
        self.t = {n: T(a) for n, a in inp.tensors.items()}
        if w.self_attn:
            self.t["x_kv"] = self.t["x_q"]
        rng = np.random.Generator(np.random.PCG64(w.seed + 1000))
        self.g = T(rng.standard_normal((w.B, w.Lq, w.d_model)).astype(np.float32))
        self.vl = None if inp.valid_lens is None else torch.from_numpy(inp.valid_lens).to(dev)
        D = w.d_model
        f32 = dict(dtype=torch.float32, device=dev)
        self.dx_q = torch.empty((w.B, w.Lq, D), **f32)
        self.dx_kv = None if w.self_attn else torch.empty((w.B, w.Lk, D), **f32)
        self.dw = [torch.empty((D, D), **f32) for _ in range(4)]
        self.db = [torch.empty((D,), **f32) for _ in range(4)]
        self.lib = _lib.load()
        need = int(self.lib.mha_backward_workspace_bytes(_lib.MHA_BF16, w.B, w.Lq, w.Lk, D, w.h))
        self.ws = torch.empty(need, dtype=torch.uint8, device=dev)
        p = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())
        t = self.t
        self.args = [_lib.MHA_BF16, p(t["x_q"]), p(t["x_kv"]), p(t["w_q"]), p(t["b_q"]), p(t["w_k"]), p(t["b_k"]),
                     p(t["w_v"]), p(t["b_v"]), p(t["w_o"]), p(self.g), p(self.dx_q), p(self.dx_kv)]
        for dw, db in zip(self.dw, self.db):
            self.args += [p(dw), p(db)]
        self.args += [w.B, w.Lq, w.Lk, D, w.h, w.d_k, p(self.vl), int(w.causal), p(self.ws), need]
        self.torch = torch

    def __call__(self):
        st = self.lib.mha_backward(*self.args, ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"mha_backward failed with status {st}")


class PreparedTrainingPair:
    """One training pass of the multi-head layer: mha_forward_train (bf16
    output, Q, K, V, the merged heads and the log-sum-exp kept) then
    mha_backward_saved on the kept tensors, arguments marshalled once."""

    def __init__(self, inp):
        import torch
        from transformer_head_scaled_sdpa_amd import _lib
        self.bwd = PreparedMhaBackward(inp)
        w = inp.workload
        dev = torch.device("cuda:0")
        t = self.bwd.t
        lib = self.lib = self.bwd.lib
        D = w.d_model
        self.out = torch.empty((w.B, w.Lq, D), dtype=torch.bfloat16, device=dev)
        sb = int(lib.mha_saved_bytes(_lib.MHA_BF16, w.B, w.Lq, w.Lk, D, w.h))
        self.saved = torch.empty(sb, dtype=torch.uint8, device=dev)
        need = int(lib.mha_backward_saved_workspace_bytes(_lib.MHA_BF16, w.B, w.Lq, w.Lk, D, w.h))
        self.ws = torch.empty(need, dtype=torch.uint8, device=dev)
        self.bwd.ws = None                      # the recomputing backward's workspace is not needed
        p = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())
        vl, bwd = p(self.bwd.vl), self.bwd
        self.fargs = [_lib.MHA_BF16, _lib.MHA_BF16, p(t["x_q"]), p(t["x_kv"]), p(t["w_q"]), p(t["b_q"]), p(t["w_k"]),
                      p(t["b_k"]), p(t["w_v"]), p(t["b_v"]), p(t["w_o"]), p(t["b_o"]), p(self.out),
                      w.B, w.Lq, w.Lk, D, w.h, w.d_k, vl, int(w.causal), p(self.saved), sb]
        self.bargs = [_lib.MHA_BF16, p(t["x_q"]), p(t["x_kv"]), p(t["w_q"]), p(t["w_k"]), p(t["w_v"]), p(t["w_o"]),
                      p(self.saved), sb, p(bwd.g), p(bwd.dx_q), p(bwd.dx_kv)]
        for dw, db in zip(bwd.dw, bwd.db):
            self.bargs += [p(dw), p(db)]
        self.bargs += [w.B, w.Lq, w.Lk, D, w.h, w.d_k, vl, int(w.causal), p(self.ws), need]
        self.torch = torch

    def __call__(self):
        s = ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)
        st = self.lib.mha_forward_train(*self.fargs, s)
        if st != 0:
            raise RuntimeError(f"mha_forward_train failed with status {st}")
        st = self.lib.mha_backward_saved(*self.bargs, s)
        if st != 0:
            raise RuntimeError(f"mha_backward_saved failed with status {st}")


class PreparedWeights:
    """sdpa_forward_ex returning the attention weights (inspection path)."""

    def __init__(self, inp):
        import torch
        from transformer_head_scaled_sdpa_amd import _lib
        w = inp.workload
        dev = torch.device("cuda:0")
        self.t = [torch.from_numpy(inp.tensors[n]).to(dev).to(torch.bfloat16) for n in "qkv"]
        self.o = torch.empty_like(self.t[0])
        self.p = torch.empty((w.B, w.h, w.Lq, w.Lk), dtype=torch.float32, device=dev)
        self.vl = None if inp.valid_lens is None else torch.from_numpy(inp.valid_lens).to(dev)
        self.lib = _lib.load()
        s4 = lambda x: _lib.Strides(*x.stride()[:3])
        p = lambda x: ctypes.c_void_p(x.data_ptr())
        q, k, v = self.t
        self.args = [_lib.MHA_BF16, _lib.MHA_BF16, p(q), s4(q), p(k), s4(k), p(v), s4(v), p(self.o), s4(self.o),
                     w.B, w.h, w.Lq, w.Lk, 64, 64, None if self.vl is None else p(self.vl), 1, int(w.causal),
                     p(self.p), s4(self.p)]
        self.torch = torch

    def __call__(self):
        st = self.lib.sdpa_forward_ex(*self.args, ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"sdpa_forward_ex failed with status {st}")


class PreparedSublayer:
    """mha_sublayer_forward (x + MHA(norm(x))) on an MHA workload's inputs,
    with the Annotated Transformer's LayerNorm (gain 1, bias 0, eps 1e-6)."""

    def __init__(self, inp):
        import torch
        from transformer_head_scaled_sdpa_amd import _lib
        self.mha = PreparedMha(inp)
        w = inp.workload
        t = self.mha.t
        self.lib = _lib.load()
        need = int(self.lib.mha_sublayer_workspace_bytes(_lib.MHA_BF16, w.B, w.Lq, w.Lk, w.d_model, w.h))
        self.ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        p = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())
        self.args = [_lib.MHA_BF16, _lib.MHA_F32, p(t["x_q"]), None, None, None, 0, 1e-6, p(t["w_q"]), p(t["b_q"]),
                     p(t["w_k"]), p(t["b_k"]), p(t["w_v"]), p(t["b_v"]), p(t["w_o"]), p(t["b_o"]), p(self.mha.out),
                     w.B, w.Lq, w.Lk, w.d_model, w.h, w.d_k, p(self.mha.vl), int(w.causal), p(self.ws), need]
        self.torch = torch

    def __call__(self):
        st = self.lib.mha_sublayer_forward(*self.args, ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"mha_sublayer_forward failed with status {st}")


def time_steps(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    return e0.elapsed_time(e1) / steps, wall / steps


def time_steps_cold(fn, steps):
    """Average step time with the caches cold: before every step a 512 MiB
    buffer is streamed (larger than the 256 MB last-level cache), and only
    the step itself lies between the two events."""
    import torch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    fn()
    for e0, e1 in evs:
        flush.fill_(1)
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    del flush
    return sum(e0.elapsed_time(e1) for e0, e1 in evs) / steps


def kernel_times(fn, steps, repeat):
    """Average duration (ms) per launch of each library kernel over `steps`
    eager steps, from the HIP event pairs the library records on the launch
    stream; each pair brackets `repeat` back-to-back launches of one kernel."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    torch.cuda.synchronize()
    with mha.kernel_timing(repeat=repeat) as kt:
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
    return {n: tot / cnt for n, (tot, cnt) in kt.result.items()}


COPY_CAL_BYTES = 1 << 30


def copy_calibration():
    """Plain streaming kernels of known size for scaling the L2-to-memory
    byte counters: a 1 GiB device-to-device copy and a 1 GiB negation, each
    reading 1 GiB and writing 1 GiB (larger than every cache level)."""
    import torch
    n = COPY_CAL_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"copy calibration: 3 x copy_ and 3 x neg of {COPY_CAL_BYTES} bytes")
    del src, dst


# ---------------------------------------------------------------------------
# measured HBM traffic (rocprofv3 FETCH_SIZE / WRITE_SIZE), valid only for
# the kernel sources it was measured on
# ---------------------------------------------------------------------------
CSRC = os.path.join(ROOT, "transformer_head_scaled_sdpa_amd", "csrc")
KERNEL_SOURCES = {
    "attn_fused_bf16": ["mha_fused.hip", "mha_fused_small.hip", "lds_tile.h", "common.h", "kernels.h"],
    "out_proj_bf16": ["gemm.hip", "lds_tile.h", "common.h", "kernels.h"],
    "sdpa_bf16": ["sdpa_bf16_pipe.hip", "common.h", "kernels.h"],
    "sdpa_decode": ["sdpa_decode.hip", "common.h", "kernels.h"],
}


def source_digest(name):
    files = KERNEL_SOURCES.get(name)
    if files is None:
        return None
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from profiles/traffic.json, or None when there is
    no record for this kernel and workload or its sources have changed since
    the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    digest = source_digest(kernel)
    for r in rec.get("kernels", []):
        if r["kernel"] == kernel and r["workload"] == workload and r["source_sha256"] == digest:
            return r["bytes_per_launch"]
    return None


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, untuned, on a bounded sample of the workload
# ---------------------------------------------------------------------------
def sampled_alg_flops(w, valid_lens, rows):
    """Algorithmic flops (4*d_k per allowed pair) of the given query rows of
    every (batch, head)."""
    vl = np.full(w.B, w.Lk) if valid_lens is None else np.asarray(valid_lens, dtype=np.int64)
    pairs = 0
    for v in vl:
        lim = w.Lk if v <= 0 else min(int(v), w.Lk)
        for i in rows:
            pairs += w.Lk if v <= 0 else (min(int(i) + 1, lim) if w.causal else lim)
    return 4 * w.d_k * w.h * pairs


def cpu_baseline(w, inp, budget_s=15.0):
    import oracle
    t = inp.tensors
    n_threads = oracle.num_threads()
    if w.kind in ("sdpa", "decode"):
        # Query rows evenly spread over the sequence, every (batch, head),
        # every key (the oracle computes every score as defined).  A first
        # call on 16 rows sizes the sample to about the time budget.
        def run(n):
            rows = np.unique(np.linspace(0, w.Lq - 1, n).astype(np.int32))
            t0 = time.perf_counter()
            oracle.sdpa(t["q"], t["k"], t["v"], valid_lens=inp.valid_lens, causal=w.causal, rows=rows)
            return rows, time.perf_counter() - t0
        rows, dt = run(min(16, w.Lq))
        n = int(min(w.Lq, max(16, 16 * budget_s / max(dt, 1e-6))))
        if n > len(rows):
            rows, dt = run(n)
        flops = sampled_alg_flops(w, inp.valid_lens, rows)
        return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": n_threads, "kind": "oracle",
                "sample": f"{len(rows)} of {w.Lq} query rows (evenly spaced) of every (batch, head), all {w.Lk} "
                          f"keys; {dt:.2f} s; rate counts the {flops / 1e9:.2f} GFLOP of mask-allowed pairs "
                          f"in the sample (4*d_k per pair), as the GPU value does"}
    # MHA: whole batches, all rows.  Time one batch, then as many batches as
    # fit the budget (at most the whole workload).
    def run(nb):
        sel = slice(0, nb)
        vl = None if inp.valid_lens is None else inp.valid_lens[sel]
        t0 = time.perf_counter()
        oracle.mha(t["x_q"][sel], t["x_kv"][sel], t["w_q"], t["w_k"], t["w_v"], t["w_o"],
                   t["b_q"], t["b_k"], t["b_v"], t["b_o"], h=w.h, valid_lens=vl, causal=w.causal)
        return time.perf_counter() - t0
    nb, dt = 1, run(1)
    fit = int(min(w.B, max(1, budget_s // max(dt, 1e-6))))
    if fit > 1:
        nb, dt = fit, run(fit)
    reps = 1
    if nb == w.B and dt < budget_s / 4:
        reps = int(max(1, (budget_s / 2) // max(dt, 1e-6)))
        dt = sum(run(nb) for _ in range(reps)) / reps
    vl = None if inp.valid_lens is None else inp.valid_lens[:nb]
    sub = workloads.Workload(w.name, w.kind, w.dtype, nb, w.Lq, w.Lk, w.h, w.d_k, w.causal, w.vl_range)
    flops = 4 * w.d_k * allowed_pairs(sub, vl)
    rep_txt = f", mean of {reps} runs" if reps > 1 else ""
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": n_threads, "kind": "oracle",
            "sample": f"{nb} of {w.B} batches, full MHA forward (projections included); {dt:.2f} s per run"
                      f"{rep_txt}; rate counts the mask-allowed attention pairs (4*d_k each)"}


HEADLINE = "sdpa_long_causal"
CONFIGS = ["mha_f32_tiny", "encoder_self", "decoder_causal", "enc_dec_source", "sdpa_long_causal"]


def measure_workload(w, inp, steps, warmup, repeat, cold=True):
    """Time one workload's step and its kernels; returns a dict with the step
    time, algorithmic rates and each kernel's roofline (the dominant one with
    the measured HBM traffic when the profiled sources still match)."""
    in_b = 2 if w.dtype == "bf16" else 4
    mfma_peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    fn = {"mha": PreparedMha, "sdpa": PreparedSdpa, "decode": PreparedDecode}[w.kind](inp)
    ms, wall_ms = time_steps(fn, steps, warmup)
    kt = kernel_times(fn, max(1, steps // repeat), repeat)
    kernels = {}
    M_q, M_kv = w.B * w.Lq, w.B * w.Lk
    for name, kms in kt.items():
        if name.startswith("sdpa_decode"):
            f, b = decode_alg(w, inp.valid_lens)
        elif name.startswith("attn_fused"):
            f, b = fused_alg(w, inp.valid_lens, in_b)
        elif name.startswith("qkv_proj"):
            f, b = gemm_alg(M_q, w.d_model, w.d_model, 1, in_b, in_b)
            f2, b2 = gemm_alg(M_kv, w.d_model, w.d_model, 2, in_b, in_b)
            f, b = f + f2, b + b2
        elif name.startswith("out_proj"):
            f, b = gemm_alg(M_q, w.d_model, w.d_model, 1, in_b, 4)
        else:
            f, b = sdpa_alg(w, inp.valid_lens, in_b, in_b if w.kind == "mha" else 2)
        kernels[name] = {"avg_us": round(kms * 1e3, 3), "alg_flops": f, "alg_bytes": b,
                         "roofline": roofline(f, b, kms, mfma_peak)}
    dom = max(kernels, key=lambda n: kernels[n]["avg_us"])
    alg_attn = 4 * w.d_k * allowed_pairs(w, inp.valid_lens)
    out = {"workload": w.description, "name": w.name, "dtype": w.dtype, "ms_per_step": round(ms, 6),
           "wall_ms_per_step": round(wall_ms, 6),
           "attention_alg_tflops": round(alg_attn / (ms * 1e-3) / 1e12, 3),
           "attention_dense_equiv_tflops": round(w.attention_flops() / (ms * 1e-3) / 1e12, 3),
           "kernels": {n: {"avg_us": k["avg_us"], "roofline_frac": k["roofline"]["frac"],
                           "bound": k["roofline"]["bound"]} for n, k in kernels.items()}}
    rl = dict(kernels[dom]["roofline"])
    rl["kernel"] = dom
    rl["traffic"] = measured_traffic(dom, w.name)
    rl["alg_per_launch"] = {"flops": kernels[dom]["alg_flops"], "bytes": kernels[dom]["alg_bytes"]}
    out["roofline"] = rl
    if w.kind == "mha":
        proj = 2 * w.d_model * w.d_model * w.B * (2 * w.Lq + 2 * w.Lk)
        out["mha_total"] = {"flops_per_step": int(proj + alg_attn),
                            "tflops": round((proj + alg_attn) / (ms * 1e-3) / 1e12, 3),
                            "frac_peak": round((proj + alg_attn) / (ms * 1e-3) / 1e12 / mfma_peak, 4),
                            "note": "projections Q, K, V, W_O (dense) plus the allowed attention pairs"}
    if cold:
        cold_ms = time_steps_cold(fn, 20)
        out["cold_cache_ms_per_step"] = round(cold_ms, 6)
    del fn
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # The clock ramps up over tens of milliseconds of sustained load (the long
    # causal kernel takes ~200 us per launch cold and ~155 us once warm), so
    # the default warm-up runs about 100 ms of steps before timing.
    ap.add_argument("--warmup", type=int, default=600)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(workloads.BY_NAME))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the headline workload (no other configs, no NEXT-row lines)")
    ap.add_argument("--repeat", type=int, default=10,
                    help="back-to-back launches per event pair when timing kernels (default 10)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run 1 GiB copy kernels (for scaling memory counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)

    if args.copy_calibration:
        copy_calibration()

    w = workloads.BY_NAME[args.workload]
    inp = workloads.make_inputs(w)
    mfma_peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    log(f"workload {w.name}: {w.description}")
    head = measure_workload(w, inp, args.steps, args.warmup, args.repeat)
    ms = head["ms_per_step"]
    alg_attn = 4 * w.d_k * allowed_pairs(w, inp.valid_lens)
    value = alg_attn / (ms * 1e-3) / 1e12
    log(f"step {ms * 1e3:.2f} us: {value:.1f} TFLOP/s algorithmic ({100 * value / mfma_peak:.1f}% of peak)")

    result = {
        "metric": "attention TFLOP/s (4*B*h*Lq*Lk*d_k) and % of MI355X bf16 MFMA peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "value_basis": "algorithmic: 4*d_k flops per mask-allowed (batch, head, query, key) pair per step / "
                       "step time (the literal 4*B*h*Lq*Lk*d_k count is reported as dense_equivalent)",
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 3),
        "dense_equivalent": {"flops_per_step": w.attention_flops(),
                             "tflops": head["attention_dense_equiv_tflops"],
                             "pct_bf16_peak": round(100 * head["attention_dense_equiv_tflops"] / PEAK_BF16_TFLOPS, 3)},
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded numpy PCG64; N(0,1) inputs, Xavier-uniform weights, zero bias)",
        "config": {"workload": w.description, "name": w.name, "B": w.B, "Lq": w.Lq, "Lk": w.Lk,
                   "d_model": w.d_model, "h": w.h, "d_k": w.d_k, "causal": w.causal,
                   "valid_lens": None if w.vl_range is None else f"U{{{w.vl_range[0]}..{w.vl_range[1]}}}",
                   "attention_alg_flops_per_step": int(alg_attn)},
        "kernels": head["kernels"],
        "roofline": head["roofline"],
        "cold_cache": {"ms_per_step": head["cold_cache_ms_per_step"],
                       "note": "512 MiB streamed before each of 20 steps; events bracket the step only"},
    }
    if "mha_total" in head:
        result["mha_total"] = head["mha_total"]

    if not args.no_extras:
        # The other configurations, each with its own dominant kernel's roofline.
        result["configs"] = {}
        for name in CONFIGS:
            if name == w.name:
                continue
            cw = workloads.BY_NAME[name]
            log(f"config {name} ...")
            result["configs"][name] = measure_workload(cw, workloads.make_inputs(cw), 100, 50, args.repeat)
        extras(result, args, w)

    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline(w, inp)
        if "configs" in result:
            # The oracle once on every other configuration too (a bounded
            # sample each), beside the GPU's step rate on the same count.
            per = {}
            for name, cfg in result["configs"].items():
                cw = workloads.BY_NAME[name]
                cb = cpu_baseline(cw, workloads.make_inputs(cw), budget_s=2.0)
                gpu = cfg.get("attention_alg_tflops")
                per[name] = {"value": cb["value"], "unit": cb["unit"], "sample": cb["sample"],
                             "gpu_over_oracle": round(gpu / cb["value"], 1) if gpu and cb["value"] else None}
            result["cpu_baseline"]["configs"] = per

    print(json.dumps(result), flush=True)


def extras(result, args, w):
    """The NEXT rows: decoding step, backward, inspection path, sublayer."""
    dw = workloads.BY_NAME["decode_step"]
    dinp = workloads.make_inputs(dw)
    df = PreparedDecode(dinp)
    dms, _ = time_steps(df, 200, 20)
    dk = sum(kernel_times(df, 20, args.repeat).values())
    f, b = decode_alg(dw, dinp.valid_lens)
    result["decode_step"] = {
        "workload": dw.description, "avg_us": round(dms * 1e3, 2),
        "alg_GBs": round(b / (dms * 1e-3) / 1e9, 1),
        "frac_hbm_peak": round(b / (dms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "kernel_us": round(dk * 1e3, 2), "kernel_frac_hbm_peak": round(b / (dk * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "note": "avg_us: calls issued back to back from Python; kernel_us: the library's events around "
                "back-to-back launches of the kernel alone"}
    del df

    ew = workloads.BY_NAME["encoder_self"]
    einp = workloads.make_inputs(ew)
    sf = PreparedSublayer(einp)
    sms, _ = time_steps(sf, 100, 10)
    result["mha_sublayer"] = {
        "workload": ew.description + ", as the pre-norm residual sublayer x + MHA(LayerNorm(x))",
        "ms_per_step": round(sms, 6)}
    del sf

    # backward: algorithmic 8*d_k flops per allowed pair (the four gradient
    # products dv, dp, dq, dk; the recomputed scores not counted)
    bw = workloads.BY_NAME["backward_causal"]
    binp = workloads.make_inputs(bw)
    pairs = allowed_pairs(bw, binp.valid_lens)
    bfl = 8 * bw.d_k * pairs
    bt = {}
    for use_lse in (True, False):
        bf = PreparedBackward(binp, use_lse)
        bt[use_lse], _ = time_steps(bf, 200, 200)
        del bf
    bms = bt[True]
    result["sdpa_backward"] = {
        "workload": bw.description + ", given the forward's log-sum-exp", "avg_us": round(bms * 1e3, 2),
        "alg_tflops": round(bfl / (bms * 1e-3) / 1e12, 2),
        "frac_bf16_mfma_peak": round(bfl / (bms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "bound": "mfma",
        "own_statistics_avg_us": round(bt[False] * 1e3, 2),
        "note": "8*d_k flops per allowed pair (dV, dP, dQ, dK products); recomputed scores not counted; "
                "own_statistics: sdpa_backward without the log-sum-exp (a pass of its own finds it)"}

    # backward of the multi-head layer on the decoder workload: algorithmic
    # work of the gradients themselves (dOcat, dW_o, the attention backward's
    # 8*d_k per allowed pair, the input and weight gradients of the three
    # input projections); the recomputed forward (Q/K/V projections and
    # attention) is reported beside it, not counted
    mw = workloads.BY_NAME["decoder_causal"]
    minp = workloads.make_inputs(mw)
    mf = PreparedMhaBackward(minp)
    mms, _ = time_steps(mf, 100, 50)
    mkt = kernel_times(mf, 10, args.repeat)
    del mf
    Mq, Mk, D = mw.B * mw.Lq, mw.B * mw.Lk, mw.d_model
    mpairs = allowed_pairs(mw, minp.valid_lens)
    grad_fl = 2 * Mq * D * D * 2 + 8 * mw.d_k * mpairs + 2 * D * D * (2 * Mq + 4 * Mk)
    recompute_fl = 2 * D * D * (Mq + 2 * Mk) + 4 * mw.d_k * mpairs
    result["mha_backward"] = {
        "workload": mw.description + ", output gradient N(0,1); all gradients fp32",
        "avg_us": round(mms * 1e3, 2),
        "alg_tflops": round(grad_fl / (mms * 1e-3) / 1e12, 2),
        "frac_bf16_mfma_peak": round(grad_fl / (mms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "with_recompute_tflops": round((grad_fl + recompute_fl) / (mms * 1e-3) / 1e12, 2),
        "kernels_us": {n: round(v * 1e3, 2) for n, v in mkt.items()},
        "note": "alg: 4*M*D^2 (dOcat, dW_o) + 8*d_k per allowed pair + 2*D^2*(2*Mq + 4*Mk) (input and weight "
                "gradients of W_Q, W_K, W_V); with_recompute adds the forward's projections and attention"}

    # the training pass (forward kept, backward on what it kept) on the same
    # workload: the forward's algorithmic work (projections, 4*d_k per
    # allowed pair) plus the gradients' above
    tf = PreparedTrainingPair(minp)
    tms, _ = time_steps(tf, 100, 50)
    tkt = kernel_times(tf, 10, args.repeat)
    del tf
    fwd_fl = 2 * D * D * (2 * Mq + 2 * Mk) + 4 * mw.d_k * mpairs
    result["mha_training_pass"] = {
        "workload": mw.description + ", mha_forward_train (bf16 output) then mha_backward_saved",
        "avg_us": round(tms * 1e3, 2),
        "alg_tflops": round((fwd_fl + grad_fl) / (tms * 1e-3) / 1e12, 2),
        "frac_bf16_mfma_peak": round((fwd_fl + grad_fl) / (tms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "kernels_us": {n: round(v * 1e3, 2) for n, v in tkt.items()},
        "note": "alg: forward 2*D^2*(2*Mq + 2*Mk) (four projections) + 4*d_k per allowed pair, plus the "
                "gradients' flops of mha_backward; nothing recomputed"}

    # inspection path: HBM-bound on the fp32 weights it writes; its matrix
    # work counted as the forward's algorithmic 4*d_k per allowed pair
    iw = workloads.BY_NAME["inspect_weights"]
    iinp = workloads.make_inputs(iw)
    wf = PreparedWeights(iinp)
    sms_w, _ = time_steps(wf, 20, 5)
    wms = sum(kernel_times(wf, 10, args.repeat).values())
    wbytes = iw.B * iw.h * (iw.Lq * iw.Lk * 4 + (2 * iw.Lq + 2 * iw.Lk) * iw.d_k * 2)
    wfl = 4 * iw.d_k * allowed_pairs(iw, iinp.valid_lens)
    result["sdpa_weights"] = {
        "workload": iw.description, "avg_us": round(wms * 1e3, 2), "bound": "hbm",
        "GBs": round(wbytes / (wms * 1e-3) / 1e9, 1), "frac_hbm_peak": round(wbytes / (wms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "alg_tflops": round(wfl / (wms * 1e-3) / 1e12, 2), "step_us": round(sms_w * 1e3, 2),
        "note": "avg_us: the library's events around back-to-back launches of the kernel; step_us: calls issued "
                "back to back from Python (bound by the host's call overhead when the kernel is shorter); bytes: "
                "fp32 weights written plus q, k, v read and o written; tflops: 4*d_k per allowed pair"}
    del wf


if __name__ == "__main__":
    main()
