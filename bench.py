"""Benchmark: multi-head attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one full multi-head attention forward (Q/K/V projections, head
split, masked softmax attention, head merge, output projection) over one
batch of seeded synthetic input already resident in HBM.  Prints ONE JSON
line: the attention throughput 4*B*h*Lq*Lk*d_k per step / step time, the
roofline of the step's dominant kernel (duration from HIP events the library
records on its launch stream), the fp64 CPU oracle timed on the host's cores,
and the fused attention kernel on the long causal workload.
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
    """sdpa_backward on q, k, v, the forward output and an output gradient."""

    def __init__(self, inp):
        import torch
        import transformer_head_scaled_sdpa_amd as mha
        from transformer_head_scaled_sdpa_amd import _lib
        w = inp.workload
        dev = torch.device("cuda:0")
        self.t = [torch.from_numpy(inp.tensors[n]).to(dev).to(torch.bfloat16) for n in "qkv"]
        rng = np.random.Generator(np.random.PCG64(w.seed + 1000))
        self.g = torch.from_numpy(rng.standard_normal(self.t[0].shape).astype(np.float32)).to(dev).to(torch.bfloat16)
        self.vl = None if inp.valid_lens is None else torch.from_numpy(inp.valid_lens).to(dev)
        self.o = mha.sdpa_forward(*self.t, valid_lens=self.vl, causal=w.causal)
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
                                                             int(w.causal), p(self.ws), need]
        self.torch = torch

    def __call__(self):
        st = self.lib.sdpa_backward(*self.args, ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"sdpa_backward failed with status {st}")


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
def cpu_baseline(w, inp, budget_s=20.0):
    import oracle
    t = inp.tensors
    n_threads = oracle.num_threads()
    if w.kind in ("sdpa", "decode"):
        # sample query rows; every (batch, head) pair, all keys
        rows = np.unique(np.linspace(0, w.Lq - 1, 16).astype(np.int32))
        t0 = time.perf_counter()
        oracle.sdpa(t["q"], t["k"], t["v"], valid_lens=inp.valid_lens, causal=w.causal, rows=rows)
        dt = time.perf_counter() - t0
        flops = 4 * w.B * w.h * len(rows) * w.Lk * w.d_k
        return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": n_threads, "kind": "oracle",
                "sample": f"{len(rows)} query rows of every (batch, head), all {w.Lk} keys; {dt:.2f} s"}
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
    # When the whole workload takes well under the budget, repeat it (about
    # half the budget in total) and report the mean.
    reps = 1
    if nb == w.B and dt < budget_s / 4:
        reps = int(max(1, (budget_s / 2) // max(dt, 1e-6)))
        dt = sum(run(nb) for _ in range(reps)) / reps
    flops = 4 * nb * w.h * w.Lq * w.Lk * w.d_k
    rep_txt = f", mean of {reps} runs" if reps > 1 else ""
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": n_threads, "kind": "oracle",
            "sample": f"{nb} of {w.B} batches, full MHA forward (projections included); {dt:.2f} s per run{rep_txt}"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="encoder_self", choices=sorted(workloads.BY_NAME))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long-sdpa", action="store_true", help="skip the long causal attention kernel line")
    ap.add_argument("--repeat", type=int, default=10,
                    help="back-to-back launches per event pair when timing kernels (default 10)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run 1 GiB copy kernels (for scaling memory counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
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
    in_b = 2 if w.dtype == "bf16" else 4
    mfma_peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    log(f"workload {w.name}: {w.description}")

    fn = {"mha": PreparedMha, "sdpa": PreparedSdpa, "decode": PreparedDecode}[w.kind](inp)
    ms, wall_ms = time_steps(fn, args.steps, args.warmup)
    cold_ms = time_steps_cold(fn, 20)
    attn_flops = w.attention_flops()
    value = attn_flops / (ms * 1e-3) / 1e12
    log(f"step {ms * 1e3:.2f} us (wall {wall_ms * 1e3:.2f} us)")

    # per-kernel durations and the dominant kernel's roofline
    kt = kernel_times(fn, max(1, args.steps // args.repeat), args.repeat)
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
    rl = dict(kernels[dom]["roofline"])
    rl["kernel"] = dom
    rl["traffic"] = measured_traffic(dom, w.name)
    rl["alg_per_launch"] = {"flops": kernels[dom]["alg_flops"], "bytes": kernels[dom]["alg_bytes"]}

    result = {
        "metric": "attention TFLOP/s (4*B*h*Lq*Lk*d_k per step / step time) and % of MI355X bf16 MFMA peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 3),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded numpy PCG64; Xavier-uniform weights, zero bias)",
        "config": {"workload": w.description, "name": w.name, "B": w.B, "Lq": w.Lq, "Lk": w.Lk,
                   "d_model": w.d_model, "h": w.h, "d_k": w.d_k, "causal": w.causal,
                   "valid_lens": None if w.vl_range is None else f"U{{{w.vl_range[0]}..{w.vl_range[1]}}}",
                   "attention_flops_per_step": attn_flops},
        "kernels": {n: {"avg_us": k["avg_us"], "roofline_frac": k["roofline"]["frac"],
                        "bound": k["roofline"]["bound"]} for n, k in kernels.items()},
        "roofline": rl,
        "cold_cache": {"ms_per_step": round(cold_ms, 6), "value": round(attn_flops / (cold_ms * 1e-3) / 1e12, 3),
                       "note": "512 MiB streamed before each of 20 steps; events bracket the step only"},
    }
    # Beside the literal formula: the attention flops the masks allow
    # (4 * d_k per allowed pair) and, for the multi-head layer, the whole
    # step's work with the projections (Q over all queries, K and V over the
    # keys, W_O over all queries).
    alg_attn = 4 * w.d_k * allowed_pairs(w, inp.valid_lens)
    result["attention_alg"] = {"flops_per_step": int(alg_attn),
                               "tflops": round(alg_attn / (ms * 1e-3) / 1e12, 3),
                               "frac_bf16_peak": round(alg_attn / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    if w.kind == "mha":
        proj = 2 * w.d_model * w.d_model * w.B * (2 * w.Lq + 2 * w.Lk)
        result["mha_total"] = {"flops_per_step": int(proj + alg_attn),
                               "tflops": round((proj + alg_attn) / (ms * 1e-3) / 1e12, 3),
                               "frac_peak": round((proj + alg_attn) / (ms * 1e-3) / 1e12 / mfma_peak, 4),
                               "note": "projections Q, K, V, W_O (dense) plus the allowed attention pairs"}

    if not args.no_long_sdpa and w.name != "sdpa_long_causal":
        lw = workloads.BY_NAME["sdpa_long_causal"]
        linp = workloads.make_inputs(lw)
        sf = PreparedSdpa(linp)
        sms, _ = time_steps(sf, 50, 20)
        f, b = sdpa_alg(lw, None, 2, 2)
        result["sdpa_long_causal"] = {
            "workload": lw.description, "avg_us": round(sms * 1e3, 2),
            "alg_tflops": round(f / (sms * 1e-3) / 1e12, 2),
            "dense_equiv_tflops": round(lw.attention_flops() / (sms * 1e-3) / 1e12, 2),
            "frac_bf16_peak_alg": round(f / (sms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del sf

    if not args.no_long_sdpa and w.name != "decode_step":
        dw = workloads.BY_NAME["decode_step"]
        dinp = workloads.make_inputs(dw)
        df = PreparedDecode(dinp)
        dms, _ = time_steps(df, 200, 20)
        f, b = decode_alg(dw, dinp.valid_lens)
        result["decode_step"] = {
            "workload": dw.description, "avg_us": round(dms * 1e3, 2),
            "alg_GBs": round(b / (dms * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(b / (dms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        del df

    if not args.no_long_sdpa and w.kind == "mha" and w.dtype == "bf16" and w.self_attn:
        sf = PreparedSublayer(inp)
        sms, _ = time_steps(sf, args.steps, args.warmup)
        result["mha_sublayer"] = {
            "workload": w.description + ", as the pre-norm residual sublayer x + MHA(LayerNorm(x))",
            "ms_per_step": round(sms, 6), "value": round(attn_flops / (sms * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
            "vs_plain_step": round(sms / ms, 3)}
        del sf

    if not args.no_long_sdpa:
        # backward: algorithmic 8*d_k flops per allowed pair (the four
        # gradient products dv, dp, dq, dk; the recomputed scores not counted)
        bw = workloads.BY_NAME["backward_causal"]
        binp = workloads.make_inputs(bw)
        bf = PreparedBackward(binp)
        bms, _ = time_steps(bf, 10, 3)
        pairs = allowed_pairs(bw, binp.valid_lens)
        bfl = 8 * bw.d_k * pairs
        result["sdpa_backward"] = {
            "workload": bw.description, "avg_us": round(bms * 1e3, 2),
            "alg_tflops": round(bfl / (bms * 1e-3) / 1e12, 2),
            "frac_bf16_mfma_peak": round(bfl / (bms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "bound": "mfma"}
        del bf
        # inspection path: the weights written (fp32) plus q, k, v read and o
        # written; on bf16 MFMA the scores run twice (2 * 2 * d_k flops per
        # allowed pair) and P.V once with P as two bf16 terms (2 * 2 * d_k)
        iw = workloads.BY_NAME["inspect_weights"]
        iinp = workloads.make_inputs(iw)
        wf = PreparedWeights(iinp)
        wms, _ = time_steps(wf, 10, 3)
        wbytes = iw.B * iw.h * (iw.Lq * iw.Lk * 4 + (2 * iw.Lq + 2 * iw.Lk) * iw.d_k * 2)
        wfl = 8 * iw.d_k * allowed_pairs(iw, iinp.valid_lens)
        result["sdpa_weights"] = {
            "workload": iw.description, "avg_us": round(wms * 1e3, 2), "bound": "hbm",
            "GBs": round(wbytes / (wms * 1e-3) / 1e9, 1), "frac_hbm_peak": round(wbytes / (wms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "mfma_tflops": round(wfl / (wms * 1e-3) / 1e12, 2),
            "frac_bf16_mfma_peak": round(wfl / (wms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del wf

    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline(w, inp)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
