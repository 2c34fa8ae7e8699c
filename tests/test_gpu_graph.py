"""The entry points under HIP graph capture: each call is captured once into a
graph and replayed on new inputs written in place; every replay must equal,
bit for bit, the eager call on the same inputs (the kernels are
deterministic: no atomics, no data-dependent reduction order).  Eager work
runs between the replays.  The library allocates nothing and records no
memset, so its launches are all it adds to a graph; the lengths are passed
as device tensors so no host copy is captured."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _graph_check(make_inputs, call, n_replays=3):
    import torch
    inputs = make_inputs(0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up outside the capture
        call(inputs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = call(inputs)
    for r in range(1, n_replays + 1):
        fresh = make_inputs(r)
        for dst, src in zip(inputs, fresh):
            if dst is not None:
                dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        eager = call(inputs)
        junk = torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")   # unrelated eager work
        torch.cuda.synchronize()
        outs_c = captured if isinstance(captured, tuple) else (captured,)
        outs_e = eager if isinstance(eager, tuple) else (eager,)
        for c, e in zip(outs_c, outs_e):
            assert torch.equal(c, e), f"replay {r} differs from the eager call"
        del junk


def _rand(shape, seed, dtype, scale=1.0):
    import torch
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype).cuda()


def test_graph_mha_forward():
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    B, L, D, h = 4, 128, 512, 8

    def make(r):
        x = _rand((B, L, D), 10 * r + 1, torch.bfloat16)
        ws = [_rand((D, D), 10 * r + 2 + i, torch.bfloat16, D ** -0.5) for i in range(4)]
        bs = [_rand((D,), 10 * r + 6 + i, torch.bfloat16, 0.1) for i in range(4)]
        vl = torch.tensor([128, 77, 1, 0], dtype=torch.int32).roll(r).cuda()
        return [x] + ws + bs + [vl]

    def call(t):
        x, wq, wk, wv, wo, bq, bk, bv, bo, vl = t
        return mha.mha_forward(x, x, wq, wk, wv, wo, bq, bk, bv, bo, h=h, valid_lens=vl)

    _graph_check(make, call)


def test_graph_sdpa_forward_causal():
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    B, h, L = 2, 4, 300

    def make(r):
        return [_rand((B, h, L, 64), 100 * r + i, torch.bfloat16) for i in range(3)]

    _graph_check(make, lambda t: mha.sdpa_forward(t[0], t[1], t[2], causal=True))


@pytest.mark.parametrize("B,h,L", [(64, 8, 512), (2, 2, 1000)])
def test_graph_sdpa_decode(B, h, L):
    """One slice written in place (B*h = 512, L = 512) and split + merge."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha

    def make(r):
        q = _rand((B, h, 64), 200 * r + 1, torch.bfloat16)
        k = _rand((B, h, L, 64), 200 * r + 2, torch.bfloat16)
        v = _rand((B, h, L, 64), 200 * r + 3, torch.bfloat16)
        rng = np.random.Generator(np.random.PCG64(r))
        lens = torch.from_numpy(rng.integers(0, L, size=B, endpoint=True).astype(np.int32)).cuda()
        return [q, k, v, lens]

    _graph_check(make, lambda t: mha.sdpa_decode(t[0], t[1], t[2], t[3]))


def test_graph_sdpa_backward():
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    B, h, L = 2, 2, 200

    def make(r):
        q, k, v, g = (_rand((B, h, L, 64), 300 * r + i, torch.bfloat16) for i in range(4))
        o = mha.sdpa_forward(q, k, v, causal=True)
        return [q, k, v, o, g]

    _graph_check(make, lambda t: mha.sdpa_backward(t[0], t[1], t[2], t[3], t[4], causal=True,
                                                   out_dtype=torch.float32))


def test_graph_sdpa_forward_and_backward_with_lse():
    """The training pair: the forward keeping each query's log-sum-exp, and
    the backward recomputing the weights from it (two launches: D and the
    statistic, then both gradient sides in one)."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    B, h, L = 2, 3, 300
    vl = torch.tensor([300, 171], dtype=torch.int32, device="cuda")

    def make(r):
        return [_rand((B, h, L, 64), 400 * r + i, torch.bfloat16) for i in range(4)]

    def call(t):
        o, lse = mha.sdpa_forward(t[0], t[1], t[2], valid_lens=vl, causal=True, return_lse=True)
        grads = mha.sdpa_backward(t[0], t[1], t[2], o, t[3], valid_lens=vl, causal=True,
                                  out_dtype=torch.float32, lse=lse)
        return (o, lse) + tuple(grads)

    _graph_check(make, call)


def test_graph_sdpa_weights_per_query_lengths():
    """The inspection path (weights exported) with one length per query."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    B, h, L = 2, 3, 150

    def make(r):
        qkv = [_rand((B, h, L, 64), 400 * r + i, torch.bfloat16) for i in range(3)]
        rng = np.random.Generator(np.random.PCG64(40 + r))
        vl = torch.from_numpy(rng.integers(0, L, size=(B, L), endpoint=True).astype(np.int32)).cuda()
        return qkv + [vl]

    _graph_check(make, lambda t: mha.sdpa_forward(t[0], t[1], t[2], valid_lens=t[3], return_weights=True))


def test_graph_mha_forward_with_weights():
    """mha_forward exporting the attention weights (projections to fp32 Q, K, V in the workspace)."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    B, L, D, h = 2, 96, 256, 4

    def make(r):
        x = _rand((B, L, D), 50 * r + 1, torch.bfloat16)
        ws = [_rand((D, D), 50 * r + 2 + i, torch.bfloat16, D ** -0.5) for i in range(4)]
        vl = torch.tensor([96, 40], dtype=torch.int32).roll(r).cuda()
        return [x] + ws + [vl]

    def call(t):
        x, wq, wk, wv, wo, vl = t
        return mha.mha_forward(x, x, wq, wk, wv, wo, h=h, valid_lens=vl, return_weights=True)

    _graph_check(make, call)


def test_graph_mha_sublayer():
    """The pre-norm sublayer x + MHA(LayerNorm(x)): layer norm, attention and the
    output projection with the residual."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    B, L, D, h = 4, 128, 512, 8

    def make(r):
        x = _rand((B, L, D), 60 * r + 1, torch.bfloat16)
        ws = [_rand((D, D), 60 * r + 2 + i, torch.bfloat16, D ** -0.5) for i in range(4)]
        g = _rand((D,), 60 * r + 7, torch.bfloat16, 0.1) + 1.0
        bb = _rand((D,), 60 * r + 8, torch.bfloat16, 0.1)
        vl = torch.tensor([128, 64, 1, 100], dtype=torch.int32).roll(r).cuda()
        return [x] + ws + [g, bb, vl]

    def call(t):
        x, wq, wk, wv, wo, g, bb, vl = t
        return mha.mha_sublayer_forward(x, wq, wk, wv, wo, h=h, ln_gain=g, ln_bias=bb, valid_lens=vl)

    _graph_check(make, call)


@pytest.mark.parametrize("self_attn", [True, False])
def test_graph_mha_backward(self_attn):
    """mha_backward's ten launches (transposes, projections, attention forward
    and backward, input and weight gradients) in one graph; outputs and
    workspace allocated once, outside the capture."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    B, L, Lk, D, h = 2, 200, 200 if self_attn else 130, 256, 4
    need = mha.library().mha_backward_workspace_bytes(mha.MHA_BF16, B, L, Lk, D, h)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def make(r):
        x = _rand((B, L, D), 10 * r + 1, torch.bfloat16)
        xkv = x if self_attn else _rand((B, Lk, D), 10 * r + 9, torch.bfloat16)
        ws_ = [_rand((D, D), 10 * r + 2 + i, torch.bfloat16, D ** -0.5) for i in range(4)]
        bs = [_rand((D,), 10 * r + 6 + i, torch.bfloat16, 0.1) for i in range(3)]
        g = _rand((B, L, D), 10 * r + 5, torch.bfloat16)
        vl = torch.tensor([Lk, 61], dtype=torch.int32).roll(r).cuda()
        return [x, None if self_attn else xkv] + ws_ + bs + [g, vl]

    def call(t):
        x, xkv = t[0], (t[0] if self_attn else t[1])
        r = mha.mha_backward(x, xkv, *t[2:6], t[9], *t[6:9], h=h, valid_lens=t[10], causal=self_attn,
                             bias_grads=True, workspace=ws)
        return tuple(r[n] for n in sorted(r) if r[n] is not None)

    _graph_check(make, call)


def test_graph_mha_training_pair():
    """mha_forward_train then mha_backward_saved (the forward's tensors kept
    in the saved buffer between the two) captured as one graph."""
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    B, L, D, h = 2, 160, 256, 4
    lib = mha.library()
    saved = torch.empty(lib.mha_saved_bytes(mha.MHA_BF16, B, L, L, D, h), dtype=torch.uint8, device="cuda")
    ws = torch.empty(lib.mha_backward_saved_workspace_bytes(mha.MHA_BF16, B, L, L, D, h), dtype=torch.uint8,
                     device="cuda")

    def make(r):
        x = _rand((B, L, D), 10 * r + 1, torch.bfloat16)
        ws_ = [_rand((D, D), 10 * r + 2 + i, torch.bfloat16, D ** -0.5) for i in range(4)]
        bs = [_rand((D,), 10 * r + 6 + i, torch.bfloat16, 0.1) for i in range(4)]
        g = _rand((B, L, D), 10 * r + 5, torch.bfloat16)
        vl = torch.tensor([L, 47], dtype=torch.int32).roll(r).cuda()
        return [x] + ws_ + bs + [g, vl]

    def call(t):
        x, wq, wk, wv, wo, bq, bk, bv, bo, g, vl = t
        out, _ = mha.mha_forward_train(x, x, wq, wk, wv, wo, bq, bk, bv, bo, h=h, valid_lens=vl, causal=True,
                                       saved=saved)
        r = mha.mha_backward(x, x, wq, wk, wv, wo, g, h=h, valid_lens=vl, causal=True, bias_grads=True,
                             workspace=ws, saved=saved)
        return (out,) + tuple(r[n] for n in sorted(r) if r[n] is not None)

    _graph_check(make, call)
