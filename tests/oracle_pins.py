"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
a value the pages print, a closed form, an invariant, a brute-force hand
computation or an independent torch float64 CPU routine.  ``test_oracle.py``
runs them against the oracle; ``test_oracle_mutations.py`` runs them against
copies of the oracle with a planted mistake and requires that one fails.
"""
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _close(a, b, tol=1e-12):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"max abs diff {err} > {tol}"


# ---------------------------------------------------------------------------
# values the pages print
# ---------------------------------------------------------------------------
def pin_scaling_example():
    """112 vs 96 (page 5, Self-Attention structure): with sqrt(64) scaling the
    weights are softmax(14, 12); unscaled (d_k = 1 gives scale 1) the second
    weight is ~1e-7, i.e. the page's 'near 0'."""
    g = {r[0]: float(r[1]) for r in _read_golden("scaling_example.txt")}
    s_self, s_other, dk = g["score_self"], g["score_other"], int(g["d_k"])
    q = np.zeros((1, 1, 1, dk)); q[..., 0] = 1.0
    k = np.zeros((1, 1, 2, dk)); k[0, 0, 0, 0] = s_self; k[0, 0, 1, 0] = s_other
    v = np.eye(2).reshape(1, 1, 2, 2)
    o, p = oracle.sdpa(q, k, v, return_weights=True)
    gap = (s_self - s_other) / math.sqrt(dk)       # 2.0
    w2 = 1.0 / (1.0 + math.exp(gap))
    _close(p[0, 0, 0], [1.0 - w2, w2], 1e-15)
    _close(o[0, 0, 0], [1.0 - w2, w2], 1e-15)
    # The unscaled softmax: a one-wide head has scale 1/sqrt(1) = 1.
    q1 = np.ones((1, 1, 1, 1))
    k1 = np.array([s_self, s_other]).reshape(1, 1, 2, 1)
    _, p1 = oracle.sdpa(q1, k1, v, return_weights=True)
    w2u = 1.0 / (1.0 + math.exp(s_self - s_other))
    _close(p1[0, 0, 0], [1.0 - w2u, w2u], 1e-15)
    assert p1[0, 0, 0, 1] < 2e-7 and p[0, 0, 0, 1] > 0.1


def pin_causal_mask_printed():
    """The printed 5x5 subsequent mask (page 4): weights are nonzero exactly
    where the mask holds 1, and exactly 0 elsewhere."""
    mask = np.array([[int(x) for x in r] for r in _read_golden("subsequent_mask_5.txt")])
    assert mask.shape == (5, 5)
    r = _rng(11)
    q, k = r.standard_normal((1, 2, 5, 8)), r.standard_normal((1, 2, 5, 8))
    v = r.standard_normal((1, 2, 5, 3))
    _, p = oracle.sdpa(q, k, v, causal=True, return_weights=True)
    for hd in range(2):
        assert np.array_equal((p[0, hd] > 0).astype(int), mask)
        assert np.all(p[0, hd][mask == 0] == 0.0)


def pin_d2l_shape():
    g = {r[0]: r[1:] for r in _read_golden("d2l_encoder_shape.txt")}
    B, L, D, h = (int(g[k][0]) for k in ("batch", "length", "d_model", "heads"))
    vl = [int(x) for x in g["valid_lens"]]
    r = _rng(12)
    x = r.standard_normal((B, L, D))
    ws = [r.uniform(-0.3, 0.3, (D, D)) for _ in range(4)]
    out = oracle.mha(x, x, *ws, h=h, valid_lens=vl)
    assert out.shape == (B, L, D)
    # batch 0 attends only its first 3 keys: what lies beyond cannot matter
    # to its first 3 query rows; batch 1 is untouched.
    x2 = x.copy()
    x2[0, 3:] = 5.0 + r.standard_normal((L - 3, D))
    out2 = oracle.mha(x2, x2, *ws, h=h, valid_lens=vl, rows=[0, 1, 2])
    _close(out2, out[:, :3], 1e-12)


def pin_single_head_shapes():
    g = {r[0]: int(r[1]) for r in _read_golden("p4_single_head_shapes.txt")}
    B, L, d = g["batch"], g["length"], g["d_k"]
    r = _rng(13)
    q, k, v = (r.standard_normal((B, 1, L, d)) for _ in range(3))
    o, p = oracle.sdpa(q, k, v, return_weights=True)
    assert o.shape == (B, 1, L, d) and p.shape == (B, 1, L, L)


# ---------------------------------------------------------------------------
# closed forms and hand-derived tiny cases
# ---------------------------------------------------------------------------
def pin_zero_query_is_mean_of_allowed():
    r = _rng(21)
    B, h, L, d = 2, 3, 7, 4
    q = np.zeros((B, h, L, d))
    k, v = r.standard_normal((B, h, L, d)), r.standard_normal((B, h, L, 5))
    vl = np.array([3, 7])
    o = oracle.sdpa(q, k, v, valid_lens=vl)
    for b in range(B):
        _close(o[b], np.broadcast_to(v[b, :, :vl[b]].mean(axis=1, keepdims=True), o[b].shape), 1e-14)
    oc = oracle.sdpa(q, k, v, causal=True, valid_lens=vl)
    for b in range(B):
        for i in range(L):
            n = min(i + 1, vl[b])
            _close(oc[b, :, i], v[b, :, :n].mean(axis=1), 1e-14)


def pin_single_allowed_key():
    r = _rng(22)
    q, k, v = (r.standard_normal((2, 2, 6, 4)) for _ in range(3))
    o = oracle.sdpa(q, k, v, valid_lens=[1, 1])
    _close(o, np.broadcast_to(v[:, :, :1], o.shape), 0.0)
    oc = oracle.sdpa(q, k, v, causal=True)
    _close(oc[:, :, 0], v[:, :, 0], 0.0)


def pin_two_keys_sigmoid():
    r = _rng(23)
    d = 16
    q, k, v = (r.standard_normal((1, 1, 3, d)) for _ in range(3))
    o, p = oracle.sdpa(q, k, v, valid_lens=[2], return_weights=True)
    for i in range(3):
        delta = (q[0, 0, i] @ k[0, 0, 0] - q[0, 0, i] @ k[0, 0, 1]) / math.sqrt(d)
        w0 = 1.0 / (1.0 + math.exp(-delta))
        _close(p[0, 0, i], [w0, 1.0 - w0, 0.0], 1e-15)
        _close(o[0, 0, i], w0 * v[0, 0, 0] + (1.0 - w0) * v[0, 0, 1], 1e-14)


def pin_identical_keys_uniform():
    r = _rng(24)
    q = r.standard_normal((1, 2, 4, 8))
    k = np.broadcast_to(r.standard_normal((1, 2, 1, 8)), (1, 2, 6, 8)).copy()
    v = r.standard_normal((1, 2, 6, 3))
    _, p = oracle.sdpa(q, k, v, valid_lens=[5], return_weights=True)
    _close(p[..., :5], np.full((1, 2, 4, 5), 0.2), 1e-15)
    assert np.all(p[..., 5] == 0.0)


def pin_fully_masked_row_is_uniform():
    """valid_len = 0: every score becomes -1e9, so the softmax is uniform over
    all Lk keys (the replace-not-add reading of the -1e9 fill)."""
    r = _rng(25)
    q, k, v = (r.standard_normal((2, 2, 5, 4)) for _ in range(3))
    q = q * 10
    o = oracle.sdpa(q, k, v, valid_lens=[0, 5])
    _close(o[0], np.broadcast_to(v[0].mean(axis=1, keepdims=True), o[0].shape), 1e-14)
    oc = oracle.sdpa(q, k, v, valid_lens=[0, 5], causal=True)
    _close(oc[0], np.broadcast_to(v[0].mean(axis=1, keepdims=True), oc[0].shape), 1e-14)


def pin_brute_force_hand_cases():
    """Tiny cases worked by hand (h = 1).

    d = 4 gives scale 1/2.  q = (2,0,0,0); keys (1,0,0,0), (0,0,0,0), (0,2,0,0)
    score 1, 0, 0; values (1,0), (0,1), (1,1):
      o = (e*1 + 1*0 + 1*1, e*0 + 1 + 1) / (e + 2) = ((e+1)/(e+2), 2/(e+2)).
    Second query (0,0,0,4): all scores 0 -> uniform -> o = (2/3, 2/3).
    With valid_len 2 the third key is dropped: o = (e/(e+1), 1/(e+1)).
    Causal: query 0 sees key 0 only -> (1, 0); query 1 sees keys 0, 1 with
    scores 0, 0 -> (1/2, 1/2).
    d = 1: q = 1, keys 0, 1, 2 -> weights prop. to 1, e, e^2.
    """
    e = math.e
    q = np.array([[2, 0, 0, 0], [0, 0, 0, 4]], dtype=float).reshape(1, 1, 2, 4)
    k = np.array([[1, 0, 0, 0], [0, 0, 0, 0], [0, 2, 0, 0]], dtype=float).reshape(1, 1, 3, 4)
    v = np.array([[1, 0], [0, 1], [1, 1]], dtype=float).reshape(1, 1, 3, 2)
    o = oracle.sdpa(q, k, v)
    _close(o[0, 0, 0], [(e + 1) / (e + 2), 2 / (e + 2)], 1e-15)
    _close(o[0, 0, 1], [2 / 3, 2 / 3], 1e-15)
    o2 = oracle.sdpa(q, k, v, valid_lens=[2])
    _close(o2[0, 0, 0], [e / (e + 1), 1 / (e + 1)], 1e-15)
    qs = np.concatenate([q, q[:, :, :1]], axis=2)   # 3 queries, square causal
    oc = oracle.sdpa(qs, k, v, causal=True)
    _close(oc[0, 0, 0], [1.0, 0.0], 0.0)
    _close(oc[0, 0, 1], [0.5, 0.5], 1e-16)
    q1 = np.ones((1, 1, 1, 1))
    k1 = np.array([0.0, 1.0, 2.0]).reshape(1, 1, 3, 1)
    v1 = np.eye(3).reshape(1, 1, 3, 3)
    _, p1 = oracle.sdpa(q1, k1, v1, return_weights=True)
    z = 1 + e + e * e
    _close(p1[0, 0, 0], [1 / z, e / z, e * e / z], 1e-15)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
def pin_rows_sum_to_one_and_masked_zero():
    r = _rng(31)
    B, h, L, d = 3, 2, 9, 8
    q, k, v = (r.standard_normal((B, h, L, d)) for _ in range(3))
    vl = np.array([4, 9, 1])
    for causal in (False, True):
        _, p = oracle.sdpa(q, k, v, valid_lens=vl, causal=causal, return_weights=True)
        assert np.max(np.abs(p.sum(-1) - 1.0)) <= 1e-15
        j = np.arange(L)
        for b in range(B):
            for i in range(L):
                masked = (j >= vl[b]) | ((j > i) if causal else False)
                assert np.all(p[b, :, i, masked] == 0.0)
                assert np.all(p[b, :, i, ~masked] > 0.0)


def pin_shift_invariances():
    r = _rng(32)
    B, h, L, d, dv = 2, 2, 8, 8, 6
    q, k = r.standard_normal((B, h, L, d)), r.standard_normal((B, h, L, d))
    v = r.standard_normal((B, h, L, dv))
    vl = [5, 8]
    o = oracle.sdpa(q, k, v, valid_lens=vl, causal=True)
    u = r.standard_normal(d)
    _close(oracle.sdpa(q, k + u, v, valid_lens=vl, causal=True), o, 1e-12)
    w = r.standard_normal(dv)
    _close(oracle.sdpa(q, k, v + w, valid_lens=vl, causal=True), o + w, 1e-12)
    v2 = r.standard_normal((B, h, L, dv))
    o2 = oracle.sdpa(q, k, v2, valid_lens=vl, causal=True)
    _close(oracle.sdpa(q, k, 2.0 * v - 3.0 * v2, valid_lens=vl, causal=True), 2.0 * o - 3.0 * o2, 1e-12)


def pin_permutations():
    r = _rng(33)
    B, h, Lq, Lk, d = 1, 2, 5, 7, 8
    q, k = r.standard_normal((B, h, Lq, d)), r.standard_normal((B, h, Lk, d))
    v = r.standard_normal((B, h, Lk, 4))
    o = oracle.sdpa(q, k, v)
    perm = r.permutation(Lk)
    _close(oracle.sdpa(q, k[:, :, perm], v[:, :, perm]), o, 1e-13)
    qp = r.permutation(Lq)
    _close(oracle.sdpa(q[:, :, qp], k, v), o[:, :, qp], 1e-13)


def pin_scale_uses_head_width():
    """Zero-padding q and k from d to 2d leaves the dot products unchanged but
    the scale becomes 1/sqrt(2d): same as q / sqrt(2) at width d."""
    r = _rng(34)
    q, k, v = r.standard_normal((1, 2, 6, 8)), r.standard_normal((1, 2, 6, 8)), r.standard_normal((1, 2, 6, 3))
    pad = lambda a: np.concatenate([a, np.zeros_like(a)], axis=-1)
    _close(oracle.sdpa(pad(q), pad(k), v), oracle.sdpa(q / math.sqrt(2.0), k, v), 1e-13)


def pin_score_variance_near_one():
    """Unit-variance q and k give q.k a variance of d_k; after the 1/sqrt(d_k)
    scaling the scores have unit variance (page 5).  Differences of log
    weights within a row are differences of scores."""
    r = _rng(35)
    d, L = 64, 2048
    q = r.standard_normal((1, 1, 16, d))
    k = r.standard_normal((1, 1, L, d))
    v = np.zeros((1, 1, L, 1))
    _, p = oracle.sdpa(q, k, v, return_weights=True)
    var = np.var(np.log(p[0, 0]), axis=-1)
    # each row's variance is |q_i|^2 / d (exact in expectation over keys)
    expect = (q[0, 0] ** 2).sum(-1) / d
    assert np.max(np.abs(var / expect - 1.0)) < 0.1
    assert abs(var.mean() - 1.0) < 0.15


def pin_valid_lens_per_query_equals_causal():
    """Per-query valid length i+1 (the d2l decoder's training-time lengths)
    gives the causal mask."""
    r = _rng(36)
    B, h, L, d = 1, 2, 6, 4
    q, k, v = (r.standard_normal((B, h, L, d)) for _ in range(3))
    oc = oracle.sdpa(q, k, v, causal=True)
    for i in range(L):
        oi = oracle.sdpa(q, k, v, valid_lens=[i + 1], rows=[i])
        _close(oi[:, :, 0], oc[:, :, i], 0.0)


def pin_valid_lens_2d_lengths_i_plus_1_equal_causal():
    """Lengths per query [B, Lq] with row i holding i + 1 (the d2l decoder's
    training-time valid lengths, one row per batch) give the causal mask, in
    one call over all rows."""
    r = _rng(41)
    B, h, L, d = 3, 2, 7, 4
    q, k, v = (r.standard_normal((B, h, L, d)) for _ in range(3))
    vl2 = np.tile(np.arange(1, L + 1, dtype=np.int32), (B, 1))
    _close(oracle.sdpa(q, k, v, valid_lens=vl2), oracle.sdpa(q, k, v, causal=True), 0.0)


def pin_valid_lens_2d_each_row_is_its_own_length():
    """Row i of batch b under lengths per query equals a one-row call with a
    per-batch length equal to vl2[b, i] (brute force over every (b, i));
    Lq != B so a transposed (b, i) index is caught."""
    r = _rng(42)
    B, h, Lq, Lk, d = 2, 2, 5, 6, 3
    q = r.standard_normal((B, h, Lq, d))
    k, v = (r.standard_normal((B, h, Lk, d)) for _ in range(2))
    vl2 = r.integers(0, Lk + 1, size=(B, Lq)).astype(np.int32)
    vl2[0, 1] = 0                            # a fully masked row
    o2 = oracle.sdpa(q, k, v, valid_lens=vl2)
    for b in range(B):
        for i in range(Lq):
            o1 = oracle.sdpa(q[b:b + 1], k[b:b + 1], v[b:b + 1], valid_lens=[vl2[b, i]], rows=[i])
            _close(o2[b:b + 1, :, i], o1[:, :, 0], 0.0)
    # closed form of the fully masked row: uniform weights over every key
    _close(o2[0, :, 1], v[0].mean(axis=1), 1e-12)


def pin_valid_lens_2d_constant_rows_equal_per_batch():
    """Lengths per query that repeat the batch's length in every row equal
    lengths per batch, for sdpa and for the multi-head layer."""
    r = _rng(43)
    B, h, Lq, Lk, d = 2, 2, 4, 5, 3
    q = r.standard_normal((B, h, Lq, d))
    k, v = (r.standard_normal((B, h, Lk, d)) for _ in range(2))
    vl = np.array([2, 5], dtype=np.int32)
    vl2 = np.repeat(vl[:, None], Lq, axis=1)
    _close(oracle.sdpa(q, k, v, valid_lens=vl2), oracle.sdpa(q, k, v, valid_lens=vl), 0.0)
    D = 8
    xq, xkv = r.standard_normal((B, Lq, D)), r.standard_normal((B, Lk, D))
    w = [r.standard_normal((D, D)) * 0.3 for _ in range(4)]
    _close(oracle.mha(xq, xkv, *w, h=2, valid_lens=vl2), oracle.mha(xq, xkv, *w, h=2, valid_lens=vl), 0.0)


def pin_mha_valid_lens_2d_lengths_i_plus_1_equal_causal():
    """The multi-head layer with query lengths i + 1 equals its causal form."""
    r = _rng(44)
    B, L, D = 2, 5, 8
    x = r.standard_normal((B, L, D))
    w = [r.standard_normal((D, D)) * 0.3 for _ in range(4)]
    vl2 = np.tile(np.arange(1, L + 1, dtype=np.int32), (B, 1))
    _close(oracle.mha(x, x, *w, h=2, valid_lens=vl2), oracle.mha(x, x, *w, h=2, causal=True), 0.0)


def _fd_grads(q, k, v, g, **mask):
    """Central finite differences of sum(sdpa(q, k, v) * g) in each element."""
    out = []
    for x in (q, k, v):
        d = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            e = 1e-6
            x[idx] += e
            up = np.sum(oracle.sdpa(q, k, v, **mask) * g)
            x[idx] -= 2 * e
            dn = np.sum(oracle.sdpa(q, k, v, **mask) * g)
            x[idx] += e
            d[idx] = (up - dn) / (2 * e)
        out.append(d)
    return out


def pin_backward_matches_finite_differences():
    """The gradients equal central differences of the forward oracle, with
    key padding (a fully masked sequence included), the causal rule, and
    lengths per query."""
    r = _rng(51)
    B, h, Lq, Lk, d = 2, 1, 3, 4, 3
    q = r.standard_normal((B, h, Lq, d))
    k = r.standard_normal((B, h, Lk, d))
    v = r.standard_normal((B, h, Lk, d))
    g = r.standard_normal((B, h, Lq, d))
    for mask in ({}, {"valid_lens": [2, 0]}, {"valid_lens": np.array([[1, 3, 0], [4, 2, 2]], np.int32)}):
        fd = _fd_grads(q, k, v, g, **mask)
        for a, b in zip(oracle.sdpa_backward(q, k, v, g, **mask), fd):
            _close(a, b, 1e-7)
    qs = r.standard_normal((1, 2, 4, d))
    ks, vs, gs = (r.standard_normal((1, 2, 4, d)) for _ in range(3))
    fd = _fd_grads(qs, ks, vs, gs, causal=True)
    for a, b in zip(oracle.sdpa_backward(qs, ks, vs, gs, causal=True), fd):
        _close(a, b, 1e-7)


def pin_backward_matches_torch_float64_autograd():
    """torch's float64 CPU autograd through its own fused attention
    (scaled_dot_product_attention, default 1/sqrt(d) scale) with a boolean
    key mask.  Every row here keeps at least one allowed key, where excluding
    a key and filling its score with -1e9 give the same weights."""
    import torch
    import torch.nn.functional as F
    r = _rng(52)
    B, h, Lq, Lk, d = 2, 3, 5, 6, 4
    q, k, v = (r.standard_normal(s) for s in ((B, h, Lq, d), (B, h, Lk, d), (B, h, Lk, d)))
    g = r.standard_normal((B, h, Lq, d))
    vl = np.array([4, 6], np.int32)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    keep = torch.arange(Lk)[None, None, None, :] < torch.tensor(vl)[:, None, None, None]
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=keep.expand(B, h, Lq, Lk))
    (o * torch.tensor(g)).sum().backward()
    for a, b in zip(oracle.sdpa_backward(q, k, v, g, valid_lens=vl), (tq.grad, tk.grad, tv.grad)):
        _close(a, b.numpy(), 1e-12)


def pin_backward_closed_forms():
    """One allowed key: the weights are constant, so dq = dk = 0 and dv of
    that key is the sum of the output gradients.  Identical keys: uniform
    weights, dq = 0 and dv_j = sum_i do_i / Lk."""
    r = _rng(53)
    B, h, Lq, Lk, d = 1, 2, 4, 5, 3
    q, k, v = (r.standard_normal(s) for s in ((B, h, Lq, d), (B, h, Lk, d), (B, h, Lk, d)))
    g = r.standard_normal((B, h, Lq, d))
    dq, dk, dv = oracle.sdpa_backward(q, k, v, g, valid_lens=[1])
    _close(dq, np.zeros_like(dq))
    _close(dk, np.zeros_like(dk))
    _close(dv[:, :, 0], g.sum(axis=2))
    _close(dv[:, :, 1:], np.zeros_like(dv[:, :, 1:]))
    ks = np.repeat(k[:, :, :1], Lk, axis=2)
    dq, dk, dv = oracle.sdpa_backward(q, ks, v, g)
    _close(dq, np.zeros_like(dq))
    _close(dv, np.repeat(g.sum(axis=2, keepdims=True) / Lk, Lk, axis=2))


def pin_layer_norm_hand_example():
    """x = [1, 2, 3, 4]: mean 2.5, squared deviations summing to 5, so the
    Annotated Transformer's std (n - 1) is sqrt(5/3) and the torch layer's
    root of the biased variance is sqrt(5/4); gain and bias act per feature."""
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    dev = np.array([-1.5, -0.5, 0.5, 1.5])
    _close(oracle.layer_norm(x, kind=0, eps=0.0)[0], dev / math.sqrt(5 / 3))
    _close(oracle.layer_norm(x, kind=1, eps=0.0)[0], dev / math.sqrt(5 / 4))
    a, b = np.array([2.0, 1.0, 0.5, -1.0]), np.array([1.0, 0.0, -2.0, 3.0])
    _close(oracle.layer_norm(x, a, b, kind=0, eps=0.5)[0], a * dev / (math.sqrt(5 / 3) + 0.5) + b)
    _close(oracle.layer_norm(x, a, b, kind=1, eps=0.75)[0], a * dev / math.sqrt(5 / 4 + 0.75) + b)


def pin_layer_norm_torch_layer_and_invariants():
    """Kind 1 is torch's layer norm (float64 CPU); the two kinds differ by
    sqrt((D-1)/D) when eps = 0; both ignore a constant shift of the row."""
    import torch
    r = _rng(61)
    x = r.standard_normal((5, 7, 24)) * 3 + 1
    a, b = r.standard_normal(24), r.standard_normal(24)
    ref = torch.nn.functional.layer_norm(torch.tensor(x), (24,), torch.tensor(a), torch.tensor(b), eps=1e-5)
    _close(oracle.layer_norm(x, a, b, kind=1, eps=1e-5), ref.numpy())
    _close(oracle.layer_norm(x, kind=0, eps=0.0), oracle.layer_norm(x, kind=1, eps=0.0) * math.sqrt(23 / 24))
    for kind in (0, 1):
        _close(oracle.layer_norm(x + 7.25, a, b, kind=kind), oracle.layer_norm(x, a, b, kind=kind), 1e-11)


def pin_sublayer_residual_closed_forms():
    """With a zero output projection the sublayer returns x + b_O; with one
    head, identity projections and a single position it returns
    x + norm(x) (attention over one key returns its value)."""
    r = _rng(62)
    B, L, D, h = 2, 5, 8, 2
    x = r.standard_normal((B, L, D))
    w = [r.standard_normal((D, D)) for _ in range(3)]
    bo = r.standard_normal(D)
    out = oracle.mha_sublayer(x, *w, np.zeros((D, D)), b_o=bo, h=h, ln_kind=1, ln_eps=1e-5)
    _close(out, x + bo)
    x1 = r.standard_normal((3, 1, D))
    g, bb = r.standard_normal(D), r.standard_normal(D)
    eye = np.eye(D)
    out = oracle.mha_sublayer(x1, eye, eye, eye, eye, h=1, ln_gain=g, ln_bias=bb)
    _close(out, x1 + oracle.layer_norm(x1, g, bb, kind=0, eps=1e-6), 1e-12)


def pin_row_subset_consistent():
    r = _rng(37)
    x = r.standard_normal((2, 9, 16))
    ws = [r.standard_normal((16, 16)) * 0.3 for _ in range(4)]
    full = oracle.mha(x, x, *ws, h=4, valid_lens=[5, 9], causal=True)
    sub = oracle.mha(x, x, *ws, h=4, valid_lens=[5, 9], causal=True, rows=[8, 0, 4])
    _close(sub, full[:, [8, 0, 4]], 1e-13)


# ---------------------------------------------------------------------------
# MHA identities
# ---------------------------------------------------------------------------
def pin_mha_single_head_identity_is_sdpa():
    r = _rng(41)
    B, L, D = 2, 7, 8
    x = r.standard_normal((B, L, D))
    I = np.eye(D)
    out = oracle.mha(x, x, I, I, I, I, h=1, valid_lens=[3, 7], causal=True)
    ref = oracle.sdpa(x[:, None], x[:, None], x[:, None], valid_lens=[3, 7], causal=True)[:, 0]
    _close(out, ref, 1e-13)


def pin_mha_output_is_sum_over_heads():
    r = _rng(42)
    B, Lq, Lk, D, h = 2, 5, 6, 12, 3
    dk = D // h
    xq, xkv = r.standard_normal((B, Lq, D)), r.standard_normal((B, Lk, D))
    wq, wk, wv, wo = (r.standard_normal((D, D)) * 0.3 for _ in range(4))
    bo = r.standard_normal(D)
    out = oracle.mha(xq, xkv, wq, wk, wv, wo, b_o=bo, h=h, valid_lens=[2, 6])
    acc = np.zeros_like(out) + bo
    for hd in range(h):
        sl = slice(hd * dk, (hd + 1) * dk)
        qh = (xq @ wq[sl].T)[:, None]
        kh = (xkv @ wk[sl].T)[:, None]
        vh = (xkv @ wv[sl].T)[:, None]
        oh = oracle.sdpa(qh, kh, vh, valid_lens=[2, 6])[:, 0]
        acc += oh @ wo[:, sl].T
    _close(out, acc, 1e-12)


def pin_linear_orientation():
    """y = x W^T + b with W stored [out, in]: a brute-force 2x3 case."""
    x = np.array([[1.0, 2.0, 3.0]])
    w = np.array([[1.0, 0.0, 0.0], [0.0, 1.0, 1.0]])
    b = np.array([10.0, 20.0])
    _close(oracle.linear(x, w, b), [[11.0, 25.0]], 0.0)


# ---------------------------------------------------------------------------
# independent library routines (torch, float64, CPU)
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def pin_sdpa_vs_torch():
    torch = _torch()
    r = _rng(51)
    B, h, Lq, Lk, d = 3, 4, 13, 13, 16
    q, k, v = (r.standard_normal((B, h, L, d)) for L in (Lq, Lk, Lk))
    vl = np.array([13, 5, 1])
    for causal in (False, True):
        o = oracle.sdpa(q, k, v, valid_lens=vl, causal=causal)
        j = np.arange(Lk)
        allowed = j[None, None, :] < vl[:, None, None]
        if causal:
            allowed = allowed & (j[None, None, :] <= np.arange(Lq)[None, :, None])
        mask = torch.from_numpy(allowed[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask).numpy()
        _close(o, ref, 1e-13)


def _torch_mha(xq, xkv, ws, bs, h, vl, causal, bf16_stages=False):
    torch = _torch()
    F = torch.nn.functional
    T = lambda a: None if a is None else torch.from_numpy(np.asarray(a, dtype=np.float64))
    xq_t, xkv_t = T(xq), T(xkv)
    B, Lq, D = xq.shape
    Lk = xkv.shape[1]
    if not bf16_stages:
        kpm = None
        if vl is not None:
            kpm = torch.arange(Lk)[None, :] >= torch.from_numpy(np.asarray(vl))[:, None]
        am = None
        if causal:
            am = torch.triu(torch.ones(Lq, Lk, dtype=torch.bool), diagonal=1)
        zero = torch.zeros(D, dtype=torch.float64)
        bias = torch.cat([T(b) if b is not None else zero for b in bs[:3]])
        out, _ = F.multi_head_attention_forward(
            xq_t.transpose(0, 1), xkv_t.transpose(0, 1), xkv_t.transpose(0, 1), D, h,
            torch.cat([T(w) for w in ws[:3]]), bias, None, None, False, 0.0,
            T(ws[3]), T(bs[3]) if bs[3] is not None else zero, training=False,
            key_padding_mask=kpm, need_weights=False, attn_mask=am)
        return out.transpose(0, 1).numpy()
    rb = lambda t: t.to(torch.bfloat16).to(torch.float64)
    q = rb(F.linear(xq_t, T(ws[0]), T(bs[0])))
    k = rb(F.linear(xkv_t, T(ws[1]), T(bs[1])))
    v = rb(F.linear(xkv_t, T(ws[2]), T(bs[2])))
    dk = D // h
    sp = lambda t: t.view(B, -1, h, dk).transpose(1, 2)
    allowed = torch.ones(B, 1, Lq, Lk, dtype=torch.bool)
    if vl is not None:
        allowed &= (torch.arange(Lk)[None, :] < torch.from_numpy(np.asarray(vl))[:, None])[:, None, None, :]
    if causal:
        allowed &= torch.tril(torch.ones(Lq, Lk, dtype=torch.bool))[None, None]
    o = F.scaled_dot_product_attention(sp(q), sp(k), sp(v), attn_mask=allowed)
    o = rb(o.transpose(1, 2).reshape(B, Lq, D))
    return F.linear(o, T(ws[3]), T(bs[3])).numpy()


def pin_mha_vs_torch():
    """Whole MHA forward against torch's own multi-head attention in float64:
    pins the weight orientation, the head split/merge order, the per-head
    scale, the shared key-padding mask and the output projection."""
    r = _rng(52)
    for (B, Lq, Lk, D, h, causal, vl) in [(2, 9, 9, 32, 4, True, [9, 4]),
                                          (3, 6, 11, 24, 3, False, [11, 2, 7]),
                                          (2, 8, 8, 16, 2, False, None)]:
        xq = r.standard_normal((B, Lq, D))
        xkv = xq if Lq == Lk and causal else r.standard_normal((B, Lk, D))
        ws = [r.standard_normal((D, D)) / math.sqrt(D) for _ in range(4)]
        bs = [r.standard_normal(D) * 0.1 for _ in range(4)]
        out = oracle.mha(xq, xkv, *ws, *bs, h=h, valid_lens=vl, causal=causal)
        ref = _torch_mha(xq, xkv, ws, bs, h, vl, causal)
        _close(out, ref, 1e-12)


def pin_mha_bf16_stages_vs_torch():
    """The bf16-storage mode: Q, K, V and the merged head output rounded to
    bf16 between steps, against the same reading written with torch's float64
    linear/SDPA and its bf16 conversion."""
    r = _rng(53)
    B, Lq, Lk, D, h = 2, 7, 10, 32, 4
    xq, xkv = r.standard_normal((B, Lq, D)), r.standard_normal((B, Lk, D))
    ws = [r.standard_normal((D, D)) / math.sqrt(D) for _ in range(4)]
    bs = [r.standard_normal(D) * 0.1 for _ in range(4)]
    out = oracle.mha(xq, xkv, *ws, *bs, h=h, valid_lens=[10, 3], bf16_stages=True)
    ref = _torch_mha(xq, xkv, ws, bs, h, [10, 3], False, bf16_stages=True)
    _close(out, ref, 1e-12)
    plain = oracle.mha(xq, xkv, *ws, *bs, h=h, valid_lens=[10, 3])
    assert np.max(np.abs(out - plain)) > 1e-4    # the rounding is really applied


def pin_round_bf16_vs_torch():
    torch = _torch()
    r = _rng(54)
    x = r.standard_normal(4000).astype(np.float32) * np.float32(10.0) ** r.integers(-30, 30, 4000)
    bits = x.view(np.uint32)
    ties = ((bits & 0xFFFF0000) | 0x8000).view(np.float32)[:500]      # exact halfway cases
    x = np.concatenate([x, ties, np.float32([0.0, -0.0, 1e-40, -3e-39, 3.39e38])])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def pin_lse_closed_forms():
    """The log of the softmax normaliser: zero queries score every key 0, so
    lse = log(number of allowed keys) (causal row i: log(i + 1); length n:
    log n); one allowed key gives exactly its scaled score; a row with every
    key masked has all scores equal to the fill: fill + log(Lk)."""
    r = _rng(60)
    B, h, L, d = 2, 2, 6, 8
    k = r.standard_normal((B, h, L, d))
    q0 = np.zeros((B, h, L, d))
    lc = oracle.sdpa_lse(q0, k, causal=True)
    _close(lc, np.broadcast_to(np.log(np.arange(1, L + 1)), lc.shape), 1e-15)
    lv = oracle.sdpa_lse(q0, k, valid_lens=[3, 5])
    _close(lv[0], np.full((h, L), math.log(3)), 1e-15)
    _close(lv[1], np.full((h, L), math.log(5)), 1e-15)
    q = r.standard_normal((B, h, L, d)) * 3
    l1 = oracle.sdpa_lse(q, k, valid_lens=[1, 1])
    _close(l1, np.einsum("bhid,bhd->bhi", q, k[:, :, 0]) / math.sqrt(d), 1e-13)
    lm = oracle.sdpa_lse(q, k, valid_lens=[0, 6])
    _close(lm[0], np.full((h, L), -1e9 + math.log(L)), 1e-6)


def pin_lse_vs_scipy_logsumexp_and_weights():
    """Against scipy's logsumexp over the allowed scores of random rows (per
    query lengths and the causal mask together), and exp(s - lse) equals the
    oracle's own weights on the allowed keys."""
    from scipy.special import logsumexp
    r = _rng(61)
    B, h, L, d = 2, 3, 9, 16
    q, k, v = (r.standard_normal((B, h, L, d)) * 2 for _ in range(3))
    vl = r.integers(1, L + 1, size=(B, L)).astype(np.int32)
    lse = oracle.sdpa_lse(q, k, valid_lens=vl, causal=True)
    _, p = oracle.sdpa(q, k, v, valid_lens=vl, causal=True, return_weights=True)
    for b in range(B):
        for hd in range(h):
            for i in range(L):
                n = min(vl[b, i], i + 1)
                s = q[b, hd, i] @ k[b, hd, :n].T / math.sqrt(d)
                _close(lse[b, hd, i], logsumexp(s), 1e-13)
                _close(np.exp(s - lse[b, hd, i]), p[b, hd, i, :n], 1e-13)


# ---------------------------------------------------------------------------
# gradients of the multi-head layer
# ---------------------------------------------------------------------------
_GRADS = ("dx_q", "dx_kv", "dw_q", "dw_k", "dw_v", "dw_o", "db_q", "db_k", "db_v", "db_o")


def _mha_case(r, B, Lq, Lk, D):
    xq, xkv = r.standard_normal((B, Lq, D)), r.standard_normal((B, Lk, D))
    ws = [r.standard_normal((D, D)) / math.sqrt(D) for _ in range(4)]
    bs = [r.standard_normal(D) * 0.1 for _ in range(4)]
    g = r.standard_normal((B, Lq, D))
    return xq, xkv, ws, bs, g


def _torch_mha_grads(xq, xkv, ws, bs, g, h, vl, causal, bf16_stages=False):
    """torch float64 CPU autograd of sum(MHA(xq, xkv) * g) through its own
    multi-head attention (in fp64) or, for the bf16-storage reading, through
    linear / scaled_dot_product_attention with a rounding step that rounds
    the value going forward and its gradient going back."""
    torch = _torch()
    F = torch.nn.functional
    leaf = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
    txq, txkv = leaf(xq), leaf(xkv)
    tw = [leaf(w) for w in ws]
    tb = [leaf(b) for b in bs]
    B, Lq, D = xq.shape
    Lk = xkv.shape[1]
    if not bf16_stages:
        kpm = None
        if vl is not None:
            kpm = torch.arange(Lk)[None, :] >= torch.tensor(np.asarray(vl))[:, None]
        am = torch.triu(torch.ones(Lq, Lk, dtype=torch.bool), diagonal=1) if causal else None
        out, _ = F.multi_head_attention_forward(
            txq.transpose(0, 1), txkv.transpose(0, 1), txkv.transpose(0, 1), D, h,
            torch.cat(tw[:3]), torch.cat(tb[:3]), None, None, False, 0.0, tw[3], tb[3], training=False,
            key_padding_mask=kpm, need_weights=False, attn_mask=am)
        out = out.transpose(0, 1)
    else:
        class Round(torch.autograd.Function):
            @staticmethod
            def forward(ctx, x):
                return x.to(torch.bfloat16).to(torch.float64)

            @staticmethod
            def backward(ctx, gr):
                return gr.to(torch.bfloat16).to(torch.float64)

        q = Round.apply(F.linear(txq, tw[0], tb[0]))
        k = Round.apply(F.linear(txkv, tw[1], tb[1]))
        v = Round.apply(F.linear(txkv, tw[2], tb[2]))
        dk = D // h
        sp = lambda t: t.view(B, -1, h, dk).transpose(1, 2)
        allowed = torch.ones(B, 1, Lq, Lk, dtype=torch.bool)
        if vl is not None:
            allowed &= (torch.arange(Lk)[None, :] < torch.tensor(np.asarray(vl))[:, None])[:, None, None, :]
        if causal:
            allowed &= torch.tril(torch.ones(Lq, Lk, dtype=torch.bool))[None, None]
        o = F.scaled_dot_product_attention(sp(q), sp(k), sp(v), attn_mask=allowed)
        o = Round.apply(o.transpose(1, 2).reshape(B, Lq, D))
        out = F.linear(o, tw[3], tb[3])
    (out * torch.tensor(g)).sum().backward()
    t = {"dx_q": txq.grad, "dx_kv": txkv.grad}
    for n, w, b in zip("qkvo", tw, tb):
        t["dw_" + n] = w.grad
        t["db_" + n] = b.grad
    return {n: a.numpy() for n, a in t.items()}


def pin_mha_backward_vs_torch_autograd():
    """Every gradient of the multi-head layer against torch's float64
    autograd through its own multi-head attention: causal self-attention with
    padding, cross-attention with padding, and no mask."""
    r = _rng(61)
    for (B, Lq, Lk, D, h, causal, vl) in [(2, 7, 7, 16, 2, True, [7, 3]),
                                          (2, 5, 9, 24, 3, False, [9, 2]),
                                          (1, 6, 4, 8, 1, False, None)]:
        xq, xkv, ws, bs, g = _mha_case(r, B, Lq, Lk, D)
        got = oracle.mha_backward(xq, xkv, *ws, g, *bs[:3], h=h, valid_lens=vl, causal=causal)
        ref = _torch_mha_grads(xq, xkv, ws, bs, g, h, vl, causal)
        for n in _GRADS:
            _close(got[n], ref[n], 1e-11)


def pin_mha_backward_bf16_stages_vs_torch():
    """The bf16-storage reading of the backward (Q, K, V, the merged heads and
    the gradients of those four rounded to bf16 where they are made) against
    torch autograd with a rounding step at the same four places."""
    r = _rng(62)
    B, Lq, Lk, D, h = 2, 6, 8, 16, 2
    xq, xkv, ws, bs, g = _mha_case(r, B, Lq, Lk, D)
    got = oracle.mha_backward(xq, xkv, *ws, g, *bs[:3], h=h, valid_lens=[8, 5], bf16_stages=True)
    ref = _torch_mha_grads(xq, xkv, ws, bs, g, h, [8, 5], False, bf16_stages=True)
    plain = oracle.mha_backward(xq, xkv, *ws, g, *bs[:3], h=h, valid_lens=[8, 5])
    for n in _GRADS:
        _close(got[n], ref[n], 1e-10)
    # the rounding is really applied, on both sides of the attention
    assert np.max(np.abs(got["dw_o"] - plain["dw_o"])) > 1e-5
    assert np.max(np.abs(got["dw_q"] - plain["dw_q"])) > 1e-5


def pin_mha_backward_finite_differences():
    """Each gradient element equals the central difference of
    sum(mha(...) * g) in that input, weight or bias (the output bias
    included), for cross-attention with padding and causal self-attention
    fed from separate query and key/value inputs."""
    r = _rng(63)
    for (B, Lq, Lk, D, h, causal, vl) in [(2, 3, 4, 4, 2, False, [4, 2]), (1, 3, 3, 4, 2, True, None)]:
        xq, xkv, ws, bs, g = _mha_case(r, B, Lq, Lk, D)
        got = oracle.mha_backward(xq, xkv, *ws, g, *bs[:3], h=h, valid_lens=vl, causal=causal)
        loss = lambda: np.sum(oracle.mha(xq, xkv, *ws, *bs, h=h, valid_lens=vl, causal=causal) * g)
        named = [("dx_q", xq), ("dx_kv", xkv)] + [("dw_" + n, w) for n, w in zip("qkvo", ws)] + \
                [("db_" + n, b) for n, b in zip("qkvo", bs)]
        for name, x in named:
            fd = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                e = 1e-6
                x[idx] += e
                up = loss()
                x[idx] -= 2 * e
                dn = loss()
                x[idx] += e
                fd[idx] = (up - dn) / (2 * e)
            _close(got[name], fd, 1e-7)


def pin_mha_backward_single_key_closed_form():
    """With one key the weights are 1 whatever the scores, so the layer is
    out_i = (x_kv W_v^T + b_v) W_o^T + b_o for every query: the query and key
    projections get no gradient, and the rest follow from two linear layers."""
    r = _rng(64)
    B, Lq, D, h = 2, 5, 8, 2
    xq, xkv, ws, bs, g = _mha_case(r, B, Lq, 1, D)
    got = oracle.mha_backward(xq, xkv, *ws, g, *bs[:3], h=h)
    for n in ("dx_q", "dw_q", "dw_k", "db_q", "db_k"):
        _close(got[n], np.zeros_like(got[n]))
    v = xkv[:, 0] @ ws[2].T + bs[2]                 # [B, D], the one value row
    gsum = g.sum(axis=1)                            # [B, D]
    dv = gsum @ ws[3]                               # gradient of each batch's value row
    _close(got["db_o"], g.sum(axis=(0, 1)))
    _close(got["dw_o"], gsum.T @ v)
    _close(got["db_v"], dv.sum(axis=0))
    _close(got["dw_v"], dv.T @ xkv[:, 0])
    _close(got["dx_kv"][:, 0], dv @ ws[2])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
