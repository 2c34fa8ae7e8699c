"""Tolerances and helpers shared by the GPU parity tests.

Floating-point bar (written here, used by every parity test):
  fp32 path : norm-wise relative error  max|g - o| / max|o|  <= 1e-5
  bf16 path : with s = max(1, rms(o)):  max|g - o| / s <= 2e-2  and
              mean|g - o| / s <= 2e-3
where g is the GPU result and o the fp64 oracle on the same (bf16-exact)
inputs.
"""
import numpy as np

FP32_REL = 1e-5
BF16_MAX = 2e-2
BF16_MEAN = 2e-3


def errors(gpu, ref):
    g = np.asarray(gpu, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    assert np.all(np.isfinite(g)), "non-finite values in the GPU result"
    d = np.abs(g - o)
    s = max(1.0, float(np.sqrt(np.mean(o * o))))
    return {
        "max_abs": float(d.max()),
        "mean_abs": float(d.mean()),
        "scale": s,
        "norm_rel": float(d.max() / max(np.abs(o).max(), 1e-300)),
    }


def assert_fp32(gpu, ref, what=""):
    e = errors(gpu, ref)
    assert e["norm_rel"] <= FP32_REL, f"{what}: fp32 norm-wise relative error {e}"
    return e


def assert_bf16(gpu, ref, what=""):
    e = errors(gpu, ref)
    assert e["max_abs"] / e["scale"] <= BF16_MAX, f"{what}: bf16 max error {e}"
    assert e["mean_abs"] / e["scale"] <= BF16_MEAN, f"{what}: bf16 mean error {e}"
    return e


# Gradients of the multi-head layer (bf16 path).  The path stores Q, K, V,
# the merged heads and the gradients of those four in bf16, each a relative
# rounding error uniform in +-2^-9 (rms 1.1e-3), and the attention backward
# multiplies bf16-rounded weights and ds; about six such steps in series
# give an rms relative error near 2.8e-3 and mean |error| near 2.2e-3 of the
# gradient's rms s, which the softmax Jacobian's cancellation (sum_j ds_ij
# = 0) raises further.  The storage roundings alone (the oracle's
# bf16-storage reading against its fp64 one) measure up to 3.4e-3 s (mean)
# and 2.7e-2 s (max) on the test cases.  Bar, against the fp64 oracle:
#   max |g - o| <= 4e-2 s  and  mean |g - o| <= 5e-3 s,
# with s = rms(o); a bias gradient takes the larger of its own rms and its
# layer's weight-gradient rms (a bias is a weight on an input fixed at 1, and
# the key bias's exact gradient is 0: softmax ignores a score shift shared by
# all keys).
# Input gradients vary in scale from row to row (under the causal mask an
# early key collects the attention of every later query), so they are held
# row by row: each row r with a nonzero reference keeps its norm-wise
# relative error ||g_r - o_r|| / ||o_r|| <= 2e-2 (the storage roundings
# alone reach 1.1e-2 on the test cases), and each sequence's mean error
# stays within GRAD_MEAN of its rows' rms.
GRAD_MAX = 4e-2
GRAD_MEAN = 5e-3
GRAD_ROW = 2e-2


def assert_grad_bf16(gpu, ref, scale, what=""):
    g = np.asarray(gpu, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values in the GPU result"
    d = np.abs(g - o)
    e = {"max_rel": float(d.max() / scale), "mean_rel": float(d.mean() / scale), "scale": float(scale)}
    assert e["max_rel"] <= GRAD_MAX, f"{what}: gradient max error {e}"
    assert e["mean_rel"] <= GRAD_MEAN, f"{what}: gradient mean error {e}"
    return e


def assert_grad_rows_bf16(gpu, ref, what=""):
    """Rows of an input gradient [L, D] (one sequence): padded rows, whose
    reference is exactly zero, must be exactly zero; the others take the
    row-wise bar and the sequence's mean bar."""
    g = np.asarray(gpu, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values in the GPU result"
    live = np.any(o != 0, axis=-1)
    assert np.all(g[~live] == 0), f"{what}: rows with a zero gradient are not zero"
    if not live.any():
        return {}
    d, ol = (g - o)[live], o[live]
    row = np.sqrt(np.sum(d * d, axis=-1) / np.sum(ol * ol, axis=-1))
    scale = float(np.sqrt(np.mean(ol * ol)))
    e = {"row_rel_max": float(row.max()), "mean_rel": float(np.mean(np.abs(d)) / scale), "scale": scale}
    assert e["row_rel_max"] <= GRAD_ROW, f"{what}: row-wise gradient error {e}"
    assert e["mean_rel"] <= GRAD_MEAN, f"{what}: gradient mean error {e}"
    return e


def to_device(x, dtype):
    """float32 numpy (bf16-exact when dtype is bf16) -> GPU tensor, exactly."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return t.to(dtype)


def to_host(t):
    return t.float().cpu().numpy().astype(np.float64)


def sample_rows(L, n_random, rng, tile=128):
    """Query rows that include tile edges, the first and the last row."""
    rows = {0, 1, L - 1, L - 2}
    for t in range(tile, L, tile):
        rows.update({t - 1, t, t + 1})
    rows = {r for r in rows if 0 <= r < L}
    extra = rng.choice(L, size=min(n_random, L), replace=False)
    rows.update(int(x) for x in extra)
    return np.array(sorted(rows), dtype=np.int32)
