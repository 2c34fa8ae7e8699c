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
