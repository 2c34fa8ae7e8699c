"""sdpa_decode_noalloc (the allocation-free decoding step) against
sdpa_decode with a caller workspace: same kernels, so the outputs must be
identical.  Two calls in a row on one GPU, the second smaller, so the second
reuses the library's array with the first call's partials still in it."""
import ctypes

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu


def _step(B, h, L, seed):
    import torch
    rng = np.random.Generator(np.random.PCG64(seed))
    q = torch.from_numpy(workloads._finish(rng.standard_normal((B, h, 64)), "bf16")).cuda().to(torch.bfloat16)
    k, v = (torch.from_numpy(workloads._finish(rng.standard_normal((B, h, L, 64)), "bf16")).cuda().to(torch.bfloat16)
            for _ in range(2))
    lens = rng.integers(1, L + 1, size=B).astype(np.int32)
    lens[0] = L
    if B > 2:
        lens[1] = 0                              # the fully masked row
    return q, k, v, torch.from_numpy(lens).cuda()


def _call_noalloc(lib, q, k, v, lens, out):
    from transformer_head_scaled_sdpa_amd import _lib
    import torch
    B, h, _ = q.shape
    L = k.shape[2]
    S3 = lambda t: _lib.Strides(t.stride(0), t.stride(1), 0)
    S4 = lambda t: _lib.Strides(*t.stride()[:3])
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    return lib.sdpa_decode_noalloc(_lib.MHA_BF16, _lib.MHA_F32 if out.dtype == torch.float32 else _lib.MHA_BF16,
                                   p(q), S3(q), p(k), S4(k), p(v), S4(v), p(out), S3(out), B, h, L, 64, 64,
                                   p(lens), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("out_f32", [False, True])
def test_noalloc_matches_workspace_entry_point(out_f32):
    import torch
    import transformer_head_scaled_sdpa_amd as mha
    from transformer_head_scaled_sdpa_amd import _lib
    lib = _lib.load()
    odt = torch.float32 if out_f32 else torch.bfloat16
    # The first step needs split partials (3000 positions: 12 slices of 256
    # keys); the second is smaller (700 positions, fewer heads and batches).
    for B, h, L, seed in ((8, 4, 3000, 11), (3, 2, 700, 12)):
        q, k, v, lens = _step(B, h, L, seed)
        out = torch.full((B, h, 64), float("nan"), dtype=odt, device="cuda")
        st = _call_noalloc(lib, q, k, v, lens, out)
        assert st == _lib.MHA_OK, _lib.status_string(st)
        ref = mha.sdpa_decode(q, k, v, lens, out_dtype=odt)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
        assert torch.equal(out, ref), f"B{B} h{h} L{L}: max diff {(out.float() - ref.float()).abs().max().item()}"


def test_noalloc_refuses_steps_beyond_its_array():
    import torch
    from transformer_head_scaled_sdpa_amd import _lib
    lib = _lib.load()
    q, k, v, lens = _step(2, 2, 64, 13)
    out = torch.empty((2, 2, 64), dtype=torch.bfloat16, device="cuda")
    # B*h*ceil(L/256) partials of 264 bytes: 64 * 8 * 256 slices exceed 16 MiB.
    # The sizes are checked before any pointer is used.
    from transformer_head_scaled_sdpa_amd import _lib as L_
    S = L_.Strides
    st = lib.sdpa_decode_noalloc(L_.MHA_BF16, L_.MHA_BF16, ctypes.c_void_p(q.data_ptr()), S(128, 64, 0),
                                 ctypes.c_void_p(k.data_ptr()), S(0, 0, 64), ctypes.c_void_p(v.data_ptr()),
                                 S(0, 0, 64), ctypes.c_void_p(out.data_ptr()), S(128, 64, 0), 64, 8, 65536, 64, 64,
                                 ctypes.c_void_p(lens.data_ptr()), None)
    assert st == L_.MHA_EWORKSPACE
