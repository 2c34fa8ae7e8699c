"""The benchmark's algorithmic work counts (CPU only): the number of pairs
the masks allow, and the flops and bytes derived from it, against brute-force
counts of the mask rule on small workloads and the closed forms of the full
sizes.  The headline rate is this count divided by the measured time, so a
wrong count would be a wrong headline."""

import numpy as np
import pytest

import bench
import workloads


def brute_pairs(B, h, Lq, Lk, causal, lens):
    """Allowed (batch, head, query, key) pairs by the rule itself: key j
    counts for query i when j < the valid length (and j <= i under the
    causal rule); a row with no allowed key weights all Lk keys."""
    total = 0
    for b in range(B):
        vl = Lk if lens is None else int(lens[b])
        for i in range(Lq):
            allowed = sum(1 for j in range(Lk) if j < min(vl, Lk) and (not causal or j <= i))
            total += Lk if (vl <= 0 or allowed == 0) else allowed
    return total * h


@pytest.mark.parametrize("causal,lens", [
    (False, None), (True, None), (False, [0, 3, 40]), (True, [1, 17, 99]), (True, [0, 40, 5]),
])
def test_allowed_pairs_matches_the_mask_rule(causal, lens):
    B, h, Lq, Lk = 3, 2, 23, (23 if causal else 31)
    w = workloads.Workload("t", "sdpa", "bf16", B, Lq, Lk, h, 64, causal, None)
    vl = None if lens is None else np.array(lens, dtype=np.int32)
    assert bench.allowed_pairs(w, vl) == brute_pairs(B, h, Lq, Lk, causal, vl)


def test_headline_flops_closed_form():
    """Long causal SDPA B4 h16 L4096 d_k 64: 4 d_k flops for each of the
    L(L+1)/2 allowed pairs of every (batch, head)."""
    w = workloads.BY_NAME["sdpa_long_causal"]
    flops, byts = bench.sdpa_alg(w, None, 2, 2)
    assert flops == 4 * 64 * 4 * 16 * 4096 * 4097 // 2 == 137472507904
    # Q, K, V read once and O written once, bf16: 4 x 4 x 16 x 4096 x 64 x 2 bytes
    assert byts == 4 * (4 * 16 * 4096 * 64 * 2) == 134217728


def test_decode_bytes_count_every_valid_cached_row_once():
    w = workloads.BY_NAME["decode_step"]
    lens = np.array([0, 1, 300, w.Lk, w.Lk + 50], dtype=np.int32)
    w5 = workloads.Workload(w.name, w.kind, w.dtype, 5, 1, w.Lk, w.h, w.d_k, False, None)
    flops, byts = bench.decode_alg(w5, lens)
    rows = w.Lk + 1 + 300 + w.Lk + w.Lk          # a length <= 0 reads the whole cache (uniform weights)
    assert flops == 4 * w.d_k * w.h * rows
    assert byts == w.h * w.d_k * 2 * (2 * rows + 2 * 5)


def test_gemm_counts():
    flops, byts = bench.gemm_alg(100, 64, 128, 3, 2, 4)
    assert flops == 2 * 100 * 64 * 128 * 3
    assert byts == 3 * ((100 * 128 + 64 * 128 + 64) * 2 + 100 * 64 * 4)


def test_workload_masks_at_full_size_match_brute_force_on_a_slice():
    """The decoder workload's counted pairs, per sequence, against the rule on
    that sequence's length (the full brute force would take minutes)."""
    w = workloads.BY_NAME["decoder_causal"]
    inp = workloads.make_inputs(w)
    for b in (0, 7, 63):
        one = workloads.Workload("t", "mha", "bf16", 1, w.Lq, w.Lk, 1, w.d_k, True, None)
        vl = inp.valid_lens[b:b + 1]
        v = int(vl[0])
        closed = sum(min(i + 1, v) for i in range(w.Lq))
        assert bench.allowed_pairs(one, vl) == closed
