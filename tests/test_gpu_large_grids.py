"""Shapes whose segment or rotation-round counts pass 65535, the most one
grid dimension holds: the kernels split such counts over two dimensions.

  * the sort with B*H*n_hashes = 131072 segments;
  * the forward with 65536 segments, matrix-core (bf16) and vector (fp32)
    chunk kernels;
  * per-head rotations with H*n_hashes = 69632 R rounds (the R preparation
    and the re-decision scan are indexed by R round).
Each is checked against the oracle on sampled segments or slices, and every
segment's permutation is checked to be one.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from oracle import oracle

lsh = pytest.importorskip("lsh_attention_fp32_amd")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lsh.load_library()


def test_sort_past_65535_segments():
    B, H, nh, L, nb = 16, 8, 1024, 64, 16
    rng = np.random.default_rng(77)
    b = rng.integers(0, nb, (B, H, nh, L)).astype(np.int32)
    perm, inv = lsh.sort(torch.from_numpy(b).to(DEV), nb)
    perm, inv = perm.cpu().numpy(), inv.cpu().numpy()
    flat_p = perm.reshape(-1, L)
    flat_i = inv.reshape(-1, L)
    flat_b = b.reshape(-1, L)
    # every segment: a permutation, (bucket, position) increasing, inv its inverse
    assert np.array_equal(np.sort(flat_p, axis=1), np.broadcast_to(np.arange(L), flat_p.shape))
    key = np.take_along_axis(flat_b, flat_p, axis=1).astype(np.int64) * L + flat_p
    assert np.all(np.diff(key, axis=1) > 0)
    assert np.array_equal(np.take_along_axis(flat_i, flat_p, axis=1),
                          np.broadcast_to(np.arange(L), flat_p.shape))
    segs = flat_p.shape[0]
    for s in list(rng.choice(segs, 200, replace=False)) + [65534, 65535, 65536, segs - 1]:
        p_ref, i_ref = oracle.sort(flat_b[s])
        assert np.array_equal(flat_p[s], p_ref) and np.array_equal(flat_i[s], i_ref)
    print(f"sort: {segs} segments, all permutations valid, 204 against the oracle")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_forward_past_65535_segments(dtype):
    w = workloads.Workload(f"segs65536_{dtype}", 4, 16, 64, 64, dtype, 4, 1024, 64, True, 78)
    qk, v, R = workloads.make_inputs(w)
    dt = torch.float32 if dtype == "fp32" else torch.bfloat16
    out = lsh.attention_fwd(torch.from_numpy(qk).to(DEV, dt), torch.from_numpy(v).to(DEV, dt),
                            torch.from_numpy(R).to(DEV), w.n_buckets, w.chunk_len, w.causal)
    out = out.float().cpu().numpy()
    assert np.isfinite(out).all()
    tol = 1e-4 if dtype == "fp32" else 2e-2
    worst, compared = 0.0, 0
    for b, h in ((0, 0), (3, 15), (2, 7)):
        ref, ex = oracle.forward(qk[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], R, w.n_buckets,
                                 w.chunk_len, w.causal, return_all=True)
        if (ex["margin"] < 1e-9).any():
            continue   # a near-tie could be decided either way
        worst = max(worst, float(np.abs(out[b, h] - ref[0, 0]).max()))
        compared += 1
    print(f"forward {dtype}: 65536 segments, {compared} slices compared, max err {worst:.3e}")
    assert compared >= 1 and worst <= tol


def test_per_head_rotations_past_65535_rounds():
    B, H, L, d, nb, nh = 1, 17, 64, 64, 4, 4096
    rng = np.random.default_rng(79)
    qk = workloads.round_to_bf16(rng.standard_normal((B, H, L, d), dtype=np.float32))
    R = rng.standard_normal((H, nh, d, nb // 2), dtype=np.float32)
    buckets, _ = lsh.hash(torch.from_numpy(qk).to(DEV, torch.bfloat16), torch.from_numpy(R).to(DEV),
                          nb)
    buckets = buckets.cpu().numpy()
    for h in (0, 8, 16):
        ref, margin = oracle.hash(qk[0, h], R[h], nb)
        assert not np.any((buckets[0, h] != ref) & (margin >= 1e-9))
    print(f"per-head hash: {H * nh} R rounds, heads 0, 8, 16 against the oracle")
