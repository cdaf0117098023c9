"""GPU parity of the backward at full workload sizes, in the configuration
bench.py's training step times (lsh_attention_fwd_train + lsh_attention_bwd
over the whole workload).

The oracle's backward over a 64K-token slice takes minutes, so it runs only
at sampled positions: ``oracle.backward_rows`` gives the rows of dqk and dv
that the full oracle backward gives there (pinned to it on the CPU), on its
own hash and sort of the slice. Slices (batch, head) are sampled, and a slice
is compared only where the GPU's bucket ids equal the oracle's everywhere (a
near-tie decided the other way changes which keys a position sees); at least
one slice must be compared. Sampled positions include the first and last
sorted slot of round 0 (the chunk with no look-back and the last chunk).
Bar, bf16 I/O: 2e-2 times the largest entry of the sampled reference rows.
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
TOL = {"fp32": 1e-4, "bf16": 2e-2}

# 500 chunks of 64 per (head, round): the backward's workgroups take runs of
# 32 chunks there, the last one ragged (20 chunks); 64 at 64K tokens
# 520 chunks, 128 segments: runs of 64 chunks with a ragged last run (8)
EXTRA = {"l32000_h8_d128_nh8": workloads.Workload("l32000_h8_d128_nh8", 1, 8, 32000, 128,
                                                  "bf16", 1000, 8, 64, True, 1017),
         "l33280_h16_d64_nh8": workloads.Workload("l33280_h16_d64_nh8", 1, 16, 33280, 64,
                                                  "bf16", 1040, 8, 64, True, 1018),
         # past the packed keys' 20-bit position field: plain permutation
         "l1m_h1_d64_nh2": workloads.Workload("l1m_h1_d64_nh2", 1, 1, (1 << 20) + 64, 64,
                                              "bf16", 64, 2, 64, True, 1019)}

# (workload, key_norm, per-head rotations)
CASES = [
    ("l64k_h8_d128_nh8", False, False),
    ("l32000_h8_d128_nh8", False, False),
    ("l33280_h16_d64_nh8", False, False),
    ("l1m_h1_d64_nh2", False, False),
    ("l64k_h8_d128_nh8", True, False),
    ("l64k_h8_d128_nh8", False, True),
    ("b8_h8_l4k_nh4", False, False),
    ("skewed_l16k_nh8", False, False),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lsh.load_library()


@pytest.mark.parametrize("name,key_norm,per_head", CASES,
                         ids=[f"{n}{'_keynorm' if k else ''}{'_perhead' if p else ''}"
                              for n, k, p in CASES])
def test_fullsize_backward_sampled_rows(name, key_norm, per_head):
    w = EXTRA[name] if name in EXTRA else workloads.WORKLOADS[name]
    qk, v, R = workloads.make_inputs(w)
    if per_head:
        R = np.random.default_rng(w.seed + 1).standard_normal(
            (w.H, w.n_hashes, w.d, w.n_buckets // 2), dtype=np.float32)
    rng = np.random.default_rng(w.seed + 17)
    g = workloads.round_to_bf16(rng.standard_normal(qk.shape, dtype=np.float32))
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qk_t = torch.from_numpy(qk).to(DEV, dt)
    v_t = torch.from_numpy(v).to(DEV, dt)
    R_t = torch.from_numpy(R).to(DEV)
    g_t = torch.from_numpy(g).to(DEV, dt)
    out, state = lsh.attention_fwd_train(qk_t, v_t, R_t, w.n_buckets, w.chunk_len, w.causal,
                                         key_norm=key_norm)
    dqk, dv = lsh.attention_bwd(qk_t, v_t, out, g_t, state, w.n_buckets, w.n_hashes,
                                w.chunk_len, w.causal, key_norm=key_norm)
    gb, _ = lsh.hash(qk_t, R_t, w.n_buckets)
    torch.cuda.synchronize()
    gb = gb.cpu().numpy()
    got_dqk = dqk.float().cpu().numpy()
    got_dv = dv.float().cpu().numpy()
    assert np.isfinite(got_dqk).all() and np.isfinite(got_dv).all()

    B, H, L = w.B, w.H, w.L
    n_bh = min(B * H, 2 if L >= 65536 else 3)
    bhs = rng.choice(B * H, size=n_bh, replace=False)
    worst, compared = 0.0, 0
    for bh in bhs:
        b, h = divmod(int(bh), H)
        Rh = R[h] if per_head else R
        x = np.ascontiguousarray(qk[b, h], dtype=np.float64)
        ref_b, _ = oracle.hash(x, Rh, w.n_buckets)
        if not np.array_equal(gb[b, h], ref_b):
            continue                  # a near-tie decided the other way
        perm0, _ = oracle.sort(ref_b[0])
        toks = set(int(t) for t in rng.choice(L, size=30, replace=False))
        toks |= {int(perm0[0]), int(perm0[L - 1])}
        toks = np.array(sorted(toks), dtype=np.int64)
        ref_dqk, ref_dv = oracle.backward_rows(x, v[b, h], Rh, g[b, h], toks,
                                               w.n_buckets, w.chunk_len, w.causal,
                                               key_norm=key_norm)
        for got, ref in ((got_dqk[b, h][toks], ref_dqk), (got_dv[b, h][toks], ref_dv)):
            err = float(np.abs(got - ref).max()) / float(np.abs(ref).max())
            worst = max(worst, err)
            assert err <= TOL[w.dtype], (name, b, h, err)
        compared += 1
    print(f"{name} key_norm={key_norm} per_head={per_head}: {compared}/{n_bh} slices x "
          f"{len(toks)} rows, worst relative error {worst:.2e}")
    assert compared >= 1
