"""GPU parity of per-head rotations (R [H, n_hashes, d, n_buckets/2],
LSH_PER_HEAD_R) against the oracle.

Head h hashes with R[h] in every batch. Bars as for the shared-R method:
bucket ids equal to the oracle's wherever its margin is >= 1e-5; outputs
max-abs 1e-4 (fp32 I/O) / 2e-2 (bf16 I/O) and gradients relative to the
slice's largest entry on slices whose GPU bucket ids equal the oracle's.
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lsh.load_library()


def _inputs(dtype, B, H, L, d, nb, nh, seed, zero_rows=()):
    rng = np.random.default_rng(seed)
    qk = rng.standard_normal((B, H, L, d), dtype=np.float32)
    v = rng.standard_normal((B, H, L, d), dtype=np.float32)
    R4 = rng.standard_normal((H, nh, d, nb // 2), dtype=np.float32)
    for b, h, t in zero_rows:
        qk[b, h, t] = 0.0        # every column ties: the full-scan re-decision
    if dtype == "bf16":
        qk = workloads.round_to_bf16(qk)
        v = workloads.round_to_bf16(v)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return qk, v, R4, torch.from_numpy(qk).to(DEV, dt), torch.from_numpy(v).to(DEV, dt), \
        torch.from_numpy(R4).to(DEV)


def _oracle_buckets(qk, R4, nb):
    B, H, L, _ = qk.shape
    nh = R4.shape[1]
    b = np.empty((B, H, nh, L), np.int32)
    mg = np.empty((B, H, nh, L))
    for bi in range(B):
        for h in range(H):
            b[bi, h], mg[bi, h] = oracle.hash(qk[bi, h], R4[h], nb)
    return b, mg


# L values that are not multiples of a hash workgroup's 256 tokens make the
# per-head workgroups end early
HASH_CASES = [("bf16", 2, 3, 320, 64, 16, 2), ("bf16", 1, 4, 1024, 128, 1024, 2),
              ("bf16", 2, 2, 999, 64, 64, 3), ("fp32", 2, 3, 320, 64, 16, 2),
              ("fp32", 1, 2, 512, 128, 64, 2)]


@pytest.mark.parametrize("dtype,B,H,L,d,nb,nh", HASH_CASES)
def test_hash_per_head_matches_oracle(dtype, B, H, L, d, nb, nh):
    qk, v, R4, qk_t, v_t, R_t = _inputs(dtype, B, H, L, d, nb, nh, 500 + L,
                                        zero_rows=[(0, H - 1, 3), (B - 1, 0, L - 1)])
    gb, refined = lsh.hash(qk_t, R_t, nb)
    ref, margin = _oracle_buckets(qk, R4, nb)
    gb = gb.cpu().numpy()
    differ = gb != ref
    assert not np.any(differ & (margin >= 1e-5)), "bucket ids differ away from near-ties"
    assert gb[0, H - 1, :, 3].tolist() == [0] * nh and gb[B - 1, 0, :, L - 1].tolist() == [0] * nh
    assert refined >= 2 * nh
    # the heads' own rotations are used: head 0's R for every head differs
    shared, _ = lsh.hash(qk_t, R_t[0].contiguous(), nb)
    assert not torch.equal(shared.cpu(), torch.from_numpy(gb)) or H == 1


def test_equal_heads_give_the_shared_result():
    qk, v, R4, qk_t, v_t, R_t = _inputs("bf16", 2, 3, 1024, 64, 64, 4, 510)
    R = R_t[1].contiguous()
    R_same = torch.stack([R] * 3).contiguous()
    a, _ = lsh.hash(qk_t, R, 64)
    b, _ = lsh.hash(qk_t, R_same, 64)
    assert torch.equal(a, b)
    oa = lsh.attention_fwd(qk_t, v_t, R, 64, 64, True)
    ob = lsh.attention_fwd(qk_t, v_t, R_same, 64, 64, True)
    assert torch.equal(oa, ob)


FWD_CASES = [("bf16", 2, 3, 1024, 64, 64, 4, 64, True), ("bf16", 1, 2, 2048, 128, 128, 3, 64, True),
             ("fp32", 2, 2, 768, 64, 16, 2, 64, False), ("bf16", 1, 2, 768, 128, 8, 2, 128, True)]


def _equal_slices(gb, rb):
    B, H = gb.shape[:2]
    return [(b, h) for b in range(B) for h in range(H) if np.array_equal(gb[b, h], rb[b, h])]


@pytest.mark.parametrize("dtype,B,H,L,d,nb,nh,m,causal", FWD_CASES)
def test_forward_and_backward_per_head_match_oracle(dtype, B, H, L, d, nb, nh, m, causal):
    qk, v, R4, qk_t, v_t, R_t = _inputs(dtype, B, H, L, d, nb, nh, 520 + L + d)
    ref, extra = oracle.forward(qk, v, R4, nb, m, causal, return_all=True)
    out = lsh.attention_fwd(qk_t, v_t, R_t, nb, m, causal)
    train, state = lsh.attention_fwd_train(qk_t, v_t, R_t, nb, m, causal)
    assert torch.equal(out, train)
    gb, _ = lsh.hash(qk_t, R_t, nb)
    slices = _equal_slices(gb.cpu().numpy(), extra["buckets"])
    assert slices
    got = out.float().cpu().numpy()
    worst = max(float(np.abs(got[b, h] - ref[b, h]).max()) for b, h in slices)
    assert worst <= TOL[dtype]
    g = np.random.default_rng(L).standard_normal(qk.shape, dtype=np.float32)
    if dtype == "bf16":
        g = workloads.round_to_bf16(g)
    dqk, dv = lsh.attention_bwd(qk_t, v_t, out, torch.from_numpy(g).to(DEV, qk_t.dtype), state,
                                nb, nh, m, causal)
    rq, rv = oracle.backward(qk, v, R4, g, nb, m, causal)
    gq, gv = dqk.float().cpu().numpy(), dv.float().cpu().numpy()
    for b, h in slices:
        for a, r in ((gq[b, h], rq[b, h]), (gv[b, h], rv[b, h])):
            assert float(np.abs(a - r).max()) / float(np.abs(r).max()) <= TOL[dtype]
    print(f"per-head {dtype} L={L}: forward worst {worst:.2e} over {len(slices)} slices")
