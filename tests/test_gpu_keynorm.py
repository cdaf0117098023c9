"""GPU parity of key normalisation (LSH_KEY_NORM) against the oracle.

With the flag, the key side of every score is the unit vector x_j / |x_j|
(the query keeps its length); the hash and the sort are unchanged. The oracle
runs the same reading (``key_norm=True``) in double precision. Bars as for
the plain method: outputs max-abs 1e-4 (fp32 I/O) / 2e-2 (bf16 I/O) on slices
whose GPU bucket ids equal the oracle's; gradients relative to the slice's
largest entry, 1e-4 / 2e-2.
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


def _wl(dtype, B, H, L, d, nb, nh, m, causal, seed, dist="normal"):
    return workloads.Workload(f"kn_{dtype}_{L}_{d}", B, H, L, d, dtype, nb, nh, m, causal, seed,
                              dist)


def _wid(w):
    return f"{w.dtype}_B{w.B}H{w.H}L{w.L}d{w.d}nb{w.n_buckets}nh{w.n_hashes}m{w.chunk_len}c{int(w.causal)}"


CASES = [
    _wl("bf16", 2, 2, 1024, 64, 64, 4, 64, True, 301),            # matrix-core path, packed keys
    _wl("bf16", 1, 2, 2048, 128, 128, 3, 64, True, 302),
    _wl("bf16", 1, 2, 1024, 64, 32, 4, 64, False, 303, "clusters"),
    _wl("fp32", 1, 2, 1024, 64, 16, 2, 64, True, 304),            # plain kernels
    _wl("fp32", 1, 1, 96 * 8, 128, 8, 2, 96, False, 305),
    _wl("bf16", 1, 1, 128 * 6, 128, 8, 2, 128, True, 306),
]


def _inputs(w, zero_rows=()):
    qk, v, R = workloads.make_inputs(w)
    qk = qk.copy()
    for b, h, t in zero_rows:
        qk[b, h, t] = 0.0     # a zero key: its normalised form is the zero vector
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return qk, v, R, torch.from_numpy(qk).to(DEV, dt), torch.from_numpy(v).to(DEV, dt), \
        torch.from_numpy(R).to(DEV)


def _equal_slices(gb, rb):
    B, H = gb.shape[:2]
    return [(b, h) for b in range(B) for h in range(H) if np.array_equal(gb[b, h], rb[b, h])]


@pytest.mark.parametrize("w", CASES, ids=_wid)
def test_forward_key_norm_matches_oracle(w):
    qk, v, R, qk_t, v_t, R_t = _inputs(w, zero_rows=[(0, 0, 5)])
    ref, extra = oracle.forward(qk, v, R, w.n_buckets, w.chunk_len, w.causal, return_all=True,
                                key_norm=True)
    plain = oracle.forward(qk, v, R, w.n_buckets, w.chunk_len, w.causal)
    out = lsh.attention_fwd(qk_t, v_t, R_t, w.n_buckets, w.chunk_len, w.causal, key_norm=True)
    train, _ = lsh.attention_fwd_train(qk_t, v_t, R_t, w.n_buckets, w.chunk_len, w.causal,
                                       key_norm=True)
    gb, _ = lsh.hash(qk_t, R_t, w.n_buckets)
    gb = gb.cpu().numpy()
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    assert torch.equal(out, train), "training forward differs from the forward"
    slices = _equal_slices(gb, extra["buckets"])
    assert slices
    worst = max(float(np.abs(got[b, h] - ref[b, h]).max()) for b, h in slices)
    # the flag must change the result: the plain method differs by far more
    moved = max(float(np.abs(plain[b, h] - ref[b, h]).max()) for b, h in slices)
    print(f"{w.name}: worst {worst:.2e}, key norm moves the output by {moved:.2e}")
    assert worst <= TOL[w.dtype]
    assert moved > 10 * TOL[w.dtype]


@pytest.mark.parametrize("w", [CASES[0], CASES[3], CASES[4]], ids=_wid)
def test_chunk_attend_key_norm_on_oracle_order(w):
    """Steps 3-4 with key normalisation on the oracle's bucket ids and order."""
    qk, v, R, qk_t, v_t, R_t = _inputs(w)
    _, extra = oracle.forward(qk, v, R, w.n_buckets, w.chunk_len, w.causal, return_all=True,
                              key_norm=True)
    rb = torch.from_numpy(extra["buckets"]).to(DEV)
    rp = torch.from_numpy(extra["perm"]).to(DEV)
    o, lse = lsh.chunk_attend(qk_t, v_t, rb, rp, w.n_buckets, w.chunk_len, w.causal,
                              key_norm=True)
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    assert float(np.abs(o - extra["o_sorted"]).max()) <= TOL[w.dtype]
    rel = np.abs(lse - extra["lse"]) / np.maximum(1.0, np.abs(extra["lse"]))
    assert float(rel.max()) <= (1e-5 if w.dtype == "fp32" else 1e-3)


BWD_CASES = [CASES[0], CASES[1], CASES[3], CASES[4], CASES[5]]


@pytest.mark.parametrize("w", BWD_CASES, ids=_wid)
def test_backward_key_norm_matches_oracle(w):
    qk, v, R, qk_t, v_t, R_t = _inputs(w, zero_rows=[(0, 0, 7)])
    rng = np.random.default_rng(w.seed + 11)
    g = rng.standard_normal(qk.shape, dtype=np.float32)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    if w.dtype == "bf16":
        g = workloads.round_to_bf16(g)
    out, state = lsh.attention_fwd_train(qk_t, v_t, R_t, w.n_buckets, w.chunk_len, w.causal,
                                         key_norm=True)
    dqk, dv = lsh.attention_bwd(qk_t, v_t, out, torch.from_numpy(g).to(DEV, dt), state,
                                w.n_buckets, w.n_hashes, w.chunk_len, w.causal, key_norm=True)
    rq, rv = oracle.backward(qk, v, R, g, w.n_buckets, w.chunk_len, w.causal, key_norm=True)
    _, extra = oracle.forward(qk, v, R, w.n_buckets, w.chunk_len, w.causal, return_all=True,
                              key_norm=True)
    gb, _ = lsh.hash(qk_t, R_t, w.n_buckets)
    slices = _equal_slices(gb.cpu().numpy(), extra["buckets"])
    assert slices
    gq, gv = dqk.float().cpu().numpy(), dv.float().cpu().numpy()
    assert np.isfinite(gq).all() and np.isfinite(gv).all()
    worst = 0.0
    for b, h in slices:
        for got, ref in ((gq[b, h], rq[b, h]), (gv[b, h], rv[b, h])):
            err = float(np.abs(got - ref).max()) / float(np.abs(ref).max())
            worst = max(worst, err)
            assert err <= TOL[w.dtype], err
    print(f"{w.name}: worst relative gradient error {worst:.2e} over {len(slices)} slices")


def test_autograd_key_norm():
    w = CASES[0]
    qk, v, R, qk_t, v_t, R_t = _inputs(w)
    a = qk_t.clone().requires_grad_(True)
    b = v_t.clone().requires_grad_(True)
    out = lsh.LSHAttention.apply(a, b, R_t, w.n_buckets, w.chunk_len, w.causal, True)
    g = torch.randn(out.shape, generator=torch.Generator().manual_seed(3)).to(DEV, out.dtype)
    out.backward(g)
    o2, state = lsh.attention_fwd_train(qk_t, v_t, R_t, w.n_buckets, w.chunk_len, w.causal,
                                        key_norm=True)
    assert torch.equal(o2, out.detach())
    dqk, dv = lsh.attention_bwd(qk_t, v_t, o2, g, state, w.n_buckets, w.n_hashes, w.chunk_len,
                                w.causal, key_norm=True)
    assert torch.equal(dqk, a.grad) and torch.equal(dv, b.grad)
