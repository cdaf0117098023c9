"""GPU parity of the input projections (lsh_qkv_project) and of the forward
that starts from token vectors (lsh_attention_fwd_x), through the C ABI.

  * projections: against the fp64 oracle on random data, within one rounding
    of the output to the I/O dtype plus the float32 accumulation error;
  * lsh_attention_fwd_x: bit-equal to lsh_qkv_project followed by
    lsh_attention_fwd, and -- on inputs whose products and sums are exact in
    float32, so both sides round the same exact projections -- within the
    forward's bar of the oracle run on the oracle's own projections.
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


def _round(a, dtype):
    return workloads.round_to_bf16(a) if dtype == "bf16" else a.astype(np.float32)


def _dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(
        DEV, torch.bfloat16 if dtype == "bf16" else torch.float32)


PROJ_CASES = [
    # dtype, B, L, d_model, H, d
    ("bf16", 2, 200, 96, 2, 64),      # tokens not a multiple of the tile; 3 k-stages
    ("bf16", 1, 512, 1024, 8, 128),   # the benchmark's model width and heads
    ("bf16", 3, 64, 64, 1, 64),       # 128 outputs: half an output tile
    ("bf16", 1, 130, 40, 2, 128),     # d_model 40: a partial k-stage
    ("fp32", 1, 100, 40, 1, 64),
    ("fp32", 2, 70, 72, 3, 128),
]


@pytest.mark.parametrize("dtype,B,L,dm,H,d", PROJ_CASES)
def test_projection_matches_oracle(dtype, B, L, dm, H, d):
    rng = np.random.default_rng(500 + L + dm)
    x = _round(rng.standard_normal((B, L, dm), dtype=np.float32), dtype)
    w_qk = _round(rng.standard_normal((H * d, dm), dtype=np.float32) / np.sqrt(dm), dtype)
    w_v = _round(rng.standard_normal((H * d, dm), dtype=np.float32) / np.sqrt(dm), dtype)
    qk_t = torch.full((B, H, L, d), float("nan"), device=DEV,
                      dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    v_t = torch.full_like(qk_t, float("nan"))
    shape = lsh.Shape(B, H, L, d, 2, 1, L, 0, lsh.LSH_BF16 if dtype == "bf16" else lsh.LSH_F32)
    lsh.lsh_qkv_project(_dev(x, dtype), _dev(w_qk, dtype), _dev(w_v, dtype), shape, dm, qk_t, v_t)
    ref_qk, ref_v = oracle.project(x, w_qk, w_v, H)
    # sum_k |x_k w_k| per output, the scale of the float32 accumulation error
    mag_qk, mag_v = oracle.project(np.abs(x), np.abs(w_qk), np.abs(w_v), H)
    rel = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -23
    for got_t, ref, mag in ((qk_t, ref_qk, mag_qk), (v_t, ref_v, mag_v)):
        got = got_t.float().cpu().numpy()
        assert np.isfinite(got).all()
        assert np.all(np.abs(got - ref) <= rel * np.abs(ref) + 2.0 ** -16 * mag)


def _exact_inputs(rng, B, L, dm, H, d):
    """x in quarters of [-1, 1], weights in 64ths of [-1/8, 1/8]: every
    product is a multiple of 2^-8 and every sum stays below 2^5, so float32
    accumulation is exact and both sides round the same exact projection."""
    x = (rng.integers(-4, 5, (B, L, dm)) / 4.0).astype(np.float32)
    w_qk = (rng.integers(-8, 9, (H * d, dm)) / 64.0).astype(np.float32)
    w_v = (rng.integers(-8, 9, (H * d, dm)) / 64.0).astype(np.float32)
    return x, w_qk, w_v


def test_fwd_x_is_projection_then_forward():
    rng = np.random.default_rng(600)
    B, L, dm, H, d, nb, nh, m = 1, 1024, 256, 2, 64, 32, 2, 64
    x = workloads.round_to_bf16(rng.standard_normal((B, L, dm), dtype=np.float32))
    w_qk = workloads.round_to_bf16(rng.standard_normal((H * d, dm), dtype=np.float32) / 16)
    w_v = workloads.round_to_bf16(rng.standard_normal((H * d, dm), dtype=np.float32) / 16)
    R = torch.from_numpy(rng.standard_normal((nh, d, nb // 2), dtype=np.float32)).to(DEV)
    xt, wq, wv = _dev(x, "bf16"), _dev(w_qk, "bf16"), _dev(w_v, "bf16")
    out = lsh.attention_fwd_x(xt, wq, wv, R, H, nb, m, True)
    qk, v = lsh.qkv_project(xt, wq, wv, H)
    ref = lsh.attention_fwd(qk, v, R, nb, m, True)
    assert torch.equal(out, ref)


@pytest.mark.parametrize("dtype,B,L,dm,H,d,nb,nh,m,causal", [
    ("bf16", 1, 1024, 256, 2, 64, 32, 4, 64, True),
    ("bf16", 2, 512, 128, 1, 128, 16, 2, 64, False),
    ("fp32", 1, 256, 64, 2, 64, 8, 2, 32, True),
])
def test_fwd_x_matches_oracle(dtype, B, L, dm, H, d, nb, nh, m, causal):
    rng = np.random.default_rng(700 + L)
    x, w_qk, w_v = _exact_inputs(rng, B, L, dm, H, d)
    R = rng.standard_normal((nh, d, nb // 2), dtype=np.float32)
    out = lsh.attention_fwd_x(_dev(x, dtype), _dev(w_qk, dtype), _dev(w_v, dtype),
                              torch.from_numpy(R).to(DEV), H, nb, m, causal)
    qk64, v64 = oracle.project(x, w_qk, w_v, H)
    qk = _round(qk64, dtype)
    v = _round(v64, dtype)
    ref, extra = oracle.forward(qk, v, R, nb, m, causal, return_all=True)
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    # a hash decision within 1e-5 of a tie may go either way; compare the
    # (batch, head) slices where the oracle saw no such near-tie
    compared = 0
    for b in range(B):
        for h in range(H):
            if np.any(extra["margin"][b, h] < 1e-5):
                continue
            compared += 1
            assert np.abs(got[b, h] - ref[b, h]).max() <= TOL[dtype]
    assert compared >= 1


def test_projection_fullsize_sampled_rows():
    """The benchmark's shape (65536 tokens, d_model 1024 -> 8 heads x 128):
    the whole projection on the GPU, sampled token rows against the oracle
    (each output row depends only on its own token vector), with the bound
    of the small cases; and lsh_attention_fwd_x bit-equal to the projection
    followed by lsh_attention_fwd at that size."""
    B, L, dm, H, d, nb, nh, m = 1, 65536, 1024, 8, 128, 1024, 8, 64
    rng = np.random.default_rng(800)
    x = workloads.round_to_bf16(rng.standard_normal((B, L, dm), dtype=np.float32))
    w_qk = workloads.round_to_bf16(rng.standard_normal((H * d, dm), dtype=np.float32) / 32)
    w_v = workloads.round_to_bf16(rng.standard_normal((H * d, dm), dtype=np.float32) / 32)
    xt, wq, wv = _dev(x, "bf16"), _dev(w_qk, "bf16"), _dev(w_v, "bf16")
    qk_t, v_t = lsh.qkv_project(xt, wq, wv, H)
    toks = np.sort(np.concatenate([[0, L - 1], rng.choice(np.arange(1, L - 1), 62,
                                                          replace=False)]))
    ref_qk, ref_v = oracle.project(x[:, toks], w_qk, w_v, H)
    mag_qk, mag_v = oracle.project(np.abs(x[:, toks]), np.abs(w_qk), np.abs(w_v), H)
    for got_t, ref, mag in ((qk_t, ref_qk, mag_qk), (v_t, ref_v, mag_v)):
        got = got_t.float().cpu().numpy()
        assert np.isfinite(got).all()
        got = got[:, :, toks]
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * mag)
    R = torch.from_numpy(rng.standard_normal((nh, d, nb // 2), dtype=np.float32)).to(DEV)
    out = lsh.attention_fwd_x(xt, wq, wv, R, H, nb, m, True)
    ref_out = lsh.attention_fwd(qk_t, v_t, R, nb, m, True)
    assert torch.equal(out, ref_out)
