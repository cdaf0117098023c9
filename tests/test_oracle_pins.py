"""Pins of the CPU oracle against facts fixed outside it (no GPU needed).

Each test names what it pins. Together they are chosen so that a plausible
slip anywhere in the oracle (a swapped half of [xR, -xR], last-index ties, a
transposed R, an unstable sort, a window that looks ahead or wraps, a wrong
score scale, a missing self or causal rule, uniform instead of logsumexp
round weights) makes at least one of them fail; ``test_oracle_mutants.py``
checks that claim by planting such slips in a copy of the oracle.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch

import workloads
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------- O1 hash

def test_hash_glossary_worked_example(oracle_mod):
    """P-a: the glossary page's printed result of its seeded hashing example."""
    g = _golden("glossary_hash_example.json")
    x, R = workloads.glossary_hash_example()
    buckets, _ = oracle_mod.hash(x, R, 16)
    assert buckets.shape == (g["rounds"], 3)
    for row, name in ((1, "near"), (2, "far")):
        cos = float(x[0] @ x[row] / np.linalg.norm(x[0]) / np.linalg.norm(x[row]))
        assert f"{cos:.2f}" == g["printed"][name]["cosine"]
        # the example averages a float32 tensor, so the share is a float32
        share = float((buckets[:, row] == buckets[:, 0]).astype(np.float32).mean(dtype=np.float32))
        assert f"{share:.0%}" == g["printed"][name]["shared_rounds"]


def test_hash_two_axis_closed_form(oracle_mod):
    """With R = [e0, e1] the bucket is the first index of max(x0, x1, -x0, -x1):
    pins the [p, -p] order and the R layout [round, dim, bucket]."""
    R = np.zeros((1, 3, 2))
    R[0, 0, 0] = 1.0   # column 0 reads x[0]
    R[0, 2, 1] = 1.0   # column 1 reads x[2] (dim 1 is ignored)
    cases = {
        (3.0, 9.0, 1.0): 0, (1.0, 9.0, 3.0): 1, (-3.0, 9.0, 1.0): 2, (1.0, 9.0, -3.0): 3,
        (-1.0, -9.0, -3.0): 3, (2.0, 0.0, -2.0): 0, (-2.0, 0.0, 2.0): 1, (0.0, 5.0, 0.0): 0,
        (-2.0, 0.0, -2.0): 2,
    }
    x = np.array(list(cases.keys()))
    b, margin = oracle_mod.hash(x, R, 4)
    assert b[0].tolist() == list(cases.values())
    # exact ties have zero margin
    assert margin[0, 5] == 0.0 and margin[0, 6] == 0.0 and margin[0, 7] == 0.0


def test_hash_sign_hashing_nb2(oracle_mod):
    """P-b: with two buckets the hash is random-hyperplane sign hashing
    (rdly.ru summary, section on LSH): bucket 0 iff x.r >= 0, and the collision
    rate of two vectors at angle theta is 1 - theta/pi (Charikar, 2002)."""
    rng = np.random.default_rng(7)
    d = 16
    x = rng.standard_normal((50, d))
    R = rng.standard_normal((4, d, 1))
    b, _ = oracle_mod.hash(x, R, 2)
    expect = np.where(np.einsum("nd,rd->rn", x, R[:, :, 0]) >= 0, 0, 1)
    assert np.array_equal(b, expect)

    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    w = rng.standard_normal(d)
    w -= (w @ u) * u
    w /= np.linalg.norm(w)
    rounds = 20000
    R = rng.standard_normal((rounds, d, 1))
    for theta in (0.3, math.pi / 3, 2.0):
        y = math.cos(theta) * u + math.sin(theta) * w
        b, _ = oracle_mod.hash(np.stack([u, y]), R, 2)
        rate = float((b[:, 0] == b[:, 1]).mean())
        assert abs(rate - (1 - theta / math.pi)) < 0.015


def test_hash_invariants(oracle_mod):
    """P-c: range, invariance to positive scaling, and h(-x) = h(x) + nb/2 mod nb."""
    rng = np.random.default_rng(11)
    nb, d = 32, 24
    x = rng.standard_normal((300, d))
    R = rng.standard_normal((3, d, nb // 2))
    b, margin = oracle_mod.hash(x, R, nb)
    assert b.min() >= 0 and b.max() < nb
    safe = margin > 1e-9
    for alpha in (2.0, 0.5, 3.7):
        b2, _ = oracle_mod.hash(alpha * x, R, nb)
        assert np.array_equal(b2[safe], b[safe])
    bn, _ = oracle_mod.hash(-x, R, nb)
    assert np.array_equal(bn[safe], ((b + nb // 2) % nb)[safe])
    # every bucket is used over many random rotations
    b_many, _ = oracle_mod.hash(x[:1], rng.standard_normal((4000, d, nb // 2)), nb)
    counts = np.bincount(b_many[:, 0], minlength=nb)
    assert counts.min() > 60


def test_hash_zero_vector_and_margin(oracle_mod):
    """Ties go to the first index: the zero vector hashes to bucket 0 with margin 0;
    the margin equals the gap between the two largest entries of [p, -p]."""
    rng = np.random.default_rng(3)
    R = rng.standard_normal((2, 8, 5))
    x = np.vstack([np.zeros(8), rng.standard_normal(8)])
    b, margin = oracle_mod.hash(x, R, 10)
    assert b[:, 0].tolist() == [0, 0] and margin[:, 0].tolist() == [0.0, 0.0]
    for r in range(2):
        p = x[1] @ R[r]
        c = np.sort(np.concatenate([p, -p]))
        assert margin[r, 1] == pytest.approx(c[-1] - c[-2], rel=1e-12)


# --------------------------------------------------------------------------- O2 sort

def test_sort_matches_stable_argsort(oracle_mod):
    """P-d: the two-level sort equals numpy's stable argsort of the buckets."""
    rng = np.random.default_rng(5)
    for L, nb in ((1, 2), (17, 4), (1000, 16), (4096, 1024)):
        bucket = rng.integers(0, nb, L).astype(np.int32)
        perm, inv = oracle_mod.sort(bucket)
        assert np.array_equal(perm, np.argsort(bucket, kind="stable"))
        assert np.array_equal(inv[perm], np.arange(L))
        key = bucket[perm].astype(np.int64) * L + perm
        assert np.all(np.diff(key) > 0)


def test_sort_skewed_and_constant(oracle_mod):
    rng = np.random.default_rng(6)
    bucket = np.where(rng.random(5000) < 0.7, 3, rng.integers(0, 64, 5000)).astype(np.int32)
    perm, _ = oracle_mod.sort(bucket)
    assert np.array_equal(perm, np.argsort(bucket, kind="stable"))
    perm, inv = oracle_mod.sort(np.zeros(300, np.int32))
    assert np.array_equal(perm, np.arange(300)) and np.array_equal(inv, np.arange(300))


# --------------------------------------------------------------------------- O3/O4 attend

def _one_round(oracle_mod, x, v, R, nb, m, causal):
    b, _ = oracle_mod.hash(x, R, nb)
    perm, inv = oracle_mod.sort(b[0])
    o, lse = oracle_mod.attend(x, v, b[0], perm, m, causal)
    return b[0], perm, inv, o, lse


@pytest.mark.parametrize("causal", [False, True])
def test_attend_one_chunk_is_dense_same_bucket(oracle_mod, causal):
    """P-e: with one chunk spanning the sequence, the output equals dense
    softmax attention restricted to same-bucket pairs."""
    rng = np.random.default_rng(21)
    L, d, nb = 48, 8, 4
    x = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    R = rng.standard_normal((1, d, nb // 2))
    b, perm, inv, o, _ = _one_round(oracle_mod, x, v, R, nb, L, causal)
    ref = brute.dense_same_bucket(x, v, b, causal)
    np.testing.assert_allclose(o[inv], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_attend_single_bucket_matches_torch_sdpa(oracle_mod, causal):
    """P-f: all tokens in one bucket and one chunk: plain softmax attention with
    scale 1/sqrt(d) (ai-scholar.tech summary, section 'Transformerの問題点とは'),
    checked against torch's scaled_dot_product_attention with an additive mask."""
    rng = np.random.default_rng(22)
    L, d = 40, 16
    x = rng.standard_normal((L, d))
    x[:, 0] = np.abs(x[:, 0]) + 0.1
    v = rng.standard_normal((L, d))
    R = np.zeros((1, d, 1))
    R[0, 0, 0] = 1.0
    b, perm, inv, o, lse = _one_round(oracle_mod, x, v, R, 2, L, causal)
    assert np.all(b == 0)
    mask = torch.zeros(L, L, dtype=torch.float64)
    mask.fill_diagonal_(-brute.SELF_PENALTY)
    if causal:
        mask.masked_fill_(torch.ones(L, L, dtype=torch.bool).triu(1), float("-inf"))
    xt = torch.from_numpy(x)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        xt, xt, torch.from_numpy(v)[None, None], attn_mask=mask)[0, 0].numpy()
    np.testing.assert_allclose(o[inv], ref, rtol=1e-10, atol=1e-12)
    # lse is the natural-log partition function of the masked scores
    s = (x @ x.T) / math.sqrt(d) + mask.numpy()
    ref_lse = np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)) + s.max(1)
    np.testing.assert_allclose(lse[inv], ref_lse, rtol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_attend_hand_built_windows(oracle_mod, causal):
    """P-l: look-back of exactly one chunk, no look-ahead, no wrap, bucket masking
    and the self rule, on a hand-derived 8-token case."""
    g = _golden("chunk_window_cases.json")
    x = np.array(g["x"], np.float64)
    R = np.array(g["R"], np.float64)
    rng = np.random.default_rng(23)
    v = rng.standard_normal((8, 2))
    b, perm, inv, o, _ = _one_round(oracle_mod, x, v, R, 2, 2, causal)
    assert b.tolist() == g["buckets"]
    assert perm.tolist() == g["perm"]
    keys = g["keys"]["causal" if causal else "non_causal"]
    for pos, ks in keys.items():
        np.testing.assert_allclose(o[inv[int(pos)]], v[ks].mean(0), rtol=1e-12, atol=1e-12)


def test_attend_slots_subset_matches_full(oracle_mod):
    rng = np.random.default_rng(24)
    L, d, nb, m = 256, 8, 8, 32
    x = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    R = rng.standard_normal((1, d, nb // 2))
    b, perm, inv, o, lse = _one_round(oracle_mod, x, v, R, nb, m, True)
    slots = np.array([0, 5, 31, 32, 100, 255])
    o2, lse2 = oracle_mod.attend(x, v, b, perm, m, True, slots=slots)
    assert np.array_equal(o2[slots], o[slots]) and np.array_equal(lse2[slots], lse[slots])
    assert np.isnan(o2[1]).all()


# --------------------------------------------------------------------------- O5 + forward

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("m", [4, 8])
def test_forward_matches_multiset_closed_form(oracle_mod, causal, m):
    """P-g: logsumexp-weighted rounds == one softmax over the multiset of hits."""
    rng = np.random.default_rng(31 + m)
    L, d, nb, nh = 32, 8, 4, 3
    qk = rng.standard_normal((1, 1, L, d))
    v = rng.standard_normal((1, 1, L, d))
    R = rng.standard_normal((nh, d, nb // 2))
    out, extra = oracle_mod.forward(qk, v, R, nb, m, causal, return_all=True)
    ref = brute.multiset_closed_form(qk[0, 0], v[0, 0], extra["buckets"][0, 0], m, causal)
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-11, atol=1e-12)


def test_forward_identity_values_give_weights(oracle_mod):
    """P-h: with V = I the output rows are the attention weights: non-negative,
    summing to one, zero above the diagonal under causality, zero on pairs
    that never share a bucket and a window."""
    rng = np.random.default_rng(41)
    L, d, nb, nh, m = 16, 16, 4, 2, 4
    qk = rng.standard_normal((1, 1, L, d))
    v = np.eye(L)[None, None]
    R = rng.standard_normal((nh, d, nb // 2))
    out, extra = oracle_mod.forward(qk, v, R, nb, m, True, return_all=True)
    w = out[0, 0]
    assert np.all(w >= 0)
    # self-only rounds carry scores near -1e5, whose ulp (~1.5e-11) bounds the rounding
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-10)
    assert np.all(np.triu(w, 1) == 0)
    c = brute.multiplicity(extra["buckets"][0, 0], m, True)
    assert np.all(w[c == 0] == 0)
    np.testing.assert_allclose(w, brute.attention_weights(qk[0, 0], extra["buckets"][0, 0], m, True),
                               rtol=1e-11, atol=1e-14)


def test_forward_convexity(oracle_mod):
    """P-i: constant V gives that constant; every output lies between the
    column-wise min and max of V."""
    rng = np.random.default_rng(42)
    B, H, L, d, nb, nh, m = 2, 2, 64, 8, 8, 3, 8
    qk = rng.standard_normal((B, H, L, d))
    R = rng.standard_normal((nh, d, nb // 2))
    vc = np.broadcast_to(rng.standard_normal(d), (B, H, L, d)).copy()
    out = oracle_mod.forward(qk, vc, R, nb, m, True)
    np.testing.assert_allclose(out, vc, rtol=1e-10)
    v = rng.standard_normal((B, H, L, d))
    out = oracle_mod.forward(qk, v, R, nb, m, False)
    lo = v.min(axis=2, keepdims=True)
    hi = v.max(axis=2, keepdims=True)
    assert np.all(out >= lo - 1e-10) and np.all(out <= hi + 1e-10)


def test_forward_round_symmetry(oracle_mod):
    """P-j: permuting the rounds leaves the output unchanged; duplicating every
    round gives the same output as the rounds once."""
    rng = np.random.default_rng(43)
    L, d, nb, nh, m = 64, 8, 8, 3, 8
    qk = rng.standard_normal((1, 2, L, d))
    v = rng.standard_normal((1, 2, L, d))
    R = rng.standard_normal((nh, d, nb // 2))
    out = oracle_mod.forward(qk, v, R, nb, m, True)
    out_p = oracle_mod.forward(qk, v, R[[2, 0, 1]], nb, m, True)
    np.testing.assert_allclose(out_p, out, rtol=1e-10, atol=1e-10)
    out_d = oracle_mod.forward(qk, v, np.concatenate([R, R]), nb, m, True)
    np.testing.assert_allclose(out_d, out, rtol=1e-10, atol=1e-10)


def test_forward_causal_first_row_is_v0(oracle_mod):
    """P-k: under causality position 0 only sees itself, in every round."""
    rng = np.random.default_rng(44)
    qk = rng.standard_normal((2, 3, 32, 8))
    v = rng.standard_normal((2, 3, 32, 8))
    R = rng.standard_normal((4, 8, 4))
    out = oracle_mod.forward(qk, v, R, 8, 4, True)
    np.testing.assert_allclose(out[:, :, 0], v[:, :, 0], rtol=1e-10)


def test_forward_steps_compose(oracle_mod):
    """forward() is exactly hash -> sort -> attend -> combine per (batch, head)."""
    rng = np.random.default_rng(45)
    B, H, L, d, nb, nh, m = 1, 2, 128, 8, 16, 2, 16
    qk = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    R = rng.standard_normal((nh, d, nb // 2))
    out, ex = oracle_mod.forward(qk, v, R, nb, m, True, return_all=True)
    for h in range(H):
        b, _ = oracle_mod.hash(qk[0, h], R, nb)
        assert np.array_equal(b, ex["buckets"][0, h])
        os_, ls_, iv_ = [], [], []
        for r in range(nh):
            perm, inv = oracle_mod.sort(b[r])
            assert np.array_equal(perm, ex["perm"][0, h, r])
            o, lse = oracle_mod.attend(qk[0, h], v[0, h], b[r], perm, m, True)
            os_.append(o), ls_.append(lse), iv_.append(inv)
        comb = oracle_mod.combine(np.stack(os_), np.stack(ls_), np.stack(iv_))
        assert np.array_equal(comb, out[0, h])


def test_forward_empty_and_errors(oracle_mod):
    R = np.ones((1, 4, 2))
    out = oracle_mod.forward(np.zeros((1, 1, 0, 4)), np.zeros((1, 1, 0, 4)), R, 4, 2, True)
    assert out.shape == (1, 1, 0, 4)
    with pytest.raises(ValueError):
        oracle_mod.forward(np.zeros((1, 1, 6, 4)), np.zeros((1, 1, 6, 4)), R, 4, 4, True)
    with pytest.raises(ValueError):
        oracle_mod.hash(np.zeros((3, 4)), np.ones((1, 4, 2)), 3)


def test_forward_bf16_inputs_widen_exactly():
    """The generator's bf16 rounding agrees with torch's conversion."""
    a = np.random.default_rng(1).standard_normal(100000).astype(np.float32) * 7
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(workloads.round_to_bf16(a), ref)


# --------------------------------------------------------------------------- P0 projections

def test_project_hand_example(oracle_mod):
    """P0: a hand-computed example; it fixes the head split, the weight
    orientation (output n of input k at w[n, k]) and which weights feed v."""
    g = _golden("projection_hand_example.json")
    qk, v = oracle_mod.project(np.array(g["x"], float), np.array(g["w_qk"], float),
                               np.array(g["w_v"], float), g["heads"])
    assert np.array_equal(qk, np.array(g["qk"], float))
    assert np.array_equal(v, np.array(g["v"], float))


def test_project_selection_weights_copy_features(oracle_mod):
    """P0: one-hot weight rows copy input features, so every output is an
    exact copy of a known input element (layout [B, H, L, d])."""
    rng = np.random.default_rng(40)
    B, L, dm, H, d = 2, 5, 12, 3, 4
    x = rng.standard_normal((B, L, dm))
    pick_q = rng.integers(0, dm, H * d)
    pick_v = rng.permutation(dm)[: H * d] if H * d <= dm else rng.integers(0, dm, H * d)
    w_qk = np.eye(dm)[pick_q]
    w_v = -2.0 * np.eye(dm)[pick_v]
    qk, v = oracle_mod.project(x, w_qk, w_v, H)
    for b in range(B):
        for h in range(H):
            for l in range(L):
                for e in range(d):
                    assert qk[b, h, l, e] == x[b, l, pick_q[h * d + e]]
                    assert v[b, h, l, e] == -2.0 * x[b, l, pick_v[h * d + e]]


def test_project_matches_einsum(oracle_mod):
    """P0: agrees with numpy's einsum (a library contraction) on random data."""
    rng = np.random.default_rng(41)
    B, L, dm, H, d = 2, 7, 24, 2, 8
    x = rng.standard_normal((B, L, dm))
    w_qk = rng.standard_normal((H * d, dm))
    w_v = rng.standard_normal((H * d, dm))
    qk, v = oracle_mod.project(x, w_qk, w_v, H)
    ref_qk = np.einsum("blk,hek->bhle", x, w_qk.reshape(H, d, dm))
    ref_v = np.einsum("blk,hek->bhle", x, w_v.reshape(H, d, dm))
    assert np.allclose(qk, ref_qk, rtol=1e-12, atol=1e-12)
    assert np.allclose(v, ref_v, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- G1 backward

def _fd_case(rng, B, H, L, d, nh, nb):
    qk = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    R = rng.standard_normal((nh, d, nb // 2))
    g = rng.standard_normal((B, H, L, d))
    return qk, v, R, g


@pytest.mark.parametrize("causal,key_norm", [(False, False), (True, False), (True, True)])
def test_backward_matches_finite_differences(oracle_mod, causal, key_norm):
    """G1: the gradient of sum(dout * forward) by central differences of the
    oracle's own forward (the hash is piecewise constant: perturbations that
    move a bucket are skipped and counted); also with normalised keys."""
    rng = np.random.default_rng(60 + causal)
    B, H, L, d, nh, nb, m = 1, 2, 16, 6, 3, 4, 4
    qk, v, R, g = _fd_case(rng, B, H, L, d, nh, nb)
    dqk, dv = oracle_mod.backward(qk, v, R, g, nb, m, causal, key_norm=key_norm)
    base_b = oracle_mod.forward(qk, v, R, nb, m, causal, return_all=True)[1]["buckets"]
    eps = 1e-6
    skipped = 0
    for which, arr, grad in (("qk", qk, dqk), ("v", v, dv)):
        for idx in np.ndindex(arr.shape):
            vals = []
            for sgn in (1.0, -1.0):
                a = arr.copy()
                a[idx] += sgn * eps
                args = (a, v) if which == "qk" else (qk, a)
                out, extra = oracle_mod.forward(*args, R, nb, m, causal, return_all=True,
                                                key_norm=key_norm)
                vals.append((float((g * out).sum()), np.array_equal(extra["buckets"], base_b)))
            if not (vals[0][1] and vals[1][1]):
                skipped += 1
                continue
            num = (vals[0][0] - vals[1][0]) / (2 * eps)
            assert abs(num - grad[idx]) <= 1e-6 * (1.0 + abs(grad[idx])), (which, idx)
    assert skipped <= 4


@pytest.mark.parametrize("causal", [False, True])
def test_backward_one_bucket_matches_torch_autograd(oracle_mod, causal):
    """G1: all tokens in one bucket and one chunk: the gradients of plain
    softmax attention with queries = keys, from torch's autograd in float64."""
    rng = np.random.default_rng(62 + causal)
    L, d = 24, 8
    x = rng.standard_normal((L, d))
    x[:, 0] = np.abs(x[:, 0]) + 0.1
    v = rng.standard_normal((L, d))
    g = rng.standard_normal((L, d))
    R = np.zeros((1, d, 1))
    R[0, 0, 0] = 1.0
    dqk, dv = oracle_mod.backward(x[None, None], v[None, None], R, g[None, None], 2, L, causal)
    xt = torch.from_numpy(x).requires_grad_(True)
    vt = torch.from_numpy(v).requires_grad_(True)
    mask = torch.zeros(L, L, dtype=torch.float64)
    mask.fill_diagonal_(-brute.SELF_PENALTY)
    if causal:
        mask.masked_fill_(torch.ones(L, L, dtype=torch.bool).triu(1), float("-inf"))
    s = xt @ xt.T / math.sqrt(d) + mask
    out = torch.softmax(s, dim=1) @ vt
    (out * torch.from_numpy(g)).sum().backward()
    np.testing.assert_allclose(dqk[0, 0], xt.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv[0, 0], vt.grad.numpy(), rtol=1e-9, atol=1e-11)


def test_backward_duplicated_round(oracle_mod):
    """G1: a round repeated ([R0, R0]) doubles every multiplicity uniformly, so
    the gradients equal those of [R0] alone."""
    rng = np.random.default_rng(64)
    qk, v, R, g = _fd_case(rng, 1, 2, 32, 8, 1, 8)
    a = oracle_mod.backward(qk, v, R, g, 8, 8, True)
    b = oracle_mod.backward(qk, v, np.concatenate([R, R]), g, 8, 8, True)
    # equal up to double rounding of sums taken in a different order
    np.testing.assert_allclose(a[0], b[0], rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-9, atol=1e-9)


@pytest.mark.parametrize("L,d,nb,nh,m,causal,key_norm", [
    (256, 16, 8, 3, 16, True, False),
    (512, 32, 16, 2, 32, False, True),
    (192, 8, 4, 4, 64, True, True),
    (64, 8, 4, 2, 64, False, False),        # one chunk
])
def test_backward_rows_equal_full_backward(oracle_mod, L, d, nb, nh, m, causal, key_norm):
    """G1 at chosen positions: every chosen row is the full backward's row,
    bit for bit (the same terms summed in the same order), including the
    positions in the first and last sorted chunk of every round."""
    rng = np.random.default_rng(66 + L + d)
    qk, v, R, g = _fd_case(rng, 1, 1, L, d, nh, nb)
    dqk, dv = oracle_mod.backward(qk, v, R, g, nb, m, causal, key_norm=key_norm)
    _, extra = oracle_mod.forward(qk, v, R, nb, m, causal, return_all=True)
    edge = {int(p) for r in range(nh) for p in (extra["perm"][0, 0, r, 0],
                                                 extra["perm"][0, 0, r, L - 1])}
    toks = np.array(sorted(edge | set(rng.choice(L, size=12, replace=False).tolist())))
    rq, rv = oracle_mod.backward_rows(qk[0, 0], v[0, 0], R, g[0, 0], toks, nb, m, causal,
                                      key_norm=key_norm)
    assert np.array_equal(rq, dqk[0, 0, toks]) and np.array_equal(rv, dv[0, 0, toks])
    # one position alone gives its row too (nothing depends on the other rows)
    q1, v1 = oracle_mod.backward_rows(qk[0, 0], v[0, 0], R, g[0, 0], toks[:1], nb, m, causal,
                                      key_norm=key_norm)
    assert np.array_equal(q1[0], dqk[0, 0, toks[0]]) and np.array_equal(v1[0], dv[0, 0, toks[0]])


def test_backward_rows_rejects_bad_positions(oracle_mod):
    rng = np.random.default_rng(67)
    qk, v, R, g = _fd_case(rng, 1, 1, 64, 8, 2, 4)
    for toks in ([3, 3], [64], [-1]):
        with pytest.raises(ValueError):
            oracle_mod.backward_rows(qk[0, 0], v[0, 0], R, g[0, 0], toks, 4, 16, True)


# --------------------------------------------------------------------------- key normalisation

def test_key_norm_unit_rows_equal_plain(oracle_mod):
    """Variant: with rows of unit length, normalising the keys changes nothing."""
    rng = np.random.default_rng(70)
    qk = rng.standard_normal((1, 2, 64, 8))
    qk /= np.linalg.norm(qk, axis=-1, keepdims=True)
    v = rng.standard_normal((1, 2, 64, 8))
    R = rng.standard_normal((2, 8, 4))
    a = oracle_mod.forward(qk, v, R, 8, 16, True)
    b = oracle_mod.forward(qk, v, R, 8, 16, True, key_norm=True)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_key_norm_single_bucket_matches_torch_sdpa(oracle_mod, causal):
    """Variant: all tokens in one bucket and one chunk: softmax attention of the
    queries against unit-length keys, from torch's scaled_dot_product_attention
    with an additive mask."""
    rng = np.random.default_rng(71)
    L, d = 40, 16
    x = rng.standard_normal((L, d)) * rng.uniform(0.5, 3.0, (L, 1))
    x[:, 0] = np.abs(x[:, 0]) + 0.1
    v = rng.standard_normal((L, d))
    R = np.zeros((1, d, 1))
    R[0, 0, 0] = 1.0
    out = oracle_mod.forward(x[None, None], v[None, None], R, 2, L, causal, key_norm=True)
    mask = torch.zeros(L, L, dtype=torch.float64)
    mask.fill_diagonal_(-brute.SELF_PENALTY)
    if causal:
        mask.masked_fill_(torch.ones(L, L, dtype=torch.bool).triu(1), float("-inf"))
    xt = torch.from_numpy(x)
    kt = xt / xt.norm(dim=1, keepdim=True)
    ref = torch.nn.functional.scaled_dot_product_attention(
        xt[None, None], kt[None, None], torch.from_numpy(v)[None, None], attn_mask=mask)[0, 0]
    np.testing.assert_allclose(out[0, 0], ref.numpy(), rtol=1e-10, atol=1e-12)


def test_per_head_rotations_equal_heads_equal_shared(oracle_mod):
    """Variant: per-head rotations that are all the same matrix give the
    shared-R method exactly."""
    rng = np.random.default_rng(80)
    qk = rng.standard_normal((2, 3, 64, 8))
    v = rng.standard_normal((2, 3, 64, 8))
    R = rng.standard_normal((2, 8, 4))
    a = oracle_mod.forward(qk, v, R, 8, 16, True)
    b = oracle_mod.forward(qk, v, np.stack([R] * 3), 8, 16, True)
    np.testing.assert_array_equal(a, b)


def test_per_head_rotations_are_each_heads_own(oracle_mod):
    """Variant: with R [H, nh, d, nb/2], slice (b, h) hashes with R[h] in every
    batch: its buckets are the plain hash of that slice by R[h], and its output
    and gradients equal the one-head method run on the slice alone with R[h]."""
    rng = np.random.default_rng(81)
    B, H, L, d, nb = 2, 3, 64, 8, 8
    qk = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    g = rng.standard_normal((B, H, L, d))
    R4 = rng.standard_normal((H, 2, d, nb // 2))
    out, extra = oracle_mod.forward(qk, v, R4, nb, 16, True, return_all=True)
    dqk, dv = oracle_mod.backward(qk, v, R4, g, nb, 16, True)
    shared = oracle_mod.forward(qk, v, R4[0], nb, 16, True)
    assert np.abs(out - shared).max() > 1e-3      # the heads' rotations matter
    for b in range(B):
        for h in range(H):
            bk, _ = oracle_mod.hash(qk[b, h], R4[h], nb)
            np.testing.assert_array_equal(extra["buckets"][b, h], bk)
            sl = (slice(b, b + 1), slice(h, h + 1))
            one = oracle_mod.forward(qk[sl], v[sl], R4[h], nb, 16, True)
            np.testing.assert_array_equal(out[b, h], one[0, 0])
            gq, gv = oracle_mod.backward(qk[sl], v[sl], R4[h], g[sl], nb, 16, True)
            np.testing.assert_array_equal(dqk[b, h], gq[0, 0])
            np.testing.assert_array_equal(dv[b, h], gv[0, 0])


def test_ffn_hand_example(oracle_mod):
    """F1: a hand-computed example; it fixes the weight orientation, where each
    bias is added and that the ReLU acts between the two maps."""
    g = _golden("ffn_hand_example.json")
    a = [np.array(g[k], float) for k in ("x", "w1", "b1", "w2", "b2")]
    for chunk in (1, 2, 5):
        assert np.array_equal(oracle_mod.ffn(*a, chunk), np.array(g["out"], float))


def test_ffn_matches_torch_linear_relu(oracle_mod):
    """F1 against torch's linear and relu in float64 on random inputs, with
    and without biases."""
    rng = np.random.default_rng(90)
    rows, dm, dff = 37, 24, 40
    x = rng.standard_normal((rows, dm))
    w1 = rng.standard_normal((dff, dm))
    w2 = rng.standard_normal((dm, dff))
    b1 = rng.standard_normal(dff)
    b2 = rng.standard_normal(dm)
    F = torch.nn.functional
    t = lambda a: torch.from_numpy(a)
    for bias in (True, False):
        ref = F.linear(F.relu(F.linear(t(x), t(w1), t(b1) if bias else None)), t(w2),
                       t(b2) if bias else None).numpy()
        got = oracle_mod.ffn(x, w1, b1 if bias else None, w2, b2 if bias else None, 8)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_ffn_chunk_size_changes_nothing(oracle_mod):
    """F1: rows are independent, so every chunk size gives the same bits."""
    rng = np.random.default_rng(91)
    x = rng.standard_normal((23, 16))
    w1 = rng.standard_normal((32, 16))
    w2 = rng.standard_normal((16, 32))
    b1 = rng.standard_normal(32)
    b2 = rng.standard_normal(16)
    ref = oracle_mod.ffn(x, w1, b1, w2, b2, 23)
    for chunk in (1, 2, 5, 22, 100):
        assert np.array_equal(oracle_mod.ffn(x, w1, b1, w2, b2, chunk), ref)


def test_ffn_relu_regions(oracle_mod):
    """F1: a very negative b1 switches every hidden unit off (out = b2
    exactly); non-negative x, W1, b1 keep them all on, where the map is the
    affine closed form x (W2 W1)^T + W2 b1 + b2 (numpy products)."""
    rng = np.random.default_rng(92)
    x = rng.standard_normal((9, 8))
    w1 = rng.standard_normal((12, 8))
    w2 = rng.standard_normal((8, 12))
    b2 = rng.standard_normal(8)
    off = oracle_mod.ffn(x, w1, np.full(12, -1e6), w2, b2, 4)
    assert np.array_equal(off, np.broadcast_to(b2, off.shape))
    xp, w1p, b1p = np.abs(x), np.abs(w1), np.abs(rng.standard_normal(12))
    on = oracle_mod.ffn(xp, w1p, b1p, w2, b2, 4)
    np.testing.assert_allclose(on, xp @ (w2 @ w1p).T + w2 @ b1p + b2, rtol=1e-12, atol=1e-12)



# --------------------------------------------------------------------------- Q1 separate Q/K

@pytest.mark.parametrize("causal", [False, True])
def test_separate_qk_hand_built_windows(oracle_mod, causal):
    """Separate queries and keys on a hand-derived 8-token case: each side
    sorted on its own, query chunk c against key chunks c-1 and c, bucket and
    causal masks, no self penalty, and a window without a key of the query's
    bucket (position 0, causal) giving a zero row and lse -inf."""
    g = _golden("separate_qk_window_cases.json")
    bq, bk = np.array(g["bucket_q"]), np.array(g["bucket_k"])
    q = np.zeros((8, 8))
    k = np.zeros((8, 8))
    q[:, 0] = np.where(bq == 0, 1.0, -1.0)
    k[:, 0] = np.where(bk == 0, 1.0, -1.0)
    R = np.zeros((1, 8, 1))
    R[0, 0, 0] = 1.0
    v = np.eye(8)
    out, ex = oracle_mod.forward_qk(q[None, None], k[None, None], v[None, None], R, 2, 2,
                                    causal, return_all=True)
    assert ex["buckets_q"][0, 0, 0].tolist() == g["bucket_q"]
    assert ex["buckets_k"][0, 0, 0].tolist() == g["bucket_k"]
    assert ex["perm_q"][0, 0, 0].tolist() == g["perm_q"]
    assert ex["perm_k"][0, 0, 0].tolist() == g["perm_k"]
    keys = g["keys"]["causal" if causal else "non_causal"]
    for pos, ks in keys.items():
        want = np.zeros(8)
        want[ks] = 1.0 / len(ks) if ks else 0.0
        np.testing.assert_allclose(out[0, 0, int(pos)], want, rtol=1e-12, atol=1e-12)
        slot = ex["inv_q"][0, 0, 0, int(pos)]
        assert np.isneginf(ex["lse"][0, 0, 0, slot]) == (not ks)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("m", [4, 8, 32])
def test_separate_qk_matches_multiset_closed_form(oracle_mod, causal, m):
    """Separate queries and keys against a brute force that takes the buckets
    from numpy's argmax and enumerates every (query, key) pair's windows from
    numpy's stable argsort of each side; m = 32 is one chunk, i.e. dense
    attention over same-bucket pairs."""
    rng = np.random.default_rng(61 + m)
    L, d, nb, nh = 32, 8, 4, 3
    q = rng.standard_normal((L, d))
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    R = rng.standard_normal((nh, d, nb // 2))
    out = oracle_mod.forward_qk(q[None, None], k[None, None], v[None, None], R, nb, m, causal)
    bq, bk = brute.angular_buckets(q, R), brute.angular_buckets(k, R)
    ref = brute.multiset_closed_form_qk(q, k, v, bq, bk, m, causal)
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-11, atol=1e-12)
    # the case must exercise queries that find no key in any round
    if causal and m == 4:
        assert (np.abs(ref).sum(1) == 0).any()


def test_separate_qk_invariants(oracle_mod):
    """Rows with a hit are convex combinations of V, rows without are zero;
    duplicating every round changes nothing; the causal first position sees
    its own key exactly when the buckets agree in some round."""
    rng = np.random.default_rng(64)
    B, H, L, d, nb, nh, m = 1, 2, 64, 8, 8, 3, 8
    q = rng.standard_normal((B, H, L, d))
    k = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    R = rng.standard_normal((nh, d, nb // 2))
    out, ex = oracle_mod.forward_qk(q, k, v, R, nb, m, True, return_all=True)
    lse_by_pos = np.take_along_axis(ex["lse"], ex["inv_q"].astype(np.int64), axis=3)
    empty = np.isneginf(lse_by_pos).all(axis=2)
    assert empty.any() and not empty.all()
    assert np.all(out[empty] == 0)
    lo = v.min(axis=2, keepdims=True)
    hi = v.max(axis=2, keepdims=True)
    inside = (out >= lo - 1e-10) & (out <= hi + 1e-10)
    assert inside[~empty].all()
    dup = oracle_mod.forward_qk(q, k, v, np.concatenate([R, R]), nb, m, True)
    np.testing.assert_allclose(dup, out, rtol=1e-10, atol=1e-12)
    same0 = (ex["buckets_q"][:, :, :, 0] == ex["buckets_k"][:, :, :, 0]).any(axis=2)
    for b in range(B):
        for h in range(H):
            want = v[b, h, 0] if same0[b, h] else np.zeros(d)
            np.testing.assert_allclose(out[b, h, 0], want, rtol=1e-12, atol=1e-14)
