"""The fused forward against the oracle on seeded random shapes.

The forward picks its kernels and launch widths from the shape (one or
several sort launches, the scatter's wave count, the chunk pass's run length,
the combine's round group). The hand-picked cases elsewhere name each choice;
these draws, from one fixed seed over the sizes the boundary accepts, meet
combinations none of them names: odd bucket counts, one to nine rounds, chunk
lengths from 16 to 128, ragged chunk counts, both I/O dtypes and both method
flags. Each case compares every (batch, head) slice whose bucket ids equal the
oracle's (a near-tie may go either way: the hash tests bound those) with the
oracle's output, at the bars of the other parity tests: max-abs 1e-4 for fp32
I/O, 2e-2 for bf16. A fourth family runs the training forward and the
backward against the oracle's gradients, relative to the largest gradient
entry of each slice at the same bars; a fifth, separate queries and keys
against the oracle's forward for that variant, where a query whose windows
hold no key of its bucket gets a zero row. The sort entry point on its
own, bit-exact against the oracle, takes a sixth family of random lengths,
bucket counts and id distributions; the projections and the chunked
feed-forward take random widths, row counts and chunkings, at the bars their
own tests derive from the arithmetic. Last, the hash on random shapes with
planted exact ties (duplicated columns of R, rows along them, zero rows),
where the first of the tied buckets must win as in the oracle.
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


# Three families: small problems over the whole range of sizes; many short
# segments (hundreds to a few thousand (batch, head, round) triples, where
# the sort and chunk launches switch to their many-segment forms); and long
# sequences spanning several sort tiles.
FAMILIES = {
    "small": dict(n=32, m=(16, 32, 64, 64, 64, 128), chunks=(1, 40), nh=(1, 9), B=(1, 3),
                  H=(1, 4), cap=120_000),
    "many": dict(n=12, m=(32, 64, 64), chunks=(1, 12), nh=(8, 32), B=(1, 4), H=(16, 64),
                 cap=1_500_000),
    "long": dict(n=8, m=(64, 64, 128), chunks=(64, 320), nh=(1, 4), B=(1, 2), H=(1, 2),
                 cap=400_000),
    # the backward: training forward and gradients
    "bwd": dict(n=16, m=(16, 32, 64, 64, 64, 128), chunks=(1, 40), nh=(1, 8), B=(1, 3),
                H=(1, 6), cap=60_000),
    # separate queries and keys (key normalisation does not apply there)
    "sep": dict(n=16, m=(16, 32, 64, 64, 64, 128), chunks=(1, 40), nh=(1, 9), B=(1, 3),
                H=(1, 6), cap=120_000),
}


def _draw(family, seed):
    f = FAMILIES[family]
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < f["n"]:
        dtype = "fp32" if rng.random() < 0.25 else "bf16"
        d = int(rng.choice([64, 128]))
        m = int(rng.choice(f["m"]))
        L = m * int(rng.integers(f["chunks"][0], f["chunks"][1] + 1))
        nb = 2 * int(round(np.exp(rng.uniform(0.0, np.log(2048.0)))))   # 2 ... 4096
        nh = int(rng.integers(f["nh"][0], f["nh"][1] + 1))
        B = int(rng.integers(f["B"][0], f["B"][1] + 1))
        H = int(rng.integers(f["H"][0], f["H"][1] + 1))
        causal = bool(rng.integers(0, 2))
        dist = "clusters" if rng.random() < 0.3 else "normal"
        per_head = bool(rng.random() < 0.25)
        key_norm = bool(rng.random() < 0.25) and family != "sep"
        # token-rounds, and the oracle's multiply-adds (a few seconds at most)
        if B * H * nh * L > f["cap"] or B * H * nh * L * (nb + 4 * m) * d > 4e10:
            continue
        i = len(cases)
        name = (f"{family}{i}_{dtype}_b{B}h{H}l{L}d{d}_nb{nb}nh{nh}m{m}"
                f"{'_causal' if causal else ''}{'_perhead' if per_head else ''}"
                f"{'_keynorm' if key_norm else ''}_{dist}")
        w = workloads.Workload(name, B, H, L, d, dtype, nb, nh, m, causal, seed + 1 + i, dist)
        cases.append((w, per_head, key_norm))
    return cases


CASES = _draw("small", 20261204) + _draw("many", 20261205) + _draw("long", 20261206)
BWD_CASES = _draw("bwd", 20261207)
SEP_CASES = [(w, ph) for w, ph, _ in _draw("sep", 20261208)]


def _draw_sort(n, seed, H=(1, 8), nh=(1, 8), Lmax=98304, max_slots=3_000_000, tag="sort"):
    """(name, B, H, nh, L, nb, kind, seed): lengths 1 to Lmax and bucket counts
    2 to 4096, both log-uniform, ids uniform, skewed (30 % in one bucket) or
    all equal."""
    Hr, nhr = H, nh
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        B = int(rng.integers(1, 4))
        H = int(rng.integers(Hr[0], Hr[1] + 1))
        nh = int(rng.integers(nhr[0], nhr[1] + 1))
        L = int(round(np.exp(rng.uniform(0.0, np.log(float(Lmax))))))
        nb = 2 * int(round(np.exp(rng.uniform(0.0, np.log(2048.0)))))
        kind = str(rng.choice(["uniform", "uniform", "skewed", "constant"]))
        if B * H * nh * L > max_slots:
            continue
        i = len(cases)
        cases.append((f"{tag}{i}_{kind}_b{B}h{H}nh{nh}l{L}_nb{nb}", B, H, nh, L, nb, kind,
                      seed + 1 + i))
    return cases


# the second family: hundreds to thousands of short segments
SORT_CASES = (_draw_sort(24, 20261209) +
              _draw_sort(8, 20261210, H=(16, 64), nh=(8, 32), Lmax=1024, tag="sortmany"))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lsh.load_library()


@pytest.mark.parametrize("w,per_head,key_norm", CASES, ids=[c[0].name for c in CASES])
def test_random_shape_forward_matches_oracle(w, per_head, key_norm):
    qk, v, R = workloads.make_inputs(w)
    if per_head:
        R = np.random.default_rng(w.seed + 1).standard_normal(
            (w.H, w.n_hashes, w.d, w.n_buckets // 2), dtype=np.float32)
    dt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    qk_t = torch.from_numpy(qk).to(DEV, dt)
    v_t = torch.from_numpy(v).to(DEV, dt)
    R_t = torch.from_numpy(R).to(DEV)
    ref, extra = oracle.forward(qk, v, R, w.n_buckets, w.chunk_len, w.causal, return_all=True,
                                key_norm=key_norm)
    buckets, _ = lsh.hash(qk_t, R_t, w.n_buckets)
    gb = buckets.cpu().numpy()
    differ = gb != extra["buckets"]
    assert not np.any(differ & (extra["margin"] >= 1e-9)), "bucket ids differ above margin 1e-9"
    out = torch.full_like(qk_t, float("nan"))
    lsh.attention_fwd(qk_t, v_t, R_t, w.n_buckets, w.chunk_len, w.causal, out=out,
                      key_norm=key_norm)
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    worst, compared = 0.0, 0
    for b in range(w.B):
        for h in range(w.H):
            if differ[b, h].any():
                continue
            compared += 1
            worst = max(worst, float(np.abs(got[b, h] - ref[b, h]).max()))
    print(f"{w.name}: slices compared {compared} of {w.B * w.H}, max |err| {worst:.2e}")
    assert compared >= 1
    assert worst <= TOL[w.dtype]


@pytest.mark.parametrize("w,per_head,key_norm", BWD_CASES, ids=[c[0].name for c in BWD_CASES])
def test_random_shape_backward_matches_oracle(w, per_head, key_norm):
    qk, v, R = workloads.make_inputs(w)
    if per_head:
        R = np.random.default_rng(w.seed + 1).standard_normal(
            (w.H, w.n_hashes, w.d, w.n_buckets // 2), dtype=np.float32)
    g = np.random.default_rng(w.seed + 2).standard_normal(qk.shape, dtype=np.float32)
    if w.dtype == "bf16":
        g = workloads.round_to_bf16(g)
    dt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    qk_t = torch.from_numpy(qk).to(DEV, dt)
    v_t = torch.from_numpy(v).to(DEV, dt)
    R_t = torch.from_numpy(R).to(DEV)
    g_t = torch.from_numpy(g).to(DEV, dt)
    _, extra = oracle.forward(qk, v, R, w.n_buckets, w.chunk_len, w.causal, return_all=True,
                              key_norm=key_norm)
    ref_dqk, ref_dv = oracle.backward(qk, v, R, g, w.n_buckets, w.chunk_len, w.causal,
                                      key_norm=key_norm)
    out, state = lsh.attention_fwd_train(qk_t, v_t, R_t, w.n_buckets, w.chunk_len, w.causal,
                                         key_norm=key_norm)
    dqk, dv = lsh.attention_bwd(qk_t, v_t, out, g_t, state, w.n_buckets, w.n_hashes,
                                w.chunk_len, w.causal, key_norm=key_norm)
    gb, _ = lsh.hash(qk_t, R_t, w.n_buckets)
    differ = gb.cpu().numpy() != extra["buckets"]
    assert not np.any(differ & (extra["margin"] >= 1e-9)), "bucket ids differ above margin 1e-9"
    got_dqk = dqk.float().cpu().numpy()
    got_dv = dv.float().cpu().numpy()
    assert np.isfinite(got_dqk).all() and np.isfinite(got_dv).all()
    worst, compared = 0.0, 0
    for b in range(w.B):
        for h in range(w.H):
            if differ[b, h].any():
                continue
            compared += 1
            for got, ref in ((got_dqk[b, h], ref_dqk[b, h]), (got_dv[b, h], ref_dv[b, h])):
                worst = max(worst, float(np.abs(got - ref).max()) / float(np.abs(ref).max()))
    print(f"{w.name}: slices compared {compared} of {w.B * w.H}, worst relative {worst:.2e}")
    assert compared >= 1
    assert worst <= TOL[w.dtype]


@pytest.mark.parametrize("w,per_head", SEP_CASES, ids=[c[0].name for c in SEP_CASES])
def test_random_shape_separate_qk_matches_oracle(w, per_head):
    q, k, v, R = workloads.make_separate_inputs(w)
    if per_head:
        R = np.random.default_rng(w.seed + 1).standard_normal(
            (w.H, w.n_hashes, w.d, w.n_buckets // 2), dtype=np.float32)
    dt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    q_t = torch.from_numpy(q).to(DEV, dt)
    k_t = torch.from_numpy(k).to(DEV, dt)
    v_t = torch.from_numpy(v).to(DEV, dt)
    R_t = torch.from_numpy(R).to(DEV)
    ref, extra = oracle.forward_qk(q, k, v, R, w.n_buckets, w.chunk_len, w.causal,
                                   return_all=True)
    gq, _ = lsh.hash(q_t, R_t, w.n_buckets)
    gk, _ = lsh.hash(k_t, R_t, w.n_buckets)
    differ = np.zeros((w.B, w.H), bool)
    for g, side in ((gq, "q"), (gk, "k")):
        d = g.cpu().numpy() != extra[f"buckets_{side}"]
        assert not np.any(d & (extra[f"margin_{side}"] >= 1e-9)), \
            f"{side} bucket ids differ above margin 1e-9"
        differ |= d.any(axis=(2, 3))
    out = torch.full_like(q_t, float("nan"))
    lsh.attention_fwd_qk(q_t, k_t, v_t, R_t, w.n_buckets, w.chunk_len, w.causal, out=out)
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    # positions none of whose rounds has a key: zero rows on both sides
    none = np.isneginf(np.take_along_axis(extra["lse"], extra["inv_q"].astype(np.int64),
                                          axis=3)).all(axis=2)
    worst, compared = 0.0, 0
    for b in range(w.B):
        for h in range(w.H):
            if differ[b, h]:
                continue
            compared += 1
            worst = max(worst, float(np.abs(got[b, h] - ref[b, h]).max()))
            assert np.all(got[b, h][none[b, h]] == 0)
    print(f"{w.name}: slices compared {compared} of {w.B * w.H}, queries with no key "
          f"{int(none.sum())}, max |err| {worst:.2e}")
    assert compared >= 1
    assert worst <= TOL[w.dtype]


@pytest.mark.parametrize("name,B,H,nh,L,nb,kind,seed", SORT_CASES, ids=[c[0] for c in SORT_CASES])
def test_random_shape_sort_matches_oracle(name, B, H, nh, L, nb, kind, seed):
    rng = np.random.default_rng(seed)
    shape = (B, H, nh, L)
    if kind == "uniform":
        b = rng.integers(0, nb, shape)
    elif kind == "skewed":
        b = np.where(rng.random(shape) < 0.3, nb // 3, rng.integers(0, nb, shape))
    else:
        b = np.full(shape, int(rng.integers(0, nb)))
    b = b.astype(np.int32)
    perm, inv = lsh.sort(torch.from_numpy(b).to(DEV), nb)
    perm, inv = perm.cpu().numpy(), inv.cpu().numpy()
    for bi in range(B):
        for h in range(H):
            for r in range(nh):
                p_ref, i_ref = oracle.sort(b[bi, h, r])
                assert np.array_equal(perm[bi, h, r], p_ref), (bi, h, r)
                assert np.array_equal(inv[bi, h, r], i_ref), (bi, h, r)


def _draw_dense(n, seed, kind):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        dtype = "fp32" if rng.random() < 0.3 else "bf16"
        dm = 8 * int(rng.integers(1, 129))
        if kind == "proj":
            # token counts: half log-uniform (small and ragged), half several tiles
            B = int(rng.integers(1, 4))
            L = (int(round(np.exp(rng.uniform(0.0, np.log(1500.0))))) if rng.random() < 0.5
                 else int(rng.integers(256, 1501)))
            H, d = int(rng.integers(1, 9)), int(rng.choice([64, 128]))
            if B * L * dm * H * d > 3e9:
                continue
            cases.append((f"proj{len(cases)}_{dtype}_b{B}l{L}dm{dm}h{H}d{d}", dtype, B, L, dm, H,
                          d, seed + 1 + len(cases)))
        else:
            rows = (int(round(np.exp(rng.uniform(0.0, np.log(3000.0))))) if rng.random() < 0.5
                    else int(rng.integers(256, 3001)))
            dff = 8 * int(rng.integers(1, 513))
            chunk = int(rng.integers(1, rows + 1))
            bias = bool(rng.integers(0, 2))
            if rows * dm * dff > 6e9:
                continue
            cases.append((f"ffn{len(cases)}_{dtype}_rows{rows}dm{dm}dff{dff}c{chunk}"
                          f"{'_bias' if bias else ''}", dtype, rows, dm, dff, chunk, bias,
                          seed + 1 + len(cases)))
    return cases


PROJ_CASES = _draw_dense(12, 20261211, "proj")
FFN_CASES = _draw_dense(12, 20261212, "ffn")


def _io(a, dtype):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return workloads.round_to_bf16(a) if dtype == "bf16" else a


@pytest.mark.parametrize("name,dtype,B,L,dm,H,d,seed", PROJ_CASES, ids=[c[0] for c in PROJ_CASES])
def test_random_shape_projection_matches_oracle(name, dtype, B, L, dm, H, d, seed):
    rng = np.random.default_rng(seed)
    x = _io(rng.standard_normal((B, L, dm), dtype=np.float32), dtype)
    w_qk = _io(rng.standard_normal((H * d, dm), dtype=np.float32) / np.sqrt(dm), dtype)
    w_v = _io(rng.standard_normal((H * d, dm), dtype=np.float32) / np.sqrt(dm), dtype)
    dt = torch.float32 if dtype == "fp32" else torch.bfloat16
    qk_t, v_t = lsh.qkv_project(*(torch.from_numpy(a).to(DEV, dt) for a in (x, w_qk, w_v)), H)
    ref_qk, ref_v = oracle.project(x, w_qk, w_v, H)
    # sum_k |x_k w_k| per output: the scale of the fp32 accumulation error;
    # bf16 outputs are rounded once more (2^-9 relative)
    mag_qk, mag_v = oracle.project(np.abs(x), np.abs(w_qk), np.abs(w_v), H)
    rel = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -23
    for got_t, ref, mag in ((qk_t, ref_qk, mag_qk), (v_t, ref_v, mag_v)):
        got = got_t.float().cpu().numpy()
        assert np.isfinite(got).all()
        assert np.all(np.abs(got - ref) <= rel * np.abs(ref) + 2.0 ** -16 * mag)


@pytest.mark.parametrize("name,dtype,rows,dm,dff,chunk,bias,seed", FFN_CASES,
                         ids=[c[0] for c in FFN_CASES])
def test_random_shape_ffn_matches_oracle(name, dtype, rows, dm, dff, chunk, bias, seed):
    rng = np.random.default_rng(seed)
    x = _io(rng.standard_normal((rows, dm), dtype=np.float32), dtype)
    w1 = _io(rng.standard_normal((dff, dm), dtype=np.float32) / np.sqrt(dm), dtype)
    w2 = _io(rng.standard_normal((dm, dff), dtype=np.float32) / np.sqrt(dff), dtype)
    b1 = _io(rng.standard_normal(dff, dtype=np.float32) * 0.1, dtype) if bias else None
    b2 = _io(rng.standard_normal(dm, dtype=np.float32) * 0.1, dtype) if bias else None
    dt = torch.float32 if dtype == "fp32" else torch.bfloat16
    dev = [None if a is None else torch.from_numpy(a).to(DEV, dt) for a in (x, w1, b1, w2, b2)]
    got = lsh.ffn(*dev, chunk).float().cpu().numpy()
    ref = oracle.ffn(x, w1, b1, w2, b2, chunk)
    # hidden activations and output rounded to the I/O dtype, fp32 sums:
    # |gpu - ref| <= rel (|ref| + sum_f |h_f w2[o, f]|) + 1e-6
    h = x.astype(np.float64) @ w1.T.astype(np.float64) + (0.0 if b1 is None else b1)
    S = np.maximum(h, 0.0) @ np.abs(w2.astype(np.float64)).T
    rel = 2.0 ** -8 if dtype == "bf16" else 2e-5
    assert np.isfinite(got).all()
    assert np.all(np.abs(got - ref) <= rel * (np.abs(ref) + S) + 1e-6)


def _draw_ties(n=10, seed=20261213):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        dtype = "fp32" if rng.random() < 0.3 else "bf16"
        d = int(rng.choice([64, 128]))
        nb = 2 * int(round(np.exp(rng.uniform(np.log(2.0), np.log(2048.0)))))   # 4 ... 4096
        nh = int(rng.integers(1, 5))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        L = int(round(np.exp(rng.uniform(np.log(64.0), np.log(8192.0)))))
        if B * H * nh * L * nb * d > 2e10:
            continue
        i = len(cases)
        cases.append((f"ties{i}_{dtype}_b{B}h{H}l{L}d{d}_nb{nb}nh{nh}",
                      workloads.Workload(f"ties{i}", B, H, L, d, dtype, nb, nh, 1, False,
                                         seed + 1 + i)))
    return cases


TIE_CASES = _draw_ties()


@pytest.mark.parametrize("name,w", TIE_CASES, ids=[c[0] for c in TIE_CASES])
def test_random_shape_hash_exact_ties(name, w):
    qk, _, R = workloads.make_inputs(w)
    rng = np.random.default_rng(w.seed + 3)
    half = w.n_buckets // 2
    # per round, up to four columns copied onto later ones: exact ties
    pairs = []
    for r in range(w.n_hashes):
        for _ in range(min(4, half // 2)):
            c1, c2 = sorted(int(c) for c in rng.choice(half, 2, replace=False))
            R[r, :, c2] = R[r, :, c1]
            pairs.append((r, c1))
    # rows: 10 % zero (every column ties), 10 % along a copied column (+ or -)
    kind = rng.random((w.B, w.H, w.L))
    qk[kind < 0.1] = 0.0
    along = (kind >= 0.1) & (kind < 0.2)
    for b, h, l in zip(*np.nonzero(along)):
        r, c = pairs[int(rng.integers(0, len(pairs)))]
        qk[b, h, l] = R[r, :, c] * (1.0 if rng.random() < 0.5 else -1.0)
    dt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    qk_t = torch.from_numpy(qk).to(DEV, dt)
    qk = qk_t.float().cpu().numpy()   # the rows as the GPU holds them
    buckets, refined = lsh.hash(qk_t, torch.from_numpy(R).to(DEV), w.n_buckets)
    got = buckets.cpu().numpy()
    ties = 0
    for b in range(w.B):
        for h in range(w.H):
            ref, margin = oracle.hash(qk[b, h], R, w.n_buckets)
            ok = (got[b, h] == ref) | ((margin > 0) & (margin < 1e-9))
            assert ok.all(), (b, h, np.argwhere(~ok)[:4].tolist())
            ties += int((margin == 0).sum())
    print(f"{name}: exact ties {ties}, re-decided {refined}")
    assert ties > 0
