"""The library's entry points under HIP graph capture.

The fused forward, and the training forward followed by the backward, are
captured once into a graph (torch.cuda.CUDAGraph begins and ends the capture
on its stream; the library only launches kernels there: no allocation,
memset, copy or synchronisation), then replayed several times with other
device work between the replays. The inputs are rewritten before each replay,
alternating between two sets, so a replay that reused stale intermediate
state would show. Every replay must equal the eager result for the same
inputs bit for bit: the kernels are deterministic.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads

lsh = pytest.importorskip("lsh_attention_fp32_amd")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lsh.load_library()


def _inputs(w, seed_shift):
    qk, v, R = workloads.make_inputs(workloads.scaled(w, seed=w.seed + seed_shift))
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return (torch.from_numpy(qk).to(DEV, dt), torch.from_numpy(v).to(DEV, dt),
            torch.from_numpy(R).to(DEV))


def _other_work(q):
    # unrelated device work between replays: a product and a reduction
    a = q.reshape(-1, q.shape[-1])[:1024].float()
    return (a @ a.T).sum()


def _warm_then_capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name", ["b8_h8_l4k_nh4", "sweep_b64_l1k_nh1", "skewed_l16k_nh8"])
def test_forward_graph_replays_equal_eager(name):
    w = workloads.WORKLOADS[name]
    sets = [_inputs(w, 0), _inputs(w, 7)]
    shape = lsh.shape_of(sets[0][0], w.n_buckets, w.n_hashes, w.chunk_len, w.causal)
    ws = torch.empty(lsh.lsh_workspace_size("fwd", shape), dtype=torch.uint8, device=DEV)
    ref = []
    for q, v, R in sets:
        out = torch.full_like(q, float("nan"))
        lsh.lsh_attention_fwd(q, v, R, shape, out, ws)
        ref.append(out)
    torch.cuda.synchronize()

    q_s, v_s, R_s = (t.clone() for t in sets[0])
    out_s = torch.full_like(q_s, float("nan"))
    ws_s = torch.empty_like(ws)
    g = _warm_then_capture(lambda: lsh.lsh_attention_fwd(q_s, v_s, R_s, shape, out_s, ws_s))
    for i in range(REPLAYS):
        k = (i + 1) % 2   # start with the set the capture did not see
        q_s.copy_(sets[k][0])
        v_s.copy_(sets[k][1])
        R_s.copy_(sets[k][2])
        out_s.fill_(float("nan"))
        _other_work(sets[k][0])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_s, ref[k]), (name, i)
    print(f"{name}: {REPLAYS} forward replays equal the eager outputs")


@pytest.mark.parametrize("name", ["b8_h8_l4k_nh4"])
def test_train_step_graph_replays_equal_eager(name):
    w = workloads.WORKLOADS[name]
    sets = [_inputs(w, 0), _inputs(w, 11)]
    gen = torch.Generator(device="cpu").manual_seed(5)
    douts = [torch.randn(sets[0][0].shape, generator=gen).to(DEV, sets[0][0].dtype)
             for _ in range(2)]
    shape = lsh.shape_of(sets[0][0], w.n_buckets, w.n_hashes, w.chunk_len, w.causal)
    sz = {k: lsh.lsh_workspace_size(k, shape) for k in ("state", "fwd", "bwd")}
    new = lambda k: torch.empty(sz[k], dtype=torch.uint8, device=DEV)

    def step(q, v, R, dout, out, state, wsf, wsb, dqk, dv):
        lsh.lsh_attention_fwd_train(q, v, R, shape, out, state, wsf)
        lsh.lsh_attention_bwd(q, v, out, dout, state, shape, dqk, dv, wsb)

    ref = []
    for (q, v, R), dout in zip(sets, douts):
        out, dqk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(v)
        step(q, v, R, dout, out, new("state"), new("fwd"), new("bwd"), dqk, dv)
        ref.append((out, dqk, dv))
    torch.cuda.synchronize()

    q_s, v_s, R_s = (t.clone() for t in sets[0])
    dout_s = douts[0].clone()
    out_s, dqk_s, dv_s = torch.empty_like(q_s), torch.empty_like(q_s), torch.empty_like(v_s)
    bufs = (new("state"), new("fwd"), new("bwd"))
    g = _warm_then_capture(lambda: step(q_s, v_s, R_s, dout_s, out_s, *bufs, dqk_s, dv_s))
    for i in range(REPLAYS):
        k = (i + 1) % 2
        for dst, src in zip((q_s, v_s, R_s, dout_s), (*sets[k], douts[k])):
            dst.copy_(src)
        for t in (out_s, dqk_s, dv_s):
            t.fill_(float("nan"))
        _other_work(sets[k][0])
        g.replay()
        torch.cuda.synchronize()
        for got, want, what in zip((out_s, dqk_s, dv_s), ref[k], ("out", "dqk", "dv")):
            assert torch.equal(got, want), (name, i, what)
    print(f"{name}: {REPLAYS} training-step replays equal the eager forward and gradients")
