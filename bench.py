"""Benchmark of the LSH-attention forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
python bench.py --sweep [--dense]     one line per workload (length sweep and the rest)
python bench.py --project             input projections (d_model 1024) and the forward from x
python bench.py --train               training forward and backward
python bench.py --separate-qk         the separate-queries-and-keys ablation

A step is one lsh_attention_fwd (hash -> sort -> chunk attention -> combine)
over one batch of synthetic input already resident in HBM. The default
workload is the 64K-token, 8-head, 8-round configuration (d_head 128,
n_buckets 1024, chunk 64, causal, bf16). Prints one JSON line.

The per-kernel durations come from lsh_attention_fwd_timed (HIP events recorded
after every kernel on the launch stream), averaged over the timed repeats; the
roofline object reports the longest-running kernel against MI355X's published
peak for the bound that limits it, with that kernel's algorithmic work.
forward_roofline sums, over the method's four steps, the larger of (flops /
peak, algorithmic bytes / HBM peak) and divides by the measured forward time.

--dense adds, per sweep line, PyTorch's scaled_dot_product_attention (a
third-party dense comparator, flash or memory-efficient backend only) at the
same shape with is_causal matched, and the analytic dense-attention floor
4 B H L^2 d / bf16 MFMA peak; with --ffn or --project it adds PyTorch's
linear (hipBLASLt) at the same shapes.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LSH-attention fwd tokens/s at L=64K, 8 heads, 8 hashes; % of MFMA/HBM roofline"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_F16_TFLOPS = 2500.0       # MI355X dense fp16 / bf16 MFMA, TFLOP/s
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 (vector / matrix), TFLOP/s


def algorithmic_work(w):
    """Per-launch algorithmic flops or HBM bytes of each kernel, by kernel name.

    Returns {name: (bound, amount, unit)} with bound 'mfma' (amount in flops),
    'alu' (flops) or 'hbm' (amount in bytes)."""
    e = 2 if w.dtype == "bf16" else 4
    T = w.B * w.H * w.L                      # token-heads
    TR = T * w.n_hashes                      # token-rounds
    d, half = w.d, w.n_buckets // 2
    compact = w.dtype == "bf16" and w.chunk_len == 64   # fp16 per-round rows
    hash_flops = 2.0 * d * half * w.n_hashes * T
    return {
        # projection x R for every round, one fp16 matrix-core pass (fp32
        # accumulation); R prep and re-decision are separate entries
        "hash_fast_mfma": ("mfma", hash_flops, "flop"),
        "hash_fast_fp32": ("alu", hash_flops, "flop"),
        # read the buckets (count); read them again and write one packed key
        # per slot (scatter, fused forward)
        "sort_count": ("hbm", 4.0 * TR, "B"),
        # per (segment, tile, bucket) count read and prefix written back, plus
        # the segment totals: not per token-round work (tiny next to the keys)
        "sort_prefix": ("hbm", 4.0 * w.B * w.H * w.n_hashes * w.n_buckets
                        * (2 * -(-w.L // 4096) + 1), "B"),
        "sort_scatter": ("hbm", 8.0 * TR, "B"),
        # gather qk and v rows once per token-round, read the sorted key (and
        # bucket id), write the round's output row: fp32 plus a separate lse
        # on the plain path, fp16 with the lse carried in the row on the bf16
        # matrix-core path
        "attend_fp32": ("hbm", TR * (2 * d * e + 8 + 4 * d + 4), "B"),
        "attend_mfma": ("hbm", TR * (2 * d * e + 4 + 2 * d), "B"),
        # read every round's output row of a token (fp16 rows carry their lse;
        # fp32 rows come with an lse and an inverse-permutation entry); write out
        "combine": ("hbm", T * (w.n_hashes * (2 * d if compact else 4 * d + 8) + d * e), "B"),
    }


def forward_roofline(w, ms_per_step):
    """Whole-forward floor: for each step of the method the larger of its
    flops at the matching peak and its algorithmic HBM bytes at 8 TB/s
    (hash: read qk, write the ids; sort: read ids, write keys; chunk pass:
    gather rows, write per-round rows; combine: read them, write out; with
    one round on the bf16 path the chunk pass writes the output itself)."""
    e = 2 if w.dtype == "bf16" else 4
    T = w.B * w.H * w.L
    TR = T * w.n_hashes
    d = w.d
    compact = w.dtype == "bf16" and w.chunk_len == 64
    hash_peak = PEAK_F16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    steps = {
        "hash": (2.0 * d * (w.n_buckets // 2) * TR, hash_peak, T * (d * e + 4 * w.n_hashes)),
        "sort": (0.0, 1.0, 12.0 * TR),
        "chunk": (8.0 * w.chunk_len * d * TR, PEAK_F16_TFLOPS if compact else PEAK_FP32_TFLOPS,
                  TR * (2 * d * e + 4 + (2 * d if compact else 4 * d + 4))),
        "combine": (3.0 * w.n_hashes * d * T, PEAK_FP32_TFLOPS,
                    T * (w.n_hashes * (2 * d if compact else 4 * d + 8) + d * e)),
    }
    if compact and w.n_hashes == 1:
        # one round: its output is the forward's, written by the chunk pass
        # (d e bytes per token instead of the fp16 row), and nothing is combined
        steps["combine"] = (0.0, 1.0, 0.0)
    per = {}
    for k, (flops, peak, nbytes) in steps.items():
        t_c = flops / (peak * 1e12) * 1e3
        t_m = nbytes / (PEAK_HBM_GBS * 1e9) * 1e3
        per[k] = {"roof_ms": max(t_c, t_m), "bound": "hbm" if t_m >= t_c else "compute"}
    t_roof = sum(x["roof_ms"] for x in per.values())
    return {"t_roof_ms": t_roof, "frac": t_roof / ms_per_step, "steps": per}


def _rotations(w, per_head_r):
    """The workload's R, or with per-head rotations R [H, nh, d, nb/2] drawn
    from a generator seeded with the workload's seed + 1."""
    import numpy as np
    import workloads
    if not per_head_r:
        return workloads.make_inputs(w)[2]
    rng = np.random.default_rng(w.seed + 1)
    return rng.standard_normal((w.H, w.n_hashes, w.d, w.n_buckets // 2), dtype=np.float32)


def measure(lsh, torch, w, steps, warmup, key_norm=False, per_head_r=False):
    """Times `steps` back-to-back forwards on synthetic inputs resident in HBM,
    then the per-kernel event intervals of a few more."""
    import numpy as np
    import workloads

    dev = torch.device("cuda:0")
    qk, v, R = workloads.make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qk_t = torch.from_numpy(qk).to(dev, dt)
    v_t = torch.from_numpy(v).to(dev, dt)
    if per_head_r:
        R = _rotations(w, True)
    R_t = torch.from_numpy(R).to(dev)
    shape = lsh.shape_of(qk_t, w.n_buckets, w.n_hashes, w.chunk_len, w.causal, key_norm,
                         per_head_r)
    ws = torch.empty(lsh.lsh_workspace_size("fwd", shape), dtype=torch.uint8, device=dev)
    out = torch.empty_like(qk_t)

    for _ in range(warmup):
        lsh.lsh_attention_fwd(qk_t, v_t, R_t, shape, out, ws)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        lsh.lsh_attention_fwd(qk_t, v_t, R_t, shape, out, ws)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(stop) / steps
    refined = int(ws[:4].view(torch.int32).item())

    # per-kernel durations, same launches with an event after each kernel
    reps = max(3, min(steps, 10))
    acc = {}
    for _ in range(reps):
        for kname, ms in lsh.lsh_attention_fwd_timed(qk_t, v_t, R_t, shape, out, ws):
            acc.setdefault(kname, []).append(ms)
    kernels = {k: float(np.mean(x)) for k, x in acc.items()}
    return {"ms_per_step": ms_per_step, "wall": wall, "refined": refined, "kernels": kernels,
            "inputs": (qk, v, R), "tensors": (qk_t, v_t)}


def measure_separate(lsh, torch, w, steps, warmup):
    """lsh_attention_fwd_qk (queries and keys hashed and sorted separately) at
    the workload's shape, next to the shared forward on the same q as qk."""
    import workloads

    dev = torch.device("cuda:0")
    q, k, v, R = workloads.make_separate_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q_t, k_t, v_t = (torch.from_numpy(a).to(dev, dt) for a in (q, k, v))
    R_t = torch.from_numpy(R).to(dev)
    shape = lsh.shape_of(q_t, w.n_buckets, w.n_hashes, w.chunk_len, w.causal)
    out = torch.empty_like(q_t)
    ws = torch.empty(lsh.lsh_workspace_size("fwd_qk", shape), dtype=torch.uint8, device=dev)
    sep_ms = _timed_ms(torch, lambda: lsh.lsh_attention_fwd_qk(q_t, k_t, v_t, R_t, shape, out,
                                                               ws), steps, warmup)
    ws2 = torch.empty(lsh.lsh_workspace_size("fwd", shape), dtype=torch.uint8, device=dev)
    shared_ms = _timed_ms(torch, lambda: lsh.lsh_attention_fwd(q_t, v_t, R_t, shape, out, ws2),
                          steps, warmup)
    return {"variant": "separate_qk", "workload": w.name, "config": w.describe(),
            "ms_per_step": sep_ms, "tokens_per_s": w.B * w.L / (sep_ms / 1e3),
            "shared_qk_ms": shared_ms}


def measure_projection(lsh, torch, w, steps, warmup, d_model=1024, dense=False):
    """lsh_qkv_project and lsh_attention_fwd_x at the workload's shape with
    model width d_model (synthetic bf16 token vectors and weights)."""
    import numpy as np

    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    x = torch.randn((w.B, w.L, d_model), generator=g).to(dev, dt)
    wq = (torch.randn((w.H * w.d, d_model), generator=g) / np.sqrt(d_model)).to(dev, dt)
    wv = (torch.randn((w.H * w.d, d_model), generator=g) / np.sqrt(d_model)).to(dev, dt)
    R = torch.randn((w.n_hashes, w.d, w.n_buckets // 2), generator=g).to(dev)
    shape = lsh.Shape(w.B, w.H, w.L, w.d, w.n_buckets, w.n_hashes, w.chunk_len, int(w.causal),
                      lsh.LSH_BF16 if w.dtype == "bf16" else lsh.LSH_F32)
    qk = torch.empty((w.B, w.H, w.L, w.d), dtype=dt, device=dev)
    v = torch.empty_like(qk)
    out = torch.empty_like(qk)
    ws = torch.empty(lsh.lsh_workspace_size("fwd_x", shape), dtype=torch.uint8, device=dev)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    p_ms = timed(lambda: lsh.lsh_qkv_project(x, wq, wv, shape, d_model, qk, v))
    f_ms = timed(lambda: lsh.lsh_attention_fwd_x(x, wq, wv, R, shape, d_model, out, ws))
    flops = 2.0 * w.B * w.L * d_model * 2 * w.H * w.d
    peak = PEAK_F16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    line = {"workload": f"{w.name}_dmodel{d_model}", "project_ms": p_ms,
            "project_tflops": flops / p_ms / 1e9, "project_frac": flops / p_ms / 1e9 / peak,
            "project_bytes": (w.B * w.L * d_model + 2 * w.H * w.d * d_model
                              + 2 * w.B * w.H * w.L * w.d) * (2 if w.dtype == "bf16" else 4),
            "fwd_x_ms": f_ms, "fwd_x_tokens_per_s": w.B * w.L / (f_ms / 1e3)}
    if dense:
        import torch.nn.functional as F
        wcat = torch.cat([wq, wv])
        x2 = x.view(-1, d_model)
        t_ms = timed(lambda: F.linear(x2, wcat))
        line["torch_linear"] = {"ms": t_ms, "tflops": flops / t_ms / 1e9,
                                "note": "one torch.nn.functional.linear of x by [W_qk; W_v] "
                                        "(hipBLASLt) into [B L, 2 H d], no head split"}
    return line


def measure_training(lsh, torch, w, steps, warmup, key_norm=False, per_head_r=False):
    """lsh_attention_fwd_train and lsh_attention_bwd at the workload's shape;
    the backward's work is counted per (query, window key) pair: the score
    and g . v recomputed, then dq, dk and dv, 10 d flops."""
    import workloads

    dev = torch.device("cuda:0")
    qk, v, R = workloads.make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qk_t = torch.from_numpy(qk).to(dev, dt)
    v_t = torch.from_numpy(v).to(dev, dt)
    R_t = torch.from_numpy(_rotations(w, True) if per_head_r else R).to(dev)
    g_t = torch.randn(qk_t.shape, generator=torch.Generator().manual_seed(w.seed)).to(dev, dt)
    shape = lsh.shape_of(qk_t, w.n_buckets, w.n_hashes, w.chunk_len, w.causal, key_norm,
                         per_head_r)
    out = torch.empty_like(qk_t)
    state = torch.empty(lsh.lsh_workspace_size("state", shape), dtype=torch.uint8, device=dev)
    ws = torch.empty(lsh.lsh_workspace_size("fwd", shape), dtype=torch.uint8, device=dev)
    bws = torch.empty(lsh.lsh_workspace_size("bwd", shape), dtype=torch.uint8, device=dev)
    dqk = torch.empty_like(qk_t)
    dv = torch.empty_like(v_t)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    f_ms = timed(lambda: lsh.lsh_attention_fwd_train(qk_t, v_t, R_t, shape, out, state, ws))
    b_ms = timed(lambda: lsh.lsh_attention_bwd(qk_t, v_t, out, g_t, state, shape, dqk, dv, bws))
    T = w.B * w.H * w.L
    pairs = T * w.n_hashes * (2 * w.chunk_len - w.chunk_len * w.chunk_len / w.L)
    flops = 10.0 * w.d * pairs
    # bf16 with chunk 64 runs on the matrix cores (bf16 products), else fp32 vector
    mfma = w.dtype == "bf16" and w.chunk_len == 64
    peak = PEAK_F16_TFLOPS if mfma else PEAK_FP32_TFLOPS
    return {"workload": w.name, "key_norm": bool(key_norm), "per_head_r": bool(per_head_r),
            "fwd_train_ms": f_ms, "bwd_ms": b_ms,
            "train_step_tokens_per_s": w.B * w.L / ((f_ms + b_ms) / 1e3),
            "bwd_pair_flops": flops, "bwd_tflops": flops / b_ms / 1e9,
            "bwd_peak": "bf16 mfma" if mfma else "fp32 vector",
            "bwd_frac": flops / b_ms / 1e9 / peak}


def measure_ffn(lsh, torch, steps, warmup, rows=65536, d_model=1024, d_ff=4096, chunk=16384,
                dense=False):
    """The chunked feed-forward at the pages' widths (d_model 1024, d_ff 4096)
    over 64K token rows in bf16, synthetic inputs resident in HBM. Work:
    2 products of 2 * rows * d_model * d_ff flops each. ``dense``: also time
    PyTorch's linear (hipBLASLt) + relu over the same chunks, a third-party
    comparator."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(1006)
    mk = lambda *sh, sc=1.0: (torch.randn(*sh, generator=g) * sc).to(dev, torch.bfloat16)
    x = mk(rows, d_model)
    w1, b1 = mk(d_ff, d_model, sc=d_model ** -0.5), mk(d_ff, sc=0.1)
    w2, b2 = mk(d_model, d_ff, sc=d_ff ** -0.5), mk(d_model, sc=0.1)
    out = torch.empty_like(x)
    ws = torch.empty(lsh.lsh_ffn_workspace_size(rows, d_ff, chunk, lsh.LSH_BF16),
                     dtype=torch.uint8, device=dev)
    run = lambda: lsh.ffn(x, w1, b1, w2, b2, chunk, ws=ws, out=out)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    flops = 4.0 * rows * d_model * d_ff
    launches = 2 * ((rows + chunk - 1) // chunk)
    line = {"workload": "ffn_rows64k_dmodel1024_dff4096", "rows": rows, "d_model": d_model,
            "d_ff": d_ff, "chunk_rows": chunk, "dtype": "bf16", "ms": ms,
            "tokens_per_s": rows / (ms / 1e3), "tflops": flops / ms / 1e9,
            "peak_tflops": PEAK_F16_TFLOPS, "frac": flops / ms / 1e9 / PEAK_F16_TFLOPS,
            "launches": launches, "ms_per_launch": ms / launches}
    if dense:
        import torch.nn.functional as F

        def ref():
            for c in range(0, rows, chunk):
                F.linear(torch.relu(F.linear(x[c:c + chunk], w1, b1)), w2, b2)
        t_ms = _timed_ms(torch, ref, steps, warmup)
        line["torch_linear"] = {"ms": t_ms, "tflops": flops / t_ms / 1e9,
                                "note": "torch.nn.functional.linear (hipBLASLt) + relu, same chunks"}
    return line


def _timed_ms(torch, fn, steps, warmup):
    for _ in range(max(1, warmup)):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def dense_comparator(torch, w, qk_t, v_t, steps=10):
    """PyTorch SDPA at the same shape (queries = keys = qk), flash or
    memory-efficient backend only; None when neither takes the shape."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    import torch.nn.functional as F

    if w.dtype != "bf16":
        return None
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
            for _ in range(2):
                F.scaled_dot_product_attention(qk_t, qk_t, v_t, is_causal=bool(w.causal))
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(steps):
                F.scaled_dot_product_attention(qk_t, qk_t, v_t, is_causal=bool(w.causal))
            b.record()
            torch.cuda.synchronize()
    except RuntimeError as ex:
        return {"ms": None, "note": str(ex).splitlines()[0][:120]}
    ms = a.elapsed_time(b) / steps
    floor = 4.0 * w.B * w.H * w.L * w.L * w.d / (PEAK_F16_TFLOPS * 1e12) * 1e3
    return {"kind": "third-party: torch scaled_dot_product_attention", "ms": ms,
            "tokens_per_s": w.B * w.L / (ms / 1e3), "analytic_dense_floor_ms": floor}


def _cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo ("unknown" elsewhere)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, qk, v, R, target_s=12.0):
    """Times the oracle (as it is) on a bounded sample of the workload: whole
    (batch, head) slices with every round, as many heads of batch row 0 as fit
    in about target_s (first shortening L if one slice alone is too long).
    A token of the metric passes through all H heads, so the sample's rate is
    scaled by (heads timed) / H."""
    from oracle import oracle

    L, heads = w.L, 1
    while True:
        t0 = time.perf_counter()
        oracle.forward(qk[:1, :heads, :L], v[:1, :heads, :L], R, w.n_buckets, w.chunk_len,
                       w.causal)
        dt = time.perf_counter() - t0
        if dt * 2.5 <= target_s and heads < w.H and L == w.L:
            heads = min(w.H, max(heads + 1, int(target_s / (dt / heads))))
            continue
        if dt <= 2.5 * target_s or L <= 4 * w.chunk_len:
            break
        L //= 2
    return {"value": L * heads / w.H / dt, "unit": "tokens/s", "cores": oracle.threads(),
            "threads": oracle.threads(), "nproc": os.cpu_count(), "cpu_model": _cpu_model(),
            "kind": "oracle",
            "sample": f"batch row 0, {heads} of {w.H} heads, first {L} positions, all "
                      f"{w.n_hashes} rounds: {dt:.1f} s; rate scaled by {heads}/{w.H} heads"}


def profile_record(name, kernel):
    """The committed rocprofv3 record of `kernel` at workload `name`
    (profiles/kernels.json: the kernel-trace average duration and, when
    counters were taken, HBM-side bytes from FETCH_SIZE / WRITE_SIZE scaled by a
    plain copy's readings and the matrix pipe's busy share), or None when the
    kernel's source has changed since it was measured."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "kernels.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get("workloads", {}).get(name, {}).get("kernels", {}).get(kernel)
    if not rec:
        return None
    src = os.path.join(ROOT, "lsh_attention_fp32_amd", "csrc", rec["source"])
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["source_sha256"]:
        return None
    return rec


def kernel_rooflines(w, name, kernels):
    """Per kernel: event-timed ms, its algorithmic work against the peak of the
    roof that binds it, and (from the committed profile, when current) the
    rocprofv3 average, counted HBM traffic and matrix-pipe busy share."""
    work = algorithmic_work(w)
    out = {}
    for k, ms in kernels.items():
        e = {"ms": ms}
        if k in work:
            bound, amount, _ = work[k]
            secs = ms / 1e3
            if bound == "hbm":
                e.update(bound="hbm", achieved=amount / secs / 1e9, unit="GB/s", peak=PEAK_HBM_GBS)
            elif bound == "mfma":
                e.update(bound="mfma", achieved=amount / secs / 1e12, unit="TFLOP/s",
                         peak=PEAK_F16_TFLOPS)
            else:
                e.update(bound="alu", achieved=amount / secs / 1e12, unit="TFLOP/s",
                         peak=PEAK_FP32_TFLOPS)
            e["frac"] = e["achieved"] / e["peak"]
        rec = profile_record(name, k)
        if rec:
            e["rocprof_ms"] = rec.get("avg_us", 0.0) / 1e3 or None
            tb = rec.get("read_bytes")
            if tb is not None:
                e["traffic_bytes"] = tb + rec["write_bytes"]
                e["hbm_gbs_counted"] = e["traffic_bytes"] / (ms / 1e3) / 1e9
            if rec.get("mfma_busy") is not None:
                e["mfma_busy"] = rec["mfma_busy"]
        out[k] = e
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (to scale HBM byte counters)")
    ap.add_argument("--sweep", action="store_true",
                    help="one JSON line per workload: the length sweep, then the others")
    ap.add_argument("--dense", action="store_true",
                    help="with --sweep: also time torch's dense SDPA at each shape; with "
                         "--ffn or --project: also time torch's linear (hipBLASLt) at the "
                         "same shapes")
    ap.add_argument("--project", action="store_true",
                    help="time the input projections and the forward that starts from x")
    ap.add_argument("--train", action="store_true",
                    help="time the training forward and the backward")
    ap.add_argument("--key-norm", action="store_true",
                    help="time the key-normalisation variant (forward, or with --train both "
                         "passes) instead of the headline line")
    ap.add_argument("--ffn", action="store_true",
                    help="time the chunked feed-forward (64K rows, 1024 -> 4096 -> 1024, bf16)")
    ap.add_argument("--ffn-chunk", type=int, default=16384,
                    help="rows per chunk of the feed-forward (with --ffn)")
    ap.add_argument("--separate-qk", action="store_true",
                    help="time the separate-queries-and-keys ablation (lsh_attention_fwd_qk) "
                         "at the workload's shape")
    ap.add_argument("--non-causal", action="store_true",
                    help="with --sweep: the sixteen length-sweep points without the causal "
                         "mask (the sweep's workloads are causal)")
    ap.add_argument("--per-head-r", action="store_true",
                    help="time the per-head rotations variant (R [H, nh, d, nb/2]); combines "
                         "with --key-norm and --train")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "launches": 3}))
        return 0
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the forward shards "
                                   "by (batch, head) with no communication, so --gpus must be 1"}))
        return 2

    import torch

    import lsh_attention_fp32_amd as lsh
    import workloads

    lsh.load_library()
    if args.sweep:
        names = [n for n in workloads.WORKLOADS if n.startswith("sweep_")]
        if not args.non_causal:
            names += [n for n in workloads.WORKLOADS if not n.startswith("sweep_")]
        for n in names:
            w = workloads.WORKLOADS[n]
            if args.non_causal:
                n = n + "_noncausal"
                w = workloads.scaled(w, name=n, causal=False)
            r = measure(lsh, torch, w, min(args.steps, 10), args.warmup)
            line = {"workload": n, "config": w.describe(), "ms_per_step": r["ms_per_step"],
                    "tokens_per_s": w.B * w.L / (r["ms_per_step"] / 1e3),
                    "kernels_ms": r["kernels"], "kernels": kernel_rooflines(w, n, r["kernels"]),
                    "hash_redecided": r["refined"],
                    "forward_roofline": forward_roofline(w, r["ms_per_step"])}
            if args.dense:
                line["dense"] = dense_comparator(torch, w, *r["tensors"])
            del r
            torch.cuda.empty_cache()
            print(json.dumps(line), flush=True)
        return 0

    if args.train:
        print(json.dumps(measure_training(lsh, torch, workloads.WORKLOADS[
            args.workload or workloads.HEADLINE], min(args.steps, 10), args.warmup,
            key_norm=args.key_norm, per_head_r=args.per_head_r)), flush=True)
        return 0

    if args.ffn:
        print(json.dumps(measure_ffn(lsh, torch, min(args.steps, 10), args.warmup,
                                     chunk=args.ffn_chunk, dense=args.dense)), flush=True)
        return 0

    if args.separate_qk:
        print(json.dumps(measure_separate(lsh, torch, workloads.WORKLOADS[
            args.workload or workloads.HEADLINE], args.steps, args.warmup)), flush=True)
        return 0

    if args.key_norm or args.per_head_r:
        name = args.workload or workloads.HEADLINE
        w = workloads.WORKLOADS[name]
        r = measure(lsh, torch, w, args.steps, args.warmup, key_norm=args.key_norm,
                    per_head_r=args.per_head_r)
        variant = "+".join(n for n, on in (("key_norm", args.key_norm),
                                           ("per_head_r", args.per_head_r)) if on)
        print(json.dumps({"variant": variant, "workload": name, "config": w.describe(),
                          "ms_per_step": r["ms_per_step"],
                          "tokens_per_s": w.B * w.L / (r["ms_per_step"] / 1e3),
                          "kernels_ms": r["kernels"],
                          "forward_roofline": forward_roofline(w, r["ms_per_step"])}),
              flush=True)
        return 0

    if args.project:
        print(json.dumps(measure_projection(lsh, torch, workloads.WORKLOADS[
            args.workload or workloads.HEADLINE], args.steps, args.warmup,
            dense=args.dense)), flush=True)
        return 0

    name = args.workload or workloads.HEADLINE
    w = workloads.WORKLOADS[name]
    r = measure(lsh, torch, w, args.steps, args.warmup)
    ms_per_step, wall, refined, kernels = r["ms_per_step"], r["wall"], r["refined"], r["kernels"]
    qk, v, R = r["inputs"]
    work = algorithmic_work(w)
    dominant = max((k for k in kernels if k in work), key=lambda k: kernels[k])
    bound, amount, _unit = work[dominant]
    secs = kernels[dominant] / 1e3
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": amount / secs / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    elif bound == "mfma":
        roof = {"bound": "mfma", "achieved": amount / secs / 1e12, "peak": PEAK_F16_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "alu", "achieved": amount / secs / 1e12, "peak": PEAK_FP32_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    rec = profile_record(name, dominant)
    roof["traffic"] = (rec["read_bytes"] + rec["write_bytes"]) if rec and "read_bytes" in rec \
        else None
    roof["kernel"] = dominant
    roof["kernel_ms"] = kernels[dominant]
    # the same fraction from the committed rocprofv3 kernel-trace average
    if rec and rec.get("avg_us"):
        roof["kernel_ms_rocprof"] = rec["avg_us"] / 1e3
        roof["frac_rocprof"] = roof["frac"] * kernels[dominant] / roof["kernel_ms_rocprof"]

    tokens = w.B * w.L
    line = {
        "metric": METRIC,
        "value": tokens / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "fp32",
        "data": "synthetic",
        "config": {"workload": name, "B": w.B, "H": w.H, "L": w.L, "d_head": w.d,
                   "n_buckets": w.n_buckets, "n_hashes": w.n_hashes, "chunk_len": w.chunk_len,
                   "causal": w.causal, "qk_dist": w.qk_dist},
        "roofline": roof,
        "forward_roofline": forward_roofline(w, ms_per_step),
        "kernels_ms": kernels,
        "kernels": kernel_rooflines(w, name, kernels),
        "hash_redecided": refined,
        "wall_s_timed": wall,
    }
    if args.dense:
        line["dense"] = dense_comparator(torch, w, *r["tensors"])
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, qk, v, R)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
