"""Seeded synthetic inputs for LSH attention, shaped like the pages' workloads.

This module only draws random inputs: it holds none of the method's
arithmetic, and both the GPU tests/benchmark and the CPU oracle take their
inputs from it.

Shapes follow the experiments the Reformer pages describe (ai-scholar.tech
summary, section "Reformerを用いた結果": 64K-token sequences, d_model 1024 split
over 8 heads, 8 hash rounds being close to full attention). The pages train on
enwik8-64K and imagenet64; those datasets are not used -- Gaussian (or
clustered Gaussian) vectors of the same shapes stand in for the projected
shared query/key and value activations.

Recipe (identical for every workload):
  * ``numpy.random.default_rng(seed)`` (PCG64), ``standard_normal`` in float32;
  * draw order: qk, then v, then R (shape [n_hashes, d, n_buckets/2], kept in
    float32);
  * bf16 workloads round qk and v to bfloat16 with round-to-nearest-even; the
    returned float32 arrays hold those exact bf16 values;
  * the "clusters" distribution (skewed buckets): 64 centres c_k ~ N(0, I_d),
    weights p_k proportional to k^-1.1 (Zipf 1.1 truncated to 64 ranks), per
    (batch, head, position) a centre k ~ p and x = c_k + 0.1 * N(0, I_d). The
    centres, then the centre choices, then the noise are drawn before v and R;
  * separate queries and keys (make_separate_inputs): q, k, v, R in that
    order from the seed + 7919, each of q and k drawn as qk would be.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    d: int
    dtype: str            # "fp32" or "bf16": the I/O dtype of qk, v and out
    n_buckets: int
    n_hashes: int
    chunk_len: int
    causal: bool
    seed: int
    qk_dist: str = "normal"   # "normal" or "clusters"

    @property
    def tokens(self) -> int:
        return self.B * self.L

    def describe(self) -> dict:
        return dataclasses.asdict(self)


def _sweep():
    out = {}
    idx = 0
    for B, L in ((64, 1024), (16, 4096), (4, 16384), (1, 65536)):
        for nh in (1, 2, 4, 8):
            name = f"sweep_b{B}_l{L // 1024}k_nh{nh}"
            out[name] = Workload(name, B, 8, L, 64, "bf16", L // 32, nh, 64, True, 1004 + idx)
            idx += 1
    return out


WORKLOADS: dict[str, Workload] = {
    # small single-head fp32 case, fast enough for the oracle in seconds
    "single_head_l1k_fp32": Workload("single_head_l1k_fp32", 1, 1, 1024, 64, "fp32", 16, 1, 64,
                                     False, 1001),
    # batch 8, 8 heads, 4K tokens, 4 rounds
    "b8_h8_l4k_nh4": Workload("b8_h8_l4k_nh4", 8, 8, 4096, 64, "bf16", 64, 4, 64, True, 1002),
    # the headline: 64K tokens, 8 heads of 128 (d_model 1024), 8 rounds
    "l64k_h8_d128_nh8": Workload("l64k_h8_d128_nh8", 1, 8, 65536, 128, "bf16", 1024, 8, 64, True,
                                 1003),
    # skewed buckets from clustered keys
    "skewed_l16k_nh8": Workload("skewed_l16k_nh8", 1, 8, 16384, 64, "bf16", 256, 8, 64, True,
                                1005, "clusters"),
}
WORKLOADS.update(_sweep())

HEADLINE = "l64k_h8_d128_nh8"


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even), kept as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    bias = ((bits >> 16) & 1) + 0x7FFF
    rounded = ((bits + bias) & 0xFFFF0000).astype(np.uint32)
    return rounded.view(np.float32)


def _cluster_qk(rng: np.random.Generator, B: int, H: int, L: int, d: int) -> np.ndarray:
    n_centres = 64
    centres = rng.standard_normal((n_centres, d), dtype=np.float32)
    w = np.arange(1, n_centres + 1, dtype=np.float64) ** -1.1
    w /= w.sum()
    choice = rng.choice(n_centres, size=(B, H, L), p=w)
    noise = rng.standard_normal((B, H, L, d), dtype=np.float32)
    return centres[choice] + np.float32(0.1) * noise


def make_inputs(w: Workload, seed: int | None = None):
    """Return (qk [B,H,L,d], v [B,H,L,d], R [n_hashes, d, n_buckets/2]) as float32."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.L, w.d)
    if w.qk_dist == "normal":
        qk = rng.standard_normal(shape, dtype=np.float32)
    elif w.qk_dist == "clusters":
        qk = _cluster_qk(rng, w.B, w.H, w.L, w.d)
    else:
        raise ValueError(f"unknown qk distribution {w.qk_dist!r}")
    v = rng.standard_normal(shape, dtype=np.float32)
    R = rng.standard_normal((w.n_hashes, w.d, w.n_buckets // 2), dtype=np.float32)
    if w.dtype == "bf16":
        qk = round_to_bf16(qk)
        v = round_to_bf16(v)
    elif w.dtype != "fp32":
        raise ValueError(f"unknown dtype {w.dtype!r}")
    return qk, v, R


def make_separate_inputs(w: Workload, seed: int | None = None):
    """Inputs for separate queries and keys: (q, k, v [B,H,L,d], R [n_hashes,
    d, n_buckets/2]) as float32. Same recipe as make_inputs with the draw
    order q, k, v, R (q and k from the workload's distribution; with
    clusters, q and k are drawn around the same centres)."""
    rng = np.random.default_rng(w.seed + 7919 if seed is None else seed)
    shape = (w.B, w.H, w.L, w.d)
    if w.qk_dist == "normal":
        q = rng.standard_normal(shape, dtype=np.float32)
        k = rng.standard_normal(shape, dtype=np.float32)
    elif w.qk_dist == "clusters":
        n_centres = 64
        centres = rng.standard_normal((n_centres, w.d), dtype=np.float32)
        p = np.arange(1, n_centres + 1, dtype=np.float64) ** -1.1
        p /= p.sum()
        q = centres[rng.choice(n_centres, size=shape[:3], p=p)] + np.float32(0.1) * \
            rng.standard_normal(shape, dtype=np.float32)
        k = centres[rng.choice(n_centres, size=shape[:3], p=p)] + np.float32(0.1) * \
            rng.standard_normal(shape, dtype=np.float32)
    else:
        raise ValueError(f"unknown qk distribution {w.qk_dist!r}")
    v = rng.standard_normal(shape, dtype=np.float32)
    R = rng.standard_normal((w.n_hashes, w.d, w.n_buckets // 2), dtype=np.float32)
    if w.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    elif w.dtype != "fp32":
        raise ValueError(f"unknown dtype {w.dtype!r}")
    return q, k, v, R


def scaled(w: Workload, **changes) -> Workload:
    """A copy of ``w`` with some fields replaced (e.g. a shorter L for a test)."""
    return dataclasses.replace(w, **changes)


def glossary_hash_example():
    """Inputs of the worked hashing example on the ultralytics.com glossary page
    (section "Atenção LSH"): torch's generator seeded with 0, a 64-dim query,
    a "near" vector = query + 0.3 * noise, an unrelated "far" vector, and
    R ~ N(0, 1) of shape [1000 rounds, 64, 16 buckets / 2], drawn in that order.

    Returns float32 arrays (x [3, 64] rows = query, near, far; R [1000, 64, 8]).
    """
    import torch

    gen = torch.Generator().manual_seed(0)
    dim, rounds, half = 64, 1000, 8
    query = torch.randn(dim, generator=gen)
    near = query + 0.3 * torch.randn(dim, generator=gen)
    far = torch.randn(dim, generator=gen)
    R = torch.randn(rounds, dim, half, generator=gen)
    x = torch.stack([query, near, far])
    return x.numpy().astype(np.float32), R.numpy().astype(np.float32)
