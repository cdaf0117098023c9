"""Host-side logic of bench.py (CPU only): the algorithmic work the roofline
fractions divide by, the whole-forward floor, the non-causal sweep's
workloads, and the rule that a committed rocprofv3 record is used only while
its kernel's source is unchanged."""
from __future__ import annotations

import hashlib
import json
import pathlib

import pytest

import bench
import workloads

HEAD = workloads.WORKLOADS[workloads.HEADLINE]


def test_headline_algorithmic_work():
    """At 64K tokens x 8 heads x 8 rounds, d 128, nb 1024 (bf16): the hash's
    projection is 2 d (nb / 2) flops per token-round (0.550 TFLOP); the chunk
    pass moves two gathered bf16 rows, the packed key and one fp16 row per
    token-round (772 B); the combine reads the 8 fp16 rows of a token-head
    and writes its bf16 output."""
    work = bench.algorithmic_work(HEAD)
    T = 8 * 65536
    assert work["hash_fast_mfma"] == ("mfma", 2.0 * 128 * 512 * 8 * T, "flop")
    assert work["hash_fast_mfma"][1] == pytest.approx(0.5497558e12, rel=1e-6)
    assert work["attend_mfma"][0] == "hbm"
    assert work["attend_mfma"][1] == T * 8 * 772
    assert work["combine"] == ("hbm", T * (8 * 256 + 256), "B")
    assert work["sort_scatter"] == ("hbm", 8.0 * T * 8, "B")


def test_headline_forward_floor():
    """The whole-forward floor at the headline: hash 0.220 ms (matrix cores),
    sort 0.006, chunk pass 0.405 and combine 0.151 ms (HBM at 8 TB/s)."""
    fr = bench.forward_roofline(HEAD, 1.0)
    steps = fr["steps"]
    assert steps["hash"]["bound"] == "compute"
    assert steps["chunk"]["bound"] == "hbm" and steps["combine"]["bound"] == "hbm"
    assert steps["hash"]["roof_ms"] == pytest.approx(0.2199, abs=5e-4)
    assert steps["sort"]["roof_ms"] == pytest.approx(0.0063, abs=5e-4)
    assert steps["chunk"]["roof_ms"] == pytest.approx(0.4047, abs=5e-4)
    assert steps["combine"]["roof_ms"] == pytest.approx(0.1510, abs=5e-4)
    assert fr["t_roof_ms"] == pytest.approx(0.782, abs=1e-3)
    assert fr["frac"] == pytest.approx(fr["t_roof_ms"])   # at 1 ms per step


def test_one_round_floor_has_no_combine():
    """With one round on the bf16 path the chunk pass writes the output
    itself: the floor counts no combine step, and the chunk step's write is
    the same 2 d bytes per token-round as the fp16 row it replaces."""
    w = workloads.WORKLOADS["sweep_b64_l1k_nh1"]
    fr = bench.forward_roofline(w, 1.0)
    assert fr["steps"]["combine"]["roof_ms"] == 0.0
    w8 = workloads.WORKLOADS["sweep_b64_l1k_nh8"]
    assert bench.forward_roofline(w8, 1.0)["steps"]["combine"]["roof_ms"] > 0.0
    assert fr["steps"]["chunk"]["roof_ms"] == pytest.approx(
        bench.forward_roofline(w8, 1.0)["steps"]["chunk"]["roof_ms"] / 8)


def test_noncausal_sweep_workloads_differ_only_in_the_mask():
    for name, w in workloads.WORKLOADS.items():
        if not name.startswith("sweep_"):
            continue
        nc = workloads.scaled(w, name=name + "_noncausal", causal=False)
        assert nc.causal is False and w.causal is True
        assert (nc.B, nc.H, nc.L, nc.d, nc.n_buckets, nc.n_hashes, nc.chunk_len, nc.seed) == \
            (w.B, w.H, w.L, w.d, w.n_buckets, w.n_hashes, w.chunk_len, w.seed)
        # same inputs: the generator does not depend on the mask
        assert nc.seed == w.seed and nc.qk_dist == w.qk_dist


def test_profile_record_only_while_the_source_is_unchanged(tmp_path, monkeypatch):
    """A record whose kernel source still hashes to the recorded value is
    returned; edit the source (or the recorded hash) and it is not."""
    root = tmp_path
    (root / "profiles").mkdir()
    csrc = root / "lsh_attention_fp32_amd" / "csrc"
    csrc.mkdir(parents=True)
    src = csrc / "lsh_hash.hip"
    src.write_text("// a kernel source\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    rec = {"rocprof_name": "k", "calls": 3, "avg_us": 600.0, "source": "lsh_hash.hip",
           "source_sha256": sha, "read_bytes": 1, "write_bytes": 2}
    (root / "profiles" / "kernels.json").write_text(json.dumps(
        {"workloads": {"w": {"kernels": {"hash_fast_mfma": rec}}}}))
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.profile_record("w", "hash_fast_mfma")["avg_us"] == 600.0
    assert bench.profile_record("w", "attend_mfma") is None
    assert bench.profile_record("other", "hash_fast_mfma") is None
    src.write_text("// the kernel source, edited\n")
    assert bench.profile_record("w", "hash_fast_mfma") is None


def test_committed_records_name_existing_sources():
    """Every committed record names a kernel source of the package and a
    64-hex-digit hash."""
    path = pathlib.Path(bench.ROOT) / "profiles" / "kernels.json"
    data = json.loads(path.read_text())
    assert data["workloads"]
    csrc = pathlib.Path(bench.ROOT) / "lsh_attention_fp32_amd" / "csrc"
    for wname, entry in data["workloads"].items():
        for kname, rec in entry["kernels"].items():
            assert (csrc / rec["source"]).exists(), (wname, kname)
            assert len(rec["source_sha256"]) == 64
            assert rec["avg_us"] > 0
