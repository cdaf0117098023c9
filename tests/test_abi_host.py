"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The library must load without a GPU, export every function that
include/lsh_attn.h declares, and reject bad arguments on the host with the
documented error codes before touching the device.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import lsh_attention_fp32_amd as lsh

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsh_attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(lsh_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not lsh.library_path().exists():
        pytest.fail("liblsh_attn.so is not built (run __graft_entry__.build())")
    return lsh.load_library()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("lsh_hash", "lsh_sort", "lsh_chunk_attend", "lsh_unsort_combine",
              "lsh_attention_fwd", "lsh_workspace_size", "lsh_last_error",
              "lsh_attention_fwd_timed", "lsh_qkv_project", "lsh_attention_fwd_x",
              "lsh_attention_fwd_train", "lsh_attention_bwd", "lsh_ffn_chunked",
              "lsh_ffn_workspace_size"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), f"{name} declared in lsh_attn.h but not exported"


def _shape(**kw):
    base = dict(B=1, H=2, L=256, d=64, n_buckets=16, n_hashes=2, chunk_len=64, causal=1,
                dtype=lsh.LSH_BF16)
    base.update(kw)
    return lsh.Shape(**base)


@pytest.mark.parametrize("kw, code", [
    (dict(n_buckets=15), -1), (dict(n_buckets=0), -1), (dict(n_hashes=0), -1),
    (dict(chunk_len=0), -1), (dict(L=100, chunk_len=64), -1), (dict(causal=2), -1),
    (dict(dtype=7), -1), (dict(B=-1), -1), (dict(d=96), -1), (dict(n_buckets=8192), -1),
    (dict(B=64, H=64, L=65536, n_hashes=8, chunk_len=64), -1),
    (dict(flags=4), -1), (dict(flags=-1), -1),
])
def test_workspace_size_rejects_bad_shapes(lib, kw, code):
    with pytest.raises(lsh.LshError) as ei:
        lsh.lsh_workspace_size("fwd", _shape(**kw))
    assert ei.value.code == code
    assert lsh.lsh_last_error()


def test_workspace_size_is_a_size_t_with_zero_on_error(lib):
    """size_t lsh_workspace_size(stage, shape): the size, with an empty
    message; 0 and a message for an unknown or NULL stage or a bad shape."""
    s = _shape()
    n = lib.lsh_workspace_size(b"fwd", ctypes.byref(s))
    assert n > 0 and lsh.lsh_last_error() == ""
    assert lib.lsh_workspace_size(b"nope", ctypes.byref(s)) == 0
    assert "unknown stage" in lsh.lsh_last_error()
    assert lib.lsh_workspace_size(None, ctypes.byref(s)) == 0
    assert "stage" in lsh.lsh_last_error()
    bad = _shape(d=96)
    assert lib.lsh_workspace_size(b"fwd", ctypes.byref(bad)) == 0
    assert "d must be 64 or 128" in lsh.lsh_last_error()
    assert lib.lsh_workspace_size(b"fwd", None) == 0
    # the message is cleared by the next successful call
    assert lib.lsh_workspace_size(b"sort", ctypes.byref(s)) > 0 and lsh.lsh_last_error() == ""
    # a valid empty problem can need no sort workspace at all: size 0, no message
    assert lib.lsh_workspace_size(b"sort", ctypes.byref(_shape(B=0))) == 0
    assert lsh.lsh_last_error() == ""
    assert lib.lsh_ffn_workspace_size(10, 12, 4, lsh.LSH_BF16) == 0 and lsh.lsh_last_error()
    assert lib.lsh_ffn_workspace_size(0, 64, 4, lsh.LSH_BF16) == 0
    assert lsh.lsh_last_error() == ""


def test_workspace_sizes_are_consistent(lib):
    # the fused forward keeps per-round outputs in fp16 on the bf16 matrix-core
    # path (chunk 64) and in fp32 otherwise; the fp16 rows carry their own lse
    # and, with packed sort keys, need no inverse, so only buckets and perm
    # remain of the four int32/fp32 per-slot arrays there
    for dtype, m, o_bytes, per_slot in ((lsh.LSH_BF16, 64, 2, 2), (lsh.LSH_F32, 64, 4, 4),
                                        (lsh.LSH_BF16, 32, 4, 4)):
        s = _shape(dtype=dtype, chunk_len=m)
        h, so, f = (lsh.lsh_workspace_size(k, s) for k in ("hash", "sort", "fwd"))
        n = s.B * s.H * s.n_hashes * s.L
        assert h > 0 and so > 0
        assert f >= h + so + n * (4 * per_slot + o_bytes * s.d)
    s = _shape()
    with pytest.raises(lsh.LshError):
        lsh.lsh_workspace_size("nope", s)


def test_entry_points_reject_on_host(lib):
    s = _shape(d=96)
    vp = ctypes.c_void_p
    assert lib.lsh_attention_fwd(None, None, None, ctypes.byref(s), None, None, 0, None) == -1
    s = _shape()
    # NULL tensors are refused before anything reaches the device
    assert lib.lsh_hash(None, None, ctypes.byref(s), None, None, 0, None) == -1
    assert lib.lsh_sort(None, ctypes.byref(s), None, None, None, 0, None) == -1
    assert lib.lsh_chunk_attend(None, None, None, None, ctypes.byref(s), None, None, None) == -1
    assert lib.lsh_unsort_combine(None, None, None, ctypes.byref(s), None, None) == -1
    # a missing or short workspace is LSH_ERR_WORKSPACE
    fake = vp(0x1000)
    assert lib.lsh_hash(fake, fake, ctypes.byref(s), fake, None, 0, None) == -2
    assert lib.lsh_hash(fake, fake, ctypes.byref(s), fake, fake, 16, None) == -2
    assert lib.lsh_sort(fake, ctypes.byref(s), fake, fake, fake, 16, None) == -2
    assert lib.lsh_attention_fwd(fake, fake, fake, ctypes.byref(s), fake, fake, 16, None) == -2
    assert b"workspace" in lib.lsh_last_error()
    assert lib.lsh_attention_fwd(None, None, None, None, None, None, 0, None) == -1
    # pointers must be 16-byte aligned; the check runs before anything is enqueued
    odd = vp(0x1008)
    assert lib.lsh_hash(odd, fake, ctypes.byref(s), fake, fake, 1 << 40, None) == -1
    assert b"aligned" in lib.lsh_last_error()
    assert lib.lsh_sort(fake, ctypes.byref(s), fake, odd, fake, 1 << 40, None) == -1
    assert lib.lsh_chunk_attend(fake, odd, fake, fake, ctypes.byref(s), fake, fake, None) == -1
    assert lib.lsh_unsort_combine(fake, fake, fake, ctypes.byref(s), odd, None) == -1
    assert lib.lsh_attention_fwd(fake, fake, fake, ctypes.byref(s), fake, odd, 1 << 40, None) == -1
    assert b"aligned" in lib.lsh_last_error()


def test_empty_problems_enqueue_nothing(lib):
    for kw in (dict(L=0), dict(B=0), dict(H=0)):
        s = _shape(**kw)
        assert lib.lsh_attention_fwd(None, None, None, ctypes.byref(s), None, None, 0, None) == 0
        assert lib.lsh_hash(None, None, ctypes.byref(s), None, None, 0, None) == 0


@pytest.mark.parametrize("d_model", [0, -8, 12, 100])
def test_projection_rejects_bad_d_model(lib, d_model):
    # host-side check, before any pointer is looked at or anything is enqueued
    s = ctypes.byref(_shape())
    assert lib.lsh_qkv_project(None, None, None, s, d_model, None, None, None) == -1
    assert "d_model" in lsh.lsh_last_error()
    assert lib.lsh_attention_fwd_x(None, None, None, None, s, d_model, None, None, 0, None) == -1
    assert "d_model" in lsh.lsh_last_error()


def test_projection_rejects_null_and_misaligned_pointers(lib):
    assert lib.lsh_qkv_project(None, None, None, ctypes.byref(_shape()), 64, None, None,
                               None) == -1
    assert "NULL" in lsh.lsh_last_error()
    p = ctypes.c_void_p(0x1008)
    rc = lib.lsh_qkv_project(p, p, p, ctypes.byref(_shape()), 64, p, p, None)
    assert rc == -1 and "aligned" in lsh.lsh_last_error()


def test_fwd_x_workspace_holds_the_projected_tensors(lib):
    for dtype, e in ((lsh.LSH_BF16, 2), (lsh.LSH_F32, 4)):
        s = _shape(dtype=dtype)
        fwd = lsh.lsh_workspace_size("fwd", s)
        fx = lsh.lsh_workspace_size("fwd_x", s)
        assert fx >= fwd + 2 * s.B * s.H * s.L * s.d * e


def test_training_state_and_backward_workspace_sizes(lib):
    s = _shape()
    n = s.B * s.H * s.n_hashes * s.L
    assert lsh.lsh_workspace_size("state", s) >= 8 * n + 4 * s.B * s.H * s.L
    assert lsh.lsh_workspace_size("bwd", s) >= 2 * 4 * n * s.d + 4 * s.B * s.H * s.L


def test_backward_rejects_small_state(lib):
    s = ctypes.byref(_shape())
    p = ctypes.c_void_p(0x1000)
    rc = lib.lsh_attention_bwd(p, p, p, p, p, 16, s, p, p, p, 1 << 40, None)
    assert rc == -2 and "state" in lsh.lsh_last_error()


def test_key_norm_workspace_holds_one_float_per_token(lib):
    """LSH_KEY_NORM adds 1 / |qk| per token (256-byte aligned) to the forward
    and backward workspaces; the other stages and the training state keep
    their size."""
    base, kn = _shape(), _shape(flags=lsh.LSH_KEY_NORM)
    tokens = base.B * base.H * base.L
    extra = -(-4 * tokens // 256) * 256
    for stage in ("hash", "sort", "state"):
        assert lsh.lsh_workspace_size(stage, kn) == lsh.lsh_workspace_size(stage, base)
    for stage in ("fwd", "fwd_x", "bwd"):
        assert lsh.lsh_workspace_size(stage, kn) == lsh.lsh_workspace_size(stage, base) + extra


def test_per_head_rotations_workspace(lib):
    """LSH_PER_HEAD_R keeps R-derived tables per (head, round): the hash
    workspace grows with H, and with one head it is the shared-R size."""
    one = _shape(H=1)
    assert lsh.lsh_workspace_size("hash", _shape(H=1, flags=lsh.LSH_PER_HEAD_R)) == \
        lsh.lsh_workspace_size("hash", one)
    assert lsh.lsh_workspace_size("hash", _shape(H=4, flags=lsh.LSH_PER_HEAD_R)) > \
        lsh.lsh_workspace_size("hash", _shape(H=4))
    both = lsh.LSH_PER_HEAD_R | lsh.LSH_KEY_NORM
    assert lsh.lsh_workspace_size("fwd", _shape(flags=both)) >= \
        lsh.lsh_workspace_size("fwd", _shape(flags=lsh.LSH_KEY_NORM))
    # the per-head queue rounds each (batch, head) up: L = 300 pads to 512 tokens
    assert lsh.lsh_workspace_size("hash", _shape(L=300, chunk_len=300, flags=lsh.LSH_PER_HEAD_R)) > \
        lsh.lsh_workspace_size("hash", _shape(L=300, chunk_len=300))


def test_rounds_of_reads_the_rotation_layout():
    import torch
    assert lsh.rounds_of(torch.empty(3, 64, 8)) == (3, False)
    assert lsh.rounds_of(torch.empty(2, 3, 64, 8)) == (3, True)
    with pytest.raises(ValueError):
        lsh.rounds_of(torch.empty(64, 8))


def test_ffn_workspace_is_one_chunk_of_the_intermediate(lib):
    assert lsh.lsh_ffn_workspace_size(65536, 4096, 8192, lsh.LSH_BF16) == 8192 * 4096 * 2
    assert lsh.lsh_ffn_workspace_size(100, 4096, 8192, lsh.LSH_F32) == 100 * 4096 * 4
    assert lsh.lsh_ffn_workspace_size(0, 64, 16, lsh.LSH_BF16) == 0
    for args in ((10, 12, 4, lsh.LSH_BF16), (10, 64, 0, lsh.LSH_BF16), (-1, 64, 4, lsh.LSH_F32),
                 (10, 64, 4, 9)):
        with pytest.raises(lsh.LshError) as ei:
            lsh.lsh_ffn_workspace_size(*args)
        assert ei.value.code == -1


def test_ffn_rejects_on_host(lib):
    import ctypes
    call = lib.lsh_ffn_chunked
    fake = ctypes.c_void_p(1 << 20)   # never dereferenced: every case fails on the host
    # d_model not a multiple of 8
    assert call(fake, fake, None, fake, None, 4, 12, 64, 4, lsh.LSH_BF16, fake, fake, 1 << 20,
                None) == -1
    # NULL x
    assert call(None, fake, None, fake, None, 4, 16, 64, 4, lsh.LSH_BF16, fake, fake, 1 << 20,
                None) == -1
    # misaligned weight
    assert call(fake, ctypes.c_void_p((1 << 20) + 2), None, fake, None, 4, 16, 64, 4,
                lsh.LSH_BF16, fake, fake, 1 << 20, None) == -1
    # workspace too small (needs 4 * 64 * 2 bytes), and missing
    assert call(fake, fake, None, fake, None, 4, 16, 64, 4, lsh.LSH_BF16, fake, fake, 511,
                None) == -2
    assert call(fake, fake, None, fake, None, 4, 16, 64, 4, lsh.LSH_BF16, fake, None, 1 << 20,
                None) == -2
    # no rows: nothing to do, no pointer is needed
    assert call(None, None, None, None, None, 0, 16, 64, 4, lsh.LSH_BF16, None, None, 0,
                None) == 0


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus 2 exits with status 2 and a JSON
    error line before touching a device."""
    import json
    import pathlib
    import subprocess
    import sys
    root = pathlib.Path(__file__).resolve().parent.parent
    res = subprocess.run([sys.executable, str(root / "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120, cwd=root)
    assert res.returncode == 2
    assert "error" in json.loads(res.stdout.strip().splitlines()[-1])


def _cpu_qk(B=1, H=2, L=256, d=64, dtype=None):
    import torch
    return torch.zeros(B, H, L, d, dtype=dtype or torch.bfloat16)


@pytest.mark.parametrize("rshape, rdtype, msg", [
    ((2, 64, 8), "bfloat16", "float32"),      # bf16 R (natural next to bf16 qk)
    ((2, 64, 4), "float32", "n_buckets/2"),   # R for 8 buckets, called with 16
    ((2, 32, 8), "float32", "n_buckets/2"),   # wrong head size
    ((3, 2, 64, 8), "float32", "n_buckets/2"),  # per-head R for 3 heads, qk has 2
    ((0, 64, 8), "float32", "n_buckets/2"),   # no rounds
])
def test_helpers_validate_R_before_any_launch(rshape, rdtype, msg):
    """R is read by kernels sized from qk and n_buckets: a mismatched or
    mistyped R is refused on the host (CPU tensors here, so nothing could be
    launched even if the check were missing: the device check comes later)."""
    import torch
    qk = _cpu_qk()
    R = torch.zeros(rshape, dtype=getattr(torch, rdtype))
    for call in (lambda: lsh.hash(qk, R, 16),
                 lambda: lsh.attention_fwd(qk, qk, R, 16, 64, True),
                 lambda: lsh.attention_fwd_train(qk, qk, R, 16, 64, True)):
        with pytest.raises(ValueError, match=msg):
            call()


def test_helpers_validate_out_and_v():
    import torch
    qk = _cpu_qk()
    R = torch.zeros(2, 64, 8)
    with pytest.raises(ValueError, match="out"):
        lsh.attention_fwd(qk, qk, R, 16, 64, True, out=torch.zeros(1, 2, 256, 64))
    with pytest.raises(ValueError, match="out"):
        lsh.attention_fwd(qk, qk, R, 16, 64, True, out=_cpu_qk(L=128))
    with pytest.raises(ValueError, match="v"):
        lsh.attention_fwd(qk, _cpu_qk(d=128), R, 16, 64, True)


def test_c_named_wrappers_check_buffer_sizes_and_dtypes():
    """The C-named Python calls check every tensor against the shape before the
    call (a short or mistyped buffer would be read past its end on the GPU)."""
    import torch
    s = _shape()
    qk = _cpu_qk()
    R = torch.zeros(2, 64, 8)
    n = s.B * s.H * s.n_hashes * s.L
    with pytest.raises(ValueError, match="buckets"):
        lsh.lsh_hash(qk, R, s, torch.zeros(n - 1, dtype=torch.int32), None)
    with pytest.raises(ValueError, match="R"):
        lsh.lsh_hash(qk, torch.zeros(2, 64, 8, dtype=torch.bfloat16), s,
                     torch.zeros(n, dtype=torch.int32), None)
    with pytest.raises(ValueError, match="qk"):
        lsh.lsh_attention_fwd(qk.float(), qk, R, s, qk, None)
    with pytest.raises(ValueError, match="inv"):
        lsh.lsh_sort(torch.zeros(n, dtype=torch.int32), s, torch.zeros(n, dtype=torch.int32),
                     torch.zeros(n, dtype=torch.int64), None)
    with pytest.raises(ValueError, match="o_sorted"):
        lsh.lsh_chunk_attend(qk, qk, torch.zeros(n, dtype=torch.int32),
                             torch.zeros(n, dtype=torch.int32), s,
                             torch.zeros(n, dtype=torch.float32), torch.zeros(n), None)
    with pytest.raises(ValueError, match="dv"):
        lsh.lsh_attention_bwd(qk, qk, qk, qk, None, s, qk, None, None)


def test_sort_noalloc_refuses_on_host(lib):
    """lsh_sort_noalloc checks the shape, the pointers and its 16 MiB static
    scratch's limit on the host, before any HIP call."""
    fake = ctypes.c_void_p(0x1000)
    big = _shape(B=1, H=1, n_hashes=8, L=1 << 20, chunk_len=64, n_buckets=4096)
    assert lib.lsh_sort_noalloc(fake, ctypes.byref(big), fake, fake, None) == -2
    assert "static scratch" in lsh.lsh_last_error()
    s = _shape()
    assert lib.lsh_sort_noalloc(None, ctypes.byref(s), fake, fake, None) == -1
    assert lib.lsh_sort_noalloc(fake, ctypes.byref(s), ctypes.c_void_p(0x1008), fake, None) == -1
    assert lib.lsh_sort_noalloc(fake, ctypes.byref(_shape(d=96)), fake, fake, None) == -1
    assert lib.lsh_sort_noalloc(None, ctypes.byref(_shape(L=0)), None, None, None) == 0


def test_debug_fail_launch_rejects_negative(lib):
    assert lib.lsh_debug_fail_launch(-1) == -1 and "n must be" in lsh.lsh_last_error()
    assert lib.lsh_debug_fail_launch(0) == 0
