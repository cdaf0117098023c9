"""Python access to the double-precision C oracle in ``lsh_oracle.c``.

TEST INFRASTRUCTURE. Only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark import this module. The GPU library never
does, and this module imports nothing from it.

Each function widens its inputs to float64 (bf16 and fp32 values widen
exactly), calls the matching C routine and returns NumPy arrays. The steps and
their sources are documented in ``lsh_oracle.c``:

  hash     -- O1, angular LSH: first argmax of [xR, -xR] per round
  sort     -- O2, positions ordered by (bucket, position)
  attend   -- O3/O4, chunk windows (own chunk + previous one), same-bucket,
              causal and self rules, softmax in double
  combine  -- O5, un-sort and logsumexp-weighted sum over rounds
  forward  -- O1..O5 over every (batch, head)
  project  -- P0, the shared query/key and the value projections of the
              token vectors, split into heads
  backward -- G1, gradients of the forward for a given output gradient
  ffn      -- F1, the chunked feed-forward relu(x W1^T + b1) W2^T + b2
  attend_qk, forward_qk -- Q1, the ablation with separate queries and keys
"""
from __future__ import annotations

import ctypes
import os
import pathlib
import subprocess

import numpy as np

_DIR = pathlib.Path(__file__).resolve().parent
_SRC = _DIR / "lsh_oracle.c"
_LIB_PATH = _DIR / "liblsh_oracle.so"
_lib = None

_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> pathlib.Path:
    """Compile the oracle with gcc (plain -O2, no FMA contraction, OpenMP)."""
    if force or not _LIB_PATH.exists():
        tmp = _LIB_PATH.with_suffix(".so.tmp")
        cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
               "-fopenmp", "-shared", "-fPIC", str(_SRC), "-o", str(tmp), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists():
            build(force=False)
        lib = ctypes.CDLL(str(_LIB_PATH))
        lib.oracle_hash.argtypes = [_f64p, ctypes.c_int64, ctypes.c_int, _f64p, ctypes.c_int,
                                    ctypes.c_int, _i32p, _f64p]
        lib.oracle_sort.argtypes = [_i32p, ctypes.c_int64, _i32p, _i32p]
        lib.oracle_attend.argtypes = [_f64p, _f64p, ctypes.c_int64, ctypes.c_int, _i32p, _i32p,
                                      ctypes.c_int, ctypes.c_int, _i64p, ctypes.c_int64, _f64p,
                                      _f64p, ctypes.c_int]
        lib.oracle_combine.argtypes = [_f64p, _f64p, _i32p, ctypes.c_int, ctypes.c_int64,
                                       ctypes.c_int, _i64p, ctypes.c_int64, _f64p]
        lib.oracle_forward.argtypes = [_f64p, _f64p, _f64p, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, _f64p, _i32p, _f64p, _i32p,
                                       _i32p, _f64p, _f64p, ctypes.c_int, ctypes.c_int]
        lib.oracle_project.argtypes = [_f64p, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                       _f64p, _f64p, ctypes.c_int, ctypes.c_int, _f64p, _f64p]
        lib.oracle_backward.argtypes = [_f64p, _f64p, _f64p, _f64p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, _f64p, _f64p, ctypes.c_int,
                                        ctypes.c_int]
        lib.oracle_backward_rows.argtypes = [_f64p, _f64p, _f64p, _f64p, ctypes.c_int64,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int, _i64p,
                                             ctypes.c_int64, _f64p, _f64p]
        lib.oracle_ffn.argtypes = [_f64p, ctypes.c_int64, ctypes.c_int, _f64p, _f64p, _f64p,
                                   _f64p, ctypes.c_int, ctypes.c_int64, _f64p]
        lib.oracle_attend_qk.argtypes = [_f64p, _f64p, _f64p, ctypes.c_int64, ctypes.c_int,
                                         _i32p, _i32p, _i32p, _i32p, ctypes.c_int, ctypes.c_int,
                                         _i64p, ctypes.c_int64, _f64p, _f64p]
        lib.oracle_forward_qk.argtypes = [_f64p, _f64p, _f64p, _f64p, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int, _f64p,
                                          _i32p, _i32p, _f64p, _f64p, _i32p, _i32p, _i32p,
                                          _f64p, _f64p, ctypes.c_int]
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = ctypes.c_int
        for fn in (lib.oracle_hash, lib.oracle_sort, lib.oracle_attend, lib.oracle_combine,
                   lib.oracle_forward, lib.oracle_project, lib.oracle_backward,
                   lib.oracle_backward_rows, lib.oracle_ffn, lib.oracle_attend_qk,
                   lib.oracle_forward_qk):
            fn.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    """Threads the oracle's OpenMP loops run on."""
    return int(_load().oracle_threads())


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p(a, t):
    return None if a is None else a.ctypes.data_as(t)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def hash(x, R, n_buckets: int):
    """O1. x: [n, d]; R: [n_hashes, d, n_buckets/2].

    Returns (buckets [n_hashes, n] int32, margin [n_hashes, n] float64).
    """
    x = _f64(x)
    R = _f64(R)
    n, d = x.shape
    nh = R.shape[0]
    if R.shape != (nh, d, n_buckets // 2):
        raise ValueError(f"R has shape {R.shape}, expected {(nh, d, n_buckets // 2)}")
    buckets = np.empty((nh, n), np.int32)
    margin = np.empty((nh, n), np.float64)
    _check(_load().oracle_hash(_p(x, _f64p), n, d, _p(R, _f64p), nh, n_buckets,
                               _p(buckets, _i32p), _p(margin, _f64p)), "hash")
    return buckets, margin


def sort(bucket):
    """O2. bucket: [L] for one round. Returns (perm [L], inv [L]) int32."""
    bucket = _i32(bucket)
    L = bucket.shape[0]
    perm = np.empty(L, np.int32)
    inv = np.empty(L, np.int32)
    _check(_load().oracle_sort(_p(bucket, _i32p), L, _p(perm, _i32p), _p(inv, _i32p)), "sort")
    return perm, inv


def attend(x, v, bucket, perm, chunk_len: int, causal: bool, slots=None, key_norm=False):
    """O3/O4 for one round. x, v: [L, d]; bucket, perm: [L].

    Returns (o [L, d], lse [L]) indexed by sorted slot. With ``slots`` only
    those query slots are computed; the other rows are NaN. ``key_norm``:
    the key side of each score uses x_j / |x_j|.
    """
    x = _f64(x)
    v = _f64(v)
    bucket = _i32(bucket)
    perm = _i32(perm)
    L, d = x.shape
    o = np.full((L, d), np.nan)
    lse = np.full(L, np.nan)
    sl = None if slots is None else np.ascontiguousarray(np.asarray(slots, dtype=np.int64))
    _check(_load().oracle_attend(_p(x, _f64p), _p(v, _f64p), L, d, _p(bucket, _i32p),
                                 _p(perm, _i32p), chunk_len, int(bool(causal)), _p(sl, _i64p),
                                 0 if sl is None else sl.shape[0], _p(o, _f64p), _p(lse, _f64p),
                                 int(bool(key_norm))),
           "attend")
    return o, lse


def combine(o, lse, inv, tokens=None):
    """O5 for one (batch, head). o: [nh, L, d]; lse, inv: [nh, L].

    Returns out [L, d] by original position (NaN rows outside ``tokens``).
    """
    o = _f64(o)
    lse = _f64(lse)
    inv = _i32(inv)
    nh, L, d = o.shape
    out = np.full((L, d), np.nan)
    tk = None if tokens is None else np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    _check(_load().oracle_combine(_p(o, _f64p), _p(lse, _f64p), _p(inv, _i32p), nh, L, d,
                                  _p(tk, _i64p), 0 if tk is None else tk.shape[0],
                                  _p(out, _f64p)), "combine")
    return out


def _rotations(R, H: int, d: int, n_buckets: int):
    """R as float64 and (n_hashes, per_head): [nh, d, nb/2] is shared by every
    head, [H, nh, d, nb/2] gives each head its own rotations."""
    R = _f64(R)
    if R.ndim == 4:
        if R.shape[0] != H or R.shape[2:] != (d, n_buckets // 2):
            raise ValueError(f"per-head R has shape {R.shape}, expected (H={H}, nh, {d}, "
                             f"{n_buckets // 2})")
        return R, R.shape[1], 1
    if R.ndim != 3 or R.shape[1:] != (d, n_buckets // 2):
        raise ValueError(f"R has shape {R.shape}, expected (nh, {d}, {n_buckets // 2})")
    return R, R.shape[0], 0


def forward(qk, v, R, n_buckets: int, chunk_len: int, causal: bool, return_all: bool = False,
            key_norm: bool = False):
    """O1..O5 over every (batch, head). qk, v: [B, H, L, d]; R: [nh, d, nb/2]
    shared by every head, or [H, nh, d, nb/2] (each head its own rotations);
    ``key_norm``: the key side of each score uses x_j / |x_j|.

    Returns out [B, H, L, d]; with ``return_all`` also a dict of the
    intermediate results (buckets, margin, perm, inv, lse, o_sorted).
    """
    qk = _f64(qk)
    v = _f64(v)
    B, H, L, d = qk.shape
    R, nh, per_head = _rotations(R, H, d, n_buckets)
    out = np.empty((B, H, L, d))
    extra = {}
    if return_all:
        extra = dict(buckets=np.empty((B, H, nh, L), np.int32),
                     margin=np.empty((B, H, nh, L)),
                     perm=np.empty((B, H, nh, L), np.int32),
                     inv=np.empty((B, H, nh, L), np.int32),
                     o_sorted=np.empty((B, H, nh, L, d)),
                     lse=np.empty((B, H, nh, L)))
    g = extra.get
    _check(_load().oracle_forward(_p(qk, _f64p), _p(v, _f64p), _p(R, _f64p), B, H, L, d,
                                  n_buckets, nh, chunk_len, int(bool(causal)), _p(out, _f64p),
                                  _p(g("buckets"), _i32p), _p(g("margin"), _f64p),
                                  _p(g("perm"), _i32p), _p(g("inv"), _i32p),
                                  _p(g("o_sorted"), _f64p), _p(g("lse"), _f64p),
                                  int(bool(key_norm)), per_head), "forward")
    return (out, extra) if return_all else out


def project(x, w_qk, w_v, n_heads: int):
    """P0: qk, v [B, H, L, d] from token vectors x [B, L, d_model] and weights
    w_qk, w_v [H * d, d_model] (output n of input k at w[n, k]); head h takes
    outputs h*d .. h*d + d - 1."""
    x = _f64(x)
    w_qk = _f64(w_qk)
    w_v = _f64(w_v)
    B, L, dm = x.shape
    n_out = w_qk.shape[0]
    if w_qk.shape != (n_out, dm) or w_v.shape != (n_out, dm) or n_out % n_heads:
        raise ValueError("weights must be [H * d, d_model] with d_model matching x")
    d = n_out // n_heads
    qk = np.zeros((B, n_heads, L, d))
    v = np.zeros((B, n_heads, L, d))
    _check(_load().oracle_project(_p(x, _f64p), B, L, dm, _p(w_qk, _f64p), _p(w_v, _f64p),
                                  n_heads, d, _p(qk, _f64p), _p(v, _f64p)), "project")
    return qk, v


def backward(qk, v, R, dout, n_buckets: int, chunk_len: int, causal: bool,
             key_norm: bool = False):
    """G1: (dqk, dv), both [B, H, L, d], for a loss whose gradient with
    respect to the forward's output is dout [B, H, L, d]; R as in forward."""
    qk = _f64(qk)
    v = _f64(v)
    dout = _f64(dout)
    B, H, L, d = qk.shape
    R, nh, per_head = _rotations(R, H, d, n_buckets)
    dqk = np.zeros((B, H, L, d))
    dv = np.zeros((B, H, L, d))
    _check(_load().oracle_backward(_p(qk, _f64p), _p(v, _f64p), _p(R, _f64p), _p(dout, _f64p),
                                   B, H, L, d, n_buckets, nh, chunk_len, int(bool(causal)),
                                   _p(dqk, _f64p), _p(dv, _f64p), int(bool(key_norm)), per_head),
           "backward")
    return dqk, dv


def backward_rows(x, v, R, dout, tokens, n_buckets: int, chunk_len: int, causal: bool,
                  key_norm: bool = False):
    """G1 at chosen positions of one (batch, head): rows (dqk[p], dv[p]) for
    each p in ``tokens`` (distinct), each as ``backward`` computes it, with
    the forward run only where those rows need it. x, v, dout: [L, d];
    R: this head's rotations [nh, d, nb/2]. Returns two [len(tokens), d]."""
    x = _f64(x)
    v = _f64(v)
    dout = _f64(dout)
    R = _f64(R)
    L, d = x.shape
    nh = R.shape[0]
    if R.shape != (nh, d, n_buckets // 2) or v.shape != x.shape or dout.shape != x.shape:
        raise ValueError("x, v, dout must be [L, d] and R [nh, d, n_buckets/2]")
    tk = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    dqk = np.empty((tk.shape[0], d))
    dv = np.empty((tk.shape[0], d))
    _check(_load().oracle_backward_rows(_p(x, _f64p), _p(v, _f64p), _p(R, _f64p),
                                        _p(dout, _f64p), L, d, n_buckets, nh, chunk_len,
                                        int(bool(causal)), int(bool(key_norm)), _p(tk, _i64p),
                                        tk.shape[0], _p(dqk, _f64p), _p(dv, _f64p)),
           "backward_rows")
    return dqk, dv


def ffn(x, w1, b1, w2, b2, chunk: int):
    """F1: out [rows, d_model] = relu(x W1^T + b1) W2^T + b2, ``chunk`` rows at
    a time. x [rows, d_model]; w1 [d_ff, d_model]; w2 [d_model, d_ff]; b1, b2
    vectors or None (zero)."""
    x = _f64(x)
    w1 = _f64(w1)
    w2 = _f64(w2)
    rows, dm = x.shape
    dff = w1.shape[0]
    if w1.shape != (dff, dm) or w2.shape != (dm, dff):
        raise ValueError("w1 must be [d_ff, d_model] and w2 [d_model, d_ff]")
    b1 = None if b1 is None else _f64(b1).reshape(dff)
    b2 = None if b2 is None else _f64(b2).reshape(dm)
    out = np.empty((rows, dm))
    _check(_load().oracle_ffn(_p(x, _f64p), rows, dm, _p(w1, _f64p), _p(b1, _f64p),
                              _p(w2, _f64p), _p(b2, _f64p), dff, chunk, _p(out, _f64p)), "ffn")
    return out


def attend_qk(q, k, v, bucket_q, bucket_k, perm_q, perm_k, chunk_len: int, causal: bool,
              slots=None):
    """Q1 for one round with separate queries and keys. q, k, v: [L, d];
    bucket_q/_k, perm_q/_k: [L]. Returns (o [L, d], lse [L]) by query slot; a
    query whose window holds no key of its bucket gets lse -inf and a zero row."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    L, d = q.shape
    o = np.full((L, d), np.nan)
    lse = np.full(L, np.nan)
    sl = None if slots is None else np.ascontiguousarray(np.asarray(slots, dtype=np.int64))
    _check(_load().oracle_attend_qk(_p(q, _f64p), _p(k, _f64p), _p(v, _f64p), L, d,
                                    _p(_i32(bucket_q), _i32p), _p(_i32(bucket_k), _i32p),
                                    _p(_i32(perm_q), _i32p), _p(_i32(perm_k), _i32p),
                                    chunk_len, int(bool(causal)), _p(sl, _i64p),
                                    0 if sl is None else sl.shape[0], _p(o, _f64p),
                                    _p(lse, _f64p)), "attend_qk")
    return o, lse


def forward_qk(q, k, v, R, n_buckets: int, chunk_len: int, causal: bool,
               return_all: bool = False):
    """Q1 over every (batch, head): queries and keys hashed with the same R,
    sorted separately, chunked attention, combine. q, k, v: [B, H, L, d];
    R as in forward. Returns out [B, H, L, d]; with ``return_all`` also a dict
    (buckets_q, buckets_k, margin_q, margin_k, perm_q, perm_k, inv_q,
    o_sorted and lse by query slot)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, d = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must have the same shape")
    R, nh, per_head = _rotations(R, H, d, n_buckets)
    out = np.empty((B, H, L, d))
    extra = {}
    if return_all:
        i32 = lambda: np.empty((B, H, nh, L), np.int32)
        f64 = lambda: np.empty((B, H, nh, L))
        extra = dict(buckets_q=i32(), buckets_k=i32(), margin_q=f64(), margin_k=f64(),
                     perm_q=i32(), perm_k=i32(), inv_q=i32(), lse=f64(),
                     o_sorted=np.empty((B, H, nh, L, d)))
    g = extra.get
    _check(_load().oracle_forward_qk(_p(q, _f64p), _p(k, _f64p), _p(v, _f64p), _p(R, _f64p),
                                     B, H, L, d, n_buckets, nh, chunk_len, int(bool(causal)),
                                     _p(out, _f64p), _p(g("buckets_q"), _i32p),
                                     _p(g("buckets_k"), _i32p), _p(g("margin_q"), _f64p),
                                     _p(g("margin_k"), _f64p), _p(g("perm_q"), _i32p),
                                     _p(g("perm_k"), _i32p), _p(g("inv_q"), _i32p),
                                     _p(g("o_sorted"), _f64p), _p(g("lse"), _f64p), per_head),
           "forward_qk")
    return (out, extra) if return_all else out
