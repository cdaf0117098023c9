"""ctypes binding of ``liblsh_attn.so`` (argument marshalling only)."""
from __future__ import annotations

import ctypes
import pathlib

import torch

LSH_F32 = 0
LSH_BF16 = 1
LSH_KEY_NORM = 1   # lsh_shape_t.flags bit: keys as unit vectors in the scores
LSH_PER_HEAD_R = 2  # lsh_shape_t.flags bit: R is [H, n_hashes, d, n_buckets/2]
_DTYPES = {torch.float32: LSH_F32, torch.bfloat16: LSH_BF16}
_ERRORS = {-1: "LSH_ERR_ARG", -2: "LSH_ERR_WORKSPACE", -3: "LSH_ERR_HIP"}

_PKG = pathlib.Path(__file__).resolve().parent
_LIB_PATH = _PKG / "liblsh_attn.so"
_lib = None


class LshError(RuntimeError):
    def __init__(self, code: int, fn: str, msg: str):
        super().__init__(f"{fn}: {_ERRORS.get(code, code)}: {msg}")
        self.code = code


class Shape(ctypes.Structure):
    """Mirror of ``lsh_shape_t``."""
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32),
                ("d", ctypes.c_int32), ("n_buckets", ctypes.c_int32),
                ("n_hashes", ctypes.c_int32), ("chunk_len", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32)]

    def __repr__(self):
        return "Shape(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


def library_path() -> pathlib.Path:
    return _LIB_PATH


def load_library():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists():
        raise RuntimeError(f"{_LIB_PATH} is missing: build it first "
                           "(python -m lsh_attention_fp32_amd.build or __graft_entry__.build())")
    lib = ctypes.CDLL(str(_LIB_PATH))
    vp, sz, i32, sp = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.POINTER(Shape)
    lib.lsh_workspace_size.argtypes = [ctypes.c_char_p, sp]
    lib.lsh_workspace_size.restype = sz
    lib.lsh_hash.argtypes = [vp, vp, sp, vp, vp, sz, vp]
    lib.lsh_sort.argtypes = [vp, sp, vp, vp, vp, sz, vp]
    lib.lsh_sort_noalloc.argtypes = [vp, sp, vp, vp, vp]
    lib.lsh_chunk_attend.argtypes = [vp, vp, vp, vp, sp, vp, vp, vp]
    lib.lsh_chunk_attend_qk.argtypes = [vp, vp, vp, vp, vp, vp, vp, sp, vp, vp, vp]
    lib.lsh_attention_fwd_qk.argtypes = [vp, vp, vp, vp, sp, vp, vp, sz, vp]
    lib.lsh_unsort_combine.argtypes = [vp, vp, vp, sp, vp, vp]
    lib.lsh_attention_fwd.argtypes = [vp, vp, vp, sp, vp, vp, sz, vp]
    lib.lsh_attention_fwd_timed.argtypes = [vp, vp, vp, sp, vp, vp, sz, vp,
                                            ctypes.POINTER(ctypes.c_float),
                                            ctypes.POINTER(ctypes.c_char_p), i32,
                                            ctypes.POINTER(i32)]
    lib.lsh_qkv_project.argtypes = [vp, vp, vp, sp, i32, vp, vp, vp]
    lib.lsh_attention_fwd_x.argtypes = [vp, vp, vp, vp, sp, i32, vp, vp, sz, vp]
    lib.lsh_attention_fwd_train.argtypes = [vp, vp, vp, sp, vp, vp, sz, vp, sz, vp]
    lib.lsh_attention_bwd.argtypes = [vp, vp, vp, vp, vp, sz, sp, vp, vp, vp, sz, vp]
    i64 = ctypes.c_int64
    lib.lsh_ffn_workspace_size.argtypes = [i64, i32, i32, i32]
    lib.lsh_ffn_workspace_size.restype = sz
    lib.lsh_ffn_chunked.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, vp, vp, sz, vp]
    for name in ("lsh_ffn_chunked", "lsh_hash", "lsh_sort", "lsh_sort_noalloc", "lsh_chunk_attend",
                 "lsh_chunk_attend_qk", "lsh_attention_fwd_qk",
                 "lsh_unsort_combine", "lsh_attention_fwd", "lsh_attention_fwd_timed",
                 "lsh_qkv_project", "lsh_attention_fwd_x", "lsh_attention_fwd_train",
                 "lsh_attention_bwd"):
        getattr(lib, name).restype = ctypes.c_int
    lib.lsh_debug_fail_launch.argtypes = [i32]
    lib.lsh_debug_fail_launch.restype = ctypes.c_int
    lib.lsh_last_error.argtypes = []
    lib.lsh_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def lsh_last_error() -> str:
    return load_library().lsh_last_error().decode()


def _check(rc: int, fn: str) -> None:
    if rc != 0:
        raise LshError(rc, fn, lsh_last_error())


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if t.numel() and not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else None


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def shape_of(qk: torch.Tensor, n_buckets: int, n_hashes: int, chunk_len: int,
             causal: bool, key_norm: bool = False, per_head_r: bool = False) -> Shape:
    """Shape for qk of shape [B, H, L, d] (float32 or bfloat16)."""
    if qk.dim() != 4:
        raise ValueError(f"qk must be [B, H, L, d], got {tuple(qk.shape)}")
    if qk.dtype not in _DTYPES:
        raise ValueError(f"qk dtype must be float32 or bfloat16, got {qk.dtype}")
    B, H, L, d = qk.shape
    return Shape(B, H, L, d, n_buckets, n_hashes, chunk_len, int(bool(causal)), _DTYPES[qk.dtype],
                 (LSH_KEY_NORM if key_norm else 0) | (LSH_PER_HEAD_R if per_head_r else 0))


def rounds_of(R) -> tuple[int, bool]:
    """(n_hashes, per-head): R [n_hashes, d, nb/2] is shared by every head,
    R [H, n_hashes, d, nb/2] gives each head its own rotations."""
    if R.dim() == 4:
        return R.shape[1], True
    if R.dim() != 3:
        raise ValueError(f"R must be [n_hashes, d, nb/2] or [H, n_hashes, d, nb/2], "
                         f"got {tuple(R.shape)}")
    return R.shape[0], False


def check_rotations(R, qk, n_buckets: int) -> tuple[int, bool]:
    """Validates R against qk [B, H, L, d] and n_buckets: a contiguous float32
    tensor on qk's device, [n_hashes, d, nb/2] or [H, n_hashes, d, nb/2].
    Returns (n_hashes, per-head)."""
    if not isinstance(R, torch.Tensor):
        raise TypeError("R must be a torch tensor")
    nh, per_head = rounds_of(R)
    B, H, L, d = qk.shape
    want = ((H,) if per_head else ()) + (nh, d, n_buckets // 2)
    if tuple(R.shape) != want or nh < 1:
        raise ValueError(f"R must be [{'H, ' if per_head else ''}n_hashes, d, n_buckets/2] = "
                         f"{want} for qk {tuple(qk.shape)} and n_buckets {n_buckets}, "
                         f"got {tuple(R.shape)}")
    if R.dtype != torch.float32:
        raise ValueError(f"R must be float32, got {R.dtype}")
    if R.device != qk.device or not R.is_contiguous():
        raise ValueError("R must be contiguous and on qk's device")
    return nh, per_head


def check_like(t, ref, what: str) -> None:
    """``t`` must match ``ref`` in shape, dtype and device, and be contiguous."""
    if (not isinstance(t, torch.Tensor) or t.shape != ref.shape or t.dtype != ref.dtype
            or t.device != ref.device or not t.is_contiguous()):
        raise ValueError(f"{what} must be a contiguous {ref.dtype} tensor of shape "
                         f"{tuple(ref.shape)} on {ref.device}")


# ---------------------------------------------------------------- C-named calls

def _size_query(n: int, fn: str) -> int:
    """A size_t result of the C ABI: 0 with a message means an error (always
    LSH_ERR_ARG for the size queries)."""
    msg = lsh_last_error()
    if msg:
        raise LshError(-1, fn, msg)
    return int(n)


def lsh_workspace_size(stage: str, shape: Shape) -> int:
    return _size_query(load_library().lsh_workspace_size(stage.encode(), ctypes.byref(shape)),
                       "lsh_workspace_size")


_TORCH_DTYPE = {LSH_F32: torch.float32, LSH_BF16: torch.bfloat16}


def _need(fn: str, what: str, t, dtype, numel: int, optional: bool = False) -> None:
    """Host check before a call: ``t`` holds at least ``numel`` elements of
    ``dtype`` (the library takes plain pointers, so it cannot see a short or
    mistyped buffer; this keeps every kernel inside its buffers)."""
    if t is None:
        if optional or numel == 0:
            return
        raise ValueError(f"{fn}: {what} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{fn}: {what} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{fn}: {what} must be {dtype}, got {t.dtype}")
    if t.numel() < numel:
        raise ValueError(f"{fn}: {what} holds {t.numel()} elements, needs {numel}")


def _io(shape: Shape):
    return _TORCH_DTYPE.get(shape.dtype, torch.float32)


def _sizes(shape: Shape):
    """(token rows B*H*L*d, per-slot entries B*H*nh*L, R elements) of a shape."""
    rows = shape.B * shape.H * shape.L * shape.d
    slots = shape.B * shape.H * shape.n_hashes * shape.L
    heads = shape.H if shape.flags & LSH_PER_HEAD_R else 1
    r = heads * shape.n_hashes * shape.d * (shape.n_buckets // 2)
    return rows, slots, r


def _need_qkvr(fn: str, shape: Shape, qk=None, v=None, R=None, out=None, with_r=True,
               with_v=True, with_out=True) -> None:
    rows, _, r = _sizes(shape)
    io = _io(shape)
    _need(fn, "qk", qk, io, rows)
    if with_v:
        _need(fn, "v", v, io, rows)
    if with_r:
        _need(fn, "R", R, torch.float32, r)
    if with_out:
        _need(fn, "out", out, io, rows)


def lsh_hash(qk, R, shape: Shape, buckets, ws, stream=None) -> None:
    _need_qkvr("lsh_hash", shape, qk, R=R, with_v=False, with_out=False)
    _need("lsh_hash", "buckets", buckets, torch.int32, _sizes(shape)[1])
    _check(load_library().lsh_hash(_ptr(qk), _ptr(R), ctypes.byref(shape), _ptr(buckets), _ptr(ws),
                                   _nbytes(ws), _stream(stream)), "lsh_hash")


def lsh_sort(buckets, shape: Shape, perm, inv, ws, stream=None) -> None:
    n = _sizes(shape)[1]
    for what, t in (("buckets", buckets), ("perm", perm), ("inv", inv)):
        _need("lsh_sort", what, t, torch.int32, n)
    _check(load_library().lsh_sort(_ptr(buckets), ctypes.byref(shape), _ptr(perm), _ptr(inv),
                                   _ptr(ws), _nbytes(ws), _stream(stream)), "lsh_sort")


def lsh_sort_noalloc(buckets, shape: Shape, perm, inv, stream=None) -> None:
    n = _sizes(shape)[1]
    for what, t in (("buckets", buckets), ("perm", perm), ("inv", inv)):
        _need("lsh_sort_noalloc", what, t, torch.int32, n)
    _check(load_library().lsh_sort_noalloc(_ptr(buckets), ctypes.byref(shape), _ptr(perm),
                                           _ptr(inv), _stream(stream)), "lsh_sort_noalloc")


def lsh_chunk_attend(qk, v, buckets, perm, shape: Shape, o_sorted, lse_sorted, stream=None) -> None:
    fn = "lsh_chunk_attend"
    _need_qkvr(fn, shape, qk, v, with_r=False, with_out=False)
    n = _sizes(shape)[1]
    _need(fn, "buckets", buckets, torch.int32, n)
    _need(fn, "perm", perm, torch.int32, n)
    _need(fn, "o_sorted", o_sorted, torch.float32, n * shape.d)
    _need(fn, "lse_sorted", lse_sorted, torch.float32, n)
    _check(load_library().lsh_chunk_attend(_ptr(qk), _ptr(v), _ptr(buckets), _ptr(perm),
                                           ctypes.byref(shape), _ptr(o_sorted), _ptr(lse_sorted),
                                           _stream(stream)), fn)


def lsh_chunk_attend_qk(q, k, v, buckets_q, buckets_k, perm_q, perm_k, shape: Shape, o_sorted,
                        lse_sorted, stream=None) -> None:
    fn = "lsh_chunk_attend_qk"
    _need_qkvr(fn, shape, q, v, with_r=False, with_out=False)
    _need(fn, "k", k, _io(shape), _sizes(shape)[0])
    n = _sizes(shape)[1]
    for what, t in (("buckets_q", buckets_q), ("buckets_k", buckets_k), ("perm_q", perm_q),
                    ("perm_k", perm_k)):
        _need(fn, what, t, torch.int32, n)
    _need(fn, "o_sorted", o_sorted, torch.float32, n * shape.d)
    _need(fn, "lse_sorted", lse_sorted, torch.float32, n)
    _check(load_library().lsh_chunk_attend_qk(
        _ptr(q), _ptr(k), _ptr(v), _ptr(buckets_q), _ptr(buckets_k), _ptr(perm_q), _ptr(perm_k),
        ctypes.byref(shape), _ptr(o_sorted), _ptr(lse_sorted), _stream(stream)), fn)


def lsh_attention_fwd_qk(q, k, v, R, shape: Shape, out, ws, stream=None) -> None:
    fn = "lsh_attention_fwd_qk"
    _need_qkvr(fn, shape, q, v, R, out)
    _need(fn, "k", k, _io(shape), _sizes(shape)[0])
    _check(load_library().lsh_attention_fwd_qk(_ptr(q), _ptr(k), _ptr(v), _ptr(R),
                                               ctypes.byref(shape), _ptr(out), _ptr(ws),
                                               _nbytes(ws), _stream(stream)), fn)


def lsh_unsort_combine(o_sorted, lse_sorted, inv, shape: Shape, out, stream=None) -> None:
    fn = "lsh_unsort_combine"
    n = _sizes(shape)[1]
    _need(fn, "o_sorted", o_sorted, torch.float32, n * shape.d)
    _need(fn, "lse_sorted", lse_sorted, torch.float32, n)
    _need(fn, "inv", inv, torch.int32, n)
    _need(fn, "out", out, _io(shape), _sizes(shape)[0])
    _check(load_library().lsh_unsort_combine(_ptr(o_sorted), _ptr(lse_sorted), _ptr(inv),
                                             ctypes.byref(shape), _ptr(out), _stream(stream)), fn)


def lsh_attention_fwd(qk, v, R, shape: Shape, out, ws, stream=None) -> None:
    _need_qkvr("lsh_attention_fwd", shape, qk, v, R, out)
    _check(load_library().lsh_attention_fwd(_ptr(qk), _ptr(v), _ptr(R), ctypes.byref(shape),
                                            _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream)),
           "lsh_attention_fwd")


def lsh_attention_fwd_timed(qk, v, R, shape: Shape, out, ws, stream=None, max_kernels: int = 16):
    """Runs the forward and returns [(kernel name, milliseconds), ...] (waits for the GPU)."""
    _need_qkvr("lsh_attention_fwd_timed", shape, qk, v, R, out)
    ms = (ctypes.c_float * max_kernels)()
    names = (ctypes.c_char_p * max_kernels)()
    n = ctypes.c_int32(0)
    _check(load_library().lsh_attention_fwd_timed(
        _ptr(qk), _ptr(v), _ptr(R), ctypes.byref(shape), _ptr(out), _ptr(ws), _nbytes(ws),
        _stream(stream), ms, names, max_kernels, ctypes.byref(n)), "lsh_attention_fwd_timed")
    return [(names[k].decode(), float(ms[k])) for k in range(n.value)]


def lsh_ffn_workspace_size(rows: int, d_ff: int, chunk_rows: int, dtype: int) -> int:
    return _size_query(load_library().lsh_ffn_workspace_size(int(rows), int(d_ff),
                                                             int(chunk_rows), int(dtype)),
                       "lsh_ffn_workspace_size")


def lsh_ffn_chunked(x, w1, b1, w2, b2, rows: int, d_model: int, d_ff: int, chunk_rows: int,
                    dtype: int, out, ws, stream=None) -> None:
    fn = "lsh_ffn_chunked"
    io = _TORCH_DTYPE.get(dtype, torch.float32)
    _need(fn, "x", x, io, rows * d_model)
    _need(fn, "w1", w1, io, d_ff * d_model)
    _need(fn, "b1", b1, io, d_ff, optional=True)
    _need(fn, "w2", w2, io, d_model * d_ff)
    _need(fn, "b2", b2, io, d_model, optional=True)
    _need(fn, "out", out, io, rows * d_model)
    _check(load_library().lsh_ffn_chunked(_ptr(x), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2),
                                          int(rows), int(d_model), int(d_ff), int(chunk_rows),
                                          int(dtype), _ptr(out), _ptr(ws), _nbytes(ws),
                                          _stream(stream)), fn)


def ffn(x, w1, b1, w2, b2, chunk_rows: int, ws=None, out=None, stream=None):
    """Chunked feed-forward relu(x W1^T + b1) W2^T + b2 over the rows of x
    [..., d_model]; w1 [d_ff, d_model], w2 [d_model, d_ff], biases [d_ff],
    [d_model] or None, all in x's dtype. Returns out shaped like x."""
    if x.dtype not in _DTYPES:
        raise ValueError(f"x dtype must be float32 or bfloat16, got {x.dtype}")
    dm = x.shape[-1]
    dff = w1.shape[0]
    if w1.shape != (dff, dm) or w2.shape != (dm, dff):
        raise ValueError("w1 must be [d_ff, d_model] and w2 [d_model, d_ff]")
    for t, n in ((b1, dff), (b2, dm)):
        if t is not None and t.shape != (n,):
            raise ValueError("biases must be [d_ff] and [d_model]")
    for t in (w1, w2, b1, b2):
        if t is not None and t.dtype != x.dtype:
            raise ValueError("weights and biases must be in x's dtype")
    rows = x.numel() // dm if dm else 0
    dtype = _DTYPES[x.dtype]
    if out is not None and (out.shape != x.shape or out.dtype != x.dtype):
        raise ValueError("out must match x in shape and dtype")
    out = torch.empty_like(x) if out is None else out
    if ws is None:
        ws = torch.empty(max(1, lsh_ffn_workspace_size(rows, dff, chunk_rows, dtype)),
                         dtype=torch.uint8, device=x.device)
    lsh_ffn_chunked(x, w1, b1, w2, b2, rows, dm, dff, chunk_rows, dtype, out, ws, stream)
    return out


def lsh_qkv_project(x, w_qk, w_v, shape: Shape, d_model: int, qk, v, stream=None) -> None:
    fn = "lsh_qkv_project"
    io = _io(shape)
    _need(fn, "x", x, io, shape.B * shape.L * d_model)
    _need(fn, "w_qk", w_qk, io, shape.H * shape.d * d_model)
    _need(fn, "w_v", w_v, io, shape.H * shape.d * d_model)
    _need_qkvr(fn, shape, qk, v, with_r=False, with_out=False)
    _check(load_library().lsh_qkv_project(_ptr(x), _ptr(w_qk), _ptr(w_v), ctypes.byref(shape),
                                          int(d_model), _ptr(qk), _ptr(v), _stream(stream)), fn)


def lsh_attention_fwd_x(x, w_qk, w_v, R, shape: Shape, d_model: int, out, ws,
                        stream=None) -> None:
    fn = "lsh_attention_fwd_x"
    io = _io(shape)
    _need(fn, "x", x, io, shape.B * shape.L * d_model)
    _need(fn, "w_qk", w_qk, io, shape.H * shape.d * d_model)
    _need(fn, "w_v", w_v, io, shape.H * shape.d * d_model)
    rows, _, r = _sizes(shape)
    _need(fn, "R", R, torch.float32, r)
    _need(fn, "out", out, io, rows)
    _check(load_library().lsh_attention_fwd_x(
        _ptr(x), _ptr(w_qk), _ptr(w_v), _ptr(R), ctypes.byref(shape), int(d_model), _ptr(out),
        _ptr(ws), _nbytes(ws), _stream(stream)), fn)


def _nbytes(t):
    return t.numel() * t.element_size() if t is not None else 0


def lsh_attention_fwd_train(qk, v, R, shape: Shape, out, state, ws, stream=None) -> None:
    _need_qkvr("lsh_attention_fwd_train", shape, qk, v, R, out)
    _check(load_library().lsh_attention_fwd_train(
        _ptr(qk), _ptr(v), _ptr(R), ctypes.byref(shape), _ptr(out), _ptr(state), _nbytes(state),
        _ptr(ws), _nbytes(ws), _stream(stream)), "lsh_attention_fwd_train")


def lsh_attention_bwd(qk, v, out, dout, state, shape: Shape, dqk, dv, ws, stream=None) -> None:
    fn = "lsh_attention_bwd"
    _need_qkvr(fn, shape, qk, v, out=out, with_r=False)
    rows = _sizes(shape)[0]
    for what, t in (("dout", dout), ("dqk", dqk), ("dv", dv)):
        _need(fn, what, t, _io(shape), rows)
    _check(load_library().lsh_attention_bwd(
        _ptr(qk), _ptr(v), _ptr(out), _ptr(dout), _ptr(state), _nbytes(state),
        ctypes.byref(shape), _ptr(dqk), _ptr(dv), _ptr(ws), _nbytes(ws), _stream(stream)), fn)


# ---------------------------------------------------------------- allocating helpers

def _workspace(stage: str, shape: Shape, device) -> torch.Tensor:
    return torch.empty(max(1, lsh_workspace_size(stage, shape)), dtype=torch.uint8, device=device)


def _rounds_shape(shape: Shape):
    return (shape.B, shape.H, shape.n_hashes, shape.L)


def hash(qk, R, n_buckets: int, ws=None, stream=None):
    """Returns (buckets [B,H,n_hashes,L] int32, number of token-rounds re-decided in fp64)."""
    nh, per_head = check_rotations(R, qk, n_buckets)
    shape = shape_of(qk, n_buckets, nh, 1, False, per_head_r=per_head)
    shape.chunk_len = max(1, shape.L)  # any divisor of L: the hash does not use it
    buckets = torch.empty(_rounds_shape(shape), dtype=torch.int32, device=qk.device)
    ws = _workspace("hash", shape, qk.device) if ws is None else ws
    lsh_hash(qk, R, shape, buckets, ws, stream)
    refined = int(ws[:4].view(torch.int32).item()) if shape.B * shape.H * shape.L else 0
    return buckets, refined


def sort(buckets, n_buckets: int, stream=None):
    """Returns (perm, inv), both [B,H,n_hashes,L] int32."""
    B, H, nh, L = buckets.shape
    shape = Shape(B, H, L, 64, n_buckets, nh, max(1, L), 0, LSH_BF16)
    perm = torch.empty_like(buckets)
    inv = torch.empty_like(buckets)
    ws = _workspace("sort", shape, buckets.device)
    lsh_sort(buckets, shape, perm, inv, ws, stream)
    return perm, inv


def chunk_attend(qk, v, buckets, perm, n_buckets: int, chunk_len: int, causal: bool, stream=None,
                 key_norm: bool = False):
    """Returns (o_sorted [B,H,n_hashes,L,d] f32, lse_sorted [B,H,n_hashes,L] f32)."""
    shape = shape_of(qk, n_buckets, buckets.shape[2], chunk_len, causal, key_norm)
    o = torch.empty(_rounds_shape(shape) + (shape.d,), dtype=torch.float32, device=qk.device)
    lse = torch.empty(_rounds_shape(shape), dtype=torch.float32, device=qk.device)
    lsh_chunk_attend(qk, v, buckets, perm, shape, o, lse, stream)
    return o, lse


def chunk_attend_qk(q, k, v, buckets_q, buckets_k, perm_q, perm_k, n_buckets: int,
                    chunk_len: int, causal: bool, stream=None):
    """Separate queries and keys: returns (o_sorted, lse_sorted) by query slot,
    [B,H,n_hashes,L,d] and [B,H,n_hashes,L] float32 (lse -inf and a zero row
    for a query whose window holds no key of its bucket)."""
    check_like(k, q, "k")
    check_like(v, q, "v")
    shape = shape_of(q, n_buckets, buckets_q.shape[2], chunk_len, causal)
    o = torch.empty(_rounds_shape(shape) + (shape.d,), dtype=torch.float32, device=q.device)
    lse = torch.empty(_rounds_shape(shape), dtype=torch.float32, device=q.device)
    lsh_chunk_attend_qk(q, k, v, buckets_q, buckets_k, perm_q, perm_k, shape, o, lse, stream)
    return o, lse


def attention_fwd_qk(q, k, v, R, n_buckets: int, chunk_len: int, causal: bool, ws=None,
                     out=None, stream=None):
    """Whole forward with separate queries and keys (the ablation); returns out
    [B,H,L,d] in q's dtype (zero rows for queries that find no key)."""
    nh, per_head = check_rotations(R, q, n_buckets)
    shape = shape_of(q, n_buckets, nh, chunk_len, causal, per_head_r=per_head)
    check_like(k, q, "k")
    check_like(v, q, "v")
    if out is not None:
        check_like(out, q, "out")
    out = torch.empty_like(q) if out is None else out
    ws = _workspace("fwd_qk", shape, q.device) if ws is None else ws
    lsh_attention_fwd_qk(q, k, v, R, shape, out, ws, stream)
    return out


def unsort_combine(o_sorted, lse_sorted, inv, dtype=torch.bfloat16, stream=None):
    """Returns out [B,H,L,d] in ``dtype``."""
    B, H, nh, L, d = o_sorted.shape
    shape = Shape(B, H, L, d, 2, nh, max(1, L), 0, _DTYPES[dtype])
    out = torch.empty((B, H, L, d), dtype=dtype, device=o_sorted.device)
    lsh_unsort_combine(o_sorted, lse_sorted, inv, shape, out, stream)
    return out


def attention_fwd(qk, v, R, n_buckets: int, chunk_len: int, causal: bool, ws=None, out=None,
                  stream=None, key_norm: bool = False):
    """Whole forward; returns out [B,H,L,d] in qk's dtype."""
    nh, per_head = check_rotations(R, qk, n_buckets)
    shape = shape_of(qk, n_buckets, nh, chunk_len, causal, key_norm, per_head)
    check_like(v, qk, "v")
    if out is not None:
        check_like(out, qk, "out")
    out = torch.empty_like(qk) if out is None else out
    ws = _workspace("fwd", shape, qk.device) if ws is None else ws
    lsh_attention_fwd(qk, v, R, shape, out, ws, stream)
    return out


def _x_shape(x, w_qk, w_v, n_heads: int, n_buckets: int, n_hashes: int, chunk_len: int,
             causal: bool, key_norm: bool = False, per_head_r: bool = False) -> Shape:
    if x.dim() != 3:
        raise ValueError(f"x must be [B, L, d_model], got {tuple(x.shape)}")
    if x.dtype not in _DTYPES:
        raise ValueError(f"x dtype must be float32 or bfloat16, got {x.dtype}")
    B, L, dm = x.shape
    n_out = w_qk.shape[0]
    if (w_qk.shape != (n_out, dm) or w_v.shape != (n_out, dm) or n_out % n_heads
            or w_qk.dtype != x.dtype or w_v.dtype != x.dtype):
        raise ValueError("w_qk and w_v must be [H * d, d_model] in x's dtype")
    return Shape(B, n_heads, L, n_out // n_heads, n_buckets, n_hashes, chunk_len,
                 int(bool(causal)), _DTYPES[x.dtype],
                 (LSH_KEY_NORM if key_norm else 0) | (LSH_PER_HEAD_R if per_head_r else 0))


def qkv_project(x, w_qk, w_v, n_heads: int, stream=None):
    """Returns (qk, v), both [B, H, L, d] in x's dtype, from x [B, L, d_model]
    and weights [H * d, d_model]."""
    shape = _x_shape(x, w_qk, w_v, n_heads, 2, 1, 1, False)
    shape.chunk_len = max(1, shape.L)
    qk = torch.empty((shape.B, shape.H, shape.L, shape.d), dtype=x.dtype, device=x.device)
    v = torch.empty_like(qk)
    lsh_qkv_project(x, w_qk, w_v, shape, x.shape[2], qk, v, stream)
    return qk, v


def attention_fwd_x(x, w_qk, w_v, R, n_heads: int, n_buckets: int, chunk_len: int, causal: bool,
                    ws=None, out=None, stream=None, key_norm: bool = False):
    """Projections, then the whole forward; returns out [B, H, L, d] in x's dtype."""
    nh, per_head = rounds_of(R)
    shape = _x_shape(x, w_qk, w_v, n_heads, n_buckets, nh, chunk_len, causal, key_norm, per_head)
    ref = torch.empty((shape.B, shape.H, shape.L, shape.d), dtype=x.dtype, device=x.device)
    check_rotations(R, ref, n_buckets)
    if out is not None:
        check_like(out, ref, "out")
    out = ref if out is None else out
    ws = _workspace("fwd_x", shape, x.device) if ws is None else ws
    lsh_attention_fwd_x(x, w_qk, w_v, R, shape, x.shape[2], out, ws, stream)
    return out


def attention_fwd_train(qk, v, R, n_buckets: int, chunk_len: int, causal: bool, stream=None,
                        key_norm: bool = False):
    """Training forward; returns (out [B,H,L,d], state) for attention_bwd."""
    nh, per_head = check_rotations(R, qk, n_buckets)
    shape = shape_of(qk, n_buckets, nh, chunk_len, causal, key_norm, per_head)
    check_like(v, qk, "v")
    out = torch.empty_like(qk)
    state = _workspace("state", shape, qk.device)
    ws = _workspace("fwd", shape, qk.device)
    lsh_attention_fwd_train(qk, v, R, shape, out, state, ws, stream)
    return out, state


def attention_bwd(qk, v, out, dout, state, n_buckets: int, n_hashes: int, chunk_len: int,
                  causal: bool, stream=None, key_norm: bool = False):
    """Returns (dqk, dv) for the output gradient dout (contiguous, qk's dtype);
    ``key_norm`` must match the training forward that wrote ``state``."""
    shape = shape_of(qk, n_buckets, n_hashes, chunk_len, causal, key_norm)
    dout = dout.to(qk.dtype).contiguous()
    dqk = torch.empty_like(qk)
    dv = torch.empty_like(v)
    ws = _workspace("bwd", shape, qk.device)
    lsh_attention_bwd(qk, v, out, dout, state, shape, dqk, dv, ws, stream)
    return dqk, dv


class LSHAttention(torch.autograd.Function):
    """out = LSH attention of (qk, v) with rotations R; differentiable in qk
    and v (the hash and the sort carry no gradient; R gets none).
    Use: ``LSHAttention.apply(qk, v, R, n_buckets, chunk_len, causal[, key_norm])``."""

    @staticmethod
    def forward(ctx, qk, v, R, n_buckets, chunk_len, causal, key_norm=False):
        qk = qk.contiguous()
        v = v.contiguous()
        out, state = attention_fwd_train(qk, v, R.contiguous(), n_buckets, chunk_len, causal,
                                         key_norm=key_norm)
        ctx.save_for_backward(qk, v, out, state)
        ctx.cfg = (n_buckets, rounds_of(R)[0], chunk_len, causal)
        ctx.key_norm = key_norm
        return out

    @staticmethod
    def backward(ctx, dout):
        qk, v, out, state = ctx.saved_tensors
        dqk, dv = attention_bwd(qk, v, out, dout, state, *ctx.cfg, key_norm=ctx.key_norm)
        return dqk, dv, None, None, None, None, None
