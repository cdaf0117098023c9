"""LSH attention (Reformer) forward pass for AMD MI355X (gfx950).

A thin ctypes binding over the C ABI of ``liblsh_attn.so`` (declared in
``include/lsh_attn.h``). Every step runs in the library's HIP kernels; this
module only checks tensors and passes their device pointers and torch's
current HIP stream. It raises if the library has not been built -- there is
no other implementation to fall back to.

Low-level functions keep the C names and argument order (tensors in place of
pointers): ``lsh_workspace_size``, ``lsh_hash``, ``lsh_sort``, ``lsh_sort_noalloc``,
``lsh_chunk_attend``, ``lsh_chunk_attend_qk``, ``lsh_unsort_combine``,
``lsh_attention_fwd``, ``lsh_attention_fwd_qk``,
``lsh_attention_fwd_timed``, ``lsh_qkv_project``, ``lsh_attention_fwd_x``,
``lsh_attention_fwd_train``, ``lsh_attention_bwd``. The allocating helpers
``hash``, ``sort``, ``chunk_attend``, ``unsort_combine``, ``attention_fwd``,
``qkv_project``, ``attention_fwd_x``, ``attention_fwd_train`` and
``attention_bwd`` create the outputs and workspaces with torch;
``LSHAttention`` is a torch.autograd.Function over the training forward and
the backward.
"""
from ._binding import (  # noqa: F401
    LSH_BF16,
    LSH_F32,
    LSH_KEY_NORM,
    LSH_PER_HEAD_R,
    LSHAttention,
    LshError,
    Shape,
    attention_bwd,
    attention_fwd,
    attention_fwd_qk,
    attention_fwd_train,
    attention_fwd_x,
    chunk_attend,
    chunk_attend_qk,
    ffn,
    hash,
    library_path,
    load_library,
    rounds_of,
    lsh_attention_fwd,
    lsh_attention_fwd_timed,
    lsh_attention_bwd,
    lsh_attention_fwd_train,
    lsh_attention_fwd_x,
    lsh_attention_fwd_qk,
    lsh_chunk_attend,
    lsh_chunk_attend_qk,
    lsh_ffn_chunked,
    lsh_ffn_workspace_size,
    lsh_hash,
    lsh_last_error,
    lsh_qkv_project,
    lsh_sort,
    lsh_sort_noalloc,
    lsh_unsort_combine,
    lsh_workspace_size,
    qkv_project,
    shape_of,
    sort,
    unsort_combine,
)
