"""lsh_sort_noalloc (the sort with its counts in the library's static device
scratch, for callers that cannot allocate) against lsh_sort with a workspace,
through the C ABI: bit-equal permutations and inverses on two calls in a row,
the second with a smaller input (so a stale first call's contents cannot
pass), and the scratch's size limit refused before any launch."""
from __future__ import annotations

import numpy as np
import pytest
import torch

lsh = pytest.importorskip("lsh_attention_fp32_amd")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lsh.load_library()


def _shape(B, H, nh, L, nb):
    return lsh.Shape(B, H, L, 64, nb, nh, max(1, L), 0, lsh.LSH_BF16)


def _both(B, H, nh, L, nb, seed):
    rng = np.random.default_rng(seed)
    b = torch.from_numpy(rng.integers(0, nb, (B, H, nh, L)).astype(np.int32)).to(DEV)
    ref_perm, ref_inv = lsh.sort(b, nb)               # lsh_sort, torch-allocated workspace
    s = _shape(B, H, nh, L, nb)
    perm = torch.full_like(b, -1)
    inv = torch.full_like(b, -1)
    lsh.lsh_sort_noalloc(b, s, perm, inv)
    torch.cuda.synchronize()
    return ref_perm, ref_inv, perm, inv


def test_noalloc_sort_equals_workspace_sort_twice():
    # the benchmark's shape (64 segments of 64K positions, 1024 buckets), then
    # a smaller one with a ragged last tile and fewer buckets
    for (B, H, nh, L, nb), seed in (((1, 8, 8, 65536, 1024), 1), ((1, 2, 3, 4096 + 192, 64), 2)):
        ref_perm, ref_inv, perm, inv = _both(B, H, nh, L, nb, seed)
        assert torch.equal(perm, ref_perm), f"perm differs at {(B, H, nh, L, nb)}"
        assert torch.equal(inv, ref_inv), f"inv differs at {(B, H, nh, L, nb)}"
        print(f"noalloc sort {(B, H, nh, L, nb)}: equal to lsh_sort")


def test_noalloc_sort_refuses_shapes_past_its_scratch():
    # 16 MiB of scratch: 8 segments x 256 tiles x 4096 buckets x 4 B = 32 MiB
    s = _shape(1, 1, 8, 1 << 20, 4096)
    need = lsh.lsh_workspace_size("sort", s)
    assert need > 16 << 20
    t = torch.empty(8, dtype=torch.int32, device=DEV)
    rc = lsh.load_library().lsh_sort_noalloc(lsh._binding._ptr(t), __import__("ctypes").byref(s),
                                             lsh._binding._ptr(t), lsh._binding._ptr(t), None)
    assert rc == -2 and "static scratch" in lsh.lsh_last_error()
