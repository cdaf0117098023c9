"""GPU parity of the chunked feed-forward (lsh_ffn_chunked) against the oracle.

Bars, element by element, from the arithmetic (S = sum_f |h_f w2[o, f]| with h
the exact hidden activations, and |ref| the exact output):
  * bf16 I/O: the hidden activations are rounded to bf16 (2^-9 relative
    each), the output too, and both products accumulate in fp32:
    |gpu - ref| <= 2^-8 (|ref| + S) + 1e-6;
  * fp32 I/O: fp32 accumulation over d_model and d_ff terms:
    |gpu - ref| <= 2e-5 (|ref| + S) + 1e-6.
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lsh.load_library()


def _inputs(dtype, rows, dm, dff, seed, bias=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, dm), dtype=np.float32)
    w1 = (rng.standard_normal((dff, dm), dtype=np.float32) / np.sqrt(dm)).astype(np.float32)
    w2 = (rng.standard_normal((dm, dff), dtype=np.float32) / np.sqrt(dff)).astype(np.float32)
    b1 = rng.standard_normal(dff, dtype=np.float32) * 0.1 if bias else None
    b2 = rng.standard_normal(dm, dtype=np.float32) * 0.1 if bias else None
    arrs = [x, w1, b1, w2, b2]
    if dtype == "bf16":
        arrs = [None if a is None else workloads.round_to_bf16(a) for a in arrs]
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = [None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV, dt)
           for a in arrs]
    return arrs, dev


def _bound(dtype, arrs, ref):
    x, w1, b1, w2, _ = (np.asarray(a, np.float64) if a is not None else None for a in arrs)
    h = x @ w1.T + (b1 if b1 is not None else 0.0)
    S = np.maximum(h, 0.0) @ np.abs(w2).T
    rel = 2.0 ** -8 if dtype == "bf16" else 2e-5
    return rel * (np.abs(ref) + S) + 1e-6


CASES = [("bf16", 1000, 256, 1024, 384, True), ("bf16", 333, 128, 512, 1000, False),
         ("bf16", 64, 1024, 4096, 64, True), ("fp32", 300, 64, 200, 128, True),
         ("fp32", 77, 128, 96, 7, False)]


@pytest.mark.parametrize("dtype,rows,dm,dff,chunk,bias", CASES)
def test_ffn_matches_oracle(dtype, rows, dm, dff, chunk, bias):
    arrs, dev = _inputs(dtype, rows, dm, dff, rows + dff, bias)
    out = lsh.ffn(*dev, chunk)
    ref = oracle.ffn(*arrs, chunk)
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    err = np.abs(got - ref)
    bound = _bound(dtype, arrs, ref)
    print(f"ffn {dtype} rows={rows} chunk={chunk}: max err {err.max():.2e}, "
          f"max err/bound {(err / bound).max():.2f}")
    assert np.all(err <= bound)


def test_ffn_chunk_size_is_bit_invisible():
    arrs, dev = _inputs("bf16", 700, 256, 512, 5)
    ref = lsh.ffn(*dev, 700)
    for chunk in (1, 128, 129, 4096):
        assert torch.equal(lsh.ffn(*dev, chunk), ref)


def test_ffn_full_size_sampled_rows():
    """The benchmark's feed-forward: 65536 rows, d_model 1024, d_ff 4096,
    chunks of 8192 rows, bf16; 48 sampled rows against the oracle."""
    rows, dm, dff, chunk = 65536, 1024, 4096, 8192
    arrs, dev = _inputs("bf16", rows, dm, dff, 1006)
    out = lsh.ffn(*dev, chunk)
    pick = np.sort(np.random.default_rng(3).choice(rows, 48, replace=False))
    pick[0], pick[-1] = 0, rows - 1
    sub = [arrs[0][pick]] + arrs[1:]
    ref = oracle.ffn(*sub, 16)
    got = out[torch.from_numpy(pick).to(DEV)].float().cpu().numpy()
    assert np.all(np.abs(got - ref) <= _bound("bf16", sub, ref))


def test_ffn_empty_rows():
    arrs, dev = _inputs("bf16", 8, 64, 128, 1)
    x0 = dev[0][:0]
    assert lsh.ffn(x0, *dev[1:], 16).shape == (0, 64)
