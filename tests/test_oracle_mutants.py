"""The pins must catch plausible slips in the oracle.

Each case plants one mistake in a temporary copy of ``oracle/lsh_oracle.c``
(the committed oracle is never touched), builds it with gcc, and runs every
pin of ``test_oracle_pins.py`` against it: at least one pin must fail.
"""
from __future__ import annotations

import importlib.util
import inspect
import pathlib
import subprocess

import numpy as np
import pytest

from tests import test_oracle_pins as pins

ROOT = pathlib.Path(__file__).resolve().parent.parent
SRC = ROOT / "oracle" / "lsh_oracle.c"
PY = ROOT / "oracle" / "oracle.py"

MUTANTS = {
    "halves_swapped": ("c[b] = p;\n                    c[b + half] = -p;",
                       "c[b] = -p;\n                    c[b + half] = p;"),
    "last_index_ties": ("if (c[b] > c[best]) best = b;", "if (c[b] >= c[best]) best = b;"),
    "R_transposed": ("R[((int64_t)r * d + k) * half + b]", "R[((int64_t)r * half + b) * d + k]"),
    "sort_position_descending": ("if (a->pos != b->pos) return a->pos < b->pos ? -1 : 1;",
                                 "if (a->pos != b->pos) return a->pos < b->pos ? 1 : -1;"),
    # windows stay within 2m slots so the mutant never writes past its buffers
    "next_chunk_instead_of_previous": (
        "const int64_t t0 = (c > 0) ? (c - 1) * m : 0; /* no look-back for chunk 0 */\n"
        "            const int64_t t1 = (c + 1) * m; ",
        "const int64_t t0 = c * m;\n"
        "            const int64_t t1 = ((c + 2) * m < L) ? (c + 2) * m : L; "),
    "own_chunk_only": ("const int64_t t0 = (c > 0) ? (c - 1) * m : 0;",
                       "const int64_t t0 = c * m;"),
    "scale_one_over_d": ("const double scale = 1.0 / sqrt((double)d);",
                         "const double scale = 1.0 / (double)d;"),
    "no_self_penalty": ("if (j == i) sc -= ORACLE_SELF_PENALTY;", "(void)0;"),
    "causal_strict": ("(!causal || j <= i)", "(!causal || j < i)"),
    "causal_ignored": ("(!causal || j <= i)", "(1)"),
    "no_bucket_mask": ("int ok = (bucket[j] == bucket[i]) &&", "int ok = 1 &&"),
    "uniform_round_weights": ("const double w = exp(lse[(int64_t)r * L + s] - z);",
                              "const double w = 1.0 / n_hashes;"),
    "combine_wrong_round_slot": ("const int64_t s = inv[(int64_t)r * L + i];",
                                 "const int64_t s = inv[i];"),
    "lse_log2": ("const double l = mx + log(sum);", "const double l = mx + log2(sum);"),
    # every index below stays inside the buffers for any shape
    "project_weights_transposed": (
        "sq += xr[k] * wq[k];",
        "sq += xr[k] * w_qk[(int64_t)k * H * d + (int64_t)h * d + e];"),
    "project_layout_bl_h": (
        "double *qo = qk + (((int64_t)b * H + h) * L + l) * d;",
        "double *qo = qk + (((int64_t)b * L + l) * H + h) * d;"),
    "project_v_from_qk_weights": ("sv += xr[k] * wv[k];", "sv += xr[k] * wq[k];"),
    "backward_no_key_gradient": ("gx[j * d + k] += ds * scale * xi[k];", "(void)0;"),
    "backward_round_lse_as_normaliser": ("const double p = exp(sc - z[i]);",
                                         "const double p = exp(sc - ls[(int64_t)r * L + s]);"),
    "backward_no_D_term": ("const double ds = p * (gdv - dd[i]);", "const double ds = p * gdv;"),
    "backward_dv_to_query": ("gv[j * d + k] += p * gi[k];", "gv[i * d + k] += p * gi[k];"),
    "key_norm_on_the_query": ("if (key_norm) sc *= inv_norm(xj, d);",
                              "if (key_norm) sc *= inv_norm(xi, d);"),
    # both stay inside R for any shape
    "per_head_rotations_of_the_batch": ("return R + (bh % H) * per_head;",
                                        "return R + ((bh / H) % H) * per_head;"),
    "per_head_rotations_ignored": ("if (!per_head_r) return R;", "return R;"),
    # w1[k * d_ff + f] stays inside w1's d_ff * d_model elements
    "ffn_w1_transposed": ("const double *w = w1 + (int64_t)f * d_model;\n"
                          "                double s = 0.0;\n"
                          "                for (int k = 0; k < d_model; ++k) s += xr[k] * w[k];",
                          "double s = 0.0;\n"
                          "                for (int k = 0; k < d_model; ++k) "
                          "s += xr[k] * w1[(int64_t)k * d_ff + f];"),
    "ffn_no_relu": ("h[i * d_ff + f] = s > 0.0 ? s : 0.0;", "h[i * d_ff + f] = s;"),
    "ffn_no_second_bias": ("if (b2) s += b2[o];", "(void)b2;"),
    "ffn_chunk_restarts_rows": ("const double *xr = x + (r0 + i) * d_model;",
                                "const double *xr = x + i * d_model;"),
    "key_norm_backward_no_projection": ("(xi[k] - dot * rn * rn * xj[k])", "(xi[k])"),
    # the chosen-rows backward: queries of the next chunk (which look back at
    # a chosen key) left out; terms landing only in a chosen key row skipped
    "backward_rows_no_next_chunk": ("if (c + 1 < n_chunks) qchunk[r * n_chunks + c + 1] = 1;",
                                    "(void)0;"),
    "backward_rows_query_side_only": ("if (row[i] < 0 && row[j] < 0) continue;",
                                      "if (row[i] < 0) continue;"),
    # separate queries and keys
    "qk_keys_in_query_order": ("const int64_t j = perm_k[t];", "const int64_t j = perm_q[t];"),
    "qk_self_penalty": ("const double sc = dot * scale;\n                score[t - t0] = sc;",
                        "const double sc = dot * scale - (j == i ? ORACLE_SELF_PENALTY : 0.0);\n"
                        "                score[t - t0] = sc;"),
    "qk_query_buckets_for_keys": ("(bucket_k[j] == bucket_q[i])", "(bucket_q[j] == bucket_q[i])"),
    "qk_empty_round_lse_zero": ("lse[s] = -INFINITY;", "lse[s] = 0.0;"),
    "qk_keys_hashed_as_queries": ("rc = oracle_hash(kk, L, d, Rh, n_hashes, n_buckets, bk, mk);",
                                  "rc = oracle_hash(qq, L, d, Rh, n_hashes, n_buckets, bk, mk);"),
    "qk_combined_through_key_order": ("oracle_combine(os, ls, iq,", "oracle_combine(os, ls, ik,"),
    "combine_empty_row_not_zero": ("if (mx == -INFINITY) {", "if (0) {"),
}


def _pin_calls():
    calls = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        params = list(inspect.signature(fn).parameters)
        if "oracle_mod" not in params:
            continue
        grid = [{}]
        for mark in getattr(fn, "pytestmark", []):
            if mark.name == "parametrize":
                argnames, values = mark.args
                names = [a.strip() for a in argnames.split(",")]
                rows = [v if len(names) > 1 else (v,) for v in values]
                grid = [dict(g, **dict(zip(names, row))) for g in grid for row in rows]
        for kw in grid:
            calls.append((name, fn, kw))
    return calls


def _load_mutant(tmp: pathlib.Path, name: str, old: str, new: str):
    text = SRC.read_text()
    assert text.count(old) >= 1, f"mutation {name}: pattern not found"
    mutated = text.replace(old, new)
    c_path = tmp / f"{name}.c"
    so_path = tmp / f"lib{name}.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-std=c11", "-O1", "-ffp-contract=off", "-fopenmp", "-shared",
                    "-fPIC", str(c_path), "-o", str(so_path), "-lm"], check=True)
    spec = importlib.util.spec_from_file_location(f"oracle_mutant_{name}", PY)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._LIB_PATH = so_path
    mod._lib = None
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    mod = _load_mutant(tmp_path, name, old, new)
    caught = []
    with np.errstate(all="ignore"):
        for pin, fn, kw in _pin_calls():
            try:
                fn(mod, **kw)
            except (AssertionError, ValueError, FloatingPointError, IndexError):
                caught.append(pin)
    assert caught, f"no pin catches the planted mistake {name!r}"


def test_unmutated_copy_passes(tmp_path):
    """Control: the copy-and-build route itself does not make pins fail."""
    mod = _load_mutant(tmp_path, "control", "#define ORACLE_SELF_PENALTY 1.0e5",
                       "#define ORACLE_SELF_PENALTY 1.0e5")
    for pin, fn, kw in _pin_calls():
        fn(mod, **kw)
