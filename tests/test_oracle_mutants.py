"""The pins are strong enough: plausible mistakes planted in the oracle (on the
CPU, in throwaway copies of its C source) each fail at least one pin.

Every mutant below is a one-line slip someone could make while writing the
orders from the bankML f16 page (Design notes): a wrong pairing at any level
of either tree, the tail summed in f32, a mis-indexed chain, a dropped tail
term, the wrong path rule, a transposed output, a rounding slip in to_f16 or
widen; and in the next rows: the wrong output column of the last layer, a
K-cache layout or head-mapping slip, an unfused or mis-indexed mad, a
mis-indexed scale.  The test builds each copy, binds the oracle's API to it and runs the
pin functions from test_oracle_orders / test_oracle_convert against it.
"""
import inspect
import os
import subprocess

import pytest

import oracle
import test_oracle_convert as tc
import test_oracle_next as tn
import test_oracle_orders as to

SRC = open(os.path.join(os.path.dirname(oracle.__file__), "f16wm_oracle.c")).read()

MUTANTS = {
    "vec_dot level 1 pairs (a0+a1)+(a2+a3)": (
        "s[l] = (acc[0][l] + acc[2][l]) + (acc[1][l] + acc[3][l]);",
        "s[l] = (acc[0][l] + acc[1][l]) + (acc[2][l] + acc[3][l]);"),
    "vec_dot halves added adjacent-first": (
        "u[i] = s[i] + s[i + 4];", "u[i] = s[2 * i] + s[2 * i + 1];"),
    "vec_dot hadd pairs (u0+u2)+(u1+u3)": (
        "float v = (u[0] + u[1]) + (u[2] + u[3]);", "float v = (u[0] + u[2]) + (u[1] + u[3]);"),
    "vec_dot tail summed in f32": (
        "d = d + (double)p;", "d = (float)(d + (double)p);"),
    "vec_dot chains interleaved lane-major": (
        "int64_t e = i + 8 * j + l;", "int64_t e = i + 4 * l + j;"),
    "vec_dot tail drops the last element": (
        "for (int64_t i = np; i < k; i++) {", "for (int64_t i = np; i + 1 < k; i++) {"),
    "vec_dot steps of 16": (
        "int64_t np = k - k % 32;", "int64_t np = k - k % 16;"),
    "vec_dot whole reduction in double": (
        "double d = (double)v;",
        "double d = ((double)acc[0][0]+acc[2][0]+acc[1][0]+acc[3][0]+acc[0][4]+acc[2][4]+acc[1][4]+acc[3][4]"
        "+acc[0][1]+acc[2][1]+acc[1][1]+acc[3][1]+acc[0][5]+acc[2][5]+acc[1][5]+acc[3][5]"
        "+acc[0][2]+acc[2][2]+acc[1][2]+acc[3][2]+acc[0][6]+acc[2][6]+acc[1][6]+acc[3][6]"
        "+acc[0][3]+acc[2][3]+acc[1][3]+acc[3][3]+acc[0][7]+acc[2][7]+acc[1][7]+acc[3][7]); (void)v;"),
    "sgemm hsum pairs (l0+l1)": (
        "return ((acc[0] + acc[4]) + (acc[2] + acc[6])) + ((acc[1] + acc[5]) + (acc[3] + acc[7]));",
        "return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));"),
    "sgemm hsum pairs (l0+l4)+(l1+l5)": (
        "return ((acc[0] + acc[4]) + (acc[2] + acc[6])) + ((acc[1] + acc[5]) + (acc[3] + acc[7]));",
        "return ((acc[0] + acc[4]) + (acc[1] + acc[5])) + ((acc[2] + acc[6]) + (acc[3] + acc[7]));"),
    "sgemm lane indexing off by one": (
        "acc[l] = fmaf(W16(x[i + l]), W16(y[i + l]), acc[l]);",
        "acc[l] = fmaf(W16(x[i + (l ^ 1)]), W16(y[i + l]), acc[l]);"),
    "takes_sgemm rows % 2": (
        "return n >= 2 && rows % 4 == 0 && k % 8 == 0;", "return n >= 2 && rows % 2 == 0 && k % 8 == 0;"),
    "takes_sgemm n >= 1": (
        "return n >= 2 && rows % 4 == 0 && k % 8 == 0;", "return n >= 1 && rows % 4 == 0 && k % 8 == 0;"),
    "takes_sgemm without the k rule": (
        "return n >= 2 && rows % 4 == 0 && k % 8 == 0;", "return n >= 2 && rows % 4 == 0;"),
    "mat_mul output transposed": (
        "j->out[c * j->rows + r] =", "j->out[r * j->n + c] ="),
    "to_f16 ties away from zero": (
        "if (rem > half || (rem == half && (N & 1u))) N += 1;", "if (rem >= half) N += 1;"),
    "to_f16 truncates": (
        "if (rem > half || (rem == half && (N & 1u))) N += 1;", "(void)half;"),
    "to_f16 flushes subnormals": (
        "if (qexp == -24 && N <= 1024)\n        enc = N;",
        "if (qexp == -24 && N <= 1024)\n        enc = (N == 1024 ? N : 0);"),
    "widen subnormal scale": (
        "ldexpf((float)f, -24)", "ldexpf((float)f, -25)"),
    "widen normal bias": (
        "ldexpf((float)(1024u + f), (int)e - 25)", "ldexpf((float)(1024u + f), (int)e - 24)"),
    "mat_mul_out takes the first column": (
        "a + (n - 1) * k, 1, out, nthreads);", "a, 1, out, nthreads);"),
    "kq maps query heads round-robin": (
        "(p * n_kv_head + h / G) * d", "(p * n_kv_head + h % n_kv_head) * d"),
    "kq reads a head-major cache": (
        "(p * n_kv_head + h / G) * d", "(h / G * n_kv + p) * d"),
    "mad rounds the product first": (
        "oracle_to_f16_one(fmaf(W16(v[e]), w[b], W16(acc[e])))",
        "oracle_to_f16_one(W16(v[e]) * w[b] + W16(acc[e]))"),
    "mad uses the first vector's weight": (
        "fmaf(W16(v[e]), w[b], W16(acc[e]))", "fmaf(W16(v[e]), w[0], W16(acc[e]))"),
    "scale uses the first vector's factor": (
        "oracle_to_f16_one(W16(acc[e]) * s[b])", "oracle_to_f16_one(W16(acc[e]) * s[0])"),
}


def _pins():
    fns = []
    for mod in (to, tc, tn):
        for name, fn in inspect.getmembers(mod, inspect.isfunction):
            if not name.startswith("test_") or fn.__module__ != mod.__name__:
                continue
            if "exhaustive_vs" in name or "fraction" in name:
                continue
            fns.append(fn)
    return fns


def _params(fn):
    """Parameter sets for a pin: its parametrize marks, else one empty call."""
    marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
    if not marks:
        return [{}]
    argnames, values = marks[0].args
    names = [a.strip() for a in argnames.split(",")] if isinstance(argnames, str) else list(argnames)
    if len(names) == 1:
        return [{names[0]: v} for v in values]
    return [dict(zip(names, v)) for v in values]


def _fails(orc, fn):
    for kw in _params(fn):
        args = {}
        sig = inspect.signature(fn).parameters
        if "orc" in sig:
            args["orc"] = orc
        if "request" in sig:
            continue
        try:
            fn(**args, **kw)
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, "mutation site not found: " + name
    src = tmp_path / "mut.c"
    src.write_text(SRC.replace(old, new))
    lib = str(tmp_path / "libmut.so")
    subprocess.check_call(["gcc", *oracle.CFLAGS, str(src), "-o", lib, "-lm"])
    orc = oracle.Oracle(lib)
    caught = [fn.__name__ for fn in _pins() if _fails(orc, fn)]
    assert caught, "no pin fails for mutant: " + name


def test_unmutated_copy_passes_every_pin(tmp_path):
    """Control: the same harness on an unmodified copy finds nothing."""
    src = tmp_path / "same.c"
    src.write_text(SRC)
    lib = str(tmp_path / "libsame.so")
    subprocess.check_call(["gcc", *oracle.CFLAGS, str(src), "-o", lib, "-lm"])
    orc = oracle.Oracle(lib)
    assert [fn.__name__ for fn in _pins() if _fails(orc, fn)] == []
