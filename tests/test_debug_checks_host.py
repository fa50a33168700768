"""The host-side permutation checks behind MOE_DEBUG, on the CPU.

The library runs these checks (csrc/debug_checks.h) on arrays it copies back
from the device; here a small shim built with g++ exposes them so that each
kind of broken permutation can be handed to them directly. A valid permutation
is built with numpy's stable argsort (the grouping the permutation call
defines: slots grouped by expert, ascending slot inside an expert).
"""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "debug_checks_shim.cpp")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")


@pytest.fixture(scope="module")
def shim(tmp_path_factory):
    so = str(tmp_path_factory.mktemp("dbg") / "debug_checks_shim.so")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-shared", "-fPIC", SRC, "-o", so], check=True)
    lib = ctypes.CDLL(so)
    P = ctypes.c_void_p
    for name, args in (("chk_offsets", [P, ctypes.c_int, ctypes.c_long]),
                       ("chk_sorted", [P, ctypes.c_long, ctypes.c_long]),
                       ("chk_rows", [P, ctypes.c_long]),
                       ("chk_permutation", [P, P, P, P, ctypes.c_int, ctypes.c_long])):
        fn = getattr(lib, name)
        fn.argtypes, fn.restype = args, ctypes.c_char_p
    return lib


def _p(a):
    return np.ascontiguousarray(a, dtype=np.int32).ctypes.data_as(ctypes.c_void_p)


def _perm(ids, E):
    ids = np.asarray(ids, dtype=np.int32)
    sorted_slots = np.argsort(ids, kind="stable").astype(np.int32)
    off = np.zeros(E + 1, dtype=np.int32)
    off[1:] = np.cumsum(np.bincount(ids, minlength=E))
    s2r = np.empty_like(sorted_slots)
    s2r[sorted_slots] = np.arange(len(ids), dtype=np.int32)
    return off, sorted_slots, s2r


def _check_perm(shim, ids, off, srt, s2r, E):
    arrs = [np.ascontiguousarray(a, dtype=np.int32) for a in (ids, off, srt, s2r)]
    return shim.chk_permutation(*[a.ctypes.data_as(ctypes.c_void_p) for a in arrs], E, len(arrs[0])).decode()


def test_valid_permutations_pass(shim):
    rng = np.random.default_rng(0)
    for S, E in ((1, 1), (7, 3), (64, 16), (1000, 16), (513, 64)):
        ids = rng.integers(0, E, S)
        if S >= 64:
            ids[: S // 2] = 0                     # a hot expert, and some experts without rows
        off, srt, s2r = _perm(ids, E)
        assert _check_perm(shim, ids, off, srt, s2r, E) == ""
        assert shim.chk_offsets(_p(off), E, S) == b""
        assert shim.chk_sorted(_p(srt), S, S) == b""
        assert shim.chk_rows(_p(s2r), S) == b""


def test_offsets_checks(shim):
    assert b"expert_offsets[0] = 1" in shim.chk_offsets(_p([1, 3, 5]), 2, 5)
    assert b"decrease at expert 1 (6 -> 4)" in shim.chk_offsets(_p([0, 6, 4, 8]), 3, 8)
    assert b"exceeds the 8 slots" in shim.chk_offsets(_p([0, 4, 9]), 2, 8)
    assert shim.chk_offsets(_p([0, 4, 6]), 2, 8) == b""    # fewer rows than slots: valid for the FFN calls
    assert shim.chk_offsets(_p([0, 0, 0]), 2, 0) == b""


def test_sorted_and_rows_checks(shim):
    assert b"sorted_slots[2] = 8 is outside [0, 8)" in shim.chk_sorted(_p([0, 1, 8, 3]), 4, 8)
    assert b"sorted_slots[1] = -1" in shim.chk_sorted(_p([0, -1]), 2, 8)
    assert b"slot 3 is held by two sorted rows (the second: 2)" in shim.chk_sorted(_p([3, 1, 3]), 3, 8)
    assert shim.chk_sorted(_p([5, 1, 8]), 2, 8) == b""        # rows past `rows` are not looked at
    assert b"slot_to_row[1] = 4" in shim.chk_rows(_p([0, 4, 1, 2]), 4)
    assert b"slot_to_row[0] = -2" in shim.chk_rows(_p([-2, 0]), 2)
    assert shim.chk_rows(_p([-1, 0, 3, 1]), 4) == b""


def test_each_broken_permutation_is_named(shim):
    """One mistake at a time in a valid permutation; each check must fire."""
    rng = np.random.default_rng(1)
    E, S = 4, 40
    ids = rng.integers(0, E, S)
    off, srt, s2r = _perm(ids, E)
    assert _check_perm(shim, ids, off, srt, s2r, E) == ""

    bad = ids.copy(); bad[5] = E
    assert "1 slots have an expert id outside [0, 4) (first: slot 5, id 4)" in _check_perm(shim, bad, off, srt, s2r, E)
    bad = ids.copy(); bad[[3, 9]] = -1
    assert "2 slots have an expert id outside" in _check_perm(shim, bad, off, srt, s2r, E)

    o = off.copy(); o[E] -= 1
    assert "expected all 40 slots" in _check_perm(shim, ids, o, srt, s2r, E)
    o = off.copy(); o[1], o[2] = o[2], o[1]
    assert "decrease" in _check_perm(shim, ids, o, srt, s2r, E) or "routed to expert" in _check_perm(shim, ids, o, srt, s2r, E)

    # two rows of one expert swapped: still a permutation, not ascending
    e = int(np.argmax(np.diff(off)))
    r = int(off[e])
    s = srt.copy(); s[r], s[r + 1] = s[r + 1], s[r]
    r2 = s2r.copy(); r2[s[r]], r2[s[r + 1]] = r, r + 1
    assert "out of ascending order" in _check_perm(shim, ids, off, s, r2, E)

    # rows of two experts swapped (the inverse kept consistent): wrong expert
    a, b = int(off[0]), int(off[E - 1])
    s = srt.copy(); s[a], s[b] = s[b], s[a]
    r2 = s2r.copy(); r2[s[a]], r2[s[b]] = a, b
    assert "routed to expert" in _check_perm(shim, ids, off, s, r2, E)

    # slot_to_row not the inverse
    r2 = s2r.copy(); r2[srt[0]], r2[srt[1]] = 1, 0
    assert "but the slot is held by sorted row" in _check_perm(shim, ids, off, srt, r2, E)
    # a duplicated slot
    s = srt.copy(); s[1] = s[0]
    assert "held by two sorted rows" in _check_perm(shim, ids, off, s, s2r, E)
