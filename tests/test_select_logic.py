"""Host unit test of the top-k selection's per-thread logic (csrc/select_logic.hpp), compiled for
the CPU from the same header the selection kernels include and driven as the kernels drive it
(a 512-thread workgroup emulated with sequential prefix sums; tests/host/select_logic_host.hip).

Checked against brute force: the threshold search over random, sparse, single-bin and
out-of-range histograms (exactly one thread claims the bin when 1 <= need <= total, none
otherwise); the full selection (bin threshold, listing, two digit passes, ordered compaction)
over random keys and adversarial ties; and the guards the final selection applies to what the
scan left (an inconsistent threshold or count selects nothing instead of reading past a list).
Order: score key descending, index ascending; output ascending, -1 padded ("DeepSeek-V4
technical report walkthrough" (cyqw.cn), section 2.2: each query keeps its top-k entries)."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "select_logic_host.hip")
INC = os.path.join(ROOT, "compressed_sparse_attention_02_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def sel(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("sel") / "libselhost.so")
    subprocess.run([HIPCC, "-x", "hip", "--cuda-host-only", "-O2", "-std=c++17", "-shared", "-fPIC", "-I", INC, SRC,
                    "-o", out], check=True, capture_output=True)
    L = ctypes.CDLL(out)
    P = ctypes.c_void_p
    L.sel_threshold_host.argtypes = [P, ctypes.c_int, ctypes.c_uint32, P, P]
    L.sel_threshold_host.restype = ctypes.c_int
    L.sel_meta_consistent_host.argtypes = [ctypes.c_int, ctypes.c_uint32, ctypes.c_uint32]
    L.sel_meta_consistent_host.restype = ctypes.c_int
    L.sel_clamp_count_host.argtypes = [ctypes.c_uint32]
    L.sel_clamp_count_host.restype = ctypes.c_uint32
    L.sel_select_host.argtypes = [P, ctypes.c_int64, ctypes.c_int, P]
    L.sel_select_host.restype = ctypes.c_int
    return L


def threshold(L, hist, need):
    h = np.ascontiguousarray(hist, np.uint32)
    T = ctypes.c_int(0)
    above = ctypes.c_uint32(0)
    claims = L.sel_threshold_host(h.ctypes.data_as(ctypes.c_void_p), h.size, int(need), ctypes.byref(T),
                                  ctypes.byref(above))
    return claims, T.value, above.value


def brute_threshold(hist, need):
    run = 0
    for b in range(len(hist) - 1, -1, -1):
        if run < need <= run + int(hist[b]):
            return b, run
        run += int(hist[b])
    return -1, 0


def select(L, keys, k):
    keys = np.ascontiguousarray(keys, np.uint32)
    out = np.empty(k, np.int32)
    rc = L.sel_select_host(keys.ctypes.data_as(ctypes.c_void_p), keys.size, k, out.ctypes.data_as(ctypes.c_void_p))
    return rc, out


def brute_select(keys, k):
    n = keys.size
    order = np.lexsort((np.arange(n), -keys.astype(np.int64)))  # key descending, index ascending
    sel = np.sort(order[:min(k, n)]).astype(np.int32)
    return np.concatenate([sel, -np.ones(k - sel.size, np.int32)])


@pytest.mark.parametrize("nbins", [4096, 1024])
def test_threshold_random_and_adversarial(sel, nbins):
    g = np.random.default_rng(11)
    hists = [g.integers(0, 5, nbins), np.where(g.random(nbins) < 0.01, g.integers(1, 3000, nbins), 0),
             np.zeros(nbins, np.int64)]
    one = np.zeros(nbins, np.int64)
    one[g.integers(nbins)] = 70000  # every key in one bin
    hists.append(one)
    edge = np.zeros(nbins, np.int64)
    edge[0], edge[-1] = 5, 3  # the lowest and the highest bin
    hists.append(edge)
    for h in hists:
        tot = int(h.sum())
        needs = {1, tot, tot + 1, max(1, tot // 2), max(1, tot - 1)} | set(int(x) for x in g.integers(1, tot + 2, 20))
        for need in sorted(needs):
            claims, T, above = threshold(sel, h, need)
            bT, babove = brute_threshold(h, need)
            if 1 <= need <= tot:
                assert claims == 1 and (T, above) == (bT, babove), (need, tot, T, above, bT, babove)
            else:
                assert claims == 0 and T == -1, (need, tot, claims)


def test_guards(sel):
    assert sel.sel_meta_consistent_host(5, 10, 64)
    assert not sel.sel_meta_consistent_host(-1, 0, 64)          # no threshold bin
    assert not sel.sel_meta_consistent_host(5, 64, 64)          # nothing left to take from bin T
    assert not sel.sel_meta_consistent_host(5, 0xFFFFFFF0, 64)  # a count that would underflow need
    assert sel.sel_clamp_count_host(12) == 12
    assert sel.sel_clamp_count_host(8192) == 8192
    assert sel.sel_clamp_count_host(8193) == 8192
    assert sel.sel_clamp_count_host(0xFFFFFFFF) == 8192


CASES = ["random", "all_equal", "few_values", "one_bin", "low_bits", "top_heavy"]


@pytest.mark.parametrize("case", CASES)
def test_select_matches_brute_force(sel, case):
    g = np.random.default_rng(30 + CASES.index(case))
    n = 20000
    if case == "random":
        keys = g.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32)
    elif case == "all_equal":
        keys = np.full(n, 0x9ABCDEF0, np.uint32)
    elif case == "few_values":  # many ties at every threshold
        keys = g.choice(np.array([0x40000000, 0x40000001, 0x80000000, 0x80100000], np.uint32), n)
    elif case == "one_bin":  # one 12-bit bin, distinct low 20 bits in a narrow range
        keys = (0x7FF00000 + g.integers(0, 3000, n)).astype(np.uint32)
    elif case == "low_bits":  # the same top 22 bits, ties decided by the second digit pass
        keys = (0x12345000 | g.integers(0, 1024, n)).astype(np.uint32)
    else:  # a few large keys, then a wide spread
        keys = g.integers(0, 2**31, n, dtype=np.uint64).astype(np.uint32)
        keys[g.integers(0, n, 40)] = 0xFFFFFFFF
    for k in (1, 2, 64, 512, 1024, 2048):
        for m in (n, 1500, 7, 0):
            rc, got = select(sel, keys[:m], k)
            assert rc == 0, (case, k, m)
            assert np.array_equal(got, brute_select(keys[:m], k)), (case, k, m)
