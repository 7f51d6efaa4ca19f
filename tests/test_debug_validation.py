"""Debug validation (host side, no GPU): the race checks of store and move ids agree
with a brute-force statement of the rule, name the first offending pair, and raise
UKV_ERR_RACE; an AddressSanitizer / UBSan build of the host library's plan, view and
check code (g++, CPU only) runs the same cases and a spec fuzz clean."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import store_gather_amd as U

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def store_races(ids):
    """Brute force: some row other than the sink row 0 named twice."""
    seen = set()
    for x in ids:
        if x != 0 and x in seen:
            return True
        seen.add(x)
    return False


def move_races(dst, src):
    """Brute force: dst repeats a row, or a source row is also a destination."""
    return len(set(dst)) != len(dst) or bool(set(dst) & set(src))


def status(fn, *a):
    try:
        fn(*a)
        return "UKV_OK"
    except U.UkvError as e:
        return e.status


@pytest.mark.parametrize("seed", range(300))
def test_checks_match_brute_force(seed):
    g = np.random.default_rng(seed)
    n = int(g.integers(0, 40))
    hi = int(g.integers(1, 4 * n + 2))
    ids = g.integers(0, hi, size=n).astype(np.int32)
    assert status(U.ukv_check_store_ids, ids) == ("UKV_ERR_RACE" if store_races(ids.tolist()) else "UKV_OK")
    dst = g.permutation(hi)[:n].astype(np.int32) if n <= hi else ids
    if g.random() < 0.3 and n:
        dst[int(g.integers(n))] = dst[0]
    src = g.integers(0, hi, size=n).astype(np.int32)
    assert status(U.ukv_check_move_ids, dst, src) == ("UKV_ERR_RACE" if move_races(dst.tolist(), src.tolist())
                                                      else "UKV_OK")


def test_messages_name_the_pair():
    with pytest.raises(U.UkvError, match=r"ids\[1\] and ids\[4\] are both row 77"):
        U.ukv_check_store_ids(np.array([5, 77, 0, 0, 77], np.int32))
    U.ukv_check_store_ids(np.array([0, 0, 0, 3, 4], np.int32))  # tombstones share the sink row
    with pytest.raises(U.UkvError, match=r"dst\[0\] and dst\[2\] are both 9"):
        U.ukv_check_move_ids(np.array([9, 1, 9], np.int32), np.array([2, 3, 4], np.int32))
    with pytest.raises(U.UkvError, match=r"src\[1\] = 1 is also dst\[1\]"):
        U.ukv_check_move_ids(np.array([9, 1, 8], np.int32), np.array([2, 1, 4], np.int32))
    U.ukv_check_move_ids(np.array([9, 1, 8], np.int32), np.array([2, 2, 4], np.int32))  # a row read twice is fine
    U.ukv_check_store_ids(np.zeros(0, np.int32))
    U.ukv_check_move_ids(np.zeros(0, np.int32), np.zeros(0, np.int32))


def test_large_inputs():
    g = np.random.default_rng(3)
    ids = g.permutation(1 << 22)[: 1 << 20].astype(np.int32)
    U.ukv_check_store_ids(ids)
    ids[777_777] = ids[12]
    with pytest.raises(U.UkvError, match="ids\\[12\\] and ids\\[777777\\]"):
        U.ukv_check_store_ids(ids)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_library_under_address_sanitizer(tmp_path):
    """ukv_plan.cpp (spec arithmetic and gates, views, race checks, status names) built
    with -fsanitize=address,undefined by g++ (CPU only; no device code is involved) and
    driven through its C entry points: specs at the gates' boundaries and a seeded fuzz
    of valid and invalid specs, views of every layer of the valid ones, and the race
    checks on random id sets.  Any sanitizer report fails the run."""
    exe = tmp_path / "ukv_host_asan"
    src = os.path.join(ROOT, "tests", "asan", "host_driver.cpp")
    lib = os.path.join(ROOT, "store_gather_amd", "csrc", "ukv_plan.cpp")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "store_gather_amd", "csrc"), "-I/opt/rocm/include", src, lib, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-3000:])
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
    assert "cases ok" in r.stdout
