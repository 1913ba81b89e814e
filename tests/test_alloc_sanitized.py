"""The host block allocator (csrc/alloc.cpp) built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven through its C API by seeded random operation sequences,
every result compared with the oracle allocator's (CPU only).

[PAG] "How paging works" (FIFO free list, a block taken only when needed), "Sharing blocks
between sequences" (reference counts, copy-on-write), "Related techniques" (blocks return to
the pool at once).  Error cases (an id out of range, a free block shared or released, an empty
pool) must come back as the documented codes, with no sanitizer report.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.paged import BlockAllocator, NoBlocksError

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KVS_OK, KVS_E_INVAL, KVS_E_NOBLOCKS, KVS_E_STATE = 0, -1, -2, -3


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("asan") / "alloc_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "kv_cache_sparsification_amd", "csrc", "alloc.cpp"),
           os.path.join(ROOT, "tests", "alloc_driver.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def _run(exe, script):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    p = subprocess.run([exe], input="\n".join(script) + "\n", capture_output=True, text=True, env=env, timeout=120)
    assert p.returncode == 0, f"sanitized allocator failed (rc {p.returncode}):\n{p.stderr[-3000:]}"
    assert "AddressSanitizer" not in p.stderr and "runtime error" not in p.stderr, p.stderr[-3000:]
    return p.stdout.splitlines()


def _expect(a: BlockAllocator, op, arg):
    """The oracle allocator's result line for one operation (the driver's output format)."""
    valid = a is not None and 0 <= arg < a.num_blocks
    if op == "alloc":
        try:
            return f"{KVS_OK} {a.alloc()}"
        except NoBlocksError:
            return f"{KVS_E_NOBLOCKS} -1"
    if op in ("incref", "decref"):
        if not valid:
            return f"{KVS_E_INVAL}"
        if a.ref[arg] == 0:
            return f"{KVS_E_STATE}"
        (a.incref if op == "incref" else a.decref)(arg)
        return f"{KVS_OK}"
    if op == "count":
        return f"{a.ref[arg]}" if valid else f"{KVS_E_INVAL}"
    if op == "cow":
        if not valid:
            return f"{KVS_E_INVAL} -1 -1"
        if a.ref[arg] == 0:
            return f"{KVS_E_STATE} -1 -1"
        if a.ref[arg] > 1 and not a.free:
            return f"{KVS_E_NOBLOCKS} -1 -1"
        nb, swapped = a.cow(arg)
        return f"{KVS_OK} {nb} {int(swapped)}"
    if op == "nfree":
        return f"{a.num_free()}"
    if op == "freelist":
        return " ".join(str(x) for x in [len(a.free)] + list(a.free))
    raise ValueError(op)


@pytest.mark.parametrize("seed", range(6))
def test_random_operations_match_the_oracle(driver, seed):
    r = np.random.default_rng(seed)
    script, expected = [], []
    for _ in range(8):                                 # several allocators per run (create / destroy)
        n = int(r.integers(1, 65))
        if r.random() < 0.5:
            order = [int(x) for x in r.permutation(n)[: int(r.integers(0, n + 1))]]
            script.append(f"create {n} " + " ".join(map(str, order)) if order else f"create {n} -1")
            if not order:
                # an empty given list is written as one bad id: creation must fail cleanly
                expected.append(f"{KVS_E_INVAL}")
                a = None
                script.append("destroy"); expected.append("0")
                continue
            a = BlockAllocator(n, order)
        else:
            script.append(f"create {n}")
            a = BlockAllocator(n)
        expected.append(f"{KVS_OK}")
        for _ in range(600):
            op = r.choice(["alloc", "alloc", "incref", "decref", "decref", "cow", "count", "nfree", "freelist"])
            arg = int(r.integers(-2, n + 2)) if r.random() < 0.1 else int(r.integers(0, n))
            script.append(op if op in ("alloc", "nfree", "freelist") else f"{op} {arg}")
            expected.append(_expect(a, op, arg))
        script.append("destroy"); expected.append("0")
    got = _run(driver, script)
    assert len(got) == len(expected)
    for i, (g, e) in enumerate(zip(got, expected)):
        assert g == e, f"line {i} ({script[i]}): got {g!r}, oracle {e!r}"


def test_bad_creation_arguments(driver):
    script = ["create 0", "create -3", "create 4 1 1", "create 4 0 4", "create 4 3 2", "count 0", "count 1",
              "freelist", "destroy"]
    expected = [f"{KVS_E_INVAL}", f"{KVS_E_INVAL}", f"{KVS_E_INVAL}", f"{KVS_E_INVAL}", f"{KVS_OK}", "1", "1",
                "2 3 2", "0"]
    assert _run(driver, script) == expected
