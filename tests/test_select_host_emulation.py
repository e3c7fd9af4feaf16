"""The exact selection among candidate lists (sel::select_candidates in select_dev.h, the
code the resolve kernels run) compiled for the host on a SIMT emulation of wave64 (one OS
thread per GPU thread, ballots and shuffles exchanged at per-wave barriers) and checked
against a brute-force selection: the k largest keys, ties to the lowest index, output
ascending [Lighthouse, "deep deepseek v4 release", section 八 item 3: top-k of the
compressed entries].  The cases put up to 32 candidates on one thread, all of them above
or equal to the threshold, which a count of fewer bits than the per-thread maximum gets
wrong."""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_attention_26_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")


@pytest.fixture(scope="module")
def emul(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("no g++")
    d = tmp_path_factory.mktemp("selemul")
    src = open(os.path.join(CSRC, "select_dev.h")).read()
    assert src.count('#include "common.h"') == 1
    open(d / "select_dev_under_test.h", "w").write(src.replace('#include "common.h"',
                                                               '#include "simt_emul.h"'))
    shutil.copy(os.path.join(HOST, "simt_emul.h"), d / "simt_emul.h")
    exe = d / "selemul"
    r = subprocess.run(["g++", "-std=c++20", "-O1", "-pthread", "-I", str(d),
                        os.path.join(HOST, "select_candidates_emul.cpp"), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return str(exe)


def brute(keys, idx, k):
    order = sorted(range(len(keys)), key=lambda i: (-int(keys[i]), int(idx[i])))
    return sorted(int(idx[i]) for i in order[:k])


def run(exe, per, keys, idx, k, L):
    lines = [f"{per} 512 {len(keys)} {k} {L}"] + [f"{int(a)} {int(b)}" for a, b in zip(keys, idx)]
    r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    return [int(x) for x in r.stdout.split()]


def sparse_indices(rng, C):
    # ascending indices with gaps, as the concatenated chunk lists hold them
    return np.cumsum(rng.integers(1, 5, size=C))


CASES = [
    # (name, PER, C, k, builder)
    ("all_tied_16000", 32, 16000, 1024, "tied"),
    ("all_tied_16384", 32, 16384, 1024, "tied"),
    ("all_tied_15873", 32, 15873, 1000, "tied"),
    ("planted_run_above", 32, 16000, 1024, "planted"),
    ("random_keys_32", 32, 16200, 1024, "random"),
    ("random_keys_16", 16, 8192, 512, "random"),
    ("tied_16", 16, 8192, 1024, "tied"),
]


@pytest.mark.parametrize("name,per,C,k,kind", CASES, ids=[c[0] for c in CASES])
def test_select_candidates_host_emulation(emul, name, per, C, k, kind):
    rng = np.random.default_rng(abs(hash(name)) % (2**32))
    L = 0x8000
    idx = sparse_indices(rng, C)
    if kind == "tied":
        keys = np.full(C, L)
    elif kind == "planted":
        # every thread holds 32 keys equal to the floor except thread 100, whose 32 keys are
        # all above it: the threshold is the floor, thread 100 contributes 32 keys above T
        keys = np.full(C, L)
        per_t = -(-C // 512)
        keys[100 * per_t: 101 * per_t] = L + 1 + rng.integers(0, 50, size=per_t)
    else:
        keys = L + rng.integers(0, 700, size=C)
    got = run(emul, per, keys, idx, k, L)
    assert got == brute(keys, idx, k)


def test_bf16_ge_mask_word_parallel_host_emulation(emul):
    """The selector's test of two bf16 keys per 32-bit word against a floor (subtracting the
    floor's raw bits from both halves at once, a byte permute gathering the flags) equals
    the key-by-key comparison on 400 000 random chunks, including +-0, the extremes, keys
    one step either side of the floor and every tail length."""
    r = subprocess.run([emul, "gemask"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    bad, runs = (int(x) for x in r.stdout.split())
    assert runs == 400000
    assert bad == 0
