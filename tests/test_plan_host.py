"""The prefill's chunk plan built for the host (tests/cpu/plan_host.cpp runs
plan_sequences, the function the GPU plan kernel runs, with one thread per
lane): its tables against the plan computed here, and its memory bounds on
invalid cu_seqlens (lengths that swing by up to 2^32, random words), where
the old 32-bit sums could wrap to a negative chunk index."""
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "cpu", "plan_host.cpp")
CSRC = os.path.join(ROOT, "long_context_attn_amd", "csrc")


@pytest.fixture(scope="module")
def plan_bin(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("plan") / "plan_host")
    subprocess.run(["g++", "-O1", "-std=c++17", "-pthread", "-I" + CSRC, SRC, "-o", exe],
                   check=True)
    return exe


def run(exe, nseq, chunk, max_chunks, cu=None, seqlen=0, total=None):
    if total is None:
        total = int(cu[-1]) if cu is not None else nseq * seqlen
    head = "%d %d %d %d %d\n" % (nseq, -1 if cu is not None else seqlen, total, chunk, max_chunks)
    body = " ".join(str(int(x)) for x in cu) + "\n" if cu is not None else ""
    out = subprocess.run([exe], input=head + body, capture_output=True, text=True, check=True)
    lines = out.stdout.split("\n")
    err, n_chunks, guards = map(int, lines[0].split())
    segs = [tuple(map(int, l.split())) for l in lines[1:1 + nseq]]
    ch = [tuple(map(int, l.split())) for l in lines[1 + nseq:1 + nseq + n_chunks]]
    return err, n_chunks, guards == 1, segs, ch


def expected(lengths, chunk):
    segs, ch, start = [], [], 0
    for s, L in enumerate(lengths):
        cnt = -(-L // chunk) if L > 0 else 0
        segs.append((len(ch), cnt))
        for c in range(cnt):
            ch.append((start + c * chunk, min(chunk, L - c * chunk), s))
        start += L
    return segs, ch


def test_valid_varlen_tables(plan_bin):
    rng = np.random.default_rng(5)
    lengths = list(rng.integers(0, 700, 1500))  # more sequences than lanes, some empty
    lengths[3] = 0
    cu = np.concatenate([[0], np.cumsum(lengths)])
    chunk = 128
    maxc = int(cu[-1]) // chunk + len(lengths)
    err, n, guards, segs, ch = run(plan_bin, len(lengths), chunk, maxc, cu=cu)
    es, ec = expected(lengths, chunk)
    assert (err, guards) == (0, True)
    assert n == len(ec) and segs == es and ch == ec


def test_uniform_rows(plan_bin):
    err, n, guards, segs, ch = run(plan_bin, 3, 64, 3 * 2 + 3, seqlen=100)
    es, ec = expected([100, 100, 100], 64)
    assert (err, guards, segs, ch) == (0, True, es, ec)


@pytest.mark.parametrize("nseq", [64, 200, 2000])
def test_swinging_lengths_stay_in_bounds(plan_bin, nseq):
    # cu[0] = 0 and cu[nseq] = total, with lengths of +-(2^32 - 1) in between:
    # 32-bit sums of the chunk counts (2^26 each at chunk 64) wrap after about
    # 32 of them (a 32-bit build of this plan faults on 200 and 2000)
    cu = [0]
    for i in range(1, nseq):
        cu.append(2**31 - 1 if i % 2 else -2**31)
    cu.append(1000)
    err, n, guards, segs, _ = run(plan_bin, nseq, 64, 1000 // 64 + nseq, cu=cu)
    assert err == 1 and n == 0 and guards
    assert all(c == 0 for _, c in segs)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_words_stay_in_bounds(plan_bin, seed):
    # an uninitialised cu_seqlens buffer
    rng = np.random.default_rng(seed)
    nseq = 3000
    cu = rng.integers(-2**31, 2**31, nseq + 1)
    total = 1 << 20
    err, n, guards, segs, _ = run(plan_bin, nseq, 64, total // 64 + nseq, cu=cu, total=total)
    assert err == 1 and n == 0 and guards
    assert all(c == 0 for _, c in segs)


def test_table_overflow_reported(plan_bin):
    # a chunk table smaller than the plan needs: error 2, nothing written past it
    lengths = [300, 500, 64]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    err, n, guards, segs, _ = run(plan_bin, 3, 64, 5, cu=cu)
    assert err == 2 and n == 0 and guards
    assert all(c == 0 for _, c in segs)
