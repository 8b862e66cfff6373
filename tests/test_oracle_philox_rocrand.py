"""Pin of the oracle's Philox-4x32-10 against an independent implementation:
rocRAND's header-only Philox-4x32-10 engine (rocrand_kernel.h, shipped with
ROCm), compiled for the host by this test and run on the CPU.

The dropout reading (keep bytes from Philox-4x32-10 of Salmon, Moraes, Dror
and Shaw, SC 2011; the FLASH-ATTN page names dropout on P, FlashAttention
"Background" and FlashAttention-2 "Background") needs the generator's round
constants to be the published ones.  The structural pins in
test_oracle_dropout_pins.py check the round function against numpy's
Philox-4x64-10; this test checks the 32-bit instance -- its two multipliers,
Weyl constants, round order and word layout -- word for word against
rocRAND.

rocRAND's engine: rocrand_init(seed, subsequence, offset) sets the key to
(seed mod 2^32, seed div 2^32) and the 128-bit counter to
subsequence * 2^64 + offset div 4, and returns word (offset mod 4) of the
block first; each block of four words is Philox-4x32-10 of the counter,
which then increments with carry (the 64-bit offset reaches counter words 0
and 1, the subsequence words 2 and 3).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pins", "rocrand_philox.cpp")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCRAND_HEADER = "/opt/rocm/include/rocrand/rocrand_kernel.h"


@pytest.fixture(scope="module")
def rocrand_exe(tmp_path_factory):
    if not (shutil.which(HIPCC) or os.path.exists(HIPCC)) or not os.path.exists(ROCRAND_HEADER):
        pytest.skip("hipcc or the rocRAND headers are not installed")
    exe = str(tmp_path_factory.mktemp("rocrand") / "rocrand_philox")
    r = subprocess.run([HIPCC, "--offload-host-only", "-O1", "-o", exe, SRC],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def rocrand_words(exe, seed, sub, off, count):
    r = subprocess.run([exe, str(seed), str(sub), str(off), str(count)], capture_output=True,
                       text=True, check=True)
    return np.array([int(x) for x in r.stdout.split()], np.uint64)


def oracle_words(seed, sub, off, count):
    """The same stream from oracle.philox(32, 10, ...): block b has counter
    sub * 2^64 + off // 4 + b (mod 2^128), split into four 32-bit words, least
    significant first; the stream starts at word off % 4 of block 0."""
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint64)
    start = sub * 2**64 + off // 4
    words, b = [], 0
    while len(words) < off % 4 + count:
        c = (start + b) % 2**128
        ctr = np.array([(c >> (32 * w)) & 0xFFFFFFFF for w in range(4)], np.uint64)
        words.extend(int(x) for x in oracle.philox(32, 10, ctr, key))
        b += 1
    return np.array(words[off % 4: off % 4 + count], np.uint64)


CASES = [
    (0, 0, 0),                                   # all-zero counter and key
    (0x123456789ABCDEF, 0, 0),                   # two key words
    (20111, 7, 4 * 1000),                        # a subsequence and an offset
    (2**64 - 1, 2**64 - 1, 4 * (2**32 - 3)),     # all-ones key and subsequence words
    (99, 3, 4 * (2**32 - 2)),                    # carry from counter word 0 into word 1
    (5, 2**32 - 1, 2**64 - 1),                   # the largest offset: word 3 of block 2^62 - 1
    (42, 0, 4 * 12345 + 3),                      # a stream that starts mid-block
    (0xDEADBEEF, 11, 2),
]


@pytest.mark.parametrize("seed,sub,off", CASES)
def test_oracle_philox_matches_rocrand(rocrand_exe, seed, sub, off):
    n = 64
    got = oracle_words(seed, sub, off, n)
    want = rocrand_words(rocrand_exe, seed, sub, off, n)
    assert want.shape == (n,)
    assert np.array_equal(got, want), (got[:8], want[:8])


def test_dropout_counter_layout_draws_from_rocrand_blocks(rocrand_exe):
    """The keep-byte contract draws block (j/4, i/4, bh, offset): as a 128-bit
    counter that is j/4 + 2^32 (i/4) + 2^64 (bh + 2^32 offset), i.e. rocRAND's
    subsequence bh + 2^32 offset at word offset 4 (j/4 + 2^32 (i/4))."""
    seed = 0x0123456789ABCDEF
    for j4, i4, bh, offw in ((0, 0, 0, 0), (5, 9, 3, 1), (511, 4095, 63, 7)):
        ctr = np.array([j4, i4, bh, offw], np.uint64)
        key = np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint64)
        want = rocrand_words(rocrand_exe, seed, bh + (offw << 32), 4 * (j4 + (i4 << 32)), 4)
        assert np.array_equal(oracle.philox(32, 10, ctr, key), want)
