"""Pins of the oracle's counter-based generator (Philox4x32-10) and of the
LoRA-dropout keep mask drawn from it (CPU only).

* Library pin: rocRAND's Philox4x32-10 -- an implementation of the same
  published generator in the ROCm headers, run here on the host -- with
  seed s, subsequence q and an offset of 4 i numbers returns, as its next
  four words, the generator at counter (i mod 2^32, i >> 32, q mod 2^32,
  q >> 32) under key (s mod 2^32, s >> 32): the oracle's counter layout.
  Skipped only on a machine without a HIP compiler.
* The mapping of a draw to eight elements, on the library's first draw.
* Statistics: keep fraction, per-position balance, uniformity, and
  independence of neighbouring draws and of different streams.
* The threshold's rounding and its limits (p = 0 keeps everything; p near 1
  keeps nothing).
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import oracle.philox as op

_PROBE = r"""
#include <rocrand/rocrand_kernel.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  const unsigned long long seed = strtoull(argv[1], 0, 0), sub = strtoull(argv[2], 0, 0),
                           off = strtoull(argv[3], 0, 0);
  const int n = atoi(argv[4]);
  rocrand_state_philox4x32_10 st;
  rocrand_init(seed, sub, off, &st);
  for (int i = 0; i < n; ++i) {
    const uint4 v = rocrand4(&st);
    printf("%u %u %u %u\n", v.x, v.y, v.z, v.w);
  }
  return 0;
}
"""


def _hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


@pytest.fixture(scope="module")
def rocrand_philox(tmp_path_factory):
    """Runs rocRAND's host-side Philox4x32-10: (seed, subsequence, offset in
    numbers, n) -> [n, 4] uint32 of consecutive four-word draws."""
    cc = _hipcc()
    if cc is None:
        pytest.skip("no HIP compiler for the rocRAND library pin")
    d = tmp_path_factory.mktemp("philox")
    src, exe = d / "probe.cpp", d / "probe"
    src.write_text(_PROBE)
    res = subprocess.run([cc, "-x", "hip", "--offload-arch=gfx950", "-O1", str(src), "-o",
                          str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr

    def run(seed, sub, off, n):
        out = subprocess.run([str(exe), str(seed), str(sub), str(off), str(n)],
                             capture_output=True, text=True, check=True).stdout
        return np.array([[int(v) for v in line.split()] for line in out.splitlines()],
                        dtype=np.uint64).astype(np.uint32)
    return run


CASES = [
    (0, 0, 0),
    (1, 0, 0),
    (0xDEADBEEFCAFEF00D, 12345, 0),
    ((1 << 64) - 1, (1 << 63) + 5, 0),
    (42, 7, 4 * ((1 << 32) - 2)),           # counter crosses into its second word
]


@pytest.mark.parametrize("seed,sub,first", CASES, ids=[str(c) for c in range(len(CASES))])
def test_generator_equals_rocrand(rocrand_philox, seed, sub, first):
    n = 48
    lib = rocrand_philox(seed, sub, first, n)
    i = np.arange(n, dtype=np.uint64) + np.uint64(first // 4)
    ctr = np.stack([i & np.uint64(0xFFFFFFFF), i >> np.uint64(32),
                    np.full(n, sub & 0xFFFFFFFF, dtype=np.uint64),
                    np.full(n, sub >> 32, dtype=np.uint64)], axis=1)
    got = oracle.philox4x32_10(ctr, (seed & 0xFFFFFFFF, seed >> 32))
    assert np.array_equal(got, lib)


def test_draw_to_element_mapping_on_the_first_draw(rocrand_philox):
    """Byte 0 under seed 0, offset 0 is the generator at counter 0: element j
    takes half j % 2 (low first) of word j / 2."""
    w = rocrand_philox(0, 0, 0, 1)[0]
    want = [(int(w[j // 2]) >> (16 * (j % 2))) & 0xFFFF for j in range(8)]
    assert list(oracle.dropout_uniforms(1, 8, 0, 0)[0]) == want
    # and the second byte of a row is the next counter
    w1 = rocrand_philox(0, 0, 4, 1)[0]
    want1 = [(int(w1[j // 2]) >> (16 * (j % 2))) & 0xFFFF for j in range(8)]
    assert list(oracle.dropout_uniforms(1, 16, 0, 0)[0, 8:]) == want1
    # the offset selects the subsequence (counter words 2, 3)
    w2 = rocrand_philox(9, 77, 0, 1)[0]
    want2 = [(int(w2[j // 2]) >> (16 * (j % 2))) & 0xFFFF for j in range(8)]
    assert list(oracle.dropout_uniforms(1, 8, 9, 77)[0]) == want2


def test_threshold_rounding_and_limits():
    assert oracle.dropout_threshold(0.0) == 0
    assert oracle.dropout_threshold(0.5) == 32768
    assert oracle.dropout_threshold(0.05) == 3277
    assert oracle.dropout_threshold(2.5 / 65536) == 2          # tie to even
    assert oracle.dropout_threshold(3.5 / 65536) == 4          # tie to even
    assert oracle.dropout_threshold(1.0 - 2.0 ** -20) == 65536
    keep = oracle.dropout_keep_philox(16, 64, 0.0, 3, 1)
    assert keep.all()
    assert not oracle.dropout_keep_philox(16, 64, 1.0 - 2.0 ** -20, 3, 1).any()


def test_keep_fraction_and_positions():
    M, K, p = 1024, 1024, 0.05
    keep = oracle.dropout_keep_philox(M, K, p, 2024, 0)
    q = 1.0 - oracle.realised_dropout(p)
    n = keep.size
    sd = np.sqrt(q * (1 - q) / n)
    assert abs(keep.mean() - q) < 5 * sd
    # each of the eight elements of a draw is balanced alike
    by_pos = keep.reshape(-1, 8).mean(axis=0)
    sd8 = np.sqrt(q * (1 - q) / (n / 8))
    assert np.all(np.abs(by_pos - q) < 5 * sd8), by_pos


def test_draws_are_uniform_and_independent():
    u = oracle.dropout_uniforms(512, 1024, 7, 3).astype(np.int64)
    n = u.size
    # top byte over 256 bins: chi-square with 255 degrees of freedom
    hist = np.bincount((u >> 8).reshape(-1), minlength=256)
    e = n / 256
    chi2 = float(((hist - e) ** 2 / e).sum())
    assert 150 < chi2 < 400, chi2
    # neighbours: within a draw (elements j, j + 1) and across draws
    # (element 7 of one counter, element 0 of the next)
    v = (u - 32767.5).reshape(-1, 8)
    lim = 5 / np.sqrt(v.shape[0])
    for j in range(7):
        c = np.corrcoef(v[:, j], v[:, j + 1])[0, 1]
        assert abs(c) < lim, (j, c)
    c = np.corrcoef(v[:-1, 7], v[1:, 0])[0, 1]
    assert abs(c) < lim, c


def test_streams_under_other_seeds_and_offsets_differ():
    M, K, p = 256, 512, 0.25
    a = oracle.dropout_keep_philox(M, K, p, 11, 0)
    q = oracle.realised_dropout(p)
    expect = 2 * q * (1 - q)                 # two independent masks disagree this often
    sd = np.sqrt(expect * (1 - expect) / a.size)
    for other in (oracle.dropout_keep_philox(M, K, p, 12, 0),
                  oracle.dropout_keep_philox(M, K, p, 11, 1),
                  oracle.dropout_keep_philox(M, K, p, 11 + (1 << 32), 0)):
        d = float(np.mean(a != other))
        assert abs(d - expect) < 5 * sd, d
    # and the same (seed, offset) replays the same mask
    assert np.array_equal(a, oracle.dropout_keep_philox(M, K, p, 11, 0))


def test_rows_of_a_mask_depend_only_on_their_bytes():
    """A mask's first rows are the mask of the first rows (the counter is the
    byte index m K / 8 + k / 8, which does not depend on M)."""
    full = oracle.dropout_keep_philox(40, 256, 0.1, 5, 9)
    assert np.array_equal(full[:17], oracle.dropout_keep_philox(17, 256, 0.1, 5, 9))


def _halves_high_first(M, K, seed, offset):
    u = _ORIG_UNIFORMS(M, K, seed, offset).reshape(-1, 2)
    return u[:, ::-1].reshape(M, K).copy()


_ORIG_UNIFORMS = op.dropout_uniforms


@pytest.mark.parametrize("name,attr,value", [
    ("key not advanced between rounds", "PHILOX_W0", 0),
    ("multipliers swapped", "PHILOX_M0", op.PHILOX_M1),
    ("seven rounds", "ROUNDS", 7),
    ("second Weyl constant dropped", "PHILOX_W1", 0),
])
def test_planted_generator_mistakes_are_caught(rocrand_philox, monkeypatch, name, attr, value):
    """Plausible mistakes in the generator, planted in the oracle, fail the
    library pin."""
    monkeypatch.setattr(op, attr, value)
    if attr == "PHILOX_M0":
        monkeypatch.setattr(op, "PHILOX_M1", 0xD2511F53)
    with pytest.raises(AssertionError):
        test_generator_equals_rocrand(rocrand_philox, *CASES[2])


def test_planted_half_order_mistake_is_caught(rocrand_philox, monkeypatch):
    monkeypatch.setattr(op, "dropout_uniforms", _halves_high_first)
    monkeypatch.setattr(oracle, "dropout_uniforms", _halves_high_first)
    with pytest.raises(AssertionError):
        test_draw_to_element_mapping_on_the_first_draw(rocrand_philox)
