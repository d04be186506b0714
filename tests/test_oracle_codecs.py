"""Pins of the oracle's scalar codecs against things outside the oracle.

* E2M1: every binary32 pattern against a brute-force nearest-grid search
  (independent C, binary64 distances) -- tests/pins/e2m1_bruteforce.c.
* E4M3: every binary32 value in [0, 464] against torch's float8_e4m3fn cast
  (an independent library rounding routine), plus the OCP decode table.
* bf16: every upper half-word with tie / near-tie lower halves against
  torch's bfloat16 cast.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_e2m1_exhaustive_against_bruteforce(orc, tmp_path):
    lib_dir = os.path.dirname(orc.build(force=False))
    exe = str(tmp_path / "e2m1bf")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-o", exe,
                    os.path.join(ROOT, "tests", "pins", "e2m1_bruteforce.c"),
                    "-L" + lib_dir, "-loracle", "-Wl,-rpath," + lib_dir, "-lm"], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True,
                         env=dict(os.environ, OMP_NUM_THREADS="8")).stdout.split()
    checked, bad = int(out[0]), int(out[1])
    assert checked == 2**32 - 2 * (2**23 - 1) - 2  # all patterns minus NaNs and +-inf
    assert bad == 0


def test_e2m1_infinities_saturate(orc):
    codes = orc.e2m1_encode(np.array([np.inf, -np.inf, 1e38, -1e38], np.float32))
    assert codes.tolist() == [7, 15, 7, 15]


def test_e2m1_decode_grid(orc):
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert [orc.e2m1_decode(c) for c in range(8)] == grid
    assert [orc.e2m1_decode(8 + c) for c in range(8)] == [-g for g in grid]
    # dec(enc(g)) = g on every grid point, both signs
    g = np.array(grid + [-v for v in grid], np.float32)
    assert np.array_equal(np.array([orc.e2m1_decode(c) for c in orc.e2m1_encode(g)], np.float32), g)


def test_e4m3_exhaustive_against_torch(orc):
    top = np.float32(464.0).view(np.uint32)
    chunk = 1 << 24
    start = 0
    while start <= top:
        stop = min(int(top) + 1, start + chunk)
        u = np.arange(start, stop, dtype=np.uint32)
        f = u.view(np.float32)
        ours = orc.e4m3_encode(f)
        ref = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        bad = np.nonzero(ours != ref)[0]
        assert bad.size == 0, "first mismatch at %r: ours %x torch %x" % (
            f[bad[0]], ours[bad[0]], ref[bad[0]])
        start = stop


def test_e4m3_saturates_above_464(orc):
    # torch turns these into NaN; the reading taken here saturates at 448.
    v = np.array([464.00003, 480, 500, 1e6, 3.4e38], np.float32)
    assert orc.e4m3_encode(v).tolist() == [0x7E] * 5


def test_e4m3_decode_table_matches_ocp(orc):
    tab = orc.e4m3_decode_table()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = codes.to(torch.float32).numpy()
    finite = np.isfinite(ref)
    assert np.array_equal(tab[finite], ref[finite])
    assert np.isnan(tab[0x7F]) and np.isnan(tab[0xFF])
    assert tab[0x7E] == 448.0 and tab[0x01] == 2.0**-9 and tab[0x08] == 2.0**-6


def test_bf16_against_torch(orc):
    hi = np.arange(65536, dtype=np.uint32) << 16
    rng = np.random.default_rng(0)
    lows = [0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000]
    lows += rng.integers(0, 65536, 8).tolist()
    for lo in lows:
        u = hi | np.uint32(lo)
        f = u.view(np.float32)
        keep = ~np.isnan(f)
        f = f[keep]
        ours = orc.bf16_from_f32(f)
        ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(ours, ref), "low half %04x" % lo


def test_bf16_widening_exact(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = orc.f32_from_bf16(h)
    ok = ~np.isnan(f)
    back = orc.bf16_from_f32(f[ok])
    assert np.array_equal(back, h[ok])
